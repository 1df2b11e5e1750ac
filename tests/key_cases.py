"""Index-key inputs whose exact sums sit on or next to a bf16 rounding boundary, shared
by the host model of the device's key rounding and the GPU parity tests of the two
calls that write index keys.  Each case is a (w, k) pair of bf16 bit vectors of 128
dims; the expected key is oracle.index_key's (the exact sum rounded once)."""
import numpy as np


def f2bf(x: float) -> int:
    """bf16 bits of a value that bf16 holds exactly."""
    b = int(np.array([x], dtype=np.float32).view(np.uint32)[0])
    assert b & 0xFFFF == 0, x
    return b >> 16


def vec(*pairs, n=128):
    w = np.zeros(n, dtype=np.uint16)
    k = np.zeros(n, dtype=np.uint16)
    for i, (a, b) in enumerate(pairs):
        w[i], k[i] = f2bf(a), f2bf(b)
    return w, k


# (w, k) lists whose exact sums sit on or next to a rounding boundary
CASES = {
    "tie_plus_tail": vec((1.0, 1.0), (2.0 ** -8, 1.0), (2.0 ** -45, 2.0 ** -45)),    # 1 + 2^-8 + 2^-90: up
    "tie_minus_tail": vec((1.0, 1.0), (2.0 ** -8, 1.0), (-2.0 ** -45, 2.0 ** -45)),  # down
    "tie_exact": vec((1.0, 1.0), (2.0 ** -8, 1.0)),                                   # even: 1
    "tie_odd_exact": vec((1.0, 1.0), (2.0 ** -7, 1.0), (2.0 ** -8, 1.0)),             # 1 + 3*2^-8: to 1 + 2^-6
    "neg_tie_plus_tail": vec((-1.0, 1.0), (-2.0 ** -8, 1.0), (-2.0 ** -45, 2.0 ** -45)),
    "cancel_to_zero": vec((1.5, 2.0), (-3.0, 1.0), (2.0 ** -100, 2.0 ** -30), (-2.0 ** -100, 2.0 ** -30)),
    "cancel_to_tiny": vec((3.0, 2.0 ** 100), (-3.0, 2.0 ** 100), (2.0 ** -120, 2.0 ** -120)),
    "subnormal_result": vec((2.0 ** -70, 2.0 ** -60), (2.0 ** -70, 2.0 ** -64)),
    "subnormal_tie": vec((2.0 ** -67, 2.0 ** -67)),                                   # 2^-134: half the quantum
    "subnormal_tie_tail": vec((2.0 ** -67, 2.0 ** -67), (2.0 ** -120, 2.0 ** -126)),
    "overflow": vec((2.0 ** 127, 2.0), (2.0 ** 127, 2.0)),
    "signed_zeros": vec((-0.0, 1.0), (0.0, -1.0), (-0.0, -0.0)),
    "huge_minus_huge_plus_unit": vec((2.0 ** 120, 2.0 ** 120), (-2.0 ** 120, 2.0 ** 120), (1.0, 1.0 + 2.0 ** -7)),
}


