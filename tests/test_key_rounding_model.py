"""Host model of the device's index-key rounding (index_key_bf16 in the library's common
device header) against the oracle's exact rule (oracle.index_key: the exact sum of the
128 products rounded once to bf16, Review, Adaptive sparse attention equation, the key
side of s_h(m, n)).

The model follows the device's steps: per lane of a 16-lane row, 8 products summed with
fp64 FMAs, the row sum on the butterfly the DPP moves take, the error-bound test that
keeps the fp64 result, and otherwise the exact integer sum in 32-bit digits with the
rounding read from its bits.  Adversarial inputs (ties with tails of either sign far
below fp64's reach, cancellation to zero and to tiny values, subnormal and overflowing
results, signed zeros) must give the oracle's bits, and the fast path must be the one
taken on ordinary inputs."""
from fractions import Fraction

import numpy as np
import pytest

from key_cases import CASES, vec
from oracle import rtp_oracle as O


def bf2f(b: int) -> float:
    return float(np.array([b << 16], dtype=np.uint32).view(np.float32)[0])


def fma(a: float, b: float, c: float) -> float:
    return float(Fraction(a) * Fraction(b) + Fraction(c))  # one rounding, nearest-even


def rne_bf16(x: float) -> int:
    return O.bf16_round(x)


def device_model(w: np.ndarray, k: np.ndarray):
    """(bits, took_exact_path) as the device computes them."""
    wf = [bf2f(int(b)) for b in w]
    kf = [bf2f(int(b)) for b in k]
    xs, As = [], []
    for lane in range(16):
        d = range(8 * lane, 8 * lane + 8)
        x = wf[d[0]] * kf[d[0]]
        A = abs(x)
        for i in list(d)[1:]:
            x = fma(wf[i], kf[i], x)
            A = fma(abs(wf[i]), abs(kf[i]), A)
        xs.append(x)
        As.append(A)
    for perm in (lambda l: l ^ 1, lambda l: l ^ 2, lambda l: (l & ~7) | (7 - (l & 7)), lambda l: 15 - l):
        xs = [xs[l] + xs[perm(l)] for l in range(16)]
        As = [As[l] + As[perm(l)] for l in range(16)]
    assert len(set(xs)) == 1 and len(set(As)) == 1  # every lane of the row agrees
    x, A = xs[0], As[0]
    if A == 0.0:
        return 0, False
    E = A * 2.0 ** -48
    lo, hi = rne_bf16(x - E), rne_bf16(x + E)
    if lo == hi:
        return lo, False
    return exact_model(w, k), True


def exact_model(w: np.ndarray, k: np.ndarray) -> int:
    """The integer path: 17 limbs of 32-bit digits, LSB 2^-266."""
    L = [0] * 17
    for a, b in zip(w.tolist(), k.tolist()):
        ea, eb = (a >> 7) & 0xFF, (b >> 7) & 0xFF
        ma, mb = (a & 0x7F) | (0x80 if ea else 0), (b & 0x7F) | (0x80 if eb else 0)
        t = (ea or 1) + (eb or 1) - 2
        v = (ma * mb) << (t & 31)
        s = -1 if (a ^ b) & 0x8000 else 1
        L[t >> 5] += s * (v & 0xFFFFFFFF)
        L[(t >> 5) + 1] += s * (v >> 32)

    def carry(L):
        for j in range(16):
            c = L[j] >> 32
            L[j] -= c << 32
            L[j + 1] += c
    carry(L)
    neg = L[16] < 0
    if neg:
        L = [-x for x in L]
        carry(L)
    V = sum(d << (32 * j) for j, d in enumerate(L))
    if V == 0:
        return 0
    top = V.bit_length() - 1
    q = max(top - 7, 133)
    Q = (V >> q) & 0x1FF
    rbit = (V >> (q - 1)) & 1
    sticky = (V & ((1 << (q - 1)) - 1)) != 0
    if rbit and (sticky or (Q & 1)):
        Q += 1
    sign = 0x8000 if neg else 0
    if top < 140:
        return sign | Q
    e = top - 266 + 127
    if Q == 256:
        Q, e = 128, e + 1
    if e >= 255:
        return sign | 0x7F80
    return sign | (e << 7) | (Q - 128)


@pytest.mark.parametrize("name", sorted(CASES))
def test_model_matches_oracle_on_boundary_cases(name):
    w, k = CASES[name]
    got, _ = device_model(w, k)
    want = int(O.index_key(w.reshape(1, 128).repeat(16, 0), k)[0])
    assert got == want, (name, hex(got), hex(want))
    assert exact_model(w, k) == want, name


def test_tie_with_tail_needs_the_exact_path():
    """The double-rounding counterexample: fp64 drops 2^-90 and lands on the tie."""
    w, k = CASES["tie_plus_tail"]
    got, exact = device_model(w, k)
    assert exact and got == 0x3F81
    x = sum(bf2f(int(a)) * bf2f(int(b)) for a, b in zip(w, k))
    assert rne_bf16(x) == 0x3F80  # what one fp64 sum rounded once more gives


def test_random_inputs_take_the_fast_path_and_agree():
    g = np.random.default_rng(5)
    n_exact = 0
    for _ in range(60):
        w = (g.standard_normal(128) / np.sqrt(128)).astype(np.float32).view(np.uint32) >> 16
        k = g.standard_normal(128).astype(np.float32).view(np.uint32) >> 16
        w, k = w.astype(np.uint16), k.astype(np.uint16)
        got, exact = device_model(w, k)
        n_exact += exact
        assert got == int(O.index_key(w.reshape(1, 128).repeat(16, 0), k)[0])
        assert exact_model(w, k) == got
    assert n_exact == 0


def test_random_ties_with_random_tails():
    """Sums built to land on a bf16 midpoint plus or minus a tail 2^-20 .. 2^-90 of the
    bf16 ulp (the tail is a product of two powers of two)."""
    g = np.random.default_rng(9)
    n_exact = 0
    for it in range(40):
        n = int(g.integers(-20, 20))
        head = float(int(g.integers(128, 256))) * 2.0 ** n   # 8 significant bits, ulp 2^n
        half = 2.0 ** (n - 1)                                  # head + half is a midpoint
        e = n - 1 - int(g.integers(20, 90))
        sgn = 1.0 if it % 2 else -1.0
        w, k = vec((head, 1.0), (half, 1.0), (sgn * 2.0 ** (e // 2), 2.0 ** (e - e // 2)))
        got, exact = device_model(w, k)
        n_exact += exact
        assert got == int(O.index_key(w.reshape(1, 128).repeat(16, 0), k)[0]), it
    assert n_exact > 10  # tails below the fp64 sum's error bound take the exact path
