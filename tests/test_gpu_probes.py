"""The two calibration probes the bench's measured ceilings come from: each computes a
result the host can predict, so a timing can only come from work that was done."""
import numpy as np
import pytest
import torch

from long_context_sparse_amd import abi

pytestmark = pytest.mark.gpu


def _bf16(x: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of float32 values that bf16 holds exactly."""
    return (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _lane_sums(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Per lane, the sum of its 16 elements of A B under v_mfma_f32_32x32x16_bf16's layout:
    lane l holds A[l % 32][8 (l / 32) + e] and B[8 (l / 32) + e][l % 32] (e < 8), and
    C[8 (r / 4) + 4 (l / 32) + r % 4][l % 32] for r < 16."""
    A = np.zeros((32, 16)); B = np.zeros((16, 32))
    for l in range(64):
        A[l % 32, 8 * (l // 32): 8 * (l // 32) + 8] = a[l]
        B[8 * (l // 32): 8 * (l // 32) + 8, l % 32] = b[l]
    C = A @ B
    return np.array([sum(C[8 * (r // 4) + 4 * (l // 32) + r % 4, l % 32] for r in range(16)) for l in range(64)])


@pytest.mark.parametrize("wgs,iters,kind", [(1, 1, "int"), (7, 3, "int"), (300, 16384, "int"), (64, 100, "normal")])
def test_mfma_rate_sums(wgs, iters, kind):
    print(f"[gpu] rtp_mfma_rate wgs={wgs} iters={iters} {kind}", flush=True)
    rng = np.random.default_rng(wgs * 7 + iters)
    if kind == "int":
        vals = rng.integers(-3, 4, size=(2, 64, 8)).astype(np.float32)
    else:
        vals = rng.standard_normal((2, 64, 8)).astype(np.float32)
        vals = (_bf16(vals).astype(np.uint32) << 16).view(np.float32)
    ops = torch.from_numpy(_bf16(vals).view(np.int16).copy()).cuda()
    out = torch.full((wgs * 256 + 5,), -1.0, dtype=torch.float32, device="cuda")
    abi.rtp_mfma_rate(ops, out, wgs, iters)
    torch.cuda.synchronize()
    h = out.cpu().numpy().astype(np.float64)
    want = np.tile(4.0 * iters * _lane_sums(vals[0].astype(np.float64), vals[1].astype(np.float64)), 4 * wgs)
    if kind == "int":
        assert np.array_equal(h[: wgs * 256], want) or np.allclose(h[: wgs * 256], want, rtol=0, atol=1e-7 * np.abs(want).max() + 1)
    else:
        assert np.allclose(h[: wgs * 256], want, rtol=1e-3, atol=1e-3 * np.abs(want).max())
    assert np.all(h[wgs * 256:] == -1.0)  # nothing past the grid's outputs is written


@pytest.mark.parametrize("nt", [True, False])
@pytest.mark.parametrize("nbytes,wgs", [(16, 1), (4096 + 48, 3), (1 << 20, 64)])
def test_stream_read_fold(nt, nbytes, wgs):
    # each workgroup's word is the XOR of every 32-bit word its lanes read: 16-byte items
    # i = tid_global + k * stride (tid_global = wg * 256 + lane, stride = wgs * 256)
    print(f"[gpu] rtp_stream_read bytes={nbytes} wgs={wgs} nt={nt}", flush=True)
    rng = np.random.default_rng(nbytes + wgs)
    words = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(words.view(np.uint8).copy()).cuda()
    sink = torch.full((wgs + 3,), 7, dtype=torch.int32, device="cuda")
    abi.rtp_stream_read(buf, sink, wgs, nt)
    torch.cuda.synchronize()
    items = words.reshape(-1, 4)
    fold = np.bitwise_xor.reduce(items, axis=1)
    owner = (np.arange(items.shape[0]) % (wgs * 256)) // 256
    want = np.zeros(wgs, dtype=np.uint32)
    for w in range(wgs):
        sel = fold[owner == w]
        want[w] = np.bitwise_xor.reduce(sel) if sel.size else 0
    got = sink.cpu().numpy().view(np.uint32)
    assert np.array_equal(got[:wgs], want)
    assert np.all(sink.cpu().numpy()[wgs:] == 7)
