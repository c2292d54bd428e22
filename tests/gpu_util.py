"""Helpers shared by the GPU parity tests: moving bf16 bit patterns between
numpy and the device, and the parity tolerance.

Tolerance for bf16 outputs: |gpu - ref| <= 1e-2 * |ref| + 1e-3 per element, both
widened exactly from bf16 to fp32.  Flag, bitmask and sentinel words are
compared bit for bit.
"""
import numpy as np
import torch

RTOL = 1e-2
ATOL = 1e-3


def device():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    return torch.device("cuda:0")


def to_dev_bf16(a):
    a = np.ascontiguousarray(a, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device())


def from_dev_bf16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def widen(u16):
    return (np.asarray(u16, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def assert_bf16_close(got, ref, what=""):
    g = widen(got).astype(np.float64)
    r = widen(ref).astype(np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert not np.isnan(g).any(), "%s: NaN in GPU output" % what
    excess = np.abs(g - r) - RTOL * np.abs(r)
    worst = np.unravel_index(np.argmax(excess), excess.shape) if excess.size else None
    ok = excess.size == 0 or excess[worst] <= ATOL
    assert ok, "%s: %d elements outside |d| <= 1e-2|ref| + 1e-3; worst at %s: gpu %r ref %r" % (
        what, int((excess > ATOL).sum()), worst, g[worst], r[worst])


def flag_words_all_set(R, owner, tiles):
    """ready_in with every flag tile of every peer segment published
    (built directly, independent of both implementations)."""
    W = (tiles + 31) // 32
    words = np.zeros((R, W), dtype=np.uint32)
    for p in range(R):
        if p == owner:
            continue
        for t in range(tiles):
            words[p, t // 32] |= np.uint32(1 << (t % 32))
    return words


def to_dev_u32(a):
    a = np.ascontiguousarray(a, dtype=np.uint32)
    return torch.from_numpy(a.view(np.int32)).to(device())


def from_dev_u32(t):
    return t.cpu().numpy().view(np.uint32)
