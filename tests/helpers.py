"""Shared helpers for the GPU parity tests (test infrastructure)."""
from __future__ import annotations

import numpy as np

import oracle


def to_dev_bf16(a: np.ndarray):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).cuda().view(torch.bfloat16)


def to_dev_codes(a: np.ndarray):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint32).view(np.int32)).cuda()


def from_dev_bf16(t) -> np.ndarray:
    import torch

    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def exhaustive_window_codes(rng: np.random.Generator, nrows: int, bits: int, shift: int = 0):
    """Code rows in which every 12-bit window value 0..4095 occurs.

    In each block, weights t = t0, t0 + s, t0 + 2s, ... (s = ceil(12/bits),
    t0 the first weight whose window does not wrap, plus `shift`) read
    disjoint bit spans, so their windows can be written freely; the remaining
    bits are random. `shift` moves the written windows to other weight
    positions (for k = 2 all of t0 + s*i share one parity).
    Returns (codes [nrows, K*bits/32], K).
    """
    s = -(-12 // bits)
    t0 = -(-(12 - bits) // bits) + shift
    slots = list(range(t0, 256, s))
    nblocks = -(-4096 // len(slots))
    k = 256 * nblocks
    wpb = 256 * bits // 32
    codes = rng.integers(0, 2 ** 32, (nrows, k * bits // 32), dtype=np.uint32)
    for r in range(nrows):
        perm = rng.permutation(4096)
        vals = np.concatenate([perm, rng.integers(0, 4096, nblocks * len(slots) - 4096)])
        for b in range(nblocks):
            blk = codes[r, b * wpb:(b + 1) * wpb]
            stream = 0
            for i, w in enumerate(blk.tolist()):
                stream |= int(w) << (32 * i)
            for i, t in enumerate(slots):
                pos = (255 - t) * bits
                stream &= ~(0xFFF << pos)
                stream |= int(vals[b * len(slots) + i]) << pos
            blk[:] = [(stream >> (32 * i)) & 0xFFFFFFFF for i in range(wpb)]
    return codes, k


def windows_np(codes: np.ndarray, k: int, bits: int) -> np.ndarray:
    """All windows [N, K] by the word-shift form (vectorised, for coverage checks)."""
    n = codes.shape[0]
    wpb = 256 * bits // 32
    blocks = codes.reshape(n, k // 256, wpb).astype(np.uint64)
    t = np.arange(256)
    pos = (255 - t) * bits
    wi = pos >> 5
    off = (pos & 31).astype(np.uint64)
    nxt = np.where(wi + 1 == wpb, 0, wi + 1)
    f = blocks[:, :, wi] | (blocks[:, :, nxt] << np.uint64(32))
    return ((f >> off) & np.uint64(0xFFF)).reshape(n, k).astype(np.uint32)


def assert_prefill_close(out_bits: np.ndarray, y: np.ndarray, a: np.ndarray, what: str = ""):
    ok = oracle.within_tolerance(out_bits, y, a)
    if not ok.all():
        idx = np.argwhere(~ok)[:5]
        outf = (out_bits.astype(np.uint32) << 16).view(np.float32)
        detail = ", ".join(f"[{i},{j}] gpu={outf[i, j]!r} f64={y[i, j]!r} A={a[i, j]!r}" for i, j in idx)
        raise AssertionError(f"{what}: {int((~ok).sum())} of {ok.size} outputs out of tolerance: {detail}")
