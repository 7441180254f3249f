"""CPU checks of the arithmetic identities the device decode relies on.

The page's weight is bf16(float32(value(code) * scale)), value(code) being the
float32 reciprocal refinement of code / 147.800537109375 (web page "mlx-bun
0.2.0 -> 0.4.0" (npm diff, page 57), section src/model/trellis-wide-prefill.ts,
kernel body). Three of the device's decode paths (the ALU path, the float16
code table and the k = 2 pair table) instead form float32(code * q) in one
rounding, with q = float32(scale * r) moved to the nearest multiple of four
units in its last place (r = float32(1 / 147.800537109375)). The ALU path gets
there through fma(1.5*2^23 + code, q, -1.5*2^23 * q); the tables through a
mixed-precision fma of the float16 code and q. This file checks, for every
code in [-510, 510] and every bf16 scale of either sign with
2^-110 <= |scale| <= 2^110, that both routes give the page's bf16 weight
(zeros compared as numbers: the sign of a zero weight does not change any
product). The page's side uses the oracle's value(); nothing here runs on the
GPU.
"""
import numpy as np

import oracle

MAGIC = np.float32(1.5 * 2 ** 23)


def bf16_rne(f32: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bits, nearest even (finite inputs)."""
    u = f32.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def all_scales(lo_exp: int = -110, hi_exp: int = 110) -> np.ndarray:
    """Every bf16 scale with lo_exp <= exponent <= hi_exp, both signs (bits)."""
    exps = np.arange(127 + lo_exp, 127 + hi_exp + 1, dtype=np.uint32)
    mant = np.arange(128, dtype=np.uint32)
    pos = ((exps[:, None] << 7) | mant[None, :]).ravel()
    return np.concatenate([pos, pos | 0x8000]).astype(np.uint16)


def same_weight(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    return (a == b) | (((a & 0x7FFF) == 0) & ((b & 0x7FFF) == 0))


def routes(codes: np.ndarray, scales: np.ndarray, round_q: bool = True):
    """(page bf16, fma-route bf16) for every (code, scale) pair."""
    vals = np.array([oracle.value(int(c)) for c in codes], dtype=np.float32)
    s = (scales.astype(np.uint32) << 16).view(np.float32)
    r = np.float32(oracle.reciprocal())
    page = bf16_rne((vals[:, None] * s[None, :]).astype(np.float32))
    q = (s * r).astype(np.float32)
    if round_q:
        q = ((q.view(np.uint32) + 2) & ~np.uint32(3)).view(np.float32)
        k = (-MAGIC * q).astype(np.float32)   # exact: q has at most 22 significant bits
        assert np.array_equal(k.astype(np.float64), -1.5 * 2 ** 23 * q.astype(np.float64))
    else:
        k = (-MAGIC * q).astype(np.float32)
    f = (MAGIC + codes.astype(np.float32)).astype(np.float32)   # 1.5*2^23 + code, exact
    # fma(f, q, k): f*q is exact in float64 (48 bits) and so is f*q + k (the
    # sum spans under 53 bits); one rounding to float32 follows
    fused = (f.astype(np.float64)[:, None] * q.astype(np.float64)[None, :] + k.astype(np.float64)[None, :])
    alu = bf16_rne(fused.astype(np.float32))
    # the tables: float32(code * q) by a mixed-precision fma with addend 0
    mix = bf16_rne((codes.astype(np.float64)[:, None] * q.astype(np.float64)[None, :]).astype(np.float32))
    return page, alu, mix


def test_fma_route_equals_page_weight_exhaustively():
    codes = np.arange(-510, 511, dtype=np.int64)
    scales = all_scales()
    bad = 0
    for i in range(0, scales.size, 4096):
        page, alu, mix = routes(codes, scales[i:i + 4096])
        bad += int((~same_weight(page, alu)).sum()) + int((~same_weight(page, mix)).sum())
    assert bad == 0


def test_fma_route_needs_the_rounded_q():
    # negative control: without moving q to a multiple of four ulps the
    # constant -1.5*2^23*q is not exact and the fused route drifts
    codes = np.arange(-510, 511, dtype=np.int64)
    scales = all_scales(-8, -6)
    page, alu, _ = routes(codes, scales, round_q=False)
    assert (~same_weight(page, alu)).sum() > 1000


def test_refinement_never_changes_a_bf16_weight():
    # A fact about the page's chain, not a requirement of the device: the
    # plain float32(code * r) misses the refined value by one float32 ulp for
    # 398 codes, yet for every bf16 scale in the range above the product with
    # the scale rounds to the same bf16 weight either way. The refinement is
    # observable in the float32 value (an oracle pin checks that) but never in
    # a bf16 weight, so a decode test of bf16 weights alone cannot tell the
    # two apart; the oracle's value() is pinned at float32 level for that
    # reason.
    codes = np.arange(-510, 511, dtype=np.int64)
    r = np.float32(oracle.reciprocal())
    vals = np.array([oracle.value(int(c)) for c in codes], dtype=np.float32)
    plain_v = (codes.astype(np.float32) * r).astype(np.float32)
    sel = plain_v != vals
    assert sel.sum() == 398
    s = (all_scales().astype(np.uint32) << 16).view(np.float32)
    page = bf16_rne((vals[sel][:, None] * s[None, :]).astype(np.float32))
    plain = bf16_rne((plain_v[sel][:, None] * s[None, :]).astype(np.float32))
    assert same_weight(page, plain).all()
