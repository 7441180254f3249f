"""Seeded synthetic inputs for the packed Trellis linear layer.

This module only draws and shapes inputs; it holds none of the layer's own
arithmetic (no window extraction, hash, normalisation or contraction). Both
the CPU oracle and the HIP path consume exactly the arrays produced here.

Shapes and distributions follow the narrow-batch prefill regime of the
Trellis wide-prefill kernel on the web page "mlx-bun 0.2.0 -> 0.4.0" (npm
diff, page 57), section ``src/model/trellis-wide-prefill.ts``: bf16
activations ``x[M, K]`` with 5 <= M <= 15, a row-major uint32 code stream
``codes[N, K*k/32]`` of k-bit codes, and one scale per output row.

Recipe (NumPy ``Generator(PCG64(seed))``, drawn in the order x, codes, scales):

* x: standard normal float32 rows, RMS-normalised with unit weight and
  eps = 1e-6 (the caller's RMSNorm output), then rounded to bf16 (RNE).
  For the down-projection shape x = bf16(silu(g) * u) with g, u standard
  normal float32, silu(g) = g * sigmoid(g) evaluated in float32.
* codes: uniform uint32 words (every bit pattern is a valid stream).
* scales: uniform float32 in [0.005, 0.02], rounded to bf16 (RNE).

bf16 values are carried as uint16 bit patterns.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

T_BLOCK = 256   # weights per code block
L_WINDOW = 12   # bits per decode window


@dataclass(frozen=True)
class Shape:
    name: str
    m: int
    k: int
    n: int
    bits: int
    seed: int
    x_kind: str = "rmsnorm"   # "rmsnorm" or "silu_mul"
    matrices: int = 1         # 2: gate and up projections of the same x
    groups: tuple = ()        # token packing: row counts of the packed inputs (sum = m)

    @property
    def words_per_row(self) -> int:
        return self.k * self.bits // 32

    @property
    def weights(self) -> int:
        return self.matrices * self.n * self.k

    @property
    def algorithmic_bytes(self) -> int:
        """Packed code bytes (every matrix) + bf16 x + bf16 out (scales excluded)."""
        return self.matrices * self.n * self.k * self.bits // 8 + 2 * self.m * self.k + 2 * self.m * self.n


# The five workloads: a tiny shape, the wide K=5120 x N=17408 shape at three
# (M, k) points, and the down projection K=17408 x N=5120.
SHAPES = {
    "tiny": Shape("tiny", 5, 512, 256, 2, 1),
    "wide_m5_k4": Shape("wide_m5_k4", 5, 5120, 17408, 4, 2),
    "wide_m8_k3": Shape("wide_m8_k3", 8, 5120, 17408, 3, 3),
    "wide_m15_k2": Shape("wide_m15_k2", 15, 5120, 17408, 2, 4),
    "down_m15_k4": Shape("down_m15_k4", 15, 17408, 5120, 4, 5, "silu_mul"),
    # small-batch (matvec) regime, M = 1..4, on the wide geometry
    "matvec_m1_k4": Shape("matvec_m1_k4", 1, 5120, 17408, 4, 6),
    "matvec_m4_k2": Shape("matvec_m4_k2", 4, 5120, 17408, 2, 7),
    # fused gate + up projections of one x (two code streams of this geometry)
    "gateup_m5_k4": Shape("gateup_m5_k4", 5, 5120, 17408, 4, 8, "rmsnorm", 2),
    # token packing: three inputs of 5 rows each through one launch
    "packed_3x5_k4": Shape("packed_3x5_k4", 15, 5120, 17408, 4, 9, "rmsnorm", 1, (5, 5, 5)),
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round to nearest even) via torch's CPU cast."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def make_x(rng: np.random.Generator, m: int, k: int, kind: str = "rmsnorm") -> np.ndarray:
    if kind == "rmsnorm":
        g = rng.standard_normal((m, k), dtype=np.float32)
        ms = np.mean(g * g, axis=1, keepdims=True, dtype=np.float32)
        x = g / np.sqrt(ms + np.float32(1e-6), dtype=np.float32)
    elif kind == "silu_mul":
        g = rng.standard_normal((m, k), dtype=np.float32)
        u = rng.standard_normal((m, k), dtype=np.float32)
        sig = np.float32(1.0) / (np.float32(1.0) + np.exp(-g, dtype=np.float32))
        x = (g * sig) * u
    else:
        raise ValueError(kind)
    return f32_to_bf16_bits(x.astype(np.float32))


def make_codes(rng: np.random.Generator, n: int, k: int, bits: int) -> np.ndarray:
    return rng.integers(0, 2**32, size=(n, k * bits // 32), dtype=np.uint32)


def make_scales(rng: np.random.Generator, n: int) -> np.ndarray:
    s = rng.uniform(0.005, 0.02, size=n).astype(np.float32)
    return f32_to_bf16_bits(s)


def generate(m: int, k: int, n: int, bits: int, seed: int, x_kind: str = "rmsnorm"):
    """Return (x_bf16[M,K] uint16, codes[N,K*bits/32] uint32, scales_bf16[N] uint16)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = make_x(rng, m, k, x_kind)
    codes = make_codes(rng, n, k, bits)
    scales = make_scales(rng, n)
    return x, codes, scales


def generate_shape(shape: Shape, m: int | None = None):
    return generate(shape.m if m is None else m, shape.k, shape.n, shape.bits, shape.seed, shape.x_kind)


def generate_gate_up(shape: Shape):
    """x and the gate matrix as generate_shape(shape); the up matrix's codes
    and scales drawn the same way from seed + 1000.
    Returns (x, codes_gate, scales_gate, codes_up, scales_up)."""
    x, cg, sg = generate_shape(shape)
    _, cu, su = generate(shape.m, shape.k, shape.n, shape.bits, shape.seed + 1000, shape.x_kind)
    return x, cg, sg, cu, su
