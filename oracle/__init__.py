"""CPU oracle for the packed Trellis-quantized linear layer.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers. The product path (the HIP library and
its Python binding) never imports this package, and this package imports
nothing from the product path.

The arithmetic lives in ``trellis_oracle.c`` (plain C, strict IEEE binary32
with ``-ffp-contract=off``; float64 for the contraction). This module loads
it with ctypes and wraps it for NumPy arrays. Source of the method: the web
page "mlx-bun 0.2.0 -> 0.4.0" (npm diff, page 57), section
``src/model/trellis-wide-prefill.ts``, Metal kernel body and host wrapper.

Pins: every function here is checked in ``tests/test_oracle_pins.py``
against facts that do not come from this code (exhaustive enumeration, exact
rational arithmetic, closed forms, a second bit-level formulation, torch's
bf16 cast, brute force). No function is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "trellis_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
GCC_FLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
             "-fno-builtin", "-shared", "-fPIC"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (strict IEEE flags). Returns the .so path."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *GCC_FLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        u32p = ctypes.POINTER(ctypes.c_uint32)
        u16p = ctypes.POINTER(ctypes.c_uint16)
        f64p = ctypes.POINTER(ctypes.c_double)
        c_int = ctypes.c_int
        L.oracle_window.argtypes = [u32p, c_int, c_int]
        L.oracle_window.restype = ctypes.c_uint32
        L.oracle_code.argtypes = [ctypes.c_uint32]
        L.oracle_code.restype = ctypes.c_int32
        L.oracle_value.argtypes = [ctypes.c_int32]
        L.oracle_value.restype = ctypes.c_float
        L.oracle_reciprocal.argtypes = []
        L.oracle_reciprocal.restype = ctypes.c_float
        L.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
        L.oracle_f32_to_bf16.restype = ctypes.c_uint16
        L.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_f32.restype = ctypes.c_float
        L.oracle_weight.argtypes = [ctypes.c_uint32, ctypes.c_uint16]
        L.oracle_weight.restype = ctypes.c_uint16
        L.oracle_decode_rows.argtypes = [u32p, u16p, c_int, c_int, c_int, c_int, u16p]
        L.oracle_decode_rows.restype = None
        L.oracle_prefill_rows.argtypes = [u16p, c_int, u32p, u16p, c_int, c_int, c_int,
                                          c_int, f64p, f64p]
        L.oracle_prefill_rows.restype = None
        L.oracle_contract.argtypes = [u16p, c_int, u16p, c_int, c_int, f64p, f64p]
        L.oracle_contract.restype = None
        L.oracle_f64_to_bf16.argtypes = [ctypes.c_double]
        L.oracle_f64_to_bf16.restype = ctypes.c_uint16
        L.oracle_gate_up_chain.argtypes = [ctypes.c_uint16, ctypes.c_uint16, ctypes.POINTER(c_int)]
        L.oracle_gate_up_chain.restype = ctypes.c_uint16
        L.oracle_gate_up_chain_n.argtypes = [u16p, u16p, ctypes.c_long, u16p, ctypes.POINTER(ctypes.c_uint8)]
        L.oracle_gate_up_chain_n.restype = None
        _lib = L
    return _lib


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


# ---- scalar steps ---------------------------------------------------------

def window(block: np.ndarray, bits: int, t: int) -> int:
    """12-bit window of weight t in one block (array of 256*bits/32 uint32)."""
    b = np.ascontiguousarray(block, dtype=np.uint32)
    assert b.size == 256 * bits // 32
    return int(lib().oracle_window(_ptr(b, ctypes.c_uint32), bits, t))


def code(win: int) -> int:
    return int(lib().oracle_code(win))


def value(c: int) -> float:
    """float32 value of an integer code (returned as a Python float)."""
    return float(lib().oracle_value(c))


def value_bits(c: int) -> int:
    return int(np.array([value(c)], dtype=np.float32).view(np.uint32)[0])


def reciprocal() -> float:
    return float(lib().oracle_reciprocal())


def f32_to_bf16(f: float) -> int:
    return int(lib().oracle_f32_to_bf16(f))


def bf16_to_f32(h: int) -> float:
    return float(lib().oracle_bf16_to_f32(h))


def weight(win: int, scale_bf16: int) -> int:
    return int(lib().oracle_weight(win, scale_bf16))


# ---- array entry points ---------------------------------------------------

def _check(codes, scales, k, bits):
    codes = np.ascontiguousarray(codes, dtype=np.uint32)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    assert k % 256 == 0 and bits in (2, 3, 4)
    assert codes.ndim == 2 and codes.shape[1] == k * bits // 32
    assert scales.shape == (codes.shape[0],)
    return codes, scales


def decode_rows(codes, scales, k: int, bits: int, row0: int = 0, nrows: int | None = None):
    """bf16 bit patterns of W[row0:row0+nrows, :K] (uint16 [nrows, K])."""
    codes, scales = _check(codes, scales, k, bits)
    n = codes.shape[0]
    nrows = n - row0 if nrows is None else nrows
    assert 0 <= row0 and row0 + nrows <= n
    w = np.empty((nrows, k), dtype=np.uint16)
    lib().oracle_decode_rows(_ptr(codes, ctypes.c_uint32), _ptr(scales, ctypes.c_uint16),
                             k, bits, row0, nrows, _ptr(w, ctypes.c_uint16))
    return w


def decode(codes, scales, k: int, bits: int):
    return decode_rows(codes, scales, k, bits)


def prefill_rows(x, codes, scales, k: int, bits: int, rows):
    """float64 y[M, len(rows)] and a[M, len(rows)] = sum |w*x| for the listed rows.

    rows is an iterable of output-row indices; consecutive runs are handed to
    the C oracle in one call.
    """
    codes, scales = _check(codes, scales, k, bits)
    x = np.ascontiguousarray(x, dtype=np.uint16)
    m = x.shape[0]
    assert x.shape == (m, k)
    rows = np.asarray(list(rows), dtype=np.int64)
    y = np.empty((m, rows.size), dtype=np.float64)
    a = np.empty((m, rows.size), dtype=np.float64)
    i = 0
    while i < rows.size:
        j = i + 1
        while j < rows.size and rows[j] == rows[j - 1] + 1:
            j += 1
        cnt = j - i
        yy = np.empty((m, cnt), dtype=np.float64)
        aa = np.empty((m, cnt), dtype=np.float64)
        lib().oracle_prefill_rows(_ptr(x, ctypes.c_uint16), m, _ptr(codes, ctypes.c_uint32),
                                  _ptr(scales, ctypes.c_uint16), k, bits, int(rows[i]), cnt,
                                  _ptr(yy, ctypes.c_double), _ptr(aa, ctypes.c_double))
        y[:, i:j] = yy
        a[:, i:j] = aa
        i = j
    return y, a


def prefill(x, codes, scales, k: int, bits: int):
    n = np.asarray(codes).shape[0]
    return prefill_rows(x, codes, scales, k, bits, range(n))


# ---- host-parallel drivers ---------------------------------------------------
# The C functions run with the GIL released (ctypes), so contiguous row
# ranges can go to a thread pool. Each thread computes whole output rows with
# the same C code as above; the arithmetic per row is unchanged.

def default_threads() -> int:
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except (AttributeError, OSError):
        return max(1, min(16, os.cpu_count() or 1))


def _row_chunks(n: int, threads: int):
    threads = max(1, min(threads, n))
    step = -(-n // threads)
    return [(r, min(n, r + step)) for r in range(0, n, step)]


def decode_parallel(codes, scales, k: int, bits: int, threads: int | None = None):
    """decode() with rows split over `threads` host threads."""
    from concurrent.futures import ThreadPoolExecutor

    codes, scales = _check(codes, scales, k, bits)
    n = codes.shape[0]
    w = np.empty((n, k), dtype=np.uint16)
    chunks = _row_chunks(n, threads or default_threads())

    def run(c):
        r0, r1 = c
        lib().oracle_decode_rows(_ptr(codes, ctypes.c_uint32), _ptr(scales, ctypes.c_uint16), k, bits, r0,
                                 r1 - r0, _ptr(w[r0:r1], ctypes.c_uint16))

    with ThreadPoolExecutor(len(chunks)) as ex:
        list(ex.map(run, chunks))
    return w


def prefill_parallel(x, codes, scales, k: int, bits: int, threads: int | None = None):
    """prefill() (float64 y and sum |w*x| for every output row) with rows split
    over `threads` host threads."""
    from concurrent.futures import ThreadPoolExecutor

    codes, scales = _check(codes, scales, k, bits)
    n = codes.shape[0]
    chunks = _row_chunks(n, threads or default_threads())
    parts = [None] * len(chunks)

    def run(i):
        r0, r1 = chunks[i]
        parts[i] = prefill_rows(x, codes, scales, k, bits, range(r0, r1))

    with ThreadPoolExecutor(len(chunks)) as ex:
        list(ex.map(run, range(len(chunks))))
    return np.concatenate([p[0] for p in parts], axis=1), np.concatenate([p[1] for p in parts], axis=1)


def contract(x, w):
    """float64 y[M, N], a[M, N] from bf16 x[M, K] and an already decoded W[N, K]."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    w = np.ascontiguousarray(w, dtype=np.uint16)
    m, k = x.shape
    n = w.shape[0]
    assert w.shape == (n, k)
    y = np.empty((m, n), dtype=np.float64)
    a = np.empty((m, n), dtype=np.float64)
    lib().oracle_contract(_ptr(x, ctypes.c_uint16), m, _ptr(w, ctypes.c_uint16), k, n,
                          _ptr(y, ctypes.c_double), _ptr(a, ctypes.c_double))
    return y, a


# ---- acceptance bound -----------------------------------------------------

def ulp_bf16(v: np.ndarray) -> np.ndarray:
    """Unit in the last place of bf16 values v (float array of bf16 values).

    2^(floor(log2|v|) - 7) for normal v; 2^-133 (the bf16 subnormal step)
    for zero and subnormal v.
    """
    v = np.abs(np.asarray(v, dtype=np.float64))
    out = np.full(v.shape, 2.0 ** -133)
    nz = v >= 2.0 ** -126
    out[nz] = np.ldexp(1.0, (np.floor(np.log2(v[nz])) - 7).astype(np.int64))
    return out


def within_tolerance(out_bf16_bits: np.ndarray, y: np.ndarray, a: np.ndarray, rel: float = 1e-5):
    """Boolean mask: |out - y| <= ulp_bf16(out) + rel * a (elementwise)."""
    out = (np.asarray(out_bf16_bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
    out = out.astype(np.float64)
    return np.abs(out - y) <= ulp_bf16(out) + rel * a


# ---- gate/up tail of an MLP ------------------------------------------------
# Page "mlx-bun 0.0.4" (npm, page 62), section src/model/minicpm5.ts, MLP
# forward: gate and up projections of the same x, then
# hidden = (gate * sigmoid(gate)) * up.

def silu(g):
    """g * sigmoid(g) = g / (1 + exp(-g)) in float64."""
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def f64_to_bf16(v: float) -> int:
    """bf16 bits of a float64 rounded to nearest even in one step."""
    return int(lib().oracle_f64_to_bf16(float(v)))


def gate_up_chain(gate_bf16, up_bf16):
    """The page's bf16 chain on bf16 gate and up arrays (bit patterns):
    h = bf16(bf16(gate * bf16(sigmoid(gate))) * up), each step exact and
    rounded once. Returns (h bits, ambiguous), where ambiguous marks elements
    whose exact sigmoid lies within 2^-21 (relative) of a bf16 rounding
    boundary, so that a float32 sigmoid may legitimately round either way."""
    g = np.ascontiguousarray(gate_bf16, dtype=np.uint16)
    u = np.ascontiguousarray(up_bf16, dtype=np.uint16)
    assert g.shape == u.shape
    h = np.empty(g.shape, dtype=np.uint16)
    amb = np.empty(g.shape, dtype=np.uint8)
    lib().oracle_gate_up_chain_n(_ptr(g, ctypes.c_uint16), _ptr(u, ctypes.c_uint16), g.size,
                                 _ptr(h, ctypes.c_uint16), _ptr(amb, ctypes.c_uint8))
    return h, amb.astype(bool)


def gate_up_rows(x, codes_g, scales_g, codes_u, scales_u, k: int, bits: int, rows):
    """Float64 reference of the fused gate/up tail for output columns `rows`.

    Returns (h, g, ag, u, au): g and u are the float64 sums of the same bf16
    products (prefill_rows), ag and au their sums of |w*x|, and
    h = silu(g) * u with no intermediate rounding.
    """
    g, ag = prefill_rows(x, codes_g, scales_g, k, bits, rows)
    u, au = prefill_rows(x, codes_u, scales_u, k, bits, rows)
    return silu(g) * u, g, ag, u, au


def gate_up_within_tolerance(h_bf16_bits, h, g, ag, u, au, rel: float = 1e-5):
    """Boolean mask: the device's h is within the bound the page's bf16 chain
    allows around the exact h = silu(g) * u.

    The device rounds gate and up to bf16 after float32 accumulation, each
    within Eg = 2 ulp_bf16(g) + rel*ag of g (resp. Eu of u), then rounds
    sigmoid(gate), gate*sigmoid(gate) and that times up to bf16. With
    |silu'| <= 1.1, S = |silu(g)| + 1.1 Eg and V = |u| + Eu bound the rounded
    operands, so
      |h_dev - h| <= (1.1 Eg + 2^-7 S) V + |silu(g)| Eu + 2^-8 S V + 2^-133,
    where 2^-7 S covers the two roundings inside silu and 2^-8 S V the last
    one (each at most half an ulp, i.e. 2^-9 relative, doubled for margin).
    """
    hd = (np.asarray(h_bf16_bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    eg = 2 * ulp_bf16(g) + rel * ag
    eu = 2 * ulp_bf16(u) + rel * au
    sg = np.abs(silu(g))
    s = sg + 1.1 * eg
    v = np.abs(u) + eu
    bound = (1.1 * eg + 2.0 ** -7 * s) * v + sg * eu + 2.0 ** -8 * s * v + 2.0 ** -133
    return np.abs(hd - h) <= bound
