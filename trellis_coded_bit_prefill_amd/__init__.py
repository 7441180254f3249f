"""Packed Trellis-quantized linear layer for narrow-batch prefill on MI355X.

Thin ctypes binding over the C ABI in ``include/trellis.h`` (library
``libtrellis.so``, hand-written HIP for gfx950). The functions here only
marshal torch tensors into device pointers, sizes and the current HIP
stream; every step of the layer runs in the library's kernels. There is no
CPU fallback: if the library is missing or fails to load, importing the
entry points raises.

Method: web page "mlx-bun 0.2.0 -> 0.4.0" (npm diff, page 57), section
src/model/trellis-wide-prefill.ts (kernel body and host wrapper).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libtrellis.so")

T_BLOCK = 256
L_WINDOW = 12
MIN_M = 5
MAX_M = 15
MATVEC_MAX_M = 4
MAX_GROUPS = 4096
MAX_GROUP_ROWS = 1 << 20

OK = 0
E_GEOMETRY = -1
E_M = -2
E_NULL = -3
E_ALIGN = -4
E_HIP = -5
E_SCRATCH = -6
NOALLOC_SCRATCH_BYTES = 32 << 20

# Every symbol declared in include/trellis.h.
EXPORTED = ("trellis_supported", "trellis_decode", "trellis_prefill", "trellis_matvec", "trellis_prefill_packed",
            "trellis_gate_up", "trellis_prefill_noalloc", "trellis_status_string")
# Test and tuning hooks (include/trellis_testing.h).
EXPORTED_TESTING = ("trellis_test_force_table",)
TABLES = {"value": 0, "code": 1, "pair": 2}


class Geom(ctypes.Structure):
    """trellis_geom: n output rows, k input columns, block t, window l, bits."""

    _fields_ = [("n", ctypes.c_int32), ("k", ctypes.c_int32), ("t", ctypes.c_int32),
                ("l", ctypes.c_int32), ("bits", ctypes.c_int32)]


def geom(n: int, k: int, bits: int, t: int = T_BLOCK, l: int = L_WINDOW) -> Geom:
    return Geom(n, k, t, l, bits)


class TrellisError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"trellis status {status}: {msg}")
        self.status = status


class TrellisValueError(TrellisError, ValueError):
    pass


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libtrellis.so (raises OSError if it is not built).

    torch is imported first. PyTorch-ROCm ships its own HIP runtime and
    links it by the plain name libamdhip64.so, while this library links the
    runtime by its versioned name. Loaded first, the library would pull the
    system runtime in, and torch would then load its own copy: two HIP
    runtimes in one process, where the library finds no device and torch's
    stream handles mean nothing to it. With torch loaded first, the library
    binds to torch's runtime.
    """
    global _lib
    if _lib is not None:
        return _lib
    import torch  # noqa: F401  (see the docstring)

    if not os.path.exists(path):
        raise OSError(f"{path} is not built; run trellis_coded_bit_prefill_amd/_build.py")
    L = ctypes.CDLL(path)
    vp = ctypes.c_void_p
    L.trellis_supported.argtypes = [Geom, ctypes.c_int32]
    L.trellis_supported.restype = ctypes.c_int
    L.trellis_status_string.argtypes = [ctypes.c_int]
    L.trellis_status_string.restype = ctypes.c_char_p
    L.trellis_decode.argtypes = [vp, vp, Geom, vp, vp]
    L.trellis_decode.restype = ctypes.c_int
    L.trellis_prefill.argtypes = [vp, ctypes.c_int32, vp, vp, Geom, vp, vp]
    L.trellis_prefill.restype = ctypes.c_int
    L.trellis_matvec.argtypes = [vp, ctypes.c_int32, vp, vp, Geom, vp, vp]
    L.trellis_matvec.restype = ctypes.c_int
    L.trellis_prefill_packed.argtypes = [vp, vp, ctypes.c_int32, vp, vp, Geom, vp, vp]
    L.trellis_prefill_packed.restype = ctypes.c_int
    L.trellis_gate_up.argtypes = [vp, ctypes.c_int32, vp, vp, vp, vp, Geom, vp, vp]
    L.trellis_gate_up.restype = ctypes.c_int
    L.trellis_prefill_noalloc.argtypes = [vp, ctypes.c_int32, vp, vp, Geom, vp, vp]
    L.trellis_prefill_noalloc.restype = ctypes.c_int
    L.trellis_test_force_table.argtypes = [ctypes.c_int]
    L.trellis_test_force_table.restype = ctypes.c_int
    _lib = L
    return L


def force_table(name):
    """Test hook: force the decode table of later calls ("value", "code",
    "pair" (k = 2 only) or None for the library's choice). Returns the
    previous setting's name."""
    kind = -1 if name is None else TABLES[name]
    prev = load_library().trellis_test_force_table(kind)
    if prev < -1:
        raise ValueError(f"bad table {name!r}")
    return None if prev == -1 else {v: k for k, v in TABLES.items()}[prev]


def status_string(status: int) -> str:
    return load_library().trellis_status_string(status).decode()


def supported(g: Geom, m: int) -> bool:
    return bool(load_library().trellis_supported(g, m))


def _raise(status: int):
    if status == OK:
        return
    msg = status_string(status)
    if status == E_HIP:
        raise TrellisError(status, msg)
    raise TrellisValueError(status, msg)


def _stream_handle(device) -> int:
    """The current stream of `device`, which must be the current device (the
    library works on the current device)."""
    import torch

    if device.index is not None and device.index != torch.cuda.current_device():
        raise ValueError(f"tensors are on {device} but the current device is cuda:{torch.cuda.current_device()}")
    return torch.cuda.current_stream(device).cuda_stream


def _check_tensor(name, t, dtypes, ndim, device=None):
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} dtype {t.dtype} not in {dtypes}")
    if t.ndim != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _dtypes():
    import torch

    return ((torch.bfloat16, torch.int16, torch.uint16),  # bf16 bit patterns
            (torch.int32, torch.uint32))                  # code words


def decode_raw(codes_ptr: int, scales_ptr: int, g: Geom, w_ptr: int, stream: int) -> None:
    """Direct C-ABI call with raw device addresses."""
    _raise(load_library().trellis_decode(codes_ptr, scales_ptr, g, w_ptr, stream))


def prefill_raw(x_ptr: int, m: int, codes_ptr: int, scales_ptr: int, g: Geom, out_ptr: int,
                stream: int) -> None:
    """Direct C-ABI call with raw device addresses."""
    _raise(load_library().trellis_prefill(x_ptr, m, codes_ptr, scales_ptr, g, out_ptr, stream))


def prefill_noalloc_raw(x_ptr: int, m: int, codes_ptr: int, scales_ptr: int, g: Geom, out_ptr: int,
                        stream: int) -> None:
    """Direct C-ABI call of the no-allocation variant (fixed device scratch)."""
    _raise(load_library().trellis_prefill_noalloc(x_ptr, m, codes_ptr, scales_ptr, g, out_ptr, stream))


def matvec_raw(x_ptr: int, m: int, codes_ptr: int, scales_ptr: int, g: Geom, out_ptr: int,
               stream: int) -> None:
    """Direct C-ABI call with raw device addresses (1 <= m <= 4)."""
    _raise(load_library().trellis_matvec(x_ptr, m, codes_ptr, scales_ptr, g, out_ptr, stream))


def prefill_packed_raw(x_ptrs, rows, codes_ptr: int, scales_ptr: int, g: Geom, out_ptrs, stream: int) -> None:
    """Direct C-ABI call: x_ptrs, rows and out_ptrs are equal-length
    sequences of raw device addresses and row counts, one per group."""
    groups = len(rows)
    if len(x_ptrs) != groups or len(out_ptrs) != groups:
        raise ValueError("x_ptrs, rows and out_ptrs must have one entry per group")
    xa = (ctypes.c_void_p * max(groups, 1))(*x_ptrs)
    ra = (ctypes.c_int32 * max(groups, 1))(*rows)
    oa = (ctypes.c_void_p * max(groups, 1))(*out_ptrs)
    _raise(load_library().trellis_prefill_packed(xa, ra, groups, codes_ptr, scales_ptr, g, oa, stream))


def gate_up_raw(x_ptr: int, m: int, codes_gate_ptr: int, scales_gate_ptr: int, codes_up_ptr: int,
                scales_up_ptr: int, g: Geom, h_ptr: int, stream: int) -> None:
    """Direct C-ABI call with raw device addresses (1 <= m <= 15)."""
    _raise(load_library().trellis_gate_up(x_ptr, m, codes_gate_ptr, scales_gate_ptr, codes_up_ptr,
                                          scales_up_ptr, g, h_ptr, stream))


@dataclass
class Layer:
    """A packed Trellis linear layer: codes [N, K*bits/32] and scales [N]."""

    codes: "object"
    scales: "object"
    n: int
    k: int
    bits: int

    @property
    def geom(self) -> Geom:
        return geom(self.n, self.k, self.bits)


def decode(codes, scales, k: int, bits: int, out=None):
    """Materialise W[N, K] (bf16) from packed codes on the current stream."""
    import torch

    bf, cw = _dtypes()
    _check_tensor("codes", codes, cw, 2)
    _check_tensor("scales", scales, bf, 1, codes.device)
    n = codes.shape[0]
    if codes.shape[1] * 32 != k * bits:
        raise ValueError(f"codes has {codes.shape[1]} words per row, expected K*bits/32 = {k * bits // 32}")
    if scales.shape[0] != n:
        raise ValueError("scales must have one entry per row")
    if out is None:
        out = torch.empty((n, k), dtype=torch.bfloat16, device=codes.device)
    _check_tensor("out", out, bf, 2, codes.device)
    if tuple(out.shape) != (n, k):
        raise ValueError("out must be [N, K]")
    decode_raw(codes.data_ptr(), scales.data_ptr(), geom(n, k, bits), out.data_ptr(),
               _stream_handle(codes.device))
    return out


def prefill(x, codes, scales, bits: int, out=None):
    """out[M, N] = x[M, K] . W^T (bf16), W decoded on the fly, current stream
    (5 <= M <= 15)."""
    return _linear(prefill_raw, x, codes, scales, bits, out)


def prefill_noalloc(x, codes, scales, bits: int, out):
    """prefill() without any device allocation by the library: `out` must be
    given, and the workspace is the library's fixed per-GPU scratch (calls on
    one GPU must not overlap)."""
    return _linear(prefill_noalloc_raw, x, codes, scales, bits, out)


def matvec(x, codes, scales, bits: int, out=None):
    """The same layer for 1 <= M <= 4 rows (decode tokens)."""
    return _linear(matvec_raw, x, codes, scales, bits, out)


def _linear(entry, x, codes, scales, bits: int, out=None):
    import torch

    bf, cw = _dtypes()
    _check_tensor("x", x, bf, 2)
    _check_tensor("codes", codes, cw, 2, x.device)
    _check_tensor("scales", scales, bf, 1, x.device)
    m, k = x.shape
    n = codes.shape[0]
    if codes.shape[1] * 32 != k * bits:
        raise ValueError(f"codes has {codes.shape[1]} words per row, expected K*bits/32 = {k * bits // 32}")
    if scales.shape[0] != n:
        raise ValueError("scales must have one entry per row")
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=x.device)
    _check_tensor("out", out, bf, 2, x.device)
    if tuple(out.shape) != (m, n):
        raise ValueError("out must be [M, N]")
    entry(x.data_ptr(), m, codes.data_ptr(), scales.data_ptr(), geom(n, k, bits), out.data_ptr(),
          _stream_handle(x.device))
    return out


def prefill_packed(xs, codes, scales, bits: int, outs=None):
    """Token packing: one pass of the layer over the rows of every x in xs
    (each [rows_i, K], any rows_i >= 0), outputs cut back per input
    ([rows_i, N] each). Rows are processed in launches of at most 15."""
    import torch

    bf, cw = _dtypes()
    if len(xs) == 0:
        raise ValueError("xs must hold at least one input")
    _check_tensor("codes", codes, cw, 2)
    _check_tensor("scales", scales, bf, 1, codes.device)
    n = codes.shape[0]
    if scales.shape[0] != n:
        raise ValueError("scales must have one entry per row")
    k = None
    for i, x in enumerate(xs):
        _check_tensor(f"xs[{i}]", x, bf, 2, codes.device)
        if k is None:
            k = x.shape[1]
        elif x.shape[1] != k:
            raise ValueError("every input must have the same K")
    if codes.shape[1] * 32 != k * bits:
        raise ValueError(f"codes has {codes.shape[1]} words per row, expected K*bits/32 = {k * bits // 32}")
    if outs is None:
        outs = [torch.empty((x.shape[0], n), dtype=torch.bfloat16, device=codes.device) for x in xs]
    if len(outs) != len(xs):
        raise ValueError("outs must have one tensor per input")
    for i, (x, o) in enumerate(zip(xs, outs)):
        _check_tensor(f"outs[{i}]", o, bf, 2, codes.device)
        if tuple(o.shape) != (x.shape[0], n):
            raise ValueError(f"outs[{i}] must be [{x.shape[0]}, {n}]")
    prefill_packed_raw([x.data_ptr() if x.shape[0] else 0 for x in xs], [x.shape[0] for x in xs],
                       codes.data_ptr(), scales.data_ptr(), geom(n, k, bits),
                       [o.data_ptr() if o.shape[0] else 0 for o in outs], _stream_handle(codes.device))
    return outs


def gate_up(x, codes_gate, scales_gate, codes_up, scales_up, bits: int, out=None):
    """h[M, N] = silu(x . Wg^T) * (x . Wu^T) with the page's bf16 roundings,
    both weight matrices decoded on the fly in one pass (1 <= M <= 15)."""
    import torch

    bf, cw = _dtypes()
    _check_tensor("x", x, bf, 2)
    for name, c, sc in (("gate", codes_gate, scales_gate), ("up", codes_up, scales_up)):
        _check_tensor(f"codes_{name}", c, cw, 2, x.device)
        _check_tensor(f"scales_{name}", sc, bf, 1, x.device)
    m, k = x.shape
    n = codes_gate.shape[0]
    if tuple(codes_up.shape) != tuple(codes_gate.shape):
        raise ValueError("gate and up codes must have the same shape")
    if codes_gate.shape[1] * 32 != k * bits:
        raise ValueError(f"codes have {codes_gate.shape[1]} words per row, expected K*bits/32 = {k * bits // 32}")
    if scales_gate.shape[0] != n or scales_up.shape[0] != n:
        raise ValueError("scales must have one entry per row")
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=x.device)
    _check_tensor("out", out, bf, 2, x.device)
    if tuple(out.shape) != (m, n):
        raise ValueError("out must be [M, N]")
    gate_up_raw(x.data_ptr(), m, codes_gate.data_ptr(), scales_gate.data_ptr(), codes_up.data_ptr(),
                scales_up.data_ptr(), geom(n, k, bits), out.data_ptr(), _stream_handle(x.device))
    return out
