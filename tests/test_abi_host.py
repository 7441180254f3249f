"""Host-side checks of the C ABI: the library loads, exports every declared
symbol, and rejects every out-of-domain call before touching the GPU."""
import os
import re

import pytest

import trellis_coded_bit_prefill_amd as tp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    """Every function declared in include/*.h."""
    import glob

    names = set()
    for path in sorted(glob.glob(os.path.join(ROOT, "include", "*.h"))):
        src = re.sub(r"/\*.*?\*/", "", open(path).read(), flags=re.S)
        names |= set(re.findall(r"\b(trellis_[a-z_]+)\s*\(", src))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(tp.LIB_PATH):
        from trellis_coded_bit_prefill_amd import _build

        _build.build()
    return tp.load_library()


def test_header_declares_the_bound_functions():
    assert declared_functions() == sorted(tp.EXPORTED + tp.EXPORTED_TESTING)


def test_table_hook_round_trips(lib):
    assert tp.force_table("code") is None
    assert tp.force_table("pair") == "code"
    assert tp.force_table(None) == "pair"
    assert lib.trellis_test_force_table(7) == -2
    assert lib.trellis_test_force_table(-3) == -2
    assert tp.force_table(None) is None


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for s in (tp.OK, tp.E_GEOMETRY, tp.E_M, tp.E_NULL, tp.E_ALIGN, tp.E_HIP, tp.E_SCRATCH):
        assert tp.status_string(s)
    assert tp.status_string(123) == "unknown status"


GOOD = dict(n=17408, k=5120, bits=4)


@pytest.mark.parametrize("n,k,bits,t,l,m,ok", [
    (17408, 5120, 4, 256, 12, 5, True),
    (17408, 5120, 3, 256, 12, 8, True),
    (17408, 5120, 2, 256, 12, 15, True),
    (5120, 17408, 4, 256, 12, 15, True),
    (256, 512, 2, 256, 12, 5, True),
    (4, 256, 2, 256, 12, 5, True),
    (17408, 5120, 4, 256, 12, 4, False),   # m below the narrow-batch range
    (17408, 5120, 4, 256, 12, 16, False),  # m above
    (17408, 5120, 1, 256, 12, 5, False),   # bits
    (17408, 5120, 5, 256, 12, 5, False),
    (17408, 5120, 8, 256, 12, 5, False),
    (17408, 5120, 4, 128, 12, 5, False),   # block length
    (17408, 5120, 4, 256, 16, 5, False),   # window length
    (17408, 5000, 4, 256, 12, 5, False),   # K not a multiple of 256
    (17408, 0, 4, 256, 12, 5, False),
    (17406, 5120, 4, 256, 12, 5, False),   # N not a multiple of 4
    (0, 5120, 4, 256, 12, 5, False),
    (-4, 5120, 4, 256, 12, 5, False),
    (17408, (1 << 18) + 256, 4, 256, 12, 5, False),
    ((1 << 22) + 4, 256, 4, 256, 12, 5, False),
])
def test_supported_truth_table(lib, n, k, bits, t, l, m, ok):
    assert tp.supported(tp.geom(n, k, bits, t, l), m) is ok


FAKE = 1 << 20  # a 16-byte aligned, never dereferenced address


def call_prefill(x=FAKE, m=5, codes=FAKE, scales=FAKE, g=None, out=FAKE):
    g = g or tp.geom(**GOOD)
    return tp.load_library().trellis_prefill(x, m, codes, scales, g, out, None)


def call_decode(codes=FAKE, scales=FAKE, g=None, w=FAKE):
    g = g or tp.geom(**GOOD)
    return tp.load_library().trellis_decode(codes, scales, g, w, None)


def test_prefill_rejects_before_launch(lib):
    assert call_prefill(g=tp.geom(17408, 5000, 4)) == tp.E_GEOMETRY
    assert call_prefill(g=tp.geom(17408, 5120, 5)) == tp.E_GEOMETRY
    assert call_prefill(m=4) == tp.E_M
    assert call_prefill(m=16) == tp.E_M
    assert call_prefill(x=None) == tp.E_NULL
    assert call_prefill(codes=None) == tp.E_NULL
    assert call_prefill(scales=None) == tp.E_NULL
    assert call_prefill(out=None) == tp.E_NULL
    assert call_prefill(x=FAKE + 2) == tp.E_ALIGN
    assert call_prefill(codes=FAKE + 4) == tp.E_ALIGN
    assert call_prefill(out=FAKE + 8) == tp.E_ALIGN
    assert call_prefill(scales=FAKE + 1) == tp.E_ALIGN
    # geometry is checked first, then m, then pointers
    assert call_prefill(g=tp.geom(17408, 5000, 4), m=4, x=None) == tp.E_GEOMETRY
    assert call_prefill(m=4, x=None) == tp.E_M


def test_decode_rejects_before_launch(lib):
    assert call_decode(g=tp.geom(17408, 5120, 4, 128)) == tp.E_GEOMETRY
    assert call_decode(g=tp.geom(17406, 5120, 4)) == tp.E_GEOMETRY
    assert call_decode(codes=None) == tp.E_NULL
    assert call_decode(scales=None) == tp.E_NULL
    assert call_decode(w=None) == tp.E_NULL
    assert call_decode(codes=FAKE + 4) == tp.E_ALIGN
    assert call_decode(w=FAKE + 2) == tp.E_ALIGN
    assert call_decode(scales=FAKE + 1) == tp.E_ALIGN


def test_python_binding_raises_value_error_on_validation(lib):
    with pytest.raises(ValueError):
        tp.prefill_raw(FAKE, 4, FAKE, FAKE, tp.geom(**GOOD), FAKE, 0)
    with pytest.raises(ValueError):
        tp.decode_raw(FAKE, FAKE, tp.geom(17408, 5120, 7), FAKE, 0)


def call_matvec(x=FAKE, m=1, codes=FAKE, scales=FAKE, g=None, out=FAKE):
    g = g or tp.geom(**GOOD)
    return tp.load_library().trellis_matvec(x, m, codes, scales, g, out, None)


def test_matvec_rejects_before_launch(lib):
    assert call_matvec(g=tp.geom(17408, 5000, 4)) == tp.E_GEOMETRY
    assert call_matvec(g=tp.geom(17408, 5120, 4, 256, 16)) == tp.E_GEOMETRY
    for m in (0, -1, 5, 15):
        assert call_matvec(m=m) == tp.E_M
    assert call_matvec(x=None) == tp.E_NULL
    assert call_matvec(codes=None) == tp.E_NULL
    assert call_matvec(scales=None) == tp.E_NULL
    assert call_matvec(out=None) == tp.E_NULL
    assert call_matvec(x=FAKE + 2) == tp.E_ALIGN
    assert call_matvec(codes=FAKE + 4) == tp.E_ALIGN
    assert call_matvec(out=FAKE + 8) == tp.E_ALIGN
    assert call_matvec(scales=FAKE + 1) == tp.E_ALIGN
    assert call_matvec(g=tp.geom(17408, 5000, 4), m=5, x=None) == tp.E_GEOMETRY
    assert call_matvec(m=5, x=None) == tp.E_M
    with pytest.raises(ValueError):
        tp.matvec_raw(FAKE, 5, FAKE, FAKE, tp.geom(**GOOD), FAKE, 0)


def call_gate_up(x=FAKE, m=5, cg=FAKE, sg=FAKE, cu=FAKE, su=FAKE, g=None, h=FAKE):
    g = g or tp.geom(**GOOD)
    return tp.load_library().trellis_gate_up(x, m, cg, sg, cu, su, g, h, None)


def test_gate_up_rejects_before_launch(lib):
    assert call_gate_up(g=tp.geom(17408, 5000, 4)) == tp.E_GEOMETRY
    for m in (0, 16, -3):
        assert call_gate_up(m=m) == tp.E_M
    for kw in ("x", "cg", "sg", "cu", "su", "h"):
        assert call_gate_up(**{kw: None}) == tp.E_NULL, kw
    assert call_gate_up(x=FAKE + 2) == tp.E_ALIGN
    assert call_gate_up(cg=FAKE + 4) == tp.E_ALIGN
    assert call_gate_up(cu=FAKE + 4) == tp.E_ALIGN
    assert call_gate_up(sg=FAKE + 1) == tp.E_ALIGN
    assert call_gate_up(su=FAKE + 1) == tp.E_ALIGN
    assert call_gate_up(h=FAKE + 8) == tp.E_ALIGN
    assert call_gate_up(g=tp.geom(17408, 5000, 4), m=0, x=None) == tp.E_GEOMETRY
    assert call_gate_up(m=0, x=None) == tp.E_M
    with pytest.raises(ValueError):
        tp.gate_up_raw(FAKE, 16, FAKE, FAKE, FAKE, FAKE, tp.geom(**GOOD), FAKE, 0)


def call_packed(xs=(FAKE, FAKE), rows=(2, 3), cd=FAKE, sc=FAKE, g=None, outs=(FAKE, FAKE), groups=None):
    import ctypes

    g = g or tp.geom(**GOOD)
    lib = tp.load_library()
    n = len(rows) if rows is not None else 2
    xa = None if xs is None else (ctypes.c_void_p * max(n, 1))(*xs)
    ra = None if rows is None else (ctypes.c_int32 * max(n, 1))(*rows)
    oa = None if outs is None else (ctypes.c_void_p * max(n, 1))(*outs)
    return lib.trellis_prefill_packed(xa, ra, n if groups is None else groups, cd, sc, g, oa, None)


def test_prefill_packed_rejects_before_launch(lib):
    assert call_packed(g=tp.geom(17408, 5000, 4)) == tp.E_GEOMETRY
    assert call_packed(xs=None) == tp.E_NULL
    assert call_packed(rows=None, groups=2) == tp.E_NULL
    assert call_packed(outs=None) == tp.E_NULL
    assert call_packed(cd=None) == tp.E_NULL
    assert call_packed(sc=None) == tp.E_NULL
    assert call_packed(groups=0) == tp.E_M
    assert call_packed(groups=tp.MAX_GROUPS + 1) == tp.E_M
    assert call_packed(rows=(2, -1)) == tp.E_M
    assert call_packed(rows=(0, 0)) == tp.E_M
    assert call_packed(rows=(2, tp.MAX_GROUP_ROWS + 1)) == tp.E_M
    assert call_packed(xs=(FAKE, None)) == tp.E_NULL
    assert call_packed(outs=(None, FAKE)) == tp.E_NULL
    assert call_packed(xs=(FAKE, FAKE + 2)) == tp.E_ALIGN
    assert call_packed(outs=(FAKE + 8, FAKE)) == tp.E_ALIGN
    assert call_packed(cd=FAKE + 4) == tp.E_ALIGN
    assert call_packed(sc=FAKE + 1) == tp.E_ALIGN
    # groups with no rows may pass NULL pointers; geometry is checked first
    assert call_packed(xs=(None, FAKE + 2), rows=(0, 3)) == tp.E_ALIGN
    assert call_packed(g=tp.geom(17408, 5000, 4), xs=None) == tp.E_GEOMETRY
    with pytest.raises(ValueError):
        tp.prefill_packed_raw([FAKE], [0], FAKE, FAKE, tp.geom(**GOOD), [FAKE], 0)


def test_one_hip_runtime_when_the_library_loads_before_torch():
    # PyTorch-ROCm links its bundled HIP runtime by the plain name
    # libamdhip64.so; the library links the runtime by its versioned name.
    # The binding imports torch before loading the library, so a process
    # that loads the library first still ends up with torch's runtime only
    # (two runtimes: the library sees no device). A fresh interpreter checks
    # the mapped files; no GPU is needed.
    import subprocess
    import sys

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = (
        "import sys; sys.path.insert(0, %r)\n"
        "import trellis_coded_bit_prefill_amd as tp\n"
        "tp.load_library()\n"
        "import torch\n"
        "print(len({l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}))\n" % root
    )
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr[-2000:]
    assert out.stdout.strip().splitlines()[-1] == "1", out.stdout
