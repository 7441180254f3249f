"""The VALU-dot contraction variant (measurement only) against the oracle.

The variant replaces each bf16 MFMA by per-lane v_dot2c_f32_bf16 dot
products (k = 4 kernel, value table, M = 5 and M = 1); it must meet the same
tolerance as the MFMA kernels before its timing means anything.
"""
import numpy as np
import pytest

import oracle
import trellis_coded_bit_prefill_amd as tp
from tests.helpers import assert_prefill_close, from_dev_bf16, to_dev_bf16, to_dev_codes
from workloads import SHAPES, generate, generate_shape

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tp.load_library()


@pytest.fixture
def valu():
    tp.force_table("value")
    tp.force_contraction("valu")
    yield
    tp.force_contraction("mfma")
    tp.force_table(None)


def run(fn, x, codes, scales, bits):
    import torch

    out = fn(to_dev_bf16(x), to_dev_codes(codes), to_dev_bf16(scales), bits)
    torch.cuda.synchronize()
    return from_dev_bf16(out)


@pytest.mark.parametrize("name", ["wide_m5_k4", "matvec_m1_k4"])
def test_valu_dot_full_shape(name, valu):
    s = SHAPES[name]
    print(f"valu dot {name}", flush=True)
    x, codes, scales = generate_shape(s)
    out = run(tp.prefill if s.m >= 5 else tp.matvec, x, codes, scales, s.bits)
    y, a = oracle.prefill_parallel(x, codes, scales, s.k, s.bits)
    assert_prefill_close(out, y, a, f"valu {name}")


@pytest.mark.parametrize("m,n,k", [(5, 324, 1792), (1, 68, 768), (5, 17408, 17408)])
def test_valu_dot_small_and_panels(m, n, k, valu):
    print(f"valu dot m={m} n={n} k={k}", flush=True)
    x, codes, scales = generate(m, k, n, 4, seed=9700 + m + n)
    out = run(tp.prefill if m >= 5 else tp.matvec, x, codes, scales, 4)
    if n > 4096:
        rows = np.arange(0, n, 7)
        y, a = oracle.prefill_rows(x, codes, scales, k, 4, rows)
        assert_prefill_close(out[:, rows], y, a, f"valu m={m} n={n} k={k}")
    else:
        y, a = oracle.prefill(x, codes, scales, k, 4)
        assert_prefill_close(out, y, a, f"valu m={m} n={n} k={k}")
