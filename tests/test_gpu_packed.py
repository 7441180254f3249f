"""GPU parity of trellis_prefill_packed (token packing) against the CPU oracle.

The rows of several independent inputs go through the layer together; each
input's output must meet trellis_prefill's tolerance against the oracle on
that input alone: |out - y| <= ulp_bf16(out) + 1e-5 * sum|w*x|, y the float64
sum of the same bf16 products. Inputs are separate device allocations, so
the kernel reads and writes rows through per-row pointers.
"""
import numpy as np
import pytest

import oracle
import trellis_coded_bit_prefill_amd as tp
from tests.helpers import assert_prefill_close, from_dev_bf16, to_dev_bf16, to_dev_codes
from workloads import SHAPES, generate, make_x

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tp.load_library()


def groups_x(rows, k, seed, kind="rmsnorm"):
    rng = np.random.Generator(np.random.PCG64(seed))
    return [make_x(rng, r, k, kind) if r else np.zeros((0, k), dtype=np.uint16) for r in rows]


def run_packed(xs, codes, scales, bits):
    import torch

    outs = tp.prefill_packed([to_dev_bf16(x) for x in xs], to_dev_codes(codes), to_dev_bf16(scales), bits)
    torch.cuda.synchronize()
    return [from_dev_bf16(o) for o in outs]


@pytest.mark.parametrize("rows", [(3, 1, 4, 2), (7, 9, 6), (0, 5, 0, 3), (1,), (15,), (2, 13), (16, 1, 15)])
@pytest.mark.parametrize("bits", [2, 3, 4])
def test_packed_groups(rows, bits):
    # One launch (<= 15 packed rows), several launches (> 15), groups with no
    # rows, single groups, and a group split across two launches.
    k, n = 1280, 132
    print(f"packed rows={rows} bits={bits}", flush=True)
    _, codes, scales = generate(5, k, n, bits, seed=7000 + bits)
    xs = groups_x(rows, k, seed=7100 + sum(rows) + bits)
    outs = run_packed(xs, codes, scales, bits)
    for i, (x, o) in enumerate(zip(xs, outs)):
        assert o.shape == (x.shape[0], n)
        if x.shape[0] == 0:
            continue
        y, a = oracle.prefill(x, codes, scales, k, bits)
        assert_prefill_close(o, y, a, f"group {i} rows={rows} bits={bits}")


def test_packed_single_group_matches_plain_call_bit_for_bit():
    # One group of m rows takes the same plan as trellis_prefill on the same
    # m, so the summation order and every output bit agree.
    import torch

    k, n, bits, m = 2048, 200, 3, 9
    x, codes, scales = generate(m, k, n, bits, seed=7201)
    xd, cd, sd = to_dev_bf16(x), to_dev_codes(codes), to_dev_bf16(scales)
    plain = tp.prefill(xd, cd, sd, bits)
    (packed,) = tp.prefill_packed([xd], cd, sd, bits)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev_bf16(plain), from_dev_bf16(packed))


def test_packed_rows_in_k_panels():
    # K = 17408 at 15 packed rows needs four K panels: staged x rows of
    # several inputs, partial tiles summed across panels.
    k, n, bits = 17408, 264, 4
    rows = (6, 5, 4)
    print(f"packed k panels rows={rows}", flush=True)
    _, codes, scales = generate(5, k, n, bits, seed=7300)
    xs = groups_x(rows, k, seed=7301, kind="silu_mul")
    outs = run_packed(xs, codes, scales, bits)
    for i, (x, o) in enumerate(zip(xs, outs)):
        y, a = oracle.prefill(x, codes, scales, k, bits)
        assert_prefill_close(o, y, a, f"group {i}")


def test_packed_wide_shape_sampled_rows():
    # The wide geometry (K = 5120, N = 17408, k = 4) with three inputs of
    # 5, 6 and 4 rows: one launch of 15 packed rows; outputs checked on
    # sampled columns.
    s = SHAPES["wide_m5_k4"]
    rows = (5, 6, 4)
    print(f"packed wide rows={rows}", flush=True)
    _, codes, scales = generate(5, s.k, s.n, s.bits, seed=s.seed)
    xs = groups_x(rows, s.k, seed=7400)
    outs = run_packed(xs, codes, scales, s.bits)
    rng = np.random.default_rng(13)
    cols = np.unique(np.concatenate([np.arange(48), np.arange(s.n - 48, s.n), rng.integers(0, s.n, 256)]))
    for i, (x, o) in enumerate(zip(xs, outs)):
        y, a = oracle.prefill_rows(x, codes, scales, s.k, s.bits, cols)
        assert_prefill_close(o[:, cols], y, a, f"wide group {i}")
