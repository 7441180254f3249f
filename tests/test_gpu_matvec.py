"""GPU parity of trellis_matvec (1 <= M <= 4) against the CPU oracle.

Same decode and tolerance as trellis_prefill: |out - y| <= ulp_bf16(out) +
1e-5 * sum|w*x|, y the float64 sum of the same bf16 products; one-hot rows
must give the decoded weights bit for bit.
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


def gpu_matvec(x, codes, scales, bits):
    import torch

    out = tp.matvec(to_dev_bf16(x), to_dev_codes(codes), to_dev_bf16(scales), bits)
    torch.cuda.synchronize()
    return from_dev_bf16(out)


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("m", [1, 2, 3, 4])
@pytest.mark.parametrize("n,k", [(4, 256), (68, 768), (324, 1792)])
def test_matvec_small_shapes(bits, m, n, k):
    print(f"matvec small m={m} n={n} k={k} bits={bits}", flush=True)
    x, codes, scales = generate(m, k, n, bits, seed=5000 + 7 * m + n + k + bits)
    out = gpu_matvec(x, codes, scales, bits)
    y, a = oracle.prefill(x, codes, scales, k, bits)
    assert_prefill_close(out, y, a, f"m={m} n={n} k={k} bits={bits}")


@pytest.mark.parametrize("name", ["matvec_m1_k4", "matvec_m4_k2"])
def test_matvec_full_shapes(name):
    s = SHAPES[name]
    print(f"matvec full shape {name}", flush=True)
    x, codes, scales = generate_shape(s)
    out = gpu_matvec(x, codes, scales, s.bits)
    assert out.shape == (s.m, s.n)
    rng = np.random.default_rng(12)
    rows = np.unique(np.concatenate([np.arange(64), np.arange(s.n - 64, s.n), rng.integers(0, s.n, 384)]))
    y, a = oracle.prefill_rows(x, codes, scales, s.k, s.bits, rows)
    assert_prefill_close(out[:, rows], y, a, name)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_matvec_one_hot_rows_equal_decoded_weights(bits):
    print(f"matvec one-hot bits={bits}", flush=True)
    k, n = 1024, 196
    _, codes, scales = generate(1, k, n, bits, seed=6000 + bits)
    w = oracle.decode(codes, scales, k, bits)
    for cols in ([0], [255, 256], [7, 511, 1023], [1, 100, 640, 768]):
        x = np.zeros((len(cols), k), dtype=np.uint16)
        x[np.arange(len(cols)), cols] = 0x3F80
        out = gpu_matvec(x, codes, scales, bits)
        got = (out.astype(np.uint32) << 16).view(np.float32)
        ref = (w[:, cols].T.astype(np.uint32) << 16).view(np.float32)
        assert np.array_equal(got, ref), cols  # +0 == -0


def test_matvec_deterministic():
    s = SHAPES["matvec_m4_k2"]
    x, codes, scales = generate_shape(s)
    a = gpu_matvec(x, codes, scales, s.bits)
    b = gpu_matvec(x, codes, scales, s.bits)
    assert np.array_equal(a, b)


def test_matvec_rejects_prefill_batch():
    import torch

    x = torch.zeros((5, 256), dtype=torch.bfloat16, device="cuda")
    codes = torch.zeros((4, 256 * 2 // 32), dtype=torch.int32, device="cuda")
    scales = torch.zeros((4,), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        tp.matvec(x, codes, scales, 2)
    with pytest.raises(ValueError):
        tp.prefill(x[:4], codes, scales, 2)
