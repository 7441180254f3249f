"""trellis_decode on the GPU: bit-exact against the CPU oracle."""
import numpy as np
import pytest

import oracle
import trellis_coded_bit_prefill_amd as tp
from workloads import SHAPES, generate
from tests.helpers import (exhaustive_window_codes, from_dev_bf16, to_dev_bf16, to_dev_codes,
                           windows_np)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tp.load_library()


def gpu_decode(codes, scales, k, bits):
    import torch

    w = tp.decode(to_dev_codes(codes), to_dev_bf16(scales), k, bits)
    torch.cuda.synchronize()
    return from_dev_bf16(w)


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("n,k", [(4, 256), (256, 512), (324, 1792)])
def test_decode_bit_exact_small(bits, n, k):
    print(f"decode small n={n} k={k} bits={bits}", flush=True)
    _, codes, scales = generate(5, k, n, bits, seed=1000 + n + k + bits)
    assert np.array_equal(gpu_decode(codes, scales, k, bits), oracle.decode(codes, scales, k, bits))


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_decode_exhaustive_windows_times_all_scales(bits):
    # Every 12-bit window in every row, one row per reachable bf16 scale
    # (0x3BA4 .. 0x3CA4, the RNE image of U[0.005, 0.02]) plus 3 more rows.
    print(f"decode exhaustive bits={bits}", flush=True)
    rng = np.random.default_rng(500 + bits)
    scales = np.concatenate([np.arange(0x3BA4, 0x3CA5, dtype=np.uint16),
                             np.array([0x3F80, 0x3C80, 0xBC00], dtype=np.uint16)])
    codes, k = exhaustive_window_codes(rng, scales.size, bits)
    wins = windows_np(codes, k, bits)
    for r in range(0, scales.size, 37):
        assert np.unique(wins[r]).size == 4096
    got = gpu_decode(codes, scales, k, bits)
    assert np.array_equal(got, oracle.decode(codes, scales, k, bits))


@pytest.mark.parametrize("name", ["tiny", "wide_m5_k4", "wide_m8_k3", "wide_m15_k2", "down_m15_k4"])
def test_decode_full_shapes_every_weight(name):
    # Every weight of W for the five workloads (oracle rows split over the
    # host's cores).
    s = SHAPES[name]
    print(f"decode full shape {name}", flush=True)
    _, codes, scales = generate(s.m, s.k, s.n, s.bits, s.seed, s.x_kind)
    got = gpu_decode(codes, scales, s.k, s.bits)
    want = oracle.decode_parallel(codes, scales, s.k, s.bits)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} weights differ, first at {bad[:3].tolist()}"
