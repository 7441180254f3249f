"""trellis_prefill on the GPU against the float64 CPU oracle.

Acceptance: |out - y| <= ulp_bf16(out) + 1e-5 * sum|w*x| elementwise, y the
float64 sum of the same bf16 products. One-hot activations make the sum a
single exact term, so those outputs must equal the decoded weights bit for
bit.
"""
import numpy as np
import pytest

import oracle
import trellis_coded_bit_prefill_amd as tp
from workloads import SHAPES, generate, generate_shape
from tests.helpers import (assert_prefill_close, exhaustive_window_codes, from_dev_bf16, to_dev_bf16,
                           to_dev_codes)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tp.load_library()


def gpu_prefill(x, codes, scales, bits):
    import torch

    out = tp.prefill(to_dev_bf16(x), to_dev_codes(codes), to_dev_bf16(scales), bits)
    torch.cuda.synchronize()
    return from_dev_bf16(out)


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("m", [5, 8, 15])
@pytest.mark.parametrize("n,k", [(4, 256), (68, 768), (324, 1792)])
def test_prefill_small_shapes(bits, m, n, k):
    print(f"prefill small m={m} n={n} k={k} bits={bits}", flush=True)
    x, codes, scales = generate(m, k, n, bits, seed=2000 + 7 * m + n + k + bits)
    out = gpu_prefill(x, codes, scales, bits)
    y, a = oracle.prefill(x, codes, scales, k, bits)
    assert_prefill_close(out, y, a, f"m={m} n={n} k={k} bits={bits}")


@pytest.mark.parametrize("m", list(range(5, 16)))
def test_prefill_every_m(m):
    print(f"prefill every m={m}", flush=True)
    x, codes, scales = generate(m, 1024, 132, 3, seed=3000 + m)
    out = gpu_prefill(x, codes, scales, 3)
    y, a = oracle.prefill(x, codes, scales, 1024, 3)
    assert_prefill_close(out, y, a, f"m={m}")


@pytest.mark.parametrize("name", ["tiny", "wide_m5_k4", "wide_m8_k3", "wide_m15_k2", "down_m15_k4"])
def test_prefill_full_shapes(name):
    # Every output of the five workloads, each checked against the float64
    # oracle (rows of the oracle split over the host's cores).
    s = SHAPES[name]
    print(f"prefill full shape {name}", flush=True)
    x, codes, scales = generate_shape(s)
    out = gpu_prefill(x, codes, scales, s.bits)
    assert out.shape == (s.m, s.n)
    y, a = oracle.prefill_parallel(x, codes, scales, s.k, s.bits)
    assert_prefill_close(out, y, a, name)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_prefill_one_hot_rows_equal_decoded_weights(bits):
    print(f"prefill one-hot bits={bits}", flush=True)
    k, n = 1024, 196
    _, codes, scales = generate(5, k, n, bits, seed=4000 + bits)
    cols = [0, 1, 7, 8, 255, 256, 257, 511, 512, 640, 767, 768, 1000, 1023, 100]
    x = np.zeros((len(cols), k), dtype=np.uint16)
    for i, c in enumerate(cols):
        x[i, c] = 0x3F80  # 1.0
    out = gpu_prefill(x, codes, scales, bits)
    w = oracle.decode(codes, scales, k, bits)
    assert np.array_equal(out, w[:, cols].T)


def test_prefill_zero_codes_closed_form():
    # All-zero codes decode every weight to bf16(v0 * s_n), v0 = value(window 0).
    k, n, m = 768, 36, 9
    x, _, scales = generate(m, k, n, 4, seed=4100)
    codes = np.zeros((n, k * 4 // 32), dtype=np.uint32)
    out = gpu_prefill(x, codes, scales, 4)
    y, a = oracle.prefill(x, codes, scales, k, 4)
    assert_prefill_close(out, y, a, "zero codes")


def test_prefill_is_deterministic():
    s = SHAPES["wide_m8_k3"]
    x, codes, scales = generate_shape(s)
    import torch

    xd, cd, sd = to_dev_bf16(x), to_dev_codes(codes), to_dev_bf16(scales)
    o1 = tp.prefill(xd, cd, sd, s.bits)
    o2 = tp.prefill(xd, cd, sd, s.bits)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_prefill_rejects_bad_m_on_device():
    import torch

    x = torch.zeros((4, 256), dtype=torch.bfloat16, device="cuda")
    codes = torch.zeros((4, 32), dtype=torch.int32, device="cuda")
    scales = torch.zeros((4,), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        tp.prefill(x, codes, scales, 4)
    x16 = torch.zeros((16, 256), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        tp.prefill(x16, codes, scales, 4)


def test_prefill_k_panels_with_whole_tiles_per_wave():
    # M=15 and K=5120 need two K panels of x in LDS; with N=65536 each wave's
    # unit range spans whole tiles, which must still be summed across panels.
    m, k, n, bits = 15, 5120, 65536, 2
    print(f"prefill panels+whole tiles m={m} k={k} n={n}", flush=True)
    x, codes, scales = generate(m, k, n, bits, seed=4200)
    out = gpu_prefill(x, codes, scales, bits)
    rng = np.random.default_rng(12)
    rows = np.unique(np.concatenate([np.arange(48), np.arange(n - 48, n), rng.integers(0, n, 256)]))
    y, a = oracle.prefill_rows(x, codes, scales, k, bits, rows)
    assert_prefill_close(out[:, rows], y, a, "panels+whole tiles")


@pytest.mark.parametrize("bits,shift,table", [(2, 0, "pair"), (2, 1, "pair"), (2, 0, "value"), (2, 0, "code"),
                                              (3, 0, "value"), (3, 0, "code"), (4, 0, "value"), (4, 0, "code")])
def test_prefill_weights_bit_exact_every_window_and_scale(bits, shift, table, force_table):
    # One-hot x rows pick single columns of W, so every output is one decoded
    # weight (sum of one exact product): prefill's in-kernel decode (the LDS
    # table named by `table` and the ALU path) must give exactly the oracle's
    # weights. Rows hold all 4096 windows; scales cover the 257 reachable
    # values, both signs, zero, and magnitudes outside 2^-110..2^110 (rows
    # that take the fallback path). For k = 2 the two shifts put the written
    # windows at odd and at even weight positions: both halves of a
    # pair-table entry.
    import torch

    force_table(table)
    print(f"prefill one-hot exhaustive bits={bits} shift={shift} table={table}", flush=True)
    rng = np.random.default_rng(600 + bits + 10 * shift)
    extra = [0x3F80, 0xBF80, 0xBC00, 0xBCA4, 0x0000, 0x8000, 0x0B00, 0x7300, 0x3FFF, 0xC07F,
             0x0600, 0x7900, 0x8600]
    scales = np.concatenate([np.arange(0x3BA4, 0x3CA5, dtype=np.uint16), np.array(extra, dtype=np.uint16)])
    scales = np.concatenate([scales, np.full((-scales.size) % 16, 0x3C00, dtype=np.uint16)])
    codes, k = exhaustive_window_codes(rng, scales.size, bits, shift)
    w_ref = oracle.decode(codes, scales, k, bits)
    cd, sd = to_dev_codes(codes), to_dev_bf16(scales)
    m = 15
    bad = 0
    for c0 in range(0, k, m):
        cols = np.arange(c0, min(c0 + m, k))
        x = np.zeros((max(5, cols.size), k), dtype=np.uint16)
        x[np.arange(cols.size), cols] = 0x3F80
        out = tp.prefill(to_dev_bf16(x), cd, sd, bits)
        torch.cuda.synchronize()
        got = (from_dev_bf16(out)[: cols.size].astype(np.uint32) << 16).view(np.float32)
        ref = (w_ref[:, cols].T.astype(np.uint32) << 16).view(np.float32)
        bad += int(np.sum(got != ref))  # +0 == -0: zero weights may differ in sign only
    assert bad == 0


@pytest.mark.parametrize("bits,table", [(2, "value"), (2, "code"), (2, "pair"), (3, "value"), (3, "code"),
                                        (4, "value"), (4, "code")])
@pytest.mark.parametrize("m,k", [(5, 1280), (15, 5120)])
def test_prefill_each_table(bits, table, m, k, force_table):
    # Every decode table on one shape with several tiles and a ragged last
    # tile; M = 15, K = 5120 needs two K panels with the value or pair table
    # and one with the code table.
    force_table(table)
    n = 84
    print(f"prefill table={table} m={m} k={k} n={n} bits={bits}", flush=True)
    x, codes, scales = generate(m, k, n, bits, seed=5000 + 3 * m + bits)
    out = gpu_prefill(x, codes, scales, bits)
    y, a = oracle.prefill(x, codes, scales, k, bits)
    assert_prefill_close(out, y, a, f"table={table} m={m} k={k} bits={bits}")


@pytest.mark.parametrize("bits,table", [(4, "value"), (4, "code"), (2, "value"), (2, "code")])
@pytest.mark.parametrize("k", [256, 512])
def test_prefill_ranges_of_one_and_two_units(bits, table, k, force_table):
    # N = 65536 rows make 4096 tiles: on 256 workgroups of 16 waves every
    # wave gets one unit with one K block (k = 256) and two with two. The
    # two-phase kernels decode a range's first unit before the prologue's
    # last barrier when the range holds two units or more and the unit's row
    # scales are all inside the ALU path's exact range. Every fifth tile
    # holds a scale of 2^115 and every tenth one of -2^-115, so first units
    # take each branch, and one-unit ranges take the plain loop.
    force_table(table)
    m, n = 5, 65536
    print(f"prefill one/two-unit ranges bits={bits} table={table} k={k}", flush=True)
    x, codes, scales = generate(m, k, n, bits, seed=4500 + k + bits)
    tiles = scales.reshape(-1, 16).copy()
    tiles[::5, 3] = 0x7900
    tiles[2::10, 7] = 0x8600
    scales = tiles.reshape(-1)
    out = gpu_prefill(x, codes, scales, bits)
    y, a = oracle.prefill_parallel(x, codes, scales, k, bits)
    assert_prefill_close(out, y, a, f"bits={bits} table={table} k={k}")


def test_prefill_workspace_grows_between_calls():
    # One stream: a small call, a call needing a larger workspace (more tiles,
    # K panels), then the small call again; the grown workspace starts with
    # zeroed counters and every result stays within the tolerance.
    cases = [(5, 512, 256, 2, 21), (15, 17408, 1040, 4, 22), (8, 768, 68, 3, 23), (15, 17408, 1040, 4, 24)]
    for m, k, n, bits, seed in cases:
        print(f"prefill workspace growth m={m} k={k} n={n} bits={bits}", flush=True)
        x, codes, scales = generate(m, k, n, bits, seed=seed)
        out = gpu_prefill(x, codes, scales, bits)
        rows = np.arange(n) if n <= 400 else np.unique(np.concatenate([np.arange(40), np.arange(n - 40, n),
                                                                        np.arange(0, n, 37)]))
        y, a = oracle.prefill_rows(x, codes, scales, k, bits, rows)
        assert_prefill_close(out[:, rows], y, a, f"growth m={m} k={k} n={n}")


def test_prefill_maximum_k():
    # K = TRELLIS_MAX_K (1024 blocks) at M = 15: x is staged in 64 K panels
    # of 16 blocks; every tile is summed across panels through the workspace.
    import torch

    m, k, n, bits = 15, 1 << 18, 36, 2
    print(f"prefill max K m={m} k={k} n={n}", flush=True)
    x, codes, scales = generate(m, k, n, bits, seed=4300)
    out = gpu_prefill(x, codes, scales, bits)
    y, a = oracle.prefill(x, codes, scales, k, bits)
    assert_prefill_close(out, y, a, "max K")


def test_prefill_maximum_n():
    # N = TRELLIS_MAX_N (2^18 tiles) with one block per row: a quarter of a
    # million tiles spread over the workgroups; sampled rows checked.
    m, k, n, bits = 7, 256, 1 << 22, 2
    print(f"prefill max N m={m} k={k} n={n}", flush=True)
    x, codes, scales = generate(m, k, n, bits, seed=4400)
    out = gpu_prefill(x, codes, scales, bits)
    rng = np.random.default_rng(14)
    rows = np.unique(np.concatenate([np.arange(40), np.arange(n - 40, n), rng.integers(0, n, 400)]))
    y, a = oracle.prefill_rows(x, codes, scales, k, bits, rows)
    assert_prefill_close(out[:, rows], y, a, "max N")
