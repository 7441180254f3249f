"""GPU parity of trellis_gate_up against the CPU oracle.

h = silu(x . Wg^T) * (x . Wu^T) with the page's bf16 roundings of every
intermediate array (page "mlx-bun 0.0.4" (npm, page 62), section
src/model/minicpm5.ts, MLP forward). Two kinds of check:

* one-hot x rows (a power of two at one column) make both projections a
  single decoded weight times that power, exact in any summation order, so h
  has one right answer: the oracle's bf16 chain (oracle.gate_up_chain) on
  those two bf16 values. The device must match it bit for bit, except where
  the exact sigmoid sits within 2^-21 of a bf16 rounding boundary (a float32
  sigmoid may round either way there); those are counted and must be rare.
* general x: the exact float64 h = silu(g) * u of the float64 projections,
  with a bound (oracle.gate_up_within_tolerance) that carries the
  projections' tolerance through silu and the product and adds the chain's
  three bf16 roundings.
"""
import numpy as np
import pytest

import oracle
import trellis_coded_bit_prefill_amd as tp
from tests.helpers import from_dev_bf16, to_dev_bf16, to_dev_codes
from workloads import SHAPES, generate, generate_gate_up

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tp.load_library()


def gpu_gate_up(x, cg, sg, cu, su, bits):
    import torch

    h = tp.gate_up(to_dev_bf16(x), to_dev_codes(cg), to_dev_bf16(sg), to_dev_codes(cu), to_dev_bf16(su), bits)
    torch.cuda.synchronize()
    return from_dev_bf16(h)


def check(h, x, cg, sg, cu, su, k, bits, rows, what):
    ref, g, ag, u, au = oracle.gate_up_rows(x, cg, sg, cu, su, k, bits, rows)
    ok = oracle.gate_up_within_tolerance(h[:, rows], ref, g, ag, u, au)
    if not ok.all():
        idx = np.argwhere(~ok)[:5]
        hv = (h[:, rows].astype(np.uint32) << 16).view(np.float32)
        detail = ", ".join(f"[{i},{j}] gpu={hv[i, j]!r} ref={ref[i, j]!r} g={g[i, j]!r} u={u[i, j]!r}"
                           for i, j in idx)
        raise AssertionError(f"{what}: {int((~ok).sum())} of {ok.size} out of bound: {detail}")


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("m", [1, 5, 15])
@pytest.mark.parametrize("n,k", [(4, 256), (68, 768), (324, 1792)])
def test_gate_up_small_shapes(bits, m, n, k):
    print(f"gate_up small m={m} n={n} k={k} bits={bits}", flush=True)
    x, cg, sg = generate(m, k, n, bits, seed=7000 + 7 * m + n + k + bits)
    _, cu, su = generate(m, k, n, bits, seed=8000 + 7 * m + n + k + bits)
    h = gpu_gate_up(x, cg, sg, cu, su, bits)
    assert h.shape == (m, n)
    check(h, x, cg, sg, cu, su, k, bits, np.arange(n), f"m={m} n={n} k={k} bits={bits}")


def test_gate_up_full_shape():
    s = SHAPES["gateup_m5_k4"]
    print("gate_up full shape", flush=True)
    x, cg, sg, cu, su = generate_gate_up(s)
    h = gpu_gate_up(x, cg, sg, cu, su, s.bits)
    rng = np.random.default_rng(13)
    rows = np.unique(np.concatenate([np.arange(64), np.arange(s.n - 64, s.n), rng.integers(0, s.n, 384)]))
    check(h, x, cg, sg, cu, su, s.k, s.bits, rows, s.name)


def test_gate_up_k_panels():
    # x too large for one LDS panel: every tile of both matrices is summed
    # across workgroups, and the last contributor writes the elementwise tail.
    print("gate_up k panels", flush=True)
    m, k, n, bits = 15, 17408, 260, 4
    x, cg, sg = generate(m, k, n, bits, seed=9001, x_kind="silu_mul")
    _, cu, su = generate(m, k, n, bits, seed=9002)
    h = gpu_gate_up(x, cg, sg, cu, su, bits)
    check(h, x, cg, sg, cu, su, k, bits, np.arange(n), "k panels")


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("m,n", [(15, 2000), (15, 17408), (8, 17408)])
def test_gate_up_barrier_combine(bits, m, n):
    # M >= 8 at K = 5120: x leaves no LDS for partial slots of both
    # matrices, so tiles shared inside a workgroup are summed after a barrier
    # in x's LDS, and the pair of partials of a piece's first tile waits in
    # global memory through the loop. N = 2000 gives one-unit pieces (about
    # twenty contributors per tile); N = 17408 gives pieces of several units
    # that start inside one tile and end in another.
    k = 5120
    print(f"gate_up barrier combine m={m} n={n} bits={bits}", flush=True)
    x, cg, sg = generate(m, k, n, bits, seed=9201 + bits + m)
    _, cu, su = generate(m, k, n, bits, seed=9301 + bits + m)
    h = gpu_gate_up(x, cg, sg, cu, su, bits)
    if n <= 2000:
        rows = np.arange(n)
    else:
        rng = np.random.default_rng(17)
        rows = np.unique(np.concatenate([np.arange(48), np.arange(n - 48, n), rng.integers(0, n, 320)]))
    check(h, x, cg, sg, cu, su, k, bits, rows, f"barrier combine m={m} n={n} bits={bits}")


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("m", [1, 5, 15])
def test_gate_up_one_hot_bit_exact_chain(bits, m):
    # n spans many tiles and a ragged tail; k has four blocks. Row i of x is
    # 2^p_i at column j_i, so gate[i, n] = 2^p_i * Wg[n, j_i] exactly (and up
    # likewise): gates from about 1e-4 to 16 cover the sigmoid's curved part.
    n, k = 2004, 1024
    print(f"gate_up one-hot m={m} bits={bits}", flush=True)
    _, cg, sg = generate(5, k, n, bits, seed=9400 + bits)
    _, cu, su = generate(5, k, n, bits, seed=9500 + bits)
    rng = np.random.default_rng(9600 + 16 * bits + m)
    cols = rng.choice(k, size=m, replace=False)
    pows = np.array([0, 2, 4, 6, 8, 1, 3, 5, 7, 0, 2, 4, 6, 8, 5])[:m]
    x = np.zeros((m, k), dtype=np.uint16)
    x[np.arange(m), cols] = (0x3F80 + (pows << 7)).astype(np.uint16)   # 2^p as bf16
    h = gpu_gate_up(x, cg, sg, cu, su, bits)
    wg = oracle.decode(cg, sg, k, bits)[:, cols].T      # [m, n] bf16 bits
    wu = oracle.decode(cu, su, k, bits)[:, cols].T
    # 2^p * w in bf16: add p to the exponent field of every nonzero weight
    def scaled(w):
        w = w.astype(np.uint32)
        nz = (w & 0x7FFF) != 0
        return np.where(nz, w + (pows[:, None].astype(np.uint32) << 7), w).astype(np.uint16)
    want, amb = oracle.gate_up_chain(scaled(wg), scaled(wu))
    same = (h == want) | (((h & 0x7FFF) == 0) & ((want & 0x7FFF) == 0))
    bad = ~same & ~amb
    assert not bad.any(), (f"{int(bad.sum())} of {h.size} differ from the chain; first "
                           f"{[(int(i), int(j), hex(h[i, j]), hex(want[i, j])) for i, j in np.argwhere(bad)[:4]]}")
    assert amb.sum() <= max(10, h.size // 100), int(amb.sum())
    print(f"  {int(amb.sum())} of {h.size} sigmoids next to a bf16 boundary; "
          f"{int((~same & amb).sum())} of them rounded the other way", flush=True)


def test_gate_up_deterministic():
    m, k, n, bits = 8, 1024, 196, 3
    x, cg, sg = generate(m, k, n, bits, seed=9101)
    _, cu, su = generate(m, k, n, bits, seed=9102)
    a = gpu_gate_up(x, cg, sg, cu, su, bits)
    b = gpu_gate_up(x, cg, sg, cu, su, bits)
    assert np.array_equal(a, b)
