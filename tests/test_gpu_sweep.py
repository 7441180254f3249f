"""Seeded random sweep: shapes, batch sizes, bit widths, decode tables and
entry points drawn together, each case checked against the CPU oracle with
the acceptance of the dedicated tests (|out - y| <= ulp_bf16(out) +
1e-5 * sum|w*x|; for gate/up the bound of oracle.gate_up_within_tolerance).

The dedicated tests walk fixed grids; this one mixes the axes (for example a
forced code table under gate/up, or packed groups over several K panels), so
a plan or combine path that only some combinations reach is still run. Every
case is small enough for the oracle to finish in well under a second.
"""
import numpy as np
import pytest

import oracle
import trellis_coded_bit_prefill_amd as tp
from tests.helpers import assert_prefill_close, from_dev_bf16, to_dev_bf16, to_dev_codes
from workloads import generate, make_x

pytestmark = pytest.mark.gpu

ENTRIES = ("prefill", "matvec", "gate_up", "packed")
MAX_WEIGHTS = 3_000_000  # per matrix, keeps each oracle call short


def draw_cases(count: int, seed: int):
    rng = np.random.Generator(np.random.PCG64(seed))
    cases = []
    for i in range(count):
        entry = ENTRIES[i % len(ENTRIES)]
        bits = int(rng.integers(2, 5))
        tables = [None, "value", "code"] + (["pair"] if bits == 2 else [])
        table = tables[int(rng.integers(0, len(tables)))]
        # K up to 17408 (several K panels at large M), N a multiple of 4
        k = 256 * int(rng.choice([1, 2, 3, 5, 8, 13, 20, 27, 40, 68]))
        n = 4 * int(rng.integers(1, 400))
        n = max(4, min(n, (MAX_WEIGHTS // k) // 4 * 4))
        if entry == "prefill":
            m = int(rng.integers(tp.MIN_M, tp.MAX_M + 1))
            groups = ()
        elif entry == "matvec":
            m = int(rng.integers(1, tp.MIN_M))
            groups = ()
        elif entry == "gate_up":
            m = int(rng.integers(1, tp.MAX_M + 1))
            groups = ()
        else:
            groups = tuple(int(r) for r in rng.integers(0, 12, int(rng.integers(1, 5))))
            if sum(groups) == 0:
                groups = groups[:-1] + (3,)
            m = sum(groups)
        cases.append((i, entry, bits, table, m, k, n, groups, int(rng.integers(1, 2**31))))
    return cases


CASES = draw_cases(48, seed=20261202)


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tp.load_library()


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-{c[1]}-k{c[2]}-{c[3] or 'auto'}-m{c[4]}-K{c[5]}-N{c[6]}")
def test_sweep(case, force_table):
    import torch

    i, entry, bits, table, m, k, n, groups, seed = case
    if table is not None:
        force_table(table)
    else:
        force_table(None)
    what = f"sweep case {i}: {entry} bits={bits} table={table} m={m} k={k} n={n} groups={groups} seed={seed}"
    print(what, flush=True)
    if entry in ("prefill", "matvec"):
        x, codes, scales = generate(m, k, n, bits, seed=seed)
        fn = tp.prefill if entry == "prefill" else tp.matvec
        out = fn(to_dev_bf16(x), to_dev_codes(codes), to_dev_bf16(scales), bits)
        torch.cuda.synchronize()
        y, a = oracle.prefill(x, codes, scales, k, bits)
        assert_prefill_close(from_dev_bf16(out), y, a, what)
    elif entry == "gate_up":
        x, cg, sg = generate(m, k, n, bits, seed=seed)
        _, cu, su = generate(m, k, n, bits, seed=seed + 1)
        h = tp.gate_up(to_dev_bf16(x), to_dev_codes(cg), to_dev_bf16(sg), to_dev_codes(cu), to_dev_bf16(su), bits)
        torch.cuda.synchronize()
        h = from_dev_bf16(h)
        ref, g, ag, u, au = oracle.gate_up_rows(x, cg, sg, cu, su, k, bits, np.arange(n))
        ok = oracle.gate_up_within_tolerance(h, ref, g, ag, u, au)
        assert ok.all(), f"{what}: {int((~ok).sum())} of {ok.size} out of bound"
    else:
        _, codes, scales = generate(1, k, n, bits, seed=seed)
        rng = np.random.Generator(np.random.PCG64(seed + 2))
        xs = [make_x(rng, r, k, "rmsnorm") if r else np.zeros((0, k), dtype=np.uint16) for r in groups]
        outs = tp.prefill_packed([to_dev_bf16(xg) for xg in xs], to_dev_codes(codes), to_dev_bf16(scales), bits)
        torch.cuda.synchronize()
        for gi, (xg, og) in enumerate(zip(xs, outs)):
            o = from_dev_bf16(og)
            assert o.shape == (xg.shape[0], n)
            if xg.shape[0] == 0:
                continue
            y, a = oracle.prefill(xg, codes, scales, k, bits)
            assert_prefill_close(o, y, a, f"{what} group {gi}")
