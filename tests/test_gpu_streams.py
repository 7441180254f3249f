"""trellis_prefill on several HIP streams and under HIP graph capture.

The library keeps one workspace (partial tiles and self-resetting per-tile
counters) per (device, stream), and the combine of shared tiles sums the
partials in a fixed order, so a call's output does not depend on the stream
it runs on or on what runs next to it. These tests hold the library to that:

* calls interleaved on two streams give the same bits as the same calls run
  one after another on one stream;
* a call captured into a HIP graph and replayed (with new inputs copied into
  the captured buffers, eager calls and synchronisations between replays)
  gives, at every replay, the bits of the eager call on the same inputs;
* two host threads calling at the same time with hipStreamPerThread (one
  handle, a different stream per thread, so a workspace per thread) get the
  one-stream bits.

Shapes are chosen so that tiles are shared across workgroups (the wide
geometry) and across K panels (M = 15, K = 17408), where the workspace and
its counters are used. Every reference output is also checked against the
float64 CPU oracle on sampled rows.
"""
import numpy as np
import pytest

import oracle
import trellis_coded_bit_prefill_amd as tp
from workloads import generate
from tests.helpers import assert_prefill_close, from_dev_bf16, to_dev_bf16, to_dev_codes

pytestmark = pytest.mark.gpu

# (m, k, n, bits): one K panel with tiles shared by neighbouring workgroups;
# four K panels, where every tile goes through the workspace.
CASES = [(5, 5120, 4352, 4), (15, 17408, 1024, 4)]
SAMPLE_ROWS = 24


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tp.load_library()


def check_against_oracle(out, x, codes, scales, k, bits, seed, what):
    rows = np.random.default_rng(seed).choice(codes.shape[0], size=SAMPLE_ROWS, replace=False)
    rows.sort()
    y, a = oracle.prefill_rows(x, codes, scales, k, bits, rows)
    assert_prefill_close(out[:, rows], y, a, what)


def inputs(case, seed):
    m, k, n, bits = case
    x, codes, scales = generate(m, k, n, bits, seed=seed)
    return x, codes, scales, (to_dev_bf16(x), to_dev_codes(codes), to_dev_bf16(scales))


@pytest.mark.parametrize("case", CASES, ids=lambda c: "m%d_k%d_n%d_b%d" % c)
def test_two_streams_interleaved(case):
    import torch

    m, k, n, bits = case
    print(f"two streams {case}", flush=True)
    sets = [inputs(case, seed=7100 + 13 * i + m) for i in range(4)]
    # References: one call after another on the current stream.
    ref = []
    for i, (x, codes, scales, dev) in enumerate(sets):
        out = tp.prefill(*dev, bits)
        torch.cuda.synchronize()
        ref.append(from_dev_bf16(out))
        check_against_oracle(ref[-1], x, codes, scales, k, bits, 7200 + i, f"{case} set {i}")
    # The same calls, alternating between two side streams, three rounds.
    main = torch.cuda.current_stream()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(main)
    outs = [[None] * len(sets) for _ in range(3)]
    for r in range(3):
        for i, (_, _, _, dev) in enumerate(sets):
            s = streams[(i + r) % 2]
            with torch.cuda.stream(s):
                o = torch.empty((m, n), dtype=torch.bfloat16, device=dev[0].device)
                tp.prefill(*dev, bits, out=o)
            outs[r][i] = o
    torch.cuda.synchronize()
    for r in range(3):
        for i in range(len(sets)):
            got = from_dev_bf16(outs[r][i])
            assert np.array_equal(got, ref[i]), f"{case}: round {r}, set {i} differs from the one-stream result"


@pytest.mark.parametrize("case", CASES, ids=lambda c: "m%d_k%d_n%d_b%d" % c)
def test_graph_capture_replay(case):
    import torch

    m, k, n, bits = case
    print(f"graph capture {case}", flush=True)
    sets = [inputs(case, seed=7300 + 17 * i + m) for i in range(3)]
    xb, cb, sb = (t.clone() for t in sets[0][3])  # the captured buffers
    out = torch.empty((m, n), dtype=torch.bfloat16, device=xb.device)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    # A first call on the capture stream allocates its workspace, so nothing
    # is allocated while the stream is being captured.
    with torch.cuda.stream(s):
        tp.prefill(xb, cb, sb, bits, out=out)
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        tp.prefill(xb, cb, sb, bits, out=out)
    torch.cuda.synchronize()
    for rep in range(6):
        x, codes, scales, dev = sets[rep % len(sets)]
        xb.copy_(dev[0])
        cb.copy_(dev[1])
        sb.copy_(dev[2])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = from_dev_bf16(out)
        eager = from_dev_bf16(tp.prefill(*dev, bits))  # eager call between replays
        torch.cuda.synchronize()
        assert np.array_equal(got, eager), f"{case}: replay {rep} differs from the eager call"
        check_against_oracle(got, x, codes, scales, k, bits, 7400 + rep, f"{case} replay {rep}")


HIP_STREAM_PER_THREAD = 2  # hipStreamPerThread: the calling host thread's own default stream


@pytest.mark.parametrize("case", CASES, ids=lambda c: "m%d_k%d_n%d_b%d" % c)
def test_per_thread_default_stream_from_two_threads(case):
    # hipStreamPerThread is one handle that names a different stream on every
    # host thread. Two threads calling with it at the same time run
    # concurrently on the GPU, so each needs its own workspace; sharing one
    # would race on the tile counters and partials. Both threads' results
    # must equal the one-stream results bit for bit.
    import threading

    import torch

    m, k, n, bits = case
    print(f"per-thread default stream {case}", flush=True)
    sets = [inputs(case, seed=7500 + 19 * i + m) for i in range(4)]
    ref = []
    for i, (x, codes, scales, dev) in enumerate(sets):
        out = tp.prefill(*dev, bits)
        torch.cuda.synchronize()
        ref.append(from_dev_bf16(out))
        check_against_oracle(ref[-1], x, codes, scales, k, bits, 7600 + i, f"{case} set {i}")
    g = tp.geom(n, k, bits)
    rounds = 6
    outs = [[torch.empty((m, n), dtype=torch.bfloat16, device=sets[0][3][0].device) for _ in range(rounds)]
            for _ in range(2)]
    torch.cuda.synchronize()
    start = threading.Barrier(2)
    errors = []

    def worker(t):
        try:
            start.wait()
            for r in range(rounds):
                xd, cd, sd = sets[(t + r) % len(sets)][3]
                tp.prefill_raw(xd.data_ptr(), m, cd.data_ptr(), sd.data_ptr(), g, outs[t][r].data_ptr(),
                               HIP_STREAM_PER_THREAD)
            # Wait here, while the thread and its per-thread stream exist: a
            # synchronisation after the thread has ended need not cover the
            # work of the stream it leaves behind.
            torch.cuda.synchronize()
        except Exception as e:  # reported below, in the test's own thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for t in range(2):
        for r in range(rounds):
            got = from_dev_bf16(outs[t][r])
            assert np.array_equal(got, ref[(t + r) % len(sets)]), f"{case}: thread {t}, call {r} differs"
