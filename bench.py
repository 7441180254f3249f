#!/usr/bin/env python3
"""Benchmark of the packed Trellis prefill layer on one MI355X.

One step = one trellis_prefill call (the whole hot path: code-stream read,
window extraction, hash decode, normalisation, scale, bf16 rounding, x . W^T)
on the wide shape M=5, K=5120, N=17408, k=4 (T=256, L=12), inputs resident
in HBM. Inputs rotate over enough independent sets that the code streams do
not fit in the 256 MB Infinity Cache ("cold"), so every step reads its codes
from HBM.

The GPU raises its clocks only after some milliseconds of sustained work, so
the default warm-up is 2000 launches (about 40 ms) before the timed region.

Prints one JSON line:
  value = packed-code GB/s = (N*K*k/8 + 2*M*K + 2*M*N) bytes / step time
  roofline = the prefill kernel's algorithmic bytes / its average duration
             (HIP events around the timed region on the launch stream, which
             holds nothing but prefill launches) against 8 TB/s
  cpu_baseline = the CPU oracle on the same workload (host cores).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# Kernel arguments in device memory (the HIP runtime's HIP_FORCE_DEV_KERNARG,
# a setting AMD recommends on MI300-class GPUs). Every wave of the prefill
# kernel reads its plan from the argument segment first thing; from host
# memory that read costs about a microsecond of each launch (kernel trace at
# M=5, K=5120, N=17408, k=4: 20.6 against 21.6 us). It must be set before
# torch loads the HIP runtime; a setting already in the environment wins,
# so HIP_FORCE_DEV_KERNARG=0 measures the runtime's default placement.
os.environ.setdefault("HIP_FORCE_DEV_KERNARG", "1")

HBM_PEAK_GBS = 8000.0
MALL_BYTES = 256 << 20
WORKLOAD = "wide_m5_k4"


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "trellis_coded_bit_prefill_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def profile_figures(workload: str, sha: str):
    """Counter figures of the layer's kernel from rocprofv3 runs kept under
    profiles/ (VALU busy share and VALU instructions per weight), if they were
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"counters_prefill_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_sha") != sha:
        return None
    return {k: rec[k] for k in ("valu_busy_profiled", "valu_ops_per_weight_profiled") if k in rec}


def traffic_from_profiles(workload: str, sha: str):
    """HBM bytes per launch measured with rocprofv3 counters, if they were
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_prefill_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_sha") != sha:
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform

    return platform.processor() or "unknown"


def cpu_baseline(shape, passes: int):
    """The CPU oracle (plain C, float64 contraction) on the full layer of
    `shape`: rows split over the host's cores (at most 16 threads, the
    machine's CPU share per GPU), and on one thread. Median of `passes`
    threaded runs and one single-thread run."""
    import numpy as np

    import oracle
    from workloads import generate_gate_up, generate_shape

    oracle.lib()
    threads = oracle.default_threads()
    if shape.matrices == 2:
        x, cg, sg, cu, su = generate_gate_up(shape)

        def run(t):
            oracle.prefill_parallel(x, cg, sg, shape.k, shape.bits, t)
            oracle.prefill_parallel(x, cu, su, shape.k, shape.bits, t)
    else:
        x, codes, scales = generate_shape(shape)

        def run(t):
            oracle.prefill_parallel(x, codes, scales, shape.k, shape.bits, t)

    def timed(t):
        t0 = time.perf_counter()
        run(t)
        return time.perf_counter() - t0

    dts = sorted(timed(threads) for _ in range(max(1, passes)))
    dt = dts[len(dts) // 2]
    dt1 = timed(1)
    del np
    return {
        "value": round(shape.algorithmic_bytes / dt / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"full {shape.name} layer (all {shape.n} rows, decode + float64 contraction), "
                  f"median of {len(dts)} passes on {threads} threads: {dt:.3f} s per pass, "
                  f"{shape.weights / dt / 1e9:.4f} Gweights/s",
        "cpu_model": cpu_model(),
        "host_cpus": os.cpu_count(),
        "one_thread": {"value": round(shape.algorithmic_bytes / dt1 / 1e9, 4), "unit": "GB/s",
                       "seconds_per_pass": round(dt1, 3),
                       "gweights_per_s": round(shape.weights / dt1 / 1e9, 5)},
    }


class Workload:
    """Device inputs of one workload: `nsets` independent input sets (set 0
    the seeded workload, the others drawn on the device with the same
    distributions) and a launcher of one step on set i."""

    def __init__(self, shape, warm: bool):
        import numpy as np
        import torch

        import trellis_coded_bit_prefill_amd as tp
        from workloads import generate_gate_up, generate_shape

        dev = torch.device("cuda:0")
        self.shape = shape
        if shape.matrices == 2:
            x0, cg0, sg0, cu0, su0 = generate_gate_up(shape)
            mats0 = [(cg0, sg0), (cu0, su0)]
        else:
            x0, c0, s0 = generate_shape(shape)
            mats0 = [(c0, s0)]

        def dev_bf16(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

        code_bytes = shape.matrices * shape.n * shape.k * shape.bits // 8
        self.nsets = nsets = 1 if warm else max(2, -(-2 * MALL_BYTES // code_bytes))
        gen = torch.Generator(device=dev)
        gen.manual_seed(shape.seed * 1000 + 1)
        sets = []
        for i in range(nsets):
            if i == 0:
                xs = dev_bf16(x0)
                mats = [(torch.from_numpy(c.view(np.int32)).to(dev), dev_bf16(sc)) for c, sc in mats0]
            else:
                xs = torch.roll(sets[0][0], shifts=i, dims=1).contiguous()
                mats = [(torch.randint(-2 ** 31, 2 ** 31, c.shape, dtype=torch.int32, device=dev, generator=gen),
                         torch.roll(sets[0][1][mi][1], shifts=i).contiguous()) for mi, (c, _) in enumerate(mats0)]
            out = torch.empty((shape.m, shape.n), dtype=torch.bfloat16, device=dev)
            sets.append((xs, mats, out))
        torch.cuda.synchronize()
        self.sets = sets
        self.stream = torch.cuda.current_stream(dev)
        self.handle = self.stream.cuda_stream
        self.g = tp.geom(shape.n, shape.k, shape.bits)
        self.ptrs = [(s[0].data_ptr(), [p.data_ptr() for cs in s[1] for p in cs], s[2].data_ptr()) for s in sets]
        self.lib = tp.load_library()
        self.tp = tp
        # M = 1..4 is the matvec entry point (same kernel and decode); two
        # matrices are the fused gate/up entry point; packed workloads pass
        # each input's rows as a separate allocation to trellis_prefill_packed.
        self.entry = self.lib.trellis_matvec if shape.m < tp.MIN_M else self.lib.trellis_prefill
        self.packed = []
        if shape.groups:
            import ctypes

            G = len(shape.groups)
            for xs, _, out in sets:
                xg, og, r0 = [], [], 0
                for r in shape.groups:
                    xg.append(xs[r0:r0 + r].clone())
                    og.append(torch.empty((r, shape.n), dtype=torch.bfloat16, device=dev))
                    r0 += r
                self.packed.append(((ctypes.c_void_p * G)(*[t.data_ptr() for t in xg]),
                                    (ctypes.c_void_p * G)(*[t.data_ptr() for t in og]), xg, og))
            self.rows_arr = (ctypes.c_int32 * G)(*shape.groups)

    def step(self, i):
        shape = self.shape
        xp, mp, op = self.ptrs[i % self.nsets]
        if shape.groups:
            xa, oa, _, _ = self.packed[i % self.nsets]
            rc = self.lib.trellis_prefill_packed(xa, self.rows_arr, len(shape.groups), mp[0], mp[1], self.g, oa,
                                                 self.handle)
        elif shape.matrices == 2:
            rc = self.lib.trellis_gate_up(xp, shape.m, mp[0], mp[1], mp[2], mp[3], self.g, op, self.handle)
        else:
            rc = self.entry(xp, shape.m, mp[0], mp[1], self.g, op, self.handle)
        if rc != 0:
            raise RuntimeError(self.tp.status_string(rc))

    def timed(self, steps: int, warmup: int):
        """Average ms per step over exactly `steps` back-to-back steps after
        `warmup` untimed ones (HIP events on the launch stream, which holds
        nothing but the layer's launches), and the wall time of the region."""
        import torch

        for i in range(warmup):
            self.step(i)
        torch.cuda.synchronize()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record(self.stream)
        t0 = time.perf_counter()
        for i in range(steps):
            self.step(i)
        ev1.record(self.stream)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / steps, time.perf_counter() - t0

    def isolated_median_ms(self, steps: int):
        """Median of per-launch event pairs (an idle GPU before each launch)."""
        import torch

        starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        for i in range(steps):
            starts[i].record(self.stream)
            self.step(i)
            ends[i].record(self.stream)
        torch.cuda.synchronize()
        durs = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))
        return durs[len(durs) // 2]

    def release(self):
        import torch

        self.sets = self.ptrs = self.packed = None
        torch.cuda.synchronize()
        torch.cuda.empty_cache()


def summary(shape, ms: float):
    gbs = shape.algorithmic_bytes / (ms * 1e-3) / 1e9
    return {"us": round(ms * 1e3, 3), "gb_per_s": round(gbs, 2), "frac_of_8tbs": round(gbs / HBM_PEAK_GBS, 4),
            "gweights_per_s": round(shape.weights / (ms * 1e-3) / 1e9, 2)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=2000)
    ap.add_argument("--workload", default=WORKLOAD)
    ap.add_argument("--warm", action="store_true", help="one input set (cache-resident codes)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-passes", type=int, default=3)
    ap.add_argument("--no-extra", action="store_true", help="skip the other workloads' figures")
    ap.add_argument("--extra-steps", type=int, default=300,
                    help="timed steps per extra workload (after --warmup warm-up steps)")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="only run a plain device copy of this many MiB (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this build has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration_mb:
        # A plain copy of known size: its FETCH_SIZE / WRITE_SIZE counter
        # readings calibrate the prefill kernel's measured HBM traffic.
        nbytes = args.copy_calibration_mb << 20
        src = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(max(1, args.steps)):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": nbytes, "launches": max(1, args.steps)}), flush=True)
        return

    import trellis_coded_bit_prefill_amd as tp
    from workloads import SHAPES

    shape = SHAPES[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    tp.load_library()

    wl = Workload(shape, args.warm)
    ms_per_step, wall = wl.timed(args.steps, args.warmup)
    # The timed region holds only the layer's launches, so its event-measured
    # average per launch is the kernel's average duration back to back.
    kernel_ms = ms_per_step
    isolated_median_ms = wl.isolated_median_ms(args.steps)
    nsets = wl.nsets
    wl.release()

    alg_bytes = shape.algorithmic_bytes
    value = alg_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = alg_bytes / (kernel_ms * 1e-3) / 1e9
    sha = kernel_source_sha()
    traffic = traffic_from_profiles(shape.name, sha)

    rec = {
        "metric": "packed-code HBM GB/s (N*K*k/8 + 2*M*K + 2*M*N bytes per step)",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": shape.name, "m": shape.m, "k": shape.k, "n": shape.n, "bits": shape.bits,
                   "T": 256, "L": 12, "matrices": shape.matrices, "groups": list(shape.groups), "input_sets": nsets,
                   "mode": "warm" if args.warm else "cold"},
        "gweights_per_s": round(shape.weights / (ms_per_step * 1e-3) / 1e9, 2),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": "prefill_kernel",
            "kernel_avg_us": round(kernel_ms * 1e3, 3),
            "isolated_launch_median_us": round(isolated_median_ms * 1e3, 3),
            "kernel_sha": sha,
        },
        "wall_s": round(wall, 4),
        "runtime_env": {"HIP_FORCE_DEV_KERNARG": os.environ.get("HIP_FORCE_DEV_KERNARG")},
    }
    prof = profile_figures(shape.name, sha)
    if prof:
        rec["roofline"].update(prof)
    if not args.no_extra and args.workload == WORKLOAD and not args.warm:
        # The other workloads of the metric (same cold protocol, their own
        # warm-up and timed steps), and the headline shape with one input set
        # (codes resident in the 256 MB Infinity Cache), labelled warm. Each
        # gets the full warm-up: its inputs are generated on the host first,
        # the GPU idles meanwhile, and after a few hundred launches its clocks
        # have not come back up (300 warm-up launches read about 2 us slow).
        extra = {}
        for name, warm in (("wide_m8_k3", False), ("wide_m15_k2", False), ("down_m15_k4", False),
                           ("wide_m5_k4", True)):
            w = Workload(SHAPES[name], warm)
            ms, _ = w.timed(args.extra_steps, args.warmup)
            w.release()
            rec_x = summary(SHAPES[name], ms)
            rec_x["mode"] = "warm" if warm else "cold"
            rec_x["steps"] = args.extra_steps
            rec_x["warmup"] = args.warmup
            p = profile_figures(name, sha)
            if p:
                rec_x.update(p)
            extra[name + ("_warm" if warm else "")] = rec_x
        rec["other_workloads"] = extra
    if not args.no_cpu:
        rec["cpu_baseline"] = cpu_baseline(shape, args.cpu_passes)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
