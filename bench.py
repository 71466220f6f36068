"""Throughput of the fused AdamW step on one MI355X, OPT-1.3B-shaped.

One bench step is the whole hot path over the OPT-1.3B parameter list (386
tensors, 1,315,753,984 parameters, each tensor its own allocation-aligned
buffer): a mixed-precision step (bf16 param/grad + fp32 master, exp_avg,
exp_avg_sq) followed by a pure-bf16 step with bf16 Kahan compensation, each one
call of adamw_multi_tensor_step (prologue + one update-kernel launch).  Inputs
are synthetic and seeded (master ~ N(0, 0.02), grads ~ N(0, 1e-3), moments 0) and
already resident in HBM when the timed region starts; the gradient buffers are
reused across steps.

value = parameter updates per second over the timed steps (2 x N per step, one
per mode), in Gparam/s.  Alongside it: per-mode Gparam/s and algorithmic HBM
GB/s (28 B/param mixed, 18 B/param Kahan), the roofline of the dominant kernel
(the mixed update) from HIP events recorded on the launch stream, and the CPU
oracle timed on a bounded sample on the host cores.

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--no-cpu]
       python bench.py --calib-copy     (plain device copy of known size, for
                                         scaling the rocprofv3 byte counters)
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published peak
BYTES = {"mixed": 28, "kahan": 18}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="opt_1_3b")
    ap.add_argument("--modes", default="mixed,kahan")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-sample", type=int, default=160_000_000,
                    help="elements of the OPT-1.3B list the oracle steps once per mode")
    ap.add_argument("--calib-copy", action="store_true")
    ap.add_argument("--chunk-elems", type=int, default=0)
    return ap.parse_args()


def calib_copy():
    """A plain copy of 4 GiB, three times: FETCH_SIZE / WRITE_SIZE of this kernel
    against the known 4 GiB per direction give the counters' scale."""
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calib_copy_bytes_each_way": n * 4, "launches": 3}), flush=True)


def make_mode_state(mode, numels, device, seed):
    import workloads
    arena = workloads.make_state(mode, numels, device, seed, align_elems=128)
    keys = workloads.STREAMS[mode]
    streams = [[arena.view(k, i) for i in range(len(numels))] for k in keys]
    return arena, streams


def cpu_baseline(numels, sample):
    """The oracle as it is (one host thread), one step per mode over the first
    `sample` elements of the list; scaled to param-updates/s of the two-mode step."""
    import numpy as np
    import torch

    import oracle
    import workloads
    n = min(sample, sum(numels))
    g = workloads.grads(n, "cpu", 7, 0, dtype=torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    w = workloads.normal(n, workloads.INIT_STD, "cpu", "master", 7).numpy()
    hp = oracle.HParams()
    secs = {}
    p16 = np.zeros(n, np.uint16)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    t0 = time.perf_counter()
    oracle.adamw_mixed(p16, g, w, m, v, hp, 1)
    secs["mixed"] = time.perf_counter() - t0
    del m, v
    pk = oracle.f32_to_bf16(w)
    del w
    mk, vk, ck = (np.zeros(n, np.uint16) for _ in range(3))
    t0 = time.perf_counter()
    oracle.adamw_kahan(pk, g, mk, vk, ck, hp, 1)
    secs["kahan"] = time.perf_counter() - t0
    per_param = secs["mixed"] / n + secs["kahan"] / n
    return {"value": round(2.0 / per_param / 1e9, 4), "unit": "Gparam/s", "cores": 1, "kind": "oracle",
            "sample": f"one mixed and one Kahan step over the first {n:,} parameters of the OPT-1.3B list "
                      f"(host-resident, 1 thread): {secs['mixed']:.2f} s + {secs['kahan']:.2f} s",
            "host_cpus": os.cpu_count()}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the step runs on one rank's share; a run on "
              f"{args.gpus} GPUs is not part of this build.", file=sys.stderr)
        sys.exit(2)
    import torch

    if args.calib_copy:
        calib_copy()
        return
    import adamw_optimizer_step_apply_amd as A
    import workloads

    if args.chunk_elems:
        A.adamw_set_chunk_elems(args.chunk_elems)
    wl = workloads.get(args.workload)
    numels = wl.numels
    N = wl.total
    modes = [m for m in args.modes.split(",") if m]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    state = {}
    for i, mode in enumerate(modes):
        arena, streams = make_mode_state(mode, numels, dev, seed=100 + i)
        state[mode] = (arena, A.TensorList(numels, streams), torch.zeros(1, dtype=torch.int32, device=dev))
    hp = A.HParams()
    code = {"mixed": A.MIXED, "kahan": A.PURE_KAHAN}

    def one(mode):
        _, tl, ctr = state[mode]
        A.adamw_multi_tensor_step(code[mode], A.BF16, tl, hp, ctr, None, stream)

    for _ in range(args.warmup):
        for mode in modes:
            one(mode)
    torch.cuda.synchronize()

    K = args.steps
    ev = {m: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
          for m in modes}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(K):
        for mode in modes:
            a, b = ev[mode][s]
            a.record(stream)
            one(mode)
            b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    per_mode = {}
    for mode in modes:
        ms = [a.elapsed_time(b) for a, b in ev[mode]]
        avg = sum(ms) / len(ms)
        per_mode[mode] = {
            "ms_avg": round(avg, 4), "ms_min": round(min(ms), 4),
            "gparam_s": round(N / (avg * 1e-3) / 1e9, 2),
            "gb_s": round(N * BYTES[mode] / (avg * 1e-3) / 1e9, 1),
            "frac_of_hbm_peak": round(N * BYTES[mode] / (avg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "bytes_per_param": BYTES[mode],
        }
    ms_step = wall / K * 1e3
    value = len(modes) * N / (wall / K) / 1e9
    dom = "mixed" if "mixed" in modes else modes[0]
    achieved = N * BYTES[dom] / (per_mode[dom]["ms_avg"] * 1e-3) / 1e9
    traffic = None
    tpath = os.path.join(ROOT, "profiles", "traffic_opt_1_3b.json")
    if os.path.exists(tpath):
        with open(tpath) as f:
            t = json.load(f)
        if t.get("kernel_source_sha") == _kernel_sha():
            traffic = t.get("traffic_bytes_per_launch", {}).get(dom)
    out = {
        "metric": "AdamW step Gparams/s + achieved HBM GB/s (% of peak), OPT-1.3B shape, 1 GPU",
        "value": round(value, 3),
        "unit": "Gparam/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: {len(numels)} tensors, {N:,} params; one step = "
                               + " then ".join({"mixed": "mixed (bf16 p/g + fp32 master/m/v)",
                                                "kahan": "pure bf16 + bf16 Kahan compensation"}[m]
                                               for m in modes),
                   "n_params": N, "n_tensors": len(numels), "modes": modes,
                   "hparams": {"lr": hp.lr, "beta1": hp.beta1, "beta2": hp.beta2, "eps": hp.eps,
                               "weight_decay": hp.weight_decay}},
        "per_mode": per_mode,
        "roofline": {"bound": "hbm", "kernel": f"update_kernel ({dom})", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic},
        "device": torch.cuda.get_device_name(dev),
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(numels, args.cpu_sample)
    print(json.dumps(out), flush=True)


def _kernel_sha():
    import hashlib
    h = hashlib.sha256()
    for f in ("kernels.hip", "plan.cpp", "layout.hpp"):
        with open(os.path.join(ROOT, "adamw_optimizer_step_apply_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


if __name__ == "__main__":
    main()
