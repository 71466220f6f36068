"""Throughput of the fused AdamW step on one MI355X, OPT-1.3B-shaped.

One bench step is the whole hot path over the OPT-1.3B parameter list (386
tensors, 1,315,753,984 parameters; params and grads each tensor its own
allocation-aligned buffer) in both of its modes: a mixed-precision step (bf16
param/grad + fp32 master, exp_avg, exp_avg_sq) and a pure-bf16 step with bf16
Kahan compensation, each one call of adamw_multi_tensor_step (prologue + one
update-kernel launch).  The optimizer owns its state, as a ZeRO shard's
optimizer does, and keeps it in the blocked layout (exp_avg, exp_avg_sq and
master or compensation interleaved per block of one buffer); with --compare the
same steps on per-tensor state buffers are timed after the headline region and
reported as per_tensor_state.  The timed region runs K mixed steps then K Kahan steps (two
consecutive phases, as two training runs would); --interleave alternates them
instead.  Inputs are synthetic and seeded (master ~ N(0, 0.02), grads ~
N(0, 1e-3), moments 0) and already resident in HBM when the timed region
starts; the gradient buffers are reused across steps.

value = parameter updates per second over the timed steps (2 x N per step, one
per mode), in Gparam/s.  Alongside it: per-mode Gparam/s and algorithmic HBM
GB/s (28 B/param mixed, 18 B/param Kahan), the time of each mode's first call
(plan build + chunk-table upload), the roofline of the dominant kernel (the
mixed update) from HIP events recorded on the launch stream, the same-mix
ceilings measured by bench_probe.hip, and the CPU oracle timed on a bounded
sample on the host cores (one thread, and one thread per range on all cores).

Usage:
  python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--no-cpu] [--no-probe] [--compare]
  python bench.py --workload ragged_10k                  (overflow check + fp16 step, 10k tensors)
  python bench.py --probe-only                            (memory ceilings only)
  python bench.py --launch-study --steps 200              (the smaller workloads: eager calls in both
                                                           launch forms against HIP-graph replays)
  python bench.py --build-probe                           (compile the ceiling probes; no GPU)
  python bench.py --calib-copy                            (plain 4 GiB copy, to scale rocprofv3 byte counters)
  python bench.py --traffic-from F.csv W.csv CF.csv CW.csv (rocprofv3 counters -> profiles/traffic_<workload>.json)
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published peak
PROBE_SRC = os.path.join(ROOT, "bench_probe.hip")
PROBE_LIB = os.path.join(ROOT, "libbench_probe.so")
BYTES = {"mixed": 28, "kahan": 18, "split": 26, "f16amp": 28, "check": 2}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="opt_1_3b")
    ap.add_argument("--modes", default=None,
                    help="comma list of mixed, kahan, split, pure-<m>-<v>-<k|n>, f16amp, each optionally -blocked")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-probe", action="store_true", help="skip the same-mix ceiling probes")
    ap.add_argument("--compare", action="store_true",
                    help="after a blocked-state headline, also time the same steps on per-tensor state "
                         "(per_tensor_state); off by default, so that each update kernel in a profile of the "
                         "default run serves the headline layout only")
    ap.add_argument("--no-compare", action="store_true", help="the default (no per-tensor-state timing)")
    ap.add_argument("--probe-only", action="store_true")
    ap.add_argument("--launch-study", action="store_true",
                    help="per-step cost of the 1M tensor, the BERT rank-0 shard and OPT-125m as eager calls "
                         "(single-launch and two-launch forms) and as HIP-graph replays")
    ap.add_argument("--build-probe", action="store_true", help="compile bench_probe.hip and exit (no GPU needed)")
    ap.add_argument("--cpu-sample", type=int, default=256_000_000,
                    help="elements of the list the oracle steps once per mode")
    ap.add_argument("--calib-copy", action="store_true")
    ap.add_argument("--traffic-from", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "CAL_FETCH_CSV", "CAL_WRITE_CSV"),
                    help="write profiles/traffic_<workload>.json from rocprofv3 --pmc counter_collection.csv files "
                         "(FETCH_SIZE and WRITE_SIZE over this bench, then over --calib-copy); needs no GPU")
    ap.add_argument("--chunk-elems", type=int, default=0)
    ap.add_argument("--interleave", action="store_true",
                    help="alternate the modes every step instead of timing them as consecutive phases")
    return ap.parse_args()


def calib_copy():
    """A plain copy of 4 GiB, three times: FETCH_SIZE / WRITE_SIZE of this kernel
    against the known 4 GiB per direction give the counters' scale."""
    import torch
    n = CALIB_COPY_BYTES // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calib_copy_bytes_each_way": n * 4, "launches": 3}), flush=True)


CALIB_COPY_BYTES = 4 << 30
# the timed kernel of each mode, as a prefix of its name in rocprofv3 output (the
# last template argument, the launch form, is left open)
KERNEL_OF = {"mixed": "update_kernel<0,", "split": "update_pure_kernel<true, true, 2,",
             "kahan": "update_pure_kernel<false, false, 1,", "f16amp": "update_kernel<1,",
             "check": "check_kernel"}


def _pmc_rows(path, counter, kernel):
    import csv
    with open(path) as f:
        return [r for r in csv.DictReader(f) if r["Counter_Name"] == counter and kernel in r["Kernel_Name"]]


def _pmc_values(path, counter, kernel):
    return [float(r["Counter_Value"]) for r in _pmc_rows(path, counter, kernel)]


def _kernel_name(path, counter, kernel):
    """The full kernel name (without its argument list) matched by `kernel`."""
    names = {r["Kernel_Name"].split("(")[0].replace("void ", "") for r in _pmc_rows(path, counter, kernel)}
    return " / ".join(sorted(names))


def write_traffic(wl_name, modes, fetch_csv, write_csv, cal_fetch_csv, cal_write_csv):
    """HBM bytes per launch of each timed kernel from two rocprofv3 --pmc passes
    (FETCH_SIZE, WRITE_SIZE: KiB per dispatch) over a bench run of `modes`,
    each scaled by what the same counter reads for the plain copy of
    --calib-copy (CALIB_COPY_BYTES each way)."""
    import workloads
    n = workloads.get(wl_name).total
    kernels = {}
    for mode in modes:
        base = mode[:-len("-blocked")] if mode.endswith("-blocked") else mode
        kernels[mode] = KERNEL_OF[base]
        if base == "f16amp":
            kernels["check"] = KERNEL_OF["check"]
    if len(set(kernels.values())) != len(kernels):
        raise SystemExit("two of the modes launch the same kernel: profile them in separate runs")
    scale = {}
    for counter, path in (("FETCH_SIZE", cal_fetch_csv), ("WRITE_SIZE", cal_write_csv)):
        vals = _pmc_values(path, counter, "copyBuffer")
        if not vals:
            raise SystemExit(f"no copy dispatches with {counter} in {path}")
        scale[counter] = sum(vals) / len(vals) * 1024 / CALIB_COPY_BYTES
    traffic, alg, per_param, raw = {}, {}, {}, {}
    for mode, kernel in kernels.items():
        fv = _pmc_values(fetch_csv, "FETCH_SIZE", kernel)
        wv = _pmc_values(write_csv, "WRITE_SIZE", kernel)
        if not fv or not wv:
            continue
        rd = sum(fv) / len(fv) * 1024 / scale["FETCH_SIZE"]
        wr = sum(wv) / len(wv) * 1024 / scale["WRITE_SIZE"]
        traffic[mode] = round(rd + wr)
        alg[mode] = BYTES[mode[:-len("-blocked")] if mode.endswith("-blocked") else mode] * n
        per_param[mode] = {"read": round(rd / n, 4), "write": round(wr / n, 4)}
        raw[mode] = {"kernel": _kernel_name(fetch_csv, "FETCH_SIZE", kernel), "FETCH_SIZE_KiB": fv,
                     "WRITE_SIZE_KiB": wv}
    if not traffic:
        raise SystemExit("no timed kernel found in the counter files")
    out = {"about": f"HBM bytes per launch on the {wl_name} list from two rocprofv3 --pmc passes (FETCH_SIZE, "
                    "then WRITE_SIZE, KiB per dispatch), each scaled by what the same counter reads for a plain "
                    f"{CALIB_COPY_BYTES >> 30} GiB device copy (bench.py --calib-copy).",
           "kernel_source_sha": _kernel_sha(),
           "counter_scale": {k: round(v, 6) for k, v in scale.items()},
           "traffic_bytes_per_launch": traffic, "algorithmic_bytes_per_launch": alg,
           "per_param": per_param, "raw": raw}
    path = os.path.join(ROOT, "profiles", f"traffic_{wl_name}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps({"wrote": path, "per_param": per_param, "counter_scale": out["counter_scale"]}), flush=True)


def default_modes(args):
    """The modes one bench step runs: both modes of the OPT-1.3B list, or the
    fp16-AMP step on an fp16 workload, with their state in the blocked layout."""
    import workloads
    if args.modes:
        return args.modes
    # Blocked state in the padded flat index (every tensor at a multiple of 8),
    # so that the ragged fp16 list's arbitrary lengths keep the vector path.
    return "f16amp-blocked" if workloads.get(args.workload).p_dtype == "f16" else "mixed-blocked,kahan-blocked"


def _time_launches(fn, reps, stream):
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    fn()
    torch.cuda.synchronize()
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    return ms[len(ms) // 2]


def build_probe(verbose: bool = False) -> str:
    """Compiles the memory-ceiling probes (bench_probe.hip, measurement support of
    this benchmark and not part of the library) into libbench_probe.so with the
    library's hipcc flags."""
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "_adamw_amd_build", os.path.join(ROOT, "adamw_optimizer_step_apply_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    mod.hipcc([PROBE_SRC], PROBE_LIB, verbose)
    return PROBE_LIB


def probes(n, stream):
    """Same-mix ceilings at n elements (median of 7 launches each), in GB/s."""
    import torch
    if not os.path.exists(PROBE_LIB):
        raise SystemExit(f"{PROBE_LIB} is missing: build it first (python bench.py --build-probe, "
                         "or __graft_entry__.build())")
    lib = ctypes.CDLL(PROBE_LIB)
    lib.probe_launch.restype = ctypes.c_int
    lib.probe_launch.argtypes = [ctypes.c_int] + [ctypes.c_void_p] * 5 + [ctypes.c_uint64, ctypes.c_void_p]
    n = n // 8 * 8
    s = stream.cuda_stream
    out = {}

    def run(kind, bufs, count, nbytes, name):
        ptrs = [b.data_ptr() for b in bufs] + [0] * (5 - len(bufs))

        def f():
            rc = lib.probe_launch(kind, *ptrs, count, s)
            if rc:
                raise RuntimeError(f"probe launch failed: {rc}")
        ms = _time_launches(f, 7, stream)
        out[name] = round(nbytes / (ms * 1e-3) / 1e9, 1)

    dev = "cuda"
    g = torch.ones(n, dtype=torch.bfloat16, device=dev)
    p = torch.ones(n, dtype=torch.bfloat16, device=dev)
    w, m, v = (torch.ones(n, dtype=torch.float32, device=dev) for _ in range(3))
    run(0, [g, w, m, v, p], n, 28 * n, "mixed_mix")
    del w, m, v
    # whole blocks of the blocked state layout: 16384 elements per block
    nb = -(-n // 16384)
    blk = torch.ones(nb * 16384 * 3, dtype=torch.float32, device=dev)
    run(6, [g, blk, p], n, 28 * n, "mixed_blocked_mix")
    del blk
    nb = -(-n // 16384)
    blk = torch.ones(nb * 16384 * 3, dtype=torch.bfloat16, device=dev)
    run(7, [g, p, blk], n, 18 * n, "kahan_blocked_mix")
    del blk
    r16 = torch.ones(n, dtype=torch.bfloat16, device=dev)
    m32, v32 = (torch.ones(n, dtype=torch.float32, device=dev) for _ in range(2))
    run(5, [g, p, r16, m32, v32], n, 26 * n, "split_mix")
    del m32, v32
    m16, v16, c16 = (torch.ones(n, dtype=torch.bfloat16, device=dev) for _ in range(3))
    run(1, [g, p, m16, v16, c16], n, 18 * n, "kahan_mix")
    del g, p, m16, v16, c16
    f = 1 << 31                                   # 8 GiB of fp32
    src = torch.ones(f, dtype=torch.float32, device=dev)
    dst = torch.zeros_like(src)
    run(2, [src, dst], f, 8 * f, "copy")
    run(3, [src, dst], f, 4 * f, "read")
    run(4, [dst], f, 4 * f, "write")
    # the same in the update kernels' shape (8 workgroups per chunk, 1 KiB tiles), 2 per CU,
    # four 16-byte words in flight per lane
    run(8, [src, dst], f, 8 * f, "copy_wide")
    run(9, [src, dst], f, 4 * f, "read_wide")
    run(10, [dst], f, 4 * f, "write_wide")
    del src, dst
    torch.cuda.empty_cache()
    return out


STATE_BLOCK_ELEMS = 16384     # elements per block of the blocked state layout (ADAMW_STATE_BLOCK_ELEMS)
BLOCKED_FLAGS = (1 << 8) | (1 << 9)   # ADAMW_BLOCKED_STATE | ADAMW_FLAT_PAD8


def state_layout(mode, numels):
    """How make_mode_state lays out a mode's buffers, apart from their base
    addresses: (arena alignment in elements of the per-tensor buffers, the
    list's flat_mask, blocks of the blocked state buffer or 0).  A "-blocked"
    mode keeps every tensor at a multiple of 8 elements in its arenas, so that a
    state arena is already the padded flat concatenation (the same offsets as
    128 when all lengths are multiples of 128, as in the OPT and BERT lists)."""
    if not mode.endswith("-blocked"):
        return 128, 0, 0
    n = sum(-(-int(m) // 8) * 8 for m in numels)     # padded flat index
    return 8, BLOCKED_FLAGS, -(-n // STATE_BLOCK_ELEMS)


def make_mode_state(mode, numels, device, seed, p_dtype="bf16", loss_scale=1.0):
    """Per-tensor buffers for every stream; a "-blocked" mode instead keeps
    exp_avg / exp_avg_sq / aux in one blocked flat buffer of the whole list
    (the optimizer-owned layout; param and grad stay per tensor), indexed by
    the padded flat index (every tensor at a multiple of 8 elements), filled
    from the per-tensor state by the library's layout copy (make_blocked_state).
    Returns (arena, streams, flat_mask)."""
    import workloads
    base = mode[:-len("-blocked")] if mode.endswith("-blocked") else mode
    align, flags, nb = state_layout(mode, numels)
    arena = workloads.make_state(base, numels, device, seed, align_elems=align, p_dtype=p_dtype,
                                 loss_scale=loss_scale)
    keys = workloads.streams_of(base)
    streams = [[arena.view(k, i) for i in range(len(numels))] for k in keys]
    if nb:
        import adamw_optimizer_step_apply_amd as A
        if base.startswith("pure"):
            m32, v32, kahan = workloads.parse_pure(base)
            code, prec = A.MIXED, A.PurePrecision(A.F32 if m32 else A.BF16, A.F32 if v32 else A.BF16, kahan)
        else:
            code, prec = {"mixed": A.MIXED, "kahan": A.PURE_KAHAN, "split": A.MIXED_SPLIT}[base], None
        dt = A.F16 if p_dtype == "f16" else A.BF16
        state = streams[2:] + [None] * (5 - len(streams))
        blocked, mask = A.make_blocked_state(code, dt, numels, *state, prec=prec)
        assert mask == flags and blocked.numel() == nb * STATE_BLOCK_ELEMS * sum(
            arena.bufs[k].element_size() for k in keys[2:])
        for k in keys[2:]:
            del arena.bufs[k]
        arena.bufs["blocked"] = blocked
        streams = streams[:2] + [[blocked], None, None]
    return arena, streams, flags


# (workload, mode, ZeRO rank or None): the smaller parity workloads in their own modes
LAUNCH_STUDY = (("single_1m", "mixed", None), ("bert_52m", "mixed", 0), ("opt_125m", "kahan", None),
                ("opt_125m", "kahan-blocked", None), ("opt_125m", "mixed-blocked", None))


def launch_study(K, dev):
    """Steps of one to a hundred million parameters last microseconds to a few
    hundred, so the host's cost per call and the prologue launch weigh.  For
    each workload of LAUNCH_STUDY, the per-step time of K calls issued back to
    back (the host's loop included, wall clock over all K) in the two-launch
    form (prologue kernel + update kernel) and in the single-launch form (the
    default for plans of at most 512 chunks, 4,096 workgroups; forced here at
    every size), the GPU time of one call (HIP events around each call on its
    stream), and the per-step time of HIP graphs holding 1 and 10 captured
    steps in the default form, replayed back to back."""
    import torch

    import adamw_optimizer_step_apply_amd as A
    import workloads
    stream = torch.cuda.Stream(dev)             # capture needs a stream other than the legacy default
    hp = A.HParams()
    rows = []
    for wname, mode, rank in LAUNCH_STUDY:
        wl = workloads.get(wname)
        numels = wl.numels
        b, e = wl.shard(rank) if rank is not None else (0, wl.total)
        with torch.cuda.stream(stream):
            arena, streams, flags = make_mode_state(mode, numels, dev, seed=300)
        torch.cuda.synchronize()
        tl = A.TensorList(numels, streams, b, e if rank is not None else -1, flags)
        base = mode[:-len("-blocked")] if mode.endswith("-blocked") else mode
        code = {"mixed": A.MIXED, "kahan": A.PURE_KAHAN}[base]
        ctr = torch.zeros(1, dtype=torch.int32, device=dev)
        s = stream.cuda_stream

        def call():
            A.adamw_multi_tensor_step(code, A.BF16, tl, hp, ctr, None, s)

        def eager():
            call()                                       # plan cached before the timed loops
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(K):
                call()
            torch.cuda.synchronize()
            wall = (time.perf_counter() - t0) / K
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
            for a, c in ev:
                a.record(stream)
                call()
                c.record(stream)
            torch.cuda.synchronize()
            gpu = sorted(a.elapsed_time(c) for a, c in ev)[K // 2] * 1e-3
            return wall, gpu

        def graphed(per_graph):
            call()
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for _ in range(per_graph):
                    call()
            torch.cuda.synchronize()
            reps = max(1, K // per_graph)
            g.replay()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(reps):
                g.replay()
            torch.cuda.synchronize()
            wall = (time.perf_counter() - t0) / (reps * per_graph)
            del g
            return wall

        chunks = len(A.adamw_plan_inspect(code, A.BF16, tl))
        forms = {}
        for form, knob in (("two_launch", 0), ("single_launch", 1 << 40)):
            A.adamw_set_single_launch_max_workgroups(knob)
            try:
                forms[form] = eager()
            finally:
                A.adamw_set_single_launch_max_workgroups(-1)
        g1, g10 = graphed(1), graphed(10)
        n = e - b
        nbytes = n * BYTES[base]

        def rate(t):
            return {"us": round(t * 1e6, 2), "gb_s": round(nbytes / t / 1e9, 1),
                    "frac_of_hbm_peak": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4)}
        rows.append({"workload": wname + (f" rank {rank} of {wl.dp_size}" if rank is not None else ""),
                     "mode": mode, "elements": n, "bytes_per_step": nbytes,
                     "chunks": chunks,
                     "default_form": "single_launch" if 8 * chunks <= 4096 else "two_launch",
                     **{f: {"eager_wall": rate(w_), "gpu_per_call": rate(g_)} for f, (w_, g_) in forms.items()},
                     "graph_1_step": rate(g1), "graph_10_steps": rate(g10)})
        del arena, streams, tl
        torch.cuda.empty_cache()
    return {"study": "launch", "steps": K, "rows": rows, "device": torch.cuda.get_device_name(dev)}


def cpu_baseline(numels, sample, modes):
    """The oracle as it is, one step per mode over the first `sample` elements
    of the list, scaled to param-updates/s of the bench step: on one host
    thread (value), and with the sample cut into equal ranges stepped by one
    host thread each (all_cores; the oracle's C loops release the GIL)."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    import torch

    import oracle
    import workloads
    modes = [m[:-len("-blocked")] if m.endswith("-blocked") else m for m in modes]
    n = min(sample, sum(numels))
    threads = max(1, min(len(os.sched_getaffinity(0)), 16))
    hp = oracle.HParams()
    w = workloads.normal(n, workloads.INIT_STD, "cpu", "master", 7).numpy()
    f16 = "f16amp" in modes
    if f16:
        g = workloads.grads(n, "cpu", 7, 0, dtype=torch.float16, scale=65536.0).view(torch.int16).numpy().view(np.uint16)
        hp = oracle.HParams(inv_scale=1.0 / 65536)
    else:
        g = workloads.grads(n, "cpu", 7, 0, dtype=torch.bfloat16).view(torch.int16).numpy().view(np.uint16)

    def zeros(dt):
        return np.full(n, 0, dt)       # written now, so no first-touch page faults land in the timed call

    def state(mode):
        if mode in ("mixed", "f16amp"):
            return (zeros(np.uint16), g, w.copy(), zeros(np.float32), zeros(np.float32))
        if mode == "split":
            ps, rs = oracle.split_make(w)
            return (ps, g, rs, zeros(np.float32), zeros(np.float32))
        return (oracle.f32_to_bf16(w), g, zeros(np.uint16), zeros(np.uint16), zeros(np.uint16))

    def step(mode, bufs, lo, hi):
        s = [x[lo:hi] for x in bufs]
        if mode == "f16amp":
            assert not oracle.any_nonfinite(s[1], True)
            oracle.adamw_mixed(s[0], s[1], s[2], s[3], s[4], hp, 1, p_is_f16=True)
        elif mode == "mixed":
            oracle.adamw_mixed(s[0], s[1], s[2], s[3], s[4], hp, 1)
        elif mode == "split":
            oracle.adamw_mixed_split(s[0], s[1], s[2], s[3], s[4], hp, 1)
        else:
            oracle.adamw_kahan(s[0], s[1], s[3], s[4], s[2], hp, 1)

    secs, secs_mt = {}, {}
    cuts = [n * i // threads for i in range(threads + 1)]
    with ThreadPoolExecutor(threads) as pool:
        for mode in [m for m in ("f16amp", "mixed", "split", "kahan") if m in modes]:
            bufs = state(mode)
            t0 = time.perf_counter()
            step(mode, bufs, 0, n)
            secs[mode] = time.perf_counter() - t0
            bufs = state(mode)
            t0 = time.perf_counter()
            list(pool.map(lambda i: step(mode, bufs, cuts[i], cuts[i + 1]), range(threads)))
            secs_mt[mode] = time.perf_counter() - t0
            del bufs

    def rate(d):
        return round(len(d) / sum(s / n for s in d.values()) / 1e9, 4)
    return {"value": rate(secs), "unit": "Gparam/s", "cores": 1, "kind": "oracle",
            "sample": f"one step per mode ({', '.join(secs)}) over the first {n:,} parameters of the list, "
                      f"host-resident, 1 thread: " + " + ".join(f"{s:.2f} s" for s in secs.values()),
            "all_cores": {"value": rate(secs_mt), "unit": "Gparam/s", "cores": threads,
                          "sample": f"the same, cut into {threads} ranges on {threads} threads: "
                                    + " + ".join(f"{s:.2f} s" for s in secs_mt.values())},
            "host_cpus": os.cpu_count(), "host_cpu_model": _cpu_model()}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _per_mode(modes, ev, K, N, first_ms):
    per_mode = {}
    for mode in modes:
        if mode.startswith("f16amp"):
            chk = [a.elapsed_time(b) for a, b, _ in ev[mode]]
            upd = [b.elapsed_time(c) for _, b, c in ev[mode]]
            c_avg = sum(chk) / K
            per_mode["check" + mode[len("f16amp"):]] = {"ms_avg": round(c_avg, 4), "gb_s": round(N * 2 / (c_avg * 1e-3) / 1e9, 1),
                                 "frac_of_hbm_peak": round(N * 2 / (c_avg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                 "bytes_per_param": 2}
            ms = upd
        else:
            ms = [a.elapsed_time(c) for a, _, c in ev[mode]]
        avg = sum(ms) / len(ms)
        key = mode + "_step" if mode.startswith("f16amp") else mode
        per_mode[key] = {
            "ms_avg": round(avg, 4), "ms_median": round(sorted(ms)[len(ms) // 2], 4), "ms_min": round(min(ms), 4),
            "gparam_s": round(N / (avg * 1e-3) / 1e9, 2),
            "gb_s": round(N * BYTES[mode] / (avg * 1e-3) / 1e9, 1),
            "frac_of_hbm_peak": round(N * BYTES[mode] / (avg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "bytes_per_param": BYTES[mode],
            "first_call_ms": round(first_ms[mode], 3),
        }
    return per_mode


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the step runs on one rank's share; runs on "
              f"{args.gpus} GPUs are not supported.", file=sys.stderr)
        sys.exit(2)
    if args.build_probe:
        print(build_probe(verbose=True))
        return
    if args.traffic_from:
        write_traffic(args.workload, default_modes(args).split(","), *args.traffic_from)
        return
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
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    if args.probe_only:
        print(json.dumps({"probes_gb_s": probes(N, stream), "n": N}), flush=True)
        return
    if args.launch_study:
        print(json.dumps(launch_study(args.steps, dev)), flush=True)
        return
    modes = default_modes(args).split(",")
    # with --compare, the same steps on per-tensor state buffers, timed after the headline region
    compare = [m[:-len("-blocked")] for m in modes if m.endswith("-blocked")] if args.compare and not args.no_compare \
        else []
    for mode in modes + compare:
        base = mode[:-len("-blocked")] if mode.endswith("-blocked") else mode
        if base.startswith("pure"):
            BYTES[mode] = workloads.pure_traffic(base)
        elif base != mode:
            BYTES[mode] = BYTES[base]

    state = {}
    for i, mode in enumerate(modes + compare):
        if mode.startswith("f16amp"):
            arena, streams, flags = make_mode_state("mixed" + mode[len("f16amp"):], numels, dev, 100 + i,
                                                    p_dtype="f16", loss_scale=wl.loss_scale)
        else:
            arena, streams, flags = make_mode_state(mode, numels, dev, seed=100 + i)
        assert A.STATE_BLOCK_ELEMS == STATE_BLOCK_ELEMS and A.BLOCKED_STATE | A.FLAT_PAD8 == BLOCKED_FLAGS
        state[mode] = (arena, A.TensorList(numels, streams, 0, -1, flags), torch.zeros(1, dtype=torch.int32, device=dev))
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    hp = A.HParams()
    # fp16 AMP keeps its loss scale on the device (growth 2, back-off 0.5, every 2000 clean steps)
    scale_state = A.loss_scale_state(wl.loss_scale)
    scaler = A.LossScaler(2.0, 0.5, 2000)

    def one(mode, ev=None):
        _, tl, ctr = state[mode]
        if mode.startswith("f16amp"):
            if ev:
                ev[0].record(stream)
            A.adamw_check_finite(A.F16, tl, flag, stream)
            if ev:
                ev[1].record(stream)
            A.adamw_multi_tensor_step_amp(A.MIXED, A.F16, tl, hp, ctr, flag, scale_state, scaler, stream)
            if ev:
                ev[2].record(stream)
            return
        if ev:
            ev[0].record(stream)
        base = mode[:-len("-blocked")] if mode.endswith("-blocked") else mode
        if base.startswith("pure"):
            m32, v32, kahan = workloads.parse_pure(base)
            prec = A.PurePrecision(A.F32 if m32 else A.BF16, A.F32 if v32 else A.BF16, kahan)
            A.adamw_pure_multi_tensor_step(prec, tl, hp, ctr, None, stream)
        else:
            code = {"mixed": A.MIXED, "kahan": A.PURE_KAHAN, "split": A.MIXED_SPLIT}[base]
            A.adamw_multi_tensor_step(code, A.BF16, tl, hp, ctr, None, stream)
        if ev:
            ev[2].record(stream)

    # the first call of each mode builds its plan and uploads the chunk table
    first_ms = {}
    for mode in modes + compare:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        one(mode)
        torch.cuda.synchronize()
        first_ms[mode] = (time.perf_counter() - t0) * 1e3
    for _ in range(args.warmup - 1):
        for mode in modes + compare:
            one(mode)
    torch.cuda.synchronize()

    # Timed region: K steps of every mode.  By default the modes run as
    # consecutive phases (K mixed steps, then K Kahan steps): they are separate
    # training configurations, and a real loop runs one of them.  --interleave
    # alternates them every step instead.
    K = args.steps

    def timed(ms_):
        ev = {m: [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(K)] for m in ms_}
        order = [(s, m) for s in range(K) for m in ms_] if args.interleave else [(s, m) for m in ms_ for s in range(K)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s, mode in order:
            one(mode, ev[mode][s])
        torch.cuda.synchronize()
        return ev, time.perf_counter() - t0

    ev, wall = timed(modes)
    per_mode = _per_mode(modes, ev, K, N, first_ms)
    if compare:
        ev_c, _ = timed(compare)
        per_tensor = _per_mode(compare, ev_c, K, N, first_ms)
    ms_step = wall / K * 1e3
    value = len(modes) * N / (wall / K) / 1e9
    dom = modes[0]
    dom_key = dom + "_step" if dom.startswith("f16amp") else dom
    achieved = per_mode[dom_key]["gb_s"]
    traffic = None
    tpath = os.path.join(ROOT, "profiles", f"traffic_{wl.name}.json")
    if os.path.exists(tpath):
        with open(tpath) as f:
            t = json.load(f)
        if t.get("kernel_source_sha") == _kernel_sha():
            traffic = t.get("traffic_bytes_per_launch", {}).get(dom)
    names = {"mixed": "mixed (bf16 p/g + fp32 master/m/v)", "kahan": "pure bf16 + bf16 Kahan compensation",
             "split": "mixed with the master split into bf16 param + int16 remainder",
             "f16amp": "fp16-AMP overflow check + mixed fp16 step with a device-resident dynamic loss scale "
                       "(65536 to start)"}
    for mode in modes:
        base = mode[:-len("-blocked")] if mode.endswith("-blocked") else mode
        if base.startswith("pure") and base not in names:
            m32, v32, kahan = workloads.parse_pure(base)
            names[base] = (f"pure bf16 params, {'fp32' if m32 else 'bf16'} exp_avg, {'fp32' if v32 else 'bf16'} "
                           f"exp_avg_sq, {('no', 'bf16 Kahan', 'fp32 Kahan')[kahan]} compensation")
        if base != mode:
            names[mode] = (names[base] + f", exp_avg/exp_avg_sq/{'master' if base == 'mixed' else 'aux'} "
                           "interleaved per block of 16384 elements of one optimizer-owned buffer")
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
                               + " then ".join(names[m] for m in modes)
                               + (" (modes alternated every step)" if args.interleave else
                                  " (timed as consecutive phases of K steps each)"),
                   "n_params": N, "n_tensors": len(numels), "modes": modes,
                   "hparams": {"lr": hp.lr, "beta1": hp.beta1, "beta2": hp.beta2, "eps": hp.eps,
                               "weight_decay": hp.weight_decay}},
        "per_mode": per_mode,
        **({"per_tensor_state": per_tensor} if compare else {}),
        "roofline": {"bound": "hbm", "kernel": f"update_kernel ({dom})", "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic},
        "device": torch.cuda.get_device_name(dev),
        "device_arch": getattr(torch.cuda.get_device_properties(dev), "gcnArchName", None),
        "hip_runtime": torch.version.hip,
    }
    if not args.no_probe:
        del state
        torch.cuda.empty_cache()
        pr = probes(N, stream)
        out["ceilings_gb_s"] = pr
        probe_of = {"mixed": "mixed_mix", "kahan": "kahan_mix", "f16amp_step": "mixed_mix", "split": "split_mix",
                    "mixed-blocked": "mixed_blocked_mix", "kahan-blocked": "kahan_blocked_mix",
                    "f16amp-blocked_step": "mixed_blocked_mix"}
        for table in (per_mode, per_tensor if compare else {}):
            for mode, row in table.items():
                key = probe_of.get(mode)
                if key:
                    row["frac_of_same_mix_probe"] = round(row["gb_s"] / pr[key], 4)
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(numels, args.cpu_sample, modes)
    print(json.dumps(out), flush=True)


def _kernel_sha():
    """Hash of the code that decides a launch's HBM traffic (kernels, planner,
    layout constants, and the header's #define lines but its version), comments and blank lines
    left out, so that a recorded counter summary stays valid across edits of the
    documentation and of declarations alone."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in ("adamw_optimizer_step_apply_amd/csrc/kernels.hip", "adamw_optimizer_step_apply_amd/csrc/plan.cpp",
              "adamw_optimizer_step_apply_amd/csrc/layout.hpp", "include/adamw.h"):
        with open(os.path.join(ROOT, f)) as fh:
            src = fh.read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        src = re.sub(r"//[^\n]*", "", src)
        lines = [ln.rstrip() for ln in src.splitlines() if ln.strip()]
        if f.endswith(".h"):    # the header's constants, its version number aside
            lines = [ln for ln in lines if ln.lstrip().startswith("#define") and "ADAMW_ABI_VERSION" not in ln]
        h.update("\n".join(lines).encode())
    return h.hexdigest()[:16]


if __name__ == "__main__":
    main()
