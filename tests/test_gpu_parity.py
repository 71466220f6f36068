"""GPU parity: the HIP library against the CPU oracle, element by element, on
seeded inputs small enough for the oracle to finish in seconds yet spanning
many workgroup chunks, peeled heads and ragged tails.  See gpu_util for the bar.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import Case, compare, free, hp_pair, join_master, same_bits, to_np

import adamw_optimizer_step_apply_amd as A

pytestmark = pytest.mark.gpu

EDGE_SIZES = [0, 1, 7, 8, 9, 15, 16, 17, 2047, 2048, 2049, 16383, 16384, 16385, 100_003, 3, 40_000]


def _run(case: Case, steps: int, hp_kw=None, label=""):
    hg, ho = hp_pair(**(hp_kw or {}))
    for s in range(steps):
        if s:
            case.refill_grads(s)
        case.gpu_step(hg)
        case.oracle_step(ho)
    stats = case.compare_all(label)
    print(label, stats, flush=True)
    return stats


def test_single_tensor_1m_mixed_10_steps():
    """One flat tensor of 1,048,576 elements, mixed bf16/fp32, 10 steps with a
    fresh seeded gradient each step (the single-tensor workload)."""
    case = Case("mixed", [1 << 20], seed=101)
    stats = _run(case, 10, label="single_1m")
    assert all(s["bit_mismatches"] == 0 for s in stats)
    free()


@pytest.mark.parametrize("align", [128, 1, 3])
@pytest.mark.parametrize("mode,p_dtype", [("mixed", "bf16"), ("mixed", "f16"), ("kahan", "bf16"),
                                          ("split", "bf16")])
def test_edge_sizes(mode, p_dtype, align):
    """Sizes around the 8-element pack and the chunk size, packed at several
    alignments (align=1 or 3 puts most tensors off a 16-byte boundary)."""
    scale = 65536.0 if p_dtype == "f16" else 1.0
    case = Case(mode, EDGE_SIZES, seed=202 + align, p_dtype=p_dtype, align_elems=align, loss_scale=scale,
                random_moments=True)
    _run(case, 4, hp_kw={"inv_scale": 1.0 / scale}, label=f"edges-{mode}-{p_dtype}-a{align}")
    free()


@pytest.mark.parametrize("shifts", [{"g": 1}, {"master": 1}, {"p": 3, "g": 3, "m": 2, "v": 2, "master": 2},
                                    {"m": 1, "v": 3}, {"g": 8}])
def test_streams_at_different_phases(shifts):
    """Streams whose tensors start at different 16-byte phases: either a common
    head peel exists or the planner falls back to element chunks."""
    case = Case("mixed", EDGE_SIZES, seed=303, shifts=shifts, random_moments=True)
    _run(case, 3, label=f"shift-{shifts}")
    free()


def test_kahan_phases():
    case = Case("kahan", EDGE_SIZES, seed=304, shifts={"c": 1, "p": 5}, random_moments=True)
    _run(case, 3, label="kahan-shift")
    free()


@pytest.mark.parametrize("hp_kw", [dict(eps=1e-3), dict(lr=1e-2, weight_decay=0.5),
                                   dict(beta1=0.0, beta2=0.0), dict(beta1=0.5, beta2=0.75, weight_decay=0.0),
                                   dict(lr=0.0, weight_decay=0.0)],
                         ids=["eps", "strong-decay", "beta0", "betas", "lr0"])
@pytest.mark.parametrize("mode", ["mixed", "kahan", "split"])
def test_hyperparameter_variants(mode, hp_kw):
    case = Case(mode, [5000, 33, 20000], seed=404, random_moments=True)
    _run(case, 3, hp_kw=hp_kw, label=f"hp-{mode}-{hp_kw}")
    free()


def test_zero_shard_union_equals_full_step():
    """Four ranks, each stepping its 1/4 shard of the flat list with its own
    step counter, leave the same state as one full-list step (the single-GPU
    form of the pages' ZeRO on/off comparison), and both match the oracle."""
    numels = [1000, 12345, 7, 50000, 16, 4099]
    total = sum(numels)
    full = Case("mixed", numels, seed=505)
    parts = Case("mixed", numels, seed=505)
    hg, ho = hp_pair()
    full.gpu_step(hg)
    full.oracle_step(ho)
    counters = []
    for r in range(4):
        b, e = r * total // 4, (r + 1) * total // 4
        ctr = torch.zeros(1, dtype=torch.int32, device="cuda")
        A.adamw_multi_tensor_step(A.MIXED, A.BF16, parts.tensor_list(b, e), hg, ctr)
        counters.append(ctr)
    torch.cuda.synchronize()
    assert [int(c.item()) for c in counters] == [1, 1, 1, 1]
    for k in parts.keys:
        assert same_bits(parts.arena.bufs[k], full.arena.bufs[k]), k
    full.compare_all("union-full")
    free()


@pytest.mark.parametrize("rank", [0, 1, 2, 3])
def test_zero_shard_vs_oracle(rank):
    """One rank's shard for 3 steps: elements outside the shard stay untouched."""
    numels = [3000, 777, 9, 65536 + 5, 128]
    total = sum(numels)
    b, e = rank * total // 4, (rank + 1) * total // 4
    case = Case("mixed", numels, seed=606, random_moments=True)
    hg, ho = hp_pair()
    for s in range(3):
        if s:
            case.refill_grads(s)
        case.gpu_step(hg, shard=(b, e))
        case.oracle_step(ho, shard=(b, e))
    case.compare_all(f"shard-r{rank}")
    free()


def test_flat_shard_buffers():
    """Gradient, master, m and v as one flat buffer of the rank's shard (a
    reduce-scattered gradient and ZeRO-sharded state), params per tensor."""
    numels = [4000, 1500, 8, 30000, 77]
    total = sum(numels)
    b, e = total // 4, 3 * total // 4
    ref = Case("mixed", numels, seed=707, align_elems=1, random_moments=True)
    flat = Case("mixed", numels, seed=707, align_elems=1, random_moments=True)
    hg, _ = hp_pair()
    # packed tight (align 1): the flat shard of a stream is a plain slice of its arena
    shard = {k: flat.arena.bufs[k][b:e].clone() for k in ("g", "m", "v", "master")}
    streams = [[flat.arena.view("p", i) for i in range(len(numels))],
               [shard["g"]], [shard["m"]], [shard["v"]], [shard["master"]]]
    tl = A.TensorList(numels, streams, b, e, flat_mask=0b11110)
    A.adamw_multi_tensor_step(A.MIXED, A.BF16, tl, hg, flat.d_step)
    ref.gpu_step(hg, shard=(b, e))
    torch.cuda.synchronize()
    assert same_bits(flat.arena.bufs["p"], ref.arena.bufs["p"])
    for k in ("m", "v", "master"):
        assert same_bits(shard[k], ref.arena.bufs[k][b:e]), k
    free()


def test_skip_flag_leaves_everything_unchanged():
    case = Case("mixed", EDGE_SIZES, seed=808, random_moments=True)
    hg, ho = hp_pair()
    case.gpu_step(hg)
    case.oracle_step(ho)
    before = {k: v.clone() for k, v in case.arena.bufs.items()}
    flag = torch.ones(1, dtype=torch.int32, device="cuda")
    case.refill_grads(1)
    before["g"] = case.arena.bufs["g"].clone()
    case.gpu_step(hg, found_inf=flag)
    torch.cuda.synchronize()
    assert int(case.d_step.item()) == 1
    for k, v in before.items():
        assert same_bits(case.arena.bufs[k], v), k
    flag.zero_()
    case.gpu_step(hg, found_inf=flag)
    case.oracle_step(ho)
    case.compare_all("after-skip")
    assert case.step == 2
    free()


@pytest.mark.parametrize("g_dtype", ["f16", "bf16"])
@pytest.mark.parametrize("bad", ["inf", "-inf", "nan"])
def test_check_finite_and_skip(g_dtype, bad):
    """fp16-AMP: the check kernel flags an inf/NaN planted at a seeded tensor and
    element; the following step is skipped; a clean gradient is not flagged."""
    scale = 65536.0 if g_dtype == "f16" else 1.0
    mode = "mixed"
    case = Case(mode, EDGE_SIZES, seed=909, p_dtype=g_dtype, loss_scale=scale, align_elems=3)
    tl = case.tensor_list()
    flag = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    A.adamw_check_finite(A.F16 if g_dtype == "f16" else A.BF16, tl, flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    rng = np.random.default_rng(11)
    for trial in range(6):
        i = int(rng.choice([j for j, n in enumerate(EDGE_SIZES) if n]))
        j = int(rng.integers(0, EDGE_SIZES[i]))
        view = case.arena.view("g", i)
        old = view[j].clone()
        view[j] = float(bad)
        A.adamw_check_finite(A.F16 if g_dtype == "f16" else A.BF16, tl, flag)
        torch.cuda.synchronize()
        assert int(flag.item()) == 1, (trial, i, j)
        host_g = to_np(case.arena.bufs["g"])
        assert oracle.any_nonfinite(host_g, g_dtype == "f16")
        before = {k: v.clone() for k, v in case.arena.bufs.items()}
        hg, _ = hp_pair(inv_scale=1.0 / scale)
        case.gpu_step(hg, tl=tl, found_inf=flag)
        torch.cuda.synchronize()
        assert int(case.d_step.item()) == 0
        for k, v in before.items():
            assert same_bits(case.arena.bufs[k], v), k
        view[j] = old
    A.adamw_check_finite(A.F16 if g_dtype == "f16" else A.BF16, tl, flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    free()


@pytest.mark.parametrize("g_dtype", ["f16", "bf16"])
def test_check_finite_all_patterns(g_dtype):
    """Every 16-bit pattern: the finite ones never raise the flag; each non-finite
    one raises it wherever it sits (vector or element chunk)."""
    is16 = g_dtype == "f16"
    allp = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    expo = 0x7C00 if is16 else 0x7F80
    finite = allp[(allp & expo) != expo]
    bad = allp[(allp & expo) == expo]
    dt = torch.float16 if is16 else torch.bfloat16
    base = torch.from_numpy(finite.view(np.int16).copy()).cuda()
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    buf = torch.zeros(finite.size + 16, dtype=torch.int16, device="cuda")
    buf[:finite.size] = base
    g = buf.view(dt)
    sizes = [1, 7, finite.size - 8]       # element chunk, element chunk, vector body + tail
    offs = [0, 1, 8]
    views = [g[o:o + n] for o, n in zip(offs, sizes)]
    tl = A.TensorList(sizes, [None, views, None, None, None])
    A.adamw_check_finite(A.F16 if is16 else A.BF16, tl, flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    rng = np.random.default_rng(12)
    positions = [0, 1, 5, 8, 9, 100, 2048 * 8 + 3, finite.size - 1]
    for pat in rng.choice(bad, size=min(64, bad.size), replace=False):
        pos = int(rng.choice(positions))
        old = int(buf[pos].item())
        buf[pos] = int(np.int16(np.uint16(pat).view(np.int16)))
        A.adamw_check_finite(A.F16 if is16 else A.BF16, tl, flag)
        torch.cuda.synchronize()
        assert int(flag.item()) == 1, hex(int(pat))
        buf[pos] = old
    free()


@pytest.mark.parametrize("p_dtype", ["bf16", "f16"])
def test_narrowing_through_the_kernel(p_dtype):
    """With lr = wd = 0 and g = 0 the master is unchanged and the 16-bit param is
    its nearest-even rounding: the kernel's conversion against the oracle's on
    4M random fp32 patterns plus rounding ties and range edges."""
    rng = np.random.default_rng(13)
    raw = rng.integers(0, 2 ** 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)
    x = raw.view(np.float32)
    x = x[np.isfinite(x)]
    ties = []
    for hi in rng.integers(0, 1 << 16, size=4000, dtype=np.uint32):
        for lo in (0x7FFF, 0x8000, 0x8001, 0x1000, 0x0FFF, 0x2000, 0x1FFF):
            ties.append((int(hi) << 16) | lo)
    t = np.array(ties, np.uint32).view(np.float32)
    sp = np.array([65504.0, 65519.99, 65520.0, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -14, 0.0, -0.0,
                   np.finfo(np.float32).max, np.finfo(np.float32).tiny, 1e-45], np.float32)
    w = np.concatenate([x, t[np.isfinite(t)], sp, -sp]).astype(np.float32)
    n = w.size
    dt = torch.float16 if p_dtype == "f16" else torch.bfloat16
    master = torch.from_numpy(w).cuda()
    p = torch.zeros(n, dtype=dt, device="cuda")
    g = torch.zeros(n, dtype=dt, device="cuda")
    m = torch.zeros(n, dtype=torch.float32, device="cuda")
    v = torch.zeros(n, dtype=torch.float32, device="cuda")
    step = torch.zeros(1, dtype=torch.int32, device="cuda")
    hg, ho = hp_pair(lr=0.0, weight_decay=0.0)
    A.adamw_step(A.MIXED, A.F16 if p_dtype == "f16" else A.BF16, n, p, g, m, v, master, hg, step)
    torch.cuda.synchronize()
    hm = w.copy()
    hp16 = np.zeros(n, np.uint16)
    oracle.adamw_mixed(hp16, np.zeros(n, np.uint16), hm, np.zeros(n, np.float32), np.zeros(n, np.float32),
                       ho, 1, p_is_f16=p_dtype == "f16")
    assert np.array_equal(to_np(master).view(np.uint32), w.view(np.uint32))
    got = to_np(p)
    assert np.array_equal(got, hp16), f"{np.count_nonzero(got != hp16)} conversions differ"
    free()


@pytest.mark.parametrize("p_dtype", ["bf16", "f16"])
def test_widening_through_the_kernel(p_dtype):
    """With beta1 = 0 the new first moment is the widened gradient: all 65,536
    16-bit patterns (inf and NaN included) through the vector and element paths."""
    allp = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    gbits = np.concatenate([allp, allp[:3]])          # 65539: vector body + a 3-element tail
    n = gbits.size
    dt = torch.float16 if p_dtype == "f16" else torch.bfloat16
    g = torch.from_numpy(gbits.view(np.int16).copy()).cuda().view(dt)
    p = torch.zeros(n, dtype=dt, device="cuda")
    m = torch.zeros(n, dtype=torch.float32, device="cuda")
    v = torch.zeros(n, dtype=torch.float32, device="cuda")
    w = torch.zeros(n, dtype=torch.float32, device="cuda")
    step = torch.zeros(1, dtype=torch.int32, device="cuda")
    hg, ho = hp_pair(beta1=0.0)
    A.adamw_step(A.MIXED, A.F16 if p_dtype == "f16" else A.BF16, n, p, g, m, v, w, hg, step)
    hs = {"p": np.zeros(n, np.uint16), "g": gbits.copy(), "m": np.zeros(n, np.float32),
          "v": np.zeros(n, np.float32), "master": np.zeros(n, np.float32)}
    oracle.adamw_mixed(hs["p"], hs["g"], hs["master"], hs["m"], hs["v"], ho, 1, p_is_f16=p_dtype == "f16")
    torch.cuda.synchronize()
    for k, t in (("m", m), ("v", v), ("master", w)):
        compare(f"widen-{k}", to_np(t), hs[k], True)
    compare("widen-p", to_np(p), hs["p"], False, p_dtype == "f16")
    free()


def test_resume_is_bitwise():
    """10 steps == 5 steps, copy every buffer and the counter to fresh memory, 5 more."""
    numels = [3000, 17, 40000]
    a = Case("kahan", numels, seed=1111, random_moments=True)
    b = Case("kahan", numels, seed=1111, random_moments=True)
    hg, _ = hp_pair()
    for s in range(10):
        if s:
            a.refill_grads(s)
        a.gpu_step(hg)
    for s in range(5):
        if s:
            b.refill_grads(s)
        b.gpu_step(hg)
    # "checkpoint": move everything to new allocations
    for k in list(b.arena.bufs):
        b.arena.bufs[k] = b.arena.bufs[k].clone()
    b.d_step = b.d_step.clone()
    for s in range(5, 10):
        b.refill_grads(s)
        b.gpu_step(hg)
    torch.cuda.synchronize()
    assert int(a.d_step.item()) == int(b.d_step.item()) == 10
    for k in a.keys:
        assert same_bits(a.arena.bufs[k], b.arena.bufs[k]), k
    free()


def test_side_streams_and_plan_cache():
    """Work on two non-default streams with alternating lists: each stream keeps
    its own workspace, and a list with new pointers is re-planned."""
    hg, ho = hp_pair()
    c1 = Case("mixed", [5000, 3], seed=1212)
    c2 = Case("mixed", [5000, 3], seed=1313)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    for it in range(3):
        for case, st in ((c1, s1), (c2, s2), (c2, s1), (c1, s2)):
            with torch.cuda.stream(st):
                case.gpu_step(hg)
            st.synchronize()
            case.oracle_step(ho)
    c1.compare_all("streams-c1")
    c2.compare_all("streams-c2")
    free()


def test_invalid_calls_enqueue_nothing():
    case = Case("mixed", [100, 200], seed=1414)
    before = {k: v.clone() for k, v in case.arena.bufs.items()}
    hg, _ = hp_pair()
    bad = [
        lambda: A.adamw_multi_tensor_step(A.MIXED, A.F32, case.tensor_list(), hg, case.d_step),
        lambda: A.adamw_multi_tensor_step(A.PURE_KAHAN, A.F16, case.tensor_list(), hg, case.d_step),
        lambda: A.adamw_multi_tensor_step(A.MIXED, A.BF16, case.tensor_list(0, 10_000), hg, case.d_step),
        lambda: A.adamw_multi_tensor_step(A.MIXED, A.BF16, case.tensor_list(), A.HParams(beta1=1.0), case.d_step),
        lambda: A.adamw_multi_tensor_step(A.MIXED, A.BF16, case.tensor_list(), A.HParams(eps=-1.0), case.d_step),
        lambda: A.adamw_multi_tensor_step(A.MIXED, A.BF16, case.tensor_list(), A.HParams(lr=float("nan")),
                                          case.d_step),
        lambda: A.adamw_multi_tensor_step(A.MIXED, A.BF16, case.tensor_list(), hg, None),
        lambda: A.adamw_step(A.MIXED, A.BF16, 100, case.arena.view("p", 0), None, case.arena.view("m", 0),
                             case.arena.view("v", 0), case.arena.view("master", 0), hg, case.d_step),
        lambda: A.adamw_step(A.MIXED, A.BF16, 100, case.arena.bufs["p"][1:].data_ptr() + 1, case.arena.bufs["g"],
                             case.arena.bufs["m"], case.arena.bufs["v"], case.arena.bufs["master"], hg, case.d_step),
    ]
    for f in bad:
        with pytest.raises(A.AdamWError):
            f()
    torch.cuda.synchronize()
    assert int(case.d_step.item()) == 0
    for k, v in before.items():
        assert same_bits(case.arena.bufs[k], v), k
    free()


def test_empty_list_advances_counter():
    step = torch.zeros(1, dtype=torch.int32, device="cuda")
    tl = A.TensorList([], [[], [], [], [], []])
    hg, _ = hp_pair()
    A.adamw_multi_tensor_step(A.MIXED, A.BF16, tl, hg, step)
    A.adamw_step(A.PURE_KAHAN, A.BF16, 0, None, None, None, None, None, hg, step)
    flag = torch.ones(1, dtype=torch.int32, device="cuda")
    A.adamw_multi_tensor_step(A.MIXED, A.BF16, tl, hg, step, flag)
    torch.cuda.synchronize()
    assert int(step.item()) == 2
    A.adamw_check_finite(A.F16, tl, flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0


def test_plan_cache_eviction_cycle():
    """More lists than the per-stream plan cache holds, cycled twice on one
    stream: every call must use its own list's table (evicted ones re-planned)."""
    hg, ho = hp_pair()
    cases = [Case("mixed" if i % 2 else "kahan", [3000 + 97 * i, 5 + i, 17000 - 31 * i], seed=1500 + i)
             for i in range(11)]
    for rnd in range(2):
        for c in cases:
            c.gpu_step(hg)
            c.oracle_step(ho)
    for i, c in enumerate(cases):
        c.compare_all(f"evict-{i}")
    free()


@pytest.mark.parametrize("mode", ["mixed", "kahan", "split", "pure-f32-bf16-k"])
def test_chunk_size_does_not_change_results(mode):
    """The same step at every legal kind of chunk size (the smallest, a middle
    one, one larger than most tensors, the largest) gives the default's bytes:
    the chunking decides only which workgroup does an element."""
    numels = [70001, 9, 4099, 2048, 300000, 17]
    ref = Case(mode, numels, seed=2700, align_elems=3, random_moments=True)
    hg, _ = hp_pair()
    ref.gpu_step(hg)
    try:
        for chunk in (2048, 6144, 262144, 1 << 22):
            c = Case(mode, numels, seed=2700, align_elems=3, random_moments=True)
            assert A.adamw_set_chunk_elems(chunk) == chunk
            c.gpu_step(hg)
            torch.cuda.synchronize()
            for k in c.keys:
                assert same_bits(c.arena.bufs[k], ref.arena.bufs[k]), (chunk, k)
            del c
    finally:
        A.adamw_set_chunk_elems(0)
    free()


def test_release_workspace_then_continue():
    """adamw_release_workspace between steps (after a synchronisation): the next
    call rebuilds its workspace and plan, and the run continues exactly."""
    case = Case("mixed", [5000, 70000, 13], seed=2800, random_moments=True)
    hg, ho = hp_pair()
    for s in range(4):
        if s:
            case.refill_grads(s)
        case.gpu_step(hg)
        case.oracle_step(ho)
        torch.cuda.synchronize()
        A.adamw_release_workspace()
    case.compare_all("release")
    free()


def test_split_master_tracks_mixed_master():
    """The split kernel on (p, r) and the mixed kernel on the fp32 master they
    encode stay bit-identical in the master and the moments over 10 steps; the
    split's bf16 half is the master's nearest bf16 (ties away from zero)."""
    numels = [70000, 9, 4099, 2048]
    sp = Case("split", numels, seed=1600, random_moments=True)
    mx = Case("mixed", numels, seed=1600, random_moments=True)
    # the mixed case starts from the master the split case encodes, with the same moments
    w0 = join_master(to_np(sp.arena.bufs["p"]), to_np(sp.arena.bufs["r"]))
    mx.arena.bufs["master"].copy_(torch.from_numpy(w0))
    for k in ("m", "v", "g"):
        mx.arena.bufs[k].copy_(sp.arena.bufs[k])
    hg, _ = hp_pair()
    for s in range(10):
        if s:
            sp.refill_grads(s)
            mx.arena.bufs["g"].copy_(sp.arena.bufs["g"])
        sp.gpu_step(hg)
        mx.gpu_step(hg)
    torch.cuda.synchronize()
    wj = join_master(to_np(sp.arena.bufs["p"]), to_np(sp.arena.bufs["r"]))
    assert np.array_equal(wj.view(np.uint32), to_np(mx.arena.bufs["master"]).view(np.uint32))
    for k in ("m", "v"):
        assert same_bits(sp.arena.bufs[k], mx.arena.bufs[k]), k
    pe, _ = oracle.split_make(wj)
    assert np.array_equal(to_np(sp.arena.bufs["p"]), pe)
    free()


@pytest.mark.parametrize("scale0,interval", [(65536.0, 3), (3e38, 2)])
def test_dynamic_loss_scale_sequence(scale0, interval):
    """fp16 AMP with the device-resident loss scale: 12 iterations of check +
    step, overflows planted at two seeded iterations.  After every iteration the
    device scale, tracker and step counter equal the oracle's, and at the end every
    buffer matches element by element.  The 3e38 start exercises a refused growth."""
    case = Case("mixed", EDGE_SIZES, seed=1700, p_dtype="f16", loss_scale=65536.0, align_elems=3)
    tl = case.tensor_list()
    hg, ho = hp_pair()
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    state = A.loss_scale_state(scale0)
    scaler = A.LossScaler(2.0, 0.5, interval)
    ls = oracle.LossScale(scale=scale0, tracker=0, growth=2.0, backoff=0.5, interval=interval)
    rng = np.random.default_rng(33)
    bad_iters = set(int(x) for x in rng.choice(np.arange(1, 12), size=2, replace=False))
    for it in range(12):
        if it:
            case.refill_grads(it)
        if it in bad_iters:
            i = int(rng.choice([j for j, n in enumerate(EDGE_SIZES) if n]))
            case.arena.view("g", i)[int(rng.integers(0, EDGE_SIZES[i]))] = float("inf")
            case.host["g"] = to_np(case.arena.bufs["g"])
        A.adamw_check_finite(A.F16, tl, flag)
        A.adamw_multi_tensor_step_amp(A.MIXED, A.F16, tl, hg, case.d_step, flag, state, scaler)
        case.step = oracle.amp_step_list("mixed", case.oracle_tensors(), ho, case.step, ls)
        torch.cuda.synchronize()
        assert int(flag.item()) == int(it in bad_iters)
        assert np.float32(state[0].item()) == np.float32(ls.scale), (it, state[0].item(), ls.scale)
        assert int(state.view(torch.int32)[1].item()) == ls.tracker, it
        assert int(case.d_step.item()) == case.step, it
    case.compare_all(f"amp-{scale0}")
    assert case.step == 12 - len(bad_iters)
    free()


@pytest.mark.parametrize("mode", ["mixed", "kahan", "split"])
@pytest.mark.parametrize("rank", [0, 1, 2, 3])
@pytest.mark.parametrize("flat_param", [False, True], ids=["param-per-tensor", "param-flat"])
def test_zero_layout_flat_grad_blocked_state(mode, rank, flat_param):
    """A ZeRO rank's layout: the reduce-scattered gradient as one flat shard
    buffer, exp_avg / exp_avg_sq / aux in the blocked layout of the shard, params
    per tensor (or, as after an all-gather into a flat buffer, flat too); 3 steps
    of rank r's quarter of the list against the oracle."""
    from gpu_util import build_blocked, compare_streams, unpack_blocked
    numels = [30592 * 8, 768, 2048 * 3, 8, 4099, 3 * 768, 40000, 1]
    total = sum(numels)
    b, e = rank * total // 4, (rank + 1) * total // 4
    case = Case(mode, numels, seed=2600 + rank, align_elems=1, random_moments=True)
    blocked = build_blocked(case, b, e)
    g_flat = case.arena.bufs["g"][b:e].clone()
    p_flat = case.arena.bufs["p"][b:e].clone()
    p_stream = [p_flat] if flat_param else [case.arena.view("p", i) for i in range(len(numels))]
    mask = A.BLOCKED_STATE | 0b10 | (0b1 if flat_param else 0)
    tl = A.TensorList(numels, [p_stream, [g_flat], [blocked], None, None], b, e, flat_mask=mask)
    hg, ho = hp_pair()
    code = {"mixed": A.MIXED, "kahan": A.PURE_KAHAN, "split": A.MIXED_SPLIT}[mode]
    for s in range(3):
        if s:
            case.refill_grads(s)
            g_flat.copy_(case.arena.bufs["g"][b:e])
        A.adamw_multi_tensor_step(code, A.BF16, tl, hg, case.d_step)
        case.oracle_step(ho, shard=(b, e))
    torch.cuda.synchronize()
    assert int(case.d_step.item()) == case.step == 3
    got = unpack_blocked(case, blocked, b, e)
    got["p"] = to_np(p_flat) if flat_param else to_np(case.arena.bufs["p"])[b:e]
    ref = {k: case.host[k][b:e] for k in case.keys}
    print(compare_streams(f"zero-{mode}-r{rank}", mode, got, ref, [k for k in case.keys if k != "g"]))
    if not flat_param:
        hp_all = to_np(case.arena.bufs["p"])
        assert np.array_equal(hp_all[:b], case.host["p"][:b]) and np.array_equal(hp_all[e:], case.host["p"][e:])
    free()


def test_blocked_state_fp16_amp_sequence():
    """fp16 AMP (check + step with the device-resident loss scale) with
    exp_avg / exp_avg_sq / master in the blocked layout: 8 iterations, an overflow
    planted at two of them; the scale, tracker and step counter after every
    iteration, and every element at the end, against the oracle."""
    from gpu_util import build_blocked, compare_streams, unpack_blocked
    numels = [30000, 7, 4099, 2048, 40000, 1, 9000]
    case = Case("mixed", numels, seed=2500, p_dtype="f16", loss_scale=65536.0, align_elems=1)
    total = sum(numels)
    blocked = build_blocked(case, 0, total)
    streams = [[case.arena.view("p", i) for i in range(len(numels))],
               [case.arena.view("g", i) for i in range(len(numels))], [blocked], None, None]
    tl = A.TensorList(numels, streams, 0, -1, flat_mask=A.BLOCKED_STATE)
    hg, ho = hp_pair()
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    state = A.loss_scale_state(65536.0)
    scaler = A.LossScaler(2.0, 0.5, 3)
    ls = oracle.LossScale(scale=65536.0, tracker=0, growth=2.0, backoff=0.5, interval=3)
    bad = {2, 5}
    for it in range(8):
        if it:
            case.refill_grads(it)
        if it in bad:
            case.arena.view("g", 4)[1234 * it] = float("inf") if it == 2 else float("nan")
            case.host["g"] = to_np(case.arena.bufs["g"])
        A.adamw_check_finite(A.F16, tl, flag)
        A.adamw_multi_tensor_step_amp(A.MIXED, A.F16, tl, hg, case.d_step, flag, state, scaler)
        case.step = oracle.amp_step_list("mixed", case.oracle_tensors(), ho, case.step, ls)
        torch.cuda.synchronize()
        assert int(flag.item()) == int(it in bad), it
        assert np.float32(state[0].item()) == np.float32(ls.scale), (it, state[0].item(), ls.scale)
        assert int(state.view(torch.int32)[1].item()) == ls.tracker, it
        assert int(case.d_step.item()) == case.step, it
    assert case.step == 6
    got = unpack_blocked(case, blocked, 0, total)
    got["p"] = to_np(case.arena.bufs["p"])
    keys = [k for k in case.keys if k != "g"]
    print(compare_streams("blocked-amp", "mixed", got, {k: case.host[k] for k in case.keys}, keys, True))
    free()


PURE_MODES = [f"pure-{m}-{v}-{k}" for m in ("f32", "bf16") for v in ("f32", "bf16") for k in ("k", "k32", "n")]


@pytest.mark.parametrize("mode", PURE_MODES)
@pytest.mark.parametrize("align", [128, 3])
def test_pure_precision_matrix(mode, align):
    """Every AnyPrecision combination (fp32/bf16 exp_avg and exp_avg_sq; no
    compensation, a bf16 or an fp32 compensation buffer) against the oracle on
    the edge sizes, from a random state, 4 steps."""
    case = Case(mode, EDGE_SIZES, seed=1800 + align, align_elems=align, random_moments=True)
    _run(case, 4, label=f"{mode}-a{align}")
    free()


def test_compensation_tracks_tiny_updates_on_the_gpu():
    """The reason for the compensation buffer, shown on the GPU: 10,000 steps of
    a constant +1e-4 update (lr 1e-4, constant gradient -1, no decay, eps 0)
    from 1.0.  The fp64 sum is 2.0; plain bf16 never leaves 1.0 (each update is
    below half an ulp); a bf16 buffer ends within 5 % of 2.0 and an fp32 buffer
    within 1e-5, with p at the bf16 nearest 2.0."""
    n, k = 256, 10_000
    hp = A.HParams(lr=1e-4, weight_decay=0.0, eps=0.0)
    one = torch.full((n,), 1.0, dtype=torch.bfloat16, device="cuda")
    g = torch.full((n,), -1.0, dtype=torch.bfloat16, device="cuda")
    got = {}
    for kahan, cdt in ((A.KAHAN_NONE, None), (A.KAHAN_BF16, torch.bfloat16), (A.KAHAN_F32, torch.float32)):
        p = one.clone()
        m = torch.zeros(n, dtype=torch.float32, device="cuda")
        v = torch.zeros(n, dtype=torch.float32, device="cuda")
        c = None if cdt is None else torch.zeros(n, dtype=cdt, device="cuda")
        tl = A.TensorList([n], [[p], [g], [m], [v], None if c is None else [c]])
        prec = A.PurePrecision(A.F32, A.F32, kahan)
        d_step = torch.zeros(1, dtype=torch.int32, device="cuda")
        for _ in range(k):
            A.adamw_pure_multi_tensor_step(prec, tl, hp, d_step)
        torch.cuda.synchronize()
        assert int(d_step.item()) == k
        total = p.double() + (0 if c is None else c.double())
        got[kahan] = (p.float().cpu(), total.cpu())
    assert bool((got[A.KAHAN_NONE][0] == 1.0).all())
    assert float((got[A.KAHAN_BF16][1] - 2.0).abs().max()) <= 0.1
    assert float((got[A.KAHAN_F32][1] - 2.0).abs().max()) <= 1e-5
    assert bool((got[A.KAHAN_F32][0] == 2.0).all())
    free()


def test_pure_bf16_kahan_equals_kahan_mode():
    """{bf16, bf16, Kahan} through adamw_pure_multi_tensor_step is ADAMW_PURE_KAHAN."""
    a = Case("kahan", [30000, 17, 4099], seed=1900, random_moments=True)
    b = Case("pure-bf16-bf16-k", [30000, 17, 4099], seed=1900, random_moments=True)
    for k in a.keys:
        b.arena.bufs[k].copy_(a.arena.bufs[k])
    hg, _ = hp_pair()
    for s in range(3):
        if s:
            a.refill_grads(s)
            b.arena.bufs["g"].copy_(a.arena.bufs["g"])
        a.gpu_step(hg)
        b.gpu_step(hg)
    torch.cuda.synchronize()
    for k in a.keys:
        assert same_bits(a.arena.bufs[k], b.arena.bufs[k]), k
    free()


def test_graph_capture_replay_matches_eager():
    """The check + step sequence captured once in a HIP graph and replayed 6
    times (with eager work and synchronisations between replays) leaves every
    buffer, the counter and the flag bit-identical to 6 eager iterations.  The
    capture stream is warmed up first so its workspace and plan already exist
    (capture records kernel launches only: no allocation, copy or memset)."""
    numels = [40000, 7, 4099, 1]
    eager = Case("mixed", numels, seed=2200, p_dtype="f16", loss_scale=65536.0, random_moments=True)
    graph = Case("mixed", numels, seed=2200, p_dtype="f16", loss_scale=65536.0, random_moments=True)
    hg, _ = hp_pair(inv_scale=1.0 / 65536)
    s = torch.cuda.Stream()
    fe = torch.zeros(1, dtype=torch.int32, device="cuda")
    fg = torch.zeros(1, dtype=torch.int32, device="cuda")
    tle, tlg = eager.tensor_list(), graph.tensor_list()

    def it_graph():
        A.adamw_check_finite(A.F16, tlg, fg, s)
        A.adamw_multi_tensor_step(A.MIXED, A.F16, tlg, hg, graph.d_step, fg, s)

    torch.cuda.synchronize()
    with torch.cuda.stream(s):          # warm-up on the capture stream (plans, workspace)
        it_graph()
    s.synchronize()
    A.adamw_check_finite(A.F16, tle, fe)
    A.adamw_multi_tensor_step(A.MIXED, A.F16, tle, hg, eager.d_step, fe)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        it_graph()
    for r in range(6):
        g.replay()
        A.adamw_check_finite(A.F16, tle, fe)
        A.adamw_multi_tensor_step(A.MIXED, A.F16, tle, hg, eager.d_step, fe)
        torch.cuda.synchronize()
        junk = torch.randn(1000, device="cuda").sum()      # unrelated eager work between replays
        del junk
        assert int(graph.d_step.item()) == int(eager.d_step.item()) == r + 2
        for k in eager.keys:
            assert same_bits(graph.arena.bufs[k], eager.arena.bufs[k]), (r, k)
    free()


def test_concurrent_host_threads_on_own_streams():
    """Four host threads, each stepping its own list on its own stream 5 times,
    concurrently (the ctypes calls release the GIL); each result equals the oracle."""
    import threading
    hg, ho = hp_pair()
    cases = [Case("mixed" if i % 2 else "kahan", [20000 + 13 * i, 9, 3000], seed=2300 + i) for i in range(4)]
    streams = [torch.cuda.Stream() for _ in cases]
    torch.cuda.synchronize()
    errors = []

    def work(c, st):
        try:
            for _ in range(5):
                tl = c.tensor_list()
                if c.mode == "mixed":
                    A.adamw_multi_tensor_step(A.MIXED, A.BF16, tl, hg, c.d_step, None, st)
                else:
                    A.adamw_multi_tensor_step(A.PURE_KAHAN, A.BF16, tl, hg, c.d_step, None, st)
            st.synchronize()
        except Exception as e:      # surfaced below
            errors.append(e)

    threads = [threading.Thread(target=work, args=(c, st)) for c, st in zip(cases, streams)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for i, c in enumerate(cases):
        for _ in range(5):
            c.oracle_step(ho)
        c.compare_all(f"thread-{i}")
    free()


@pytest.mark.parametrize("mode", ["mixed", "kahan", "split", "pure-f32-bf16-n", "pure-f32-f32-k"])
@pytest.mark.parametrize("shard", [(0, None), (37, 60013), (4096, 4096 * 3 + 13)], ids=["all", "odd", "aligned"])
def test_blocked_state_layout(mode, shard):
    """exp_avg / exp_avg_sq / aux in one blocked buffer of the shard (8,192-element
    blocks, stream after stream), param and grad per tensor: 3 steps against the
    oracle run on the ordinary per-stream arrays."""
    from gpu_util import build_blocked, unpack_blocked, pure_precision
    numels = [30000, 7, 4099, 2048, 40000, 1]
    case = Case(mode, numels, seed=2400, align_elems=1, random_moments=True)
    total = sum(numels)
    b, e = shard[0], shard[1] if shard[1] is not None else total
    blocked = build_blocked(case, b, e)
    streams = [[case.arena.view("p", i) for i in range(len(numels))],
               [case.arena.view("g", i) for i in range(len(numels))], [blocked], None, None]
    tl = A.TensorList(numels, streams, b, e, flat_mask=A.BLOCKED_STATE)
    hg, ho = hp_pair()
    for s in range(3):
        if s:
            case.refill_grads(s)
        if mode.startswith("pure"):
            A.adamw_pure_multi_tensor_step(pure_precision(mode), tl, hg, case.d_step)
        else:
            code = {"mixed": A.MIXED, "kahan": A.PURE_KAHAN, "split": A.MIXED_SPLIT}[mode]
            A.adamw_multi_tensor_step(code, A.BF16, tl, hg, case.d_step)
        case.oracle_step(ho, shard=(b, e))
    torch.cuda.synchronize()
    assert int(case.d_step.item()) == case.step == 3
    got = unpack_blocked(case, blocked, b, e)
    got["p"] = to_np(case.arena.bufs["p"])[b:e]
    ref = {k: case.host[k][b:e] for k in case.keys}
    keys = [k for k in case.keys if k != "g"]
    from gpu_util import compare_streams
    stats = compare_streams(f"blocked-{mode}", mode, got, ref, keys)
    print(stats)
    # the params outside the shard are untouched
    hp_all = to_np(case.arena.bufs["p"])
    assert np.array_equal(hp_all[:b], case.host["p"][:b]) and np.array_equal(hp_all[e:], case.host["p"][e:])
    free()


def test_mixed_step_tracks_torch_adamw():
    """A user-facing cross-check against torch.optim.AdamW on the GPU (fp32 params,
    gradients that are exact bf16 values): after 5 steps the fp32 master and the
    moments agree with PyTorch's to a few units in the last place.  torch orders
    the operations differently (moments by lerp, sqrt(v)/sqrt(1-b2^t)), so this is
    not the bitwise bar of the oracle comparisons."""
    torch.manual_seed(11)
    shapes = [(513, 77), (4099,), (64, 64, 3)]
    ref = [torch.randn(s, device="cuda") * 0.02 for s in shapes]
    hp = dict(lr=2e-4, betas=(0.9, 0.95), eps=1e-8, weight_decay=0.1)
    tparams = [torch.nn.Parameter(w.clone()) for w in ref]
    opt = torch.optim.AdamW(tparams, foreach=False, **hp)
    master = [w.clone() for w in ref]
    p16 = [w.to(torch.bfloat16) for w in ref]
    m = [torch.zeros_like(w) for w in ref]
    v = [torch.zeros_like(w) for w in ref]
    g16 = [torch.empty(s, dtype=torch.bfloat16, device="cuda") for s in shapes]
    tl = A.TensorList([w.numel() for w in ref], [p16, g16, m, v, master])
    step = torch.zeros(1, dtype=torch.int32, device="cuda")
    hg = A.HParams(lr=hp["lr"], beta1=0.9, beta2=0.95, eps=hp["eps"], weight_decay=hp["weight_decay"])
    gmax = [torch.zeros_like(w) for w in ref]
    for _ in range(5):
        for i, (g, tp) in enumerate(zip(g16, tparams)):
            g.copy_((torch.randn_like(tp) * 1e-3).to(torch.bfloat16))
            tp.grad = g.float()
            gmax[i] = torch.maximum(gmax[i], tp.grad.abs())
        opt.step()
        A.adamw_multi_tensor_step(A.MIXED, A.BF16, tl, hg, step)
    torch.cuda.synchronize()
    # Bounds relative to the terms each quantity is formed from (a result near 0 can
    # come from cancelling terms): the master moves by at most lr * |u| <= 2 lr per
    # step; exp_avg is a decaying sum of gradients; exp_avg_sq of squares (no
    # cancellation).  8 units in the last place of those magnitudes.
    ulp = 8 * 2.0 ** -23
    for i, tp in enumerate(tparams):
        st = opt.state[tp]
        w_t, m_t, v_t = tp.detach(), st["exp_avg"], st["exp_avg_sq"]
        checks = (("master", master[i], w_t, ref[i].abs() + w_t.abs() + 10 * hp["lr"]),
                  ("exp_avg", m[i], m_t, m_t.abs() + gmax[i]),
                  ("exp_avg_sq", v[i], v_t, v_t.abs()))
        for name, ours, theirs, scale in checks:
            diff = (ours - theirs).abs()
            assert bool((diff <= ulp * scale).all()), (i, name, float((diff / scale).max()))
        assert torch.equal(p16[i], master[i].to(torch.bfloat16))
    assert int(step.item()) == 5
    free()


@pytest.mark.parametrize("mode,p_dtype", [("mixed", "bf16"), ("mixed", "f16"), ("kahan", "bf16"), ("split", "bf16"),
                                          ("pure-bf16-f32-k32", "bf16"), ("pure-f32-bf16-n", "bf16")])
def test_arbitrary_bit_patterns_in_every_stream(mode, p_dtype):
    """IEEE semantics end to end: every stream (params, gradients, moments,
    master, compensation, remainder) filled with uniformly random bit patterns --
    NaNs, infinities, subnormals, negative second moments and signed zeros
    included -- and stepped twice.  Every result, NaN or not, must have the
    oracle's bit pattern (a NaN's payload aside)."""
    case = Case(mode, [70_000, 5, 4099, 1], seed=1700, p_dtype=p_dtype)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1701)
    for k in case.keys:
        buf = case.arena.bufs[k]
        raw = buf.view(torch.int32) if buf.element_size() == 4 else buf.view(torch.int16)
        info = torch.iinfo(raw.dtype)
        raw.copy_(torch.randint(info.min, info.max, raw.shape, generator=gen, device="cuda", dtype=raw.dtype))
        case.host[k] = to_np(buf)
    hg, ho = hp_pair()
    for s in range(2):
        case.gpu_step(hg)
        case.oracle_step(ho)
    case.compare_all(f"bits-{mode}-{p_dtype}")
    free()
