"""GPU: the two launch forms of a step give the same bits.  Grids of at most
adamw_set_single_launch_max_workgroups workgroups (8 per chunk of a step) run
as one launch of the update kernel, which forms the step's scalars in every workgroup and lets the last
workgroup advance the counter; larger plans run the prologue kernel first.
Every element, the counter and the skip behaviour must not depend on the form,
and both must match the oracle."""
import pytest
import torch

import adamw_optimizer_step_apply_amd as A
from gpu_util import Case, free, hp_pair, same_bits

pytestmark = pytest.mark.gpu

SIZES = [0, 1, 7, 8, 9, 2047, 2048, 2049, 16385, 100_003, 3, 40_000]


@pytest.fixture
def single_launch_limit():
    """Sets the single-launch limit for one test and restores the default."""
    def set_limit(n):
        return A.adamw_set_single_launch_max_workgroups(n)
    yield set_limit
    A.adamw_set_single_launch_max_workgroups(-1)


def _plan_chunks(case: Case) -> int:
    """Chunks of the case's plan (mixed, kahan and split lists)."""
    code = {"mixed": A.MIXED, "kahan": A.PURE_KAHAN, "split": A.MIXED_SPLIT}[case.mode]
    dt = A.F16 if case.p_dtype == "f16" else A.BF16
    return len(A.adamw_plan_inspect(code, dt, case.tensor_list()))


@pytest.mark.parametrize("mode,p_dtype", [("mixed", "bf16"), ("mixed", "f16"), ("kahan", "bf16"), ("split", "bf16"),
                                          ("pure-f32-f32-k", "bf16"), ("pure-bf16-f32-n", "bf16"),
                                          ("pure-bf16-bf16-k32", "bf16")])
def test_forms_are_bit_identical_and_match_the_oracle(mode, p_dtype, single_launch_limit):
    """The same list stepped 4 times in each form (one copy each), a skipped step
    in the middle: every buffer and the counter bitwise equal between the forms,
    and the single-launch copy within the bar of the oracle."""
    scale = 65536.0 if p_dtype == "f16" else 1.0
    kw = dict(p_dtype=p_dtype, align_elems=3, loss_scale=scale, random_moments=True)
    one, two = Case(mode, SIZES, seed=911, **kw), Case(mode, SIZES, seed=911, **kw)
    if not mode.startswith("pure"):
        assert 0 < 8 * _plan_chunks(one) <= 4096
    hg, ho = hp_pair(inv_scale=1.0 / scale)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    for s in range(5):
        if s:
            one.refill_grads(s)
            two.refill_grads(s)
        flag.fill_(1 if s == 2 else 0)
        single_launch_limit(-1)
        one.gpu_step(hg, found_inf=flag)
        single_launch_limit(0)
        two.gpu_step(hg, found_inf=flag)
        if s != 2:
            one.oracle_step(ho)
    torch.cuda.synchronize()
    assert int(one.d_step.item()) == int(two.d_step.item()) == 4
    for k in one.keys:
        assert same_bits(one.arena.bufs[k], two.arena.bufs[k]), f"{mode}: stream {k} differs between the forms"
    one.compare_all(f"single-launch-{mode}-{p_dtype}")
    free()


@pytest.mark.parametrize("extra", [0, 1])
def test_limit_boundary(extra, single_launch_limit):
    """A grid of exactly the limit (8 workgroups per chunk) runs as one launch;
    one workgroup more takes the prologue.  Both match the oracle over 3 steps."""
    case = Case("mixed", SIZES, seed=912, align_elems=3, random_moments=True)
    k = _plan_chunks(case)
    single_launch_limit(8 * k - extra)
    hg, ho = hp_pair()
    for s in range(3):
        if s:
            case.refill_grads(s)
        case.gpu_step(hg)
        case.oracle_step(ho)
    case.compare_all(f"boundary-{extra}")
    free()


def test_forms_alternate_on_one_stream(single_launch_limit):
    """Two lists on one stream, stepped in turn while the form changes every
    call: the single-launch completion count must be back at zero after each
    launch, and each counter must advance once per step."""
    a = Case("mixed", SIZES, seed=913, random_moments=True)
    b = Case("kahan", [5000, 70, 4099, 1], seed=914, random_moments=True)
    hg, ho = hp_pair()
    for s in range(8):
        for i, case in enumerate((a, b)):
            if s:
                case.refill_grads(s)
            single_launch_limit(-1 if (s + i) % 2 == 0 else 0)
            case.gpu_step(hg)
            case.oracle_step(ho)
    a.compare_all("alternate-mixed")
    b.compare_all("alternate-kahan")
    free()


def test_single_launch_graph_replays(single_launch_limit):
    """A single-launch step captured in a HIP graph and replayed 5 times, with
    eager work between the replays, equals 5 eager steps bit for bit."""
    single_launch_limit(-1)
    numels = [5000, 70, 4099, 1, 20000]
    eager, graphed = Case("mixed", numels, seed=915), Case("mixed", numels, seed=915)
    hg, _ = hp_pair()
    tl_e, tl_g = eager.tensor_list(), graphed.tensor_list()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        # one warm-up call on the capture stream builds its workspace and plan
        A.adamw_multi_tensor_step(A.MIXED, A.BF16, tl_g, hg, graphed.d_step, None, s)
        A.adamw_multi_tensor_step(A.MIXED, A.BF16, tl_e, hg, eager.d_step, None, s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        A.adamw_multi_tensor_step(A.MIXED, A.BF16, tl_g, hg, graphed.d_step, None, s)
    for r in range(5):
        g.replay()
        with torch.cuda.stream(s):
            A.adamw_multi_tensor_step(A.MIXED, A.BF16, tl_e, hg, eager.d_step, None, s)
        torch.cuda.synchronize()
        _ = torch.ones(1 << 20, device="cuda").sum().item()   # unrelated eager work between replays
        assert int(graphed.d_step.item()) == int(eager.d_step.item()) == r + 2
        for k in eager.keys:
            assert same_bits(graphed.arena.bufs[k], eager.arena.bufs[k]), (r, k)
    del g
    free()


@pytest.mark.parametrize("start", [999_999, 2**31 - 3])
def test_forms_agree_at_large_step_counts(start, single_launch_limit):
    """Resuming at a large step counter: both forms form the same scalars (the
    bias corrections are then 1 to within fp32) and store the same counter,
    and both match the oracle, for 2 steps."""
    one, two = (Case("mixed", SIZES, seed=916, random_moments=True) for _ in range(2))
    for c in (one, two):
        c.d_step.fill_(start)
        c.step = start
    hg, ho = hp_pair()
    for s in range(2):
        if s:
            one.refill_grads(s)
            two.refill_grads(s)
        single_launch_limit(-1)
        one.gpu_step(hg)
        single_launch_limit(0)
        two.gpu_step(hg)
        one.oracle_step(ho)
        two.oracle_step(ho)
    one.compare_all(f"large-step-single-{start}")
    two.compare_all(f"large-step-two-{start}")
    for k in one.keys:
        assert same_bits(one.arena.bufs[k], two.arena.bufs[k]), k
    free()


@pytest.mark.parametrize("g_dtype", ["f16", "bf16"])
def test_check_forms_agree(g_dtype, single_launch_limit):
    """The overflow check in one launch (the last workgroup stores the flag)
    and in two (zero the flag, then OR into it): the same flag as the oracle's
    scan for clean gradients and for one planted inf/NaN at seeded positions,
    with the flag holding a stale value before every call."""
    import numpy as np
    import oracle
    from gpu_util import to_np
    is16 = g_dtype == "f16"
    case = Case("mixed", SIZES, seed=917, p_dtype=g_dtype, align_elems=3, loss_scale=65536.0 if is16 else 1.0)
    tl = case.tensor_list()
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    rng = np.random.default_rng(918)
    bad_bits = (0x7C00, 0xFC00, 0x7E00) if is16 else (0x7F80, 0xFF80, 0x7FC0)
    nonempty = [i for i, n in enumerate(SIZES) if n]
    for trial in range(12):
        planted = None
        if trial % 3:
            i = int(rng.choice(nonempty))
            e = int(rng.integers(0, SIZES[i]))
            view = case.arena.view("g", i).view(torch.int16)
            planted = (view, e, int(view[e].item()))
            view[e] = int(np.int16(np.uint16(bad_bits[trial % 3]).view(np.int16)))
        want = oracle.any_nonfinite(to_np(case.arena.bufs["g"]), is16)
        got = []
        for lim in (-1, 0):
            single_launch_limit(lim)
            flag.fill_(7)
            A.adamw_check_finite(A.F16 if is16 else A.BF16, tl, flag)
            torch.cuda.synchronize()
            got.append(int(flag.item()))
        assert got == [int(want)] * 2, (trial, got, want)
        if planted:
            planted[0][planted[1]] = planted[2]
    free()


def test_amp_sequence_forms_agree(single_launch_limit):
    """fp16 AMP with the device-resident loss scale, 10 iterations of check +
    step with overflows planted at two of them, run in one launch each and in
    two launches each on identical copies: flag, scale, tracker, counter after
    every iteration and every buffer at the end are bitwise equal, and the
    single-launch copy matches the oracle."""
    import numpy as np
    import oracle
    one = Case("mixed", SIZES, seed=919, p_dtype="f16", loss_scale=65536.0, align_elems=3)
    two = Case("mixed", SIZES, seed=919, p_dtype="f16", loss_scale=65536.0, align_elems=3)
    hg, ho = hp_pair()
    scaler = A.LossScaler(2.0, 0.5, 3)
    ls = oracle.LossScale(scale=65536.0, tracker=0, growth=2.0, backoff=0.5, interval=3)
    runs = []
    for case, lim in ((one, -1), (two, 0)):
        runs.append((case, lim, case.tensor_list(), torch.zeros(1, dtype=torch.int32, device="cuda"),
                     A.loss_scale_state(65536.0)))
    bad_iters = {3, 7}
    for it in range(10):
        for case, lim, tl, flag, state in runs:
            if it:
                case.refill_grads(it)
            if it in bad_iters:
                case.arena.view("g", 9)[12345 % SIZES[9]] = float("inf")
            single_launch_limit(lim)
            A.adamw_check_finite(A.F16, tl, flag)
            A.adamw_multi_tensor_step_amp(A.MIXED, A.F16, tl, hg, case.d_step, flag, state, scaler)
        from gpu_util import to_np
        one.host["g"] = to_np(one.arena.bufs["g"])
        one.step = oracle.amp_step_list("mixed", one.oracle_tensors(), ho, one.step, ls)
        torch.cuda.synchronize()
        (_, _, _, f1, s1), (_, _, _, f2, s2) = runs
        assert int(f1.item()) == int(f2.item()) == int(it in bad_iters), it
        assert same_bits(s1, s2), (it, s1.tolist(), s2.tolist())
        assert np.float32(s1[0].item()) == np.float32(ls.scale) and int(s1.view(torch.int32)[1].item()) == ls.tracker
        assert int(one.d_step.item()) == int(two.d_step.item()) == one.step, it
    for k in one.keys:
        assert same_bits(one.arena.bufs[k], two.arena.bufs[k]), k
    one.compare_all("amp-single-launch")
    free()


@pytest.mark.parametrize("mode,amp", [("kahan", False), ("mixed", True)])
def test_single_launch_forced_on_a_large_grid(mode, amp, single_launch_limit):
    """The single launch does not depend on the grid's size: forced on the
    OPT-125m list (7,760 chunks, 62,080 workgroups, about 1,940 per first-level
    completion counter) it equals the two-launch form bit for bit over 4 steps
    with a skipped one, and stores the same counter (and, with a dynamic loss
    scale, the same scale and tracker, including a back-off and a growth)."""
    import workloads
    wl = workloads.get("opt_125m")
    numels = wl.numels
    p_dtype = "f16" if amp else "bf16"
    scale = 1024.0 if amp else 1.0
    arenas = [workloads.make_state(mode, numels, "cuda", 917, p_dtype=p_dtype, loss_scale=scale,
                                   random_moments=True) for _ in range(2)]
    keys = workloads.streams_of(mode)
    lists = [A.TensorList(numels, [[a.view(k, i) for i in range(len(numels))] for k in keys]) for a in arenas]
    steps = [torch.zeros(1, dtype=torch.int32, device="cuda") for _ in range(2)]
    scales = [A.loss_scale_state(scale) for _ in range(2)]
    scaler = A.LossScaler(2.0, 0.5, 2)
    code = {"mixed": A.MIXED, "kahan": A.PURE_KAHAN}[mode]
    dt = A.F16 if amp else A.BF16
    hg, _ = hp_pair()
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    assert 8 * len(A.adamw_plan_inspect(code, dt, lists[0])) > 60_000
    for s in range(4):
        if s:
            for a in arenas:
                workloads.refill_grads(a, 917, s, p_dtype=p_dtype, loss_scale=scale)
        flag.fill_(1 if s == 1 else 0)
        for i, limit in enumerate((1 << 40, 0)):
            single_launch_limit(limit)
            if amp:
                A.adamw_multi_tensor_step_amp(code, dt, lists[i], hg, steps[i], flag, scales[i], scaler)
            else:
                A.adamw_multi_tensor_step(code, dt, lists[i], hg, steps[i], flag)
    torch.cuda.synchronize()
    assert int(steps[0].item()) == int(steps[1].item()) == 3
    if amp:
        assert same_bits(scales[0], scales[1])
        st = scales[0].view(torch.int32)
        assert float(scales[0][0]) == scale and int(st[1]) == 0     # backed off to 512, grown back after 2 clean steps
    for k in keys:
        assert same_bits(arenas[0].bufs[k], arenas[1].bufs[k]), f"{mode}: stream {k} differs between the forms"
    del arenas, lists
    free()


def test_many_single_launches_in_a_row(single_launch_limit):
    """2,000 single-launch steps back to back, an overflow check between them
    (both single-launch kernels sharing the stream's completion counters): the
    counter ends at exactly 2,000 and the state equals 2,000 two-launch steps
    bit for bit, so no launch ever miscounts its grid."""
    numels = [70_000, 3, 4099, 1, 16384 * 3 + 5]
    one, two = (Case("mixed", numels, seed=918, random_moments=True) for _ in range(2))
    tl1, tl2 = one.tensor_list(), two.tensor_list()
    hg = A.HParams(lr=1e-6)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    k = 2000
    single_launch_limit(-1)
    assert 8 * _plan_chunks(one) <= 4096
    for _ in range(k):
        A.adamw_check_finite(A.BF16, tl1, flag)
        A.adamw_multi_tensor_step(A.MIXED, A.BF16, tl1, hg, one.d_step, flag)
    single_launch_limit(0)
    for _ in range(k):
        A.adamw_check_finite(A.BF16, tl2, flag)
        A.adamw_multi_tensor_step(A.MIXED, A.BF16, tl2, hg, two.d_step, flag)
    torch.cuda.synchronize()
    assert int(one.d_step.item()) == int(two.d_step.item()) == k and int(flag.item()) == 0
    for key in one.keys:
        assert same_bits(one.arena.bufs[key], two.arena.bufs[key]), key
    free()
