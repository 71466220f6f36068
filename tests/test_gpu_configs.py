"""GPU parity at the workloads' full sizes, in the launch configuration that
bench.py times (allocation-aligned arenas, default chunking).  The oracle steps
every element (on all host threads) and every element of every stream is
compared, the arenas' untouched parts included; only the tensor past 2^32
elements is followed on samples.  Bar: see gpu_util.  The OPT-1.3B list is in
test_gpu_full_size.py."""
import numpy as np
import pytest
import torch

import adamw_optimizer_step_apply_amd as A
import oracle
import workloads
from gpu_util import Case, FullCase, SampledCase, build_blocked_padded, free, hp_pair, same_bits, to_np

pytestmark = pytest.mark.gpu


def _print(*a):
    print(*a, flush=True)


def test_bert_rank0_shard_all_elements_20_steps():
    """The BERT list at DP=4, rank 0's shard (13,059,840 elements, inside the
    word embedding), 20 steps, compared element by element over the whole list
    (the other ranks' elements must stay untouched)."""
    wl = workloads.get("bert_52m")
    b, e = wl.shard(0)
    case = Case("mixed", wl.numels, seed=2001)
    hg, ho = hp_pair()
    for s in range(wl.steps):
        if s:
            case.refill_grads(s)
        case.gpu_step(hg, shard=(b, e))
        case.oracle_step(ho, shard=(b, e))
    stats = case.compare_all("bert-r0")
    _print(stats)
    free()


@pytest.mark.parametrize("rank", [1, 2, 3])
def test_bert_other_rank_shards_all_elements(rank):
    """Ranks 1-3: shards that start and end inside tensors and span several;
    20 steps, every element of the list compared (the other ranks' elements
    must stay untouched)."""
    wl = workloads.get("bert_52m")
    shard = wl.shard(rank)
    case = FullCase("mixed", wl.numels, seed=2100 + rank)
    hg, ho = hp_pair()
    tl = case.tensor_list(*shard)
    for s in range(wl.steps):
        if s:
            case.refill_grads(s)
        A.adamw_multi_tensor_step(A.MIXED, A.BF16, tl, hg, case.d_step)
        case.oracle_step(ho, shard=shard)
    _print(case.compare_all(f"bert-r{rank}"))
    free()


def test_opt125m_kahan_100_steps_warmup():
    """OPT-125m list, pure bf16 + Kahan, 100 steps of the linear warmup schedule
    (lr 2e-4 * t/500), a fresh seeded gradient every step; every element
    compared at t = 10 and t = 100."""
    wl = workloads.get("opt_125m")
    case = FullCase("kahan", wl.numels, seed=3001)
    tl = case.tensor_list()
    for s in range(wl.steps):
        if s:
            case.refill_grads(s)
        lr = oracle.warmup_linear_lr(s + 1)
        hg, ho = hp_pair(lr=lr)
        A.adamw_multi_tensor_step(A.PURE_KAHAN, A.BF16, tl, hg, case.d_step)
        case.oracle_step(ho)
        if s + 1 in (10, 100):
            _print(case.compare_all(f"opt125m-t{s + 1}"))
    free()


BIG = 2 ** 32 + 6157     # one tensor past 2^32 elements, with a ragged tail of 5 after its last pack


@pytest.mark.parametrize("mode,shard", [("mixed", (0, -1)), ("mixed", (2 ** 31 + 5, 2 ** 32 + 100)),
                                        ("kahan", (0, -1))])
def test_single_tensor_beyond_32_bit_offsets(mode, shard):
    """The largest sizes: a tensor of 4,294,973,453 elements (68.7 GB of mixed
    state) and a short tensor behind it, whole or through a shard that starts
    at an unaligned position past 2^31 and ends past 2^32.  Two steps; the
    oracle follows 2M uniform samples plus every element within 24 of 2^31,
    2^32, the shard edges and the tensor ends."""
    numels = [BIG, 1000]
    total = sum(numels)
    b, e = shard[0], (total if shard[1] < 0 else shard[1])
    marks = [2 ** 31, 2 ** 32, b, e, BIG - 5, BIG]
    extra = sorted({x + d for x in marks for d in range(-24, 24)})
    _print(f"beyond-2^32 {mode} shard={shard}: allocating")
    case = SampledCase(mode, numels, seed=4301 if mode == "mixed" else 4302, shard=shard, extra=extra)
    tl = case.tensor_list()
    hg, ho = hp_pair()
    code = {"mixed": A.MIXED, "kahan": A.PURE_KAHAN}[mode]
    for s in range(2):
        if s:
            case.refill_grads(s)
        A.adamw_multi_tensor_step(code, A.BF16, tl, hg, case.d_step)
        case.oracle_step(ho)
    _print(case.compare_all(f"beyond-2^32-{mode}-{shard}"))
    del case, tl
    free()


def _host_any_nonfinite(g: torch.Tensor, block=1 << 28) -> bool:
    for i in range(0, g.numel(), block):
        if oracle.any_nonfinite(to_np(g[i:i + block]), True):
            return True
    return False


def test_ragged_10k_fp16_overflow_skip():
    """10,000 tensors, log-uniform sizes in [1, 2^22] (2.77e9 elements), fp16
    params and grads scaled by 65536, fp32 master/m/v.  Every step runs the
    overflow check, then the step with the flag.  One seeded step plants +inf at
    a seeded tensor and element: the flag must be set (as the oracle's scan of
    all gradients says) and every buffer and the counter left bit-identical.
    Every element compared at the end."""
    wl = workloads.get("ragged_10k")
    scale = wl.loss_scale
    case = FullCase("mixed", wl.numels, seed=5001, p_dtype="f16", loss_scale=scale)
    tl = case.tensor_list()
    hg, ho = hp_pair(inv_scale=1.0 / scale)
    rng = np.random.default_rng(np.random.SeedSequence([5, 1]))
    inject_step = int(rng.integers(1, wl.steps + 1))
    t_inj = int(rng.integers(0, len(wl.numels)))
    e_inj = int(rng.integers(0, wl.numels[t_inj]))
    _print("inject at step", inject_step, "tensor", t_inj, "element", e_inj, "of", wl.numels[t_inj])
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    for s in range(wl.steps + 1):
        if s:
            case.refill_grads(s)
        if s == inject_step:
            case.arena.view("g", t_inj)[e_inj] = float("inf")
        A.adamw_check_finite(A.F16, tl, flag)
        torch.cuda.synchronize()
        want = _host_any_nonfinite(case.arena.bufs["g"])
        assert int(flag.item()) == int(want) == int(s == inject_step), (s, int(flag.item()), want)
        if want:
            before = {k: case.arena.bufs[k].clone() for k in ("p", "m", "v", "master")}
            step_before = int(case.d_step.item())
        A.adamw_multi_tensor_step(A.MIXED, A.F16, tl, hg, case.d_step, flag)
        case.oracle_step(ho, skip=want)
        if want:
            torch.cuda.synchronize()
            assert int(case.d_step.item()) == step_before
            for k, v in before.items():
                assert same_bits(case.arena.bufs[k], v), f"{k} changed on a skipped step"
            del before
        _print(f"ragged10k: step {s} done")
    _print(case.compare_all("ragged10k"))
    del case, tl
    free()


def test_ragged_10k_fp16_blocked_padded_state():
    """The 10,000-tensor fp16 list in the launch configuration bench.py times for
    it: exp_avg / exp_avg_sq / master in the blocked layout of the padded flat
    index (every tensor at a multiple of 8), params and grads per tensor.  Check
    + step for 3 steps, an overflow planted in the second (skipped: nothing
    written, counter kept); every element of every stream against the oracle."""
    wl = workloads.get("ragged_10k")
    scale = wl.loss_scale
    case = FullCase("mixed", wl.numels, seed=5101, p_dtype="f16", loss_scale=scale, align_elems=8)
    state = case.keys[2:]
    blocked = build_blocked_padded(case.arena, state, wl.numels)
    for k in state:                      # the per-tensor copies are not stepped: let them go
        case.arena.bufs[k] = case.arena.bufs[k][:0]
    free()
    streams = [[case.arena.view(k, i) for i in range(len(wl.numels))] for k in case.keys[:2]]
    tl = A.TensorList(wl.numels, streams + [[blocked], None, None], 0, -1, A.BLOCKED_STATE | A.FLAT_PAD8)
    hg, ho = hp_pair(inv_scale=1.0 / scale)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    t_inj = int(np.argmax(wl.numels))
    for s in range(3):
        if s:
            case.refill_grads(s)
        if s == 1:
            case.arena.view("g", t_inj)[12345] = float("inf")
        A.adamw_check_finite(A.F16, tl, flag)
        A.adamw_multi_tensor_step(A.MIXED, A.F16, tl, hg, case.d_step, flag)
        case.oracle_step(ho, skip=(s == 1), flat_align=8)
        torch.cuda.synchronize()
        assert int(flag.item()) == int(s == 1), s
        _print(f"ragged10k-blocked: step {s} done")
    assert case.step == 2
    _print(case.compare_all("ragged10k-blocked", skip_keys=state))
    _print(case.compare_blocked(blocked, "ragged10k-blocked"))
    del case, tl, blocked
    free()


def test_bert_zero_shard_with_flat_grad_and_state():
    """The ZeRO layout proper: rank 2 of 4 holds its gradient shard and its
    optimizer state (fp32 master, exp_avg, exp_avg_sq) as flat buffers of the
    shard's length, while the params stay the model's per-tensor tensors.  20
    steps of the BERT list, a fresh reduce-scattered gradient each step; every
    element compared (the flat buffers written back to their place in the list)."""
    wl = workloads.get("bert_52m")
    b, e = wl.shard(2)
    case = FullCase("mixed", wl.numels, seed=2200, align_elems=1)
    assert case.arena.offsets[-1] + wl.numels[-1] == wl.total      # the arenas are the flat index itself
    flat = {k: case.arena.bufs[k][b:e].clone() for k in ("g", "m", "v", "master")}
    params = [case.arena.view("p", i) for i in range(len(wl.numels))]
    tl = A.TensorList(wl.numels, [params, [flat["g"]], [flat["m"]], [flat["v"]], [flat["master"]]], b, e,
                      0b11110)
    hg, ho = hp_pair()
    for s in range(wl.steps):
        if s:
            case.refill_grads(s)
            flat["g"].copy_(case.arena.bufs["g"][b:e])
        A.adamw_multi_tensor_step(A.MIXED, A.BF16, tl, hg, case.d_step)
        case.oracle_step(ho, shard=(b, e))
    for k in ("m", "v", "master"):
        case.arena.bufs[k][b:e].copy_(flat[k])
    _print(case.compare_all("bert-r2-flat"))
    del case, tl, flat, params
    free()
