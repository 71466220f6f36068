"""Randomised GPU parity: seeded draws over the whole configuration space of the
C ABI, each checked element by element against the oracle.

Every case draws a mode (mixed bf16 / fp16, Kahan, split master, the twelve
AnyPrecision combinations), a ragged tensor list (empty tensors included), a
ZeRO shard range, the flat index (back to back, or padded to multiples of 8),
buffer alignment, the layout of param, grad and state (per tensor, flat shard
buffer, or the blocked state layout), random
hyper-parameters, 1-3 steps with fresh gradients and, in fp16 runs, an overflow
planted in one step (check + skip).  Bar: see gpu_util."""
import numpy as np
import pytest
import torch

import adamw_optimizer_step_apply_amd as A
import oracle
from gpu_util import Case, build_blocked, compare_streams, hp_pair, pure_precision, to_np, unpack_blocked, free

pytestmark = pytest.mark.gpu

PURE = [f"pure-{m}-{v}-{k}" for m in ("f32", "bf16") for v in ("f32", "bf16") for k in ("k", "k32", "n")]
MODES = ["mixed", "mixed-f16", "kahan", "split"] + PURE


def _draw(seed):
    rng = np.random.default_rng(np.random.SeedSequence([31, seed]))
    mode = MODES[int(rng.integers(len(MODES)))]
    nt = int(rng.integers(1, 9))
    numels = [0 if rng.random() < 0.1 else int(np.exp(rng.uniform(0, np.log(70000)))) for _ in range(nt)]
    if sum(numels) == 0:
        numels[0] = 1 + int(rng.integers(5000))
    pad8 = bool(rng.random() < 0.35)
    state = ["tensor", "flat", "blocked"][int(rng.integers(3))]
    grad_flat = bool(rng.random() < 0.5)
    param_flat = bool(rng.random() < 0.3)
    tight = state != "tensor" or grad_flat or param_flat
    # a tight arena puts every element at its flat index (padded: align 8)
    if tight:
        align = 8 if pad8 else 1
    else:
        align = int(rng.choice([8, 128] if pad8 else [1, 3, 8, 128]))
    ends = np.cumsum([-(-n // 8) * 8 if pad8 else n for n in numels])
    # the flat index's last position; flat and blocked buffers are cut from the arena, which ends
    # at the last tensor's last element
    total = int(ends[-1]) if not tight else int(ends[-1] - (-(-numels[-1] // 8) * 8 - numels[-1] if pad8 else 0))
    if rng.random() < 0.4:
        shard = (0, total)
    else:
        b = int(rng.integers(0, total))
        if pad8 and rng.random() < 0.5:
            b = b // 8 * 8
        shard = (b, int(rng.integers(b + 1, total + 1)))
    hp = dict(lr=float(10 ** rng.uniform(-5, -2)), beta1=float(rng.uniform(0.5, 0.99)),
              beta2=float(rng.uniform(0.9, 0.9999)), eps=float(10 ** rng.uniform(-8, -6)),
              weight_decay=float(rng.uniform(0, 0.3)))
    steps = int(rng.integers(1, 4))
    plant = mode == "mixed-f16" and rng.random() < 0.8
    return dict(mode=mode, numels=numels, shard=shard, state=state, grad_flat=grad_flat, param_flat=param_flat,
                align=align, pad8=pad8, hp=hp, steps=steps, plant=plant, random_moments=bool(rng.random() < 0.7),
                rng=rng)


@pytest.mark.parametrize("seed", range(200))
def test_random_configuration(seed):
    d = _draw(seed)
    f16 = d["mode"] == "mixed-f16"
    mode = "mixed" if f16 else d["mode"]
    scale = 65536.0 if f16 else 1.0
    print(f"seed {seed}: {d['mode']} tensors={d['numels']} shard={d['shard']} state={d['state']} "
          f"grad_flat={d['grad_flat']} param_flat={d['param_flat']} align={d['align']} pad8={d['pad8']} "
          f"steps={d['steps']} "
          f"plant={d['plant']}", flush=True)
    case = Case(mode, d["numels"], seed=4000 + seed, p_dtype="f16" if f16 else "bf16", align_elems=d["align"],
                loss_scale=scale, random_moments=d["random_moments"])
    b, e = d["shard"]
    nt = len(d["numels"])
    hg, ho = hp_pair(inv_scale=1.0 / scale, **d["hp"])
    keys = case.keys

    flat = {}
    streams = []
    mask = 0
    for s, k in enumerate(keys):
        if s >= 2 and d["state"] == "blocked":
            streams.append(None)
            continue
        if (s == 0 and d["param_flat"]) or (s == 1 and d["grad_flat"]) or (s >= 2 and d["state"] == "flat"):
            flat[k] = case.arena.bufs[k][b:e].clone()
            streams.append([flat[k]])
            mask |= 1 << s
        else:
            streams.append([case.arena.view(k, i) for i in range(nt)])
    blocked = None
    if d["state"] == "blocked":
        blocked = build_blocked(case, b, e)
        streams[2] = [blocked]
        mask |= A.BLOCKED_STATE
    streams += [None] * (5 - len(streams))
    if d["pad8"]:
        mask |= A.FLAT_PAD8
    tl = A.TensorList(d["numels"], streams, b, e, flat_mask=mask)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    flat_align = 8 if d["pad8"] else 1
    pieces = list(oracle.shard_pieces(d["numels"], b, e, flat_align))   # the shard's real elements
    plant_step = int(d["rng"].integers(d["steps"])) if d["plant"] and pieces else -1

    for s in range(d["steps"]):
        if s:
            case.refill_grads(s)
        if s == plant_step:
            # a real element inside the shard, at its tensor's place in the arena
            t, lo, hi, _ = pieces[int(d["rng"].integers(len(pieces)))]
            case.arena.bufs["g"][case.arena.offsets[t] + int(d["rng"].integers(lo, hi))] = float("inf")
            case.host["g"] = to_np(case.arena.bufs["g"])
        if "g" in flat:
            flat["g"].copy_(case.arena.bufs["g"][b:e])
        if f16:
            A.adamw_check_finite(A.F16, tl, flag)
            A.adamw_multi_tensor_step(A.MIXED, A.F16, tl, hg, case.d_step, flag)
        elif mode.startswith("pure"):
            A.adamw_pure_multi_tensor_step(pure_precision(mode), tl, hg, case.d_step)
        else:
            code = {"mixed": A.MIXED, "kahan": A.PURE_KAHAN, "split": A.MIXED_SPLIT}[mode]
            A.adamw_multi_tensor_step(code, A.BF16, tl, hg, case.d_step)
        case.oracle_step(ho, shard=(b, e), check_overflow=f16, flat_align=flat_align)
    torch.cuda.synchronize()
    assert int(case.d_step.item()) == case.step
    if f16:
        assert int(flag.item()) == int(plant_step == d["steps"] - 1)

    # gather the GPU's results in the arena's index space
    got = {k: to_np(case.arena.bufs[k]) for k in keys}
    for k, buf in flat.items():
        got[k][b:e] = to_np(buf)
    if blocked is not None:
        for k, v in unpack_blocked(case, blocked, b, e).items():
            got[k][b:e] = v
    out_keys = [k for k in keys if k != "g"]
    compare_streams(f"random-{seed}", mode, got, case.host, out_keys, f16)
    free()
