"""GPU: adamw_blocked_state_copy / make_blocked_state, the layout-only copy
between per-tensor state buffers and the blocked state buffer.

* Packing gives, byte for byte, the buffer the tests build on their own
  (gpu_util.build_blocked_padded, or blocked_gather at every position).
* Unpacking a packed buffer into cleared per-tensor buffers gives back the
  original state bit for bit, and leaves the blocked padding untouched.
* A step on packed state equals the same step on per-tensor state: after 3
  steps, the unpacked blocked state and the per-tensor run are bitwise equal.
Lists: arenas at multiples of 8 and at arbitrary element offsets, with and
without the padded index, whole lists and ZeRO shards, flat state buffers, every
state precision (mixed, Kahan, split master, the pure matrix).
"""
import numpy as np
import pytest
import torch

import adamw_optimizer_step_apply_amd as A
import workloads
from gpu_util import Case, blocked_gather, build_blocked_padded, free, hp_pair, same_bits

pytestmark = pytest.mark.gpu

NUMELS = [16384 * 2 + 5, 7, 4099, 1, 0, 20000, 16384, 3]
CODE = {"mixed": A.MIXED, "kahan": A.PURE_KAHAN, "split": A.MIXED_SPLIT}


def _code_prec(mode):
    if mode.startswith("pure"):
        m32, v32, k = workloads.parse_pure(mode)
        return A.MIXED, A.PurePrecision(A.F32 if m32 else A.BF16, A.F32 if v32 else A.BF16, k)
    return CODE[mode], None


def _state_list(case, shard=(0, -1), pad8=True):
    keys = case.keys[2:] + (None,) * (3 - len(case.keys[2:]))
    streams = [None, None] + [None if k is None else [case.arena.view(k, i) for i in range(len(case.numels))]
                              for k in keys]
    return A.TensorList(case.numels, streams, shard[0], shard[1], A.FLAT_PAD8 if pad8 else 0)


@pytest.mark.parametrize("mode", ["mixed", "kahan", "split", "pure-f32-bf16-k", "pure-bf16-f32-n", "pure-bf16-bf16-k32"])
def test_pack_matches_the_tests_own_layout(mode):
    case = Case(mode, NUMELS, seed=8100, align_elems=8, random_moments=True)
    code, prec = _code_prec(mode)
    tl = _state_list(case)
    nbytes = A.adamw_blocked_state_bytes(code, A.BF16, tl, prec)
    blocked = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    A.adamw_blocked_state_copy(code, A.BF16, tl, blocked, True, prec)
    # the arenas' gaps between tensors hold random values: the reference's
    # padding must be the untouched zeros of the packed buffer
    offs = list(case.arena.offsets) + [case.arena.bufs["g"].numel()]
    for k in case.keys[2:]:
        for i, n in enumerate(NUMELS):
            case.arena.bufs[k][offs[i] + n:offs[i + 1]] = 0
    want = build_blocked_padded(case.arena, case.keys[2:], NUMELS)
    assert want.numel() == nbytes
    assert torch.equal(blocked.view(-1), want.view(-1))
    free()


@pytest.mark.parametrize("mode", ["mixed", "kahan", "split"])
@pytest.mark.parametrize("pad8,shard", [(True, (0, -1)), (False, (0, -1)), (False, (5000, 40000)),
                                        (True, (16384, 53256))])
def test_round_trip_and_padding(mode, pad8, shard):
    """Arenas at arbitrary element offsets (streams shifted against each other),
    the plain and the padded index, whole list and shards."""
    shifts = {"mixed": {"m": 3, "master": 1}, "kahan": {"m": 3, "c": 5}, "split": {"m": 3, "r": 2}}[mode]
    case = Case(mode, NUMELS, seed=8200, align_elems=1, random_moments=True, shifts=shifts)
    code, prec = _code_prec(mode)
    tl = _state_list(case, shard, pad8)
    nbytes = A.adamw_blocked_state_bytes(code, A.BF16, tl, prec)
    blocked = torch.full((nbytes,), 0xA5, dtype=torch.uint8, device="cuda")    # padding sentinel
    A.adamw_blocked_state_copy(code, A.BF16, tl, blocked, True, prec)
    # every owned element at its blocked position; everything else still the sentinel
    fa = 8 if pad8 else 1
    starts = np.concatenate([[0], np.cumsum([-(-n // fa) * fa for n in NUMELS])]).astype(np.int64)
    b = shard[0]
    e = int(starts[-1]) if shard[1] < 0 else shard[1]
    flat, tens, elem = [], [], []
    for i, n in enumerate(NUMELS):
        lo, hi = max(b, int(starts[i])), min(e, int(starts[i]) + n)
        if hi > lo:
            flat.append(np.arange(lo, hi))
            tens.append(np.full(hi - lo, i))
            elem.append(np.arange(lo, hi) - starts[i])
    flat, tens, elem = (np.concatenate(x) for x in (flat, tens, elem))
    keys = case.keys[2:]
    dtypes = {k: case.arena.bufs[k].dtype for k in keys}
    B = A.STATE_BLOCK_ELEMS
    nb = -(-(e - b) // B)
    assert nbytes == nb * B * sum(torch.empty(0, dtype=d).element_size() for d in dtypes.values())
    got = blocked_gather(blocked.view(nb, -1), dtypes, torch.from_numpy(flat - b).to("cuda"))
    arena_idx = torch.from_numpy(np.asarray(case.arena.offsets)[tens] + elem).to("cuda")
    for k in keys:
        assert same_bits(got[k], case.arena.bufs[k][arena_idx]), k
    touched = torch.zeros(nbytes, dtype=torch.bool, device="cuda")
    col = 0
    rel = torch.from_numpy(flat - b).to("cuda")
    for k, d in dtypes.items():
        es = torch.empty(0, dtype=d).element_size()
        start = (rel // B) * (B * sum(torch.empty(0, dtype=x).element_size() for x in dtypes.values())) + col + (rel % B) * es
        for j in range(es):
            touched[start + j] = True
        col += B * es
    assert bool((blocked[~touched] == 0xA5).all()), "padding written"
    # back into cleared per-tensor buffers
    before = {k: case.arena.bufs[k].clone() for k in keys}
    for k in keys:
        case.arena.bufs[k].zero_()
    A.adamw_blocked_state_copy(code, A.BF16, tl, blocked, False, prec)
    torch.cuda.synchronize()
    for k in keys:
        ref = before[k].clone()
        mask = torch.zeros(ref.numel(), dtype=torch.bool, device="cuda")
        mask[arena_idx] = True
        ref[~mask] = 0
        assert same_bits(case.arena.bufs[k], ref), k
    free()


@pytest.mark.parametrize("mode", ["mixed", "kahan", "split", "pure-f32-f32-k", "pure-f32-bf16-k32"])
def test_steps_on_packed_state_equal_per_tensor_steps(mode):
    """make_blocked_state from the per-tensor state, then 3 steps each way."""
    a = Case(mode, NUMELS, seed=8300, align_elems=8, random_moments=True)
    b = Case(mode, NUMELS, seed=8300, align_elems=8, random_moments=True)
    code, prec = _code_prec(mode)
    keys = a.keys[2:]
    views = [[b.arena.view(k, i) for i in range(len(NUMELS))] for k in keys]
    blocked, mask = A.make_blocked_state(code, A.BF16, NUMELS, *views, prec=prec)
    tl_b = A.TensorList(NUMELS, [[b.arena.view(k, i) for i in range(len(NUMELS))] for k in b.keys[:2]]
                        + [[blocked], None, None], 0, -1, mask)
    hg, _ = hp_pair()
    for s in range(3):
        if s:
            a.refill_grads(s)
            b.refill_grads(s)
        a.gpu_step(hg)
        if prec is None:
            A.adamw_multi_tensor_step(code, A.BF16, tl_b, hg, b.d_step)
        else:
            A.adamw_pure_multi_tensor_step(prec, tl_b, hg, b.d_step)
    A.adamw_blocked_state_copy(code, A.BF16, _state_list(b), blocked, False, prec)
    torch.cuda.synchronize()
    assert int(a.d_step.item()) == int(b.d_step.item()) == 3
    for k in a.keys:
        assert same_bits(a.arena.bufs[k], b.arena.bufs[k]), k
    free()


def test_flat_state_shard():
    """A ZeRO rank's state as flat shard buffers (flat_mask bits 2-4), packed."""
    numels = [30000, 17, 9000, 40000]
    case = Case("mixed", numels, seed=8400, align_elems=1, random_moments=True)
    b, e = 12345, 70011
    flat = {k: case.arena.bufs[k][b:e].clone() for k in ("m", "v", "master")}
    tl = A.TensorList(numels, [None, None, [flat["m"]], [flat["v"]], [flat["master"]]], b, e, 0b11100)
    nbytes = A.adamw_blocked_state_bytes(A.MIXED, A.BF16, tl)
    blocked = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    A.adamw_blocked_state_copy(A.MIXED, A.BF16, tl, blocked, True)
    B = A.STATE_BLOCK_ELEMS
    nb = -(-(e - b) // B)
    got = blocked_gather(blocked.view(nb, -1), {k: torch.float32 for k in ("m", "v", "master")},
                         torch.arange(e - b, device="cuda"))
    for k in ("m", "v", "master"):
        assert same_bits(got[k], flat[k]), k
    free()


def test_invalid_copy_is_refused_before_any_work():
    case = Case("mixed", [100, 7], seed=8500)
    tl = _state_list(case)
    blocked = torch.zeros(A.adamw_blocked_state_bytes(A.MIXED, A.BF16, tl) + 64, dtype=torch.uint8, device="cuda")
    with pytest.raises(A.AdamWError, match="16-byte"):
        A.adamw_blocked_state_copy(A.MIXED, A.BF16, tl, blocked.data_ptr() + 8, True)
    bad = A.TensorList(case.numels, [None, None, [case.arena.view("m", i) for i in range(2)], None,
                                     [case.arena.view("master", i) for i in range(2)]], 0, -1, A.FLAT_PAD8)
    with pytest.raises(A.AdamWError, match="exp_avg_sq"):
        A.adamw_blocked_state_copy(A.MIXED, A.BF16, bad, blocked, True)
    assert bool((blocked == 0).all())
    free()


def test_copy_under_graph_capture_is_refused():
    """The copy allocates its table and waits for itself: on a stream under
    capture it is refused before anything is recorded, and the capture goes on
    (the graph holds the other work and replays it)."""
    case = Case("mixed", [100, 7], seed=8600)
    tl = _state_list(case)
    blocked = torch.zeros(A.adamw_blocked_state_bytes(A.MIXED, A.BF16, tl), dtype=torch.uint8, device="cuda")
    x = torch.zeros(4, device="cuda")
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        x.add_(1.0)
        with pytest.raises(A.AdamWError, match="cannot be captured"):
            A.adamw_blocked_state_copy(A.MIXED, A.BF16, tl, blocked, True, stream=s)
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    assert float(x[0]) == 2.0
    assert bool((blocked == 0).all())
    del g
    free()


def test_full_size_checkpoint_round_trip():
    """Checkpointing blocked state at the OPT-1.3B size: 3 mixed steps on blocked
    state, then the state unpacked into fresh per-tensor tensors (the usual
    checkpoint form) and packed again into a new blocked buffer; the two buffers
    are byte-identical, and 2 more steps from each (each with its own copy of the
    params) stay bit-identical with each other."""
    wl = workloads.get("opt_1_3b")
    numels = wl.numels
    arena = workloads.make_state("mixed", numels, "cuda", 8700, align_elems=8, random_moments=True)
    view = lambda k: [arena.view(k, i) for i in range(len(numels))]   # noqa: E731
    blocked_a, mask = A.make_blocked_state(A.MIXED, A.BF16, numels, view("m"), view("v"), view("master"))
    for k in ("m", "v", "master"):
        arena.bufs[k] = arena.bufs[k][:0]        # the per-tensor state is not used again
    free()
    params_a = arena.bufs["p"]
    grads = view("g")
    hg, _ = hp_pair()
    d_a = torch.zeros(1, dtype=torch.int32, device="cuda")
    tl_a = A.TensorList(numels, [view("p"), grads, [blocked_a], None, None], 0, -1, mask)
    for _ in range(3):
        A.adamw_multi_tensor_step(A.MIXED, A.BF16, tl_a, hg, d_a)
    # checkpoint: out to per-tensor tensors, then into a new blocked buffer
    ck = {k: [torch.empty(n, dtype=torch.float32, device="cuda") for n in numels] for k in ("m", "v", "master")}
    state_tl = A.TensorList(numels, [None, None, ck["m"], ck["v"], ck["master"]], 0, -1, A.FLAT_PAD8)
    A.adamw_blocked_state_copy(A.MIXED, A.BF16, state_tl, blocked_a, False)
    blocked_b, mask_b = A.make_blocked_state(A.MIXED, A.BF16, numels, ck["m"], ck["v"], ck["master"])
    assert mask_b == mask and same_bits(blocked_a, blocked_b)
    del ck, state_tl
    free()
    params_b = params_a.clone()
    d_b = d_a.clone()
    offs = arena.offsets
    tl_b = A.TensorList(numels, [[params_b[o:o + n] for o, n in zip(offs, numels)], grads, [blocked_b], None, None],
                        0, -1, mask)
    for _ in range(2):
        A.adamw_multi_tensor_step(A.MIXED, A.BF16, tl_a, hg, d_a)
        A.adamw_multi_tensor_step(A.MIXED, A.BF16, tl_b, hg, d_b)
    torch.cuda.synchronize()
    assert int(d_a.item()) == int(d_b.item()) == 5
    assert same_bits(blocked_a, blocked_b) and same_bits(params_a, params_b)
    del tl_a, tl_b, blocked_a, blocked_b, params_b, arena
    free()
