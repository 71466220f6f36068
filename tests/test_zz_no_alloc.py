"""GPU: adamw_multi_tensor_step_noalloc, the allocation-free form of
adamw_multi_tensor_step, against that entry point.

Twin copies of the same seeded state take the same steps, one through each
entry point (called through the C ABI); after every call every buffer and the
counter must be bitwise equal, and the allocation-free copy is also held to
the oracle.  Two calls in a row, the second with a smaller list (so the
workspace's table is replaced by a shorter one), in both launch forms, then
the first list again, a skipped step, and a list whose table does not fit,
which must be refused with nothing enqueued.
"""
import pytest
import torch

import adamw_optimizer_step_apply_amd as A
from gpu_util import Case, build_blocked_padded, free, hp_pair, same_bits

pytestmark = pytest.mark.gpu

LARGE = [40000, 7, 4099, 1, 16384 * 5 + 3, 0, 2048]
SMALL = [9, 100, 3]
CODE = {"mixed": A.MIXED, "kahan": A.PURE_KAHAN, "split": A.MIXED_SPLIT}


@pytest.fixture
def single_launch_limit():
    yield A.adamw_set_single_launch_max_workgroups
    A.adamw_set_single_launch_max_workgroups(-1)


def _pair(mode, numels, seed, p_dtype="bf16"):
    scale = 65536.0 if p_dtype == "f16" else 1.0
    a = Case(mode, numels, seed=seed, p_dtype=p_dtype, loss_scale=scale, random_moments=True)
    b = Case(mode, numels, seed=seed, p_dtype=p_dtype, loss_scale=scale, random_moments=True)
    return a, b


def _same(a, b, label):
    torch.cuda.synchronize()
    assert int(a.d_step.item()) == int(b.d_step.item()), label
    for k in a.keys:
        assert same_bits(a.arena.bufs[k], b.arena.bufs[k]), f"{label}: {k}"


def _both(mode, a, b, hg, flag=None):
    dt = A.F16 if a.p_dtype == "f16" else A.BF16
    A.adamw_multi_tensor_step_noalloc(CODE[mode], dt, a.tensor_list(), hg, a.d_step, flag)
    A.adamw_multi_tensor_step(CODE[mode], dt, b.tensor_list(), hg, b.d_step, flag)


@pytest.mark.parametrize("limit", [-1, 0])
@pytest.mark.parametrize("mode,p_dtype", [("mixed", "bf16"), ("mixed", "f16"), ("kahan", "bf16"), ("split", "bf16")])
def test_noalloc_matches_the_allocating_step(mode, p_dtype, limit, single_launch_limit):
    single_launch_limit(limit)
    scale = 65536.0 if p_dtype == "f16" else 1.0
    hg, ho = hp_pair(inv_scale=1.0 / scale)
    big_a, big_b = _pair(mode, LARGE, 7100, p_dtype)
    small_a, small_b = _pair(mode, SMALL, 7101, p_dtype)
    # two calls in a row, the second with a smaller input; the oracle follows
    # the allocation-free copy
    _both(mode, big_a, big_b, hg)
    big_a.oracle_step(ho)
    _same(big_a, big_b, "large list")
    _both(mode, small_a, small_b, hg)
    small_a.oracle_step(ho)
    _same(small_a, small_b, "smaller list")
    # the larger list again (its table goes back in), twice (the second call reuses it)
    for s in range(2):
        big_a.refill_grads(s + 1)
        big_b.refill_grads(s + 1)
        _both(mode, big_a, big_b, hg)
        big_a.oracle_step(ho)
        _same(big_a, big_b, f"large list again ({s})")
    # a skipped step changes nothing in either
    flag = torch.ones(1, dtype=torch.int32, device="cuda")
    _both(mode, small_a, small_b, hg, flag)
    _same(small_a, small_b, "skipped")
    big_a.compare_all(f"noalloc-{mode}-{p_dtype}-{limit}")
    small_a.compare_all(f"noalloc-small-{mode}-{p_dtype}-{limit}")
    free()


def test_noalloc_refuses_a_table_too_large():
    """300,000 one-element tensors: 300,000 segments of 64 bytes exceed the
    workspace; the call is refused and neither the buffers nor the counter
    change.  A list that fits still runs afterwards."""
    n = 300_000
    case = Case("mixed", [1] * n, seed=7200, align_elems=8)
    before = {k: case.arena.bufs[k].clone() for k in case.keys}
    # the list's addresses, element i of every arena (integers: no 1.5M tensor views)
    streams = [[case.arena.bufs[k].data_ptr() + 8 * i * case.arena.bufs[k].element_size() for i in range(n)]
               for k in case.keys]
    tl = A.TensorList([1] * n, streams)
    hg, _ = hp_pair()
    with pytest.raises(A.AdamWError, match="allocation-free step holds at most"):
        A.adamw_multi_tensor_step_noalloc(A.MIXED, A.BF16, tl, hg, case.d_step)
    torch.cuda.synchronize()
    assert int(case.d_step.item()) == 0
    for k, v in before.items():
        assert same_bits(case.arena.bufs[k], v), k
    a, b = _pair("mixed", SMALL, 7201)
    _both("mixed", a, b, hg)
    _same(a, b, "after a refused call")
    free()


def test_noalloc_on_a_side_stream_and_blocked_state():
    """A side stream, and the OPT-shaped blocked-state layout of bench.py at a
    reduced size (the table holds one segment per 16384-element block)."""
    numels = [16384 * 3, 2048, 16384 * 2 + 8, 8]
    # arenas at multiples of 8 elements: the padded flat index itself
    a, b = (Case("mixed", numels, seed=7300, align_elems=8, random_moments=True) for _ in range(2))
    tl = {}
    for name, c in (("a", a), ("b", b)):
        blocked = build_blocked_padded(c.arena, c.keys[2:], numels)
        streams = [[c.arena.view(k, i) for i in range(len(numels))] for k in c.keys[:2]]
        tl[name] = (A.TensorList(numels, streams + [[blocked], None, None], 0, -1, A.BLOCKED_STATE | A.FLAT_PAD8),
                    blocked)
    hg, _ = hp_pair()
    s = torch.cuda.Stream()
    for _ in range(3):
        A.adamw_multi_tensor_step_noalloc(A.MIXED, A.BF16, tl["a"][0], hg, a.d_step, None, s)
        A.adamw_multi_tensor_step(A.MIXED, A.BF16, tl["b"][0], hg, b.d_step, None, s)
    s.synchronize()
    assert int(a.d_step.item()) == int(b.d_step.item()) == 3
    assert same_bits(tl["a"][1], tl["b"][1])
    assert same_bits(a.arena.bufs["p"], b.arena.bufs["p"])
    free()


def test_noalloc_table_pinned_by_a_captured_graph():
    """A step captured into a HIP graph through the allocation-free entry point
    pins the table that its replays read: a later call with another list is
    refused with nothing enqueued, calls with the same list still run, and every
    replay matches the allocating entry point's eager step bit for bit (and the
    oracle).  adamw_release_workspace releases the pin: the other list runs
    afterwards."""
    hg, ho = hp_pair()
    g_case, e_case = _pair("mixed", LARGE, 7400)
    other_a, other_b = _pair("mixed", SMALL, 7401)
    tl_g, tl_e = g_case.tensor_list(), e_case.tensor_list()
    s = torch.cuda.Stream()

    def eager_pair(noalloc=True):
        if noalloc:
            A.adamw_multi_tensor_step_noalloc(A.MIXED, A.BF16, tl_g, hg, g_case.d_step, None, s)
        A.adamw_multi_tensor_step(A.MIXED, A.BF16, tl_e, hg, e_case.d_step, None, s)
        s.synchronize()
        g_case.oracle_step(ho)
        _same(g_case, e_case, "eager")

    eager_pair()                         # the table goes in outside capture
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        A.adamw_multi_tensor_step_noalloc(A.MIXED, A.BF16, tl_g, hg, g_case.d_step, None, s)
    torch.cuda.synchronize()
    before = {k: other_a.arena.bufs[k].clone() for k in other_a.keys}
    with pytest.raises(A.AdamWError, match="captured into a graph"):
        A.adamw_multi_tensor_step_noalloc(A.MIXED, A.BF16, other_a.tensor_list(), hg, other_a.d_step, None, s)
    torch.cuda.synchronize()
    assert int(other_a.d_step.item()) == 0
    for k, v in before.items():
        assert same_bits(other_a.arena.bufs[k], v), k
    for r in range(3):
        with torch.cuda.stream(s):
            graph.replay()
        eager_pair(noalloc=False)
        assert int(g_case.d_step.item()) == r + 2
    eager_pair()                         # the same list, eagerly, while pinned
    g_case.compare_all("noalloc-graph")
    del graph
    torch.cuda.synchronize()
    A.adamw_release_workspace()
    _both("mixed", other_a, other_b, hg)
    other_a.oracle_step(ho)
    _same(other_a, other_b, "after the release")
    other_a.compare_all("noalloc-after-release")
    free()
