"""GPU: the step counter's range and HIP-graph capture against the plan cache.

* A step runs only from a counter in [0, INT32_MAX): from INT32_MAX - 1 the
  step t = INT32_MAX is taken (and matches the oracle at that t); from
  INT32_MAX, or from a negative counter, the call writes nothing at all -- no
  buffer, no counter, no loss scale -- in both launch forms.
* A step captured into a graph keeps working after the capture stream has
  stepped 11 other lists (more than the stream's 8 cached plans, one of them
  with a larger chunk table): the captured plan slot is pinned.  A capture
  whose table was never uploaded is refused before anything is recorded.
"""
import pytest
import torch

import adamw_optimizer_step_apply_amd as A
from gpu_util import Case, free, hp_pair, same_bits

pytestmark = pytest.mark.gpu

INT32_MAX = 2 ** 31 - 1
SIZES = [0, 1, 7, 8, 9, 2047, 2048, 2049, 16385, 100_003, 3, 40_000]


@pytest.fixture
def single_launch_limit():
    yield A.adamw_set_single_launch_max_workgroups
    A.adamw_set_single_launch_max_workgroups(-1)


def _snapshot(case):
    return {k: case.arena.bufs[k].clone() for k in case.keys}


def _unchanged(case, snap, label):
    torch.cuda.synchronize()
    for k, v in snap.items():
        assert same_bits(case.arena.bufs[k], v), f"{label}: {k} written"


@pytest.mark.parametrize("limit", [-1, 0])
@pytest.mark.parametrize("mode", ["mixed", "kahan", "split"])
def test_counter_saturates_without_writing(mode, limit, single_launch_limit):
    """limit -1: the single-launch form (the list is small); 0: prologue + update."""
    single_launch_limit(limit)
    case = Case(mode, SIZES, seed=6100, random_moments=True)
    case.d_step.fill_(INT32_MAX - 1)
    case.step = INT32_MAX - 1
    hg, ho = hp_pair()
    case.gpu_step(hg)
    case.oracle_step(ho)
    case.compare_all(f"saturate-{mode}-{limit}-last")
    assert case.step == INT32_MAX
    for s, start in enumerate([INT32_MAX, -1, -1000]):
        case.d_step.fill_(start)
        case.refill_grads(s + 1)
        snap = _snapshot(case)
        case.gpu_step(hg)
        _unchanged(case, snap, f"counter {start}")
        assert int(case.d_step.item()) == start
    free()


@pytest.mark.parametrize("limit", [-1, 0])
def test_counter_saturation_keeps_the_loss_scale(limit, single_launch_limit):
    single_launch_limit(limit)
    case = Case("mixed", SIZES, seed=6101, p_dtype="f16", loss_scale=1024.0)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    scale = A.loss_scale_state(1024.0)
    hg, _ = hp_pair()
    tl = case.tensor_list()
    for found_inf in (0, 1):
        case.d_step.fill_(INT32_MAX)
        flag.fill_(found_inf)
        snap = _snapshot(case)
        before = scale.clone()
        A.adamw_multi_tensor_step_amp(A.MIXED, A.F16, tl, hg, case.d_step, flag, scale, A.LossScaler(2.0, 0.5, 1))
        _unchanged(case, snap, f"amp found_inf={found_inf}")
        assert int(case.d_step.item()) == INT32_MAX
        assert same_bits(scale, before), "loss scale advanced on a saturated counter"
    free()


def test_capture_survives_plan_cache_cycling():
    numels = [40000, 7, 4099, 1, 16384 * 3 + 5]
    graphed = Case("mixed", numels, seed=6200, random_moments=True)
    eager = Case("mixed", numels, seed=6200, random_moments=True)
    hg, ho = hp_pair()
    s = torch.cuda.Stream()
    tlg, tle = graphed.tensor_list(), eager.tensor_list()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):          # warm-up: workspace and plan on the capture stream
        A.adamw_multi_tensor_step(A.MIXED, A.BF16, tlg, hg, graphed.d_step, None, s)
    s.synchronize()
    A.adamw_multi_tensor_step(A.MIXED, A.BF16, tle, hg, eager.d_step)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        A.adamw_multi_tensor_step(A.MIXED, A.BF16, tlg, hg, graphed.d_step, None, s)
    # 11 other lists on the capture stream: more than its 8 unpinned plan slots;
    # the last one needs a larger table than any slot holds
    others = [Case("kahan", [1000 + 97 * i, 3 + i], seed=6300 + i) for i in range(10)]
    others.append(Case("kahan", [16384 * 40 + 1] * 6 + [5] * 300, seed=6399))
    for o in others:
        A.adamw_multi_tensor_step(A.PURE_KAHAN, A.BF16, o.tensor_list(), hg, o.d_step, None, s)
    s.synchronize()
    for r in range(3):
        g.replay()
        A.adamw_multi_tensor_step(A.MIXED, A.BF16, tle, hg, eager.d_step)
        torch.cuda.synchronize()
        assert int(graphed.d_step.item()) == int(eager.d_step.item()) == r + 2
        for k in eager.keys:
            assert same_bits(graphed.arena.bufs[k], eager.arena.bufs[k]), (r, k)
    # and the replayed steps are the oracle's steps
    for _ in range(4):
        graphed.oracle_step(ho)
    graphed.compare_all("capture-after-cycling")
    del g, others
    free()


def test_capture_of_an_unplanned_list_is_refused():
    case = Case("mixed", [1000, 9], seed=6400)
    other = Case("mixed", [333, 4097], seed=6401)
    hg, _ = hp_pair()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        A.adamw_multi_tensor_step(A.MIXED, A.BF16, case.tensor_list(), hg, case.d_step, None, s)
    s.synchronize()
    snap = _snapshot(other)
    x = torch.zeros(16, device="cuda")
    g = torch.cuda.CUDAGraph()
    with pytest.raises(A.AdamWError, match="before capturing"):
        with torch.cuda.graph(g, stream=s):
            x.add_(1.0)                   # the graph holds some work besides the refused call
            A.adamw_multi_tensor_step(A.MIXED, A.BF16, other.tensor_list(), hg, other.d_step, None, s)
    torch.cuda.synchronize()
    _unchanged(other, snap, "refused capture")
    assert int(other.d_step.item()) == 0
    # the stream still works eagerly with that list afterwards
    A.adamw_multi_tensor_step(A.MIXED, A.BF16, other.tensor_list(), hg, other.d_step, None, s)
    s.synchronize()
    assert int(other.d_step.item()) == 1
    del g
    free()
