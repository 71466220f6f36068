"""Address-level check of the launch plan, on the CPU (no GPU, no HIP call).

For every chunk of a plan, ``adamw_plan_inspect_bytes`` returns the byte range
[lo, hi) of each stream that the chunk's workgroups read and write, taken from
the very segment and chunk tables the kernels receive.  These tests rebuild,
independently of the planner, where every element of the list lives in each
stream for the layout the caller handed in (per-tensor buffers, one flat shard
buffer, or the blocked state buffer of the padded flat index) and require:

* per chunk and stream: the range is exactly that of the chunk's elements
  (tensor, offset and count from ``adamw_plan_inspect``) at their addresses in
  that stream, and a blocked-state range stays inside one block's sub-array;
* per stream: the chunks' ranges never overlap, and their union is exactly the
  bytes of the elements the step owns -- so nothing outside the caller's
  buffers (or in the padding of the padded index) is touched, and no element
  is updated twice;
* vector chunks hold whole 8-element packs at 16-byte-aligned addresses in
  every stream (the kernels' dwordx4 accesses).

Layouts: the exact ones bench.py builds (the 10,000-tensor fp16 list on
blocked state in the padded index, and per tensor; OPT-1.3B on both), the BERT
list's four ZeRO shards, 200 seeded random lists, and 150 more that hypothesis
draws (and shrinks on a failure).  Base addresses are synthetic
(never dereferenced); torch allocations start on 2 MiB boundaries for buffers
this large, which the synthetic bases follow.
"""
import numpy as np
import pytest

import adamw_optimizer_step_apply_amd as A
import bench
import workloads

B = A.STATE_BLOCK_ELEMS
MiB2 = 1 << 21

# element sizes of the five streams per launch kind
ESZ = {
    ("mixed", "bf16"): (2, 2, 4, 4, 4), ("mixed", "f16"): (2, 2, 4, 4, 4),
    ("kahan", "bf16"): (2, 2, 2, 2, 2), ("split", "bf16"): (2, 2, 4, 4, 2),
    ("check", "f16"): (0, 2, 0, 0, 0), ("check", "bf16"): (0, 2, 0, 0, 0),
}
CODE = {"mixed": A.MIXED, "kahan": A.PURE_KAHAN, "split": A.MIXED_SPLIT}
DT = {"bf16": A.BF16, "f16": A.F16}


def pure_esz(m32, v32, kahan):
    """Element sizes of a pure step's streams; kahan 0 (none), 1 (bf16) or 2 (fp32 compensation)."""
    return (2, 2, 4 if m32 else 2, 4 if v32 else 2, (0, 2, 4)[int(kahan)])


class Spec:
    """A tensor list as handed to the library: per stream either per-tensor
    start addresses, one flat shard buffer, or (streams 2-4) the blocked buffer."""

    def __init__(self, numels, esz, ptrs, shard=(0, -1), flat_mask=0):
        self.numels = np.asarray(numels, dtype=np.int64)
        self.esz = tuple(esz)
        self.ptrs = ptrs                  # list of 5: list of ints, or None
        self.b, self.shard_end = shard
        self.flat_mask = flat_mask
        self.blocked = bool(flat_mask & A.BLOCKED_STATE) and any(self.esz[2:])
        fa = 8 if flat_mask & A.FLAT_PAD8 else 1
        padded = -(-self.numels // fa) * fa
        self.start = np.concatenate([[0], np.cumsum(padded)[:-1]]).astype(np.int64)
        self.total = int(padded.sum())
        self.e = self.total if self.shard_end < 0 else self.shard_end
        # blocked state: [exp_avg x B][exp_avg_sq x B][aux x B] per block
        self.soff = [0] * 5
        acc = 0
        for s in (2, 3, 4):
            self.soff[s] = acc
            acc += B * self.esz[s]
        self.block_bytes = acc

    def tensor_list(self):
        return A.TensorList(self.numels.tolist(), self.ptrs, self.b, self.shard_end, self.flat_mask)

    def kind(self, s):
        if self.blocked and s >= 2:
            return "blocked"
        return "flat" if (self.flat_mask >> s) & 1 else "tensor"

    def addr(self, s, t, flat):
        """Addresses in stream s of flat positions `flat` of tensors `t` (arrays)."""
        k, e = self.kind(s), self.esz[s]
        if k == "tensor":
            base = np.asarray(self.ptrs[s], dtype=np.int64)[t]
            return base + (flat - self.start[t]) * e
        if k == "flat":
            return self.ptrs[s][0] + (flat - self.b) * e
        rel = flat - self.b
        return self.ptrs[2][0] + (rel // B) * self.block_bytes + self.soff[s] + (rel % B) * e

    def owned_intervals(self):
        """(tensor, flat lo, flat hi) of the elements the step owns, split at
        block edges when the state is blocked."""
        lo = np.maximum(self.start, self.b)
        hi = np.minimum(self.start + self.numels, self.e)
        keep = hi > lo
        t, lo, hi = np.flatnonzero(keep), lo[keep], hi[keep]
        if not self.blocked:
            return t, lo, hi
        k0 = (lo - self.b) // B
        k1 = (hi - 1 - self.b) // B
        reps = (k1 - k0 + 1).astype(np.int64)
        t, lo_r, hi_r, k0_r = (np.repeat(x, reps) for x in (t, lo, hi, k0))
        j = np.arange(reps.sum()) - np.repeat(np.cumsum(reps) - reps, reps)
        blk = k0_r + j
        plo = np.maximum(lo_r, self.b + blk * B)
        phi = np.minimum(hi_r, self.b + (blk + 1) * B)
        return t, plo, phi


def merge(lo, hi):
    """Sorted, merged [lo, hi) intervals; asserts that the inputs do not overlap."""
    o = np.argsort(lo, kind="stable")
    lo, hi = lo[o], hi[o]
    if lo.size > 1:
        bad = np.flatnonzero(lo[1:] < hi[:-1])
        assert bad.size == 0, f"overlapping ranges at {lo[bad[0]]:#x}..{hi[bad[0]]:#x} / {lo[bad[0] + 1]:#x}"
    if lo.size == 0:
        return lo, hi
    starts = np.concatenate([[True], lo[1:] != hi[:-1]])
    ends = np.concatenate([lo[1:] != hi[:-1], [True]])
    return lo[starts], hi[ends]


def check_plan(spec, code, dt, for_check=False, prec=None):
    tl = spec.tensor_list()
    rows, rng = A.adamw_plan_inspect_bytes(code, dt, tl, for_check, prec)
    rng = rng.astype(np.int64)
    if prec is None:
        # the same plan through the row-only export
        assert np.array_equal(rows, np.asarray(A.adamw_plan_inspect(code, dt, tl, for_check),
                                               dtype=np.int64).reshape(-1, 6))
    t, off, cnt, vec, flat = rows[:, 0], rows[:, 1], rows[:, 2], rows[:, 3].astype(bool), rows[:, 4]
    assert np.all(cnt > 0)
    assert np.array_equal(flat, spec.start[t] + off), "chunk flat position disagrees with its tensor offset"
    # vector chunks: whole packs
    assert np.all(cnt[vec] % 8 == 0)
    t_own, lo_own, hi_own = spec.owned_intervals()
    for s in range(5):
        e = spec.esz[s]
        lo, hi = rng[:, s, 0], rng[:, s, 1]
        if e == 0:
            assert not lo.any() and not hi.any(), f"stream {s} is not used but has ranges"
            continue
        # per chunk: exactly the chunk's elements at their addresses in this stream
        want = spec.addr(s, t, flat)
        assert np.array_equal(lo, want), f"stream {s}: chunk start address differs"
        assert np.array_equal(hi - lo, cnt * e), f"stream {s}: chunk length differs"
        if spec.kind(s) == "blocked":
            assert np.all((flat - spec.b) % B + cnt <= B), f"stream {s}: chunk crosses a state block"
        assert np.all(lo[vec] % 16 == 0), f"stream {s}: vector chunk not 16-byte aligned"
        # per stream: disjoint, and together exactly the owned elements' bytes
        got_lo, got_hi = merge(lo, hi)
        exp_lo, exp_hi = merge(spec.addr(s, t_own, lo_own), spec.addr(s, t_own, lo_own) + (hi_own - lo_own) * e)
        assert np.array_equal(got_lo, exp_lo) and np.array_equal(got_hi, exp_hi), \
            f"stream {s}: bytes touched differ from the owned elements' bytes"
    return rows.shape[0]


def arena_ptrs(base, numels, align, esz):
    offs, _ = workloads.aligned_offsets([int(n) for n in numels], align)
    return [base + o * esz for o in offs]


def bench_spec(mode, numels, esz):
    """The list exactly as bench.make_mode_state and bench.main build it."""
    align, flags, nb = bench.state_layout(mode, numels)
    bases = [(1 << 40) + k * (1 << 38) for k in range(6)]     # one 2 MiB-aligned allocation per arena
    ptrs = [arena_ptrs(bases[s], numels, align, esz[s]) if esz[s] else None for s in range(5)]
    if nb:
        ptrs[2], ptrs[3], ptrs[4] = [bases[5]], None, None
    return Spec(numels, esz, ptrs, (0, -1), flags)


@pytest.mark.parametrize("mode", ["f16amp-blocked", "f16amp"])
def test_ragged_10k_bench_layout(mode):
    """The 10,000-tensor fp16 list (2.77e9 elements) as bench.py lays it out:
    the step plan and the overflow check's plan."""
    wl = workloads.get("ragged_10k")
    spec = bench_spec(mode.replace("f16amp", "mixed"), wl.numels, ESZ[("mixed", "f16")])
    n = check_plan(spec, A.MIXED, A.F16)
    assert n > 169_000
    chk = Spec(wl.numels, ESZ[("check", "f16")], [None, spec.ptrs[1], None, None, None], (0, -1), spec.flat_mask)
    check_plan(chk, A.MIXED, A.F16, for_check=True)


@pytest.mark.parametrize("mode", ["mixed", "kahan", "split"])
@pytest.mark.parametrize("blocked", [True, False])
def test_opt13b_bench_layout(mode, blocked):
    wl = workloads.get("opt_1_3b")
    m = mode + ("-blocked" if blocked else "")
    check_plan(bench_spec(m, wl.numels, ESZ[(mode, "bf16")]), CODE[mode], A.BF16)


@pytest.mark.parametrize("rank", [0, 1, 2, 3])
@pytest.mark.parametrize("layout", ["per_tensor", "flat_state", "blocked_state"])
def test_bert_zero_shards(rank, layout):
    """The BERT list at DP=4: each rank's shard with per-tensor buffers (the GPU
    tests' layout), with flat shard buffers for grad and state (a ZeRO rank's
    reduce-scattered grads and its own state), and with blocked state."""
    wl = workloads.get("bert_52m")
    b, e = wl.shard(rank)
    esz = ESZ[("mixed", "bf16")]
    bases = [(1 << 40) + k * (1 << 36) for k in range(6)]
    ptrs = [arena_ptrs(bases[s], wl.numels, 128, esz[s]) for s in range(5)]
    mask = 0
    if layout == "flat_state":
        mask = 0b11110
        for s in range(1, 5):
            ptrs[s] = [bases[s] + 64 * s]
    elif layout == "blocked_state":
        mask = A.BLOCKED_STATE
        ptrs[2], ptrs[3], ptrs[4] = [bases[5]], None, None
    check_plan(Spec(wl.numels, esz, ptrs, (b, e), mask), A.MIXED, A.BF16)


def _random_spec(rng):
    kinds = [("mixed", "bf16"), ("mixed", "f16"), ("kahan", "bf16"), ("split", "bf16"), ("pure", "bf16"),
             ("check", "f16"), ("check", "bf16")]
    kind, dt = kinds[int(rng.integers(len(kinds)))]
    prec = None
    if kind == "pure":
        m32, v32 = (bool(rng.integers(2)) for _ in range(2))
        kahan = int(rng.integers(3))
        prec = A.PurePrecision(A.F32 if m32 else A.BF16, A.F32 if v32 else A.BF16, kahan)
        esz = pure_esz(m32, v32, kahan)
    else:
        esz = ESZ[(kind, dt)]
    nt = int(rng.integers(0, 40))
    size_kind = rng.integers(3, size=nt)
    numels = np.where(size_kind == 0, rng.integers(0, 9, size=nt),
                      np.where(size_kind == 1, rng.integers(9, 3000, size=nt), rng.integers(3000, 70000, size=nt)))
    blocked = kind != "check" and bool(rng.integers(2))
    pad8 = bool(rng.integers(2))
    mask = (A.BLOCKED_STATE if blocked else 0) | (A.FLAT_PAD8 if pad8 else 0)
    fa = 8 if pad8 else 1
    total = int((-(-numels // fa) * fa).sum())
    if rng.integers(2) and total:
        b = int(rng.integers(0, total + 1))
        e = int(rng.integers(b, total + 1))
        if pad8 and rng.integers(2):
            b -= b % 8
        shard = (b, e)
    else:
        shard = (0, -1)
    L = (total if shard[1] < 0 else shard[1]) - shard[0]
    ptrs = []
    for s in range(5):
        if not esz[s]:
            ptrs.append(None)
            continue
        base = (1 << 40) + s * (1 << 34) + MiB2 * int(rng.integers(0, 64))
        flat = not (blocked and s >= 2) and bool(rng.integers(2)) and (shard[1] >= 0 or rng.integers(2))
        if flat:
            mask |= 1 << s
            ptrs.append([base + esz[s] * int(rng.integers(0, 8))])    # element-aligned, any 16-byte phase
            continue
        shift = int(rng.integers(0, 8)) if rng.integers(2) else 0
        align = int(rng.choice([1, 8, 128]))
        ptrs.append(arena_ptrs(base + shift * esz[s], numels, align, esz[s]))
    if blocked:
        ptrs[2], ptrs[3], ptrs[4] = [(1 << 40) + 5 * (1 << 34) + 256 * int(rng.integers(0, 64))], None, None
    del L
    return Spec(numels, esz, ptrs, shard, mask), kind, dt, prec


def test_random_lists():
    rng = np.random.default_rng(np.random.SeedSequence([8, 200]))
    seen = set()
    for _ in range(200):
        spec, kind, dt, prec = _random_spec(rng)
        code = CODE.get(kind, A.MIXED)
        check_plan(spec, code, DT[dt], for_check=kind == "check", prec=prec)
        seen.add((kind, spec.blocked, bool(spec.flat_mask & A.FLAT_PAD8)))
    assert len(seen) >= 12


def test_checker_is_not_vacuous():
    """The checker must fail when its picture of the layout is off by one
    element in a tensor start, or by one element in a blocked sub-array."""
    numels = [1000, 7, 20000, 3]
    esz = ESZ[("mixed", "bf16")]

    def spec(mask=0):
        ptrs = [arena_ptrs((1 << 40) + s * (1 << 34), numels, 8, esz[s]) for s in range(5)]
        if mask & A.BLOCKED_STATE:
            ptrs[2], ptrs[3], ptrs[4] = [(1 << 40) + 5 * (1 << 34)], None, None
        return Spec(numels, esz, ptrs, (0, -1), mask)

    check_plan(spec(), A.MIXED, A.BF16)
    check_plan(spec(A.BLOCKED_STATE | A.FLAT_PAD8), A.MIXED, A.BF16)
    bad = spec()
    bad.start = bad.start + np.array([0, 1, 1, 1])
    with pytest.raises(AssertionError):
        check_plan(bad, A.MIXED, A.BF16)
    bad = spec(A.BLOCKED_STATE | A.FLAT_PAD8)
    bad.soff[4] += 4
    with pytest.raises(AssertionError):
        check_plan(bad, A.MIXED, A.BF16)


@pytest.mark.parametrize("mode,prec,state_bytes", [
    ("mixed", None, 12), ("kahan", None, 6), ("split", None, 10),
    ("pure", (True, False, True), 8), ("pure", (False, True, False), 6), ("pure", (False, False, 2), 8)])
@pytest.mark.parametrize("pad8,shard", [(True, (0, -1)), (False, (0, -1)), (False, (1000, 300000)),
                                        (True, (16384, 16384 * 3 + 8))])
def test_blocked_state_bytes(mode, prec, state_bytes, pad8, shard):
    """Whole blocks of 16384 elements over the shard's length, each holding the
    state streams' bytes (no GPU: the query plans only)."""
    numels = [100_000, 7, 65_536, 3, 250_001]
    pc = None if prec is None else A.PurePrecision(A.F32 if prec[0] else A.BF16, A.F32 if prec[1] else A.BF16,
                                                   prec[2])
    esz = pure_esz(*prec) if prec else ESZ[(mode, "bf16")]
    ptrs = [None, None] + [arena_ptrs((1 << 40) + s * (1 << 34), numels, 8, esz[s]) if esz[s] else None
                           for s in (2, 3, 4)]
    tl = A.TensorList(numels, ptrs, shard[0], shard[1], A.FLAT_PAD8 if pad8 else 0)
    fa = 8 if pad8 else 1
    total = sum(-(-n // fa) * fa for n in numels)
    length = (total if shard[1] < 0 else shard[1]) - shard[0]
    assert A.adamw_blocked_state_bytes(CODE.get(mode, A.MIXED), A.BF16, tl, pc) == \
        -(-length // B) * B * state_bytes


def test_blocked_state_bytes_refuses_bad_lists():
    numels = [1000, 5]
    ptrs = [None, None] + [arena_ptrs((1 << 40) + s * (1 << 34), numels, 8, 4) for s in (2, 3, 4)]
    with pytest.raises(A.AdamWError, match="BLOCKED_STATE"):
        A.adamw_blocked_state_bytes(A.MIXED, A.BF16, A.TensorList(numels, ptrs, 0, -1, A.BLOCKED_STATE))
    bad = list(ptrs)
    bad[3] = None
    with pytest.raises(A.AdamWError, match="exp_avg_sq"):
        A.adamw_blocked_state_bytes(A.MIXED, A.BF16, A.TensorList(numels, bad))
    misaligned = list(ptrs)
    misaligned[4] = [p + 2 for p in ptrs[4]]
    with pytest.raises(A.AdamWError, match="aligned"):
        A.adamw_blocked_state_bytes(A.MIXED, A.BF16, A.TensorList(numels, misaligned))


# The same check driven by hypothesis: it draws the list, the layout and the
# shard itself, and shrinks a failing case to a small one.
from hypothesis import HealthCheck, given, settings  # noqa: E402
from hypothesis import strategies as st  # noqa: E402

_KINDS = [("mixed", "bf16"), ("mixed", "f16"), ("kahan", "bf16"), ("split", "bf16"), ("pure", "bf16"),
          ("check", "f16")]


@st.composite
def _plans(draw):
    kind, dt = draw(st.sampled_from(_KINDS))
    prec = None
    if kind == "pure":
        m32, v32 = draw(st.booleans()), draw(st.booleans())
        kahan = draw(st.integers(0, 2))
        prec = A.PurePrecision(A.F32 if m32 else A.BF16, A.F32 if v32 else A.BF16, kahan)
        esz = pure_esz(m32, v32, kahan)
    else:
        esz = ESZ[(kind, dt)]
    numels = np.array(draw(st.lists(st.one_of(st.integers(0, 20), st.integers(0, 3 * B + 17)), max_size=12)),
                      dtype=np.int64)
    blocked = kind != "check" and draw(st.booleans())
    pad8 = draw(st.booleans())
    mask = (A.BLOCKED_STATE if blocked else 0) | (A.FLAT_PAD8 if pad8 else 0)
    fa = 8 if pad8 else 1
    total = int((-(-numels // fa) * fa).sum())
    shard = (0, -1)
    if total and draw(st.booleans()):
        b = draw(st.integers(0, total))
        shard = (b, -1 if draw(st.booleans()) else draw(st.integers(b, total)))   # -1: to the list's end
    ptrs = []
    for s in range(5):
        if not esz[s]:
            ptrs.append(None)
            continue
        base = (1 << 40) + s * (1 << 34) + MiB2 * draw(st.integers(0, 7))
        if not (blocked and s >= 2) and shard != (0, -1) and draw(st.booleans()):
            mask |= 1 << s                                   # one flat shard buffer, any element phase
            ptrs.append([base + esz[s] * draw(st.integers(0, 7))])
            continue
        shift, align = draw(st.integers(0, 7)), draw(st.sampled_from([1, 8, 128]))
        ptrs.append(arena_ptrs(base + shift * esz[s], numels, align, esz[s]))
    if blocked:
        ptrs[2], ptrs[3], ptrs[4] = [(1 << 40) + 5 * (1 << 34) + 256 * draw(st.integers(0, 63))], None, None
    return Spec(numels, esz, ptrs, shard, mask), kind, dt, prec


@settings(max_examples=150, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(_plans())
def test_random_plans_hypothesis(case):
    spec, kind, dt, prec = case
    check_plan(spec, CODE.get(kind, A.MIXED), DT[dt], for_check=kind == "check", prec=prec)
