"""Helpers of the GPU parity tests: run the HIP library and the CPU oracle on the
same seeded bytes and compare to the stated bar.

Bar (per element, after the last step):
* fp32 state (master, exp_avg, exp_avg_sq of mixed mode): relative error
  |gpu - oracle| / |oracle| <= 2e-6, and exact equality where the oracle is 0;
* 16-bit outputs (param, bf16 moments, Kahan compensation): at most 1 ulp apart,
  measured as the distance of the sign-magnitude codes on the ordered line;
* NaN on one side only is a failure; step counters and skip flags exactly equal.
The kernels are designed to be bit-exact with the oracle (same operation order,
no contraction, correctly rounded sqrt/div, RNE narrowing), so every comparison
also asserts that no bit pattern differs (a NaN's sign and payload aside): the
tolerance above is the reported bar, bit equality the enforced one.
"""
from __future__ import annotations

import numpy as np
import torch

import adamw_optimizer_step_apply_amd as A
import oracle
import workloads

MODE = {"mixed": A.MIXED, "kahan": A.PURE_KAHAN, "split": A.MIXED_SPLIT}
DT = {"bf16": A.BF16, "f16": A.F16}
F32_KEYS = {"mixed": ("m", "v", "master"), "kahan": (), "split": ("m", "v")}


def f32_keys(mode):
    if mode.startswith("pure"):
        m32, v32, kahan = workloads.parse_pure(mode)
        return tuple(k for k, f in (("m", m32), ("v", v32), ("c", kahan == 2)) if f)
    return F32_KEYS[mode]


def pure_precision(mode):
    m32, v32, kahan = workloads.parse_pure(mode)
    return A.PurePrecision(A.F32 if m32 else A.BF16, A.F32 if v32 else A.BF16, kahan)


def join_master(p: np.ndarray, r: np.ndarray) -> np.ndarray:
    """fp32 masters encoded by split (bf16 high half p, int16 remainder r)."""
    w = (p.astype(np.int64) << 16) + r.view(np.int16).astype(np.int64)
    return (w & 0xFFFFFFFF).astype(np.uint32).view(np.float32)


def compare_streams(label, mode, got: dict, ref: dict, keys, p_is_f16=False):
    """compare() over a mode's streams; a split master is compared as the joined
    fp32 master (the fp32 bar) plus its bf16 half (the 16-bit bar)."""
    stats = []
    for k in keys:
        if mode == "split" and k == "r":
            stats.append(compare(f"{label}:master(p,r)", join_master(got["p"], got["r"]),
                                 join_master(ref["p"], ref["r"]), True))
            continue
        stats.append(compare(f"{label}:{k}", got[k], ref[k], k in f32_keys(mode), p_is_f16))
    return stats
REL_TOL = 2e-6
ULP_TOL = 1


def to_np(t: torch.Tensor) -> np.ndarray:
    t = t.detach()
    if t.dtype in (torch.bfloat16, torch.float16, torch.int16):
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.contiguous().cpu().numpy()


def ordered16(a: np.ndarray) -> np.ndarray:
    a = a.astype(np.int32)
    return np.where(a & 0x8000, -(a & 0x7FFF), a)


def compare(name: str, got: np.ndarray, ref: np.ndarray, is_f32: bool, p_is_f16: bool = False) -> dict:
    """Checks one stream against the bar; returns statistics (raises on failure)."""
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    word = np.uint32 if is_f32 else np.uint16
    if np.array_equal(got.view(word), ref.view(word)):
        # identical bits: no error of any size, the same NaNs and infinities
        return {"stream": name, "n": int(got.size), "bit_mismatches": 0,
                ("max_rel" if is_f32 else "max_ulp"): 0.0 if is_f32 else 0}
    if is_f32:
        gb, rb = got.view(np.uint32), ref.view(np.uint32)
        gn, rn = np.isnan(got), np.isnan(ref)
    else:
        gb, rb = got, ref
        expo = 0x7C00 if p_is_f16 else 0x7F80
        gn = ((got & expo) == expo) & ((got & (0x3FF if p_is_f16 else 0x7F)) != 0)
        rn = ((ref & expo) == expo) & ((ref & (0x3FF if p_is_f16 else 0x7F)) != 0)
    assert np.array_equal(gn, rn), f"{name}: NaN pattern differs at {np.flatnonzero(gn != rn)[:8]}"
    ok = ~rn
    diff_bits = int(np.count_nonzero(gb[ok] != rb[ok]))
    stats = {"stream": name, "n": int(got.size), "bit_mismatches": diff_bits}
    if is_f32:
        # an infinity on either side must be the same infinity; the relative bar
        # covers the pairs that are both finite
        inf = np.isinf(got[ok]) | np.isinf(ref[ok])
        assert np.array_equal(gb[ok][inf], rb[ok][inf]), f"{name}: infinities differ"
        g64, r64 = got[ok][~inf].astype(np.float64), ref[ok][~inf].astype(np.float64)
        zero = r64 == 0
        assert np.all(g64[zero] == 0), f"{name}: nonzero where the oracle is 0"
        nz = ~zero
        rel = np.abs(g64[nz] - r64[nz]) / np.abs(r64[nz])
        stats["max_rel"] = float(rel.max()) if rel.size else 0.0
        assert stats["max_rel"] <= REL_TOL, f"{name}: max relative error {stats['max_rel']:.3e} > {REL_TOL}"
    else:
        mag = (0x7C00 if p_is_f16 else 0x7F80)
        inf = ((got[ok] & 0x7FFF) == mag) | ((ref[ok] & 0x7FFF) == mag)
        assert np.array_equal(got[ok][inf], ref[ok][inf]), f"{name}: infinities differ"
        d = np.abs(ordered16(got[ok]) - ordered16(ref[ok]))
        stats["max_ulp"] = int(d.max()) if d.size else 0
        assert stats["max_ulp"] <= ULP_TOL, f"{name}: {stats['max_ulp']} ulp apart"
    if diff_bits:
        first = np.flatnonzero(ok & (gb != rb))[:4]
        raise AssertionError(f"{name}: {diff_bits} of {got.size} elements differ from the oracle in their bits "
                             f"(within the tolerance: {stats}); first at {first.tolist()}: "
                             f"gpu {gb[first].tolist()} oracle {rb[first].tolist()}")
    return stats


def merge_stats(name: str, parts) -> dict:
    """One stream's statistics from those of its pieces."""
    parts = list(parts)
    out = {"stream": name, "n": sum(p["n"] for p in parts), "bit_mismatches": sum(p["bit_mismatches"] for p in parts)}
    for key in ("max_rel", "max_ulp"):
        vals = [p[key] for p in parts if key in p]
        if vals:
            out[key] = max(vals)
    return out


def shift_stream(arena: workloads.Arena, key: str, shift: int):
    """Moves stream ``key`` of the arena ``shift`` elements up in a fresh buffer,
    so its tensors start at a different 16-byte phase than the other streams."""
    if not shift:
        return
    old = arena.bufs[key]
    buf = torch.empty(old.numel() + shift, dtype=old.dtype, device=old.device)
    buf[:shift].zero_()
    buf[shift:].copy_(old)
    arena.bufs[key] = buf[shift:]
    arena.bufs["_" + key + "_owner"] = buf


class Case:
    """A tensor list on the GPU (one arena per stream) and its host mirror."""

    def __init__(self, mode, numels, seed, *, p_dtype="bf16", align_elems=128, loss_scale=1.0,
                 random_moments=False, shifts=None, device="cuda"):
        self.mode, self.p_dtype, self.seed, self.loss_scale = mode, p_dtype, seed, loss_scale
        self.numels = [int(n) for n in numels]
        self.arena = workloads.make_state(mode, self.numels, device, seed, p_dtype=p_dtype,
                                          align_elems=align_elems, loss_scale=loss_scale,
                                          random_moments=random_moments)
        for k, s in (shifts or {}).items():
            shift_stream(self.arena, k, s)
        self.keys = workloads.streams_of(mode)
        self.host = {k: to_np(self.arena.bufs[k]) for k in self.keys}
        self.d_step = torch.zeros(1, dtype=torch.int32, device=device)
        self.step = 0

    # -- lists ------------------------------------------------------------
    def tensor_list(self, shard_begin=0, shard_end=-1):
        streams = [[self.arena.view(k, i) for i in range(len(self.numels))] for k in self.keys]
        return A.TensorList(self.numels, streams, shard_begin, shard_end)

    def oracle_tensors(self):
        return [{k: self.host[k][o:o + n] for k in self.keys}
                for o, n in zip(self.arena.offsets, self.numels)]

    # -- steps ------------------------------------------------------------
    def refill_grads(self, step_index: int):
        workloads.refill_grads(self.arena, self.seed, step_index, p_dtype=self.p_dtype,
                               loss_scale=self.loss_scale)
        self.host["g"] = to_np(self.arena.bufs["g"])

    def gpu_step(self, hp: A.HParams, shard=(0, -1), found_inf=None, tl=None):
        tl = tl or self.tensor_list(*shard)
        if self.mode.startswith("pure"):
            A.adamw_pure_multi_tensor_step(pure_precision(self.mode), tl, hp, self.d_step, found_inf)
        else:
            A.adamw_multi_tensor_step(MODE[self.mode], DT[self.p_dtype], tl, hp, self.d_step, found_inf)

    def oracle_step(self, hp: oracle.HParams, shard=(0, -1), check_overflow=False, flat_align=1):
        self.step = oracle.step_list(self.mode, self.oracle_tensors(), hp, self.step,
                                     p_is_f16=self.p_dtype == "f16", check_overflow=check_overflow,
                                     shard_begin=shard[0], shard_end=shard[1], flat_align=flat_align)

    def compare_all(self, label=""):
        torch.cuda.synchronize()
        assert int(self.d_step.item()) == self.step, f"{label}: step counter {int(self.d_step.item())} != {self.step}"
        got = {k: to_np(self.arena.bufs[k]) for k in self.keys}
        stats = compare_streams(label, self.mode, got, self.host, self.keys, self.p_dtype == "f16")
        log_stats(stats)
        return stats


def log_stats(stats):
    """Appends comparison statistics to $PARITY_STATS (JSON lines) when set."""
    import json
    import os
    path = os.environ.get("PARITY_STATS")
    if path:
        with open(path, "a") as f:
            for st in stats:
                f.write(json.dumps(st) + "\n")


def hp_pair(lr=2e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, inv_scale=1.0):
    """The same fp32 hyper-parameters for the library and the oracle."""
    f = [float(np.float32(x)) for x in (lr, beta1, beta2, eps, weight_decay, inv_scale)]
    return A.HParams(*f), oracle.HParams(*f)


def same_bits(a: torch.Tensor, b: torch.Tensor) -> bool:
    """Bitwise equality (torch.equal treats NaN as unequal to itself)."""
    view = {1: torch.uint8, 2: torch.int16, 4: torch.int32, 8: torch.int64}[a.element_size()]
    return a.dtype == b.dtype and torch.equal(a.view(view), b.view(view))


def free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


class SampledCase:
    """A full-size workload on the GPU with the oracle following a sample of its
    elements.  The update is elementwise, so the oracle stepping only the sampled
    elements (with the same per-step scalars) is exact for them.

    Samples: the first and last 8 elements of every tensor, plus ``n_random``
    uniform positions of the flat list and the flat positions in ``extra``;
    optionally restricted bookkeeping for a
    ZeRO shard [b, e): samples outside it must come back unchanged."""

    def __init__(self, mode, numels, seed, *, p_dtype="bf16", loss_scale=1.0, n_random=1 << 21,
                 shard=(0, -1), align_elems=128, device="cuda", extra=()):
        self.mode, self.p_dtype, self.seed, self.loss_scale = mode, p_dtype, seed, loss_scale
        self.numels = [int(n) for n in numels]
        self.arena = workloads.make_state(mode, self.numels, device, seed, p_dtype=p_dtype,
                                          align_elems=align_elems, loss_scale=loss_scale)
        self.keys = workloads.streams_of(mode)
        total = sum(self.numels)
        b, e = shard[0], (total if shard[1] < 0 else shard[1])
        self.shard = (b, shard[1])
        starts = np.concatenate([[0], np.cumsum(self.numels)]).astype(np.int64)
        rng = np.random.default_rng(np.random.SeedSequence([seed, 77]))
        flat = [rng.integers(0, total, size=n_random, dtype=np.int64),
                np.asarray([x for x in extra if 0 <= x < total], dtype=np.int64)]
        for i, n in enumerate(self.numels):
            k = min(8, n)
            flat.append(starts[i] + np.arange(k))
            flat.append(starts[i] + n - k + np.arange(k))
        flat = np.unique(np.concatenate(flat))
        tens = np.searchsorted(starts, flat, side="right") - 1
        arena_idx = np.asarray(self.arena.offsets, np.int64)[tens] + (flat - starts[tens])
        self.flat = flat
        self.inside = (flat >= b) & (flat < e)
        self.idx = torch.from_numpy(arena_idx).to(device)
        self.host = {k: to_np(self.arena.bufs[k][self.idx]) for k in self.keys}
        self.initial = {k: v.copy() for k, v in self.host.items()}
        self.d_step = torch.zeros(1, dtype=torch.int32, device=device)
        self.step = 0

    def tensor_list(self):
        streams = [[self.arena.view(k, i) for i in range(len(self.numels))] for k in self.keys]
        return A.TensorList(self.numels, streams, *self.shard)

    def refill_grads(self, step_index):
        workloads.refill_grads(self.arena, self.seed, step_index, p_dtype=self.p_dtype, loss_scale=self.loss_scale)
        self.host["g"] = to_np(self.arena.bufs["g"][self.idx])

    def oracle_step(self, ho: oracle.HParams, skip=False):
        if skip:
            return
        t = self.step + 1
        sel = np.flatnonzero(self.inside)
        sub = {k: np.ascontiguousarray(self.host[k][sel]) for k in self.keys}
        if self.mode == "mixed":
            oracle.adamw_mixed(sub["p"], sub["g"], sub["master"], sub["m"], sub["v"], ho, t,
                               p_is_f16=self.p_dtype == "f16")
        elif self.mode == "split":
            oracle.adamw_mixed_split(sub["p"], sub["g"], sub["r"], sub["m"], sub["v"], ho, t)
        elif self.mode.startswith("pure"):
            oracle.adamw_pure(sub["p"], sub["g"], sub["m"], sub["v"], sub.get("c"), ho, t)
        else:
            oracle.adamw_kahan(sub["p"], sub["g"], sub["m"], sub["v"], sub["c"], ho, t)
        for k in self.keys:
            self.host[k][sel] = sub[k]
        self.step = t

    def compare_all(self, label=""):
        torch.cuda.synchronize()
        assert int(self.d_step.item()) == self.step, f"{label}: step counter {int(self.d_step.item())} != {self.step}"
        got = {k: to_np(self.arena.bufs[k][self.idx]) for k in self.keys}
        stats = compare_streams(label, self.mode, got, self.host, self.keys, self.p_dtype == "f16")
        out = ~self.inside
        for k in self.keys:
            if k != "g" and out.any():
                assert np.array_equal(got[k][out], self.initial[k][out]), f"{label}:{k} changed outside the shard"
        log_stats(stats)
        return stats


STATE_KEYS = ("m", "v")


def blocked_state_keys(case) -> tuple:
    """The state streams (exp_avg, exp_avg_sq[, aux]) of a case, in block order."""
    return tuple(case.keys[2:])


def state_block_of(dtypes) -> int:
    """Elements per block of a blocked state buffer (the same for every set of state dtypes)."""
    return A.STATE_BLOCK_ELEMS


def build_blocked(case, b, e) -> torch.Tensor:
    """The blocked state buffer of the shard [b, e) of a tightly packed case
    (arena index == flat index): per block of B elements (32 KiB of the widest
    state stream), each state stream's values one after another, as raw bytes."""
    B = state_block_of([case.arena.bufs[k].dtype for k in blocked_state_keys(case)])
    L = e - b
    nb = -(-L // B)
    cols = []
    for k in blocked_state_keys(case):
        x = case.arena.bufs[k][b:e]
        pad = torch.zeros(nb * B - L, dtype=x.dtype, device=x.device)
        cols.append(torch.cat([x, pad]).view(nb, B).view(torch.uint8))
    return torch.cat(cols, dim=1).contiguous()


def padded_starts(numels) -> np.ndarray:
    """Each tensor's start in the padded flat index (multiples of 8), plus the total."""
    return np.concatenate([[0], np.cumsum([-(-int(n) // 8) * 8 for n in numels])]).astype(np.int64)


def build_blocked_padded(arena, keys, numels) -> torch.Tensor:
    """The blocked state buffer of a whole list in the padded flat index, from
    an arena whose tensors already sit at their padded positions (aligned to 8
    elements, or to any multiple of 8 when every length is one)."""
    B = state_block_of([arena.bufs[k].dtype for k in keys])
    starts = padded_starts(numels)
    assert list(arena.offsets) == [int(x) for x in starts[:-1]], "arena is not in the padded flat index"
    nb = -(-int(starts[-1]) // B)
    cols = []
    for k in keys:
        src = arena.bufs[k]
        flat = torch.cat([src, torch.zeros(nb * B - src.numel(), dtype=src.dtype, device=src.device)])
        cols.append(flat.view(nb, B).view(torch.uint8))
        del flat
    out = torch.cat(cols, dim=1).contiguous()
    del cols
    return out


def blocked_gather(blocked: torch.Tensor, dtypes: dict, pos: torch.Tensor) -> dict:
    """Values at flat positions `pos` (device int64) of each state stream of a
    whole-list blocked buffer; `dtypes` maps the streams, in block order, to
    their torch dtypes."""
    B = state_block_of(list(dtypes.values()))
    blk, off = pos // B, pos % B
    out, col = {}, 0
    for k, dt in dtypes.items():
        width = B * torch.empty(0, dtype=dt).element_size()
        out[k] = blocked[:, col:col + width].contiguous().view(dt)[blk, off]
        col += width
    return out


def unpack_blocked(case, blocked: torch.Tensor, b, e) -> dict:
    """Per-stream host arrays (flat order, length e - b) from a blocked buffer."""
    B = state_block_of([case.arena.bufs[k].dtype for k in blocked_state_keys(case)])
    L = e - b
    out, col = {}, 0
    for k in blocked_state_keys(case):
        dt = case.arena.bufs[k].dtype
        nbytes = B * torch.empty(0, dtype=dt).element_size()
        part = blocked[:, col:col + nbytes].contiguous().view(dt).reshape(-1)[:L]
        out[k] = to_np(part)
        col += nbytes
    return out


PIECE = 1 << 26          # elements per comparison piece (a multiple of the state block)
RANGE = 1 << 24          # elements per oracle work item


def host_threads() -> int:
    """Host threads for the oracle: the affinity set, at most 16 (the CPU share one GPU gets)."""
    import os
    return max(1, min(16, len(os.sched_getaffinity(0))))


def oracle_ranges(mode, host: dict, ranges, ho: oracle.HParams, t: int, p_is_f16=False):
    """Steps the arena ranges [a, b) of `host` in place on all host threads: the
    update is elementwise, so any cut of a tensor's elements steps them as the
    whole tensor would, and the oracle's C loops release the GIL."""
    from concurrent.futures import ThreadPoolExecutor
    work = [(a + o, min(b, a + o + RANGE)) for a, b in ranges for o in range(0, b - a, RANGE)]

    def run(ab):
        a, b = ab
        h = {k: v[a:b] for k, v in host.items()}
        if mode == "mixed":
            oracle.adamw_mixed(h["p"], h["g"], h["master"], h["m"], h["v"], ho, t, p_is_f16=p_is_f16)
        elif mode == "split":
            oracle.adamw_mixed_split(h["p"], h["g"], h["r"], h["m"], h["v"], ho, t)
        elif mode == "kahan":
            oracle.adamw_kahan(h["p"], h["g"], h["m"], h["v"], h["c"], ho, t)
        else:
            oracle.adamw_pure(h["p"], h["g"], h["m"], h["v"], h.get("c"), ho, t)

    with ThreadPoolExecutor(host_threads()) as pool:
        list(pool.map(run, work))


class FullCase(Case):
    """A full-size workload compared on every element: the oracle steps the
    owned pieces of the arenas on all host threads, and the comparison runs
    over the whole arenas in pieces (untouched elements and gaps included)."""

    def oracle_step(self, hp: oracle.HParams, shard=(0, -1), skip=False, flat_align=1):
        if skip:
            return
        t = self.step + 1
        end = None if shard[1] < 0 else shard[1]
        ranges = [(self.arena.offsets[i] + lo, self.arena.offsets[i] + hi)
                  for i, lo, hi, _ in oracle.shard_pieces(self.numels, shard[0], end, flat_align)]
        oracle_ranges(self.mode, self.host, ranges, hp, t, self.p_dtype == "f16")
        self.step = t

    def compare_all(self, label="", skip_keys=()):
        torch.cuda.synchronize()
        assert int(self.d_step.item()) == self.step, f"{label}: step counter {int(self.d_step.item())} != {self.step}"
        stats = []
        f16 = self.p_dtype == "f16"
        for k in self.keys:
            if k == "g" or k in skip_keys:
                continue
            n = self.arena.bufs[k].numel()
            parts = [compare(f"{label}:{k}", to_np(self.arena.bufs[k][a:a + PIECE]), self.host[k][a:a + PIECE],
                             k in f32_keys(self.mode), f16) for a in range(0, n, PIECE)]
            stats.append(merge_stats(f"{label}:{k}", parts))
        log_stats(stats)
        return stats

    def compare_blocked(self, blocked: torch.Tensor, label=""):
        """The state streams read out of a blocked buffer of the whole list whose
        padded flat index is this case's arena index (arenas at multiples of 8),
        against the host arenas, every element (gaps carried over at packing)."""
        torch.cuda.synchronize()
        B = A.STATE_BLOCK_ELEMS
        rows = PIECE // B
        col, stats = 0, []
        for k in self.keys[2:]:
            dt = self.arena.bufs[k].dtype
            width = B * torch.empty(0, dtype=dt).element_size()
            n = self.host[k].size
            parts = []
            for r0 in range(0, blocked.shape[0], rows):
                a = r0 * B
                if a >= n:
                    break
                piece = blocked[r0:r0 + rows, col:col + width].contiguous().view(dt).reshape(-1)
                m = min(piece.numel(), n - a)
                parts.append(compare(f"{label}:{k}", to_np(piece[:m]), self.host[k][a:a + m], k in f32_keys(self.mode),
                                     self.p_dtype == "f16"))
            stats.append(merge_stats(f"{label}:{k}", parts))
            col += width
        log_stats(stats)
        return stats
