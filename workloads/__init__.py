"""Seeded synthetic workloads for the AdamW step: shapes and input generators.

This module holds no optimizer arithmetic.  It only says which tensors a
workload has and fills them with seeded random numbers; the same bytes then go
to the GPU library and to the CPU oracle.  Nothing here imports either of them.

The tensor lists follow the model shapes of the pages' runs (the pages train on
datasets and checkpoints that are not used here; the step's cost and result do
not depend on where the numbers come from, so seeded normal draws stand in):

* ``single_1m``   -- one flat tensor of 1,048,576 elements.
* ``bert_52m``    -- the Megatron-BERT list of "Distributed optimizer support
  for BERT" (A40/A100 tables, 4-way data parallel): word embedding 30592x768,
  position embedding 512x768, 4 layers of QKV 768x2304, proj 768x768,
  fc1 768x3072, fc2 3072x768 (each with a bias) and 2 LayerNorms (gamma, beta),
  52,239,360 elements in 50 tensors.
* ``opt_125m``    -- OPT-125m ("[pure bf16 training] w/ AnyPrecisionAdamW and
  Kahan summation", the opt-125m runs): 196 tensors, 125,239,296 elements.
* ``opt_1_3b``    -- OPT-1.3B (same page, the opt-1.3b run and its memory
  table): 386 tensors, 1,315,753,984 elements (the final LayerNorm is not in
  the list, as the workload is written).
* ``ragged_10k``  -- 10,000 tensors with log-uniform sizes in [1, 2^22].
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np


@dataclass
class Workload:
    name: str
    shapes: list            # list of (name, numel)
    mode: str               # "mixed" or "kahan" (the default mode of the run)
    p_dtype: str            # "bf16" or "f16"
    steps: int
    loss_scale: float = 1.0
    warmup_lr: bool = False
    dp_size: int = 1        # ZeRO data-parallel degree; rank r owns 1/dp of the flat list
    notes: str = ""

    @property
    def numels(self):
        return [n for _, n in self.shapes]

    @property
    def total(self) -> int:
        return int(sum(self.numels))

    def shard(self, rank: int):
        """[begin, end) of ``rank``'s equal share of the flat concatenation."""
        n = self.total
        return rank * n // self.dp_size, (rank + 1) * n // self.dp_size


def _linear(name, fan_in, fan_out):
    return [(f"{name}.weight", fan_in * fan_out), (f"{name}.bias", fan_out)]


def _ln(name, d):
    return [(f"{name}.gamma", d), (f"{name}.beta", d)]


def bert_shapes():
    d, ff = 768, 3072
    s = [("word_emb", 30592 * d), ("pos_emb", 512 * d)]
    for i in range(4):
        s += _linear(f"l{i}.qkv", d, 3 * d) + _linear(f"l{i}.proj", d, d)
        s += _linear(f"l{i}.fc1", d, ff) + _linear(f"l{i}.fc2", ff, d)
        s += _ln(f"l{i}.ln1", d) + _ln(f"l{i}.ln2", d)
    return s


def opt_shapes(d, ff, layers, vocab=50272, pos=2050, final_ln=True):
    s = [("embed_tokens", vocab * d), ("embed_positions", pos * d)]
    for i in range(layers):
        for proj in ("q", "k", "v", "out"):
            s += _linear(f"l{i}.{proj}_proj", d, d)
        s += _linear(f"l{i}.fc1", d, ff) + _linear(f"l{i}.fc2", ff, d)
        s += _ln(f"l{i}.self_attn_ln", d) + _ln(f"l{i}.final_ln", d)
    if final_ln:
        s += _ln("final_layer_norm", d)
    return s


def ragged_sizes(count=10_000, max_numel=1 << 22, seed=0):
    """Log-uniform sizes: floor(exp(U(0, ln(max+1)))) clipped to [1, max]."""
    rng = np.random.default_rng(np.random.SeedSequence([5, seed]))
    x = np.floor(np.exp(rng.uniform(0.0, math.log(max_numel + 1), size=count)))
    return np.clip(x, 1, max_numel).astype(np.int64)


def get(name: str) -> Workload:
    if name == "single_1m":
        return Workload(name, [("flat", 1 << 20)], "mixed", "bf16", 10)
    if name == "bert_52m":
        return Workload(name, bert_shapes(), "mixed", "bf16", 20, dp_size=4)
    if name == "opt_125m":
        return Workload(name, opt_shapes(768, 3072, 12), "kahan", "bf16", 100, warmup_lr=True)
    if name == "opt_1_3b":
        return Workload(name, opt_shapes(2048, 8192, 24, final_ln=False), "mixed", "bf16", 10)
    if name == "ragged_10k":
        sizes = ragged_sizes()
        return Workload(name, [(f"t{i}", int(n)) for i, n in enumerate(sizes)], "mixed", "f16", 3,
                        loss_scale=65536.0)
    raise KeyError(name)


NAMES = ("single_1m", "bert_52m", "opt_125m", "opt_1_3b", "ragged_10k")

# Spread of the synthetic draws (the workload recipe): master weights N(0, 0.02),
# gradients N(0, 1e-3) before loss scaling.
INIT_STD = 0.02
GRAD_STD = 1e-3


def seed_of(*parts) -> int:
    """A 63-bit seed derived from a tuple of ints/strings (stable across runs)."""
    ss = np.random.SeedSequence([abs(hash_str(p)) if isinstance(p, str) else int(p) for p in parts])
    return int(ss.generate_state(2, np.uint64)[0] >> np.uint64(1))


def hash_str(s: str) -> int:
    h = 1469598103934665603
    for ch in s.encode():
        h = ((h ^ ch) * 1099511628211) & ((1 << 64) - 1)
    return h >> 1


def aligned_offsets(numels, align_elems: int):
    """Start offsets of tensors packed one after another in one arena, each
    start rounded up to a multiple of ``align_elems`` (1 = packed tight)."""
    offs, pos = [], 0
    for n in numels:
        pos = -(-pos // align_elems) * align_elems
        offs.append(pos)
        pos += int(n)
    return offs, pos


# ---------------------------------------------------------------------------
# torch-based generators (device or CPU); imported lazily so that the shapes
# above stay usable without torch.
# ---------------------------------------------------------------------------

def _gen(device, *parts):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed_of(*parts))
    return g


def normal(n, std, device, *seed_parts, dtype=None):
    """``n`` draws of N(0, std^2) as float32, rounded to ``dtype`` if given."""
    import torch
    x = torch.empty(int(n), dtype=torch.float32, device=device)
    if n:
        x.normal_(0.0, std, generator=_gen(device, *seed_parts))
    return x if dtype is None else x.to(dtype)


def randint16(n, device, *seed_parts):
    """``n`` uniformly random 16-bit patterns (as an int16 tensor)."""
    import torch
    x = torch.empty(int(n), dtype=torch.int16, device=device)
    if n:
        x.random_(-32768, 32768, generator=_gen(device, *seed_parts))
    return x


def grads(n, device, *seed_parts, dtype, scale=1.0):
    """Gradients N(0, GRAD_STD^2), multiplied by ``scale`` (the loss scale),
    then rounded to the 16-bit ``dtype``."""
    import torch
    x = normal(n, GRAD_STD, device, "grad", *seed_parts)
    if scale != 1.0:
        x = x * torch.tensor(scale, dtype=torch.float32, device=device)
    return x.to(dtype)


@dataclass
class Arena:
    """One flat buffer per stream with every tensor of the list carved out of it.

    ``offsets[i]`` is tensor ``i``'s first element in every stream buffer.
    """
    numels: list
    offsets: list
    bufs: dict = field(default_factory=dict)

    def view(self, key, i):
        o = self.offsets[i]
        return self.bufs[key][o:o + self.numels[i]]


def make_state(mode, numels, device, seed, *, p_dtype="bf16", align_elems=128, loss_scale=1.0,
               random_moments=False):
    """Allocate and fill the optimizer state of a tensor list in one arena per stream.

    mixed: p (bf16|f16) = round(master), g (same 16-bit dtype), master/m/v fp32.
    split: p = bf16 round(N(0, 0.02)), r = uniform random int16, m/v fp32.
    kahan: p, g, m, v, c all bf16; p = round(N(0, 0.02)).
    m = v = c = 0 unless ``random_moments`` (then m ~ N(0, 1e-3), v ~ N(0, 1e-3)^2,
    and for Kahan c ~ N(0, 1e-6)), to start the update from a generic state.
    """
    import torch
    half = torch.bfloat16 if p_dtype == "bf16" else torch.float16
    offs, total = aligned_offsets(numels, align_elems)
    a = Arena(list(map(int, numels)), offs)
    master = normal(total, INIT_STD, device, "master", seed)
    a.bufs["g"] = grads(total, device, seed, 0, dtype=half, scale=loss_scale)
    if mode == "mixed":
        a.bufs["master"] = master
        a.bufs["p"] = master.to(half)
        if random_moments:
            a.bufs["m"] = normal(total, GRAD_STD, device, "m", seed)
            a.bufs["v"] = normal(total, GRAD_STD, device, "v", seed).square()
        else:
            a.bufs["m"] = torch.zeros(total, dtype=torch.float32, device=device)
            a.bufs["v"] = torch.zeros(total, dtype=torch.float32, device=device)
    elif mode == "split":
        # the master as two 16-bit halves: a bf16 high half and a uniformly random
        # int16 low half (every pair encodes some fp32 master near the bf16 value)
        a.bufs["p"] = master.to(torch.bfloat16)
        del master
        a.bufs["r"] = randint16(total, device, "remainder", seed)
        if random_moments:
            a.bufs["m"] = normal(total, GRAD_STD, device, "m", seed)
            a.bufs["v"] = normal(total, GRAD_STD, device, "v", seed).square()
        else:
            a.bufs["m"] = torch.zeros(total, dtype=torch.float32, device=device)
            a.bufs["v"] = torch.zeros(total, dtype=torch.float32, device=device)
    elif mode.startswith("pure"):
        m32, v32, kahan = parse_pure(mode)
        a.bufs["p"] = master.to(torch.bfloat16)
        del master
        for k, f32 in (("m", m32), ("v", v32)):
            x = normal(total, GRAD_STD, device, k, seed) if random_moments else \
                torch.zeros(total, dtype=torch.float32, device=device)
            if random_moments and k == "v":
                x = x.square()
            a.bufs[k] = x if f32 else x.to(torch.bfloat16)
        if kahan:
            cdt = torch.float32 if kahan == 2 else torch.bfloat16
            a.bufs["c"] = (normal(total, 1e-6, device, "c", seed, dtype=cdt) if random_moments else
                           torch.zeros(total, dtype=cdt, device=device))
    elif mode == "kahan":
        a.bufs["p"] = master.to(torch.bfloat16)
        del master
        if random_moments:
            a.bufs["m"] = normal(total, GRAD_STD, device, "m", seed, dtype=torch.bfloat16)
            a.bufs["v"] = normal(total, GRAD_STD, device, "v", seed).square().to(torch.bfloat16)
            a.bufs["c"] = normal(total, 1e-6, device, "c", seed, dtype=torch.bfloat16)
        else:
            for k in ("m", "v", "c"):
                a.bufs[k] = torch.zeros(total, dtype=torch.bfloat16, device=device)
    else:
        raise ValueError(mode)
    return a


def refill_grads(arena: Arena, seed, step, *, p_dtype="bf16", loss_scale=1.0):
    """Overwrite the gradient arena with the seeded draw of ``step``."""
    import torch
    half = torch.bfloat16 if p_dtype == "bf16" else torch.float16
    g = arena.bufs["g"]
    g.copy_(grads(g.numel(), g.device, seed, step, dtype=half, scale=loss_scale))


# Buffers of each mode in the order of the C ABI's streams:
# param, grad, exp_avg, exp_avg_sq, aux (fp32 master in mixed mode, bf16 Kahan compensation otherwise).
STREAMS = {"mixed": ("p", "g", "m", "v", "master"), "kahan": ("p", "g", "m", "v", "c"),
           "split": ("p", "g", "m", "v", "r")}


def parse_pure(mode: str):
    """'pure-<m>-<v>-<k|k32|n>' with m, v in {f32, bf16}: (fp32 exp_avg, fp32
    exp_avg_sq, compensation), the compensation 0 (n: none), 1 (k: a bf16
    buffer) or 2 (k32: an fp32 buffer)."""
    _, m, v, k = mode.split("-")
    assert m in ("f32", "bf16") and v in ("f32", "bf16") and k in ("k", "k32", "n"), mode
    return m == "f32", v == "f32", {"n": 0, "k": 1, "k32": 2}[k]


def streams_of(mode: str):
    """Buffer keys of a mode in the C ABI's stream order (param, grad, exp_avg, exp_avg_sq[, aux])."""
    if mode.startswith("pure"):
        return ("p", "g", "m", "v", "c") if parse_pure(mode)[2] else ("p", "g", "m", "v")
    return STREAMS[mode]


def pure_traffic(mode: str) -> int:
    """Bytes moved per parameter by a pure-bf16 step of this precision."""
    m32, v32, kahan = parse_pure(mode)
    state = (4 if m32 else 2) + (4 if v32 else 2) + (0, 2, 4)[kahan]
    return (2 + 2 + state) + (2 + state)

# Resident bytes per parameter of each stream layout (what one rank holds).
RESIDENT_BYTES = {
    "mixed": {"p": 2, "g": 2, "master": 4, "m": 4, "v": 4},
    "kahan": {"p": 2, "g": 2, "m": 2, "v": 2, "c": 2},
    "bf16_naive": {"p": 2, "g": 2, "m": 2, "v": 2},
    "split": {"p": 2, "g": 2, "m": 4, "v": 4, "r": 2},
}

# Bytes moved per parameter by one step: what is read plus what is written.
# mixed: read g, master, m, v; write master, m, v, p (p is derived, never read).
# kahan: read g, p, m, v, c; write p, m, v, c.
TRAFFIC_BYTES = {
    "mixed": {"read": {"g": 2, "master": 4, "m": 4, "v": 4}, "write": {"master": 4, "m": 4, "v": 4, "p": 2}},
    "kahan": {"read": {"g": 2, "p": 2, "m": 2, "v": 2, "c": 2}, "write": {"p": 2, "m": 2, "v": 2, "c": 2}},
    "check_f16": {"read": {"g": 2}, "write": {}},
    "split": {"read": {"g": 2, "p": 2, "r": 2, "m": 4, "v": 4}, "write": {"p": 2, "r": 2, "m": 4, "v": 4}},
}


def traffic_per_param(kind: str) -> int:
    t = TRAFFIC_BYTES[kind]
    return sum(t["read"].values()) + sum(t["write"].values())
