"""CPU oracle for the fused AdamW optimizer step.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import this package.  It shares no
code with the GPU library (``adamw_optimizer_step_apply_amd``) and never imports
it; the two meet only on the bytes of their inputs and outputs.

The arithmetic lives in ``adamw_oracle.c`` (plain scalar C, built by gcc with
``-ffp-contract=off``); this module is a ctypes wrapper over numpy arrays plus
the step bookkeeping that the definition needs around the element loop:

* the step counter ``t`` (1-based, advanced only when the step is taken) and the
  Adam bias correction it feeds (Kingma & Ba, Algorithm 1);
* the skip rule of fp16 loss scaling: any inf/NaN gradient anywhere leaves every
  buffer and the counter unchanged (the fp16-amp run on the page
  "[pure bf16 training] w/ AnyPrecisionAdamW and Kahan summation");
* a ZeRO shard: one data-parallel rank updates only the elements of the list's
  flat concatenation in ``[shard_begin, shard_end)`` ("Distributed optimizer
  support for BERT", the A40 table and the expected-saving remark below it).
  The update is elementwise, so the shard step is the full-list step restricted
  to those elements.

Arrays: 16-bit floats (bf16 / fp16) are carried as ``numpy.uint16`` bit patterns,
fp32 state as ``numpy.float32``.  All updates are in place.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "adamw_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

# Flags that keep the C compiler on plain IEEE binary32 arithmetic: no
# contraction into FMA, no fast-math reassociation, no auto-vectorised
# reductions that could reorder anything.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math", "-ffp-contract=off",
          "-fno-tree-vectorize", "-fno-math-errno"]


def build(src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile ``src`` with gcc into the shared library ``out`` and return its path."""
    tmp = out + ".tmp"
    subprocess.run(["gcc", *CFLAGS, "-o", tmp, src, "-lm"], check=True)
    os.replace(tmp, out)
    return out


_U16P = np.ctypeslib.ndpointer(np.uint16, flags="C_CONTIGUOUS")
_F32P = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
_U32P = np.ctypeslib.ndpointer(np.uint32, flags="C_CONTIGUOUS")
_I64 = ctypes.c_int64
_F = ctypes.c_float


def _bind(lib: ctypes.CDLL) -> ctypes.CDLL:
    sig = {
        "oracle_bf16_to_f32_n": (None, [_U16P, _F32P, _I64]),
        "oracle_f16_to_f32_n": (None, [_U16P, _F32P, _I64]),
        "oracle_f32_to_bf16_n": (None, [_F32P, _U16P, _I64]),
        "oracle_f32_to_f16_n": (None, [_F32P, _U16P, _I64]),
        "oracle_scalars": (None, [_I64, _F, _F, _F, _F, _F32P]),
        "oracle_any_nonfinite_f16": (ctypes.c_int, [_U16P, _I64]),
        "oracle_any_nonfinite_bf16": (ctypes.c_int, [_U16P, _I64]),
        "oracle_adamw_mixed": (None, [_I64, ctypes.c_int, _U16P, _U16P, _F32P, _F32P, _F32P,
                                      _F, _F, _F, _F, _F, _F, _I64]),
        "oracle_adamw_kahan": (None, [_I64, _U16P, _U16P, _U16P, _U16P, _U16P,
                                      _F, _F, _F, _F, _F, _F, _I64]),
        "oracle_adamw_bf16_naive": (None, [_I64, _U16P, _U16P, _U16P, _U16P,
                                           _F, _F, _F, _F, _F, _F, _I64]),
        "oracle_adamw_mixed_split": (None, [_I64, _U16P, _U16P, _U16P, _F32P, _F32P,
                                            _F, _F, _F, _F, _F, _F, _I64]),
        "oracle_split_make_n": (None, [_U32P, _U16P, _U16P, _I64]),
        "oracle_split_join_n": (None, [_U16P, _U16P, _U32P, _I64]),
        "oracle_inv_scale": (_F, [_F]),
        "oracle_adamw_pure": (None, [_I64, _U16P, _U16P, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                     ctypes.c_int, ctypes.c_void_p, ctypes.c_int, _F, _F, _F, _F, _F, _F, _I64]),
        "oracle_update_loss_scale": (None, [ctypes.POINTER(_F), ctypes.POINTER(ctypes.c_int32), ctypes.c_int,
                                            _F, _F, ctypes.c_int32]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_cache: dict[str, ctypes.CDLL] = {}


def load(path: str | None = None) -> ctypes.CDLL:
    """Load (building first if absent) the oracle library at ``path``."""
    path = path or _LIB_PATH
    if path not in _cache:
        if path == _LIB_PATH and (not os.path.exists(path)
                                  or os.path.getmtime(path) < os.path.getmtime(_SRC)):
            build()
        _cache[path] = _bind(ctypes.CDLL(path))
    return _cache[path]


# --------------------------------------------------------------------------
# 16-bit conversions
# --------------------------------------------------------------------------

def _u16(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.uint16)


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32)


def bf16_to_f32(bits, lib=None) -> np.ndarray:
    lib = lib or load()
    bits = _u16(bits)
    out = np.empty(bits.shape, np.float32)
    lib.oracle_bf16_to_f32_n(bits.reshape(-1), out.reshape(-1), bits.size)
    return out


def f16_to_f32(bits, lib=None) -> np.ndarray:
    lib = lib or load()
    bits = _u16(bits)
    out = np.empty(bits.shape, np.float32)
    lib.oracle_f16_to_f32_n(bits.reshape(-1), out.reshape(-1), bits.size)
    return out


def f32_to_bf16(x, lib=None) -> np.ndarray:
    lib = lib or load()
    x = _f32(x)
    out = np.empty(x.shape, np.uint16)
    lib.oracle_f32_to_bf16_n(x.reshape(-1), out.reshape(-1), x.size)
    return out


def f32_to_f16(x, lib=None) -> np.ndarray:
    lib = lib or load()
    x = _f32(x)
    out = np.empty(x.shape, np.uint16)
    lib.oracle_f32_to_f16_n(x.reshape(-1), out.reshape(-1), x.size)
    return out


# --------------------------------------------------------------------------
# Hyper-parameters and per-launch scalars
# --------------------------------------------------------------------------

@dataclass
class HParams:
    """AdamW hyper-parameters, entered as fp32 values.

    Defaults are the opt-1.3b recipe on the AnyPrecisionAdamW page
    (--learning_rate 0.0002 --adam_beta1 0.9 --adam_beta2 0.95
    --weight_decay 0.1); eps is not on the pages and takes Adam's usual 1e-8.
    ``inv_scale`` multiplies every gradient before use (1/loss-scale in fp16
    AMP, 1.0 otherwise).
    """
    lr: float = 2e-4
    beta1: float = 0.9
    beta2: float = 0.95
    eps: float = 1e-8
    weight_decay: float = 0.1
    inv_scale: float = 1.0

    def f32(self):
        return tuple(float(np.float32(x)) for x in
                     (self.lr, self.beta1, self.beta2, self.eps, self.weight_decay, self.inv_scale))


def scalars(t: int, hp: HParams, lib=None) -> dict:
    """The per-launch scalars of step ``t`` (1-based), as fp32 values."""
    lib = lib or load()
    lr, b1, b2, _eps, wd, _s = hp.f32()
    out = np.zeros(6, np.float32)
    lib.oracle_scalars(int(t), lr, b1, b2, wd, out)
    return dict(zip(("step_size", "rbc2", "decay", "lrwd", "omb1", "omb2"), out.tolist()))


# --------------------------------------------------------------------------
# Element updates on one contiguous range (in place)
# --------------------------------------------------------------------------

def adamw_mixed(p16, g16, master, m, v, hp: HParams, t: int, p_is_f16=False, lib=None):
    """Mixed precision step on one range: 16-bit p/g, fp32 master/m/v."""
    lib = lib or load()
    n = master.size
    for a, dt in ((p16, np.uint16), (g16, np.uint16), (master, np.float32),
                  (m, np.float32), (v, np.float32)):
        assert a.dtype == dt and a.flags.c_contiguous and a.size == n
    lr, b1, b2, eps, wd, s = hp.f32()
    lib.oracle_adamw_mixed(n, int(bool(p_is_f16)), p16.reshape(-1), g16.reshape(-1),
                           master.reshape(-1), m.reshape(-1), v.reshape(-1),
                           lr, b1, b2, eps, wd, s, int(t))


def adamw_kahan(p, g, m, v, c, hp: HParams, t: int, lib=None):
    """Pure bf16 step with bf16 Kahan compensation on one range."""
    lib = lib or load()
    n = p.size
    for a in (p, g, m, v, c):
        assert a.dtype == np.uint16 and a.flags.c_contiguous and a.size == n
    lr, b1, b2, eps, wd, s = hp.f32()
    lib.oracle_adamw_kahan(n, p.reshape(-1), g.reshape(-1), m.reshape(-1), v.reshape(-1),
                           c.reshape(-1), lr, b1, b2, eps, wd, s, int(t))


def adamw_bf16_naive(p, g, m, v, hp: HParams, t: int, lib=None):
    """Pure bf16 step without compensation (control for the Kahan pins)."""
    lib = lib or load()
    n = p.size
    lr, b1, b2, eps, wd, s = hp.f32()
    lib.oracle_adamw_bf16_naive(n, p.reshape(-1), g.reshape(-1), m.reshape(-1), v.reshape(-1),
                                lr, b1, b2, eps, wd, s, int(t))


def split_make(w, lib=None):
    """Split fp32 masters (any array viewable as uint32 bits) into (p, r) uint16 halves."""
    lib = lib or load()
    wb = np.ascontiguousarray(np.asarray(w).view(np.uint32)).reshape(-1)
    p = np.empty(wb.size, np.uint16)
    r = np.empty(wb.size, np.uint16)
    lib.oracle_split_make_n(wb, p, r, wb.size)
    return p, r


def split_join(p, r, lib=None) -> np.ndarray:
    """The fp32 masters (as float32) that (p, r) halves encode."""
    lib = lib or load()
    p, r = _u16(p).reshape(-1), _u16(r).reshape(-1)
    w = np.empty(p.size, np.uint32)
    lib.oracle_split_join_n(p, r, w, p.size)
    return w.view(np.float32)


def adamw_mixed_split(p, g, r, m, v, hp: HParams, t: int, lib=None):
    """Mixed step on the split master: bf16 p (read and written), int16 remainder r
    (as uint16 bits), fp32 m/v."""
    lib = lib or load()
    n = m.size
    for a, dt in ((p, np.uint16), (g, np.uint16), (r, np.uint16), (m, np.float32), (v, np.float32)):
        assert a.dtype == dt and a.flags.c_contiguous and a.size == n
    lr, b1, b2, eps, wd, s = hp.f32()
    lib.oracle_adamw_mixed_split(n, p.reshape(-1), g.reshape(-1), r.reshape(-1), m.reshape(-1), v.reshape(-1),
                                 lr, b1, b2, eps, wd, s, int(t))


def adamw_pure(p, g, m, v, c, hp: HParams, t: int, lib=None):
    """Pure bf16 step with chosen state precisions: m and v are float32 (fp32
    state) or uint16 (bf16 bits) arrays; c is the compensation buffer, float32
    (fp32) or uint16 (bf16 bits), or None (no Kahan summation)."""
    lib = lib or load()
    n = p.size
    for a in (p, g):
        assert a.dtype == np.uint16 and a.flags.c_contiguous and a.size == n
    for a in (m, v) + (() if c is None else (c,)):
        assert a.dtype in (np.float32, np.uint16) and a.flags.c_contiguous and a.size == n
    lr, b1, b2, eps, wd, s = hp.f32()
    lib.oracle_adamw_pure(n, p.reshape(-1), g.reshape(-1), m.ctypes.data, int(m.dtype == np.float32),
                          v.ctypes.data, int(v.dtype == np.float32), None if c is None else c.ctypes.data,
                          int(c is not None and c.dtype == np.float32), lr, b1, b2, eps, wd, s, int(t))


def any_nonfinite(g16, is_f16: bool, lib=None) -> bool:
    """True iff any 16-bit gradient is inf or NaN (exponent field all ones)."""
    lib = lib or load()
    g16 = _u16(g16).reshape(-1)
    fn = lib.oracle_any_nonfinite_f16 if is_f16 else lib.oracle_any_nonfinite_bf16
    return bool(fn(g16, g16.size))


# --------------------------------------------------------------------------
# The whole step over a tensor list (with shard restriction and skip rule)
# --------------------------------------------------------------------------

MIXED = "mixed"
KAHAN = "kahan"
SPLIT = "split"


def _place(n: int, flat_align: int) -> int:
    """Room a tensor of n elements takes in the flat concatenation."""
    return -(-n // flat_align) * flat_align


def shard_pieces(numels, shard_begin: int = 0, shard_end: int | None = None, flat_align: int = 1):
    """Intersect the list's flat concatenation with ``[shard_begin, shard_end)``.

    The concatenation places the tensors in list order, each starting at a
    multiple of ``flat_align`` elements (1: back to back; 8: the padded flat
    index, whose gaps hold no element).  Yields ``(tensor_index, lo, hi,
    flat_lo)``: elements ``lo..hi`` of that tensor, which sit at flat position
    ``flat_lo`` of the concatenation.
    """
    total = int(sum(_place(int(n), flat_align) for n in numels))
    if shard_end is None or shard_end < 0:
        shard_end = total
    base = 0
    for i, n in enumerate(numels):
        n = int(n)
        lo = max(shard_begin, base)
        hi = min(shard_end, base + n)
        if lo < hi:
            yield i, lo - base, hi - base, lo
        base += _place(n, flat_align)


def step_list(mode: str, tensors: list, hp: HParams, step: int, *, p_is_f16=False,
              check_overflow=False, shard_begin=0, shard_end=None, flat_align=1, lib=None) -> int:
    """Take one AdamW step over a tensor list; return the new step counter.

    ``tensors`` is a list of dicts of flat numpy arrays: mixed mode uses keys
    ``p, g, master, m, v``; split mode ``p, g, r, m, v``; Kahan mode ``p, g, m, v, c``;
    a "pure..." mode ``p, g, m, v`` (m, v float32 or uint16) and ``c`` when compensated.  With
    ``check_overflow`` the step is skipped (nothing written, counter kept) when
    any gradient of the whole list is inf/NaN.  Only elements inside
    ``[shard_begin, shard_end)`` of the flat concatenation (tensors placed at
    multiples of ``flat_align``, see shard_pieces) are updated.
    """
    lib = lib or load()
    if check_overflow and any(any_nonfinite(tt["g"], p_is_f16, lib) for tt in tensors):
        return step
    t = step + 1
    numels = [tt["g"].size for tt in tensors]
    for i, lo, hi, _ in shard_pieces(numels, shard_begin, shard_end, flat_align):
        tt = tensors[i]
        if mode == MIXED:
            sl = {k: np.ascontiguousarray(tt[k][lo:hi]) for k in ("p", "g", "master", "m", "v")}
            adamw_mixed(sl["p"], sl["g"], sl["master"], sl["m"], sl["v"], hp, t, p_is_f16, lib)
            for k in ("p", "master", "m", "v"):
                tt[k][lo:hi] = sl[k]
        elif mode == SPLIT:
            sl = {k: np.ascontiguousarray(tt[k][lo:hi]) for k in ("p", "g", "r", "m", "v")}
            adamw_mixed_split(sl["p"], sl["g"], sl["r"], sl["m"], sl["v"], hp, t, lib)
            for k in ("p", "r", "m", "v"):
                tt[k][lo:hi] = sl[k]
        elif mode.startswith("pure"):
            keys = ["p", "g", "m", "v"] + (["c"] if "c" in tt else [])
            sl = {k: np.ascontiguousarray(tt[k][lo:hi]) for k in keys}
            adamw_pure(sl["p"], sl["g"], sl["m"], sl["v"], sl.get("c"), hp, t, lib)
            for k in keys:
                if k != "g":
                    tt[k][lo:hi] = sl[k]
        elif mode == KAHAN:
            sl = {k: np.ascontiguousarray(tt[k][lo:hi]) for k in ("p", "g", "m", "v", "c")}
            adamw_kahan(sl["p"], sl["g"], sl["m"], sl["v"], sl["c"], hp, t, lib)
            for k in ("p", "m", "v", "c"):
                tt[k][lo:hi] = sl[k]
        else:
            raise ValueError(f"unknown mode {mode!r}")
    return t


@dataclass
class LossScale:
    """Dynamic loss-scale state and rule (fp32 scale, int32 growth tracker)."""
    scale: float = 65536.0
    tracker: int = 0
    growth: float = 2.0
    backoff: float = 0.5
    interval: int = 2000

    def inv(self, lib=None) -> float:
        lib = lib or load()
        return float(lib.oracle_inv_scale(float(np.float32(self.scale))))

    def update(self, found_inf: bool, lib=None):
        lib = lib or load()
        s = _F(float(np.float32(self.scale)))
        t = ctypes.c_int32(int(self.tracker))
        lib.oracle_update_loss_scale(ctypes.byref(s), ctypes.byref(t), int(bool(found_inf)),
                                     float(np.float32(self.growth)), float(np.float32(self.backoff)),
                                     int(self.interval))
        self.scale, self.tracker = float(s.value), int(t.value)


def amp_step_list(mode: str, tensors: list, hp: HParams, step: int, ls: LossScale, *, p_is_f16=True,
                  shard_begin=0, shard_end=None, flat_align=1, lib=None) -> int:
    """fp16-AMP step with a dynamic loss scale: the overflow test over every
    gradient of the list, the step (unless skipped) with the gradient multiplier
    1/scale, then the scale update from the test's outcome.  Returns the new
    step counter; ``ls`` is updated in place."""
    lib = lib or load()
    found = any(any_nonfinite(tt["g"], p_is_f16, lib) for tt in tensors)
    hps = HParams(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, ls.inv(lib))
    new_step = step if found else step_list(mode, tensors, hps, step, p_is_f16=p_is_f16,
                                            shard_begin=shard_begin, shard_end=shard_end,
                                            flat_align=flat_align, lib=lib)
    ls.update(found, lib)
    return new_step


def warmup_linear_lr(t: int, base_lr: float = 2e-4, warmup: int = 500) -> float:
    """Learning rate of 1-based step ``t`` under the linear schedule with warmup
    (the opt-125m command: --learning_rate 0.0002 --lr_scheduler_type linear
    --warmup_steps 500).  Inside the warmup it rises linearly, lr * t / warmup;
    the decay phase needs the total step count, which the bounded runs here
    never reach.  Returned as the fp32 value both sides receive."""
    return float(np.float32(base_lr * min(1.0, t / warmup)))
