"""Python binding of the MI355X fused AdamW step (``libadamw_amd.so``).

Argument marshalling only: every step of the optimizer runs in the library's
HIP kernels.  The functions carry the names of the C ABI in ``include/adamw.h``
and accept torch tensors (their ``data_ptr()`` is passed) or raw integer device
addresses.  PyTorch supplies device memory and streams; with ``stream=None`` the
work goes on ``torch.cuda.current_stream()``.

There is no fallback: if the shared library has not been built the import
fails, and every non-OK status raises :class:`AdamWError`.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Sequence

import torch  # loads the HIP runtime the library then binds to

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libadamw_amd.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python adamw_optimizer_step_apply_amd/build.py` "
                      "(or __graft_entry__.build())")

_lib = None

# enums of adamw.h
OK, E_INVALID, E_UNSUPPORTED, E_NOMEM, E_HIP = 0, 1, 2, 3, 4
F32, BF16, F16 = 0, 1, 2
MIXED, PURE_KAHAN, MIXED_SPLIT = 0, 1, 2
KAHAN_NONE, KAHAN_BF16, KAHAN_F32 = 0, 1, 2   # compensation buffer of a pure-bf16 step (PurePrecision.kahan)
STREAM_PARAM, STREAM_GRAD, STREAM_EXP_AVG, STREAM_EXP_AVG_SQ, STREAM_AUX = range(5)
BLOCKED_STATE = 1 << 8        # flat_mask bit: exp_avg / exp_avg_sq / aux in one blocked buffer
FLAT_PAD8 = 1 << 9            # flat_mask bit: every tensor starts at a multiple of 8 in the flat index
STATE_BLOCK_ELEMS = 16384     # elements per block of a blocked state buffer (ADAMW_STATE_BLOCK_ELEMS)
NOALLOC_SCRATCH_BYTES = 16 << 20   # the allocation-free step's per-GPU workspace (ADAMW_NOALLOC_SCRATCH_BYTES)
NUM_STREAMS = 5
_STATUS = {0: "ADAMW_OK", 1: "ADAMW_E_INVALID", 2: "ADAMW_E_UNSUPPORTED", 3: "ADAMW_E_NOMEM", 4: "ADAMW_E_HIP"}


EXPORTED = ("adamw_step", "adamw_multi_tensor_step", "adamw_multi_tensor_step_noalloc", "adamw_multi_tensor_step_amp",
            "adamw_pure_multi_tensor_step",
            "adamw_check_finite",
            "adamw_last_error", "adamw_release_workspace", "adamw_abi_version", "adamw_plan_inspect",
            "adamw_plan_inspect_bytes", "adamw_set_chunk_elems", "adamw_set_single_launch_max_workgroups",
            "adamw_blocked_state_bytes", "adamw_blocked_state_copy")


class adamw_hparams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float), ("inv_loss_scale", ctypes.c_float)]


class adamw_pure_precision(ctypes.Structure):
    _fields_ = [("exp_avg", ctypes.c_int), ("exp_avg_sq", ctypes.c_int), ("kahan", ctypes.c_int32)]


class adamw_loss_scaler(ctypes.Structure):
    _fields_ = [("growth_factor", ctypes.c_float), ("backoff_factor", ctypes.c_float),
                ("growth_interval", ctypes.c_int32)]


class adamw_tensor_list(ctypes.Structure):
    _fields_ = [("n_tensors", ctypes.c_int64), ("numel", ctypes.POINTER(ctypes.c_int64)),
                ("ptr", ctypes.POINTER(ctypes.c_void_p) * NUM_STREAMS),
                ("shard_begin", ctypes.c_int64), ("shard_end", ctypes.c_int64), ("flat_mask", ctypes.c_uint32)]


_vp = ctypes.c_void_p


def _load(path: str) -> None:
    """Loads the library at ``path`` and declares its C signatures."""
    global _lib
    lib = ctypes.CDLL(path)
    _declare(lib)
    _lib = lib


def _declare(_lib):
    _lib.adamw_step.restype = ctypes.c_int
    _lib.adamw_step.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int64, _vp, _vp, _vp, _vp, _vp,
                                ctypes.POINTER(adamw_hparams), _vp, _vp, _vp]
    _lib.adamw_multi_tensor_step.restype = ctypes.c_int
    _lib.adamw_multi_tensor_step.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(adamw_tensor_list),
                                             ctypes.POINTER(adamw_hparams), _vp, _vp, _vp]
    _lib.adamw_multi_tensor_step_noalloc.restype = ctypes.c_int
    _lib.adamw_multi_tensor_step_noalloc.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(adamw_tensor_list),
                                                     ctypes.POINTER(adamw_hparams), _vp, _vp, _vp]
    _lib.adamw_multi_tensor_step_amp.restype = ctypes.c_int
    _lib.adamw_multi_tensor_step_amp.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(adamw_tensor_list),
                                                 ctypes.POINTER(adamw_hparams), _vp, _vp, _vp,
                                                 ctypes.POINTER(adamw_loss_scaler), _vp]
    _lib.adamw_pure_multi_tensor_step.restype = ctypes.c_int
    _lib.adamw_pure_multi_tensor_step.argtypes = [ctypes.POINTER(adamw_pure_precision),
                                                  ctypes.POINTER(adamw_tensor_list), ctypes.POINTER(adamw_hparams),
                                                  _vp, _vp, _vp]
    _lib.adamw_check_finite.restype = ctypes.c_int
    _lib.adamw_check_finite.argtypes = [ctypes.c_int, ctypes.POINTER(adamw_tensor_list), _vp, _vp]
    _lib.adamw_last_error.restype = ctypes.c_char_p
    _lib.adamw_last_error.argtypes = []
    _lib.adamw_release_workspace.restype = None
    _lib.adamw_release_workspace.argtypes = []
    _lib.adamw_abi_version.restype = ctypes.c_int
    _lib.adamw_abi_version.argtypes = []
    _lib.adamw_plan_inspect.restype = ctypes.c_int64
    _lib.adamw_plan_inspect.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(adamw_tensor_list), ctypes.c_int,
                                        ctypes.POINTER(ctypes.c_int64), ctypes.c_int64]
    _lib.adamw_plan_inspect_bytes.restype = ctypes.c_int64
    _lib.adamw_plan_inspect_bytes.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(adamw_pure_precision),
                                              ctypes.POINTER(adamw_tensor_list), ctypes.c_int,
                                              ctypes.POINTER(ctypes.c_uint64), ctypes.c_int64]
    _lib.adamw_blocked_state_bytes.restype = ctypes.c_int64
    _lib.adamw_blocked_state_bytes.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(adamw_pure_precision),
                                               ctypes.POINTER(adamw_tensor_list)]
    _lib.adamw_blocked_state_copy.restype = ctypes.c_int
    _lib.adamw_blocked_state_copy.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(adamw_pure_precision),
                                              ctypes.POINTER(adamw_tensor_list), _vp, ctypes.c_int, _vp]
    _lib.adamw_set_chunk_elems.restype = ctypes.c_int64
    _lib.adamw_set_chunk_elems.argtypes = [ctypes.c_int64]
    _lib.adamw_set_single_launch_max_workgroups.restype = ctypes.c_int64
    _lib.adamw_set_single_launch_max_workgroups.argtypes = [ctypes.c_int64]


_load(LIB_PATH)
ABI_VERSION = 8               # ADAMW_ABI_VERSION of the header this binding follows
if _lib.adamw_abi_version() != ABI_VERSION:
    raise ImportError(f"{LIB_PATH} has ABI version {_lib.adamw_abi_version()}, this binding expects {ABI_VERSION}: "
                      "rebuild the library")


class AdamWError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


@dataclass
class HParams:
    """AdamW hyper-parameters (fp32 in the library).  Defaults: the opt-1.3b
    recipe of "[pure bf16 training] w/ AnyPrecisionAdamW and Kahan summation"
    (lr 0.0002, betas 0.9/0.95, weight decay 0.1) and eps 1e-8."""
    lr: float = 2e-4
    beta1: float = 0.9
    beta2: float = 0.95
    eps: float = 1e-8
    weight_decay: float = 0.1
    inv_loss_scale: float = 1.0

    def c(self) -> adamw_hparams:
        return adamw_hparams(self.lr, self.beta1, self.beta2, self.eps, self.weight_decay, self.inv_loss_scale)


def _addr(x) -> int:
    if x is None:
        return 0
    if isinstance(x, torch.Tensor):
        return x.data_ptr()
    return int(x)


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _check(status: int):
    if status != OK:
        raise AdamWError(status, (_lib.adamw_last_error() or b"").decode())


def _hp(hp) -> adamw_hparams:
    if isinstance(hp, adamw_hparams):
        return hp
    if hp is None:
        hp = HParams()
    return hp.c()


class TensorList:
    """Marshals a tensor list into an ``adamw_tensor_list`` and keeps the ctypes
    arrays, and every tensor given, alive as long as it lives (addresses given
    as integers are the caller's to keep valid).  ``streams`` is a sequence of
    5 sequences (param, grad, exp_avg, exp_avg_sq, aux) of tensors or
    addresses; a stream flagged in ``flat_mask`` holds one flat shard buffer;
    ``None`` leaves a stream unset."""

    def __init__(self, numels: Sequence[int], streams, shard_begin: int = 0, shard_end: int = -1,
                 flat_mask: int = 0):
        n = len(numels)
        self._numel = (ctypes.c_int64 * max(n, 1))(*[int(x) for x in numels])
        self._arrays = []
        self._tensors = [x for items in streams if items is not None for x in items if isinstance(x, torch.Tensor)]
        s = adamw_tensor_list()
        s.n_tensors = n
        s.numel = ctypes.cast(self._numel, ctypes.POINTER(ctypes.c_int64))
        for k in range(NUM_STREAMS):
            items = streams[k] if k < len(streams) else None
            if items is None:
                s.ptr[k] = ctypes.POINTER(ctypes.c_void_p)()
                continue
            arr = (ctypes.c_void_p * max(len(items), 1))(*[_addr(x) for x in items])
            self._arrays.append(arr)
            s.ptr[k] = ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))
        s.shard_begin = int(shard_begin)
        s.shard_end = int(shard_end)
        s.flat_mask = int(flat_mask)
        self.c = s
        self.numels = [int(x) for x in numels]


def adamw_step(mode: int, p_dtype: int, n: int, param, grad, exp_avg, exp_avg_sq, aux, hp, d_step,
               d_found_inf=None, stream=None) -> None:
    """One AdamW step over one contiguous range of ``n`` elements (C ABI adamw_step)."""
    h = _hp(hp)
    _check(_lib.adamw_step(mode, p_dtype, int(n), _addr(param), _addr(grad), _addr(exp_avg), _addr(exp_avg_sq),
                           _addr(aux), ctypes.byref(h), _addr(d_step), _addr(d_found_inf), _stream(stream)))


def adamw_multi_tensor_step(mode: int, p_dtype: int, tensors: TensorList, hp, d_step, d_found_inf=None,
                            stream=None) -> None:
    """One AdamW step over a tensor list or its ZeRO shard (C ABI adamw_multi_tensor_step)."""
    h = _hp(hp)
    _check(_lib.adamw_multi_tensor_step(mode, p_dtype, ctypes.byref(tensors.c), ctypes.byref(h), _addr(d_step),
                                        _addr(d_found_inf), _stream(stream)))


def adamw_multi_tensor_step_noalloc(mode: int, p_dtype: int, tensors: TensorList, hp, d_step, d_found_inf=None,
                                    stream=None) -> None:
    """adamw_multi_tensor_step without any device allocation: the workspace is
    the library's static per-GPU array (C ABI adamw_multi_tensor_step_noalloc)."""
    h = _hp(hp)
    _check(_lib.adamw_multi_tensor_step_noalloc(mode, p_dtype, ctypes.byref(tensors.c), ctypes.byref(h),
                                                _addr(d_step), _addr(d_found_inf), _stream(stream)))


@dataclass
class LossScaler:
    """Dynamic loss-scaling rule (growth after growth_interval clean steps,
    back-off on an inf/NaN gradient)."""
    growth_factor: float = 2.0
    backoff_factor: float = 0.5
    growth_interval: int = 2000

    def c(self) -> adamw_loss_scaler:
        return adamw_loss_scaler(self.growth_factor, self.backoff_factor, int(self.growth_interval))


def loss_scale_state(scale: float = 65536.0, device="cuda") -> torch.Tensor:
    """A device adamw_loss_scale_state {float scale; int32 growth_tracker} as an
    8-byte tensor (view it as float32 for the scale, int32 for the tracker)."""
    t = torch.zeros(2, dtype=torch.float32, device=device)
    t[0] = scale
    return t


def adamw_multi_tensor_step_amp(mode: int, p_dtype: int, tensors: TensorList, hp, d_step, d_found_inf,
                                d_scale, scaler: LossScaler = None, stream=None) -> None:
    """AdamW step that unscales by a device-resident dynamic loss scale and then
    advances it from the overflow flag (C ABI adamw_multi_tensor_step_amp)."""
    h = _hp(hp)
    sc = (scaler or LossScaler()).c()
    _check(_lib.adamw_multi_tensor_step_amp(mode, p_dtype, ctypes.byref(tensors.c), ctypes.byref(h), _addr(d_step),
                                            _addr(d_found_inf), _addr(d_scale), ctypes.byref(sc),
                                            _stream(stream)))


@dataclass
class PurePrecision:
    """State precisions of a pure-bf16 step: exp_avg / exp_avg_sq dtype (F32 or
    BF16) and the aux stream's compensation buffer: KAHAN_NONE (False),
    KAHAN_BF16 (True) or KAHAN_F32."""
    exp_avg: int = BF16
    exp_avg_sq: int = BF16
    kahan: int = KAHAN_BF16

    def c(self) -> adamw_pure_precision:
        return adamw_pure_precision(int(self.exp_avg), int(self.exp_avg_sq), int(self.kahan))

    @classmethod
    def from_optim_args(cls, text: str) -> "PurePrecision":
        """The precisions named by an AnyPrecisionAdamW option string of the
        form used with ``--optim_args`` ("key=value, ..."): momentum_dtype and
        variance_dtype (bfloat16 or float32, default bfloat16),
        use_kahan_summation (true/false, default false) and
        compensation_buffer_dtype (bfloat16 or float32, default bfloat16).
        Other keys, or other values, raise ValueError."""
        dtypes = {"bfloat16": BF16, "torch.bfloat16": BF16, "float32": F32, "torch.float32": F32}
        opts = {"momentum_dtype": "bfloat16", "variance_dtype": "bfloat16", "use_kahan_summation": "false",
                "compensation_buffer_dtype": "bfloat16"}
        for item in filter(None, (x.strip() for x in text.split(","))):
            key, sep, value = (x.strip() for x in item.partition("="))
            if not sep or key not in opts:
                raise ValueError(f"optim_args: unknown or malformed entry {item!r}")
            opts[key] = value.lower()
        for key in ("momentum_dtype", "variance_dtype", "compensation_buffer_dtype"):
            if opts[key] not in dtypes:
                raise ValueError(f"optim_args: {key}={opts[key]} (bfloat16 or float32)")
        if opts["use_kahan_summation"] not in ("true", "false", "1", "0"):
            raise ValueError(f"optim_args: use_kahan_summation={opts['use_kahan_summation']} (true or false)")
        kahan = KAHAN_NONE
        if opts["use_kahan_summation"] in ("true", "1"):
            kahan = KAHAN_F32 if dtypes[opts["compensation_buffer_dtype"]] == F32 else KAHAN_BF16
        return cls(dtypes[opts["momentum_dtype"]], dtypes[opts["variance_dtype"]], kahan)


def adamw_pure_multi_tensor_step(prec: PurePrecision, tensors: TensorList, hp, d_step, d_found_inf=None,
                                 stream=None) -> None:
    """Pure-bf16 step with chosen state precisions (C ABI adamw_pure_multi_tensor_step)."""
    h = _hp(hp)
    pc = prec.c()
    _check(_lib.adamw_pure_multi_tensor_step(ctypes.byref(pc), ctypes.byref(tensors.c), ctypes.byref(h),
                                             _addr(d_step), _addr(d_found_inf), _stream(stream)))


def adamw_check_finite(g_dtype: int, grads: TensorList, d_found_inf, stream=None) -> None:
    """Zero ``d_found_inf``, then set it to 1 if any gradient is inf/NaN (C ABI adamw_check_finite)."""
    _check(_lib.adamw_check_finite(g_dtype, ctypes.byref(grads.c), _addr(d_found_inf), _stream(stream)))


def adamw_last_error() -> str:
    return (_lib.adamw_last_error() or b"").decode()


def adamw_release_workspace() -> None:
    _lib.adamw_release_workspace()


def adamw_abi_version() -> int:
    return _lib.adamw_abi_version()


def adamw_plan_inspect(mode: int, p_dtype: int, tensors: TensorList, for_check: bool = False):
    """The chunk plan as a list of (tensor, offset_in_tensor, count, is_vector, flat_pos, segment)."""
    n = _lib.adamw_plan_inspect(mode, p_dtype, ctypes.byref(tensors.c), int(for_check), None, 0)
    if n < 0:
        raise AdamWError(E_INVALID, adamw_last_error())
    buf = (ctypes.c_int64 * (6 * max(n, 1)))()
    n2 = _lib.adamw_plan_inspect(mode, p_dtype, ctypes.byref(tensors.c), int(for_check), buf, n)
    assert n2 == n
    return [tuple(buf[6 * i:6 * i + 6]) for i in range(n)]


def adamw_plan_inspect_bytes(mode: int, p_dtype: int, tensors: TensorList, for_check: bool = False,
                             prec: "PurePrecision" = None):
    """The chunk plan with the device bytes of every chunk: (rows, ranges), rows
    an int64 array (chunks, 6) of adamw_plan_inspect's fields, ranges a uint64
    array (chunks, 5, 2) of [lo, hi) per stream, (0, 0) for an untouched stream."""
    import numpy as np
    pc = ctypes.byref(prec.c()) if prec is not None else None
    n = _lib.adamw_plan_inspect_bytes(mode, p_dtype, pc, ctypes.byref(tensors.c), int(for_check), None, 0)
    if n < 0:
        raise AdamWError(E_INVALID, adamw_last_error())
    out = np.zeros((max(n, 1), 16), dtype=np.uint64)
    n2 = _lib.adamw_plan_inspect_bytes(mode, p_dtype, pc, ctypes.byref(tensors.c), int(for_check),
                                       out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)), n)
    assert n2 == n
    out = out[:n]
    return out[:, :6].view(np.int64), out[:, 6:].reshape(n, NUM_STREAMS, 2)


def adamw_blocked_state_bytes(mode: int, p_dtype: int, tensors: TensorList, prec: "PurePrecision" = None) -> int:
    """Bytes of the blocked state buffer for the per-tensor state that ``tensors``
    describes (C ABI adamw_blocked_state_bytes)."""
    pc = ctypes.byref(prec.c()) if prec is not None else None
    n = _lib.adamw_blocked_state_bytes(mode, p_dtype, pc, ctypes.byref(tensors.c))
    if n < 0:
        raise AdamWError(E_INVALID, adamw_last_error())
    return n


def adamw_blocked_state_copy(mode: int, p_dtype: int, tensors: TensorList, blocked, to_blocked: bool = True,
                             prec: "PurePrecision" = None, stream=None) -> None:
    """Copies the state between per-tensor buffers and a blocked buffer, either way
    (C ABI adamw_blocked_state_copy); returns when the copy is done."""
    pc = ctypes.byref(prec.c()) if prec is not None else None
    _check(_lib.adamw_blocked_state_copy(mode, p_dtype, pc, ctypes.byref(tensors.c), _addr(blocked),
                                         int(bool(to_blocked)), _stream(stream)))


def make_blocked_state(mode: int, p_dtype: int, numels: Sequence[int], exp_avg, exp_avg_sq, aux=None,
                       shard_begin: int = 0, shard_end: int = -1, pad8: bool = True, flat_mask: int = 0,
                       prec: "PurePrecision" = None, stream=None, device=None):
    """Optimizer-owned state in the blocked layout, filled from per-tensor state.

    ``exp_avg``, ``exp_avg_sq`` and ``aux`` are sequences of per-tensor tensors
    (one per entry of ``numels``; with flat_mask bits 2-4, one flat shard tensor)
    holding the state to start from -- e.g. zero moments and the fp32 master
    weights (tensors, or device addresses with ``device`` given).  Allocates one
    zero-filled uint8 tensor on their device, copies the state in with the
    library's copy kernel, and returns ``(blocked, step_mask)``:
    a step then takes ``TensorList(numels, [params, grads, [blocked], None, None],
    shard_begin, shard_end, step_mask)``.  ``pad8`` lays the buffer out in the
    padded flat index (ADAMW_FLAT_PAD8), which keeps every tensor of any length on
    the 16-byte vector path when params and grads are 16-byte aligned."""
    streams = [None, None, list(exp_avg), list(exp_avg_sq), None if aux is None else list(aux)]
    mask = (flat_mask & 0x1c) | (FLAT_PAD8 if pad8 else 0)
    tl = TensorList(numels, streams, shard_begin, shard_end, mask)
    nbytes = adamw_blocked_state_bytes(mode, p_dtype, tl, prec)
    if device is None:
        tensors = [t for t in streams[2] if isinstance(t, torch.Tensor)]
        if not tensors:
            raise ValueError("make_blocked_state: pass device= when the state is given as addresses")
        device = tensors[0].device
    blocked = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=device)
    adamw_blocked_state_copy(mode, p_dtype, tl, blocked, True, prec, stream)
    return blocked, mask | BLOCKED_STATE


def adamw_set_chunk_elems(elems: int) -> int:
    r = _lib.adamw_set_chunk_elems(int(elems))
    if r < 0:
        raise AdamWError(E_INVALID, f"chunk size {elems} rejected")
    return r


def adamw_set_single_launch_max_workgroups(max_workgroups: int) -> int:
    """Largest grid (in workgroups: 8 per chunk of a step, 1 per check chunk)
    that runs as one launch; 0 = always two launches, < 0 = the default.
    Returns the value now in force."""
    return _lib.adamw_set_single_launch_max_workgroups(int(max_workgroups))


def library_path() -> str:
    return LIB_PATH
