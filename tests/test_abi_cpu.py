"""The C ABI without a GPU: the library loads, exports every function that
include/adamw.h declares, rejects bad arguments before any HIP call, and the
planner partitions lists and shards correctly (through adamw_plan_inspect)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest
import torch

import adamw_optimizer_step_apply_amd as A

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "adamw.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(adamw_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) >= {"adamw_step", "adamw_multi_tensor_step", "adamw_check_finite"}
    lib = ctypes.CDLL(A.library_path())
    for n in names:
        assert hasattr(lib, n), f"{n} declared in adamw.h but not exported"
    assert set(names) == set(A.EXPORTED)


def test_abi_version():
    src = open(HEADER).read()
    v = int(re.search(r"#define ADAMW_ABI_VERSION (\d+)", src).group(1))
    assert A.adamw_abi_version() == v == A.ABI_VERSION


def test_binding_constants_match_the_header():
    """The binding restates the header's enums and layout constants: they must agree."""
    src = open(HEADER).read()

    def define(name):
        m = re.search(rf"#define {name} \(?(\d+)u?(?: << (\d+)\))?", src)
        return int(m.group(1)) << int(m.group(2) or 0)

    assert define("ADAMW_BLOCKED_STATE") == A.BLOCKED_STATE
    assert define("ADAMW_FLAT_PAD8") == A.FLAT_PAD8
    assert define("ADAMW_STATE_BLOCK_ELEMS") == A.STATE_BLOCK_ELEMS == 16384
    for name, value in (("ADAMW_OK", A.OK), ("ADAMW_E_INVALID", A.E_INVALID), ("ADAMW_E_UNSUPPORTED", A.E_UNSUPPORTED),
                        ("ADAMW_E_NOMEM", A.E_NOMEM), ("ADAMW_E_HIP", A.E_HIP), ("ADAMW_F32", A.F32),
                        ("ADAMW_BF16", A.BF16), ("ADAMW_F16", A.F16), ("ADAMW_MIXED", A.MIXED),
                        ("ADAMW_PURE_KAHAN", A.PURE_KAHAN), ("ADAMW_MIXED_SPLIT", A.MIXED_SPLIT),
                        ("ADAMW_STREAM_PARAM", A.STREAM_PARAM), ("ADAMW_STREAM_GRAD", A.STREAM_GRAD),
                        ("ADAMW_STREAM_EXP_AVG", A.STREAM_EXP_AVG), ("ADAMW_STREAM_EXP_AVG_SQ", A.STREAM_EXP_AVG_SQ),
                        ("ADAMW_STREAM_AUX", A.STREAM_AUX), ("ADAMW_NUM_STREAMS", A.NUM_STREAMS)):
        assert int(re.search(rf"\b{name} = (\d+)", src).group(1)) == value, name
    for name, value in (("ADAMW_KAHAN_NONE", A.KAHAN_NONE), ("ADAMW_KAHAN_BF16", A.KAHAN_BF16),
                        ("ADAMW_KAHAN_F32", A.KAHAN_F32)):
        assert define(name) == value, name


LAYOUT_PROGRAM = r"""
#include <stddef.h>
#include <stdio.h>
#include "adamw.h"
#define F(T, m) printf(#T "." #m " %zu\n", offsetof(T, m))
int main(void)
{
    printf("adamw_hparams %zu\n", sizeof(adamw_hparams));
    F(adamw_hparams, lr); F(adamw_hparams, beta1); F(adamw_hparams, beta2); F(adamw_hparams, eps);
    F(adamw_hparams, weight_decay); F(adamw_hparams, inv_loss_scale);
    printf("adamw_pure_precision %zu\n", sizeof(adamw_pure_precision));
    F(adamw_pure_precision, exp_avg); F(adamw_pure_precision, exp_avg_sq); F(adamw_pure_precision, kahan);
    printf("adamw_loss_scaler %zu\n", sizeof(adamw_loss_scaler));
    F(adamw_loss_scaler, growth_factor); F(adamw_loss_scaler, backoff_factor); F(adamw_loss_scaler, growth_interval);
    printf("adamw_tensor_list %zu\n", sizeof(adamw_tensor_list));
    F(adamw_tensor_list, n_tensors); F(adamw_tensor_list, numel); F(adamw_tensor_list, ptr);
    F(adamw_tensor_list, shard_begin); F(adamw_tensor_list, shard_end); F(adamw_tensor_list, flat_mask);
    printf("adamw_loss_scale_state %zu\n", sizeof(adamw_loss_scale_state));
    F(adamw_loss_scale_state, scale); F(adamw_loss_scale_state, growth_tracker);
    return 0;
}
"""


def test_binding_structs_match_the_c_layout(tmp_path):
    """Sizes and field offsets of the binding's ctypes structures equal the C
    compiler's for the header (a mismatch would pass garbage across the ABI)."""
    src = tmp_path / "layout.c"
    src.write_text(LAYOUT_PROGRAM)
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)], check=True)
    c = dict(line.rsplit(" ", 1) for line in subprocess.run([str(exe)], capture_output=True, text=True,
                                                               check=True).stdout.splitlines())
    c = {k: int(v) for k, v in c.items()}
    for cls in (A.adamw_hparams, A.adamw_pure_precision, A.adamw_loss_scaler, A.adamw_tensor_list):
        assert ctypes.sizeof(cls) == c[cls.__name__], cls.__name__
        for name, _ in cls._fields_:
            assert getattr(cls, name).offset == c[f"{cls.__name__}.{name}"], (cls.__name__, name)
    # the device-resident loss-scale state: fp32 scale, then int32 tracker
    assert c["adamw_loss_scale_state"] == 8 and c["adamw_loss_scale_state.scale"] == 0
    assert c["adamw_loss_scale_state.growth_tracker"] == 4
    st = A.loss_scale_state(1024.0, device="cpu")
    assert st.numel() * st.element_size() == 8 and float(st[0]) == 1024.0 and int(st.view(torch.int32)[1]) == 0


FAKE = 0x7f0000000000     # never dereferenced: validation fails before any HIP call


def _tl(numels, base=FAKE, esz=(2, 2, 4, 4, 4), **kw):
    streams = []
    for s in range(5):
        offs = np.concatenate([[0], np.cumsum(numels)[:-1]]) if numels else []
        streams.append([base + s * (1 << 36) + int(o) * esz[s] for o in offs])
    return A.TensorList(numels, streams, **kw)


@pytest.mark.parametrize("call,needle", [
    (lambda: A.adamw_multi_tensor_step(A.MIXED, A.F32, _tl([10]), A.HParams(), FAKE, stream=0), "p_dtype"),
    (lambda: A.adamw_multi_tensor_step(A.PURE_KAHAN, A.F16, _tl([10]), A.HParams(), FAKE, stream=0), "BF16"),
    (lambda: A.adamw_multi_tensor_step(7, A.BF16, _tl([10]), A.HParams(), FAKE, stream=0), "mode"),
    (lambda: A.adamw_multi_tensor_step(A.MIXED, A.BF16, _tl([10]), A.HParams(beta2=1.0), FAKE, stream=0), "beta"),
    (lambda: A.adamw_multi_tensor_step(A.MIXED, A.BF16, _tl([10]), A.HParams(eps=-1e-8), FAKE, stream=0), "eps"),
    (lambda: A.adamw_multi_tensor_step(A.MIXED, A.BF16, _tl([10]), A.HParams(lr=float("inf")), FAKE, stream=0),
     "finite"),
    (lambda: A.adamw_multi_tensor_step(A.MIXED, A.BF16, _tl([10]), A.HParams(inv_loss_scale=0.0), FAKE, stream=0),
     "inv_loss_scale"),
    (lambda: A.adamw_multi_tensor_step(A.MIXED, A.BF16, _tl([10]), A.HParams(), 0, stream=0), "d_step"),
    (lambda: A.adamw_multi_tensor_step(A.MIXED, A.BF16, _tl([10]), A.HParams(), FAKE + 2, stream=0), "aligned"),
    (lambda: A.adamw_multi_tensor_step(A.MIXED, A.BF16, _tl([10, -1]), A.HParams(), FAKE, stream=0), "numel"),
    (lambda: A.adamw_multi_tensor_step(A.MIXED, A.BF16, _tl([10, 5], shard_begin=3, shard_end=16), A.HParams(),
                                       FAKE, stream=0), "shard"),
    (lambda: A.adamw_multi_tensor_step(A.MIXED, A.BF16, _tl([10, 5], shard_begin=6, shard_end=5), A.HParams(),
                                       FAKE, stream=0), "shard"),
    (lambda: A.adamw_multi_tensor_step(A.MIXED, A.BF16, _tl([10], flat_mask=1 << 5), A.HParams(), FAKE, stream=0),
     "flat_mask"),
    (lambda: A.adamw_multi_tensor_step(A.MIXED, A.BF16, _tl([10], base=FAKE + 1), A.HParams(), FAKE, stream=0),
     "aligned"),
    (lambda: A.adamw_multi_tensor_step(A.MIXED, A.BF16, A.TensorList([10], [[FAKE], [0], [FAKE], [FAKE], [FAKE]]),
                                       A.HParams(), FAKE, stream=0), "grad"),
    (lambda: A.adamw_multi_tensor_step(A.MIXED, A.BF16, A.TensorList([10], [[FAKE], None, [FAKE], [FAKE], [FAKE]]),
                                       A.HParams(), FAKE, stream=0), "grad"),
    (lambda: A.adamw_step(A.MIXED, A.BF16, -1, FAKE, FAKE, FAKE, FAKE, FAKE, A.HParams(), FAKE, stream=0), "n < 0"),
    (lambda: A.adamw_step(A.MIXED, A.BF16, 5, FAKE, 0, FAKE, FAKE, FAKE, A.HParams(), FAKE, stream=0), "null"),
    (lambda: A.adamw_multi_tensor_step_amp(A.MIXED, A.F16, _tl([10]), A.HParams(), FAKE, 0, FAKE, stream=0),
     "d_found_inf"),
    (lambda: A.adamw_multi_tensor_step_amp(A.MIXED, A.F16, _tl([10]), A.HParams(), FAKE, FAKE, 0, stream=0),
     "d_scale"),
    (lambda: A.adamw_multi_tensor_step_amp(A.MIXED, A.F16, _tl([10]), A.HParams(), FAKE, FAKE, FAKE,
                                           A.LossScaler(0.5, 0.5, 10), stream=0), "growth_factor"),
    (lambda: A.adamw_multi_tensor_step_amp(A.MIXED, A.F16, _tl([10]), A.HParams(), FAKE, FAKE, FAKE,
                                           A.LossScaler(2.0, 0.0, 10), stream=0), "backoff_factor"),
    (lambda: A.adamw_multi_tensor_step_amp(A.MIXED, A.F16, _tl([10]), A.HParams(), FAKE, FAKE, FAKE,
                                           A.LossScaler(2.0, 0.5, 0), stream=0), "growth_interval"),
    (lambda: A.adamw_multi_tensor_step(A.MIXED_SPLIT, A.F16, _tl([10], esz=(2, 2, 4, 4, 2)), A.HParams(), FAKE,
                                       stream=0), "MIXED_SPLIT"),
    (lambda: A.adamw_pure_multi_tensor_step(A.PurePrecision(A.BF16, A.BF16, 3), _tl([10], esz=(2, 2, 2, 2, 2)),
                                            A.HParams(), FAKE, stream=0), "ADAMW_KAHAN_F32"),
    (lambda: A.adamw_check_finite(A.F32, _tl([10]), FAKE, stream=0), "g_dtype"),
    (lambda: A.adamw_check_finite(A.F16, _tl([10]), 0, stream=0), "d_found_inf"),
    (lambda: A.adamw_check_finite(A.F16, _tl([10, 3], shard_begin=0, shard_end=14), FAKE, stream=0), "shard"),
])
def test_rejected_before_any_hip_call(call, needle):
    """Each bad call returns an error naming the problem.  None of them gets as
    far as a HIP call: on this GPU-less host that would fail with ADAMW_E_HIP."""
    with pytest.raises(A.AdamWError) as ei:
        call()
    assert ei.value.status in (A.E_INVALID, A.E_UNSUPPORTED)
    assert needle.lower() in str(ei.value).lower(), str(ei.value)


def test_valid_call_reaches_hip():
    """A valid call passes validation and fails only at the first HIP call here."""
    with pytest.raises(A.AdamWError) as ei:
        A.adamw_multi_tensor_step(A.MIXED, A.BF16, _tl([10, 20]), A.HParams(), FAKE, stream=0)
    assert ei.value.status == A.E_HIP


# ---------------------------------------------------------------------------
# planner
# ---------------------------------------------------------------------------

# workgroup size x 8 of each kernel family
DEFAULT_CHUNK = {A.MIXED: 16384, A.MIXED_SPLIT: 16384, A.PURE_KAHAN: 16384}


def check_plan(rows, numels, b, e, ptrs, esz, chunk_elems):
    """Rows partition [b, e) in flat order; each row lies in one tensor; vector
    rows hold a multiple of 8 elements, 16-byte aligned in every stream."""
    starts = np.concatenate([[0], np.cumsum(numels)]).astype(np.int64)
    pos = b
    for (t, off, n, vec, flat, seg) in rows:
        assert flat == pos and n > 0
        assert starts[t] + off == flat and off + n <= numels[t]
        if vec:
            assert n % 8 == 0 and n <= chunk_elems
            for s in range(5):
                if esz[s]:
                    assert (ptrs[s][t] + off * esz[s]) % 16 == 0
        else:
            assert n <= 4096
        pos += n
    assert pos == e


@pytest.mark.parametrize("seed", range(40))
def test_plan_partitions_random_lists(seed):
    rng = np.random.default_rng(seed)
    nt = int(rng.integers(0, 30))
    numels = [int(x) for x in rng.choice([0, 1, 3, 7, 8, 9, 16, 100, 2049, 16384, 16391, 70000], size=nt)]
    total = sum(numels)
    b = int(rng.integers(0, total + 1))
    e = int(rng.integers(b, total + 1))
    mode = A.MIXED if seed % 2 == 0 else A.PURE_KAHAN
    esz = (2, 2, 4, 4, 4) if mode == A.MIXED else (2, 2, 2, 2, 2)
    # per-stream base phase: all aligned, or random element phases
    phase = [0] * 5 if seed % 3 == 0 else [int(rng.integers(0, 8)) * esz[s] % 16 for s in range(5)]
    ptrs = []
    for s in range(5):
        base = FAKE + s * (1 << 36) + phase[s]
        offs = np.concatenate([[0], np.cumsum(numels)[:-1]]) if nt else []
        ptrs.append([base + int(o) * esz[s] + 256 * i for i, o in enumerate(offs)])
    tl = A.TensorList(numels, ptrs, b, e if rng.random() < 0.8 or e != total else -1)
    rows = A.adamw_plan_inspect(mode, A.BF16, tl)
    check_plan(rows, numels, b, e, ptrs, esz, DEFAULT_CHUNK[mode])
    if seed % 3 == 0:
        # all streams at one phase: at most 2 element rows per segment
        segs = {}
        for r in rows:
            segs.setdefault(r[5], []).append(r)
        for rs in segs.values():
            assert sum(1 for r in rs if not r[3]) <= 2 or sum(r[2] for r in rs) < 16


def test_plan_bert_shards():
    """The BERT list at DP=4: rank 0's shard lies inside the word embedding;
    ranks 1-3 cover several tensors with split ends."""
    import workloads
    wl = workloads.get("bert_52m")
    numels = wl.numels
    esz = (2, 2, 4, 4, 4)
    offs = np.concatenate([[0], np.cumsum(numels)[:-1]])
    ptrs = [[FAKE + s * (1 << 40) + int(o) * esz[s] for o in offs] for s in range(5)]
    nseg = []
    for r in range(4):
        b, e = wl.shard(r)
        tl = A.TensorList(numels, ptrs, b, e)
        rows = A.adamw_plan_inspect(A.MIXED, A.BF16, tl)
        check_plan(rows, numels, b, e, ptrs, esz, DEFAULT_CHUNK[A.MIXED])
        nseg.append(len({row[5] for row in rows}))
    assert nseg[0] == 1 and all(n > 1 for n in nseg[1:])


def test_plan_check_mode_uses_grad_stream_only():
    numels = [100, 5]
    ptrs = [None, [FAKE + 2, FAKE + 2 + 256], None, None, None]
    tl = A.TensorList(numels, ptrs)
    rows = A.adamw_plan_inspect(A.MIXED, A.F16, tl, for_check=True)
    assert rows[0][3] == 0 and rows[0][2] == 7       # head peel to the next 16-byte boundary
    assert sum(r[2] for r in rows) == 105


def test_chunk_size_knob():
    numels = [100_000]
    tl = _tl(numels)
    try:
        assert A.adamw_set_chunk_elems(8192) == 8192
        rows = A.adamw_plan_inspect(A.MIXED, A.BF16, tl)
        assert max(r[2] for r in rows) == 8192
        with pytest.raises(A.AdamWError):
            A.adamw_set_chunk_elems(1000)
    finally:
        A.adamw_set_chunk_elems(0)
    assert A.adamw_set_chunk_elems(0) == 0
    rows = A.adamw_plan_inspect(A.MIXED, A.BF16, tl)
    assert max(r[2] for r in rows) == 16384
    rows = A.adamw_plan_inspect(A.PURE_KAHAN, A.BF16, _tl(numels, esz=(2, 2, 2, 2, 2)))
    assert max(r[2] for r in rows) == 16384


C_PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "adamw.h"

int main(void)
{
    if (adamw_abi_version() != ADAMW_ABI_VERSION) return 1;
    adamw_hparams hp = {2e-4f, 0.9f, 0.95f, 1e-8f, 0.1f, 1.0f};
    int64_t numel[2] = {100, 37};
    void* p0[2] = {(void*)0x7f0000000000, (void*)0x7f0000010000};
    adamw_tensor_list list;
    memset(&list, 0, sizeof list);
    list.n_tensors = 2;
    list.numel = numel;
    for (int s = 0; s < ADAMW_NUM_STREAMS; ++s) list.ptr[s] = p0;
    list.shard_end = -1;
    /* bad dtype: rejected before any HIP call */
    if (adamw_multi_tensor_step(ADAMW_MIXED, ADAMW_F32, &list, &hp, (int32_t*)0x7f0000020000, NULL, NULL)
        != ADAMW_E_UNSUPPORTED) return 2;
    if (strstr(adamw_last_error(), "p_dtype") == NULL) return 3;
    /* plan introspection works without a GPU */
    int64_t rows[6 * 16];
    int64_t n = adamw_plan_inspect(ADAMW_MIXED, ADAMW_BF16, &list, 0, rows, 16);
    if (n <= 0 || rows[2] <= 0) return 4;
    adamw_pure_precision prec = {ADAMW_F32, ADAMW_BF16, 1};
    hp.beta1 = 1.0f;
    if (adamw_pure_multi_tensor_step(&prec, &list, &hp, (int32_t*)0x7f0000020000, NULL, NULL) != ADAMW_E_INVALID)
        return 5;
    printf("ok %lld chunks\n", (long long)n);
    return 0;
}
"""


def test_header_is_plain_c_and_library_callable_from_c(tmp_path):
    """adamw.h compiles as C99 and a C program links the library and gets the
    documented error codes (no GPU needed: every call here fails validation or
    only plans)."""
    import subprocess
    src = tmp_path / "abi.c"
    src.write_text(C_PROGRAM)
    exe = tmp_path / "abi"
    libdir = os.path.dirname(A.library_path())
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), str(src),
                    "-o", str(exe), "-L", libdir, "-ladamw_amd", f"-Wl,-rpath,{libdir}"], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    assert r.stdout.startswith("ok")


@pytest.mark.parametrize("seed", range(12))
def test_plan_blocked_state_never_straddles_a_block(seed):
    """With the blocked state layout every chunk lies inside one state block
    (block k = shard elements [k*B, (k+1)*B)), and the rows still partition the shard."""
    rng = np.random.default_rng(100 + seed)
    numels = [int(x) for x in rng.choice([1, 7, 8, 100, 2047, 2048, 2049, 5000, 8191, 8192, 8193, 20000, 40000], size=rng.integers(1, 12))]
    total = sum(numels)
    b = int(rng.integers(0, total))
    e = int(rng.integers(b + 1, total + 1))
    esz = (2, 2, 4, 4, 4)
    offs = np.concatenate([[0], np.cumsum(numels)[:-1]])
    ptrs = [[FAKE + s * (1 << 36) + int(o) * esz[s] for o in offs] for s in range(2)]
    ptrs += [[FAKE + 7 * (1 << 36)], None, None]
    tl = A.TensorList(numels, ptrs, b, e, flat_mask=A.BLOCKED_STATE)
    rows = A.adamw_plan_inspect(A.MIXED, A.BF16, tl)
    pos = b
    for (t, off, n, vec, flat, seg) in rows:
        assert flat == pos
        assert (flat - b) // A.STATE_BLOCK_ELEMS == (flat + n - 1 - b) // A.STATE_BLOCK_ELEMS
        pos += n
    assert pos == e


@pytest.mark.parametrize("seed", range(16))
def test_plan_padded_flat_index(seed):
    """ADAMW_FLAT_PAD8: tensors sit at multiples of 8 in the flat index.  The rows
    cover exactly the real elements of [b, e) in that padded space (written out
    slot by slot here); with 16-byte aligned per-tensor param/grad buffers, a
    blocked state and a shard start that is a multiple of 8, the only element
    rows are the last numel % 8 elements of a tensor or the shard's end."""
    rng = np.random.default_rng(500 + seed)
    numels = [int(x) for x in rng.choice([0, 1, 3, 7, 9, 100, 2049, 8191, 8193, 16391, 40001], size=rng.integers(1, 14))]
    slots = []
    for i, n in enumerate(numels):
        slots += [(i, j) for j in range(n)]
        slots += [None] * (-len(slots) % 8)
    total = len(slots)
    b = int(rng.integers(0, total // 8 + 1)) * 8 if seed % 2 == 0 else int(rng.integers(0, total + 1))
    e = int(rng.integers(b, total + 1))
    esz = (2, 2, 4, 4, 4)
    ptrs = [[FAKE + s * (1 << 36) + (1 << 20) * i for i in range(len(numels))] for s in range(2)]
    ptrs += [[FAKE + 7 * (1 << 36)], None, None]
    tl = A.TensorList(numels, ptrs, b, e, flat_mask=A.BLOCKED_STATE | A.FLAT_PAD8)
    rows = A.adamw_plan_inspect(A.MIXED, A.BF16, tl)
    covered = []
    for (t, off, n, vec, flat, seg) in rows:
        assert slots[flat] == (t, off)
        assert (flat - b) // A.STATE_BLOCK_ELEMS == (flat + n - 1 - b) // A.STATE_BLOCK_ELEMS
        covered += [(t, off + j) for j in range(n)]
        if seed % 2 == 0 and not vec:
            assert n < 8 and (off + n == numels[t] or flat + n == e), (t, off, n, numels[t])
    assert covered == [sl for sl in slots[b:e] if sl is not None]
    with pytest.raises(A.AdamWError, match="shard range"):
        A.adamw_plan_inspect(A.MIXED, A.BF16, A.TensorList(numels, ptrs, 0, total + 1,
                                                          flat_mask=A.BLOCKED_STATE | A.FLAT_PAD8))


def test_check_plan_ignores_blocked_bit():
    """The overflow check reads only grads: with the blocked bit its plan is the
    plan without it (no splits at state-block edges), and it needs no state buffer."""
    numels = [30000, 7, 20000, 1, 40000]
    offs = np.concatenate([[0], np.cumsum(numels)[:-1]])
    g = [FAKE + (1 << 36) + int(o) * 2 for o in offs]
    plain = A.adamw_plan_inspect(A.MIXED, A.F16, A.TensorList(numels, [None, g, None, None, None]), True)
    blocked = A.adamw_plan_inspect(A.MIXED, A.F16, A.TensorList(numels, [None, g, None, None, None],
                                                                flat_mask=A.BLOCKED_STATE), True)
    assert blocked == plain
    B = A.STATE_BLOCK_ELEMS
    assert any(flat // B != (flat + n - 1) // B for (_, _, n, _, flat, _) in plain)   # a blocked plan would cut here


@pytest.mark.parametrize("mode,esz", [(A.MIXED, (2, 2, 4, 4, 4)), (A.PURE_KAHAN, (2, 2, 2, 2, 2))])
def test_blocked_state_blocks_cut_the_plan(mode, esz):
    """B = 16384 elements in every mode: the segments of a blocked plan are
    exactly the pieces of the list cut at tensor edges and at multiples of B
    from the shard start, and no more."""
    block = A.STATE_BLOCK_ELEMS
    rng = np.random.default_rng(7)
    numels = [int(x) for x in rng.integers(1, 60000, size=9)]
    total = sum(numels)
    b, e = 12345, total - 777
    offs = np.concatenate([[0], np.cumsum(numels)[:-1]])
    ptrs = [[FAKE + s * (1 << 36) + int(o) * esz[s] for o in offs] for s in range(2)]
    ptrs += [[FAKE + 7 * (1 << 36)], None, None]
    rows = A.adamw_plan_inspect(mode, A.BF16, A.TensorList(numels, ptrs, b, e, flat_mask=A.BLOCKED_STATE))
    starts = set(int(x) for x in np.concatenate([[0], np.cumsum(numels)]))
    cuts = {x for x in starts if b < x < e} | {x for x in range(b + block, e, block)}
    want_segments = len(cuts) + 1
    assert len({r[5] for r in rows}) == want_segments
    for (t, off, n, vec, flat, seg) in rows:
        assert (flat - b) // block == (flat + n - 1 - b) // block


def test_validation_is_not_skipped_for_a_changed_list():
    """A list validated once is not walked again on the next call, but any change
    (one pointer, one size, the shard, the mode) is validated afresh: errors in a
    list that differs from a validated one in a single field are still caught
    before any HIP call."""
    numels = [5000, 70, 4099]
    esz = (2, 2, 4, 4, 4)
    offs = np.concatenate([[0], np.cumsum(numels)[:-1]])
    ptrs = [[FAKE + s * (1 << 36) + int(o) * esz[s] for o in offs] for s in range(5)]
    for _ in range(2):
        with pytest.raises(A.AdamWError) as e:          # valid: passes validation, then needs a GPU
            A.adamw_multi_tensor_step(A.MIXED, A.BF16, A.TensorList(numels, ptrs), A.HParams(), FAKE, stream=0)
        assert e.value.status in (A.E_HIP, A.E_NOMEM), e.value
    bad = [list(p) for p in ptrs]
    bad[2][1] += 2                                      # exp_avg of tensor 1 misaligned for fp32
    with pytest.raises(A.AdamWError, match="aligned"):
        A.adamw_multi_tensor_step(A.MIXED, A.BF16, A.TensorList(numels, bad), A.HParams(), FAKE, stream=0)
    with pytest.raises(A.AdamWError, match="shard"):
        A.adamw_multi_tensor_step(A.MIXED, A.BF16, A.TensorList(numels, ptrs, 0, sum(numels) + 1),
                                  A.HParams(), FAKE, stream=0)


def test_blocked_state_needs_aligned_buffer():
    numels = [100]
    ptrs = [[FAKE], [FAKE + (1 << 36)], [FAKE + 2 * (1 << 36) + 8], None, None]
    with pytest.raises(A.AdamWError, match="blocked"):
        A.adamw_multi_tensor_step(A.MIXED, A.BF16, A.TensorList(numels, ptrs, 0, -1, A.BLOCKED_STATE),
                                  A.HParams(), FAKE, stream=0)


def test_plan_beyond_the_grid_limit_is_rejected():
    """A launch's grid holds at most 2^32 - 1 lanes: with 8 workgroups of 256
    lanes per chunk a step plan may have at most 2,097,151 chunks.  One flat
    shard of exactly that many 16384-element chunks is counted without building
    the table and passes validation (then needs a GPU); one chunk more is
    rejected before any HIP call."""
    limit = (2 ** 32 - 1) // (8 * 256)
    for n_chunks, ok in ((limit, True), (limit + 1, False)):
        n = n_chunks * 16384
        ptrs = [[FAKE + s * (1 << 40)] for s in range(5)]
        tl = A.TensorList([n], ptrs, 0, -1, 0x1f)
        with pytest.raises(A.AdamWError) as e:
            A.adamw_multi_tensor_step(A.MIXED, A.BF16, tl, A.HParams(), FAKE, stream=0)
        if ok:
            assert e.value.status in (A.E_HIP, A.E_NOMEM), e.value
        else:
            assert e.value.status == A.E_INVALID and "chunks in one launch" in str(e.value), e.value


def test_many_tiny_tensors_count_one_chunk_each():
    """Tensors shorter than a pack run as one element chunk each, so the chunk
    count of a list of tiny tensors is its length (planner count = inspected rows)."""
    numels = [1, 3, 7, 2, 5] * 40
    offs = np.concatenate([[0], np.cumsum(numels)[:-1]])
    esz = (2, 2, 4, 4, 4)
    ptrs = [[FAKE + s * (1 << 36) + int(o) * esz[s] for o in offs] for s in range(5)]
    rows = A.adamw_plan_inspect(A.MIXED, A.BF16, A.TensorList(numels, ptrs))
    assert len(rows) == len(numels)
    assert all(r[3] == 0 for r in rows)
    assert [r[2] for r in rows] == numels


def test_single_launch_limit_knob():
    """The single-launch limit: any value >= 0 is taken as given, a negative one
    restores the default (4096 workgroups), and the call needs no GPU."""
    try:
        assert A.adamw_set_single_launch_max_workgroups(0) == 0
        assert A.adamw_set_single_launch_max_workgroups(123) == 123
        assert A.adamw_set_single_launch_max_workgroups(-1) == 4096
        assert A.adamw_set_single_launch_max_workgroups(-7) == 4096
    finally:
        A.adamw_set_single_launch_max_workgroups(-1)


def _plan_rows(mode, tl):
    """adamw_plan_inspect's rows as an (n, 6) int64 array (for plans of millions of chunks)."""
    lib = A._lib
    n = lib.adamw_plan_inspect(mode, A.BF16, ctypes.byref(tl.c), 0, None, 0)
    assert n >= 0, A.adamw_last_error()
    buf = (ctypes.c_int64 * (6 * max(n, 1)))()
    assert lib.adamw_plan_inspect(mode, A.BF16, ctypes.byref(tl.c), 0, buf, n) == n
    return np.frombuffer(buf, dtype=np.int64, count=6 * n).reshape(n, 6)


@pytest.mark.parametrize("mode", [A.MIXED, A.PURE_KAHAN])
@pytest.mark.parametrize("shard", [(0, -1), (2 ** 31 + 5, 2 ** 32 + 100), (2 ** 32 - 3, 2 ** 32 + 6157 + 40)])
def test_plan_beyond_32_bit_offsets(shard, mode):
    """One tensor longer than 2^32 elements (a ragged tail of 5 after the last
    pack) and a short one behind it: the plan covers the range exactly, with
    64-bit offsets inside the tensor, whole 16,384-element vector chunks between
    the peeled ends, and every row inside its tensor (the layout of the GPU test
    at this size: arenas with tensors at 128-element offsets)."""
    big = 2 ** 32 + 6157
    numels = [big, 1000]
    esz = (2, 2, 4, 4, 4) if mode == A.MIXED else (2, 2, 2, 2, 2)
    offs = [0, -(-big // 128) * 128]
    ptrs = [[FAKE + s * (1 << 40) + o * esz[s] for o in offs] for s in range(5)]
    total = sum(numels)
    b, e = shard[0], (total if shard[1] < 0 else shard[1])
    rows = _plan_rows(mode, A.TensorList(numels, ptrs, *shard))
    t, off, n, vec, flat, _ = rows.T
    starts = np.array([0, big], dtype=np.int64)
    assert flat[0] == b and np.array_equal(flat[1:], flat[:-1] + n[:-1]) and flat[-1] + n[-1] == e
    assert (n > 0).all() and np.array_equal(starts[t] + off, flat)
    assert (off + n <= np.array(numels, dtype=np.int64)[t]).all()
    assert off.max() > 2 ** 32 if e > 2 ** 32 else True
    v = vec == 1
    assert (n[v] % 8 == 0).all() and (n[v] <= 16384).all() and (n[~v] <= 4096).all()
    for s in range(5):
        base = np.array([ptrs[s][0], ptrs[s][1]], dtype=np.int64)
        assert ((base[t[v]] + off[v] * esz[s]) % 16 == 0).all()
    # inside the big tensor, only its peeled ends run element-wise
    big_rows = t == 0
    assert (~v[big_rows]).sum() <= 2 and (n[big_rows & v] == 16384).sum() >= (min(e, big) - b) // 16384 - 2


XCD_MAP_PROGRAM = r"""
#include <stdio.h>
#include <vector>
#include "layout.hpp"
// every grid size up to 20000 and a few large ones (the OPT-1.3B plan, the grid
// limit): each workgroup lands in [0, nb), every chunk is taken exactly once,
// and the workgroups of one XCD (b % 8) take one contiguous run in b order
static int check(uint32_t nb) {
    std::vector<unsigned char> seen(nb, 0);
    long last[8];
    for (int x = 0; x < 8; ++x) last[x] = -1;
    for (uint32_t b = 0; b < nb; ++b) {
        const uint32_t c = adamw::xcd_chunk(b, nb);
        if (c >= nb || seen[c]) return 1;
        seen[c] = 1;
        const int x = (int)(b & 7u);
        if (last[x] >= 0 && (long)c != last[x] + 1) return 2;
        last[x] = (long)c;
    }
    return 0;
}
// the lanes of an update chunk's parts take each of its packs exactly once
static int check_tiles(uint32_t block, uint32_t p) {
    const uint32_t packs = adamw::kXcdParts * block;
    std::vector<unsigned char> seen(packs, 0);
    for (uint32_t part = 0; part < (uint32_t)adamw::kXcdParts; ++part)
        for (uint32_t tid = 0; tid < block; ++tid) {
            const uint32_t k = adamw::tile_pack(tid, part, p);
            if (k >= packs || seen[k]) return 1;
            seen[k] = 1;
            // a tile of p packs lies with one part
            if ((k / p) % adamw::kXcdParts != part) return 2;
        }
    return 0;
}
int main() {
    const uint32_t shapes[][2] = {{(uint32_t)adamw::kBlockMixed, (uint32_t)adamw::kTilePacksMixed},
                                  {(uint32_t)adamw::kBlockMixed, (uint32_t)adamw::kTilePacks},
                                  {(uint32_t)adamw::kBlockPure, (uint32_t)adamw::kTilePacks},
                                  {256u, 1u}, {256u, 256u}, {128u, 16u}};
    for (auto& sp : shapes)
        if (int e = check_tiles(sp[0], sp[1])) { printf("tiles %u/%u err=%d\n", sp[0], sp[1], e); return 1; }
    for (uint32_t nb = 1; nb <= 20000; ++nb)
        if (int e = check(nb)) { printf("nb=%u err=%d\n", nb, e); return 1; }
    const uint32_t big[] = {642458u, 1283467u, 16777215u};
    for (uint32_t nb : big)
        if (int e = check(nb)) { printf("nb=%u err=%d\n", nb, e); return 1; }
    printf("ok\n");
    return 0;
}
"""


def test_xcd_chunk_map_is_a_bijection(tmp_path):
    """The overflow check's workgroup -> chunk map, and the update kernels'
    (part, lane) -> pack map inside a chunk (constexpr in layout.hpp, compiled
    here by the host compiler from the same header): each a bijection."""
    src = tmp_path / "xcd.cpp"
    src.write_text(XCD_MAP_PROGRAM)
    exe = tmp_path / "xcd"
    subprocess.run(["g++", "-std=c++17", "-O2", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                    "-I", os.path.join(ROOT, "adamw_optimizer_step_apply_amd", "csrc"), str(src), "-o", str(exe)],
                   check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0 and r.stdout.startswith("ok"), (r.returncode, r.stdout, r.stderr)


def test_precision_from_the_pages_optim_args():
    """The option string of the pages' pure-bf16 runs names the ADAMW_PURE_KAHAN
    precisions; other spellings map to the other instances, and bad entries are
    refused (no GPU: parsing only)."""
    import json
    hp = json.load(open(os.path.join(ROOT, "tests", "golden", "pages_recipe_hparams.json")))
    text = ", ".join(f"{k}={str(v).lower()}" for k, v in hp["optim_args"].items())
    assert A.PurePrecision.from_optim_args(text) == A.PurePrecision(A.BF16, A.BF16, A.KAHAN_BF16)
    assert A.PurePrecision.from_optim_args("momentum_dtype=float32, variance_dtype=bfloat16") == \
        A.PurePrecision(A.F32, A.BF16, A.KAHAN_NONE)
    assert A.PurePrecision.from_optim_args(
        "use_kahan_summation=True,compensation_buffer_dtype=torch.float32,variance_dtype=float32") == \
        A.PurePrecision(A.BF16, A.F32, A.KAHAN_F32)
    assert A.PurePrecision.from_optim_args("") == A.PurePrecision(A.BF16, A.BF16, A.KAHAN_NONE)
    for bad in ("momentum_dtype=float16", "use_kahan=true", "use_kahan_summation=maybe", "momentum_dtype"):
        with pytest.raises(ValueError):
            A.PurePrecision.from_optim_args(bad)
