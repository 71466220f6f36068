"""Pins for the CPU oracle: facts fixed by the pages, by the mathematics of
AdamW, or by independent library routines -- never by the oracle itself.

Every test here runs on the CPU.  Each pin is chosen so that a plausible slip in
the oracle (a dropped term, a swapped beta, eps in the wrong place, a wrong sign
in the compensation, an off-by-one in the shard walk, a wrong bit mask in the
overflow test) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import HParams

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
U = 2.0 ** -24  # unit roundoff of binary32


def ulp32(x):
    """Spacing of binary32 numbers at |x| (elementwise, as float64)."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    x = np.maximum(x, np.float64(np.finfo(np.float32).tiny))
    return np.exp2(np.floor(np.log2(x)) - 23)


def f32(x):
    return float(np.float32(x))


def bf16_bits(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_val(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------------------
# P1: 16-bit conversions vs library routines
# ---------------------------------------------------------------------------

def test_bf16_widen_exhaustive(olib):
    a = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.bf16_to_f32(a, olib)
    ref = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))


def test_f16_widen_exhaustive(olib):
    a = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.f16_to_f32(a, olib)
    ref = a.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours.view(np.uint32)[~nan], ref.view(np.uint32)[~nan])
    assert np.array_equal(np.signbit(ours[nan]), np.signbit(ref[nan]))


def _narrow_cases():
    rng = np.random.default_rng(1)
    raw = rng.integers(0, 2 ** 32, size=4_000_000, dtype=np.uint64).astype(np.uint32)
    spread = (rng.standard_normal(4_000_000) * np.exp2(rng.integers(-30, 18, 4_000_000))).astype(np.float32)
    # ties and near-ties for both formats, max finite, overflow edges, subnormals
    edge_bits = []
    for hi in rng.integers(0, 1 << 16, size=2000, dtype=np.uint32):
        for lo in (0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x1000, 0x0FFF, 0x2000):
            edge_bits.append((int(hi) << 16) | lo)
    edges = np.array(edge_bits, np.uint32).view(np.float32)
    special = np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 65536.0, -65520.0, 2.0 ** -24, 2.0 ** -25,
                        3 * 2.0 ** -26, 2.0 ** -14, 2.0 ** -14 - 2.0 ** -25, 2.0 ** -15, np.inf, -np.inf,
                        np.finfo(np.float32).max, np.finfo(np.float32).tiny, 1e-45, 3.3895313892515355e38],
                       np.float32)
    return np.concatenate([raw.view(np.float32), spread, edges, special])


def test_bf16_narrow_vs_torch(olib):
    x = _narrow_cases()
    ours = oracle.f32_to_bf16(x, olib)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.all((ours[nan] & 0x7F80) == 0x7F80) and np.all(ours[nan] & 0x007F)


def test_f16_narrow_vs_numpy(olib):
    x = _narrow_cases()
    ours = oracle.f32_to_f16(x, olib)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.all((ours[nan] & 0x7C00) == 0x7C00) and np.all(ours[nan] & 0x03FF)


# ---------------------------------------------------------------------------
# Per-launch scalars vs the library pow
# ---------------------------------------------------------------------------

def test_scalars_match_library_pow(olib):
    hp = HParams()
    lr, b1, b2, _, wd, _ = hp.f32()
    for t in list(range(1, 2001)) + [10_000, 123_457, 10 ** 6]:
        s = oracle.scalars(t, hp, olib)
        exp_ss = np.float32(lr / (1.0 - math.pow(b1, t)))
        exp_rb = np.float32(1.0 / (1.0 - math.pow(b2, t)))
        # fp64 pow and square-and-multiply agree to ~1e-16; after rounding to fp32
        # they may differ by one fp32 step only at a rounding boundary
        assert abs(s["step_size"] - exp_ss) <= ulp32(exp_ss)
        assert abs(s["rbc2"] - exp_rb) <= ulp32(exp_rb)
    s = oracle.scalars(10 ** 6, hp, olib)
    assert s["step_size"] == f32(2e-4) and s["rbc2"] == 1.0
    s = oracle.scalars(1, hp, olib)
    assert s["decay"] == f32(1.0 - f32(2e-4) * f32(0.1))
    assert s["omb1"] == f32(1.0 - f32(0.9)) and s["omb2"] == f32(1.0 - f32(0.95))


# ---------------------------------------------------------------------------
# P2: first step from zero moments -- closed form -lr * g / (|g| + eps)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("eps", [1e-8, 1e-3])
def test_step1_closed_form(olib, eps):
    """After bias correction, m_hat = g and sqrt(v_hat) = |g| exactly at t = 1,
    so the Adam direction is g / (|g| + eps) (~ sign(g) for |g| >> eps).  With
    w0 = 0 the decay term vanishes and w1 = -lr * g / (|g| + eps)."""
    rng = np.random.default_rng(2)
    n = 200_000
    g = bf16_bits(rng.standard_normal(n) * 1e-3)
    hp = HParams(eps=eps)
    p16 = np.zeros(n, np.uint16)
    master = np.zeros(n, np.float32)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    oracle.adamw_mixed(p16, g.copy(), master, m, v, hp, 1, lib=olib)
    gv = bf16_val(g).astype(np.float64)
    lr = hp.f32()[0]
    expect = -lr * gv / (np.abs(gv) + np.float64(np.float32(eps)))
    # about a dozen binary32 roundings feed the result; 16 u is a safe bound
    nz = gv != 0
    rel = np.abs(master[nz] - expect[nz]) / np.abs(expect[nz])
    assert rel.max() <= 16 * U, rel.max()
    assert np.all(master[~nz] == 0)
    if eps == 1e-8:
        # the pages' reading of "update ~ lr * sign(g)": within 1e-4 of lr for |g| > 1e-4
        big = np.abs(gv) > 1e-4
        assert np.allclose(master[big], -lr * np.sign(gv[big]), rtol=1e-4, atol=0)
    # p16 is the master rounded to bf16
    assert np.array_equal(p16, bf16_bits(master))


def test_step1_decay_only_from_nonzero_weight(olib):
    """With g = 0 the first step is the pure decoupled decay w * (1 - lr*wd)."""
    rng = np.random.default_rng(3)
    n = 100_000
    w0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    hp = HParams(lr=1e-2, weight_decay=0.5)
    master = w0.copy()
    z = np.zeros(n, np.float32)
    oracle.adamw_mixed(np.zeros(n, np.uint16), np.zeros(n, np.uint16), master, z.copy(), z.copy(), hp, 1,
                       lib=olib)
    lr, wd = hp.f32()[0], hp.f32()[4]
    expect = w0.astype(np.float64) * (1.0 - lr * wd)
    # one rounding of the decay factor (<= u) and one of the product (<= u/2)
    assert np.all(np.abs(master - expect) <= 1.5 * U * np.abs(expect) + 1e-45)


# ---------------------------------------------------------------------------
# P3: constant gradient -- m_hat = g, v_hat = g^2 at every step
# ---------------------------------------------------------------------------

def test_constant_gradient_closed_form(olib):
    """With a constant gradient the bias-corrected moments equal g and g^2 at
    every t, so every step moves w by -lr * g/(|g| + eps) after the decay:
    w_k = w0 D^k - lr u (1 - D^k)/(1 - D), D = 1 - lr*wd (geometric series)."""
    rng = np.random.default_rng(4)
    n, k = 20_000, 50
    g = bf16_bits(rng.standard_normal(n) * 1e-3)
    w0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    hp = HParams()
    lr, _, _, eps, wd, _ = hp.f32()
    master, m, v = w0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    p16 = np.zeros(n, np.uint16)
    for t in range(1, k + 1):
        oracle.adamw_mixed(p16, g, master, m, v, hp, t, lib=olib)
    gv = bf16_val(g).astype(np.float64)
    u = gv / (np.abs(gv) + eps)
    D = 1.0 - lr * wd
    expect = w0 * D ** k - lr * u * (1 - D ** k) / (1 - D)
    # per step: the decay factor's own rounding (u relative), two roundings of
    # the weight (u/2 each, relative to |w|) and ~16 u relative on the lr*u term
    mag = np.abs(w0) + k * lr
    tol = k * (2.5 * U * mag + 16 * U * lr)
    assert np.all(np.abs(master - expect) <= tol)
    # the moments themselves track g (1 - beta^t) and g^2 (1 - beta^t)
    b1, b2 = hp.f32()[1], hp.f32()[2]
    assert np.allclose(m, gv * (1 - b1 ** k), rtol=k * 4 * U, atol=0)
    assert np.allclose(v, gv * gv * (1 - b2 ** k), rtol=k * 6 * U, atol=0)


# ---------------------------------------------------------------------------
# P4: zero gradient -- moments stay 0, weights decay geometrically
# ---------------------------------------------------------------------------

def test_zero_gradient_mixed_decay(olib):
    rng = np.random.default_rng(5)
    n, k = 50_000, 1000
    w0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    hp = HParams()
    master, m, v = w0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    z16 = np.zeros(n, np.uint16)
    p16 = np.zeros(n, np.uint16)
    for t in range(1, k + 1):
        oracle.adamw_mixed(p16, z16, master, m, v, hp, t, lib=olib)
    assert np.all(m == 0) and np.all(v == 0)
    lr, wd = hp.f32()[0], hp.f32()[4]
    dec32 = float(np.float32(1.0 - lr * wd))
    exact = w0.astype(np.float64) * (1.0 - lr * wd) ** k
    with_f32_factor = w0.astype(np.float64) * dec32 ** k
    # k roundings of the product, each <= u/2 relative
    assert np.all(np.abs(master - with_f32_factor) <= k * 0.5 * U * np.abs(with_f32_factor) * 1.001)
    # and the fp32 factor is within u of 1 - lr*wd
    assert np.all(np.abs(master - exact) <= k * 1.5 * U * np.abs(exact) * 1.001)
    assert np.array_equal(p16, bf16_bits(master))


def test_zero_gradient_kahan_tracks_decay(olib):
    """1000 steps of pure decay with lr*wd = 2e-5, far below bf16's half-ulp
    (2^-9 relative): without compensation the bf16 weight never moves; with the
    compensation buffer p + c follows w0 (1 - lr*wd)^k (a 2% total decay)."""
    rng = np.random.default_rng(6)
    n, k = 100_000, 1000
    p0 = bf16_bits(rng.standard_normal(n) * 0.02)
    hp = HParams()
    p, m, v, c = p0.copy(), np.zeros(n, np.uint16), np.zeros(n, np.uint16), np.zeros(n, np.uint16)
    pn, mn, vn = p0.copy(), np.zeros(n, np.uint16), np.zeros(n, np.uint16)
    z = np.zeros(n, np.uint16)
    for t in range(1, k + 1):
        oracle.adamw_kahan(p, z, m, v, c, hp, t, lib=olib)
        oracle.adamw_bf16_naive(pn, z, mn, vn, hp, t, lib=olib)
    lr, wd = hp.f32()[0], hp.f32()[4]
    truth = bf16_val(p0).astype(np.float64) * (1.0 - lr * wd) ** k
    got = bf16_val(p).astype(np.float64) + bf16_val(c).astype(np.float64)
    nz = truth != 0
    rel = np.abs(got[nz] - truth[nz]) / np.abs(truth[nz])
    assert np.median(rel) <= 2e-3 and rel.max() <= 5e-3, (np.median(rel), rel.max())
    assert np.array_equal(pn, p0)                 # naive bf16 never moves
    assert np.all(m == 0) and np.all(v == 0)


# ---------------------------------------------------------------------------
# P5: beta1 = beta2 = 0 -- history-free signSGD with decoupled decay
# ---------------------------------------------------------------------------

def test_beta_zero_is_decayed_sign_sgd(olib):
    rng = np.random.default_rng(7)
    n, k = 20_000, 20
    hp = HParams(beta1=0.0, beta2=0.0, lr=1e-3, weight_decay=0.1)
    lr, _, _, eps, wd, _ = hp.f32()
    w0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    master, m, v, p16 = w0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.uint16)
    ref = w0.astype(np.float64)
    err_budget = np.zeros(n)
    for t in range(1, k + 1):
        g = bf16_bits(rng.standard_normal(n) * 1e-3)
        oracle.adamw_mixed(p16, g, master, m, v, hp, t, lib=olib)
        gv = bf16_val(g).astype(np.float64)
        ref = ref * (1 - lr * wd) - lr * gv / (np.abs(gv) + eps)
        err_budget += 2.5 * U * (np.abs(ref) + lr) + 16 * U * lr
        assert np.all(np.abs(master - ref) <= err_budget)
        assert np.array_equal(m, bf16_val(g))     # m = g exactly when beta1 = 0


# ---------------------------------------------------------------------------
# P6: special cases that reduce to torch.optim.AdamW (an independent library)
# ---------------------------------------------------------------------------

def _torch_adamw(w0, grads, hp, dtype):
    lr, b1, b2, eps, wd, _ = hp.f32()
    p = torch.nn.Parameter(torch.from_numpy(w0.astype(np.float64)).to(dtype))
    opt = torch.optim.AdamW([p], lr=lr, betas=(b1, b2), eps=eps, weight_decay=wd, foreach=False)
    for g in grads:
        p.grad = torch.from_numpy(g.astype(np.float64)).to(dtype)
        opt.step()
    st = opt.state[p]
    return (p.detach().double().numpy(), st["exp_avg"].double().numpy(), st["exp_avg_sq"].double().numpy())


@pytest.mark.parametrize("hp", [HParams(), HParams(lr=1e-2, weight_decay=0.5, eps=1e-4),
                                HParams(lr=5e-3, beta1=0.5, beta2=0.75, weight_decay=0.0, eps=1e-3)],
                         ids=["recipe", "strong-decay", "other-betas"])
def test_mixed_matches_torch_adamw_fp64(olib, hp):
    """torch.optim.AdamW in float64 is the same algorithm (decoupled decay
    applied to the pre-step weight, bias-corrected moments, eps outside the
    square root).  Our binary32 result must stay within the rounding budget of
    binary32 arithmetic, checked per element."""
    rng = np.random.default_rng(8)
    n, k = 20_000, 10
    w0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    grads = [bf16_val(bf16_bits(rng.standard_normal(n) * 1e-3)) for _ in range(k)]
    master, m, v, p16 = w0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.uint16)
    for t, g in enumerate(grads, 1):
        oracle.adamw_mixed(p16, bf16_bits(g), master, m, v, hp, t, lib=olib)
    tw, tm, tv = _torch_adamw(w0, grads, hp, torch.float64)
    lr = hp.f32()[0]
    gmax = np.max(np.abs(np.stack(grads)), axis=0).astype(np.float64)
    mag = np.abs(w0) + 2 * k * lr
    assert np.all(np.abs(master - tw) <= k * (2.5 * U * mag + 32 * U * lr))
    assert np.all(np.abs(m - tm) <= k * 3 * U * gmax)
    assert np.all(np.abs(v - tv) <= k * 4 * U * gmax * gmax)


def test_mixed_close_to_torch_adamw_fp32(olib):
    """torch's own binary32 AdamW evaluates in a different order; expect a few ulp."""
    rng = np.random.default_rng(9)
    n, k = 20_000, 10
    hp = HParams()
    w0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    grads = [bf16_val(bf16_bits(rng.standard_normal(n) * 1e-3)) for _ in range(k)]
    master, m, v, p16 = w0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.uint16)
    for t, g in enumerate(grads, 1):
        oracle.adamw_mixed(p16, bf16_bits(g), master, m, v, hp, t, lib=olib)
    tw, _, _ = _torch_adamw(w0, grads, hp, torch.float32)
    assert np.all(np.abs(master - tw) <= 8 * k * ulp32(np.abs(w0) + 2 * k * 2e-4))


def test_lr_zero_wd_zero_leaves_weights(olib):
    rng = np.random.default_rng(10)
    n = 10_000
    w0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    hp = HParams(lr=0.0, weight_decay=0.0)
    master, m, v, p16 = w0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.uint16)
    for t in range(1, 4):
        oracle.adamw_mixed(p16, bf16_bits(rng.standard_normal(n) * 1e-3), master, m, v, hp, t, lib=olib)
    assert np.array_equal(master, w0)
    pk, ck = bf16_bits(w0), np.zeros(n, np.uint16)
    p0 = pk.copy()
    mk, vk = np.zeros(n, np.uint16), np.zeros(n, np.uint16)
    for t in range(1, 4):
        oracle.adamw_kahan(pk, bf16_bits(rng.standard_normal(n) * 1e-3), mk, vk, ck, hp, t, lib=olib)
    assert np.array_equal(pk, p0) and np.all(bf16_val(ck) == 0)


# ---------------------------------------------------------------------------
# P7: Kahan compensation tracks an fp64 accumulation of tiny updates
# ---------------------------------------------------------------------------

def test_kahan_tracks_constant_tiny_updates(olib):
    """p0 = 1, 10,000 updates of +1e-4 (below bf16's half-ulp 2^-8 at 1.0):
    the fp64 sum reaches 2.0; naive bf16 stays at 1.0; p + c must be within 5%.

    The update is produced by the optimizer itself: wd = 0, eps = 0 and a
    constant gradient g = -1 give u = -1 (to a few ulp), so d = +lr."""
    n, k = 64, 10_000
    hp = HParams(lr=1e-4, weight_decay=0.0, eps=0.0)
    one = bf16_bits(np.ones(n))
    g = bf16_bits(-np.ones(n))
    p, m, v, c = one.copy(), np.zeros(n, np.uint16), np.zeros(n, np.uint16), np.zeros(n, np.uint16)
    pn, mn, vn = one.copy(), np.zeros(n, np.uint16), np.zeros(n, np.uint16)
    for t in range(1, k + 1):
        oracle.adamw_kahan(p, g, m, v, c, hp, t, lib=olib)
        oracle.adamw_bf16_naive(pn, g, mn, vn, hp, t, lib=olib)
    got = bf16_val(p).astype(np.float64) + bf16_val(c)
    assert np.all(np.abs(got - 2.0) <= 0.05 * 2.0), got[:4]
    assert np.all(bf16_val(pn) == 1.0)


def test_kahan_tracks_random_tiny_updates(olib):
    """Independent random-signed updates of about 1e-4 per step, 10,000 steps
    from p0 = 1.  With beta1 = beta2 = 0, eps = 1 and wd = 0 the direction is
    u = g / (|g| + 1) (~ g for small g), so g ~ N(0, 1e-2), lr = 1e-2 gives every
    element its own delta of ~N(0, 1e-4) per step.

    Expected errors.  Naive bf16 cannot move (|d| << half an ulp of 1.0), so its
    error is the whole walk, RMS ~ 1e-4 * sqrt(1e4) = 1e-2.  Kahan's only loss
    is the bf16 rounding of c each step: |c| < 2^-8, rounding error uniform in
    half an ulp of c, RMS ~ 3.3e-6 per step, so ~ 3.3e-4 after 1e4 steps, a
    ratio near 30.  Require 10x, with 1024 independent elements."""
    rng = np.random.default_rng(11)
    n, k = 1024, 10_000
    hp = HParams(lr=1e-2, beta1=0.0, beta2=0.0, eps=1.0, weight_decay=0.0)
    lr = hp.f32()[0]
    one = bf16_bits(np.ones(n))
    p, m, v, c = one.copy(), np.zeros(n, np.uint16), np.zeros(n, np.uint16), np.zeros(n, np.uint16)
    pn, mn, vn = one.copy(), np.zeros(n, np.uint16), np.zeros(n, np.uint16)
    truth = np.ones(n)
    for t in range(1, k + 1):
        g = bf16_bits(rng.standard_normal(n) * 1e-2)
        oracle.adamw_kahan(p, g, m, v, c, hp, t, lib=olib)
        oracle.adamw_bf16_naive(pn, g, mn, vn, hp, t, lib=olib)
        gv = bf16_val(g).astype(np.float64)
        truth -= lr * gv / (np.abs(gv) + 1.0)
    kahan_rms = np.sqrt(np.mean((bf16_val(p) + bf16_val(c).astype(np.float64) - truth) ** 2))
    naive_rms = np.sqrt(np.mean((bf16_val(pn) - truth) ** 2))
    assert np.array_equal(pn, one)
    assert kahan_rms * 10 <= naive_rms, (kahan_rms, naive_rms)
    assert kahan_rms <= 1e-3


def test_kahan_step1_agrees_with_mixed(olib):
    """From the same state (master = the bf16 weight, zero moments) one Kahan
    step and one mixed step compute the same fp32 moments, so the stored bf16
    moments are the mixed ones rounded, and p + c equals the mixed master up to
    the rounding of c (half a bf16 ulp of c) and the fp32 roundings."""
    rng = np.random.default_rng(12)
    n = 100_000
    p0 = bf16_bits(rng.standard_normal(n) * 0.02)
    g = bf16_bits(rng.standard_normal(n) * 1e-3)
    hp = HParams()
    master = bf16_val(p0).copy()
    mm, vm, p16 = np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.uint16)
    oracle.adamw_mixed(p16, g, master, mm, vm, hp, 1, lib=olib)
    pk, mk, vk, ck = p0.copy(), np.zeros(n, np.uint16), np.zeros(n, np.uint16), np.zeros(n, np.uint16)
    oracle.adamw_kahan(pk, g, mk, vk, ck, hp, 1, lib=olib)
    assert np.array_equal(mk, bf16_bits(mm)) and np.array_equal(vk, bf16_bits(vm))
    got = bf16_val(pk).astype(np.float64) + bf16_val(ck)
    # the fp32 roundings are relative to the operands (|p0| and the step ~lr), not to
    # the result, which can cancel to near zero
    tol = (np.exp2(np.floor(np.log2(np.maximum(np.abs(bf16_val(ck)), 1e-38))) - 8)
           + 4 * ulp32(np.abs(bf16_val(p0)) + hp.f32()[0]))
    assert np.all(np.abs(got - master) <= tol)


# ---------------------------------------------------------------------------
# fp16 AMP: scaled fp16 gradients give the same fp32 step as the unscaled bf16 ones
# ---------------------------------------------------------------------------

def test_f16_scaled_equals_bf16_unscaled(olib):
    """A bf16 gradient times 2^16 is exact in fp16 (8 significant bits, in range),
    and multiplying by 2^-16 undoes it exactly; so the fp16-AMP step with loss
    scale 65536 must give bit-identical master/m/v to the bf16 step."""
    rng = np.random.default_rng(13)
    n, k = 50_000, 5
    w0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    s_b = [w0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)]
    s_h = [w0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)]
    pb, ph = np.zeros(n, np.uint16), np.zeros(n, np.uint16)
    hb = HParams()
    hh = HParams(inv_scale=1.0 / 65536)
    for t in range(1, k + 1):
        gb = bf16_bits(rng.standard_normal(n) * 1e-3)
        gh = (bf16_val(gb) * np.float32(65536)).astype(np.float16).view(np.uint16)
        assert np.array_equal(gh.view(np.float16).astype(np.float32) / 65536, bf16_val(gb))
        oracle.adamw_mixed(pb, gb, *s_b, hb, t, p_is_f16=False, lib=olib)
        oracle.adamw_mixed(ph, gh, *s_h, hh, t, p_is_f16=True, lib=olib)
    for a, b in zip(s_b, s_h):
        assert np.array_equal(a, b)
    assert np.array_equal(ph, s_h[0].astype(np.float16).view(np.uint16))


# ---------------------------------------------------------------------------
# P9: the overflow skip
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("bad", [0x7C00, 0xFC00, 0x7E00, 0x7C01, 0xFFFF])
def test_skip_on_nonfinite_f16(olib, bad):
    rng = np.random.default_rng(14)
    sizes = [5, 1000, 1, 333]
    tensors = []
    for n in sizes:
        w = (rng.standard_normal(n) * 0.02).astype(np.float32)
        g = (rng.standard_normal(n) * 65.536).astype(np.float16).view(np.uint16)
        tensors.append(dict(p=w.astype(np.float16).view(np.uint16), g=g, master=w,
                            m=np.zeros(n, np.float32), v=np.zeros(n, np.float32)))
    tensors[2]["g"][0] = bad
    before = [{k: a.copy() for k, a in tt.items()} for tt in tensors]
    step = oracle.step_list("mixed", tensors, HParams(inv_scale=1 / 65536), 7, p_is_f16=True,
                            check_overflow=True, lib=olib)
    assert step == 7
    for tt, bb in zip(tensors, before):
        for k in tt:
            assert np.array_equal(tt[k], bb[k])
    # the largest finite values do not trip it
    tensors[2]["g"][0] = 0x7BFF
    assert oracle.step_list("mixed", tensors, HParams(inv_scale=1 / 65536), 7, p_is_f16=True,
                            check_overflow=True, lib=olib) == 8
    assert not np.array_equal(tensors[1]["master"], before[1]["master"])


def test_nonfinite_masks_exhaustive(olib):
    a = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f16 = a.view(np.float16).astype(np.float32)
    bf = bf16_val(a)
    for i in range(0, 65536, 4096):
        blk = a[i:i + 4096]
        assert oracle.any_nonfinite(blk, True, olib) == bool(np.any(~np.isfinite(f16[i:i + 4096])))
        assert oracle.any_nonfinite(blk, False, olib) == bool(np.any(~np.isfinite(bf[i:i + 4096])))
    for x in a:
        if not np.isfinite(f16[x]):
            assert oracle.any_nonfinite(np.array([x], np.uint16), True, olib)
        if not np.isfinite(bf[x]):
            assert oracle.any_nonfinite(np.array([x], np.uint16), False, olib)
    fin16 = a[np.isfinite(f16)]
    finb = a[np.isfinite(bf)]
    assert not oracle.any_nonfinite(fin16, True, olib)
    assert not oracle.any_nonfinite(finb, False, olib)


# ---------------------------------------------------------------------------
# P10: shard walk and the shard-union invariant
# ---------------------------------------------------------------------------

def test_shard_pieces_brute_force():
    rng = np.random.default_rng(15)
    for _ in range(300):
        numels = list(rng.integers(0, 9, size=rng.integers(1, 8)))
        total = int(sum(numels))
        b = int(rng.integers(0, total + 1))
        e = int(rng.integers(b, total + 1))
        owner = np.concatenate([np.full(n, i) for i, n in enumerate(numels)] + [np.zeros(0)]).astype(int)
        local = np.concatenate([np.arange(n) for n in numels] + [np.zeros(0)]).astype(int)
        got = []
        for i, lo, hi, flo in oracle.shard_pieces(numels, b, e):
            assert owner[flo] == i and local[flo] == lo
            got += [(i, j) for j in range(lo, hi)]
        assert got == [(owner[f], local[f]) for f in range(b, e)]


def test_shard_pieces_padded_flat_index_brute_force():
    """The padded flat index: each tensor's elements followed by empty slots up
    to the next multiple of 8, written out one slot at a time."""
    rng = np.random.default_rng(16)
    for _ in range(300):
        numels = list(rng.integers(0, 20, size=rng.integers(1, 8)))
        slots = []                      # (tensor, element) or None for a gap
        for i, n in enumerate(numels):
            slots += [(i, j) for j in range(n)]
            while len(slots) % 8:
                slots.append(None)
        total = len(slots)
        b = int(rng.integers(0, total + 1))
        e = int(rng.integers(b, total + 1))
        got = []
        for i, lo, hi, flo in oracle.shard_pieces(numels, b, e, flat_align=8):
            assert slots[flo] == (i, lo)
            got += [(i, j) for j in range(lo, hi)]
        assert got == [sl for sl in slots[b:e] if sl is not None]


def test_shard_union_equals_full_step(olib):
    """The single-GPU form of the pages' ZeRO on/off comparison (same losses in
    the A40/A100 tables): four rank shards stepped one after another equal one
    full-list step, bit for bit."""
    numels = [37, 1, 4096, 513, 7, 2048, 999]
    def fresh():
        r = np.random.default_rng(17)
        ts = []
        for n in numels:
            w = (r.standard_normal(n) * 0.02).astype(np.float32)
            ts.append(dict(p=bf16_bits(w), g=bf16_bits(r.standard_normal(n) * 1e-3), master=w,
                           m=np.zeros(n, np.float32), v=np.zeros(n, np.float32)))
        return ts
    full, parts = fresh(), fresh()
    oracle.step_list("mixed", full, HParams(), 0, lib=olib)
    total = sum(numels)
    for r in range(4):
        b, e = r * total // 4, (r + 1) * total // 4
        assert oracle.step_list("mixed", parts, HParams(), 0, shard_begin=b, shard_end=e, lib=olib) == 1
    for a, b in zip(full, parts):
        for k in a:
            assert np.array_equal(a[k], b[k])


# ---------------------------------------------------------------------------
# P13: learning-rate schedule of the opt-125m run
# ---------------------------------------------------------------------------

def test_warmup_schedule():
    hp = json.load(open(os.path.join(GOLDEN, "pages_recipe_hparams.json")))
    base, warm = hp["learning_rate"], hp["warmup_steps"]
    assert oracle.warmup_linear_lr(1, base, warm) == f32(4e-7)
    assert oracle.warmup_linear_lr(100, base, warm) == f32(4e-5)
    assert oracle.warmup_linear_lr(250, base, warm) == f32(1e-4)
    assert oracle.warmup_linear_lr(500, base, warm) == f32(2e-4)
    assert oracle.warmup_linear_lr(501, base, warm) == f32(2e-4)


def test_recipe_defaults():
    hp = json.load(open(os.path.join(GOLDEN, "pages_recipe_hparams.json")))
    d = HParams()
    assert (d.lr, d.beta1, d.beta2, d.weight_decay) == (hp["learning_rate"], hp["adam_beta1"],
                                                        hp["adam_beta2"], hp["weight_decay"])
    assert hp["optim_args"]["momentum_dtype"] == hp["optim_args"]["compensation_buffer_dtype"] == "bfloat16"


# ---------------------------------------------------------------------------
# Split master (16-bit param + 16-bit remainder)
# ---------------------------------------------------------------------------

def _pattern_sweep(n_random=1 << 22):
    rng = np.random.default_rng(21)
    stride = np.arange(0, 1 << 32, 4099, dtype=np.uint64).astype(np.uint32)     # ~1M patterns over the whole space
    rnd = rng.integers(0, 1 << 32, size=n_random, dtype=np.uint64).astype(np.uint32)
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF], np.uint32)
    his = rng.integers(0, 1 << 16, size=20000, dtype=np.uint64).astype(np.uint32)
    edges = ((his[:, None] << 16) | lows[None, :]).reshape(-1)
    special = np.array([0x7F7FFFFF, 0xFF7FFFFF, 0x7F800000, 0xFF800000, 0x00000000, 0x80000000,
                        0x00008000, 0x80008000, 0x0000FFFF, 0x7F7F8000], np.uint32)
    return np.concatenate([stride, rnd, edges, special])


def test_split_join_roundtrip(olib):
    """join(split(w)) == w bit for bit for every non-NaN pattern tried (a stride
    through all 2^32 patterns, 4M random ones, and every rounding boundary), and a
    NaN master joins back to a NaN."""
    w = _pattern_sweep()
    p, r = oracle.split_make(w, olib)
    back = oracle.split_join(p, r, olib).view(np.uint32)
    nan = np.isnan(w.view(np.float32))
    assert np.array_equal(back[~nan], w[~nan])
    assert np.all(np.isnan(back[nan].view(np.float32)))


def test_split_param_is_a_nearest_bf16(olib):
    """The bf16 half is a nearest bf16 to the master: it equals torch's
    round-to-nearest-even except on exact ties, where it is the one of larger
    magnitude; the remainder always fits in int16."""
    w = _pattern_sweep()
    w = w[np.isfinite(w.view(np.float32))]
    p, r = oracle.split_make(w, olib)
    rne = bf16_bits(w.view(np.float32))
    tie = (w & 0xFFFF) == 0x8000
    assert np.array_equal(p[~tie], rne[~tie])
    assert np.array_equal(p[tie].astype(np.uint32), (w[tie] >> 16) + 1)
    rem = r.view(np.int16).astype(np.int64)
    assert np.array_equal((p.astype(np.int64) << 16) + rem, w.astype(np.int64))


@pytest.mark.parametrize("hp", [HParams(), HParams(lr=1e-2, weight_decay=0.5, eps=1e-4)], ids=["recipe", "strong"])
def test_split_step_equals_mixed_step(olib, hp):
    """The split master is an exact encoding of the fp32 master, so k split steps
    leave join(p, r) bit-identical to k mixed steps from the same master, with the
    same moments, and p is the split of that master."""
    rng = np.random.default_rng(22)
    n, k = 50_000, 8
    w0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    w0[:64] = np.array([0x3C808000 + i for i in range(64)], np.uint32).view(np.float32)   # ties
    master, mm, vm, p16 = w0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.uint16)
    ps, rs = oracle.split_make(w0, olib)
    ms, vs = np.zeros(n, np.float32), np.zeros(n, np.float32)
    for t in range(1, k + 1):
        g = bf16_bits(rng.standard_normal(n) * 1e-3)
        oracle.adamw_mixed(p16, g, master, mm, vm, hp, t, lib=olib)
        oracle.adamw_mixed_split(ps, g, rs, ms, vs, hp, t, lib=olib)
    assert np.array_equal(oracle.split_join(ps, rs, olib).view(np.uint32), master.view(np.uint32))
    assert np.array_equal(ms, mm) and np.array_equal(vs, vm)
    pe, _ = oracle.split_make(master, olib)
    assert np.array_equal(ps, pe)


# ---------------------------------------------------------------------------
# Dynamic loss scaling (fp16 AMP)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("growth,backoff,interval,scale0", [
    (2.0, 0.5, 3, 65536.0), (2.0, 0.5, 1, 1.0), (1.5, 0.25, 4, 1000.0), (2.0, 0.5, 2, 3e38),
    (2.0, 0.5, 5, 1e-30), (1.0, 1.0, 3, 7.0)])
def test_loss_scale_rule_matches_torch(olib, growth, backoff, interval, scale0):
    """The scale/tracker trajectory over a random overflow pattern equals torch's
    own loss-scale update (torch._amp_update_scale_, the op behind GradScaler.update),
    including the growth that would overflow fp32 and is refused."""
    rng = np.random.default_rng(31)
    flags = (rng.random(300) < 0.15).astype(int)
    ls = oracle.LossScale(scale=scale0, tracker=0, growth=growth, backoff=backoff, interval=interval)
    ts = torch.tensor([scale0], dtype=torch.float32)
    tt = torch.tensor([0], dtype=torch.int32)
    for f in flags:
        ls.update(bool(f), olib)
        torch._amp_update_scale_(ts, tt, torch.tensor([float(f)]), growth, backoff, interval)
        assert np.float32(ls.scale) == np.float32(ts.item()) and ls.tracker == int(tt.item())


def test_inv_scale(olib):
    ls = oracle.LossScale()
    for e in range(-20, 40):
        ls.scale = float(2.0 ** e)
        assert ls.inv(olib) == 2.0 ** -e
    for x in (3.0, 1000.0, 12345.678):
        ls.scale = float(np.float32(x))
        assert ls.inv(olib) == float(np.float32(1.0 / np.float64(np.float32(x))))


def test_amp_step_skips_and_backs_off(olib):
    """An overflow leaves every buffer and the counter unchanged and halves the
    scale; clean steps unscale by 1/scale, i.e. act like the bf16-equivalent step."""
    rng = np.random.default_rng(32)
    n = 4000
    w = (rng.standard_normal(n) * 0.02).astype(np.float32)
    g = (rng.standard_normal(n) * 65.536).astype(np.float16).view(np.uint16)
    t = [dict(p=w.astype(np.float16).view(np.uint16), g=g.copy(), master=w.copy(),
              m=np.zeros(n, np.float32), v=np.zeros(n, np.float32))]
    ref = [{k: a.copy() for k, a in t[0].items()}]
    ls = oracle.LossScale(scale=65536.0, interval=2)
    step = oracle.amp_step_list("mixed", t, HParams(), 0, ls, lib=olib)
    assert step == 1 and ls.scale == 65536.0 and ls.tracker == 1
    oracle.step_list("mixed", ref, HParams(inv_scale=1 / 65536), 0, p_is_f16=True, lib=olib)
    for k in t[0]:
        assert np.array_equal(t[0][k], ref[0][k])
    t[0]["g"][17] = 0x7C00
    before = {k: a.copy() for k, a in t[0].items()}
    step = oracle.amp_step_list("mixed", t, HParams(), step, ls, lib=olib)
    assert step == 1 and ls.scale == 32768.0 and ls.tracker == 0
    for k in t[0]:
        assert np.array_equal(t[0][k], before[k])


# ---------------------------------------------------------------------------
# AnyPrecision state dtypes (pure bf16 params)
# ---------------------------------------------------------------------------

def _pure_state(n, rng, m32, v32, kahan):
    p = bf16_bits(rng.standard_normal(n) * 0.02)
    m = np.zeros(n, np.float32) if m32 else np.zeros(n, np.uint16)
    v = np.zeros(n, np.float32) if v32 else np.zeros(n, np.uint16)
    c = np.zeros(n, np.uint16) if kahan else None
    return p, m, v, c


def test_pure_bf16_state_reduces_to_kahan_and_naive(olib):
    """bf16 moments with compensation is the Kahan step; without it, the naive bf16 step."""
    rng = np.random.default_rng(41)
    n = 30_000
    for kahan in (True, False):
        p, m, v, c = _pure_state(n, rng, False, False, kahan)
        p2, m2, v2, c2 = p.copy(), m.copy(), v.copy(), None if c is None else c.copy()
        for t in range(1, 6):
            g = bf16_bits(rng.standard_normal(n) * 1e-3)
            oracle.adamw_pure(p, g, m, v, c, HParams(), t, lib=olib)
            if kahan:
                oracle.adamw_kahan(p2, g, m2, v2, c2, HParams(), t, lib=olib)
            else:
                oracle.adamw_bf16_naive(p2, g, m2, v2, HParams(), t, lib=olib)
        assert np.array_equal(p, p2) and np.array_equal(m, m2) and np.array_equal(v, v2)
        if kahan:
            assert np.array_equal(c, c2)


@pytest.mark.parametrize("m32,v32", [(True, True), (True, False), (False, True)])
def test_pure_fp32_moments_follow_the_mixed_moments(olib, m32, v32):
    """fp32 moments evolve exactly as the pinned mixed oracle's (the moment update
    does not read the weight); bf16 ones are its fp32 values rounded at step 1.
    Without compensation the new param is the rounding of the mixed step's
    master when that master starts at the bf16 param."""
    rng = np.random.default_rng(42)
    n = 30_000
    p, m, v, _ = _pure_state(n, rng, m32, v32, False)
    w = bf16_val(p).copy()
    mm, vm, p16 = np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.uint16)
    g = bf16_bits(rng.standard_normal(n) * 1e-3)
    oracle.adamw_pure(p, g, m, v, None, HParams(), 1, lib=olib)
    oracle.adamw_mixed(p16, g, w, mm, vm, HParams(), 1, lib=olib)
    assert np.array_equal(p, p16)
    assert np.array_equal(m, mm) if m32 else np.array_equal(m, bf16_bits(mm))
    assert np.array_equal(v, vm) if v32 else np.array_equal(v, bf16_bits(vm))
    if m32 and v32:
        for t in range(2, 8):
            g = bf16_bits(rng.standard_normal(n) * 1e-3)
            oracle.adamw_pure(p, g, m, v, None, HParams(), t, lib=olib)
            w = bf16_val(p).copy()        # the mixed master restarted from the bf16 param
            oracle.adamw_mixed(p16, g, w, mm, vm, HParams(), t, lib=olib)
        assert np.array_equal(m, mm) and np.array_equal(v, vm)


def test_pure_fp32_moments_kahan_tracks_tiny_updates(olib):
    """Compensation with fp32 moments: 10,000 constant +1e-4 updates from 1.0 land
    within 5% of the fp64 sum (naive bf16 stays at 1.0)."""
    n, k = 64, 10_000
    hp = HParams(lr=1e-4, weight_decay=0.0, eps=0.0)
    p = bf16_bits(np.ones(n))
    m, v, c = np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.uint16)
    pn, mn, vn = p.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    g = bf16_bits(-np.ones(n))
    for t in range(1, k + 1):
        oracle.adamw_pure(p, g, m, v, c, hp, t, lib=olib)
        oracle.adamw_pure(pn, g, mn, vn, None, hp, t, lib=olib)
    got = bf16_val(p).astype(np.float64) + bf16_val(c)
    assert np.all(np.abs(got - 2.0) <= 0.1) and np.all(bf16_val(pn) == 1.0)


def test_pure_fp32_compensation_tracks_tiny_updates_closely(olib):
    """An fp32 compensation buffer (compensation_buffer_dtype=float32): 10,000
    constant +1e-4 updates from 1.0 bring p + c within 1e-5 of the fp64 sum 2.0
    (a bf16 buffer only gets within 5 %: it rounds each residual to 8 bits), and p
    itself reaches the bf16 nearest to 2.0."""
    n, k = 64, 10_000
    hp = HParams(lr=1e-4, weight_decay=0.0, eps=0.0)
    p = bf16_bits(np.ones(n))
    m, v, c = np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.float32)
    pb, mb, vb, cb = p.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.uint16)
    g = bf16_bits(-np.ones(n))
    for t in range(1, k + 1):
        oracle.adamw_pure(p, g, m, v, c, hp, t, lib=olib)
        oracle.adamw_pure(pb, g, mb, vb, cb, hp, t, lib=olib)
    got = bf16_val(p).astype(np.float64) + c
    got_b = bf16_val(pb).astype(np.float64) + bf16_val(cb)
    assert np.all(np.abs(got - 2.0) <= 1e-5), np.abs(got - 2.0).max()
    assert np.all(bf16_val(p) == 2.0)
    assert np.all(np.abs(got_b - 2.0) > 1e-3)      # the bf16 buffer is measurably coarser


def test_pure_fp32_compensation_follows_the_mixed_master(olib):
    """bf16 p plus an fp32 compensation c carry an fp32 master: after 10 steps
    from w = p (c = 0), p + c stays within the bound that the two rules' one
    difference allows of the mixed step's fp32 master w.  Per step that
    difference is the decay of c, which the Kahan reading leaves undecayed
    (|lr*wd*c| with |c| at most half a bf16 ulp of p, <= 2^-8 |p|), plus a few
    fp32 roundings; the fp32 moments are the mixed ones exactly.  A bf16
    compensation buffer lands outside the same bound on many elements."""
    rng = np.random.default_rng(43)
    n, steps = 30_000, 10
    hp = HParams()
    p = bf16_bits(rng.standard_normal(n) * 0.02)
    w = bf16_val(p).copy()
    m, v = np.zeros(n, np.float32), np.zeros(n, np.float32)
    c = np.zeros(n, np.float32)
    pb, mb, vb, cb = p.copy(), m.copy(), v.copy(), np.zeros(n, np.uint16)
    mm, vm, p16 = np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.uint16)
    for t in range(1, steps + 1):
        g = bf16_bits(rng.standard_normal(n) * 1e-3)
        oracle.adamw_pure(p, g, m, v, c, hp, t, lib=olib)
        oracle.adamw_pure(pb, g, mb, vb, cb, hp, t, lib=olib)
        oracle.adamw_mixed(p16, g, w, mm, vm, hp, t, lib=olib)
    assert np.array_equal(m, mm) and np.array_equal(v, vm)
    aw = np.abs(w).astype(np.float64)
    ulp = np.spacing(np.float32(1.0)) * np.maximum(aw, hp.lr)        # an fp32 ulp of w (or of one step)
    bound = steps * (hp.lr * hp.weight_decay * 2.0 ** -8 * aw + 4 * ulp)
    err = np.abs(bf16_val(p).astype(np.float64) + c - w)
    assert np.all(err <= bound), (err / bound).max()
    err_b = np.abs(bf16_val(pb).astype(np.float64) + bf16_val(cb) - w)
    assert (err_b > bound).mean() > 1 / 3          # the bound is not vacuous


@pytest.mark.parametrize("m32,v32", [(True, True), (False, False), (True, False)])
def test_compensation_dtype_changes_only_the_residual(olib, m32, v32):
    """The compensation buffer's dtype touches nothing but the residual: over 6
    steps the moments are bit-identical with an fp32 buffer, a bf16 buffer and
    none (the moment update reads neither p nor c), and after the first step
    from c = 0 both buffers give the same param while the bf16 residual is the
    fp32 residual rounded to nearest even."""
    rng = np.random.default_rng(44)
    n = 20_000
    p0 = bf16_bits(rng.standard_normal(n) * 0.02)
    runs = {}
    for name, c in (("f32", np.zeros(n, np.float32)), ("bf16", np.zeros(n, np.uint16)), ("none", None)):
        runs[name] = [p0.copy(), np.zeros(n, np.float32) if m32 else np.zeros(n, np.uint16),
                      np.zeros(n, np.float32) if v32 else np.zeros(n, np.uint16), c]
    for t in range(1, 7):
        g = bf16_bits(rng.standard_normal(n) * 1e-3)
        for r in runs.values():
            oracle.adamw_pure(r[0], g, r[1], r[2], r[3], HParams(), t, lib=olib)
        if t == 1:
            assert np.array_equal(runs["f32"][0], runs["bf16"][0])
            assert np.array_equal(runs["bf16"][3], bf16_bits(runs["f32"][3]))
            assert np.any(runs["f32"][3] != bf16_val(runs["bf16"][3]))
    for k in (1, 2):
        assert np.array_equal(runs["f32"][k], runs["bf16"][k]) and np.array_equal(runs["f32"][k], runs["none"][k])
