"""The pins catch plausible mistakes: each mutant below plants one mistake in a
copy of the oracle's C source (built into a temporary directory; the real
oracle is untouched) and at least one pin of test_oracle_pins must fail on it.
"""
import ctypes
import os
import subprocess
import tempfile

import pytest

import test_oracle_pins as pins
from oracle import _SRC, CFLAGS, _bind

# (name, original text, planted mistake)
MUTANTS = [
    ("beta swapped in m", "float mi = beta1 * *m + omb1 * g;", "float mi = beta2 * *m + omb1 * g;"),
    ("g not squared in v", "float vi = beta2 * *v + omb2 * (g * g);", "float vi = beta2 * *v + omb2 * g;"),
    ("eps inside sqrt", "return mi / (sqrtf(vi * rbc2) + eps);", "return mi / sqrtf(vi * rbc2 + eps);"),
    ("no bias correction of m", "out[0] = (float)((double)lr / (1.0 - b1t));", "out[0] = lr;"),
    ("no bias correction of v", "out[1] = (float)(1.0 / (1.0 - b2t));", "out[1] = 1.0f;"),
    ("t off by one", "double b1t = pow_by_squaring((double)beta1, t);",
     "double b1t = pow_by_squaring((double)beta1, t + 1);"),
    ("wrong bit in powering", "if (t & 1) r = r * b;", "if (t & 2) r = r * b;"),
    ("decay dropped (mixed)", "float w = master[i] * decay - step_size * u;", "float w = master[i] - step_size * u;"),
    ("decay is 1-wd", "out[2] = (float)(1.0 - (double)lr * (double)wd);", "out[2] = (float)(1.0 - (double)wd);"),
    ("update sign (mixed)", "float w = master[i] * decay - step_size * u;", "float w = master[i] * decay + step_size * u;"),
    ("no unscale (mixed)", ": oracle_bf16_to_f32(g16[i])) * inv_scale;", ": oracle_bf16_to_f32(g16[i]));"),
    ("Kahan compensation sign", "c[i] = oracle_f32_to_bf16(sum - absorbed);", "c[i] = oracle_f32_to_bf16(sum + absorbed);"),
    ("Kahan compensation dropped", "float sum = oracle_bf16_to_f32(c[i]) + d;", "float sum = d;"),
    ("Kahan decay dropped", "float d = -(lrwd * pf) - step_size * u;", "float d = -step_size * u;"),
    ("Kahan m/v stores swapped", "m[i] = oracle_f32_to_bf16(mi);", "m[i] = oracle_f32_to_bf16(vi);"),
    ("bf16 ties away from zero", "if (drop > 0x8000u || (drop == 0x8000u && (keep & 1u))) keep += 1u;",
     "if (drop >= 0x8000u) keep += 1u;"),
    ("bf16 truncation", "if (drop > 0x8000u || (drop == 0x8000u && (keep & 1u))) keep += 1u;", ";"),
    ("f16 subnormal boundary", "int q_exp = (e < -14) ? -24 : e - 10;", "int q_exp = (e < -15) ? -24 : e - 10;"),
    ("f16 overflow threshold", "if (a >= 65520.0)", "if (a >= 65504.0)"),
    ("f16 widen exponent bias", "mag = ldexpf((float)(1024 + f), e - 25);", "mag = ldexpf((float)(1024 + f), e - 24);"),
    ("NaN not detected (f16)", "if ((g[i] & 0x7c00u) == 0x7c00u) return 1;",
     "if ((g[i] & 0x7fffu) == 0x7c00u) return 1;"),
    ("f16 ties", "if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) == 1.0)) r += 1.0;",
     "if (frac >= 0.5) r += 1.0;"),
    ("split tie goes down", "hi = (w >> 16) + (low >= 0x8000u ? 1u : 0u);", "hi = (w >> 16) + (low > 0x8000u ? 1u : 0u);"),
    ("split truncates", "hi = (w >> 16) + (low >= 0x8000u ? 1u : 0u);", "hi = (w >> 16);"),
    ("remainder zero-extended", "int32_t rem = (int32_t)(int16_t)r;", "int32_t rem = (int32_t)r;"),
    ("growth one step early", "if (run == interval) {", "if (run + 1 >= interval) {"),
    ("backoff keeps tracker", "*scale = *scale * backoff;\n        *tracker = 0;", "*scale = *scale * backoff;"),
    ("growth without finiteness test", "if (isfinite(grown)) *scale = grown;", "*scale = grown;"),
    ("inverse scale in float", "return (float)(1.0 / (double)scale);", "return 1.0f / (scale * 1.0000001f);"),
    ("split decay dropped", "w = w * decay - step_size * u;\n        oracle_split_make", "w = w - step_size * u;\n        oracle_split_make"),
    ("pure fp32 residual rounded to bf16", "if (c_f32) cf[i] = rest;",
     "if (c_f32) cf[i] = oracle_bf16_to_f32(oracle_f32_to_bf16(rest));"),
    ("pure fp32 compensation never read", "float sum = (c_f32 ? cf[i] : oracle_bf16_to_f32(ch[i])) + d;",
     "float sum = (c_f32 ? 0.0f : oracle_bf16_to_f32(ch[i])) + d;"),
    ("pure residual sign", "float rest = sum - (oracle_bf16_to_f32(pn) - pf);",
     "float rest = sum + (oracle_bf16_to_f32(pn) - pf);"),
    ("pure fp32 moment kept from before", "if (m_f32) mf[i] = mi;", "if (m_f32) mf[i] = mf[i];"),
]

# fastest first; each entry is (pin, extra args)
PINS = [
    (pins.test_scalars_match_library_pow, ()),
    (pins.test_step1_closed_form, (1e-8,)),
    (pins.test_step1_closed_form, (1e-3,)),
    (pins.test_step1_decay_only_from_nonzero_weight, ()),
    (pins.test_f16_scaled_equals_bf16_unscaled, ()),
    (pins.test_kahan_step1_agrees_with_mixed, ()),
    (pins.test_constant_gradient_closed_form, ()),
    (pins.test_beta_zero_is_decayed_sign_sgd, ()),
    (pins.test_skip_on_nonfinite_f16, (0x7C01,)),
    (pins.test_skip_on_nonfinite_f16, (0x7C00,)),
    (pins.test_bf16_widen_exhaustive, ()),
    (pins.test_f16_widen_exhaustive, ()),
    (pins.test_bf16_narrow_vs_torch, ()),
    (pins.test_f16_narrow_vs_numpy, ()),
    (pins.test_kahan_tracks_constant_tiny_updates, ()),
    (pins.test_zero_gradient_kahan_tracks_decay, ()),
]
AMP_PINS = [
    (pins.test_loss_scale_rule_matches_torch, (2.0, 0.5, 3, 65536.0)),
    (pins.test_loss_scale_rule_matches_torch, (2.0, 0.5, 2, 3e38)),
    (pins.test_inv_scale, ()),
    (pins.test_amp_step_skips_and_backs_off, ()),
]
PURE_PINS = [
    (pins.test_pure_bf16_state_reduces_to_kahan_and_naive, ()),
    (pins.test_pure_fp32_moments_follow_the_mixed_moments, (True, True)),
    (pins.test_pure_fp32_compensation_tracks_tiny_updates_closely, ()),
    (pins.test_pure_fp32_compensation_follows_the_mixed_master, ()),
    (pins.test_compensation_dtype_changes_only_the_residual, (False, False)),
]
SPLIT_PINS = [
    (pins.test_split_step_equals_mixed_step, (pins.HParams(),)),
    (pins.test_split_join_roundtrip, ()),
    (pins.test_split_param_is_a_nearest_bf16, ()),
]


@pytest.fixture(scope="module")
def tmpdir_mut():
    with tempfile.TemporaryDirectory() as d:
        yield d


@pytest.mark.parametrize("name,orig,bad", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_killed(tmpdir_mut, name, orig, bad):
    src = open(_SRC).read()
    assert src.count(orig) >= 1, f"mutation site for {name!r} not found"
    mutated = src.replace(orig, bad, 1)
    tag = "".join(ch if ch.isalnum() else "_" for ch in name)
    csrc = os.path.join(tmpdir_mut, f"{tag}.c")
    so = os.path.join(tmpdir_mut, f"lib{tag}.so")
    open(csrc, "w").write(mutated)
    subprocess.run(["gcc", *CFLAGS, "-o", so, csrc, "-lm"], check=True)
    lib = _bind(ctypes.CDLL(so))
    amp = any(w in name for w in ("growth", "backoff", "inverse scale"))
    split = name.startswith("split") or "remainder" in name
    if name.startswith("pure"):
        order = PURE_PINS
    else:
        order = AMP_PINS + PINS + SPLIT_PINS if amp else SPLIT_PINS + PINS + AMP_PINS if split else \
            PINS + SPLIT_PINS + AMP_PINS
    for pin, args in order:
        try:
            pin(lib, *args)
        except AssertionError:
            return  # killed
    pytest.fail(f"mutant {name!r} survived every pin")
