/*
 * adamw_oracle.c -- plain scalar CPU oracle for the fused AdamW optimizer step.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the package's
 * smoke check and the benchmark's CPU-baseline leg may load this library.  It
 * shares no source, header, table or helper with the GPU library: the two are
 * written separately and meet only on the bytes of their inputs and outputs.
 *
 * What it computes, and where it comes from:
 *   - The optimizer is AdamW: Adam's first/second moment estimates with bias
 *     correction (Kingma & Ba, "Adam", ICLR 2015, Algorithm 1) plus weight
 *     decay decoupled from the gradient (Loshchilov & Hutter, "Decoupled
 *     Weight Decay Regularization", ICLR 2019, Algorithm 2).  The pages name the
 *     optimizer and its hyper-parameters but never print the update rule:
 *       "Distributed optimizer support for BERT", Usage (fused_adam /
 *       distributed_fused_adam) and the A40/A100 tables ("BF16 with O2");
 *       "[pure bf16 training] w/ AnyPrecisionAdamW and Kahan summation",
 *       the opt-1.3b training command (--weight_decay 0.1 --adam_beta1 0.9
 *       --adam_beta2 0.95 --learning_rate 0.0002, linear schedule, 500 warmup).
 *   - Mixed ("O2") mode: 16-bit model parameter + fp32 master copy + fp32
 *     moments ("BF16 with O2 optimizations"; the bf16-mixed memory breakdown
 *     8 optim + 2 grad + 4+2 weights bytes per parameter).
 *   - Pure bf16 mode with Kahan compensation: bf16 parameter, bf16 moments and
 *     a bf16 compensation buffer (the --optim_args string
 *     use_kahan_summation=true, momentum_dtype=bfloat16,
 *     variance_dtype=bfloat16, compensation_buffer_dtype=bfloat16; the bf16-pure
 *     breakdown 4+2 optim + 2 grad + 2 weights).
 *   - fp16 AMP: gradients carry a loss scale; any inf/NaN gradient skips the
 *     whole step (the opt-125m fp16-amp run on the AnyPrecisionAdamW page).
 *
 * Arithmetic contract (the readings where the pages are silent):
 *   - Per-launch scalars are formed in IEEE double from +, -, *, / only and
 *     rounded once to float.  beta^t is formed by right-to-left binary
 *     powering (square-and-multiply), so the sequence of double products is
 *     fixed.
 *   - Per-element math is IEEE binary32, every operation rounded to nearest
 *     even, in the written order; no fused multiply-add (build with
 *     -ffp-contract=off), correctly rounded sqrtf and division, subnormals kept.
 *   - Narrowing to bf16/fp16 rounds to nearest, ties to even; NaN stays NaN.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* ------------------------------------------------------------------------- */
/* 16-bit floating point formats, decoded from their IEEE-style definitions.  */
/* ------------------------------------------------------------------------- */

static float bits_to_f32(uint32_t u) { float f; memcpy(&f, &u, sizeof f); return f; }
static uint32_t f32_to_bits(float f) { uint32_t u; memcpy(&u, &f, sizeof u); return u; }

/* bfloat16 is the upper 16 bits of a binary32 value: widening is exact. */
float oracle_bf16_to_f32(uint16_t h) { return bits_to_f32((uint32_t)h << 16); }

/* binary16: sign (1), exponent (5, bias 15), fraction (10). */
float oracle_f16_to_f32(uint16_t h)
{
    uint32_t sign = (uint32_t)(h >> 15) << 31;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    if (e == 0x1f) {
        if (f == 0) return bits_to_f32(sign | 0x7f800000u);          /* +-inf */
        return bits_to_f32(sign | 0x7fc00000u | ((uint32_t)f << 13)); /* quiet NaN */
    }
    float mag;
    if (e == 0) mag = ldexpf((float)f, -24);              /* subnormal: f * 2^-24 */
    else mag = ldexpf((float)(1024 + f), e - 25);         /* normal: 1.f * 2^(e-15) */
    return sign ? -mag : mag;
}

/* Round a binary32 value to bfloat16, nearest, ties to even.  The 16 dropped
 * bits are compared with one half unit in the last kept place (0x8000). */
uint16_t oracle_f32_to_bf16(float x)
{
    uint32_t u = f32_to_bits(x);
    if (isnan(x)) return (uint16_t)((u >> 16) | 0x0040u);   /* quiet, sign kept */
    uint32_t keep = u >> 16;
    uint32_t drop = u & 0xffffu;
    if (drop > 0x8000u || (drop == 0x8000u && (keep & 1u))) keep += 1u; /* carry may reach inf */
    return (uint16_t)keep;
}

/* Round a binary32 value to binary16, nearest, ties to even, written on the
 * exact value: scale |x| by the binary16 quantum of its binade, round the
 * quotient to an integer, and encode. */
uint16_t oracle_f32_to_f16(float x)
{
    uint32_t u = f32_to_bits(x);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    if (isnan(x)) return (uint16_t)(sign | 0x7e00u | ((u >> 13) & 0x3ffu));
    double a = fabs((double)x);
    if (a >= 65520.0) return (uint16_t)(sign | 0x7c00u);   /* >= max + half ulp: inf */
    if (a == 0.0) return sign;
    int ex;
    (void)frexp(a, &ex);                 /* a = m * 2^ex, m in [0.5, 1) */
    int e = ex - 1;                      /* floor(log2 a) */
    int q_exp = (e < -14) ? -24 : e - 10;  /* quantum: 2^-24 below 2^-14, else 2^(e-10) */
    double n = ldexp(a, -q_exp);         /* exact */
    double r = floor(n);
    double frac = n - r;                 /* exact */
    if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) == 1.0)) r += 1.0;
    uint32_t ir = (uint32_t)r;
    if (e < -14) return (uint16_t)(sign | ir);   /* subnormal (ir == 1024 encodes 2^-14) */
    /* normal: value = ir * 2^(e-10), ir in [1024, 2048]; the leading bit of ir
     * lands in the exponent field, so ir == 2048 moves to the next binade. */
    return (uint16_t)(sign | (((uint32_t)(e + 14) << 10) + ir));
}

/* Exhaustive/batch helpers for the conversion pins. */
void oracle_bf16_to_f32_n(const uint16_t* in, float* out, int64_t n)
{ for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_to_f32(in[i]); }
void oracle_f16_to_f32_n(const uint16_t* in, float* out, int64_t n)
{ for (int64_t i = 0; i < n; ++i) out[i] = oracle_f16_to_f32(in[i]); }
void oracle_f32_to_bf16_n(const float* in, uint16_t* out, int64_t n)
{ for (int64_t i = 0; i < n; ++i) out[i] = oracle_f32_to_bf16(in[i]); }
void oracle_f32_to_f16_n(const float* in, uint16_t* out, int64_t n)
{ for (int64_t i = 0; i < n; ++i) out[i] = oracle_f32_to_f16(in[i]); }

/* ------------------------------------------------------------------------- */
/* Per-launch scalars.                                                        */
/* ------------------------------------------------------------------------- */

/* beta^t in double by right-to-left binary powering. */
static double pow_by_squaring(double b, int64_t t)
{
    double r = 1.0;
    while (t > 0) {
        if (t & 1) r = r * b;
        b = b * b;
        t >>= 1;
    }
    return r;
}

/* out[0] step_size = lr / (1 - beta1^t)            (bias correction of m)
 * out[1] rbc2      = 1 / (1 - beta2^t)             (bias correction of v)
 * out[2] decay     = 1 - lr*wd                     (decoupled weight decay factor)
 * out[3] lrwd      = lr*wd
 * out[4] omb1      = 1 - beta1   (in float)
 * out[5] omb2      = 1 - beta2   (in float)
 * t is the 1-based index of the step being taken. */
void oracle_scalars(int64_t t, float lr, float beta1, float beta2, float wd, float* out)
{
    double b1t = pow_by_squaring((double)beta1, t);
    double b2t = pow_by_squaring((double)beta2, t);
    out[0] = (float)((double)lr / (1.0 - b1t));
    out[1] = (float)(1.0 / (1.0 - b2t));
    out[2] = (float)(1.0 - (double)lr * (double)wd);
    out[3] = (float)((double)lr * (double)wd);
    out[4] = 1.0f - beta1;
    out[5] = 1.0f - beta2;
}

/* ------------------------------------------------------------------------- */
/* Overflow check (fp16 AMP): any gradient whose exponent field is all ones   */
/* (inf or NaN) makes the whole step a no-op.                                 */
/* ------------------------------------------------------------------------- */

int oracle_any_nonfinite_f16(const uint16_t* g, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        if ((g[i] & 0x7c00u) == 0x7c00u) return 1;
    return 0;
}

int oracle_any_nonfinite_bf16(const uint16_t* g, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        if ((g[i] & 0x7f80u) == 0x7f80u) return 1;
    return 0;
}

/* Dynamic loss scaling (fp16 AMP): a step with an inf/NaN gradient multiplies
 * the scale by `backoff`; growth_interval consecutive clean steps multiply it
 * by `growth`, unless that product is not finite; either event restarts the
 * count.  The step itself unscales by 1/scale formed in double, rounded to
 * float (exact for the power-of-two scales of the fp16-amp run). */
float oracle_inv_scale(float scale) { return (float)(1.0 / (double)scale); }

void oracle_update_loss_scale(float* scale, int32_t* tracker, int found_inf,
                              float growth, float backoff, int32_t interval)
{
    if (found_inf) {
        *scale = *scale * backoff;
        *tracker = 0;
        return;
    }
    int32_t run = *tracker + 1;
    if (run == interval) {
        float grown = *scale * growth;
        if (isfinite(grown)) *scale = grown;
        *tracker = 0;
    } else {
        *tracker = run;
    }
}

/* ------------------------------------------------------------------------- */
/* The element update.                                                        */
/* ------------------------------------------------------------------------- */

/* Adam direction: with m, v the updated moments,
 *   m_hat = m / (1 - beta1^t),  v_hat = v / (1 - beta2^t),
 *   u = m_hat / (sqrt(v_hat) + eps).
 * The 1/(1 - beta1^t) factor is carried by step_size, so the direction
 * evaluated here is m / (sqrt(v * rbc2) + eps). */
static float adam_moments(float g, float* m, float* v,
                          float beta1, float beta2, float omb1, float omb2,
                          float rbc2, float eps)
{
    float mi = beta1 * *m + omb1 * g;
    float vi = beta2 * *v + omb2 * (g * g);
    *m = mi;
    *v = vi;
    return mi / (sqrtf(vi * rbc2) + eps);
}

/* Mixed ("O2") precision: 16-bit gradient, fp32 master weight, fp32 moments.
 *   w <- w * (1 - lr*wd) - (lr / (1 - beta1^t)) * u
 *   p16 <- round(w)                     (the 16-bit parameter is write-only)
 * p_is_f16 selects binary16 (fp16 AMP) instead of bfloat16 for p and g. */
void oracle_adamw_mixed(int64_t n, int p_is_f16,
                        uint16_t* p16, const uint16_t* g16,
                        float* master, float* m, float* v,
                        float lr, float beta1, float beta2, float eps, float wd,
                        float inv_scale, int64_t t)
{
    float s[6];
    oracle_scalars(t, lr, beta1, beta2, wd, s);
    float step_size = s[0], rbc2 = s[1], decay = s[2];
    for (int64_t i = 0; i < n; ++i) {
        float g = (p_is_f16 ? oracle_f16_to_f32(g16[i]) : oracle_bf16_to_f32(g16[i])) * inv_scale;
        float u = adam_moments(g, &m[i], &v[i], beta1, beta2, s[4], s[5], rbc2, eps);
        float w = master[i] * decay - step_size * u;
        master[i] = w;
        p16[i] = p_is_f16 ? oracle_f32_to_f16(w) : oracle_f32_to_bf16(w);
    }
}

/* Pure bf16 with a bf16 Kahan compensation buffer c (Kahan, "Further remarks
 * on reducing truncation errors", CACM 8(1), 1965).  The decoupled decay and
 * the Adam step form one delta d that is added to p through the compensated
 * sum, so increments far below bf16's resolution still accumulate:
 *   d  = -(lr*wd) * p - step_size * u
 *   s  = c + d                  (pending increment, fp32)
 *   p' = round_bf16(p + s)
 *   c' = round_bf16(s - (p' - p))   (the part of s that p' did not absorb)
 * The moments are updated in fp32 from their bf16 values and stored rounded. */
void oracle_adamw_kahan(int64_t n, uint16_t* p, const uint16_t* g,
                        uint16_t* m, uint16_t* v, uint16_t* c,
                        float lr, float beta1, float beta2, float eps, float wd,
                        float inv_scale, int64_t t)
{
    float s[6];
    oracle_scalars(t, lr, beta1, beta2, wd, s);
    float step_size = s[0], rbc2 = s[1], lrwd = s[3];
    for (int64_t i = 0; i < n; ++i) {
        float gi = oracle_bf16_to_f32(g[i]) * inv_scale;
        float mi = oracle_bf16_to_f32(m[i]);
        float vi = oracle_bf16_to_f32(v[i]);
        float u = adam_moments(gi, &mi, &vi, beta1, beta2, s[4], s[5], rbc2, eps);
        float pf = oracle_bf16_to_f32(p[i]);
        float d = -(lrwd * pf) - step_size * u;
        float sum = oracle_bf16_to_f32(c[i]) + d;
        uint16_t pn = oracle_f32_to_bf16(pf + sum);
        float absorbed = oracle_bf16_to_f32(pn) - pf;
        c[i] = oracle_f32_to_bf16(sum - absorbed);
        p[i] = pn;
        m[i] = oracle_f32_to_bf16(mi);
        v[i] = oracle_f32_to_bf16(vi);
    }
}

/* Split master: the fp32 master w is held as two 16-bit halves, the bf16 model
 * parameter p and an int16 remainder r, with w's bit pattern equal to
 * (p << 16) + r in 32-bit two's-complement arithmetic (a reading of the 16-bit
 * master copy counted in the ZeRO saving estimate of "Distributed optimizer
 * support for BERT").  Splitting picks the p that leaves the smallest remainder: the
 * nearest bf16, ties away from zero, which keeps r within [-32768, 32767]; a
 * NaN master keeps a quiet-NaN p. */
uint32_t oracle_split_join(uint16_t p, uint16_t r)
{
    int32_t rem = (int32_t)(int16_t)r;
    return (uint32_t)(((uint32_t)p << 16) + (uint32_t)rem);
}

void oracle_split_make(uint32_t w, uint16_t* p, uint16_t* r)
{
    uint32_t hi;
    if (isnan(bits_to_f32(w))) {
        hi = (w >> 16) | 0x0040u;
    } else {
        uint32_t low = w & 0xffffu;
        hi = (w >> 16) + (low >= 0x8000u ? 1u : 0u);   /* nearest; the tie goes up in magnitude */
    }
    *p = (uint16_t)hi;
    *r = (uint16_t)(w - (hi << 16));
}

/* Mixed step with the split master: join, the mixed update of w, split. */
void oracle_adamw_mixed_split(int64_t n, uint16_t* p, const uint16_t* g16, uint16_t* r,
                              float* m, float* v,
                              float lr, float beta1, float beta2, float eps, float wd,
                              float inv_scale, int64_t t)
{
    float s[6];
    oracle_scalars(t, lr, beta1, beta2, wd, s);
    float step_size = s[0], rbc2 = s[1], decay = s[2];
    for (int64_t i = 0; i < n; ++i) {
        float g = oracle_bf16_to_f32(g16[i]) * inv_scale;
        float u = adam_moments(g, &m[i], &v[i], beta1, beta2, s[4], s[5], rbc2, eps);
        float w = bits_to_f32(oracle_split_join(p[i], r[i]));
        w = w * decay - step_size * u;
        oracle_split_make(f32_to_bits(w), &p[i], &r[i]);
    }
}

/* Batch forms for the tests. */
void oracle_split_make_n(const uint32_t* w, uint16_t* p, uint16_t* r, int64_t n)
{ for (int64_t i = 0; i < n; ++i) oracle_split_make(w[i], &p[i], &r[i]); }
void oracle_split_join_n(const uint16_t* p, const uint16_t* r, uint32_t* w, int64_t n)
{ for (int64_t i = 0; i < n; ++i) w[i] = oracle_split_join(p[i], r[i]); }

/* Pure bf16 parameters with separately chosen state precisions (the
 * AnyPrecisionAdamW knobs of "[pure bf16 training] w/ AnyPrecisionAdamW and
 * Kahan summation": momentum_dtype, variance_dtype, use_kahan_summation and
 * compensation_buffer_dtype).  m_f32 / v_f32 select fp32 moments (float arrays)
 * instead of bf16 ones (uint16 bit arrays); c == NULL means no compensation:
 * then p' = round_bf16(p * (1 - lr*wd) - step_size * u).  With c, the Kahan rule
 * of oracle_adamw_kahan, the compensation held in bf16 (uint16 bits) or, with
 * c_f32, in fp32 (a float array): the same sum, with the residual kept as the
 * fp32 value it is computed in instead of rounded to bf16. */
void oracle_adamw_pure(int64_t n, uint16_t* p, const uint16_t* g, void* m, int m_f32, void* v, int v_f32,
                       void* c, int c_f32, float lr, float beta1, float beta2, float eps, float wd,
                       float inv_scale, int64_t t)
{
    float s[6];
    oracle_scalars(t, lr, beta1, beta2, wd, s);
    float step_size = s[0], rbc2 = s[1], decay = s[2], lrwd = s[3];
    float* mf = (float*)m;
    float* vf = (float*)v;
    uint16_t* mh = (uint16_t*)m;
    uint16_t* vh = (uint16_t*)v;
    float* cf = (float*)c;
    uint16_t* ch = (uint16_t*)c;
    for (int64_t i = 0; i < n; ++i) {
        float gi = oracle_bf16_to_f32(g[i]) * inv_scale;
        float mi = m_f32 ? mf[i] : oracle_bf16_to_f32(mh[i]);
        float vi = v_f32 ? vf[i] : oracle_bf16_to_f32(vh[i]);
        float u = adam_moments(gi, &mi, &vi, beta1, beta2, s[4], s[5], rbc2, eps);
        float pf = oracle_bf16_to_f32(p[i]);
        if (c) {
            float d = -(lrwd * pf) - step_size * u;
            float sum = (c_f32 ? cf[i] : oracle_bf16_to_f32(ch[i])) + d;
            uint16_t pn = oracle_f32_to_bf16(pf + sum);
            float rest = sum - (oracle_bf16_to_f32(pn) - pf);
            if (c_f32) cf[i] = rest; else ch[i] = oracle_f32_to_bf16(rest);
            p[i] = pn;
        } else {
            p[i] = oracle_f32_to_bf16(pf * decay - step_size * u);
        }
        if (m_f32) mf[i] = mi; else mh[i] = oracle_f32_to_bf16(mi);
        if (v_f32) vf[i] = vi; else vh[i] = oracle_f32_to_bf16(vi);
    }
}

/* Pure bf16 without compensation: the same step applied directly to bf16 p.
 * Used by the tests as the control that Kahan summation is measured against. */
void oracle_adamw_bf16_naive(int64_t n, uint16_t* p, const uint16_t* g,
                             uint16_t* m, uint16_t* v,
                             float lr, float beta1, float beta2, float eps, float wd,
                             float inv_scale, int64_t t)
{
    float s[6];
    oracle_scalars(t, lr, beta1, beta2, wd, s);
    float step_size = s[0], rbc2 = s[1], decay = s[2];
    for (int64_t i = 0; i < n; ++i) {
        float gi = oracle_bf16_to_f32(g[i]) * inv_scale;
        float mi = oracle_bf16_to_f32(m[i]);
        float vi = oracle_bf16_to_f32(v[i]);
        float u = adam_moments(gi, &mi, &vi, beta1, beta2, s[4], s[5], rbc2, eps);
        float w = oracle_bf16_to_f32(p[i]) * decay - step_size * u;
        p[i] = oracle_f32_to_bf16(w);
        m[i] = oracle_f32_to_bf16(mi);
        v[i] = oracle_f32_to_bf16(vi);
    }
}
