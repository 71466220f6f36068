/* oracle_check.c -- the CPU oracle (oracle/adamw_oracle.c) under
 * AddressSanitizer and UndefinedBehaviorSanitizer.  Built by
 * tests/test_sanitizers.py with gcc together with the oracle's source.
 *
 * Every exported oracle function runs on every length from 0 to 70 and a few
 * longer ones, each array in its own heap allocation of exactly that length
 * (so an access one element past the end is reported), on random bit patterns
 * that include NaN, infinities and subnormals, at step indices from 1 up to
 * 2^40.  The conversions also run over every 16-bit pattern.  The program
 * prints "oracle_check ok" and a checksum of every output, which the test
 * compares with the same program built without the sanitizers (so the
 * sanitizers change nothing the oracle computes).  A NaN output counts as "a
 * NaN", whatever its sign and payload: which NaN an operation with NaN
 * operands returns depends on the order the compiler gives a commutative
 * operation's operands and on whether sqrt is inlined, and the parity bar
 * compares NaNs as a class.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

float oracle_bf16_to_f32(uint16_t h);
float oracle_f16_to_f32(uint16_t h);
uint16_t oracle_f32_to_bf16(float x);
uint16_t oracle_f32_to_f16(float x);
void oracle_bf16_to_f32_n(const uint16_t* in, float* out, int64_t n);
void oracle_f16_to_f32_n(const uint16_t* in, float* out, int64_t n);
void oracle_f32_to_bf16_n(const float* in, uint16_t* out, int64_t n);
void oracle_f32_to_f16_n(const float* in, uint16_t* out, int64_t n);
void oracle_scalars(int64_t t, float lr, float beta1, float beta2, float wd, float* out);
int oracle_any_nonfinite_f16(const uint16_t* g, int64_t n);
int oracle_any_nonfinite_bf16(const uint16_t* g, int64_t n);
float oracle_inv_scale(float scale);
void oracle_update_loss_scale(float* scale, int32_t* tracker, int found_inf, float growth, float backoff,
                              int32_t interval);
void oracle_adamw_mixed(int64_t n, int p_is_f16, uint16_t* p16, const uint16_t* g16, float* master, float* m,
                        float* v, float lr, float beta1, float beta2, float eps, float wd, float inv_scale,
                        int64_t t);
void oracle_adamw_kahan(int64_t n, uint16_t* p, const uint16_t* g, uint16_t* m, uint16_t* v, uint16_t* c,
                        float lr, float beta1, float beta2, float eps, float wd, float inv_scale, int64_t t);
void oracle_adamw_bf16_naive(int64_t n, uint16_t* p, const uint16_t* g, uint16_t* m, uint16_t* v, float lr,
                             float beta1, float beta2, float eps, float wd, float inv_scale, int64_t t);
void oracle_adamw_mixed_split(int64_t n, uint16_t* p, const uint16_t* g16, uint16_t* r, float* m, float* v,
                              float lr, float beta1, float beta2, float eps, float wd, float inv_scale, int64_t t);
void oracle_split_make_n(const uint32_t* w, uint16_t* p, uint16_t* r, int64_t n);
void oracle_split_join_n(const uint16_t* p, const uint16_t* r, uint32_t* w, int64_t n);
void oracle_adamw_pure(int64_t n, uint16_t* p, const uint16_t* g, void* m, int m_f32, void* v, int v_f32,
                       void* c, int c_f32, float lr, float beta1, float beta2, float eps, float wd, float inv_scale,
                       int64_t t);

static uint64_t g_rng = 0x243f6a8885a308d3ull, g_sum = 1469598103934665603ull;

static uint64_t next(void)
{
    g_rng ^= g_rng << 13;
    g_rng ^= g_rng >> 7;
    g_rng ^= g_rng << 17;
    return g_rng;
}

static void mix(uint32_t x) { g_sum = (g_sum ^ x) * 1099511628211ull; }

/* fp32 outputs (read bytewise: the arrays hold float or uint32 objects), every
 * NaN mixed in as one value */
static void mix_f32(const void* p, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) {
        uint32_t u;
        memcpy(&u, (const char*)p + 4 * i, 4);
        mix((u & 0x7fffffffu) > 0x7f800000u ? 0x7fc00000u : u);
    }
}

/* 16-bit float outputs (f16: binary16, else bfloat16), every NaN as one value */
static void mix_h(const uint16_t* h, int64_t n, int f16)
{
    const uint32_t expo = f16 ? 0x7c00u : 0x7f80u;
    for (int64_t i = 0; i < n; ++i) {
        const uint32_t x = h[i];
        mix((x & expo) == expo && (x & ~(expo | 0x8000u)) ? 0x10000u : x);
    }
}

/* A heap array of exactly n elements of `size` bytes (at least one byte, so
 * that malloc(0) never stands for a valid empty array with data). */
static void* arr(int64_t n, size_t size)
{
    void* p = malloc(n ? (size_t)n * size : 1);
    if (!p) abort();
    return p;
}

/* Random 32-bit patterns: a mix of moderate floats, zeros, subnormals,
 * infinities, NaNs and arbitrary bits. */
static uint32_t rand_f32_bits(void)
{
    const uint64_t k = next() % 8;
    uint32_t u = (uint32_t)next();
    switch (k) {
    case 0: return u & 0x807fffffu;                  /* zero or subnormal */
    case 1: return (u & 0x80000000u) | 0x7f800000u;   /* infinity */
    case 2: return u | 0x7f800001u;                   /* NaN */
    case 3: return u;                                 /* anything */
    default: {
        float f = (float)((int32_t)(u % 2000001u) - 1000000) * 1e-8f;
        uint32_t b;
        memcpy(&b, &f, 4);
        return b;
    }
    }
}

static uint16_t rand_16(int finite_only, int f16)
{
    uint16_t h = (uint16_t)next();
    if (finite_only) {
        const uint16_t expo = f16 ? 0x7c00u : 0x7f80u;
        if ((h & expo) == expo) h &= (uint16_t)~0x4000u;
    }
    return h;
}

static void fill_f32(float* x, int64_t n, int finite_small)
{
    for (int64_t i = 0; i < n; ++i) {
        uint32_t b = finite_small ? 0 : rand_f32_bits();
        if (finite_small) {
            float f = (float)((int32_t)(next() % 20001u) - 10000) * 1e-6f;
            memcpy(&b, &f, 4);
        }
        memcpy(&x[i], &b, 4);
    }
}

static void fill_16(uint16_t* x, int64_t n, int finite_only, int f16)
{
    for (int64_t i = 0; i < n; ++i) x[i] = rand_16(finite_only, f16);
}

static void run_length(int64_t n)
{
    static const int64_t steps[] = {1, 2, 17, 1000, 2147483647, (int64_t)1 << 40};
    for (size_t si = 0; si < sizeof steps / sizeof steps[0]; ++si) {
        const int64_t t = steps[si];
        const int generic = (int)(next() % 2);   /* 0: finite moderate values, 1: any bit patterns */
        /* mixed, bf16 and fp16 */
        for (int f16 = 0; f16 < 2; ++f16) {
            uint16_t* p = arr(n, 2);
            uint16_t* g = arr(n, 2);
            float* w = arr(n, 4);
            float* m = arr(n, 4);
            float* v = arr(n, 4);
            fill_16(p, n, 0, f16);
            fill_16(g, n, !generic, f16);
            fill_f32(w, n, !generic);
            fill_f32(m, n, !generic);
            for (int64_t i = 0; i < n; ++i) v[i] = generic ? (float)(next() % 1000) * 1e-9f : 0.0f;
            oracle_adamw_mixed(n, f16, p, g, w, m, v, 2e-4f, 0.9f, 0.95f, 1e-8f, 0.1f,
                               f16 ? 1.0f / 65536.0f : 1.0f, t);
            mix_h(p, n, f16);
            mix_f32(w, n);
            mix_f32(m, n);
            mix_f32(v, n);
            g_sum ^= (uint64_t)oracle_any_nonfinite_f16(g, n) << 1 | (uint64_t)oracle_any_nonfinite_bf16(g, n);
            free(p); free(g); free(w); free(m); free(v);
        }
        /* Kahan, naive bf16 and split */
        {
            uint16_t* p = arr(n, 2);
            uint16_t* g = arr(n, 2);
            uint16_t* m = arr(n, 2);
            uint16_t* v = arr(n, 2);
            uint16_t* c = arr(n, 2);
            fill_16(p, n, 0, 0);
            fill_16(g, n, !generic, 0);
            fill_16(m, n, 0, 0);
            fill_16(v, n, 0, 0);
            fill_16(c, n, 0, 0);
            oracle_adamw_kahan(n, p, g, m, v, c, 2e-4f, 0.9f, 0.95f, 1e-8f, 0.1f, 1.0f, t);
            mix_h(p, n, 0);
            mix_h(c, n, 0);
            oracle_adamw_bf16_naive(n, p, g, m, v, 2e-4f, 0.9f, 0.95f, 1e-8f, 0.1f, 1.0f, t);
            mix_h(p, n, 0);
            mix_h(m, n, 0);
            float* m32 = arr(n, 4);
            float* v32 = arr(n, 4);
            fill_f32(m32, n, 1);
            for (int64_t i = 0; i < n; ++i) v32[i] = (float)(next() % 1000) * 1e-9f;
            oracle_adamw_mixed_split(n, p, g, c, m32, v32, 2e-4f, 0.9f, 0.95f, 1e-8f, 0.1f, 1.0f, t);
            /* the split master as the fp32 value it encodes (a NaN master's
             * remainder holds NaN payload bits) */
            uint32_t* joined = arr(n, 4);
            oracle_split_join_n(p, c, joined, n);
            mix_f32(joined, n);
            mix_f32(m32, n);
            free(joined);
            fill_16(p, n, 0, 0);
            fill_16(c, n, 0, 0);
            fill_f32(m32, n, 1);
            float* c32 = arr(n, 4);
            for (int64_t i = 0; i < n; ++i) c32[i] = (float)((int64_t)(next() % 2001) - 1000) * 1e-9f;
            for (int mf = 0; mf < 2; ++mf)
                for (int vf = 0; vf < 2; ++vf)
                    for (int k = 0; k < 3; ++k) {   /* no compensation, bf16, fp32 */
                        oracle_adamw_pure(n, p, g, mf ? (void*)m32 : (void*)m, mf, vf ? (void*)v32 : (void*)v, vf,
                                          k == 0 ? NULL : k == 1 ? (void*)c : (void*)c32, k == 2, 2e-4f, 0.9f,
                                          0.95f, 1e-8f, 0.1f, 1.0f, t);
                        mix_h(p, n, 0);
                    }
            mix_f32(c32, n);
            free(c32);
            uint32_t* w = arr(n, 4);
            for (int64_t i = 0; i < n; ++i) w[i] = rand_f32_bits();
            oracle_split_make_n(w, p, c, n);
            uint32_t* back = arr(n, 4);
            oracle_split_join_n(p, c, back, n);
            for (int64_t i = 0; i < n; ++i)
                if ((w[i] & 0x7fffffffu) <= 0x7f800000u && back[i] != w[i]) abort();   /* exact round trip */
            mix_f32(back, n);
            free(p); free(g); free(m); free(v); free(c); free(m32); free(v32); free(w); free(back);
        }
    }
}

int main(void)
{
    /* conversions over every 16-bit pattern, and random fp32 patterns narrowed */
    {
        const int64_t n = 65536;
        uint16_t* h = arr(n, 2);
        float* f = arr(n, 4);
        for (int64_t i = 0; i < n; ++i) h[i] = (uint16_t)i;
        oracle_bf16_to_f32_n(h, f, n);
        mix_f32(f, n);
        oracle_f16_to_f32_n(h, f, n);
        mix_f32(f, n);
        for (int64_t i = 0; i < n; ++i) {
            uint32_t b = (i & 1) ? rand_f32_bits() : (uint32_t)next();
            memcpy(&f[i], &b, 4);
        }
        oracle_f32_to_bf16_n(f, h, n);
        mix_h(h, n, 0);
        oracle_f32_to_f16_n(f, h, n);
        mix_h(h, n, 1);
        free(h);
        free(f);
    }
    /* scalars and the loss scale over their whole input ranges */
    {
        static const int64_t ts[] = {1, 2, 3, 10, 500, 65535, 2147483647, (int64_t)1 << 40};
        static const float betas[] = {0.0f, 0.5f, 0.9f, 0.95f, 0.999f, 0.99999994f};
        float out[6];
        for (size_t a = 0; a < sizeof ts / sizeof ts[0]; ++a)
            for (size_t b = 0; b < sizeof betas / sizeof betas[0]; ++b) {
                oracle_scalars(ts[a], 2e-4f, betas[b], betas[(b + 1) % 6], 0.1f, out);
                mix_f32(out, 6);
            }
        float s = 65536.0f;
        int32_t tr = 0;
        for (int i = 0; i < 5000; ++i) {
            oracle_update_loss_scale(&s, &tr, (next() % 97) == 0, 2.0f, 0.5f, 7);
            if (tr < 0 || tr >= 7) abort();
        }
        float big = 3e38f;
        tr = 0;
        oracle_update_loss_scale(&big, &tr, 0, 2.0f, 0.5f, 1);   /* growth refused: not finite */
        mix_f32(&big, 1);
        mix_f32(&s, 1);
        float inv = oracle_inv_scale(65536.0f);
        mix_f32(&inv, 1);
    }
    for (int64_t n = 0; n <= 70; ++n) run_length(n);
    run_length(4096 + 5);
    run_length(65536 + 3);
    printf("oracle_check ok %016llx\n", (unsigned long long)g_sum);
    return 0;
}
