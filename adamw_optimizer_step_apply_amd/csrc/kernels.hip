// kernels.hip -- gfx950 (CDNA4) kernels of the fused AdamW step.
//
// The step is a pure stream: every element is read once and written once, with
// no reuse, so there is nothing to stage in LDS and no contraction for the
// matrix cores.  The kernels are shaped for HBM: every lane moves whole 16-byte
// words (8 elements of a 16-bit stream, 4 of an fp32 stream), consecutive lanes
// touch consecutive words, and each lane issues all loads of its 8-element pack
// (one to two 16-byte words per stream) before it computes.  The math is fp32
// in registers.
//
// Kernels:
//   prologue_kernel      one lane: reads the skip flag and the step counter,
//                        forms the step's scalars in binary64, advances the counter
//   update_kernel<MODE, FUSED> / update_pure_kernel<M32, V32, AUX, FUSED>
//                        eight workgroups per chunk, one on each XCD, the chunk
//                        interleaved between them in tiles of 256 or 512
//                        elements: the AdamW element update;
//                        FUSED: without a prologue, for small plans (each
//                        workgroup forms the scalars, the last one advances
//                        the counter)
//   zero_flag_kernel /
//   check_kernel<F16, FUSED>  the fp16-AMP overflow test (any inf/NaN gradient);
//                        FUSED: one launch that also sets the flag to 0 or 1
//   state_copy_kernel    layout only: state between per-tensor buffers and the
//                        blocked buffer
//   zero_words_kernel    clears the completion counters of a new workspace
//
// Element rule (the AdamW of Loshchilov & Hutter, Algorithm 2, with Adam's bias
// correction from Kingma & Ba, Algorithm 1; named on the pages "Distributed
// optimizer support for BERT", Usage, and "[pure bf16 training] w/
// AnyPrecisionAdamW and Kahan summation", the opt-1.3b command):
//   m = b1*m + (1-b1)*g ; v = b2*v + (1-b2)*(g*g) ; u = m / (sqrt(v*rbc2) + eps)
//   mixed: w = w*decay - step_size*u, p = round16(w)
//   Kahan: d = -(lrwd*p) - step_size*u ; s = c + d ; p' = rbf16(p + s) ; c = rbf16(s - (p' - p))
//          (with an fp32 compensation buffer c = s - (p' - p), unrounded)
// Each operation is one binary32 operation in that order; the library is
// compiled with -ffp-contract=off so no multiply-add is fused, sqrt and
// division are the correctly rounded ones, and fp32 subnormals are kept.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "adamw.h"
#include "layout.hpp"

namespace adamw {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Device addresses taken from the segment table are plain integers; casting them
// to the global address space lets the compiler emit global_load/global_store
// (rather than flat accesses, which also test the LDS aperture).
#define GLOBAL __attribute__((address_space(1)))
template <typename T>
__device__ __forceinline__ GLOBAL T* gptr(uint64_t addr, uint64_t elem_off)
{
    return reinterpret_cast<GLOBAL T*>(addr) + elem_off;
}
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// 16-bit <-> fp32.  A 32-bit word holds two 16-bit elements, the lower-addressed
// one in the low half.
// ---------------------------------------------------------------------------

template <bool F16>
__device__ __forceinline__ f32x2 widen2(uint32_t w)
{
    if constexpr (F16) {
        return __builtin_convertvector(__builtin_bit_cast(f16x2, w), f32x2);   // v_cvt_f32_f16 (exact)
    } else {
        f32x2 r;
        r.x = __uint_as_float(w << 16);            // bf16 is the top half of an fp32
        r.y = __uint_as_float(w & 0xffff0000u);
        return r;
    }
}

// Round two fp32 values to nearest-even 16-bit and pack them (v_cvt_pk_bf16_f32 /
// v_cvt_pk_f16_f32 under the default round-to-nearest-even mode).
template <bool F16>
__device__ __forceinline__ uint32_t narrow2(float lo, float hi)
{
    f32x2 x = {lo, hi};
    if constexpr (F16) return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, f16x2));
    else return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
}

template <bool F16>
__device__ __forceinline__ float widen1(uint16_t h)
{
    if constexpr (F16) return (float)__builtin_bit_cast(_Float16, h);
    else return __uint_as_float((uint32_t)h << 16);
}

template <bool F16>
__device__ __forceinline__ uint16_t narrow1(float x)
{
    if constexpr (F16) return __builtin_bit_cast(uint16_t, (_Float16)x);
    else return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// ---------------------------------------------------------------------------
// Element math
// ---------------------------------------------------------------------------

struct Coef {
    float step_size, rbc2, decay, lrwd, omb1, omb2, beta1, beta2, eps, inv_scale;
};

// Moments and the bias-corrected Adam direction u = m_hat / (sqrt(v_hat) + eps),
// with 1/(1-b1^t) carried by step_size.
__device__ __forceinline__ float adam_dir(float g, float& m, float& v, const Coef& c)
{
    m = c.beta1 * m + c.omb1 * g;
    v = c.beta2 * v + c.omb2 * (g * g);
    return m / (__builtin_sqrtf(v * c.rbc2) + c.eps);
}

// Mixed precision: fp32 master w (in place); returns the new w.
__device__ __forceinline__ float mixed_elem(float g16, float& w, float& m, float& v, const Coef& c)
{
    const float g = g16 * c.inv_scale;
    const float u = adam_dir(g, m, v, c);
    w = w * c.decay - c.step_size * u;
    return w;
}

// Kahan: returns the fp32 sum p + s to be rounded into the new bf16 p, and the
// pending increment s through `s_out`.
__device__ __forceinline__ float kahan_sum(float g16, float pf, float cf, float& m, float& v, const Coef& c,
                                           float& s_out)
{
    const float g = g16 * c.inv_scale;
    const float u = adam_dir(g, m, v, c);
    const float d = -(c.lrwd * pf) - c.step_size * u;
    const float s = cf + d;
    s_out = s;
    return pf + s;
}

// Split master: w's bits = (p << 16) + r, r an int16 (two's complement, mod 2^32).
__device__ __forceinline__ uint32_t join_bits(uint32_t p16, uint32_t r16)
{
    return (p16 << 16) + (uint32_t)(int32_t)(int16_t)(uint16_t)r16;
}

// p = nearest bf16 of w, ties away from zero (bit 15 of the dropped half rounds the
// magnitude up), so the remainder w - (p << 16) lies in [-32768, 32767]; a NaN
// keeps its high half with the quiet bit set.  Returns p; r through `r16`.
// Both candidates are formed and one is picked with a mask: written as a
// conditional, the NaN case compiled to a divergent branch per element.
__device__ __forceinline__ uint32_t split_bits(uint32_t w, uint32_t& r16)
{
    const uint32_t nan_mask = 0u - (uint32_t)((w & 0x7fffffffu) > 0x7f800000u);
    const uint32_t rounded = (w >> 16) + ((w >> 15) & 1u);
    const uint32_t quieted = (w >> 16) | 0x0040u;
    const uint32_t hi = (rounded & ~nan_mask) | (quieted & nan_mask);
    r16 = (w - (hi << 16)) & 0xffffu;
    return hi & 0xffffu;
}

// ---------------------------------------------------------------------------
// Prologue: one lane.  skip = *found_inf != 0; otherwise t = *step + 1, the
// step's scalars, and *step = t.  With a loss-scale state, the unscale factor
// is 1/scale and the state advances by the dynamic loss-scaling rule.
// ---------------------------------------------------------------------------

__device__ double pow_sq(double b, int64_t t)
{
    // beta^t by right-to-left binary powering: square the base every round,
    // multiply it into the result for every set bit of t.
    double r = 1.0;
    for (; t > 0; t >>= 1) {
        if (t & 1) r = r * b;
        b = b * b;
    }
    return r;
}

// The scalars of step t: binary64 from +, -, *, / only, each rounded once to
// binary32.  The prologue kernel and the single-launch form share this code.
__device__ __forceinline__ Coef step_coef(const adamw_hparams& hp, int64_t t, float inv_scale)
{
    const double lr = (double)hp.lr, wd = (double)hp.weight_decay;
    const double b1t = pow_sq((double)hp.beta1, t);
    const double b2t = pow_sq((double)hp.beta2, t);
    Coef c;
    c.step_size = (float)(lr / (1.0 - b1t));
    c.rbc2 = (float)(1.0 / (1.0 - b2t));
    c.decay = (float)(1.0 - lr * wd);
    c.lrwd = (float)(lr * wd);
    c.omb1 = 1.0f - hp.beta1;
    c.omb2 = 1.0f - hp.beta2;
    c.beta1 = hp.beta1;
    c.beta2 = hp.beta2;
    c.eps = hp.eps;
    c.inv_scale = inv_scale;
    return c;
}

// The dynamic loss-scaling rule, applied once per step after the step's
// unscale factor 1/scale has been read: back off on an overflow, grow after
// growth_interval clean steps in a row (a growth that would overflow binary32
// is refused).  One lane of the grid runs it.
__device__ __forceinline__ void advance_loss_scale(adamw_loss_scale_state* amp, const adamw_loss_scaler& scaler,
                                                   float scale, bool skip)
{
    if (skip) {
        amp->scale = scale * scaler.backoff_factor;
        amp->growth_tracker = 0;
    } else {
        const int32_t run = amp->growth_tracker + 1;
        if (run == scaler.growth_interval) {
            const float grown = scale * scaler.growth_factor;
            if (__builtin_isfinite(grown)) amp->scale = grown;
            amp->growth_tracker = 0;
        } else {
            amp->growth_tracker = run;
        }
    }
}

// A step is taken only from a counter in [0, INT32_MAX): the step it takes,
// t = counter + 1, must be a positive int32.  From any other value the call
// writes nothing at all (no buffer, no counter, no loss scale), as on a skip.
__device__ __forceinline__ bool counter_in_range(int32_t step) { return step >= 0 && step != INT32_MAX; }

__global__ void prologue_kernel(adamw_hparams hp, int32_t* __restrict__ step, const int32_t* __restrict__ found_inf,
                                LaunchScalars* __restrict__ out, adamw_loss_scale_state* __restrict__ amp,
                                adamw_loss_scaler scaler)
{
    if (threadIdx.x != 0 || blockIdx.x != 0) return;
    LaunchScalars s{};
    const int32_t step0 = *step;
    if (!counter_in_range(step0)) {
        // no step t = step0 + 1 exists in int32: write nothing but the skip mark
        s.skip = 1;
        *out = s;
        return;
    }
    const bool skip = found_inf && *found_inf != 0;
    float inv_scale = hp.inv_loss_scale;
    if (amp) {
        // this step unscales by the current scale; the scale for the next step
        // follows from the flag
        const float scale = amp->scale;
        inv_scale = (float)(1.0 / (double)scale);
        advance_loss_scale(amp, scaler, scale, skip);
    }
    if (skip) {
        s.skip = 1;
        *out = s;
        return;
    }
    const int64_t t = (int64_t)step0 + 1;
    const Coef c = step_coef(hp, t, inv_scale);
    s.skip = 0;
    s.t = (int32_t)t;
    s.step_size = c.step_size;
    s.rbc2 = c.rbc2;
    s.decay = c.decay;
    s.lrwd = c.lrwd;
    s.omb1 = c.omb1;
    s.omb2 = c.omb2;
    s.beta1 = c.beta1;
    s.beta2 = c.beta2;
    s.eps = c.eps;
    s.inv_scale = c.inv_scale;
    *out = s;
    *step = (int32_t)t;
}

// ---------------------------------------------------------------------------
// Update kernel
// ---------------------------------------------------------------------------

// The cache policy of the streaming accesses per mode: bit 0 = non-temporal
// loads, bit 1 = non-temporal stores (every element is touched exactly once
// per step).
#ifndef ADAMW_NT_MIXED
#define ADAMW_NT_MIXED 2
#endif
// The mixed family loads the gradient, which nothing writes back, non-temporally
// on top of ADAMW_NT_MIXED: measured +2-2.5 % for the mixed and split steps on
// MI355X, while non-temporal loads of the read-modify-write state streams cost 9 %.
#ifndef ADAMW_NT_MIXED_GRAD
#define ADAMW_NT_MIXED_GRAD 1
#endif
// The pure family (every stream alike, the gradient included): non-temporal loads
// and stores while the state is bf16 or has one fp32 moment; in the wide mixes
// (both moments fp32, or an fp32 compensation buffer; the split master)
// non-temporal stores only, measured on MI355X (OPT-1.3B list, blocked state)
// 5-6 % faster with fp32 moments and compensation, 3.5 % with fp32 moments
// alone, and 57 % -> 77 % of peak with bf16 moments and an fp32 compensation
// buffer, while the bf16 Kahan step loses 8 % without non-temporal loads and
// the one-fp32-moment mixes tie.
#ifndef ADAMW_NT_PURE
#define ADAMW_NT_PURE 3
#endif
#ifndef ADAMW_NT_PURE_WIDE
#define ADAMW_NT_PURE_WIDE 2
#endif
#ifndef ADAMW_NT_SPLIT
#define ADAMW_NT_SPLIT 2
#endif
#ifndef ADAMW_NT_CHECK
#define ADAMW_NT_CHECK 1
#endif
constexpr int kCheckUnroll = kCheckChunkMult;

template <int NT, typename T>
__device__ __forceinline__ T ld(const GLOBAL T* p)
{
    if constexpr (NT & 1) return __builtin_nontemporal_load(p);
    else return *p;
}

template <int NT, typename T>
__device__ __forceinline__ void st(GLOBAL T* p, T v)
{
    if constexpr (NT & 2) __builtin_nontemporal_store(v, p);
    else *p = v;
}

// The overflow check's workgroup -> chunk map: xcd_chunk (layout.hpp), under
// which each XCD walks one contiguous run of chunks.
__device__ __forceinline__ uint32_t chunk_index(uint32_t b, uint32_t nb) { return xcd_chunk(b, nb); }

// An update kernel's chunk is processed by kXcdParts consecutive workgroups,
// part = blockIdx.x % kXcdParts running on XCD `part`; lane tid takes the pack
// tile_pack(tid, part, P) (layout.hpp) of every kXcdParts * BLOCK packs of the
// chunk.  Element-wise chunks go to the parts in strides of the workgroup size.
template <int P, int BLOCK>
__device__ __forceinline__ uint32_t first_pack(uint32_t tid, uint32_t part)
{
    static_assert(BLOCK % P == 0, "a workgroup covers whole tiles");
    return tile_pack(tid, part, P);
}

__device__ __forceinline__ Coef load_coef(const LaunchScalars* sc)
{
    Coef c;
    c.step_size = sc->step_size;
    c.rbc2 = sc->rbc2;
    c.decay = sc->decay;
    c.lrwd = sc->lrwd;
    c.omb1 = sc->omb1;
    c.omb2 = sc->omb2;
    c.beta1 = sc->beta1;
    c.beta2 = sc->beta2;
    c.eps = sc->eps;
    c.inv_scale = sc->inv_scale;
    return c;
}

// Start of a step in an update kernel.  Two-launch form: the prologue kernel
// has written the skip flag and the scalars.  Single launch: the workgroup
// reads the flag, the counter and (with a dynamic loss scale) the scale
// itself; its scalars are formed by fused_coef once its data loads are in
// flight.  Returns false on a skipped step (uniform over the grid: nothing is
// written, the counter is kept; workgroup 0 backs the loss scale off) and on a
// counter out of range (nothing is written at all).
template <bool FUSED>
__device__ __forceinline__ bool begin_step(const LaunchScalars* sc, const FusedStep& fs, Coef& c, int64_t& t,
                                           float& scale)
{
    if constexpr (FUSED) {
        // All three reads come before the one store a workgroup may make here,
        // so that the compiler can issue them as scalar loads (a store ahead of
        // a load in the kernel would turn it into a vector load with a full
        // wait before the data loads start).
        const int32_t flag = fs.found_inf ? *fs.found_inf : 0;
        const int32_t step = *fs.step;
        scale = fs.amp ? fs.amp->scale : 0.0f;
        if (!counter_in_range(step)) return false;
        if (flag != 0) {
            if (fs.amp && blockIdx.x == 0 && threadIdx.x == 0) advance_loss_scale(fs.amp, fs.scaler, scale, true);
            return false;
        }
        t = (int64_t)step + 1;   // as the prologue: no int32 overflow in the scalars
    } else {
        if (sc->skip) return false;
        c = load_coef(sc);
    }
    return true;
}

template <bool FUSED>
__device__ __forceinline__ void fused_coef(const FusedStep& fs, int64_t t, float scale, Coef& c)
{
    if constexpr (FUSED) c = step_coef(fs.hp, t, fs.amp ? (float)(1.0 / (double)scale) : fs.hp.inv_loss_scale);
}

// The grid's completion count, shared by the single-launch kernels.  Each
// workgroup counts itself in a first-level counter (b % kDoneLanes); the
// workgroup completing a first-level count rearms it and counts once in the
// second level, and the one completing that rearms it and returns true.
// Spreading the count over separate 256-byte lines keeps the same-address
// atomics, which the memory side serialises, to about nb / kDoneLanes +
// kDoneLanes per launch.  The counts order nothing but reads that every wave
// has consumed before the workgroup's barrier, so the atomics are relaxed:
// acquire-release ones at device scope would write back and invalidate the
// XCD's L2 in every workgroup.
struct DoneLane {
    uint32_t lanes, j, in_lane;
};

__device__ __forceinline__ DoneLane done_lane()
{
    const uint32_t nb = gridDim.x, b = blockIdx.x;
    const uint32_t lanes = nb < (uint32_t)kDoneLanes ? nb : (uint32_t)kDoneLanes;
    const uint32_t j = b % lanes;
    return DoneLane{lanes, j, nb / lanes + (j < nb % lanes ? 1u : 0u)};
}

// The count alone, on 32-bit words (the low words of the counter lines).
__device__ __forceinline__ bool grid_done(uint32_t* done)
{
    const DoneLane d = done_lane();
    uint32_t* first = done + (size_t)d.j * kDoneStrideWords;
    uint32_t* second = done + (size_t)kDoneLanes * kDoneStrideWords;
    if (__hip_atomic_fetch_add(first, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != d.in_lane - 1) return false;
    __hip_atomic_store(first, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (__hip_atomic_fetch_add(second, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != d.lanes - 1) return false;
    __hip_atomic_store(second, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return true;
}

// The count with a 0/1 verdict per workgroup, on 64-bit words: the count in the
// low half and the number of raised verdicts in the high half, so the verdicts
// travel in the atomics' own values.  The completer gets the number of lanes
// with a raised verdict in *lanes_hit.  Both forms leave every counter word at
// zero, so the update and check kernels of one stream share the lines.
__device__ __forceinline__ bool grid_done_verdict(uint32_t* done, uint32_t verdict, uint32_t* lanes_hit)
{
    const DoneLane d = done_lane();
    uint64_t* first = reinterpret_cast<uint64_t*>(done + (size_t)d.j * kDoneStrideWords);
    uint64_t* second = reinterpret_cast<uint64_t*>(done + (size_t)kDoneLanes * kDoneStrideWords);
    const uint64_t prev = __hip_atomic_fetch_add(first, 1ull + ((uint64_t)verdict << 32), __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    if ((uint32_t)prev != d.in_lane - 1) return false;
    __hip_atomic_store(first, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t hit = ((prev >> 32) + verdict) != 0 ? 1ull : 0ull;
    const uint64_t prev2 = __hip_atomic_fetch_add(second, 1ull + (hit << 32), __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
    if ((uint32_t)prev2 != d.lanes - 1) return false;
    __hip_atomic_store(second, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *lanes_hit = (uint32_t)(prev2 >> 32) + (uint32_t)hit;
    return true;
}

// End of a single-launch step: once every wave of this workgroup is past its
// reads of the counter and the loss scale, one lane counts the workgroup; the
// last one of the grid stores the new counter and advances the loss scale.
template <bool FUSED>
__device__ __forceinline__ void end_step(const FusedStep& fs, int64_t t, float scale)
{
    if constexpr (FUSED) {
        __syncthreads();
        if (threadIdx.x == 0 && grid_done(fs.done)) {
            __hip_atomic_store(fs.step, (int32_t)t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (fs.amp) advance_loss_scale(fs.amp, fs.scaler, scale, false);
        }
    }
}

// MODE 0: mixed bf16, 1: mixed fp16 (the split-master step is a pure-family
// kernel below: its param is read as well as written)
template <int MODE, bool FUSED>
__global__ __launch_bounds__(kBlockMixed) void update_kernel(const DevSeg* __restrict__ segs,
                                                        const DevChunk* __restrict__ chunks,
                                                        const LaunchScalars* __restrict__ sc, FusedStep fs)
{
    Coef c{};
    int64_t t = 0;
    float scale = 0.0f;
    if (!begin_step<FUSED>(sc, fs, c, t, scale)) return;
    constexpr bool F16 = (MODE == 1);
    constexpr int NTM = ADAMW_NT_MIXED;
    constexpr int NTG = NTM | (ADAMW_NT_MIXED_GRAD ? 1 : 0);   // the gradient's loads
    constexpr int P = kTilePacksMixed;   // tiles of 256 elements
    constexpr uint32_t kStride = kXcdParts * kBlockMixed;
    const uint32_t part = blockIdx.x % kXcdParts;
    const DevChunk ch = chunks[blockIdx.x / kXcdParts];
    const DevSeg& sg = segs[ch.seg];
    const uint32_t n = ch.n_kind & kCountMask;
    const uint64_t off = ch.off;
    const uint32_t tid = threadIdx.x;

    GLOBAL uint16_t* __restrict__ p = gptr<uint16_t>(sg.ptr[ADAMW_STREAM_PARAM], off);
    const GLOBAL uint16_t* __restrict__ g = gptr<const uint16_t>(sg.ptr[ADAMW_STREAM_GRAD], off);
    GLOBAL float* __restrict__ m = gptr<float>(sg.ptr[ADAMW_STREAM_EXP_AVG], off);
    GLOBAL float* __restrict__ v = gptr<float>(sg.ptr[ADAMW_STREAM_EXP_AVG_SQ], off);
    GLOBAL float* __restrict__ w = gptr<float>(sg.ptr[ADAMW_STREAM_AUX], off);
    if (ch.n_kind & kVecBit) {
        const uint32_t npack = n / kPack;
        const GLOBAL u32x4* __restrict__ g4 = reinterpret_cast<const GLOBAL u32x4*>(g);
        GLOBAL u32x4* __restrict__ p4 = reinterpret_cast<GLOBAL u32x4*>(p);
        GLOBAL f32x4* __restrict__ m4 = reinterpret_cast<GLOBAL f32x4*>(m);
        GLOBAL f32x4* __restrict__ v4 = reinterpret_cast<GLOBAL f32x4*>(v);
        GLOBAL f32x4* __restrict__ w4 = reinterpret_cast<GLOBAL f32x4*>(w);
        for (uint32_t k = first_pack<P, kBlockMixed>(tid, part); k < npack; k += kStride) {
            const u32x4 G = ld<NTG>(g4 + k);
            f32x4 W[2] = {ld<NTM>(w4 + 2 * k), ld<NTM>(w4 + 2 * k + 1)};
            f32x4 M[2] = {ld<NTM>(m4 + 2 * k), ld<NTM>(m4 + 2 * k + 1)};
            f32x4 V[2] = {ld<NTM>(v4 + 2 * k), ld<NTM>(v4 + 2 * k + 1)};
            fused_coef<FUSED>(fs, t, scale, c);   // while the loads are in flight
            float* wf = reinterpret_cast<float*>(W);
            float* mf = reinterpret_cast<float*>(M);
            float* vf = reinterpret_cast<float*>(V);
            const uint32_t gw[4] = {G.x, G.y, G.z, G.w};
            uint32_t pw[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x2 gg = widen2<F16>(gw[j]);
                const float a = mixed_elem(gg.x, wf[2 * j], mf[2 * j], vf[2 * j], c);
                const float b = mixed_elem(gg.y, wf[2 * j + 1], mf[2 * j + 1], vf[2 * j + 1], c);
                pw[j] = narrow2<F16>(a, b);
            }
            st<NTM>(w4 + 2 * k, W[0]); st<NTM>(w4 + 2 * k + 1, W[1]);
            st<NTM>(m4 + 2 * k, M[0]); st<NTM>(m4 + 2 * k + 1, M[1]);
            st<NTM>(v4 + 2 * k, V[0]); st<NTM>(v4 + 2 * k + 1, V[1]);
            st<NTM>(p4 + k, u32x4{pw[0], pw[1], pw[2], pw[3]});
        }
    } else {
        fused_coef<FUSED>(fs, t, scale, c);
        for (uint32_t i = part * kBlockMixed + tid; i < n; i += kStride) {
            float wi = w[i], mi = m[i], vi = v[i];
            const float nw = mixed_elem(widen1<F16>(g[i]), wi, mi, vi, c);
            w[i] = wi;
            m[i] = mi;
            v[i] = vi;
            p[i] = narrow1<F16>(nw);
        }
    }
    end_step<FUSED>(fs, t, scale);
}

// The aux stream of a pure-family step.
constexpr int kAuxNone = 0;    // no aux stream: p' = round(p * decay - step_size * u)
constexpr int kAuxKahan = 1;   // bf16 Kahan compensation c
constexpr int kAuxSplit = 2;   // int16 remainder r of the split fp32 master w = join(p, r)
constexpr int kAuxKahan32 = 3; // fp32 Kahan compensation c (the residual kept unrounded)

// Steps whose param is read as well as written, over bf16 params: the pure-bf16
// family with chosen state precisions (M32 / V32 = fp32 exp_avg / exp_avg_sq,
// else bf16; aux none, bf16 or fp32 compensation; <false, false, kAuxKahan> is
// the pure-bf16 Kahan mode), and the split-master mixed step (<true, true,
// kAuxSplit>).
template <bool M32, bool V32, int AUX, bool FUSED>
__global__ __launch_bounds__(kBlockPure) void update_pure_kernel(const DevSeg* __restrict__ segs,
                                                                            const DevChunk* __restrict__ chunks,
                                                                            const LaunchScalars* __restrict__ sc,
                                                                            FusedStep fs)
{
    Coef c{};
    int64_t t = 0;
    float scale = 0.0f;
    if (!begin_step<FUSED>(sc, fs, c, t, scale)) return;
    constexpr bool KAHAN = AUX == kAuxKahan, SPLIT = AUX == kAuxSplit, KAHAN32 = AUX == kAuxKahan32;
    static_assert(!SPLIT || (M32 && V32), "the split master keeps fp32 moments");
    // The wide pure-family mixes (both moments in fp32, or an fp32
    // compensation buffer: 8-14 B of state per element, half or more of it in
    // fp32 streams): non-temporal stores only and the mixed family's occupancy.
    constexpr bool WIDE = (M32 && V32) || KAHAN32;
    constexpr int NT = SPLIT ? ADAMW_NT_SPLIT : WIDE ? ADAMW_NT_PURE_WIDE : ADAMW_NT_PURE;
    // tiles of 256 elements (split master) or 512 (the rest)
    constexpr int P = SPLIT ? kTilePacksSplit : WIDE ? kTilePacksPureWide : kTilePacks;
    constexpr uint32_t kStride = kXcdParts * kBlockPure;
    const uint32_t part = blockIdx.x % kXcdParts;
    const DevChunk ch = chunks[blockIdx.x / kXcdParts];
    const DevSeg& sg = segs[ch.seg];
    const uint32_t n = ch.n_kind & kCountMask;
    const uint64_t off = ch.off;
    const uint32_t tid = threadIdx.x;
    using MT = typename std::conditional<M32, float, uint16_t>::type;
    using VT = typename std::conditional<V32, float, uint16_t>::type;
    GLOBAL uint16_t* __restrict__ p = gptr<uint16_t>(sg.ptr[ADAMW_STREAM_PARAM], off);
    const GLOBAL uint16_t* __restrict__ g = gptr<const uint16_t>(sg.ptr[ADAMW_STREAM_GRAD], off);
    GLOBAL MT* __restrict__ m = gptr<MT>(sg.ptr[ADAMW_STREAM_EXP_AVG], off);
    GLOBAL VT* __restrict__ v = gptr<VT>(sg.ptr[ADAMW_STREAM_EXP_AVG_SQ], off);
    using CT = typename std::conditional<KAHAN32, float, uint16_t>::type;
    GLOBAL CT* __restrict__ cc = gptr<CT>(sg.ptr[ADAMW_STREAM_AUX], off);

    if (ch.n_kind & kVecBit) {
        const uint32_t npack = n / kPack;
        const GLOBAL u32x4* __restrict__ g4 = reinterpret_cast<const GLOBAL u32x4*>(g);
        GLOBAL u32x4* __restrict__ p4 = reinterpret_cast<GLOBAL u32x4*>(p);
        GLOBAL u32x4* __restrict__ c4 = reinterpret_cast<GLOBAL u32x4*>(cc);
        // a pack of 8 moments (or compensations) is one dwordx4 in bf16, two in fp32
        constexpr int MW = M32 ? 2 : 1, VW = V32 ? 2 : 1, CW = KAHAN32 ? 2 : 1;
        GLOBAL u32x4* __restrict__ m4 = reinterpret_cast<GLOBAL u32x4*>(m);
        GLOBAL u32x4* __restrict__ v4 = reinterpret_cast<GLOBAL u32x4*>(v);
        for (uint32_t k = first_pack<P, kBlockPure>(tid, part); k < npack; k += kStride) {
            const u32x4 G = ld<NT>(g4 + k), Pv = ld<NT>(p4 + k);
            u32x4 C[CW], M[MW], V[VW];
#pragma unroll
            for (int q = 0; q < MW; ++q) M[q] = ld<NT>(m4 + MW * k + q);
#pragma unroll
            for (int q = 0; q < VW; ++q) V[q] = ld<NT>(v4 + VW * k + q);
            if constexpr (AUX != kAuxNone) {
#pragma unroll
                for (int q = 0; q < CW; ++q) C[q] = ld<NT>(c4 + CW * k + q);
            }
            fused_coef<FUSED>(fs, t, scale, c);   // while the loads are in flight
            const uint32_t* gw = reinterpret_cast<const uint32_t*>(&G);
            const uint32_t* pw = reinterpret_cast<const uint32_t*>(&Pv);
            uint32_t* cw = reinterpret_cast<uint32_t*>(C);   // 4 (bf16) or 8 (fp32) words
            uint32_t* mw = reinterpret_cast<uint32_t*>(M);   // 4 (bf16) or 8 (fp32) words
            uint32_t* vw = reinterpret_cast<uint32_t*>(V);
            uint32_t po[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x2 gg = widen2<false>(gw[j]);
                const f32x2 pp = widen2<false>(pw[j]);
                float ma, mb, va, vb;
                if constexpr (M32) {
                    ma = __uint_as_float(mw[2 * j]);
                    mb = __uint_as_float(mw[2 * j + 1]);
                } else {
                    const f32x2 t2 = widen2<false>(mw[j]);
                    ma = t2.x;
                    mb = t2.y;
                }
                if constexpr (V32) {
                    va = __uint_as_float(vw[2 * j]);
                    vb = __uint_as_float(vw[2 * j + 1]);
                } else {
                    const f32x2 t2 = widen2<false>(vw[j]);
                    va = t2.x;
                    vb = t2.y;
                }
                if constexpr (SPLIT) {
                    float wa = __uint_as_float(join_bits(pw[j] & 0xffffu, cw[j] & 0xffffu));
                    float wb = __uint_as_float(join_bits(pw[j] >> 16, cw[j] >> 16));
                    mixed_elem(gg.x, wa, ma, va, c);
                    mixed_elem(gg.y, wb, mb, vb, c);
                    uint32_t ra, rb;
                    const uint32_t pa = split_bits(__float_as_uint(wa), ra);
                    const uint32_t pb = split_bits(__float_as_uint(wb), rb);
                    po[j] = pa | (pb << 16);
                    cw[j] = ra | (rb << 16);
                } else if constexpr (KAHAN) {
                    const f32x2 cf = widen2<false>(cw[j]);
                    float sa, sb;
                    const float ta = kahan_sum(gg.x, pp.x, cf.x, ma, va, c, sa);
                    const float tb = kahan_sum(gg.y, pp.y, cf.y, mb, vb, c, sb);
                    po[j] = narrow2<false>(ta, tb);
                    const f32x2 pn = widen2<false>(po[j]);
                    cw[j] = narrow2<false>(sa - (pn.x - pp.x), sb - (pn.y - pp.y));
                } else if constexpr (KAHAN32) {
                    float sa, sb;
                    const float ta = kahan_sum(gg.x, pp.x, __uint_as_float(cw[2 * j]), ma, va, c, sa);
                    const float tb = kahan_sum(gg.y, pp.y, __uint_as_float(cw[2 * j + 1]), mb, vb, c, sb);
                    po[j] = narrow2<false>(ta, tb);
                    const f32x2 pn = widen2<false>(po[j]);
                    cw[2 * j] = __float_as_uint(sa - (pn.x - pp.x));
                    cw[2 * j + 1] = __float_as_uint(sb - (pn.y - pp.y));
                } else {
                    float wa = pp.x, wb = pp.y;
                    mixed_elem(gg.x, wa, ma, va, c);
                    mixed_elem(gg.y, wb, mb, vb, c);
                    po[j] = narrow2<false>(wa, wb);
                }
                if constexpr (M32) {
                    mw[2 * j] = __float_as_uint(ma);
                    mw[2 * j + 1] = __float_as_uint(mb);
                } else {
                    mw[j] = narrow2<false>(ma, mb);
                }
                if constexpr (V32) {
                    vw[2 * j] = __float_as_uint(va);
                    vw[2 * j + 1] = __float_as_uint(vb);
                } else {
                    vw[j] = narrow2<false>(va, vb);
                }
            }
            st<NT>(p4 + k, u32x4{po[0], po[1], po[2], po[3]});
#pragma unroll
            for (int q = 0; q < MW; ++q) st<NT>(m4 + MW * k + q, M[q]);
#pragma unroll
            for (int q = 0; q < VW; ++q) st<NT>(v4 + VW * k + q, V[q]);
            if constexpr (AUX != kAuxNone) {
#pragma unroll
                for (int q = 0; q < CW; ++q) st<NT>(c4 + CW * k + q, C[q]);
            }
        }
    } else {
        fused_coef<FUSED>(fs, t, scale, c);
        for (uint32_t i = part * kBlockPure + tid; i < n; i += kStride) {
            const float pf = widen1<false>(p[i]);
            float mi, vi;
            if constexpr (M32) mi = m[i]; else mi = widen1<false>(m[i]);
            if constexpr (V32) vi = v[i]; else vi = widen1<false>(v[i]);
            const float gi = widen1<false>(g[i]);
            if constexpr (SPLIT) {
                float w = __uint_as_float(join_bits(p[i], cc[i]));
                mixed_elem(gi, w, mi, vi, c);
                uint32_t ri;
                const uint32_t pi = split_bits(__float_as_uint(w), ri);
                p[i] = (uint16_t)pi;
                cc[i] = (uint16_t)ri;
            } else if constexpr (KAHAN) {
                float s;
                const float tot = kahan_sum(gi, pf, widen1<false>(cc[i]), mi, vi, c, s);
                const uint16_t pn = narrow1<false>(tot);
                cc[i] = narrow1<false>(s - (widen1<false>(pn) - pf));
                p[i] = pn;
            } else if constexpr (KAHAN32) {
                float s;
                const float tot = kahan_sum(gi, pf, cc[i], mi, vi, c, s);
                const uint16_t pn = narrow1<false>(tot);
                cc[i] = s - (widen1<false>(pn) - pf);
                p[i] = pn;
            } else {
                float w = pf;
                mixed_elem(gi, w, mi, vi, c);
                p[i] = narrow1<false>(w);
            }
            if constexpr (M32) m[i] = mi; else m[i] = narrow1<false>(mi);
            if constexpr (V32) v[i] = vi; else v[i] = narrow1<false>(vi);
        }
    }
    end_step<FUSED>(fs, t, scale);
}

// ---------------------------------------------------------------------------
// Overflow check
// ---------------------------------------------------------------------------

__global__ void zero_flag_kernel(int32_t* __restrict__ flag)
{
    if (threadIdx.x == 0 && blockIdx.x == 0) *flag = 0;
}

// Nonzero iff one of the two 16-bit elements in w has an all-ones exponent
// field (EXP = 0x7c00 for fp16, 0x7f80 for bf16).
template <uint32_t EXP>
__device__ __forceinline__ uint32_t nonfinite2(uint32_t w)
{
    const uint32_t x = ~w & (EXP | (EXP << 16));
    return (uint32_t)((x & 0xffffu) == 0) | (uint32_t)((x >> 16) == 0);
}

// FUSED: a single launch that also replaces the zeroing of the flag: the
// workgroups count themselves with their verdicts (grid_done_verdict), and the last
// one stores the flag, 1 if any workgroup saw a non-finite value, else 0.
template <bool F16, bool FUSED>
__global__ __launch_bounds__(kBlockCheck) void check_kernel(const DevSeg* __restrict__ segs,
                                                       const DevChunk* __restrict__ chunks,
                                                       int32_t* __restrict__ flag, uint32_t* __restrict__ done)
{
    constexpr uint32_t EXP = F16 ? 0x7c00u : 0x7f80u;
    const DevChunk ch = chunks[chunk_index(blockIdx.x, gridDim.x)];
    const GLOBAL uint16_t* __restrict__ g = gptr<const uint16_t>(segs[ch.seg].ptr[ADAMW_STREAM_GRAD], ch.off);
    const uint32_t n = ch.n_kind & kCountMask;
    uint32_t bad = 0;
    if (ch.n_kind & kVecBit) {
        // each lane issues kCheckUnroll loads before testing any: one pass
        // covers a default check chunk
        const GLOBAL u32x4* __restrict__ g4 = reinterpret_cast<const GLOBAL u32x4*>(g);
        const uint32_t npack = n / kPack;
        for (uint32_t k0 = threadIdx.x; k0 < npack; k0 += kBlockCheck * kCheckUnroll) {
            u32x4 q[kCheckUnroll];
#pragma unroll
            for (int u = 0; u < kCheckUnroll; ++u) {
                const uint32_t k = k0 + u * kBlockCheck;
                q[u] = k < npack ? ld<ADAMW_NT_CHECK>(g4 + k) : u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int u = 0; u < kCheckUnroll; ++u)
                bad |= nonfinite2<EXP>(q[u].x) | nonfinite2<EXP>(q[u].y) | nonfinite2<EXP>(q[u].z) |
                       nonfinite2<EXP>(q[u].w);
        }
    } else {
        for (uint32_t i = threadIdx.x; i < n; i += kBlockCheck) bad |= (uint32_t)((g[i] & EXP) == EXP);
    }
    if constexpr (FUSED) {
        const int any = __syncthreads_or((int)bad);
        uint32_t hit = 0;
        if (threadIdx.x == 0 && grid_done_verdict(done, any ? 1u : 0u, &hit))
            __hip_atomic_store(flag, hit ? 1 : 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
        // one atomic per wavefront that saw a non-finite value
        if (__any((int)bad) && (threadIdx.x % warpSize) == 0)
            __hip_atomic_fetch_or(flag, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------

hipError_t launch_prologue(const adamw_hparams& hp, int32_t* d_step, const int32_t* d_found_inf,
                           LaunchScalars* d_scalars, adamw_loss_scale_state* d_amp, const adamw_loss_scaler& scaler,
                           hipStream_t stream)
{
    hipLaunchKernelGGL(prologue_kernel, dim3(1), dim3(64), 0, stream, hp, d_step, d_found_inf, d_scalars, d_amp,
                       scaler);
    return hipGetLastError();
}

// Occupancy cap, per kernel family: the update kernels use no LDS, but
// reserving this much per workgroup leaves room for only 160 KiB / bytes
// workgroups on a CU.  Measured on MI355X with the OPT-1.3B list, 8 waves per CU
// (mixed: two 256-lane workgroups) and 16 (pure: four 256-lane workgroups)
// stream faster than the register-limited 20-32 waves: fewer concurrent address
// streams per CU keep more DRAM rows open.  The wide pure-bf16 mixes (both
// moments fp32, or an fp32 compensation buffer) run at the mixed family's 8
// waves: 4 % faster than at 16 with fp32 moments and compensation on blocked
// state, while the bf16-state steps lost 2-5 % at 8.
#ifndef ADAMW_LDS_MIXED
#define ADAMW_LDS_MIXED 81920
#endif
#ifndef ADAMW_LDS_PURE
#define ADAMW_LDS_PURE 40960
#endif
#ifndef ADAMW_LDS_PURE_WIDE
#define ADAMW_LDS_PURE_WIDE 81920
#endif
#ifndef ADAMW_LDS_SPLIT
#define ADAMW_LDS_SPLIT 81920
#endif

// Two-launch form (fused == nullptr): the update kernel reads the prologue's
// scalars at d_scalars.  Single launch: the kernel forms them from *fused.
template <bool FUSED>
static hipError_t launch_update_as(int kernel, const DevSeg* segs, const DevChunk* chunks, int64_t n_chunks,
                                   const LaunchScalars* d_scalars, const FusedStep& fs, hipStream_t stream)
{
    // kXcdParts workgroups per chunk (the plan's chunk limit keeps the grid in range)
    const dim3 grid((unsigned)(n_chunks * kXcdParts)), block(kBlockMixed), block_pure(kBlockPure);
    switch (kernel) {
    case kKernelMixedBf16:
        hipLaunchKernelGGL((update_kernel<0, FUSED>), grid, block, ADAMW_LDS_MIXED, stream, segs, chunks, d_scalars, fs);
        break;
    case kKernelMixedF16:
        hipLaunchKernelGGL((update_kernel<1, FUSED>), grid, block, ADAMW_LDS_MIXED, stream, segs, chunks, d_scalars, fs);
        break;
    case kKernelSplit:
        hipLaunchKernelGGL((update_pure_kernel<true, true, kAuxSplit, FUSED>), grid, block_pure, ADAMW_LDS_SPLIT, stream,
                           segs, chunks, d_scalars, fs);
        break;
#define ADAMW_PURE_CASE(M, V, K)                                                                          \
    case kKernelPure + (M) * 4 + (V) * 2 + (K):                                                            \
        hipLaunchKernelGGL((update_pure_kernel<M, V, (K) ? kAuxKahan : kAuxNone, FUSED>), grid, block_pure,    \
                           (M) && (V) ? ADAMW_LDS_PURE_WIDE : ADAMW_LDS_PURE, stream, segs,                     \
                           chunks, d_scalars, fs);                                                         \
        break;
        ADAMW_PURE_CASE(0, 0, 0) ADAMW_PURE_CASE(0, 0, 1) ADAMW_PURE_CASE(0, 1, 0) ADAMW_PURE_CASE(0, 1, 1)
        ADAMW_PURE_CASE(1, 0, 0) ADAMW_PURE_CASE(1, 0, 1) ADAMW_PURE_CASE(1, 1, 0) ADAMW_PURE_CASE(1, 1, 1)
#undef ADAMW_PURE_CASE
#define ADAMW_PURE_C32_CASE(M, V)                                                                         \
    case kKernelPureC32 + (M) * 2 + (V):                                                                   \
        hipLaunchKernelGGL((update_pure_kernel<M, V, kAuxKahan32, FUSED>), grid, block_pure,                 \
                           ADAMW_LDS_PURE_WIDE, stream, segs, chunks, d_scalars, fs);                     \
        break;
        ADAMW_PURE_C32_CASE(0, 0) ADAMW_PURE_C32_CASE(0, 1) ADAMW_PURE_C32_CASE(1, 0) ADAMW_PURE_C32_CASE(1, 1)
#undef ADAMW_PURE_C32_CASE
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_update(int kernel, const DevSeg* segs, const DevChunk* chunks, int64_t n_chunks,
                         const LaunchScalars* d_scalars, const FusedStep* fused, hipStream_t stream)
{
    if (n_chunks <= 0) return hipSuccess;
    if (fused) return launch_update_as<true>(kernel, segs, chunks, n_chunks, nullptr, *fused, stream);
    return launch_update_as<false>(kernel, segs, chunks, n_chunks, d_scalars, FusedStep{}, stream);
}

// ---------------------------------------------------------------------------
// State copy between per-tensor (or flat) state buffers and the blocked buffer
// ---------------------------------------------------------------------------

// One workgroup per chunk of the copy plan: the chunk's elements of each state
// stream, element by element (the two sides need not share their alignment).
template <typename T>
__device__ __forceinline__ void copy_elems(uint64_t dst, uint64_t src, uint64_t off, uint32_t n)
{
    GLOBAL T* __restrict__ d = gptr<T>(dst, off);
    const GLOBAL T* __restrict__ s = gptr<const T>(src, off);
    for (uint32_t i = threadIdx.x; i < n; i += blockDim.x) d[i] = s[i];
}

__global__ __launch_bounds__(kBlockCopy) void state_copy_kernel(const DevCopySeg* __restrict__ segs,
                                                         const DevChunk* __restrict__ chunks, int esz_m, int esz_v,
                                                         int esz_aux, int to_blocked)
{
    const DevChunk ch = chunks[blockIdx.x];
    const DevCopySeg& sg = segs[ch.seg];
    const uint32_t n = ch.n_kind & kCountMask;
    const int esz[3] = {esz_m, esz_v, esz_aux};
    for (int s = 0; s < 3; ++s) {
        const uint64_t dst = to_blocked ? sg.blocked_side[s] : sg.tensor_side[s];
        const uint64_t src = to_blocked ? sg.tensor_side[s] : sg.blocked_side[s];
        if (esz[s] == 4) copy_elems<uint32_t>(dst, src, ch.off, n);
        else if (esz[s] == 2) copy_elems<uint16_t>(dst, src, ch.off, n);
    }
}

hipError_t launch_state_copy(const DevCopySeg* segs, const DevChunk* chunks, int64_t n_chunks, const int esz[3],
                             bool to_blocked, hipStream_t stream)
{
    if (n_chunks <= 0) return hipSuccess;
    hipLaunchKernelGGL(state_copy_kernel, dim3((unsigned)n_chunks), dim3(kBlockCopy), 0, stream, segs, chunks, esz[0],
                       esz[1], esz[2], to_blocked ? 1 : 0);
    return hipGetLastError();
}

__global__ void zero_words_kernel(uint32_t* __restrict__ p, int64_t n)
{
    for (int64_t i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0u;
}

// Zeroes n 32-bit words (a fill kernel rather than a memset, so that it may
// sit in a captured graph).
hipError_t launch_zero_words(uint32_t* p, int64_t n, hipStream_t stream)
{
    hipLaunchKernelGGL(zero_words_kernel, dim3(1), dim3(256), 0, stream, p, n);
    return hipGetLastError();
}

// fused: one launch of the check (it stores the flag itself, through the
// completion counters at done); else zero the flag, then the check ORs into it.
hipError_t launch_check(adamw_dtype g_dtype, const DevSeg* segs, const DevChunk* chunks, int64_t n_chunks,
                        int32_t* d_flag, uint32_t* done, bool fused, hipStream_t stream)
{
    const dim3 grid((unsigned)(n_chunks > 0 ? n_chunks : 1)), block(kBlockCheck);
    if (fused && n_chunks > 0) {
        if (g_dtype == ADAMW_F16)
            hipLaunchKernelGGL((check_kernel<true, true>), grid, block, 0, stream, segs, chunks, d_flag, done);
        else
            hipLaunchKernelGGL((check_kernel<false, true>), grid, block, 0, stream, segs, chunks, d_flag, done);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(zero_flag_kernel, dim3(1), dim3(64), 0, stream, d_flag);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || n_chunks <= 0) return e;
    if (g_dtype == ADAMW_F16)
        hipLaunchKernelGGL((check_kernel<true, false>), grid, block, 0, stream, segs, chunks, d_flag, nullptr);
    else
        hipLaunchKernelGGL((check_kernel<false, false>), grid, block, 0, stream, segs, chunks, d_flag, nullptr);
    return hipGetLastError();
}

}  // namespace adamw
