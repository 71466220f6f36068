/*
 * adamw.h -- C ABI of the MI355X (gfx950) fused AdamW optimizer step.
 *
 * One call updates a whole list of parameter tensors (or one data-parallel
 * rank's share of it) in place on the GPU: one HBM pass over param, grad,
 * exp_avg, exp_avg_sq and an auxiliary buffer, with the arithmetic in fp32
 * registers.
 *
 * The operation.  AdamW: Adam's bias-corrected moment estimates (Kingma & Ba,
 * "Adam", ICLR 2015, Algorithm 1) with weight decay decoupled from the
 * gradient (Loshchilov & Hutter, "Decoupled Weight Decay Regularization",
 * ICLR 2019, Algorithm 2).  The pages that motivate this library name it and
 * its settings without printing the rule: "Distributed optimizer support for
 * BERT" (Usage: fused_adam / distributed_fused_adam; the A40 and A100 tables,
 * "BF16 with O2 optimizations") and "[pure bf16 training] w/ AnyPrecisionAdamW
 * and Kahan summation" (the opt-1.3b command: lr 0.0002, betas 0.9/0.95,
 * weight decay 0.1; --optim_args with bf16 momentum, variance and Kahan
 * compensation buffer).  With t the 1-based index of the step being taken:
 *
 *   g   = grad * inv_loss_scale
 *   m   = beta1*m + (1-beta1)*g
 *   v   = beta2*v + (1-beta2)*g*g
 *   u   = m / (sqrt(v / (1-beta2^t)) + eps)
 *   ADAMW_MIXED:      w = w*(1 - lr*wd) - (lr/(1-beta1^t))*u;  param = round16(w)
 *   ADAMW_PURE_KAHAN: d = -(lr*wd)*p - (lr/(1-beta1^t))*u
 *                     s = c + d;  p' = round_bf16(p + s);  c = round_bf16(s - (p' - p))
 *   ADAMW_MIXED_SPLIT: the ADAMW_MIXED rule on w = join(param, remainder), then
 *                     (param, remainder) = split(w), where join(p, r) is the fp32 whose
 *                     bit pattern is (p << 16) + r in 32-bit two's complement (r read as
 *                     int16) and split(w) takes p = w's nearest bf16, ties away from zero
 *                     (so r = w - (p << 16) always fits int16), and p = w's high half with
 *                     the quiet bit set for a NaN w.  join(split(w)) == w for every
 *                     non-NaN w, so the master is exact fp32 (a reading of the 16-bit
 *                     master copy counted in the ZeRO saving estimate of "Distributed
 *                     optimizer support for BERT").
 *
 * Numerics: every element operation is one IEEE binary32 operation rounded to
 * nearest even, in the order written above, without fused multiply-add;
 * sqrt and division are correctly rounded; subnormals are kept.  The
 * per-launch scalars 1/(1-beta1^t) etc. are formed in binary64 from +,-,*,/
 * (beta^t by right-to-left square-and-multiply) and rounded once to fp32.
 * Narrowing to bf16/fp16 rounds to nearest even.
 *
 * Streams.  Index s of the five per-element buffers:
 *   0 param       ADAMW_MIXED: bf16 or fp16 (= p_dtype), written only
 *                 ADAMW_PURE_KAHAN: bf16, read and written
 *   1 grad        same 16-bit dtype as param; read only, never unscaled in place
 *   2 exp_avg     ADAMW_MIXED: fp32 / ADAMW_PURE_KAHAN: bf16 (first moment m)
 *   3 exp_avg_sq  ADAMW_MIXED: fp32 / ADAMW_PURE_KAHAN: bf16 (second moment v)
 *   4 aux         ADAMW_MIXED: fp32 master weight w / ADAMW_PURE_KAHAN: bf16
 *                 compensation c / ADAMW_MIXED_SPLIT: int16 remainder of the master
 *   (ADAMW_MIXED_SPLIT: param is bf16 and read as well as written; exp_avg and
 *   exp_avg_sq are fp32.)
 * Every buffer is contiguous, 1-D, in device memory, aligned to its element
 * size.  16-byte alignment is not required but is what the fast path uses;
 * misaligned heads and tails are peeled, and a segment whose streams cannot
 * be aligned together is processed element by element.
 *
 * Step counter and skip flag.  *d_step (device int32) is the number of steps
 * taken so far; a step that is taken uses t = *d_step + 1 and stores t.  If
 * d_found_inf is non-null and *d_found_inf != 0 when the step runs (stream
 * order), nothing is written at all and *d_step is left as it is: the fp16
 * loss-scaling skip.  The caller fills the flag with adamw_check_finite.
 * The counter must lie in [0, INT32_MAX) when the step runs: at INT32_MAX (or
 * below 0) no step t fits in int32, and the call writes nothing at all -- no
 * buffer, no counter, no loss scale -- so the parameters stay finite and a
 * caller can detect the saturated counter by reading it.
 *
 * Ownership and execution.  The caller owns every tensor, d_step, d_found_inf
 * and the stream; the library never frees or reallocates them.  All work is
 * enqueued on hip_stream (a hipStream_t; NULL = the null stream of the calling
 * thread's current device) and the call returns without synchronising.  Every
 * buffer must live on the stream's device.  The library owns only a small
 * device workspace per (device, stream), on the stream's device, holding the
 * launch scalars, the single-launch completion counters (about 8.7 KB) and the
 * chunk table, grown on demand and kept until adamw_release_workspace().  The
 * host arrays inside adamw_tensor_list are read during the call only.
 *
 * HIP graphs.  After one call on a stream with a given list (which allocates
 * the workspace and uploads the list's chunk table), the same call captured on
 * that stream records kernel launches only: no allocation, copy or memset.  A
 * call under capture whose table is not yet on the device (or on a stream
 * without a workspace) is refused with ADAMW_E_INVALID.  A captured step may be
 * replayed any number of times.  It uses the capture stream's workspace
 * (launch scalars, completion counters, chunk table).  The chunk table a
 * capture used is pinned: later calls on the stream, with however many other
 * lists, never evict, move or rewrite it (the stream keeps up to 8 unpinned
 * tables besides the pinned ones); pinned tables are freed only by
 * adamw_release_workspace(), which therefore must not run while such a graph
 * is in use.  A replay must not overlap other work that uses that workspace:
 * steps enqueued on the capture stream, or replays of other graphs captured on
 * it.  Replaying on the capture stream itself keeps all of these in stream
 * order.
 *
 * Errors.  Arguments are validated before anything is enqueued; on an error
 * nothing is enqueued, no buffer is touched, and adamw_last_error() describes
 * it.  A HIP failure while enqueuing returns ADAMW_E_HIP.  Faults inside a
 * kernel surface at the caller's next synchronisation.  One launch's grid
 * holds at most 2^32 - 1 lanes, so a step plan of more than 2,097,151 chunks
 * (8 workgroups of 256 lanes each: about 34e9 elements at the default chunk,
 * or that many tensors of under 8 elements), or a check plan of more than
 * 16,777,215, is rejected with ADAMW_E_INVALID.
 *
 * Concurrency.  Calls may come from several host threads.  Calls on different
 * streams run independently (each stream has its own workspace); two calls
 * must not update the same buffers concurrently.
 */
#ifndef ADAMW_H
#define ADAMW_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ADAMW_ABI_VERSION 8

typedef enum {
    ADAMW_OK = 0,
    ADAMW_E_INVALID = 1,      /* bad argument: null, negative size, range, alignment, hyper-parameter */
    ADAMW_E_UNSUPPORTED = 2,  /* mode / dtype combination not provided */
    ADAMW_E_NOMEM = 3,        /* workspace allocation failed */
    ADAMW_E_HIP = 4           /* a HIP call failed while enqueuing */
} adamw_status;

typedef enum { ADAMW_F32 = 0, ADAMW_BF16 = 1, ADAMW_F16 = 2 } adamw_dtype;

typedef enum {
    ADAMW_MIXED = 0,       /* 16-bit param/grad (bf16 or fp16) + fp32 master, exp_avg, exp_avg_sq */
    ADAMW_PURE_KAHAN = 1,  /* bf16 param, grad, exp_avg, exp_avg_sq + bf16 Kahan compensation */
    ADAMW_MIXED_SPLIT = 2  /* ADAMW_MIXED with the fp32 master split into the bf16 param and an
                              int16 remainder: 14 B/param resident instead of 16, 26 B moved */
} adamw_mode;

enum {
    ADAMW_STREAM_PARAM = 0,
    ADAMW_STREAM_GRAD = 1,
    ADAMW_STREAM_EXP_AVG = 2,
    ADAMW_STREAM_EXP_AVG_SQ = 3,
    ADAMW_STREAM_AUX = 4,
    ADAMW_NUM_STREAMS = 5
};

/* Hyper-parameters, as fp32.  Requirements: all finite; 0 <= beta1, beta2 < 1;
 * eps >= 0; lr >= 0; weight_decay >= 0; inv_loss_scale > 0 (1.0f = no
 * unscaling; 1/65536 for fp16 loss scale 65536). */
typedef struct {
    float lr;
    float beta1;
    float beta2;
    float eps;
    float weight_decay;
    float inv_loss_scale;
} adamw_hparams;

/* A ragged list of tensors, optionally restricted to one data-parallel rank's
 * ZeRO shard: the elements [shard_begin, shard_end) of the list's flat
 * concatenation in list order (the optimizer-state sharding of "Distributed
 * optimizer support for BERT": each rank keeps and updates 1/DP of the
 * state).  Tensors may straddle the shard's edges; only their elements inside
 * the range are touched.  shard_begin = 0, shard_end = -1 means the whole list.
 *
 * ptr[s] is a host array of device pointers for stream s:
 *   flat_mask bit s == 0: ptr[s][i] is tensor i's buffer (numel[i] elements);
 *   flat_mask bit s == 1: ptr[s][0] is ONE flat buffer of shard_end-shard_begin
 *                         elements holding this rank's share, element 0 being
 *                         flat position shard_begin (e.g. a reduce-scattered
 *                         gradient shard, or ZeRO-sharded master/m/v).
 *   flat_mask & ADAMW_BLOCKED_STATE, flat_mask & ADAMW_FLAT_PAD8: see below.
 * numel is a host array of n_tensors element counts (each >= 0). */
/* flat_mask bit: the blocked state layout.  exp_avg, exp_avg_sq and aux share
 * ONE flat buffer of the shard, ptr[2][0] (16-byte aligned; ptr[3], ptr[4] and
 * flat_mask bits 2-4 are ignored), made of ceil((shard_end - shard_begin) / B)
 * blocks of B = ADAMW_STATE_BLOCK_ELEMS = 16384 elements (every mode).  Block k
 * holds the state of the shard's elements [k*B, (k+1)*B), stream after stream:
 *     [exp_avg x B][exp_avg_sq x B][aux x B]
 * each in its stream's dtype (an unused aux stream takes no room; a block is
 * 192 KiB in ADAMW_MIXED, 160 KiB in ADAMW_MIXED_SPLIT, 96 KiB in
 * ADAMW_PURE_KAHAN, B times the three streams' element sizes for the other
 * pure-bf16 precisions); the last block is padded to B.  For optimizer-owned ZeRO state: the step's per-element
 * state traffic becomes one contiguous region per block instead of three
 * separate streams (fewer concurrently open DRAM rows; measured faster on
 * MI355X).  B is one default update chunk, so splitting work at block edges
 * never leaves a workgroup's lanes idle.  param and grad keep their own layout
 * (adamw_check_finite, which reads only grads, ignores the bit).  The 16-byte
 * vector path needs an element's state address and its param/grad addresses
 * to share their alignment: with per-tensor param/grad buffers that start
 * 16-byte aligned, a tensor whose flat start is not a multiple of 8 elements
 * runs element-wise (correct, but slower: on 10,000 tensors of random lengths
 * the mixed fp16 step fell from 5.6 to 4.2 TB/s on MI355X), so give such lists
 * tensor lengths, or padding, that are multiples of 8 (see ADAMW_FLAT_PAD8). */
#define ADAMW_BLOCKED_STATE (1u << 8)
#define ADAMW_STATE_BLOCK_ELEMS 16384
/* flat_mask bit: the padded flat index.  The list's flat concatenation places
 * every tensor at a multiple of 8 elements: tensor i starts at the sum over
 * j < i of numel[j] rounded up to a multiple of 8, and the gaps hold no
 * element (nothing reads or writes them).  shard_begin and shard_end, flat
 * shard buffers and the blocked state are all indexed in this padded space,
 * as in ZeRO implementations that pad each tensor inside their flat buffers;
 * shard_end may reach the padded total.  With per-tensor buffers that start
 * 16-byte aligned and a shard_begin that is a multiple of 8, every tensor of
 * any length keeps the 16-byte vector path in every layout. */
#define ADAMW_FLAT_PAD8 (1u << 9)

typedef struct {
    int64_t n_tensors;
    const int64_t* numel;
    void* const* ptr[ADAMW_NUM_STREAMS];
    int64_t shard_begin;
    int64_t shard_end;
    uint32_t flat_mask;
} adamw_tensor_list;

/* One AdamW step over one contiguous range of n elements: a single tensor, or
 * one data-parallel rank's flat shard with every pointer already offset to it
 * -- the unit of work of the ZeRO-sharded optimizer of "Distributed optimizer
 * support for BERT" (the remark under the 4 x A40 table: each of the DP ranks
 * keeps the fp32 optimizer state and the 16-bit master copy of 1/DP of the
 * parameters, and steps only that share).
 * param, grad, exp_avg, exp_avg_sq, aux: device buffers of n elements in the
 * layouts above.  p_dtype: ADAMW_BF16 or ADAMW_F16 in ADAMW_MIXED, ADAMW_BF16
 * in ADAMW_PURE_KAHAN and ADAMW_MIXED_SPLIT.  n == 0 is valid (the counter
 * still advances unless skipped).  See the file comment for d_step /
 * d_found_inf. */
adamw_status adamw_step(adamw_mode mode, adamw_dtype p_dtype, int64_t n,
                        void* param, const void* grad, void* exp_avg, void* exp_avg_sq, void* aux,
                        const adamw_hparams* hp, int32_t* d_step, const int32_t* d_found_inf,
                        void* hip_stream);

/* One AdamW step over a ragged tensor list (or its shard), in one launch of
 * the update kernel: the chunked multi-tensor form of the fused optimizer
 * ("fused_adam" in "Distributed optimizer support for BERT").  Same element
 * rule, dtypes, counter and skip semantics as adamw_step. */
adamw_status adamw_multi_tensor_step(adamw_mode mode, adamw_dtype p_dtype, const adamw_tensor_list* list,
                                     const adamw_hparams* hp, int32_t* d_step, const int32_t* d_found_inf,
                                     void* hip_stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the step of
 * adamw_multi_tensor_step -- same arguments, same results bit for bit -- with
 * no device allocation, free or allocating library call.  Its workspace (the
 * launch scalars, the single-launch completion counters and the list's chunk
 * table) lives in one static device array of ADAMW_NOALLOC_SCRATCH_BYTES per
 * GPU, which the library's code object holds on every GPU it runs on until
 * the process ends.  The chunk table takes 64 bytes per segment and 16 per
 * chunk (adamw_plan_inspect lists both) and must fit in
 * ADAMW_NOALLOC_SCRATCH_BYTES - 16384 bytes: about a million chunks of a few
 * large tensors (every chunk 16384 elements: some 1.7e10 elements), about
 * 200,000 of a list with blocked state (one segment per block: some 3.3e9
 * elements; OPT-1.3B takes 6.4 MB).  A larger list is rejected with
 * ADAMW_E_INVALID before anything is enqueued.  A call copies the list's table
 * into the array (a host-to-device copy on hip_stream) unless the last call on
 * this GPU used the same list; under graph capture that copy is refused, as in
 * adamw_multi_tensor_step.  A call captured into a graph pins the table it
 * used, since every replay reads it: later calls on that GPU with another list
 * are then refused with ADAMW_E_INVALID (calls with the same list still run)
 * until adamw_release_workspace(), which unpins it and must not run while
 * such a graph may still be replayed.  Every call on a GPU shares that GPU's
 * array and its contents: calls on one GPU that may overlap (on different
 * streams, or from host threads without an order between them) race on it and
 * must be ordered by the caller, e.g. by issuing them on one stream. */
#define ADAMW_NOALLOC_SCRATCH_BYTES (16u << 20)
adamw_status adamw_multi_tensor_step_noalloc(adamw_mode mode, adamw_dtype p_dtype, const adamw_tensor_list* list,
                                             const adamw_hparams* hp, int32_t* d_step, const int32_t* d_found_inf,
                                             void* hip_stream);

/* State precisions of a pure-bf16 step (the AnyPrecisionAdamW knobs of
 * "[pure bf16 training] w/ AnyPrecisionAdamW and Kahan summation":
 * momentum_dtype, variance_dtype, use_kahan_summation and
 * compensation_buffer_dtype). */
#define ADAMW_KAHAN_NONE 0   /* no compensation: stream 4 (aux) is unused */
#define ADAMW_KAHAN_BF16 1   /* stream 4 (aux) is a bf16 compensation buffer */
#define ADAMW_KAHAN_F32 2    /* stream 4 (aux) is an fp32 compensation buffer */
typedef struct {
    adamw_dtype exp_avg;     /* ADAMW_F32 or ADAMW_BF16 */
    adamw_dtype exp_avg_sq;  /* ADAMW_F32 or ADAMW_BF16 */
    int32_t kahan;           /* ADAMW_KAHAN_NONE, ADAMW_KAHAN_BF16 or ADAMW_KAHAN_F32; other values are rejected */
} adamw_pure_precision;

/* Pure-bf16 step with chosen state precisions: param and grad bf16, exp_avg and
 * exp_avg_sq in the dtypes of *prec (fp32 moments are kept and used exactly;
 * bf16 ones are widened, updated in fp32 and stored rounded to nearest even).
 * With a compensation buffer: the ADAMW_PURE_KAHAN rule, the residual
 * s - (p' - p) stored rounded to bf16 (ADAMW_KAHAN_BF16) or kept as the fp32
 * value it is computed in (ADAMW_KAHAN_F32: 2 more bytes per element each way,
 * and p + c then carries an fp32 master); without: p = round_bf16(p*(1 - lr*wd)
 * - (lr/(1-beta1^t))*u).  {ADAMW_BF16, ADAMW_BF16, ADAMW_KAHAN_BF16} is
 * ADAMW_PURE_KAHAN.
 * Everything else (list, shard, counter, skip flag, errors) as
 * adamw_multi_tensor_step. */
adamw_status adamw_pure_multi_tensor_step(const adamw_pure_precision* prec, const adamw_tensor_list* list,
                                          const adamw_hparams* hp, int32_t* d_step, const int32_t* d_found_inf,
                                          void* hip_stream);

/* Dynamic loss scaling state, in device memory owned by the caller (8 bytes,
 * 4-byte aligned).  growth_tracker counts consecutive steps taken since the
 * scale last changed and must start in [0, growth_interval). */
typedef struct {
    float scale;
    int32_t growth_tracker;
} adamw_loss_scale_state;

/* Dynamic loss scaling rule (host values): after growth_interval consecutive
 * steps without an inf/NaN gradient the scale is multiplied by growth_factor
 * (kept unchanged if the product is not finite); a step with an inf/NaN gradient
 * multiplies it by backoff_factor.  Either event resets the tracker.
 * Requirements: growth_factor finite and >= 1; 0 < backoff_factor <= 1;
 * growth_interval >= 1.  The pages show an fp16-amp run but not its scaler's
 * constants; the usual choice is growth 2, backoff 0.5, interval 2000. */
typedef struct {
    float growth_factor;
    float backoff_factor;
    int32_t growth_interval;
} adamw_loss_scaler;

/* fp16-AMP step with a device-resident dynamic loss scale: as
 * adamw_multi_tensor_step with d_found_inf required, except that the gradient
 * multiplier is (float)(1 / (double)d_scale->scale) read on the device when the
 * step runs (hp->inv_loss_scale is ignored), and that the same launch then
 * advances *d_scale by the rule above using *d_found_inf -- whether or not the
 * step itself was skipped.  No host synchronisation is involved.  Typical
 * sequence per iteration: adamw_check_finite, then this call with the same flag
 * (the opt-125m fp16-amp run on the page "[pure bf16 training] w/
 * AnyPrecisionAdamW and Kahan summation"). */
adamw_status adamw_multi_tensor_step_amp(adamw_mode mode, adamw_dtype p_dtype, const adamw_tensor_list* list,
                                         const adamw_hparams* hp, int32_t* d_step, const int32_t* d_found_inf,
                                         adamw_loss_scale_state* d_scale, const adamw_loss_scaler* scaler,
                                         void* hip_stream);

/* fp16-AMP overflow check, for the fp16 mixed-precision training of the
 * "opt-125m / fp16-amp training from scratch" run on the page "[pure bf16
 * training] w/ AnyPrecisionAdamW and Kahan summation": its loss is scaled, and
 * a step whose scaled gradients hold an inf or NaN must be skipped (see the
 * skip flag in the file comment).  Stores 0 to *d_found_inf (stream
 * ordered), then 1 if any gradient element of the list (stream 1 only; shard range and
 * flat_mask bit 1 honoured) has an all-ones exponent field, i.e. is inf or NaN.
 * g_dtype: ADAMW_F16 or ADAMW_BF16.  Scaled gradients are tested as stored,
 * before any unscaling.  Intended order: adamw_check_finite, then the step
 * with the same d_found_inf (an all-reduce(max) of the flag across ranks
 * would sit between the two in a multi-GPU job). */
adamw_status adamw_check_finite(adamw_dtype g_dtype, const adamw_tensor_list* grads, int32_t* d_found_inf,
                                void* hip_stream);

/* Description of the last error on the calling thread ("" if none).  Valid
 * until the next call into the library on that thread. */
const char* adamw_last_error(void);

/* Frees every workspace the library holds (all devices and streams) and
 * releases the allocation-free entry point's table on every GPU (its static
 * array stays).  The caller must make sure no enqueued step is still running,
 * no graph holding a captured step will be replayed again, and no other
 * thread is inside a library call. */
void adamw_release_workspace(void);

/* ADAMW_ABI_VERSION of the built library. */
int adamw_abi_version(void);

/* Optimizer-owned state in the blocked layout (ADAMW_BLOCKED_STATE), set up and
 * read back from ordinary per-tensor (or flat) state buffers: the layout of the
 * fastest steps made easy to adopt, and a blocked state checkpointed in the
 * usual per-tensor form.  Layout only, no arithmetic.
 *
 * `list` describes the per-tensor state as a step of (mode, p_dtype) -- or,
 * with prec non-null, of adamw_pure_multi_tensor_step with *prec -- would see
 * it WITHOUT ADAMW_BLOCKED_STATE: numel, the shard range, ptr[2..4] and
 * flat_mask bits 2-4 for exp_avg, exp_avg_sq and aux, and ADAMW_FLAT_PAD8,
 * which selects the flat index the blocked buffer is laid out in.  ptr[0] and
 * ptr[1] (param, grad) are not used.  The blocked buffer then serves the step
 * whose list has the same numel, shard and ADAMW_FLAT_PAD8 choice,
 * ADAMW_BLOCKED_STATE set and ptr[2][0] = the buffer.
 *
 * adamw_blocked_state_bytes: the size in bytes of that blocked buffer (whole
 * blocks of ADAMW_STATE_BLOCK_ELEMS elements), or -1 on an invalid argument.
 * No GPU work, no HIP call.
 *
 * adamw_blocked_state_copy: copies every element of the shard's state between
 * the per-tensor buffers and `blocked` (device memory, 16-byte aligned,
 * adamw_blocked_state_bytes long): to_blocked != 0 fills the blocked buffer
 * from the per-tensor buffers, 0 the reverse.  The blocked buffer's padding
 * (the ends of the last block and, with ADAMW_FLAT_PAD8, the gaps between
 * tensors) is neither read nor written.  The copy runs on hip_stream, after
 * the work already queued there, and the call returns once it is done (it
 * allocates and frees a small device table: a setup and checkpoint routine,
 * not for the training loop; on a stream under graph capture it is refused
 * with ADAMW_E_INVALID). */
int64_t adamw_blocked_state_bytes(adamw_mode mode, adamw_dtype p_dtype, const adamw_pure_precision* prec,
                                  const adamw_tensor_list* list);
adamw_status adamw_blocked_state_copy(adamw_mode mode, adamw_dtype p_dtype, const adamw_pure_precision* prec,
                                      const adamw_tensor_list* list, void* blocked, int to_blocked, void* hip_stream);

/* Planner introspection, for tests: no GPU work, no HIP call.  Builds the
 * chunk plan that adamw_multi_tensor_step (for_check = 0) or
 * adamw_check_finite (for_check = 1) would launch, and writes up to cap rows
 * of 6 int64 each to out:
 *   {tensor index, element offset inside the tensor, element count,
 *    kind (0 = element-wise, 1 = 16-byte vector), flat position, segment}.
 * Returns the number of chunks (which may exceed cap), or -1 on an invalid
 * argument (see adamw_last_error). */
int64_t adamw_plan_inspect(adamw_mode mode, adamw_dtype p_dtype, const adamw_tensor_list* list, int for_check,
                           int64_t* out, int64_t cap);

/* Planner introspection, for tests: no GPU work, no HIP call.  The device
 * bytes each chunk of the plan covers: for the step of (mode, p_dtype), or with
 * prec non-null the step of adamw_pure_multi_tensor_step with *prec (mode and
 * p_dtype ignored), or with for_check the check of adamw_check_finite
 * (g_dtype = p_dtype), writes up to cap rows of 16 uint64 to out:
 *   {the 6 fields of an adamw_plan_inspect row, lo[0], hi[0], ..., lo[4], hi[4]}
 * where [lo[s], hi[s]) is the address range of stream s that the chunk's
 * workgroups read and write (lo = hi = 0 for a stream the launch does not
 * touch; a blocked state buffer shows as streams 2-4 at their places inside
 * the blocks).  Returns the number of chunks, or -1 on an invalid argument. */
int64_t adamw_plan_inspect_bytes(adamw_mode mode, adamw_dtype p_dtype, const adamw_pure_precision* prec,
                                 const adamw_tensor_list* list, int for_check, uint64_t* out, int64_t cap);

/* Launch form.  A step whose grid has at most max_workgroups workgroups
 * (default 4096: 512 chunks of 16384 elements, about 8.4e6 elements) runs as
 * ONE kernel launch: every workgroup reads *d_found_inf, *d_step and the loss
 * scale itself, forms the step's scalars (the same binary64 formulas, so the
 * same bits), and the last workgroup to finish stores t into *d_step and
 * advances the loss scale.  Larger plans and empty lists run a one-lane
 * prologue kernel first.  Likewise adamw_check_finite over a grid of at most
 * max_workgroups (one per check chunk) is one launch whose last workgroup
 * stores the flag, instead of a zeroing kernel and the check.  The results are
 * bit-identical either way; the single launch saves a kernel launch and its
 * dependency, which dominate steps of a few million elements.  An update plan
 * of c chunks launches 8c workgroups.  max_workgroups: 0 = always two
 * launches, < 0 = restore the default.  Affects later calls on every stream.
 * Returns the value now in force. */
int64_t adamw_set_single_launch_max_workgroups(int64_t max_workgroups);

/* Tuning knob: elements per vector chunk, a multiple of 2048 in [2048, 1<<22],
 * for every kernel (an update chunk is shared by 8 workgroups, one per XCD,
 * each lane taking one 8-element pack per 16384 elements; a check chunk is one
 * workgroup's); 0 restores the built-in defaults (16384 for the update kernels
 * and the check).  Affects plans built after the call.  Returns the value now
 * in force (0 = defaults), or -1 if rejected. */
int64_t adamw_set_chunk_elems(int64_t elems);

#ifdef __cplusplus
}
#endif

#endif /* ADAMW_H */
