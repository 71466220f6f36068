// api.cpp -- the C ABI declared in include/adamw.h: validation, plan caching,
// per-(device, stream) workspace, and the launch sequence
//   [check: zero flag -> check kernel]   (adamw_check_finite)
//   [step:  prologue  -> update kernel]  (adamw_step / adamw_multi_tensor_step[_amp])
//   small grids (up to a few thousand workgroups): the check kernel alone, the
//   update kernel alone
// Nothing here synchronises with the device except when a workspace has to
// grow (the old buffer may still be read by work queued on its stream).
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <map>
#include <memory>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "adamw.h"
#include "layout.hpp"
#include "plan.hpp"
#include "step.hpp"

namespace adamw {

namespace {
thread_local std::string g_err;
}  // namespace

adamw_status fail(adamw_status st, const std::string& msg)
{
    g_err = msg;
    return st;
}

void clear_error() { g_err.clear(); }

adamw_status hip_fail(const char* what, hipError_t e)
{
    g_err = std::string(what) + ": " + hipGetErrorString(e);
    return ADAMW_E_HIP;
}

namespace {

// A device-resident copy of one plan (segment table followed by chunk table),
// uploaded through a pinned staging buffer.
struct PlanSlot {
    void* dev = nullptr;
    size_t dev_cap = 0;
    void* host = nullptr;
    size_t host_cap = 0;
    hipEvent_t uploaded = nullptr;
    bool upload_in_flight = false;
    std::vector<int64_t> key;
    bool valid = false;
    bool pinned = false;   // used under graph capture: never evicted, resized or rewritten
    int64_t n_segs = 0, n_chunks = 0;

    const DevSeg* segs() const { return static_cast<const DevSeg*>(dev); }
    const DevChunk* chunks() const
    {
        return reinterpret_cast<const DevChunk*>(static_cast<const char*>(dev) + n_segs * sizeof(DevSeg));
    }

    void release()
    {
        if (dev) (void)hipFree(dev);
        if (host) (void)hipHostFree(host);
        if (uploaded) (void)hipEventDestroy(uploaded);
        dev = host = nullptr;
        uploaded = nullptr;
        dev_cap = host_cap = 0;
        valid = false;
        pinned = false;
        key.clear();
    }
};

// Plans cached per stream, most recently used first: at most this many slots
// that no captured graph holds, plus every pinned one.  A training loop that
// alternates a few lists (e.g. two parameter groups, or a step and its
// overflow check) keeps each one's table resident instead of re-uploading it.
constexpr size_t kPlansPerStream = 8;

struct StreamWorkspace {
    int device = 0;                     // the stream's device: the workspace lives there
    LaunchScalars* scalars = nullptr;   // device, kWorkspaceBytes: scalars, then the completion counters
    std::vector<std::unique_ptr<PlanSlot>> plans;
    std::mutex mu;                      // one call at a time per stream
};

std::mutex g_mu;
std::map<std::pair<int, uintptr_t>, std::unique_ptr<StreamWorkspace>> g_ws;
std::atomic<int64_t> g_chunk_elems{0};   // 0: each kernel's own default chunk
// Grids of at most this many workgroups run as one launch (the update kernel
// forms the step's scalars itself) instead of prologue + update kernel.
std::atomic<int64_t> g_single_launch_max_workgroups{kSingleLaunchMaxWorkgroups};

// The chunk limit of a plan for `tag` (an update kernel id, or -1 for the
// overflow check): the grid of one launch holds at most 2^32 - 1 lanes.
int64_t max_chunks_of(int64_t tag) { return tag < 0 ? kMaxCheckChunks : kMaxUpdateChunks; }

// The workspace of a stream, on the stream's own device.
adamw_status get_workspace(hipStream_t stream, StreamWorkspace** out)
{
    int dev = 0;
    adamw_status st = stream_device(stream, &dev);
    if (st != ADAMW_OK) return st;
    std::lock_guard<std::mutex> lk(g_mu);
    auto& ws = g_ws[{dev, (uintptr_t)stream}];
    if (!ws) {
        ws.reset(new StreamWorkspace());
        ws->device = dev;
    }
    *out = ws.get();
    return ADAMW_OK;
}

// Returns (in *out) a slot of `ws` holding the device plan of (mode, dtype,
// list, for_check): a cached one if every input matches (the key holds every
// input the plan depends on, so a hit was validated when it was built), else
// the list is validated and planned, and a slot chosen by choose_plan_slot
// takes the new plan.  An invalid list returns its error before any HIP call
// and leaves the cache as it was.
//
// Under graph capture the graph records the slot's device address: a hit pins
// the slot, so that later calls never evict, resize or rewrite it while the
// graph may replay (pinned slots are freed by adamw_release_workspace only).
// A miss under capture is refused: uploading a table would need a copy, and a
// table that grows a stream synchronisation, neither of which belongs in the
// graph.
adamw_status ensure_plan(StreamWorkspace& ws, int64_t tag, const int esz[kStreams], const adamw_tensor_list* list,
                         int64_t chunk_elems, hipStream_t stream, bool under_capture, PlanSlot** out)
{
    std::vector<int64_t> key;
    plan_key(tag, esz, list, chunk_elems, key);
    auto& plans = ws.plans;
    for (size_t i = 0; i < plans.size(); ++i) {
        if (plans[i]->valid && plans[i]->key == key) {
            std::rotate(plans.begin(), plans.begin() + (ptrdiff_t)i, plans.begin() + (ptrdiff_t)i + 1);
            *out = plans.front().get();
            if (under_capture) (*out)->pinned = true;
            return ADAMW_OK;
        }
    }
    Plan plan;
    std::string err;
    adamw_status st = build_plan(esz, list, chunk_elems, max_chunks_of(tag), &plan, err);
    if (st != ADAMW_OK) return fail(st, err);
    if (under_capture)
        return fail(ADAMW_E_INVALID,
                    "this list's chunk table is not on the device: make the same call once on this stream "
                    "before capturing it into a graph");

    std::vector<bool> pinned(plans.size());
    for (size_t i = 0; i < plans.size(); ++i) pinned[i] = plans[i]->pinned;
    const size_t pick = choose_plan_slot(pinned, kPlansPerStream);
    if (pick == plans.size()) plans.emplace_back(new PlanSlot());
    std::rotate(plans.begin(), plans.begin() + (ptrdiff_t)pick, plans.begin() + (ptrdiff_t)pick + 1);
    PlanSlot& slot = *plans.front();
    slot.valid = false;
    *out = &slot;

    const size_t seg_bytes = plan.segs.size() * sizeof(DevSeg);
    const size_t bytes = seg_bytes + plan.chunks.size() * sizeof(DevChunk);
    hipError_t e;
    if (!slot.uploaded) {
        e = hipEventCreateWithFlags(&slot.uploaded, hipEventDisableTiming);
        if (e != hipSuccess) return hip_fail("hipEventCreate", e);
    }
    // the staging buffer may still feed the previous upload
    if (slot.upload_in_flight) {
        e = hipEventSynchronize(slot.uploaded);
        if (e != hipSuccess) return hip_fail("hipEventSynchronize", e);
        slot.upload_in_flight = false;
    }
    if (bytes > slot.host_cap) {
        if (slot.host) (void)hipHostFree(slot.host);
        slot.host = nullptr;
        size_t cap = bytes + bytes / 4 + 4096;
        e = hipHostMalloc(&slot.host, cap, hipHostMallocDefault);
        if (e != hipSuccess) { slot.host_cap = 0; slot.valid = false; return fail(ADAMW_E_NOMEM, "hipHostMalloc failed"); }
        slot.host_cap = cap;
    }
    if (bytes > slot.dev_cap) {
        if (slot.dev) {
            // queued kernels on this stream may still read the old table
            e = hipStreamSynchronize(stream);
            if (e != hipSuccess) return hip_fail("hipStreamSynchronize", e);
            (void)hipFree(slot.dev);
            slot.dev = nullptr;
        }
        size_t cap = bytes + bytes / 4 + 4096;
        e = hipMalloc(&slot.dev, cap);
        if (e != hipSuccess) { slot.dev_cap = 0; slot.valid = false; return fail(ADAMW_E_NOMEM, "hipMalloc of the chunk table failed"); }
        slot.dev_cap = cap;
    }
    if (bytes) {
        memcpy(slot.host, plan.segs.data(), seg_bytes);
        memcpy(static_cast<char*>(slot.host) + seg_bytes, plan.chunks.data(), plan.chunks.size() * sizeof(DevChunk));
        e = hipMemcpyAsync(slot.dev, slot.host, bytes, hipMemcpyHostToDevice, stream);
        if (e != hipSuccess) { slot.valid = false; return hip_fail("hipMemcpyAsync (chunk table)", e); }
        e = hipEventRecord(slot.uploaded, stream);
        if (e != hipSuccess) { slot.valid = false; return hip_fail("hipEventRecord", e); }
        slot.upload_in_flight = true;
    }
    slot.n_segs = (int64_t)plan.segs.size();
    slot.n_chunks = (int64_t)plan.chunks.size();
    slot.key.swap(key);
    slot.valid = true;
    return ADAMW_OK;
}

// Keys of the lists validated most recently (full keys, not hashes).  A call
// whose key is here skips the validation walk, which for a blocked-state list
// of 10^5-10^6 pieces costs milliseconds of host time per call; a new key is
// validated before any HIP call.
constexpr size_t kValidatedKeys = 16;
std::mutex g_validated_mu;
std::vector<std::vector<int64_t>> g_validated;   // most recent first

bool validated_before(const std::vector<int64_t>& key)
{
    std::lock_guard<std::mutex> lk(g_validated_mu);
    for (size_t i = 0; i < g_validated.size(); ++i) {
        if (g_validated[i] == key) {
            std::rotate(g_validated.begin(), g_validated.begin() + (ptrdiff_t)i,
                        g_validated.begin() + (ptrdiff_t)i + 1);
            return true;
        }
    }
    return false;
}

void remember_validated(const std::vector<int64_t>& key)
{
    std::lock_guard<std::mutex> lk(g_validated_mu);
    if (g_validated.size() >= kValidatedKeys) g_validated.pop_back();
    g_validated.insert(g_validated.begin(), key);
}

// Validates the list for a plan of `tag` (unless the same key passed before),
// with no HIP call.
adamw_status validate_list(int64_t tag, const int esz[kStreams], const adamw_tensor_list* list, int64_t chunk_elems)
{
    std::vector<int64_t> key;
    plan_key(tag, esz, list, chunk_elems, key);
    if (validated_before(key)) return ADAMW_OK;
    std::string err;
    adamw_status st = build_plan(esz, list, chunk_elems, max_chunks_of(tag), nullptr, err);
    if (st != ADAMW_OK) return fail(st, err);
    remember_validated(key);
    return ADAMW_OK;
}

adamw_status check_hparams(const adamw_hparams* hp)
{
    std::string err;
    adamw_status st = adamw::check_hparams(hp, err);
    return st == ADAMW_OK ? st : fail(st, err);
}

adamw_status basic_list_check(const adamw_tensor_list* list)
{
    std::string err;
    adamw_status st = adamw::basic_list_check(list, err);
    return st == ADAMW_OK ? st : fail(st, err);
}

adamw_status check_scaler(const adamw_loss_scaler* sc)
{
    std::string err;
    adamw_status st = adamw::check_scaler(sc, err);
    return st == ADAMW_OK ? st : fail(st, err);
}

// The stream's 256-byte scalar block and the single-launch completion counters
// after it, allocated on first use (the counters start at zero, and every
// single launch leaves them at zero).  Returns the counters in *done.
adamw_status ensure_workspace_block(StreamWorkspace& ws, hipStream_t stream, bool under_capture, uint32_t** done)
{
    if (!ws.scalars) {
        if (under_capture)
            return fail(ADAMW_E_INVALID,
                        "this stream has no workspace yet: make the same call once on it before capturing it "
                        "into a graph");
        hipError_t e = hipMalloc(reinterpret_cast<void**>(&ws.scalars), kWorkspaceBytes);
        if (e != hipSuccess) { ws.scalars = nullptr; return fail(ADAMW_E_NOMEM, "hipMalloc of the scalar block failed"); }
        uint32_t* d = reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(ws.scalars) + kDoneOffset);
        e = launch_zero_words(d, kDoneWords, stream);
        if (e != hipSuccess) {
            (void)hipFree(ws.scalars);
            ws.scalars = nullptr;
            return hip_fail("workspace initialisation", e);
        }
    }
    *done = reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(ws.scalars) + kDoneOffset);
    return ADAMW_OK;
}

// Whether a grid of n_workgroups (> 0) runs as one launch.
bool single_launch(int64_t n_workgroups)
{
    return n_workgroups > 0 && n_workgroups <= g_single_launch_max_workgroups.load(std::memory_order_relaxed);
}

int kernel_block(int kernel) { return kernel == kKernelSplit || kernel >= kKernelPure ? kBlockPure : kBlockMixed; }

int64_t check_chunk_elems()
{
    const int64_t c = g_chunk_elems.load(std::memory_order_relaxed);
    return c ? c : kCheckChunkElems;
}

// Row i of adamw_plan_inspect: {tensor, offset in the tensor, count, kind, flat position, segment}.
void inspect_row(const Plan& plan, size_t i, int64_t* r)
{
    const DevChunk& c = plan.chunks[i];
    const SegInfo& si = plan.info[c.seg];
    r[0] = si.tensor;
    r[1] = si.tensor_off + (int64_t)c.off;
    r[2] = (int64_t)(c.n_kind & kCountMask);
    r[3] = (c.n_kind & kVecBit) ? 1 : 0;
    r[4] = si.flat + (int64_t)c.off;
    r[5] = (int64_t)c.seg;
}

// One step through the stream's workspace and plan cache.
adamw_status do_step(const StepKind& kind, const adamw_tensor_list* list, const adamw_hparams* hp, int32_t* d_step,
                     const int32_t* d_found_inf, void* hip_stream, adamw_loss_scale_state* d_amp = nullptr,
                     const adamw_loss_scaler* scaler = nullptr)
{
    adamw_status st;
    if ((st = check_step_call(kind, list, hp, d_step, d_found_inf)) != ADAMW_OK) return st;
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    StreamWorkspace* ws = nullptr;
    if ((st = get_workspace(stream, &ws)) != ADAMW_OK) return st;
    std::lock_guard<std::mutex> lk(ws->mu);
    DeviceGuard dg(ws->device);
    bool cap = false;
    if ((st = capturing(stream, &cap)) != ADAMW_OK) return st;
    uint32_t* done = nullptr;
    if ((st = ensure_workspace_block(*ws, stream, cap, &done)) != ADAMW_OK) return st;
    PlanSlot* plan = nullptr;
    if ((st = ensure_plan(*ws, kind.kernel, kind.esz, list, chunk_elems_of(kind.kernel), stream, cap, &plan)) !=
        ADAMW_OK)
        return st;
    return enqueue_step(kind, plan->segs(), plan->chunks(), plan->n_chunks, ws->scalars, done, *hp, d_step,
                        d_found_inf, d_amp, scaler, stream);
}

}  // namespace

StepKind kind_of_pure(const adamw_pure_precision& prec)
{
    const int m32 = prec.exp_avg == ADAMW_F32, v32 = prec.exp_avg_sq == ADAMW_F32;
    const int kahan = prec.kahan != ADAMW_KAHAN_NONE, c32 = prec.kahan == ADAMW_KAHAN_F32;
    StepKind kind{};
    kind.kernel = c32 ? kKernelPureC32 + 2 * m32 + v32 : kKernelPure + 4 * m32 + 2 * v32 + kahan;
    kind.esz[ADAMW_STREAM_PARAM] = 2;
    kind.esz[ADAMW_STREAM_GRAD] = 2;
    kind.esz[ADAMW_STREAM_EXP_AVG] = m32 ? 4 : 2;
    kind.esz[ADAMW_STREAM_EXP_AVG_SQ] = v32 ? 4 : 2;
    kind.esz[ADAMW_STREAM_AUX] = c32 ? 4 : kahan ? 2 : 0;
    return kind;
}

StepKind kind_of_mode(adamw_mode mode, adamw_dtype p_dtype)
{
    StepKind k{};
    mode_esizes(mode, p_dtype, false, k.esz);
    k.kernel = mode == ADAMW_PURE_KAHAN ? kKernelKahan
             : mode == ADAMW_MIXED_SPLIT ? kKernelSplit
             : p_dtype == ADAMW_F16 ? kKernelMixedF16 : kKernelMixedBf16;
    return k;
}

adamw_status mode_kind(adamw_mode mode, adamw_dtype p_dtype, StepKind* out)
{
    std::string err;
    adamw_status st = check_mode(mode, p_dtype, false, err);
    if (st != ADAMW_OK) return fail(st, err);
    *out = kind_of_mode(mode, p_dtype);
    return ADAMW_OK;
}

adamw_status check_step_call(const StepKind& kind, const adamw_tensor_list* list, const adamw_hparams* hp,
                             const int32_t* d_step, const int32_t* d_found_inf)
{
    adamw_status st;
    if ((st = check_hparams(hp)) != ADAMW_OK) return st;
    if (!d_step) return fail(ADAMW_E_INVALID, "d_step is null");
    if ((uintptr_t)d_step % 4 || (uintptr_t)d_found_inf % 4)
        return fail(ADAMW_E_INVALID, "d_step / d_found_inf must be 4-byte aligned");
    if ((st = basic_list_check(list)) != ADAMW_OK) return st;
    // the whole list is validated before the first HIP call
    return validate_list(kind.kernel, kind.esz, list, chunk_elems_of(kind.kernel));
}

adamw_status enqueue_step(const StepKind& kind, const DevSeg* segs, const DevChunk* chunks, int64_t n_chunks,
                          LaunchScalars* scalars, uint32_t* done, const adamw_hparams& hp, int32_t* d_step,
                          const int32_t* d_found_inf, adamw_loss_scale_state* d_amp, const adamw_loss_scaler* scaler,
                          hipStream_t stream)
{
    const adamw_loss_scaler rule = scaler ? *scaler : adamw_loss_scaler{1.0f, 1.0f, 1};
    hipError_t e;
    // Small plans: one launch.  An empty plan, whose step still advances the
    // counter (and the loss scale), keeps the prologue kernel.
    if (single_launch(n_chunks * kXcdParts)) {
        const FusedStep fs{hp, d_step, d_found_inf, done, d_amp, rule};
        e = launch_update(kind.kernel, segs, chunks, n_chunks, nullptr, &fs, stream);
        if (e != hipSuccess) return hip_fail("update launch", e);
        return ADAMW_OK;
    }
    e = launch_prologue(hp, d_step, d_found_inf, scalars, d_amp, rule, stream);
    if (e != hipSuccess) return hip_fail("prologue launch", e);
    e = launch_update(kind.kernel, segs, chunks, n_chunks, scalars, nullptr, stream);
    if (e != hipSuccess) return hip_fail("update launch", e);
    return ADAMW_OK;
}

adamw_status stream_device(hipStream_t stream, int* dev)
{
    hipError_t e = stream ? hipStreamGetDevice(stream, dev) : hipGetDevice(dev);
    if (e != hipSuccess) return hip_fail(stream ? "hipStreamGetDevice" : "hipGetDevice", e);
    return ADAMW_OK;
}

// Whether `stream` is being captured into a HIP graph right now.
adamw_status capturing(hipStream_t stream, bool* out)
{
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(stream, &cs);
    if (e != hipSuccess) return hip_fail("hipStreamIsCapturing", e);
    *out = cs != hipStreamCaptureStatusNone;
    return ADAMW_OK;
}

int64_t chunk_elems_of(int kernel)
{
    const int64_t c = g_chunk_elems.load(std::memory_order_relaxed);
    return c ? c : update_chunk_elems(kernel_block(kernel));
}

}  // namespace adamw

using namespace adamw;

extern "C" {

adamw_status adamw_multi_tensor_step(adamw_mode mode, adamw_dtype p_dtype, const adamw_tensor_list* list,
                                     const adamw_hparams* hp, int32_t* d_step, const int32_t* d_found_inf,
                                     void* hip_stream)
{
    g_err.clear();
    StepKind kind;
    adamw_status st = mode_kind(mode, p_dtype, &kind);
    if (st != ADAMW_OK) return st;
    return do_step(kind, list, hp, d_step, d_found_inf, hip_stream);
}

adamw_status adamw_pure_multi_tensor_step(const adamw_pure_precision* prec, const adamw_tensor_list* list,
                                          const adamw_hparams* hp, int32_t* d_step, const int32_t* d_found_inf,
                                          void* hip_stream)
{
    g_err.clear();
    std::string err;
    adamw_status st = check_pure_precision(prec, err);
    if (st != ADAMW_OK) return fail(st, err);
    return do_step(kind_of_pure(*prec), list, hp, d_step, d_found_inf, hip_stream);
}

adamw_status adamw_multi_tensor_step_amp(adamw_mode mode, adamw_dtype p_dtype, const adamw_tensor_list* list,
                                         const adamw_hparams* hp, int32_t* d_step, const int32_t* d_found_inf,
                                         adamw_loss_scale_state* d_scale, const adamw_loss_scaler* scaler,
                                         void* hip_stream)
{
    g_err.clear();
    if (!d_found_inf) return fail(ADAMW_E_INVALID, "d_found_inf is required with a dynamic loss scale");
    if (!d_scale || (uintptr_t)d_scale % 4) return fail(ADAMW_E_INVALID, "d_scale is null or not 4-byte aligned");
    adamw_status st = check_scaler(scaler);
    if (st != ADAMW_OK) return st;
    StepKind kind;
    if ((st = mode_kind(mode, p_dtype, &kind)) != ADAMW_OK) return st;
    return do_step(kind, list, hp, d_step, d_found_inf, hip_stream, d_scale, scaler);
}

adamw_status adamw_step(adamw_mode mode, adamw_dtype p_dtype, int64_t n, void* param, const void* grad,
                        void* exp_avg, void* exp_avg_sq, void* aux, const adamw_hparams* hp, int32_t* d_step,
                        const int32_t* d_found_inf, void* hip_stream)
{
    g_err.clear();
    if (n < 0) return fail(ADAMW_E_INVALID, "n < 0");
    void* p0 = param;
    void* p1 = const_cast<void*>(grad);
    void* p2 = exp_avg;
    void* p3 = exp_avg_sq;
    void* p4 = aux;
    void* const a0[1] = {p0};
    void* const a1[1] = {p1};
    void* const a2[1] = {p2};
    void* const a3[1] = {p3};
    void* const a4[1] = {p4};
    const int64_t numel[1] = {n};
    adamw_tensor_list list;
    list.n_tensors = 1;
    list.numel = numel;
    list.ptr[0] = a0;
    list.ptr[1] = a1;
    list.ptr[2] = a2;
    list.ptr[3] = a3;
    list.ptr[4] = a4;
    list.shard_begin = 0;
    list.shard_end = -1;
    list.flat_mask = 0;
    if (n > 0 && (!param || !grad || !exp_avg || !exp_avg_sq || !aux))
        return fail(ADAMW_E_INVALID, "a required buffer pointer is null");
    StepKind kind;
    adamw_status st = mode_kind(mode, p_dtype, &kind);
    if (st != ADAMW_OK) return st;
    return do_step(kind, &list, hp, d_step, d_found_inf, hip_stream);
}

adamw_status adamw_check_finite(adamw_dtype g_dtype, const adamw_tensor_list* grads, int32_t* d_found_inf,
                                void* hip_stream)
{
    g_err.clear();
    std::string err;
    adamw_status st = check_mode(ADAMW_MIXED, g_dtype, true, err);
    if (st != ADAMW_OK) return fail(st, err);
    if (!d_found_inf || (uintptr_t)d_found_inf % 4) return fail(ADAMW_E_INVALID, "d_found_inf is null or misaligned");
    if ((st = basic_list_check(grads)) != ADAMW_OK) return st;
    const int64_t chunk_elems = check_chunk_elems();
    int esz[kStreams];
    mode_esizes(ADAMW_MIXED, g_dtype, true, esz);
    if ((st = validate_list(-1, esz, grads, chunk_elems)) != ADAMW_OK) return st;
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    StreamWorkspace* ws = nullptr;
    if ((st = get_workspace(stream, &ws)) != ADAMW_OK) return st;
    std::lock_guard<std::mutex> lk(ws->mu);
    DeviceGuard dg(ws->device);
    bool cap = false;
    if ((st = capturing(stream, &cap)) != ADAMW_OK) return st;
    uint32_t* done = nullptr;
    if ((st = ensure_workspace_block(*ws, stream, cap, &done)) != ADAMW_OK) return st;
    PlanSlot* plan = nullptr;
    if ((st = ensure_plan(*ws, -1, esz, grads, chunk_elems, stream, cap, &plan)) != ADAMW_OK) return st;
    hipError_t e = launch_check(g_dtype, plan->segs(), plan->chunks(), plan->n_chunks, d_found_inf, done,
                                single_launch(plan->n_chunks), stream);
    if (e != hipSuccess) return hip_fail("check launch", e);
    return ADAMW_OK;
}

const char* adamw_last_error(void) { return g_err.c_str(); }

void adamw_release_workspace(void)
{
    std::lock_guard<std::mutex> lk(g_mu);
    for (auto& kv : g_ws) {
        StreamWorkspace* ws = kv.second.get();
        if (ws->scalars) (void)hipFree(ws->scalars);
        ws->scalars = nullptr;
        for (auto& p : ws->plans) p->release();
        ws->plans.clear();
    }
    g_ws.clear();
    release_noalloc_tables();
}

int adamw_abi_version(void) { return ADAMW_ABI_VERSION; }

int64_t adamw_plan_inspect(adamw_mode mode, adamw_dtype p_dtype, const adamw_tensor_list* list, int for_check,
                           int64_t* out, int64_t cap)
{
    g_err.clear();
    Plan plan;
    std::string err;
    adamw_status st = check_mode(mode, p_dtype, for_check != 0, err);
    int esz[kStreams];
    mode_esizes(mode, p_dtype, for_check != 0, esz);
    const int64_t chunk = for_check ? check_chunk_elems()
                                    : chunk_elems_of(st == ADAMW_OK ? kind_of_mode(mode, p_dtype).kernel : 0);
    if (st == ADAMW_OK) st = build_plan(esz, list, chunk, for_check ? kMaxCheckChunks : kMaxUpdateChunks, &plan, err);
    if (st != ADAMW_OK) {
        g_err = err;
        return -1;
    }
    const int64_t n = (int64_t)plan.chunks.size();
    for (int64_t i = 0; i < n && i < cap && out; ++i) inspect_row(plan, (size_t)i, out + 6 * i);
    return n;
}

int64_t adamw_plan_inspect_bytes(adamw_mode mode, adamw_dtype p_dtype, const adamw_pure_precision* prec,
                                 const adamw_tensor_list* list, int for_check, uint64_t* out, int64_t cap)
{
    g_err.clear();
    std::string err;
    adamw_status st = ADAMW_OK;
    StepKind kind{};
    int64_t chunk = 0, max_chunks = kMaxUpdateChunks;
    if (for_check) {
        st = check_mode(mode, p_dtype, true, err);
        mode_esizes(mode, p_dtype, true, kind.esz);
        chunk = check_chunk_elems();
        max_chunks = kMaxCheckChunks;
    } else if (prec) {
        st = check_pure_precision(prec, err);
        if (st == ADAMW_OK) kind = kind_of_pure(*prec);
    } else {
        st = check_mode(mode, p_dtype, false, err);
        if (st == ADAMW_OK) kind = kind_of_mode(mode, p_dtype);
    }
    if (st == ADAMW_OK && !for_check) chunk = chunk_elems_of(kind.kernel);
    Plan plan;
    if (st == ADAMW_OK) st = build_plan(kind.esz, list, chunk, max_chunks, &plan, err);
    if (st != ADAMW_OK) {
        g_err = err;
        return -1;
    }
    const int64_t n = (int64_t)plan.chunks.size();
    constexpr int64_t kRow = 6 + 2 * kStreams;
    for (int64_t i = 0; i < n && i < cap && out; ++i) {
        uint64_t* r = out + kRow * i;
        inspect_row(plan, (size_t)i, reinterpret_cast<int64_t*>(r));
        uint64_t lo[kStreams], hi[kStreams];
        chunk_bytes(plan, (size_t)i, kind.esz, lo, hi);
        for (int s = 0; s < kStreams; ++s) {
            r[6 + 2 * s] = lo[s];
            r[6 + 2 * s + 1] = hi[s];
        }
    }
    return n;
}

// The element sizes of a step of (mode, p_dtype), or of the pure step of *prec.
static adamw_status state_kind(adamw_mode mode, adamw_dtype p_dtype, const adamw_pure_precision* prec, StepKind* kind)
{
    if (!prec) return mode_kind(mode, p_dtype, kind);
    std::string err;
    adamw_status st = check_pure_precision(prec, err);
    if (st != ADAMW_OK) return fail(st, err);
    *kind = kind_of_pure(*prec);
    return ADAMW_OK;
}

int64_t adamw_blocked_state_bytes(adamw_mode mode, adamw_dtype p_dtype, const adamw_pure_precision* prec,
                                  const adamw_tensor_list* list)
{
    g_err.clear();
    StepKind kind;
    if (state_kind(mode, p_dtype, prec, &kind) != ADAMW_OK) return -1;
    CopyPlan cp;
    std::string err;
    // the blocked side's base is only an address to plan with: nothing is accessed
    if (build_copy_plan(kind.esz, list, 4096, &cp, err) != ADAMW_OK) {
        g_err = err;
        return -1;
    }
    return cp.blocked_bytes;
}

adamw_status adamw_blocked_state_copy(adamw_mode mode, adamw_dtype p_dtype, const adamw_pure_precision* prec,
                                      const adamw_tensor_list* list, void* blocked, int to_blocked, void* hip_stream)
{
    g_err.clear();
    StepKind kind;
    adamw_status st = state_kind(mode, p_dtype, prec, &kind);
    if (st != ADAMW_OK) return st;
    if (!blocked || (uintptr_t)blocked % 16) return fail(ADAMW_E_INVALID, "blocked buffer is null or not 16-byte aligned");
    CopyPlan cp;
    std::string err;
    if ((st = build_copy_plan(kind.esz, list, (uint64_t)(uintptr_t)blocked, &cp, err)) != ADAMW_OK) return fail(st, err);
    if (cp.chunks.empty()) return ADAMW_OK;
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    int dev = 0;
    if ((st = stream_device(stream, &dev)) != ADAMW_OK) return st;
    bool cap = false;
    if ((st = capturing(stream, &cap)) != ADAMW_OK) return st;
    if (cap)
        return fail(ADAMW_E_INVALID,
                    "adamw_blocked_state_copy allocates and waits for the copy: it cannot be captured into a graph");
    DeviceGuard dg(dev);
    const size_t seg_bytes = cp.segs.size() * sizeof(DevCopySeg);
    const size_t bytes = seg_bytes + cp.chunks.size() * sizeof(DevChunk);
    std::vector<unsigned char> host(bytes);
    memcpy(host.data(), cp.segs.data(), seg_bytes);
    memcpy(host.data() + seg_bytes, cp.chunks.data(), cp.chunks.size() * sizeof(DevChunk));
    void* table = nullptr;
    hipError_t e = hipMalloc(&table, bytes);
    if (e != hipSuccess) return fail(ADAMW_E_NOMEM, "hipMalloc of the copy table failed");
    const int esz[3] = {kind.esz[2], kind.esz[3], kind.esz[4]};
    e = hipMemcpyAsync(table, host.data(), bytes, hipMemcpyHostToDevice, stream);
    if (e == hipSuccess)
        e = launch_state_copy(static_cast<const DevCopySeg*>(table),
                              reinterpret_cast<const DevChunk*>(static_cast<char*>(table) + seg_bytes),
                              (int64_t)cp.chunks.size(), esz, to_blocked != 0, stream);
    // the table is freed once the copy has run: the call returns with the copy done
    const hipError_t e2 = hipStreamSynchronize(stream);
    (void)hipFree(table);
    if (e != hipSuccess) return hip_fail("state copy", e);
    if (e2 != hipSuccess) return hip_fail("hipStreamSynchronize (state copy)", e2);
    return ADAMW_OK;
}

int64_t adamw_set_single_launch_max_workgroups(int64_t max_workgroups)
{
    const int64_t v = max_workgroups < 0 ? kSingleLaunchMaxWorkgroups : max_workgroups;
    g_single_launch_max_workgroups.store(v, std::memory_order_relaxed);
    return v;
}

int64_t adamw_set_chunk_elems(int64_t elems)
{
    if (elems != 0 && (elems < 2048 || elems > (INT64_C(1) << 22) || elems % 2048)) return -1;
    g_chunk_elems.store(elems, std::memory_order_relaxed);
    return elems;
}

}  // extern "C"
