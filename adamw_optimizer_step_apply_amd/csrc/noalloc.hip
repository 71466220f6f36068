// noalloc.hip -- adamw_multi_tensor_step_noalloc: the step of
// adamw_multi_tensor_step for callers that cannot allocate device memory.
//
// The regular entry points keep a workspace per stream, allocated on first
// use: the launch scalars, the single-launch completion counters and each
// list's chunk table.  This one keeps the same three things in `scratch`, a
// static device array that the code object holds on every GPU the library
// runs on, and allocates nothing: no hipMalloc, hipFree or allocating library
// call.  Layout of the array:
//   [0, 256)                   launch scalars (written by the prologue kernel)
//   [256, 256 + 8448)          completion counters (zero between launches)
//   [kTableOffset, end)        segment table, then chunk table
// Host code never uses the array's name as an address (there it is only a
// host-side handle): each device's address comes from hipGetSymbolAddress,
// taken once per device with that device current, and every kernel argument
// and copy uses that address.
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <string.h>

#include <map>
#include <memory>
#include <mutex>
#include <string>
#include <vector>

#include "adamw.h"
#include "step.hpp"

static __device__ __align__(256) unsigned char scratch[ADAMW_NOALLOC_SCRATCH_BYTES];

namespace adamw {
namespace {

constexpr int64_t kTableOffset = 16384;
static_assert(kWorkspaceBytes <= kTableOffset, "the scalars and counters fit before the table");
static_assert(kTableOffset % alignof(DevSeg) == 0, "the segment table is aligned");
constexpr int64_t kTableBytes = (int64_t)ADAMW_NOALLOC_SCRATCH_BYTES - kTableOffset;

struct DeviceScratch {
    std::mutex mu;                     // one call at a time per device
    unsigned char* ptr = nullptr;      // this device's `scratch` (hipGetSymbolAddress)
    std::vector<int64_t> key;          // the plan whose table the array holds (empty: none)
    bool pinned = false;               // a graph captured a step with that table
    int64_t n_segs = 0, n_chunks = 0;
    std::vector<unsigned char> table;  // host image of that table
};

std::mutex g_mu;
std::map<int, std::unique_ptr<DeviceScratch>> g_dev;

DeviceScratch& device_scratch(int dev)
{
    std::lock_guard<std::mutex> lk(g_mu);
    auto& d = g_dev[dev];
    if (!d) d.reset(new DeviceScratch());
    return *d;
}

// First call on a device (that device current): the array's address on it,
// and its completion counters cleared (static device memory starts at zero,
// and every single launch leaves the counters at zero; clearing them here
// makes the start explicit).  A fill kernel, not a memset, so that it may sit
// in a captured graph.
adamw_status init_device(DeviceScratch& ds, hipStream_t stream)
{
    if (ds.ptr) return ADAMW_OK;
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return hip_fail("hipGetSymbolAddress (allocation-free workspace)", e);
    e = launch_zero_words(reinterpret_cast<uint32_t*>(static_cast<unsigned char*>(p) + kDoneOffset), kDoneWords,
                          stream);
    if (e != hipSuccess) return hip_fail("allocation-free workspace initialisation", e);
    ds.ptr = static_cast<unsigned char*>(p);
    return ADAMW_OK;
}

// Makes the array hold the plan of (kind, list): the table is planned on the
// host and copied in on `stream`, unless the array already holds it.  A call
// under capture pins the table it uses: the graph reads it at every replay, so
// from then on a call with another list is refused instead of rewriting it,
// until adamw_release_workspace.
adamw_status ensure_table(DeviceScratch& ds, const StepKind& kind, const adamw_tensor_list* list, hipStream_t stream)
{
    const int64_t chunk_elems = chunk_elems_of(kind.kernel);
    std::vector<int64_t> key;
    plan_key(kind.kernel, kind.esz, list, chunk_elems, key);
    bool cap = false;
    adamw_status st = capturing(stream, &cap);
    if (st != ADAMW_OK) return st;
    if (!ds.key.empty() && key == ds.key) {
        if (cap) ds.pinned = true;
        return ADAMW_OK;
    }
    if (cap)
        return fail(ADAMW_E_INVALID,
                    "the allocation-free workspace holds another list's table: make this call once outside "
                    "graph capture first");
    if (ds.pinned)
        return fail(ADAMW_E_INVALID,
                    "the allocation-free workspace holds the table of a step captured into a graph, which "
                    "replays read: it serves only that list until adamw_release_workspace()");
    Plan plan;
    std::string err;
    st = build_plan(kind.esz, list, chunk_elems, kMaxUpdateChunks, &plan, err);
    if (st != ADAMW_OK) return fail(st, err);
    const int64_t seg_bytes = (int64_t)(plan.segs.size() * sizeof(DevSeg));
    const int64_t bytes = seg_bytes + (int64_t)(plan.chunks.size() * sizeof(DevChunk));
    if (bytes > kTableBytes) {
        char buf[256];
        snprintf(buf, sizeof buf,
                 "the list's launch table takes %lld bytes (%zu segments, %zu chunks); the allocation-free step "
                 "holds at most %lld: use adamw_multi_tensor_step",
                 (long long)bytes, plan.segs.size(), plan.chunks.size(), (long long)kTableBytes);
        return fail(ADAMW_E_INVALID, buf);
    }
    ds.key.clear();   // until the copy below is enqueued, the array's table is unknown
    ds.table.resize((size_t)bytes);
    if (bytes) {
        memcpy(ds.table.data(), plan.segs.data(), (size_t)seg_bytes);
        memcpy(ds.table.data() + seg_bytes, plan.chunks.data(), plan.chunks.size() * sizeof(DevChunk));
        // A copy from pageable host memory: the source has been consumed when
        // the call returns, so the host image may change afterwards.
        hipError_t e = hipMemcpyAsync(ds.ptr + kTableOffset, ds.table.data(), (size_t)bytes, hipMemcpyHostToDevice,
                                      stream);
        if (e != hipSuccess) return hip_fail("hipMemcpyAsync (allocation-free chunk table)", e);
    }
    ds.n_segs = (int64_t)plan.segs.size();
    ds.n_chunks = (int64_t)plan.chunks.size();
    ds.key.swap(key);
    return ADAMW_OK;
}

}  // namespace

// Called by adamw_release_workspace: forgets every device's table and its pin
// (the array itself stays; the next call uploads its list's table again).
void release_noalloc_tables()
{
    std::lock_guard<std::mutex> lk(g_mu);
    for (auto& kv : g_dev) {
        std::lock_guard<std::mutex> lk2(kv.second->mu);
        kv.second->key.clear();
        kv.second->pinned = false;
    }
}

}  // namespace adamw

using namespace adamw;

extern "C" adamw_status adamw_multi_tensor_step_noalloc(adamw_mode mode, adamw_dtype p_dtype,
                                                        const adamw_tensor_list* list, const adamw_hparams* hp,
                                                        int32_t* d_step, const int32_t* d_found_inf, void* hip_stream)
{
    clear_error();
    StepKind kind;
    adamw_status st = mode_kind(mode, p_dtype, &kind);
    if (st != ADAMW_OK) return st;
    if ((st = check_step_call(kind, list, hp, d_step, d_found_inf)) != ADAMW_OK) return st;
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    int dev = 0;
    if ((st = stream_device(stream, &dev)) != ADAMW_OK) return st;
    DeviceScratch& ds = device_scratch(dev);
    std::lock_guard<std::mutex> lk(ds.mu);
    DeviceGuard dg(dev);
    if ((st = init_device(ds, stream)) != ADAMW_OK) return st;
    if ((st = ensure_table(ds, kind, list, stream)) != ADAMW_OK) return st;
    const DevSeg* segs = reinterpret_cast<const DevSeg*>(ds.ptr + kTableOffset);
    const DevChunk* chunks = reinterpret_cast<const DevChunk*>(ds.ptr + kTableOffset + ds.n_segs * sizeof(DevSeg));
    return enqueue_step(kind, segs, chunks, ds.n_chunks, reinterpret_cast<LaunchScalars*>(ds.ptr),
                        reinterpret_cast<uint32_t*>(ds.ptr + kDoneOffset), *hp, d_step, d_found_inf, nullptr, nullptr,
                        stream);
}
