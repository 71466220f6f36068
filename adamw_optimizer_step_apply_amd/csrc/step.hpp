// step.hpp -- the host side of one step, shared by the entry points of api.cpp
// (which keep a workspace per stream) and noalloc.hip (which keeps its
// workspace in a static device array): error reporting, the checks made
// before any HIP call, and the launch sequence over a device plan.
#pragma once

#include <hip/hip_runtime.h>

#include <string>

#include "adamw.h"
#include "layout.hpp"
#include "plan.hpp"

namespace adamw {

// The calling thread's last-error text (adamw_last_error) is set to `msg`
// (or to `what` and the HIP error string); returns the status given.
adamw_status fail(adamw_status st, const std::string& msg);
void clear_error();
adamw_status hip_fail(const char* what, hipError_t e);

// What one step launches: the update kernel and its streams' element sizes.
struct StepKind {
    int kernel;
    int esz[kStreams];
};
adamw_status mode_kind(adamw_mode mode, adamw_dtype p_dtype, StepKind* out);
StepKind kind_of_pure(const adamw_pure_precision& prec);
// Elements per vector chunk of an update kernel's plan (the tuning knob, or
// the kernel's default).
int64_t chunk_elems_of(int kernel);

// Every check of a step call that needs no device: hyper-parameters, the
// counter and flag pointers, and the whole list (validated once per key).
adamw_status check_step_call(const StepKind& kind, const adamw_tensor_list* list, const adamw_hparams* hp,
                             const int32_t* d_step, const int32_t* d_found_inf);

// Enqueues one step over a plan already on the device: small grids as one
// launch of the update kernel (which uses the completion counters at `done`),
// others as the prologue kernel (writing the scalars at `scalars`) and the
// update kernel.  d_amp / scaler: the dynamic loss scale, or null.
adamw_status enqueue_step(const StepKind& kind, const DevSeg* segs, const DevChunk* chunks, int64_t n_chunks,
                          LaunchScalars* scalars, uint32_t* done, const adamw_hparams& hp, int32_t* d_step,
                          const int32_t* d_found_inf, adamw_loss_scale_state* d_amp, const adamw_loss_scaler* scaler,
                          hipStream_t stream);

// The device a stream belongs to (the null stream: the calling thread's
// current device), and whether the stream is being captured into a graph.
adamw_status stream_device(hipStream_t stream, int* dev);
adamw_status capturing(hipStream_t stream, bool* out);

// Forgets the allocation-free entry point's table on every device, and its pin
// (noalloc.hip; part of adamw_release_workspace).
void release_noalloc_tables();

// Makes `dev` the current device for the lifetime of the guard (allocations
// and launches of a call then land on its stream's device).
class DeviceGuard {
public:
    explicit DeviceGuard(int dev)
    {
        if (hipGetDevice(&prev_) == hipSuccess && prev_ != dev && hipSetDevice(dev) == hipSuccess) switched_ = true;
    }
    ~DeviceGuard()
    {
        if (switched_) (void)hipSetDevice(prev_);
    }
    DeviceGuard(const DeviceGuard&) = delete;
    DeviceGuard& operator=(const DeviceGuard&) = delete;

private:
    int prev_ = 0;
    bool switched_ = false;
};

// Kernel launchers (kernels.hip).
hipError_t launch_prologue(const adamw_hparams& hp, int32_t* d_step, const int32_t* d_found_inf,
                           LaunchScalars* d_scalars, adamw_loss_scale_state* d_amp, const adamw_loss_scaler& scaler,
                           hipStream_t stream);
hipError_t launch_update(int kernel, const DevSeg* segs, const DevChunk* chunks, int64_t n_chunks,
                         const LaunchScalars* d_scalars, const FusedStep* fused, hipStream_t stream);
hipError_t launch_zero_words(uint32_t* p, int64_t n, hipStream_t stream);
hipError_t launch_check(adamw_dtype g_dtype, const DevSeg* segs, const DevChunk* chunks, int64_t n_chunks,
                        int32_t* d_flag, uint32_t* done, bool fused, hipStream_t stream);
hipError_t launch_state_copy(const DevCopySeg* segs, const DevChunk* chunks, int64_t n_chunks, const int esz[3],
                             bool to_blocked, hipStream_t stream);

}  // namespace adamw
