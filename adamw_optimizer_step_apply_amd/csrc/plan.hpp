// plan.hpp -- host-side logic of the fused AdamW launch, free of HIP calls:
// the planner (tensor list, or ZeRO shard of it -> segments and workgroup
// chunks) and the argument checks made before anything is enqueued.
#pragma once

#include <stdint.h>

#include <string>
#include <vector>

#include "adamw.h"
#include "layout.hpp"

namespace adamw {

struct SegInfo {
    int64_t tensor;     // index in the list
    int64_t tensor_off; // first element inside the tensor
    int64_t flat;       // flat position of that element in the list's concatenation
    int64_t count;
};

struct Plan {
    std::vector<DevSeg> segs;
    std::vector<DevChunk> chunks;
    std::vector<SegInfo> info;   // parallel to segs
    int64_t total = 0;           // elements covered
};

// Checks the mode/dtype pair.  Returns ADAMW_OK or an error with `err` set.
adamw_status check_mode(adamw_mode mode, adamw_dtype p_dtype, bool for_check, std::string& err);

// Element sizes of the five streams for a step in `mode` (or, with for_check,
// for the overflow check, which reads the gradient only); 0 = stream unused.
void mode_esizes(adamw_mode mode, adamw_dtype p_dtype, bool for_check, int esz[kStreams]);

// Validates the list against per-stream element sizes `esz` (0 = stream
// unused) and, if `out` is non-null, builds the plan with vector chunks of
// `chunk_elems` elements; a plan of more than `max_chunks` chunks (the grid
// limit of the kernel that runs it) is rejected.  No HIP call.
adamw_status build_plan(const int esz[kStreams], const adamw_tensor_list* list, int64_t chunk_elems,
                        int64_t max_chunks, Plan* out, std::string& err);

// The plan of a state copy between per-tensor (or flat) state buffers and one
// blocked buffer: `list` describes the state as a step would see it without
// ADAMW_BLOCKED_STATE (streams 2-4, flat_mask bits 2-4 and ADAMW_FLAT_PAD8 as for
// a step; streams 0 and 1 are not used), `esz` the step's element sizes.  The
// pieces are those of the blocked plan (split at block edges), one copy segment
// each, with both sides' addresses; `blocked_bytes` is the blocked buffer's size.
struct CopyPlan {
    std::vector<DevCopySeg> segs;
    std::vector<DevChunk> chunks;
    int64_t blocked_bytes = 0;
};
adamw_status build_copy_plan(const int esz[kStreams], const adamw_tensor_list* list, uint64_t blocked,
                             CopyPlan* out, std::string& err);

// Device bytes of chunk `c` of `plan` in each stream: [lo[s], hi[s]) holds the
// elements [off, off + count) of the chunk's segment at the stream's element
// size esz[s]; lo = hi = 0 for a stream the plan does not touch.  These are
// exactly the bytes the kernels read and write for the chunk: a vector chunk's
// lanes take its 8-element packs [0, count / 8), an element chunk's lanes its
// elements [0, count).
void chunk_bytes(const Plan& plan, size_t c, const int esz[kStreams], uint64_t lo[kStreams], uint64_t hi[kStreams]);

// The argument checks of the entry points (error text in `err`).
adamw_status check_hparams(const adamw_hparams* hp, std::string& err);
adamw_status check_scaler(const adamw_loss_scaler* sc, std::string& err);
adamw_status basic_list_check(const adamw_tensor_list* list, std::string& err);
adamw_status check_pure_precision(const adamw_pure_precision* prec, std::string& err);

// Plan cache policy of one stream.  `pinned` lists the stream's slots in
// most-recently-used order, true for a slot that a captured HIP graph holds
// (its device table must stay as it is for as long as the graph may replay).
// Returns the slot a new plan goes to: `pinned.size()` (a new slot) while fewer
// than `cap` slots are unpinned, else the least recently used unpinned slot.
// A pinned slot is never chosen.
size_t choose_plan_slot(const std::vector<bool>& pinned, size_t cap);

// The exact inputs a plan depends on, for caching (`tag` distinguishes kernels).
void plan_key(int64_t tag, const int esz[kStreams], const adamw_tensor_list* list, int64_t chunk_elems,
              std::vector<int64_t>& key);

}  // namespace adamw
