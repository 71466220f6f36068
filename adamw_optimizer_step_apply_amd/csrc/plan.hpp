// plan.hpp -- host-side planner: tensor list (or ZeRO shard of it) -> segments
// and workgroup chunks for the fused AdamW kernels.
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

// The exact inputs a plan depends on, for caching (`tag` distinguishes kernels).
void plan_key(int64_t tag, const int esz[kStreams], const adamw_tensor_list* list, int64_t chunk_elems,
              std::vector<int64_t>& key);

}  // namespace adamw
