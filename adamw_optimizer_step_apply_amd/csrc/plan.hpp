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

// Element size in bytes of stream s for this mode/dtype (0 = stream unused).
int stream_esize(adamw_mode mode, adamw_dtype p_dtype, int s, bool for_check);

// Checks the mode/dtype pair.  Returns ADAMW_OK or an error with `err` set.
adamw_status check_mode(adamw_mode mode, adamw_dtype p_dtype, bool for_check, std::string& err);

// Validates the list and, if `out` is non-null, builds the plan into it.
// No HIP call.
adamw_status build_plan(adamw_mode mode, adamw_dtype p_dtype, const adamw_tensor_list* list, bool for_check,
                        int64_t chunk_elems, Plan* out, std::string& err);

// The exact inputs a plan depends on, for caching.
void plan_key(adamw_mode mode, adamw_dtype p_dtype, const adamw_tensor_list* list, bool for_check,
              int64_t chunk_elems, std::vector<int64_t>& key);

}  // namespace adamw
