// Host-side pieces of the C ABI shared between its source files.  Not
// installed; the public ABI is include/spd.h.
#pragma once

#include "spd.h"
#include "spd_internal.h"

namespace spd {

// The host checks and plan of sparse_decode_attn_ex, shared with its
// allocation-free variant: on SPD_OK either *empty (N == 0: nothing to
// launch) or *a holds every argument but the workspace and *plan the plan.
spd_status prepare_attn_ex(const void* q, const void* unified_kv, int64_t num_rows,
                           const int32_t* kv_indices, const int32_t* kv_indptr,
                           const float* attn_sink, float softmax_scale, void* out, int32_t N,
                           int32_t H, int32_t D, int32_t max_len, int32_t split_rows, int32_t mode,
                           AttnArgs* a, AttnPlan* plan, bool* empty);

}  // namespace spd
