// Internal declarations shared by the host API and the kernel launchers of
// libspd.  Not installed; the public ABI is include/spd.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace spd {

// Work decompositions (values match spd_mode in include/spd.h).
constexpr int kModeAuto = 0;
constexpr int kModeHeads = 1;  // waves of a workgroup split the heads, share the rows
constexpr int kModeRows = 2;   // waves of a workgroup split the rows, share 16 heads
constexpr int kModeWide = 3;   // heads mode on 32-head waves, asked for explicitly
constexpr int kModeSplit = 4;  // (token, heads, partition) workgroups merged in-kernel

// Work decomposition of one attention call, fixed by scalar arguments only so
// that the grid never depends on device data.
struct AttnPlan {
  int mode;            // kModeHeads, kModeRows or kModeSplit
  int waves;           // waves per workgroup
  int heads_per_group; // heads per workgroup
  int head_groups;     // ceil(H / heads_per_group)
  int wide;            // heads mode with 32-head waves (attn_wide_kernel); FP8 plans:
                       // the wide_waves of launch_attention_fp8 (0, 2, 3 or 4)
  int splits;          // partitions of a slice (1 = no split-L)
  int split_rows;      // rows per partition (multiple of 32); huge when splits == 1
  int parities;        // split mode: waves per head block (2 or 4); 1 otherwise
  int bal_slots;       // split mode: > 0 for a balanced plan (workgroups per head group,
                       // partitions sized in the kernel from the slices' lengths); 0 otherwise
  size_t workspace_bytes;
};

bool attn_supported(int32_t H, int32_t D);
// Returns false when the arguments cannot form a plan.
bool make_attn_plan(int32_t N, int32_t H, int32_t D, int32_t max_len, int32_t split_rows,
                    int32_t mode, AttnPlan* plan);
// Plan of an attention call over an FP8 pool: split mode as make_attn_plan
// chooses it (D >= 128), else rows mode or one of the 32-head-wave
// decompositions (plan->wide).  mode: kModeAuto, kModeRows, kModeWide or
// kModeSplit.  False when the arguments cannot form a plan.
bool make_fp8_plan(int32_t N, int32_t H, int32_t D, int32_t max_len, int32_t split_rows,
                   int32_t mode, AttnPlan* plan);

struct AttnArgs {
  const uint16_t* q;         // [N][H][D] bf16 bits
  const uint16_t* kv;        // [num_rows][D] bf16 bits
  const int32_t* kv_indices;
  const int32_t* kv_indptr;  // [N+1]
  const float* sink;         // [H]
  uint16_t* out;             // [N][H][D] bf16 bits
  float* ws;                 // split partials (splits > 1)
  float qk_scale;            // softmax_scale * log2(e)
  int32_t N, H, head_groups, splits, split_rows;
  // split mode: 1 when the whole grid can be resident at once (one
  // workgroup per CU), so that a merging workgroup may wait a bounded time
  // for the other partitions; 0 = never wait (the last arrival merges)
  int32_t split_wait;
  // split mode, balanced plan (> 0): the workgroups of a head group, whose
  // partitions the kernel sizes from kv_indptr (split_rows and splits unused)
  int32_t bal_slots;
  // Page transform (sparse_decode_attn_paged): when paged != 0 each token's
  // rows are derived from these, as build_decode_indices derives them, and
  // kv_indices / kv_indptr are not read.  win + topk <= kPagedMaxLen, no split.
  int32_t paged;
  const int32_t* state_slot;   // [N]
  const int32_t* swa_len;      // [N]
  const int32_t* comp_pos;     // [N][topk] or null
  const int32_t* block_table;  // [N][max_blocks]
  int32_t topk, max_blocks, win, k_per_block, swa_pages;
  uint32_t comp_limit;         // min(max_blocks * k_per_block, 2^31)
  // Shared-window prefill (sparse_prefill_attn): kv_indices is one index
  // stream and token t attends to kv_indices[win_start[t] : + win_len[t]];
  // a workgroup takes tokens_per_group consecutive tokens, whose
  // tokens_per_group * H query rows fill its 2 or 4 waves of 32 heads.
  const int32_t* win_start;    // [N]
  const int32_t* win_len;      // [N]
  int64_t stream_len;
  int32_t tokens_per_group;
  // FP8 pool (sparse_decode_attn_fp8): row r is kv_scale[r] * e4m3(kv8[r][:]);
  // kv is not read.
  const uint8_t* kv8;          // [num_rows][D] OCP e4m3 codes
  const float* kv_scale;       // [num_rows]
};

// Longest per-token list the paged entry point accepts (win + topk): the
// whole list is built in LDS before the first row is loaded.
constexpr int kPagedMaxLen = 2048;

hipError_t launch_attention(const AttnArgs& args, int D, const AttnPlan& plan, hipStream_t stream);

// Split mode (attn_split.hip): workgroup = (token, heads_per_group heads,
// partition), the partitions of a (token, head group) merged inside the
// kernel.  Fixed plans cut every slice into partitions of split_rows rows
// (grid N x head_groups x splits); balanced plans (bal_slots > 0) give each
// head group bal_slots workgroups, which the kernel deals out as the
// partitions of this call's slices.  The workspace holds one softmax state per
// workgroup and the arrival counters of every (token, head group); the
// counters must be zero before the first call and every call leaves them
// zero.
size_t split_workspace_bytes(int32_t N, int32_t D, const AttnPlan& plan);
// Offset of the arrival counters in that workspace (they run from there to
// its end).
size_t split_counters_offset(int32_t N, int32_t D, const AttnPlan& plan);
// fp8: the rows are args.kv8 / args.kv_scale (D >= 128), else args.kv.
hipError_t launch_split(const AttnArgs& args, int D, const AttnPlan& plan, bool fp8,
                        hipStream_t stream);

// Attention over an FP8 pool (args.kv8 / args.kv_scale replace args.kv), in
// the plan of make_fp8_plan: split mode (attn_split.hip), or no split with
// plan.wide = 0: rows decomposition (workgroup = token x 16 heads); 2 or 4:
// workgroups of 32 * wide heads on 32-head waves (H % (32 * wide) == 0,
// D >= 128); 3: workgroups of 64 heads on four 32-head waves, two parities of
// each head block (H % 64 == 0, D >= 128).
hipError_t launch_attention_fp8(const AttnArgs& args, int D, const AttnPlan& plan,
                                hipStream_t stream);

// Shared-window prefill: 32-head waves, two or four per workgroup
// (tokens_per_group x H = 64 or 128 query rows), no split.
hipError_t launch_prefill(const AttnArgs& args, int D, hipStream_t stream);

struct BuildArgs {
  const int32_t* state_slot;
  const int32_t* swa_len;
  const int32_t* comp_pos;
  const int32_t* block_table;
  int32_t* kv_indptr;
  int32_t* kv_indices;
  int32_t topk, max_blocks, N, win, k_per_block, swa_pages;
  int32_t comp_vec4;    // comp_pos rows are 16-byte aligned (aligned base, topk % 4 == 0)
  uint32_t comp_limit;  // min(max_blocks * k_per_block, 2^31): entry p is valid iff 0 <= p < it
};

hipError_t launch_build_indices(const BuildArgs& args, hipStream_t stream);

hipError_t launch_validate_indices(const int32_t* kv_indices, int64_t num_indices,
                                   const int32_t* kv_indptr, int32_t N, int64_t num_rows,
                                   unsigned long long* first_bad_dev, hipStream_t stream);

}  // namespace spd
