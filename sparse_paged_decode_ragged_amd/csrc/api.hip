// api.hip -- the exported C ABI of libspd (declared in include/spd.h).
//
// Every argument check runs on the host before the first HIP call, so the
// validation paths work (and are tested) on machines without a GPU.  No entry
// point but spd_validate_indices allocates or synchronises.
#include <math.h>
#include <stdint.h>

#include "api_internal.h"
#include "spd.h"
#include "spd_internal.h"
#include "store_internal.h"

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

constexpr double kLog2eD = 1.4426950408889634073599;

// The mode and shape checks of sparse_decode_attn_fp8_ex (host only).
spd_status fp8_mode_status(int32_t H, int32_t D, int32_t split_rows, int32_t mode) {
  if (mode != SPD_MODE_AUTO && mode != SPD_MODE_HEADS && mode != SPD_MODE_ROWS &&
      mode != SPD_MODE_WIDE && mode != SPD_MODE_SPLIT)
    return SPD_ERR_INVALID_ARG;
  if (!spd::attn_supported(H, D) || mode == SPD_MODE_HEADS) return SPD_ERR_UNSUPPORTED;
  // split and wide modes need D >= 128 (wide: H % 64 == 0); only split mode
  // (asked for, or taken by the automatic plan) cuts slices into split_rows
  if ((mode == SPD_MODE_SPLIT || mode == SPD_MODE_WIDE || split_rows != 0) && D < 128)
    return SPD_ERR_UNSUPPORTED;
  if (mode == SPD_MODE_WIDE && H % 64 != 0) return SPD_ERR_UNSUPPORTED;
  if (mode != SPD_MODE_SPLIT && mode != SPD_MODE_AUTO && split_rows != 0) return SPD_ERR_UNSUPPORTED;
  return SPD_OK;
}

}  // namespace

namespace spd {

spd_status prepare_attn_ex(const void* q, const void* unified_kv, int64_t num_rows,
                           const int32_t* kv_indices, const int32_t* kv_indptr,
                           const float* attn_sink, float softmax_scale, void* out, int32_t N,
                           int32_t H, int32_t D, int32_t max_len, int32_t split_rows, int32_t mode,
                           AttnArgs* a, AttnPlan* plan, bool* empty) {
  *empty = false;
  if (N < 0 || H <= 0 || D <= 0 || num_rows <= 0 || max_len < 0 || split_rows < 0)
    return SPD_ERR_INVALID_ARG;
  if (mode != SPD_MODE_AUTO && mode != SPD_MODE_HEADS && mode != SPD_MODE_ROWS &&
      mode != SPD_MODE_WIDE && mode != SPD_MODE_SPLIT)
    return SPD_ERR_INVALID_ARG;
  if (mode == SPD_MODE_ROWS && split_rows != 0) return SPD_ERR_UNSUPPORTED;
  if (!isfinite(softmax_scale)) return SPD_ERR_INVALID_ARG;
  if (!attn_supported(H, D)) return SPD_ERR_UNSUPPORTED;
  if (mode == SPD_MODE_WIDE && (split_rows != 0 || H % 64 != 0)) return SPD_ERR_UNSUPPORTED;
  if (N == 0) {
    *empty = true;
    return SPD_OK;
  }
  if (!q || !unified_kv || !kv_indices || !kv_indptr || !attn_sink || !out)
    return SPD_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(unified_kv, 16) || !aligned(out, 16) || !aligned(kv_indices, 4) ||
      !aligned(kv_indptr, 4) || !aligned(attn_sink, 4))
    return SPD_ERR_INVALID_ARG;
  if (num_rows > (int64_t)1 << 40) return SPD_ERR_INVALID_ARG;
  const size_t qo_bytes = (size_t)N * H * D * 2;
  if (overlap(out, qo_bytes, q, qo_bytes) ||
      overlap(out, qo_bytes, unified_kv, (size_t)num_rows * D * 2) ||
      overlap(out, qo_bytes, attn_sink, (size_t)H * 4) ||
      overlap(out, qo_bytes, kv_indptr, (size_t)(N + 1) * 4))
    return SPD_ERR_INVALID_ARG;
  if (!make_attn_plan(N, H, D, max_len, split_rows, mode, plan)) return SPD_ERR_INVALID_ARG;
  a->q = static_cast<const uint16_t*>(q);
  a->kv = static_cast<const uint16_t*>(unified_kv);
  a->kv_indices = kv_indices;
  a->kv_indptr = kv_indptr;
  a->sink = attn_sink;
  a->out = static_cast<uint16_t*>(out);
  a->ws = nullptr;
  a->qk_scale = (float)((double)softmax_scale * kLog2eD);
  a->N = N;
  a->H = H;
  a->head_groups = plan->head_groups;
  a->splits = plan->splits;
  a->split_rows = plan->split_rows;
  return SPD_OK;
}

}  // namespace spd

extern "C" {

SPD_API const char* spd_status_string(spd_status s) {
  switch (s) {
    case SPD_OK: return "SPD_OK";
    case SPD_ERR_INVALID_ARG: return "SPD_ERR_INVALID_ARG";
    case SPD_ERR_UNSUPPORTED: return "SPD_ERR_UNSUPPORTED";
    case SPD_ERR_WORKSPACE: return "SPD_ERR_WORKSPACE";
    case SPD_ERR_HIP: return "SPD_ERR_HIP";
  }
  return "SPD_ERR_UNKNOWN";
}

SPD_API int spd_version(void) { return 400; }

SPD_API int sparse_decode_attn_can_use(int32_t H, int32_t D) {
  return spd::attn_supported(H, D) ? 1 : 0;
}

SPD_API size_t sparse_decode_attn_workspace_size(int32_t N, int32_t H, int32_t D, int32_t max_len,
                                                 int32_t split_rows, int32_t mode) {
  spd::AttnPlan plan;
  if (!spd::make_attn_plan(N, H, D, max_len, split_rows, mode, &plan)) return 0;
  return plan.workspace_bytes;
}

SPD_API spd_status sparse_decode_attn_plan_info(int32_t N, int32_t H, int32_t D, int32_t max_len,
                                                int32_t split_rows, int32_t mode, int32_t* info) {
  if (!info || N < 0 || H <= 0 || D <= 0 || max_len < 0 || split_rows < 0) return SPD_ERR_INVALID_ARG;
  if (mode != SPD_MODE_AUTO && mode != SPD_MODE_HEADS && mode != SPD_MODE_ROWS &&
      mode != SPD_MODE_WIDE && mode != SPD_MODE_SPLIT)
    return SPD_ERR_INVALID_ARG;
  if (!spd::attn_supported(H, D)) return SPD_ERR_UNSUPPORTED;
  if (mode == SPD_MODE_ROWS && split_rows != 0) return SPD_ERR_UNSUPPORTED;
  if (mode == SPD_MODE_WIDE && (split_rows != 0 || H % 64 != 0)) return SPD_ERR_UNSUPPORTED;
  spd::AttnPlan plan;
  if (!spd::make_attn_plan(N, H, D, max_len, split_rows, mode, &plan)) return SPD_ERR_INVALID_ARG;
  info[0] = plan.mode;
  info[1] = plan.heads_per_group;
  info[2] = plan.head_groups;
  info[3] = plan.splits;
  info[4] = plan.split_rows;
  info[5] = plan.wide;
  info[6] = plan.parities;
  return SPD_OK;
}

SPD_API spd_status sparse_decode_attn_ex(const void* q, const void* unified_kv, int64_t num_rows,
                                         const int32_t* kv_indices, const int32_t* kv_indptr,
                                         const float* attn_sink, float softmax_scale, void* out,
                                         int32_t N, int32_t H, int32_t D, int32_t max_len,
                                         int32_t split_rows, int32_t mode, void* workspace,
                                         size_t workspace_bytes, void* stream) {
  spd::AttnArgs a{};
  spd::AttnPlan plan{};
  bool empty = false;
  const spd_status st =
      spd::prepare_attn_ex(q, unified_kv, num_rows, kv_indices, kv_indptr, attn_sink, softmax_scale,
                           out, N, H, D, max_len, split_rows, mode, &a, &plan, &empty);
  if (st != SPD_OK || empty) return st;
  if (plan.workspace_bytes > 0) {
    if (!workspace || workspace_bytes < plan.workspace_bytes) return SPD_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return SPD_ERR_INVALID_ARG;
  }
  a.ws = static_cast<float*>(workspace);
  const hipError_t e = spd::launch_attention(a, D, plan, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SPD_OK : SPD_ERR_HIP;
}

SPD_API spd_status sparse_decode_attn(const void* q, const void* unified_kv, int64_t num_rows,
                                      const int32_t* kv_indices, const int32_t* kv_indptr,
                                      const float* attn_sink, float softmax_scale, void* out,
                                      int32_t N, int32_t H, int32_t D, void* stream) {
  return sparse_decode_attn_ex(q, unified_kv, num_rows, kv_indices, kv_indptr, attn_sink,
                               softmax_scale, out, N, H, D, 0, 0, SPD_MODE_AUTO, nullptr, 0,
                               stream);
}

SPD_API spd_status sparse_decode_attn_paged(
    const void* q, const void* unified_kv, int64_t num_rows, const int32_t* state_slot,
    const int32_t* swa_len, const int32_t* comp_pos, int32_t topk, const int32_t* block_table,
    int32_t max_blocks, int32_t win, int32_t k_per_block, int32_t swa_pages,
    const float* attn_sink, float softmax_scale, void* out, int32_t N, int32_t H, int32_t D,
    int32_t mode, void* stream) {
  if (N < 0 || H <= 0 || D <= 0 || num_rows <= 0) return SPD_ERR_INVALID_ARG;
  if (topk < 0 || win <= 0 || k_per_block <= 0 || swa_pages < 0 || max_blocks < 0)
    return SPD_ERR_INVALID_ARG;
  if (comp_pos == nullptr && topk > 0) return SPD_ERR_INVALID_ARG;
  if (comp_pos != nullptr && topk > 0 && (block_table == nullptr || max_blocks <= 0))
    return SPD_ERR_INVALID_ARG;
  if (mode != SPD_MODE_AUTO && mode != SPD_MODE_HEADS && mode != SPD_MODE_ROWS &&
      mode != SPD_MODE_WIDE)
    return SPD_ERR_INVALID_ARG;
  if (!isfinite(softmax_scale)) return SPD_ERR_INVALID_ARG;
  if (!spd::attn_supported(H, D)) return SPD_ERR_UNSUPPORTED;
  if (mode == SPD_MODE_WIDE && H % 64 != 0) return SPD_ERR_UNSUPPORTED;
  if ((int64_t)win + topk > spd::kPagedMaxLen) return SPD_ERR_UNSUPPORTED;
  if (N == 0) return SPD_OK;
  if (!q || !unified_kv || !state_slot || !swa_len || !attn_sink || !out) return SPD_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(unified_kv, 16) || !aligned(out, 16) || !aligned(state_slot, 4) ||
      !aligned(swa_len, 4) || !aligned(attn_sink, 4) ||
      (topk > 0 && (!aligned(comp_pos, 4) || !aligned(block_table, 4))))
    return SPD_ERR_INVALID_ARG;
  if (num_rows > (int64_t)1 << 40) return SPD_ERR_INVALID_ARG;
  const size_t qo_bytes = (size_t)N * H * D * 2;
  if (overlap(out, qo_bytes, q, qo_bytes) ||
      overlap(out, qo_bytes, unified_kv, (size_t)num_rows * D * 2) ||
      overlap(out, qo_bytes, attn_sink, (size_t)H * 4))
    return SPD_ERR_INVALID_ARG;

  // Each token's list is built whole in LDS, so no split-L (max_len 0 asks
  // the planner for none).
  spd::AttnPlan plan;
  if (!spd::make_attn_plan(N, H, D, 0, 0, mode, &plan) || plan.splits != 1)
    return SPD_ERR_INVALID_ARG;

  spd::AttnArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.kv = static_cast<const uint16_t*>(unified_kv);
  a.sink = attn_sink;
  a.out = static_cast<uint16_t*>(out);
  a.qk_scale = (float)((double)softmax_scale * kLog2eD);
  a.N = N;
  a.H = H;
  a.head_groups = plan.head_groups;
  a.splits = 1;
  a.split_rows = plan.split_rows;
  a.paged = 1;
  a.state_slot = state_slot;
  a.swa_len = swa_len;
  a.comp_pos = topk > 0 ? comp_pos : nullptr;
  a.block_table = block_table;
  a.topk = topk;
  a.max_blocks = max_blocks;
  a.win = win;
  a.k_per_block = k_per_block;
  a.swa_pages = swa_pages;
  const int64_t lim = (int64_t)max_blocks * k_per_block;
  a.comp_limit = (uint32_t)(lim < (int64_t(1) << 31) ? lim : (int64_t(1) << 31));
  const hipError_t e = spd::launch_attention(a, D, plan, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SPD_OK : SPD_ERR_HIP;
}

SPD_API spd_status sparse_prefill_attn(const void* q, const void* unified_kv, int64_t num_rows,
                                       const int32_t* kv_stream, int64_t stream_len,
                                       const int32_t* win_start, const int32_t* win_len,
                                       const float* attn_sink, float softmax_scale, void* out,
                                       int32_t N, int32_t H, int32_t D, int32_t tokens_per_group,
                                       void* stream) {
  if (N < 0 || H <= 0 || D <= 0 || num_rows <= 0 || stream_len < 0 || tokens_per_group < 0)
    return SPD_ERR_INVALID_ARG;
  if (!isfinite(softmax_scale)) return SPD_ERR_INVALID_ARG;
  if ((D != 64 && D != 128 && D != 256 && D != 512) || (H != 32 && H != 64 && H != 128))
    return SPD_ERR_UNSUPPORTED;
  // automatic: 64 query rows (two 32-head waves) per workgroup, one token at
  // H = 64; H = 128 needs four waves for one token
  const int T = tokens_per_group > 0 ? tokens_per_group : (H == 128 ? 1 : 64 / H);
  if ((long long)T * H != 64 && (long long)T * H != 128) return SPD_ERR_UNSUPPORTED;
  if (stream_len > 0x7fffffffLL || num_rows > (int64_t)1 << 40) return SPD_ERR_INVALID_ARG;
  if (N == 0) return SPD_OK;
  if (!q || !unified_kv || !win_start || !win_len || !attn_sink || !out ||
      (stream_len > 0 && !kv_stream))
    return SPD_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(unified_kv, 16) || !aligned(out, 16) || !aligned(win_start, 4) ||
      !aligned(win_len, 4) || !aligned(attn_sink, 4) || (kv_stream && !aligned(kv_stream, 4)))
    return SPD_ERR_INVALID_ARG;
  const size_t qo_bytes = (size_t)N * H * D * 2;
  if (overlap(out, qo_bytes, q, qo_bytes) ||
      overlap(out, qo_bytes, unified_kv, (size_t)num_rows * D * 2) ||
      overlap(out, qo_bytes, attn_sink, (size_t)H * 4) ||
      overlap(out, qo_bytes, win_start, (size_t)N * 4) ||
      overlap(out, qo_bytes, win_len, (size_t)N * 4) ||
      (kv_stream && overlap(out, qo_bytes, kv_stream, (size_t)stream_len * 4)))
    return SPD_ERR_INVALID_ARG;

  spd::AttnArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.kv = static_cast<const uint16_t*>(unified_kv);
  a.kv_indices = kv_stream;
  a.sink = attn_sink;
  a.out = static_cast<uint16_t*>(out);
  a.qk_scale = (float)((double)softmax_scale * kLog2eD);
  a.N = N;
  a.H = H;
  a.head_groups = 1;
  a.splits = 1;
  a.split_rows = 1 << 30;
  a.win_start = win_start;
  a.win_len = win_len;
  a.stream_len = stream_len;
  a.tokens_per_group = T;
  const hipError_t e = spd::launch_prefill(a, D, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SPD_OK : SPD_ERR_HIP;
}

SPD_API size_t sparse_decode_attn_fp8_workspace_size(int32_t N, int32_t H, int32_t D,
                                                     int32_t max_len, int32_t split_rows,
                                                     int32_t mode) {
  spd::AttnPlan plan;
  if (!spd::make_fp8_plan(N, H, D, max_len, split_rows, mode, &plan)) return 0;
  return plan.workspace_bytes;
}

SPD_API spd_status sparse_decode_attn_fp8_plan_info(int32_t N, int32_t H, int32_t D,
                                                    int32_t max_len, int32_t split_rows,
                                                    int32_t mode, int32_t* info) {
  if (!info || N < 0 || H <= 0 || D <= 0 || max_len < 0 || split_rows < 0) return SPD_ERR_INVALID_ARG;
  const spd_status ms = fp8_mode_status(H, D, split_rows, mode);
  if (ms != SPD_OK) return ms;
  spd::AttnPlan plan;
  if (!spd::make_fp8_plan(N, H, D, max_len, split_rows, mode, &plan)) return SPD_ERR_INVALID_ARG;
  info[0] = plan.mode;
  info[1] = plan.heads_per_group;
  info[2] = plan.head_groups;
  info[3] = plan.splits;
  info[4] = plan.split_rows;
  info[5] = plan.wide;
  info[6] = plan.parities;
  return SPD_OK;
}

SPD_API spd_status sparse_decode_attn_fp8_ex(const void* q, const void* kv_fp8,
                                             const float* kv_scale, int64_t num_rows,
                                             const int32_t* kv_indices, const int32_t* kv_indptr,
                                             const float* attn_sink, float softmax_scale,
                                             void* out, int32_t N, int32_t H, int32_t D,
                                             int32_t max_len, int32_t split_rows, int32_t mode,
                                             void* workspace, size_t workspace_bytes,
                                             void* stream) {
  if (N < 0 || H <= 0 || D <= 0 || num_rows <= 0 || max_len < 0 || split_rows < 0)
    return SPD_ERR_INVALID_ARG;
  if (!isfinite(softmax_scale)) return SPD_ERR_INVALID_ARG;
  const spd_status ms = fp8_mode_status(H, D, split_rows, mode);
  if (ms != SPD_OK) return ms;
  if (N == 0) return SPD_OK;
  if (!q || !kv_fp8 || !kv_scale || !kv_indices || !kv_indptr || !attn_sink || !out)
    return SPD_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(kv_fp8, 16) || !aligned(out, 16) || !aligned(kv_scale, 4) ||
      !aligned(kv_indices, 4) || !aligned(kv_indptr, 4) || !aligned(attn_sink, 4))
    return SPD_ERR_INVALID_ARG;
  if (num_rows > (int64_t)1 << 40) return SPD_ERR_INVALID_ARG;
  const size_t qo_bytes = (size_t)N * H * D * 2;
  if (overlap(out, qo_bytes, q, qo_bytes) ||
      overlap(out, qo_bytes, kv_fp8, (size_t)num_rows * D) ||
      overlap(out, qo_bytes, kv_scale, (size_t)num_rows * 4) ||
      overlap(out, qo_bytes, attn_sink, (size_t)H * 4) ||
      overlap(out, qo_bytes, kv_indptr, (size_t)(N + 1) * 4))
    return SPD_ERR_INVALID_ARG;
  spd::AttnPlan plan;
  if (!spd::make_fp8_plan(N, H, D, max_len, split_rows, mode, &plan)) return SPD_ERR_INVALID_ARG;
  if (plan.workspace_bytes > 0) {
    if (!workspace || workspace_bytes < plan.workspace_bytes) return SPD_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return SPD_ERR_INVALID_ARG;
  }

  spd::AttnArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.kv8 = static_cast<const uint8_t*>(kv_fp8);
  a.kv_scale = kv_scale;
  a.kv_indices = kv_indices;
  a.kv_indptr = kv_indptr;
  a.sink = attn_sink;
  a.out = static_cast<uint16_t*>(out);
  a.ws = static_cast<float*>(workspace);
  a.qk_scale = (float)((double)softmax_scale * kLog2eD);
  a.N = N;
  a.H = H;
  a.head_groups = plan.head_groups;
  a.splits = plan.splits;
  a.split_rows = plan.split_rows;
  const hipError_t e = spd::launch_attention_fp8(a, D, plan, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SPD_OK : SPD_ERR_HIP;
}

SPD_API spd_status sparse_decode_attn_fp8(const void* q, const void* kv_fp8,
                                          const float* kv_scale, int64_t num_rows,
                                          const int32_t* kv_indices, const int32_t* kv_indptr,
                                          const float* attn_sink, float softmax_scale, void* out,
                                          int32_t N, int32_t H, int32_t D, void* stream) {
  return sparse_decode_attn_fp8_ex(q, kv_fp8, kv_scale, num_rows, kv_indices, kv_indptr,
                                   attn_sink, softmax_scale, out, N, H, D, 0, 0, SPD_MODE_AUTO,
                                   nullptr, 0, stream);
}

SPD_API spd_status quantize_kv_fp8(const void* src, const int32_t* slots, int32_t n, int32_t D,
                                   void* kv_fp8, float* kv_scale, int64_t num_rows, void* stream) {
  if (n < 0 || D <= 0 || num_rows <= 0) return SPD_ERR_INVALID_ARG;
  if (D != 64 && D != 128 && D != 256 && D != 512) return SPD_ERR_UNSUPPORTED;
  if (n == 0) return SPD_OK;
  if (!src || !kv_fp8 || !kv_scale) return SPD_ERR_INVALID_ARG;
  if (!aligned(src, 16) || !aligned(kv_fp8, 16) || !aligned(kv_scale, 4) ||
      (slots && !aligned(slots, 4)))
    return SPD_ERR_INVALID_ARG;
  if (!slots && n > num_rows) return SPD_ERR_INVALID_ARG;
  if (num_rows > (int64_t)1 << 40) return SPD_ERR_INVALID_ARG;
  const size_t src_bytes = (size_t)n * D * 2;
  if (overlap(src, src_bytes, kv_fp8, (size_t)num_rows * D) ||
      overlap(src, src_bytes, kv_scale, (size_t)num_rows * 4) ||
      overlap(kv_fp8, (size_t)num_rows * D, kv_scale, (size_t)num_rows * 4) ||
      (slots && (overlap(slots, (size_t)n * 4, kv_fp8, (size_t)num_rows * D) ||
                 overlap(slots, (size_t)n * 4, kv_scale, (size_t)num_rows * 4))))
    return SPD_ERR_INVALID_ARG;

  spd::QuantArgs a{};
  a.src = static_cast<const uint16_t*>(src);
  a.slots = slots;
  a.kv8 = static_cast<uint8_t*>(kv_fp8);
  a.kv_scale = kv_scale;
  a.n = n;
  a.num_rows = num_rows;
  const hipError_t e = spd::launch_quantize_fp8(a, D, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SPD_OK : SPD_ERR_HIP;
}

SPD_API spd_status fused_qk_norm_rope_swa_store(
    const void* q, void* q_out, const void* kv, const float* q_weight, const float* kv_weight,
    float eps, const int32_t* positions, const float* cos_sin, int32_t max_pos, int32_t rope_dim,
    const int32_t* state_slot, int32_t win, void* unified_kv, void* kv_fp8, float* kv_scale,
    int64_t num_rows, int32_t N, int32_t H, int32_t D, void* stream) {
  if (N < 0 || H <= 0 || D <= 0 || win <= 0 || max_pos < 0 || num_rows <= 0)
    return SPD_ERR_INVALID_ARG;
  if (rope_dim < 0 || rope_dim > D || (rope_dim & 1) || !(eps >= 0.0f) || !isfinite(eps))
    return SPD_ERR_INVALID_ARG;
  if (D != 64 && D != 128 && D != 256 && D != 512) return SPD_ERR_UNSUPPORTED;
  if (!unified_kv && !kv_fp8) return SPD_ERR_INVALID_ARG;  // the KV row must go somewhere
  if (kv_fp8 && !kv_scale) return SPD_ERR_INVALID_ARG;
  if ((int64_t)N * H > ((int64_t)1 << 40) || num_rows > ((int64_t)1 << 40)) return SPD_ERR_INVALID_ARG;
  if (N == 0) return SPD_OK;
  if (!q || !q_out || !kv || !q_weight || !kv_weight || !positions || !state_slot ||
      (rope_dim > 0 && (!cos_sin || max_pos == 0)))
    return SPD_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(q_out, 16) || !aligned(kv, 16) || !aligned(q_weight, 4) ||
      !aligned(kv_weight, 4) || !aligned(positions, 4) || !aligned(state_slot, 4) ||
      (cos_sin && !aligned(cos_sin, 4)) || (unified_kv && !aligned(unified_kv, 16)) ||
      (kv_fp8 && !aligned(kv_fp8, 16)) || (kv_scale && !aligned(kv_scale, 4)))
    return SPD_ERR_INVALID_ARG;
  const size_t qb = (size_t)N * H * D * 2, kvb = (size_t)N * D * 2;
  const size_t pool16 = (size_t)num_rows * D * 2, pool8 = (size_t)num_rows * D;
  // q_out may be q itself (in place), but no other overlap
  if ((q_out != q && overlap(q_out, qb, q, qb)) || overlap(q_out, qb, kv, kvb) ||
      (unified_kv && (overlap(unified_kv, pool16, q_out, qb) || overlap(unified_kv, pool16, q, qb) ||
                      overlap(unified_kv, pool16, kv, kvb))) ||
      (kv_fp8 && (overlap(kv_fp8, pool8, q_out, qb) || overlap(kv_fp8, pool8, q, qb) ||
                  overlap(kv_fp8, pool8, kv, kvb) || overlap(kv_scale, (size_t)num_rows * 4, kv_fp8, pool8) ||
                  overlap(kv_scale, (size_t)num_rows * 4, q_out, qb))) ||
      (unified_kv && kv_fp8 && (overlap(unified_kv, pool16, kv_fp8, pool8) ||
                                overlap(unified_kv, pool16, kv_scale, (size_t)num_rows * 4))))
    return SPD_ERR_INVALID_ARG;

  spd::ProducerArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.q_out = static_cast<uint16_t*>(q_out);
  a.kv = static_cast<const uint16_t*>(kv);
  a.q_weight = q_weight;
  a.kv_weight = kv_weight;
  a.eps = eps;
  a.positions = positions;
  a.cos_sin = cos_sin;
  a.max_pos = max_pos;
  a.rope_dim = rope_dim;
  a.state_slot = state_slot;
  a.win = win;
  a.kv_bf16 = static_cast<uint16_t*>(unified_kv);
  a.kv8 = static_cast<uint8_t*>(kv_fp8);
  a.kv_scale = kv_scale;
  a.num_rows = num_rows;
  a.N = N;
  a.H = H;
  const hipError_t e = spd::launch_producer(a, D, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SPD_OK : SPD_ERR_HIP;
}

SPD_API spd_status build_decode_indices(const int32_t* state_slot, const int32_t* swa_len,
                                        const int32_t* comp_pos, int32_t topk,
                                        const int32_t* block_table, int32_t max_blocks, int32_t N,
                                        int32_t win, int32_t k_per_block, int32_t swa_pages,
                                        int32_t* kv_indptr, int32_t* kv_indices,
                                        int64_t indices_capacity, void* stream) {
  if (N < 0 || topk < 0 || win <= 0 || k_per_block <= 0 || swa_pages < 0 || max_blocks < 0 ||
      indices_capacity < 0)
    return SPD_ERR_INVALID_ARG;
  if (comp_pos == nullptr && topk > 0) return SPD_ERR_INVALID_ARG;
  if (comp_pos != nullptr && topk > 0 && (block_table == nullptr || max_blocks <= 0))
    return SPD_ERR_INVALID_ARG;
  const int64_t need = (int64_t)N * ((int64_t)win + topk);
  if (need > 0x7fffffffLL || indices_capacity < need) return SPD_ERR_INVALID_ARG;
  if (kv_indptr == nullptr) return SPD_ERR_INVALID_ARG;
  if (N > 0 && (state_slot == nullptr || swa_len == nullptr || kv_indices == nullptr))
    return SPD_ERR_INVALID_ARG;

  spd::BuildArgs a{};
  a.state_slot = state_slot;
  a.swa_len = swa_len;
  a.comp_pos = topk > 0 ? comp_pos : nullptr;
  a.block_table = block_table;
  a.kv_indptr = kv_indptr;
  a.kv_indices = kv_indices;
  a.topk = topk;
  a.max_blocks = max_blocks;
  a.N = N;
  a.win = win;
  a.k_per_block = k_per_block;
  a.swa_pages = swa_pages;
  a.comp_vec4 = a.comp_pos != nullptr && topk % 4 == 0 &&
                (reinterpret_cast<uintptr_t>(comp_pos) & 15) == 0;
  const int64_t lim = (int64_t)max_blocks * k_per_block;
  a.comp_limit = (uint32_t)(lim < (int64_t(1) << 31) ? lim : (int64_t(1) << 31));
  const hipError_t e = spd::launch_build_indices(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SPD_OK : SPD_ERR_HIP;
}

SPD_API spd_status spd_validate_indices(const int32_t* kv_indices, int64_t num_indices,
                                        const int32_t* kv_indptr, int32_t N, int64_t num_rows,
                                        int64_t* first_bad, void* stream) {
  if (N < 0 || num_indices < 0 || num_rows < 0 || !kv_indptr || !first_bad)
    return SPD_ERR_INVALID_ARG;
  if (num_indices > 0 && !kv_indices) return SPD_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  unsigned long long* dev = nullptr;
  if (hipMalloc(&dev, sizeof(unsigned long long)) != hipSuccess) return SPD_ERR_HIP;
  spd_status st = SPD_OK;
  unsigned long long host = ~0ULL;
  if (hipMemcpyAsync(dev, &host, sizeof host, hipMemcpyHostToDevice, s) != hipSuccess ||
      spd::launch_validate_indices(kv_indices, num_indices, kv_indptr, N, num_rows, dev, s) !=
          hipSuccess ||
      hipMemcpyAsync(&host, dev, sizeof host, hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    st = SPD_ERR_HIP;
  (void)hipFree(dev);
  if (st == SPD_OK) *first_bad = host == ~0ULL ? -1 : (int64_t)host;
  return st;
}

}  // extern "C"
