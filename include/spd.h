/*
 * spd.h -- C ABI of libspd: sparse decode attention over a unified paged KV
 * pool, and the decode index builder that feeds it, for AMD Instinct MI355X
 * (gfx950).
 *
 * Source of the contract: sglang PR #28392 summary page, "key source snippet"
 * section (the paged_decode.py module docstring), and the same page's
 * "implementation" and "key files" sections naming the decode index builder
 * write_v4_paged_decode_indices.
 *
 * Conventions for every call:
 *   - All tensor arguments are DEVICE pointers owned by the caller, row-major
 *     and contiguous.  The library keeps no reference after the call returns
 *     (the work is asynchronous on `stream`; buffers must stay alive until
 *     the stream reaches that point).
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *   - Calls never synchronise, never read device data on the host, never
 *     allocate, and launch a grid that depends only on the scalar arguments,
 *     so they may be captured in a HIP graph (the page designs the decode
 *     kernel for graph capture).  spd_validate_indices is the one exception
 *     (a debug call that allocates and synchronises).
 *   - Errors are returned as spd_status; nothing is thrown or aborted across
 *     the ABI.  Argument checks run on the host before any HIP call, so they
 *     also work on a machine without a GPU.
 *   - bf16 means IEEE binary32 truncated to its top 16 bits (1-8-7).
 */
#ifndef SPD_H_
#define SPD_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPD_API __attribute__((visibility("default")))

typedef enum spd_status {
  SPD_OK = 0,
  SPD_ERR_INVALID_ARG = 1, /* null pointer, negative size, bad scalar, misalignment */
  SPD_ERR_UNSUPPORTED = 2, /* shape this library does not implement (see *_can_use) */
  SPD_ERR_WORKSPACE = 3,   /* workspace missing or smaller than *_workspace_size */
  SPD_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed */
} spd_status;

/* Human-readable name of a status code (static string, never NULL). */
SPD_API const char* spd_status_string(spd_status s);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH (0.2.0: SPD_MODE_SPLIT;
 * 0.3.0: sparse_decode_attn_fp8_ex and its split mode; 0.4.0: split plans
 * whose partitions the kernel sizes from the slice lengths). */
SPD_API int spd_version(void);

/*
 * 1 when sparse_decode_attn supports heads H and head width D, else 0.
 * Supported: D in {64, 128, 256, 512}, 1 <= H <= 1024.  Callers own the
 * fallback for anything else (the call then returns SPD_ERR_UNSUPPORTED).
 */
SPD_API int sparse_decode_attn_can_use(int32_t H, int32_t D);

/*
 * Sparse decode attention (page: "key source snippet", caller contract and
 * numerics).  For each query token t and head h:
 *
 *   J = kv_indices[kv_indptr[t] : kv_indptr[t+1]]          (a multiset)
 *   s_j = softmax_scale * dot(q[t,h,:], unified_kv[J_j,:])
 *   out[t,h,:] = sum_j e^(s_j) unified_kv[J_j,:] / (e^(attn_sink[h]) + sum_j e^(s_j))
 *   out[t,h,:] = 0 when J is empty (also when attn_sink[h] = -inf)
 *
 * computed as an online softmax in the log2 domain with
 * qk_scale = softmax_scale * log2(e); one pool row is both key and value; the
 * sink acts as a virtual key in the denominator.  fp32 accumulation, output
 * rounded to bf16 with round-to-nearest-even.
 *
 *   q            [N, H, D] bf16, 16-byte aligned
 *   unified_kv   [num_rows, D] bf16 (page_size 1), 16-byte aligned.  Slots
 *                [0, swa_pages) hold sliding-window entries and slots from
 *                swa_pages on hold compressed entries; this call does not
 *                need to know the split.
 *   kv_indices   [kv_indptr[N]] int32: every entry must lie in [0, num_rows)
 *   kv_indptr    [N+1] int32: kv_indptr[0] == 0, non-decreasing (true prefix
 *                sums; a graph-padded token has kv_indptr[t+1] == kv_indptr[t])
 *   attn_sink    [H] fp32, natural-log logit in the units of the scaled score
 *                (-inf disables the sink)
 *   out          [N, H, D] bf16, 16-byte aligned, must not overlap the inputs
 *
 * The kernel does not check the index preconditions (as on the page, there is
 * no per-entry sentinel test); breaking them is undefined behaviour.  Use
 * spd_validate_indices in debug builds.  N == 0 returns SPD_OK and does
 * nothing.  This form never splits a token's slice across workgroups, so it
 * needs no workspace; sparse_decode_attn_ex adds split-L for long slices.
 */
SPD_API spd_status sparse_decode_attn(const void* q, const void* unified_kv, int64_t num_rows,
                                      const int32_t* kv_indices, const int32_t* kv_indptr,
                                      const float* attn_sink, float softmax_scale, void* out,
                                      int32_t N, int32_t H, int32_t D, void* stream);

/*
 * Work decompositions of sparse_decode_attn_ex.  Both give the same result
 * within the accumulation tolerance; they differ in how the work of one token
 * is spread over workgroups:
 *   SPD_MODE_HEADS: a workgroup takes (token, up to 128 heads, partition);
 *                   its waves split the heads and share every gathered row.
 *                   Waves take 16 heads, or 32 (64 or 128 heads per
 *                   workgroup) when H % 64 == 0, nothing is split and the
 *                   batch gives enough workgroups to fill the chip.
 *   SPD_MODE_ROWS:  a workgroup takes (token, 16 heads); its 4 waves split
 *                   the rows and merge in LDS -- more workgroups for small
 *                   batches without partial results in memory.  No split-L.
 *   SPD_MODE_WIDE:  SPD_MODE_HEADS on 32-head waves whatever the batch size:
 *                   needs H % 64 == 0 and no split-L (SPD_ERR_UNSUPPORTED
 *                   otherwise).
 *   SPD_MODE_SPLIT: a workgroup takes (token, 64 heads, partition) -- 32
 *                   heads when H <= 32 and D >= 128 -- its 4 waves two (or
 *                   four) 16-row streams of each 32-head block; the
 *                   partitions of one (token, head group) are merged inside
 *                   the same kernel, each partition merging a share of the
 *                   columns (no combine kernel).  Up to 32 partitions a
 *                   slice.  With split_rows given, every slice is cut into
 *                   partitions of that many rows.  With split_rows == 0 and
 *                   at most 256 (token, head group) pairs (N <= 512), the
 *                   grid is 256 workgroups, which the kernel deals out as the
 *                   partitions of this call's slices, sized from kv_indptr: the
 *                   least partition length (a multiple of 32 rows, 64 when a
 *                   workgroup takes 32 heads) for which every slice's
 *                   partitions fit sets each slice's partition count, and a
 *                   split slice's rows are then shared evenly among its
 *                   partitions (in whole 32- or 64-row tiles, the last
 *                   partition taking the rest), so a long slice among short
 *                   ones takes more workgroups.  Otherwise with split_rows == 0
 *                   the plan cuts slices only when the batch gives fewer
 *                   than 256 workgroups.  Its workspace holds arrival counters: see
 *                   sparse_decode_attn_ex.
 *   SPD_MODE_AUTO:  SPLIT when split_rows == 0, the batch gives at most
 *                   256 HEADS-mode workgroups and max_len >= 2048 (a batch
 *                   of long slices, partitions sized from the lengths); else
 *                   ROWS when split_rows == 0 and the batch gives fewer than
 *                   256 HEADS-mode workgroups; else HEADS.
 */
typedef enum spd_mode {
  SPD_MODE_AUTO = 0,
  SPD_MODE_HEADS = 1,
  SPD_MODE_ROWS = 2,
  SPD_MODE_WIDE = 3,
  SPD_MODE_SPLIT = 4
} spd_mode;

/*
 * Workspace bytes that sparse_decode_attn_ex needs for (N, H, D, max_len,
 * split_rows, mode); 0 when the plan does not split.  Returns 0 for
 * unsupported or invalid arguments (the call itself then reports the error).
 */
SPD_API size_t sparse_decode_attn_workspace_size(int32_t N, int32_t H, int32_t D, int32_t max_len,
                                                 int32_t split_rows, int32_t mode);

/*
 * The plan sparse_decode_attn_ex would use for these arguments, for callers
 * that size buffers or report what runs: info[0] = mode actually used
 * (SPD_MODE_HEADS, SPD_MODE_ROWS or SPD_MODE_SPLIT), info[1] = heads per
 * workgroup, info[2] = head groups, info[3] = split-L partitions (1 = none;
 * for partitions sized in the kernel, the most a slice can take), info[4] =
 * rows per partition (0 = sized in the kernel from the slice lengths),
 * info[5] = 1 when the heads mode runs on
 * 32-head waves (64 or 128 heads per workgroup) else 0, info[6] = waves per
 * 32-head block (SPD_MODE_SPLIT: 2, or 4 when a workgroup takes 32 heads,
 * the waves taking alternate 16-row tiles of the same heads; else 1).  info is
 * a host array of 7 int32.  Returns
 * SPD_ERR_INVALID_ARG or SPD_ERR_UNSUPPORTED exactly when
 * sparse_decode_attn_ex would.
 */
SPD_API spd_status sparse_decode_attn_plan_info(int32_t N, int32_t H, int32_t D, int32_t max_len,
                                                int32_t split_rows, int32_t mode, int32_t* info);

/*
 * sparse_decode_attn with a chosen plan.  max_len is a capacity bound on
 * every slice length, used only to size the grid and the workspace (a longer
 * slice is still computed correctly, by its last partition); 0 = unknown.
 * split_rows fixes the split-L partition length (rounded up to a multiple of
 * 32; HEADS or SPLIT mode, SPD_ERR_UNSUPPORTED with SPD_MODE_ROWS or
 * SPD_MODE_WIDE); 0 lets the plan choose from N, H and max_len, and in SPLIT
 * mode with at most 256 (token, head group) pairs lets the kernel size the
 * partitions from the slice lengths.  mode is an spd_mode.  HEADS-mode
 * partitions of one token are merged by a combine kernel, SPLIT-mode ones
 * inside the attention kernel (the attention sink is counted once either way).
 * workspace/workspace_bytes: a caller-owned device buffer of at least
 * sparse_decode_attn_workspace_size bytes, 16-byte aligned (may be NULL when
 * that size is 0).  HEADS-mode split-L keeps no state in it between calls.
 * When the plan is SPD_MODE_SPLIT (asked for, or chosen by SPD_MODE_AUTO; see
 * plan_info) the last N * ceil(H / heads per workgroup) * D / (2 * info[6])
 * bytes are arrival counters that must be zero when the call starts: zero the buffer
 * once after allocating it (and again after another plan has used it).  Every
 * call leaves them zero, so one buffer serves any number of calls issued one
 * after another; two calls that run at the same time on one buffer race.
 */
SPD_API spd_status sparse_decode_attn_ex(const void* q, const void* unified_kv, int64_t num_rows,
                                         const int32_t* kv_indices, const int32_t* kv_indptr,
                                         const float* attn_sink, float softmax_scale, void* out,
                                         int32_t N, int32_t H, int32_t D, int32_t max_len,
                                         int32_t split_rows, int32_t mode, void* workspace,
                                         size_t workspace_bytes, void* stream);

/*
 * sparse_decode_attn_ex for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments but the workspace, the same plans, kernels
 * and results, bit for bit.  A plan that needs a workspace (split-L, split
 * mode) uses a static device array of SPD_NOALLOC_WORKSPACE_BYTES (96 MiB)
 * that the library holds on each GPU it runs on until the process ends; the
 * call allocates and frees nothing.  A split-mode call first clears the
 * plan's arrival counters in that array with a small kernel on `stream`.
 *
 * Every call on one GPU shares that GPU's array: two calls that may run at
 * the same time (other streams, other host threads) race on it and give
 * wrong results.  stream must belong to the current device
 * (SPD_ERR_INVALID_ARG otherwise).  SPD_ERR_WORKSPACE when the plan needs
 * more than SPD_NOALLOC_WORKSPACE_BYTES (sparse_decode_attn_workspace_size
 * reports the need; the automatic plans need at most about 68 MB); other
 * errors as sparse_decode_attn_ex.
 */
#define SPD_NOALLOC_WORKSPACE_BYTES ((size_t)96 << 20)
SPD_API spd_status sparse_decode_attn_noalloc(const void* q, const void* unified_kv,
                                              int64_t num_rows, const int32_t* kv_indices,
                                              const int32_t* kv_indptr, const float* attn_sink,
                                              float softmax_scale, void* out, int32_t N, int32_t H,
                                              int32_t D, int32_t max_len, int32_t split_rows,
                                              int32_t mode, void* stream);

/*
 * Decode index builder, the page's write_v4_paged_decode_indices ("paged
 * decode index scatter kernel"): packs sliding-window ring slots and
 * compressed paged slots into ragged CSR indices with no sentinels.
 * For each token t, in token order:
 *   window part:     state_slot[t] * win + r            for r = 0 .. swa_len[t]-1
 *   compressed part: swa_pages + block_table[t][c / k_per_block] * k_per_block
 *                              + c % k_per_block
 *                    for each entry c of comp_pos[t][0 .. topk-1] with c >= 0,
 *                    in row order
 *   kv_indptr[0] = 0, kv_indptr[t+1] = kv_indptr[t] + entries of token t.
 * A padded token (swa_len 0, no valid comp_pos) gets a zero-length slice.
 *
 *   state_slot   [N] int32        swa_len [N] int32, each in [0, win]
 *   comp_pos     [N, topk] int32, negative = no entry; NULL with topk == 0
 *   block_table  [N, max_blocks] int32 (NULL allowed when comp_pos is NULL)
 *   kv_indptr    [N+1] int32 (out)   kv_indices [indices_capacity] int32 (out)
 *
 * Host checks: win > 0, k_per_block > 0, N >= 0, topk >= 0, swa_pages >= 0,
 * indices_capacity >= N * (win + topk) and N * (win + topk) < 2^31.
 * Device-side: swa_len is clamped to [0, win] and a comp_pos entry whose block
 * lookup falls outside [0, max_blocks) is dropped, so bad metadata cannot
 * make the builder read or write out of bounds.  Caller precondition (not
 * checked): the produced slots lie inside the pool.
 */
SPD_API spd_status build_decode_indices(const int32_t* state_slot, const int32_t* swa_len,
                                        const int32_t* comp_pos, int32_t topk,
                                        const int32_t* block_table, int32_t max_blocks, int32_t N,
                                        int32_t win, int32_t k_per_block, int32_t swa_pages,
                                        int32_t* kv_indptr, int32_t* kv_indices,
                                        int64_t indices_capacity, void* stream);

/*
 * sparse_decode_attn with the page transform fused into the attention kernel:
 * each workgroup derives its token's row list from the builder's inputs, by
 * exactly the rule of build_decode_indices above (window slots, then the
 * valid compressed slots in comp_pos order), and gathers those rows; the
 * ragged kv_indices / kv_indptr are never materialised.  The result equals
 * build_decode_indices followed by sparse_decode_attn on its output, bit for
 * bit: the rows are the same and are visited in the same order.  (The page
 * transform as a structure of its own that several kernels share: prhub
 * sglang attention-tag page, entry of 2026-09-16 on the DSV4.1 indexer
 * kernels; the slot formulas: sglang PR #28392 summary page, "key source
 * snippet".)
 *
 *   q, unified_kv, attn_sink, softmax_scale, out, N, H, D: as sparse_decode_attn
 *   state_slot, swa_len, comp_pos, topk, block_table, max_blocks, win,
 *   k_per_block, swa_pages: as build_decode_indices (same host checks, same
 *                device-side clamping of swa_len and dropping of comp_pos
 *                entries outside [0, max_blocks * k_per_block))
 *   mode         an spd_mode; never splits a token across workgroups, so no
 *                workspace
 *
 * win + topk must not exceed 2048 (a token's whole list is built in LDS before
 * its first row is loaded): SPD_ERR_UNSUPPORTED otherwise.  Caller
 * precondition (not checked): the produced slots lie in [0, num_rows).
 */
SPD_API spd_status sparse_decode_attn_paged(
    const void* q, const void* unified_kv, int64_t num_rows, const int32_t* state_slot,
    const int32_t* swa_len, const int32_t* comp_pos, int32_t topk, const int32_t* block_table,
    int32_t max_blocks, int32_t win, int32_t k_per_block, int32_t swa_pages,
    const float* attn_sink, float softmax_scale, void* out, int32_t N, int32_t H, int32_t D,
    int32_t mode, void* stream);

/*
 * Sparse attention for a batch of query tokens whose row lists are windows of
 * one shared index stream (prefill-shaped batches, where consecutive tokens
 * share most of their rows: sglang PR #28392 summary page, "implementation
 * breakdown" and "key files", the paged prefill module beside the decode
 * one).  Token t attends to
 *
 *   J_t = kv_stream[win_start[t] : win_start[t] + win_len[t]]
 *
 * with exactly the operation and numerics of sparse_decode_attn (sink,
 * log2-domain softmax, empty window -> zeros).  A CSR batch is the case of
 * windows that do not overlap (win_start = kv_indptr[t], win_len = its
 * length).  A workgroup serves tokens_per_group consecutive tokens (their
 * tokens_per_group * H query rows, 64 or 128, fill two or four waves of 32
 * heads), gathers the union of their windows once, and each token masks the
 * rows outside its own window, so overlapping windows are read once per group;
 * the cost grows with the union's span, so tokens of one group should overlap.
 * tokens_per_group = 0 picks one token per workgroup at H = 64 and 128 and two
 * at H = 32 (on the prefill batch of this library's measurements, two tokens a
 * workgroup at H = 64 gathered fewer bytes but ran slower: the rows they share
 * were already L2 hits, and each wave still reads every row it uses from LDS).
 *
 *   q, unified_kv, attn_sink, softmax_scale, out, N, D: as sparse_decode_attn
 *   H            32, 64 or 128, and tokens_per_group * H in {64, 128}
 *                (SPD_ERR_UNSUPPORTED otherwise)
 *   kv_stream    [stream_len] int32 pool rows, each in [0, num_rows)
 *                (NULL allowed when stream_len == 0); stream_len < 2^31
 *   win_start, win_len  [N] int32; a window with win_len <= 0, win_start < 0
 *                or win_start + win_len > stream_len counts as empty
 *
 * No workspace, no split; graph-capturable.
 */
SPD_API spd_status sparse_prefill_attn(const void* q, const void* unified_kv, int64_t num_rows,
                                       const int32_t* kv_stream, int64_t stream_len,
                                       const int32_t* win_start, const int32_t* win_len,
                                       const float* attn_sink, float softmax_scale, void* out,
                                       int32_t N, int32_t H, int32_t D, int32_t tokens_per_group,
                                       void* stream);

/*
 * FP8 pool.  The page's caches have FP8 variants, filled by stores that
 * quantise rows as they scatter them into the pool (sglang PR #25898 summary
 * page, "key files": the fused norm/RoPE/store kernel and the store-cache
 * kernels); a review on that page ("comment highlights", "risks and impact")
 * asks for round-to-nearest-even in the conversion, not round-half-up.
 * Format: row r of the pool is D OCP e4m3 codes (1 sign, 4 exponent bits with
 * bias 7, 3 mantissa bits; no infinities; 0x7f / 0xff are NaN) in
 * kv_fp8[r][0 .. D) plus one fp32 scale kv_scale[r]; its value is
 * kv_scale[r] * e4m3(code).
 */

/*
 * sparse_decode_attn over an FP8 pool: the same operation (same index
 * contract, sink and numerics) with the row value kv_scale[r] * e4m3(code),
 * used as both key and value.  fp32 accumulation; the codes are converted to
 * bf16 exactly, the scale multiplies the row's scores and its softmax weight.
 * Work decomposition as sparse_decode_attn_fp8_ex with max_len 0 and
 * SPD_MODE_AUTO (no split, no workspace).
 *
 *   q, kv_indices, kv_indptr, attn_sink, softmax_scale, out, N, H, D:
 *                as sparse_decode_attn (same alignment and preconditions:
 *                every index in [0, num_rows))
 *   kv_fp8       [num_rows, D] uint8 e4m3 codes, 16-byte aligned
 *   kv_scale     [num_rows] fp32, 4-byte aligned
 *
 * Returns SPD_ERR_UNSUPPORTED where sparse_decode_attn_can_use(H, D) is 0.
 */
SPD_API spd_status sparse_decode_attn_fp8(const void* q, const void* kv_fp8,
                                          const float* kv_scale, int64_t num_rows,
                                          const int32_t* kv_indices, const int32_t* kv_indptr,
                                          const float* attn_sink, float softmax_scale, void* out,
                                          int32_t N, int32_t H, int32_t D, void* stream);

/*
 * sparse_decode_attn_fp8 with a chosen plan, as sparse_decode_attn_ex is
 * for the bf16 pool (same max_len, split_rows, workspace and arrival-counter
 * rules).  Modes:
 *   SPD_MODE_ROWS:  workgroup = (token, 16 heads), its 4 waves splitting the
 *                   rows (any supported H and D).
 *   SPD_MODE_WIDE:  workgroups of 128 heads (H % 128 == 0) or 64 heads on
 *                   32-head waves sharing 32-row tiles of codes; D >= 128,
 *                   H % 64 == 0.
 *   SPD_MODE_SPLIT: the split mode of sparse_decode_attn_ex over codes
 *                   (D >= 128): partitions of a slice merged inside the
 *                   kernel, each gathered row entering one CU per 64 heads.
 *   SPD_MODE_AUTO:  SPLIT when split_rows != 0, or when D >= 128, the batch
 *                   gives at most 256 workgroups of 64 heads (16 or 32
 *                   when H is smaller) and max_len >= 2048; else WIDE on 128-head
 *                   workgroups when H % 128 == 0, D >= 128 and N * H / 128 >=
 *                   256; on 64-head workgroups of two waves when H % 64 == 0
 *                   and N * H / 64 >= 512, or of four waves (two parities of
 *                   each 32-head block) when it is in [256, 512); else ROWS.
 * SPD_MODE_HEADS (no FP8 kernel), SPLIT, WIDE or split_rows != 0 with
 * D < 128, WIDE with H % 64 != 0 and split_rows != 0 with ROWS or WIDE give
 * SPD_ERR_UNSUPPORTED.  Other arguments and errors as sparse_decode_attn_fp8
 * and sparse_decode_attn_ex.
 */
SPD_API spd_status sparse_decode_attn_fp8_ex(const void* q, const void* kv_fp8,
                                             const float* kv_scale, int64_t num_rows,
                                             const int32_t* kv_indices, const int32_t* kv_indptr,
                                             const float* attn_sink, float softmax_scale,
                                             void* out, int32_t N, int32_t H, int32_t D,
                                             int32_t max_len, int32_t split_rows, int32_t mode,
                                             void* workspace, size_t workspace_bytes,
                                             void* stream);

/*
 * Workspace bytes sparse_decode_attn_fp8_ex needs (0 when its plan does not
 * split, or for arguments it rejects), and its plan in the layout of
 * sparse_decode_attn_plan_info, except info[5] = 0 (ROWS), 2 or 4 (WIDE:
 * waves of 32 heads a workgroup) or 3 (64 heads on four waves, two parities).
 * plan_info returns SPD_ERR_UNSUPPORTED for every mode and shape the call
 * rejects as unsupported, SPD_ERR_INVALID_ARG for invalid sizes or modes.
 */
SPD_API size_t sparse_decode_attn_fp8_workspace_size(int32_t N, int32_t H, int32_t D,
                                                     int32_t max_len, int32_t split_rows,
                                                     int32_t mode);
SPD_API spd_status sparse_decode_attn_fp8_plan_info(int32_t N, int32_t H, int32_t D,
                                                    int32_t max_len, int32_t split_rows,
                                                    int32_t mode, int32_t* info);

/*
 * Quantising store into an FP8 pool: bf16 row i of src goes to pool row
 * slots[i] (row i when slots is NULL) as codes plus a scale:
 *   amax = max_d |x_d|;  amax < 2^-64 (a zero row): scale 0, every code 0;
 *   else scale = amax / 448 and inv = 448 / amax (fp32, correctly rounded),
 *        y_d = clamp(x_d * inv, -448, 448) (fp32),
 *        code_d = y_d rounded to the nearest e4m3 value, ties to even
 *        (448 is the largest finite e4m3 value, so |x| = amax stores +-448).
 * The inputs must be finite (a row holding an infinity or a NaN stores
 * unspecified codes).
 *
 *   src       [n, D] bf16, 16-byte aligned;  D in {64, 128, 256, 512}
 *   slots     [n] int32 destination rows, or NULL; a slot outside
 *             [0, num_rows) skips its row (nothing is written for it).  Two
 *             rows with the same slot race.
 *   kv_fp8    [num_rows, D] uint8 (out), 16-byte aligned
 *   kv_scale  [num_rows] fp32 (out)
 *
 * Host checks: n >= 0, num_rows > 0, n <= num_rows when slots is NULL, no
 * overlap between the source and the pool.  n == 0 returns SPD_OK.
 */
SPD_API spd_status quantize_kv_fp8(const void* src, const int32_t* slots, int32_t n, int32_t D,
                                   void* kv_fp8, float* kv_scale, int64_t num_rows, void* stream);

/*
 * The decode-step producer: writes the rows the attention reads.  sglang PR
 * #25898 summary page, "key files": one fused kernel does the q per-head
 * RMSNorm, the KV RMSNorm, RoPE, the FP8 quantisation and the paged
 * sliding-window store.  For each token t with position p = positions[t]:
 *
 *   RMSNorm(x, w) = x_d * w_d / sqrt(mean_d(x_d^2) + eps)        (fp32)
 *   RoPE: on the last rope_dim entries (o = D - rope_dim), GPT-J pairs:
 *     for i < rope_dim/2, c = cos_sin[p][i], s = cos_sin[p][rope_dim/2 + i]:
 *     (y[o+2i], y[o+2i+1]) <- (y[o+2i] c - y[o+2i+1] s, y[o+2i] s + y[o+2i+1] c)
 *   q_out[t,h,:] = bf16(RoPE(RMSNorm(q[t,h,:], q_weight)))       for every head h
 *   row          = bf16(RoPE(RMSNorm(kv[t,:], kv_weight)))
 *   slot         = state_slot[t] * win + p mod win                (the window ring)
 *   unified_kv[slot,:] = row;  and/or  (kv_fp8[slot,:], kv_scale[slot]) = the
 *   quantize_kv_fp8 store of row.
 *
 *   q, q_out   [N, H, D] bf16, 16-byte aligned; q_out may be q (in place),
 *              no other overlap
 *   kv         [N, D] bf16, each token's new KV row
 *   q_weight, kv_weight  [D] fp32;  eps >= 0
 *   positions  [N] int32; cos_sin [max_pos, rope_dim] fp32 (cos, then sin),
 *              may be NULL when rope_dim == 0; rope_dim even, 0 <= rope_dim <= D
 *   state_slot [N] int32;  win > 0
 *   unified_kv [num_rows, D] bf16 pool, or NULL;  kv_fp8 [num_rows, D] codes
 *              with kv_scale [num_rows], or NULL; at least one pool
 *
 * A token whose position is negative, or (when rope_dim > 0) not below
 * max_pos, is skipped (nothing is written for it); a KV row whose slot lies
 * outside [0, num_rows) is not stored.  D in {64, 128, 256, 512} (SPD_ERR_UNSUPPORTED otherwise).  One
 * launch; graph-capturable.
 */
SPD_API spd_status fused_qk_norm_rope_swa_store(
    const void* q, void* q_out, const void* kv, const float* q_weight, const float* kv_weight,
    float eps, const int32_t* positions, const float* cos_sin, int32_t max_pos, int32_t rope_dim,
    const int32_t* state_slot, int32_t win, void* unified_kv, void* kv_fp8, float* kv_scale,
    int64_t num_rows, int32_t N, int32_t H, int32_t D, void* stream);

/*
 * Debug check of the attention call's index preconditions: kv_indptr[0] == 0,
 * kv_indptr non-decreasing, kv_indptr[N] <= num_indices (the length of the
 * kv_indices buffer), and every kv_indices[j], j < kv_indptr[N], in
 * [0, num_rows).  *first_bad (host pointer) receives -1 when all hold, else
 * the smallest offending position: t (0..N) for a kv_indptr violation, or
 * N + 1 + j for kv_indices[j].  Allocates a few bytes of device memory and
 * synchronises `stream`: not for the hot path and not capturable.
 */
SPD_API spd_status spd_validate_indices(const int32_t* kv_indices, int64_t num_indices,
                                        const int32_t* kv_indptr, int32_t N, int64_t num_rows,
                                        int64_t* first_bad, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPD_H_ */
