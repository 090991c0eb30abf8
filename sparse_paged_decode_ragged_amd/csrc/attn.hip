// attn.hip -- sparse decode attention over a unified paged KV pool, gfx950.
//
// Operation (sglang PR #28392 summary page, "key source snippet": the
// paged_decode.py module docstring): token t attends to the pool rows
// kv_indices[kv_indptr[t] : kv_indptr[t+1]]; each bf16 row of width D is both
// key and value; attn_sink[H] is a virtual key in the softmax denominator;
// the softmax is computed online in the log2 domain with
// qk_scale = softmax_scale * log2(e); an empty slice gives zeros.
//
// Kernel design (MI355X-first, not a translation of the page's kernel):
//   * rows are gathered straight into LDS with LDS-DMA loads
//     (global_load_lds_dwordx4: one 1 KiB row per wave instruction at D=512),
//     XOR-swizzled by row so that both LDS read patterns below are
//     bank-conflict free; the row indices of a partition are staged into LDS
//     first (global_load_lds_dword, 64 per instruction), so issuing a row load
//     never waits on memory;
//   * S^T = K Q^T on MFMA bf16 with A = K rows from LDS and B = Q^T held in
//     VGPRs for the whole slice; the S^T accumulator layout (lane = head, four
//     rows per lane) is exactly the B operand layout of O^T += V^T P^T, so P
//     never leaves registers; V^T is read from the same LDS rows with
//     ds_read_b64_tr_b16 (the 16-lane transpose read of gfx950);
//   * the online-softmax state lives per lane (lane = head); its reference
//     maximum is fixed at the state's first tile, so the accumulator (held in
//     AGPRs by the MFMAs) is never rescaled inside the loop; a score more than
//     2^64 above that reference sends the workgroup through a second pass with
//     the true maximum, which the first pass tracked;
//   * two decompositions of the work of one token:
//       heads  -- workgroup = (token, 16*W heads, partition); wave w owns 16
//                 heads and all waves share each 32-row tile (for batches
//                 that already provide hundreds of workgroups);
//       rows   -- workgroup = (token, 16 heads); its 4 waves take every 4th
//                 16-row tile into private LDS stages (no barriers in the
//                 loop) and merge their (m, l, O) in LDS at the end (for
//                 small batches: 4x the workgroups, no partials in memory);
//   * long slices may also be split across workgroups (split-L); partials
//     (m, l, O) go to a workspace and a combine kernel merges them, counting
//     the sink once.
#include "attn_device.h"

namespace spd {
namespace {

// ---------------------------------------------------------------------------
// heads mode: workgroup = (token, 16*W heads, partition); 32-row shared tiles.
template <int D, int W, bool kPaged>
__global__ void __launch_bounds__(64 * W) attn_heads_kernel(AttnArgs a) {
  constexpr int kTile = 32;
  constexpr int kRowBytes = 2 * D;
  constexpr int kStageBytes = kTile * kRowBytes;
  constexpr int kKSteps = D / 32;
  constexpr int kDTiles = D / 16;
  constexpr int kRowsPerLoad = 1024 / kRowBytes;  // rows filled by one 64-lane x 16 B load
  constexpr int kLoadsPerTile = kTile / kRowsPerLoad;
  constexpr int kLoadsPerWave = kLoadsPerTile / W;
  constexpr int kHeads = 16 * W;
  static_assert(D % 64 == 0 && D <= 512, "unsupported D");
  static_assert(kLoadsPerTile % W == 0, "loads must divide among waves");
  // 32-row tiles in flight; a wave's outstanding loads must fit the 6-bit vmcnt
  constexpr int kAhead = 2 * kLoadsPerWave <= 63 ? 3 : 2;
  constexpr int kStages = kAhead + 1;
  static_assert((kStages & (kStages - 1)) == 0 || kStages == 3, "stage count");

  __shared__ __attribute__((aligned(1024))) unsigned char smem[kStages * kStageBytes];
  __shared__ __attribute__((aligned(256))) int sidx[kIdxCap];
  __shared__ __attribute__((aligned(256))) float ssink[64];
  __shared__ int sflag[W];
  __shared__ int scount[8 * W];  // page transform: valid entries per (group slot, wave)

  // Work item: partition c of (token, head group) th.  With split-L and a
  // number of (token, head group) pairs divisible by 8, the k-th workgroup an
  // XCD receives (the dispatcher deals workgroups to the 8 XCDs in turn)
  // takes partition S - 1 - k / Tx of pair 8 (k mod Tx) + x.  Every XCD holds
  // every 8th pair, so empty and short tokens (a padded batch tail, say)
  // spread over all XCDs.  It deals the last partitions of all its pairs
  // first: those exist only for the longest slices (the others exit at once),
  // so the tails of long slices start at the beginning and the partitions
  // every token has fill the CUs as they free.
  int c, th;
  {
    const int T = a.N * a.head_groups;
    if (a.splits > 1 && (T & 7) == 0) {
      const int x = blockIdx.x & 7, k = blockIdx.x >> 3, tx = T >> 3;
      const int r = k / tx;
      c = a.splits - 1 - r;
      th = 8 * (k - r * tx) + x;
    } else {
      const int it = xcd_item(blockIdx.x, gridDim.x);
      c = it % a.splits;
      th = it / a.splits;
    }
  }
  const int item = th * a.splits + c;  // its workspace slot
  const int hg = th % a.head_groups;
  const int t = th / a.head_groups;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n16 = lane & 15;
  const int g = lane >> 4;

  int L;
  const int32_t* part = nullptr;
  if constexpr (kPaged) {  // no split: c == 0
    L = stage_paged_list<64 * W>(a, t, sidx, scount);
  } else {
    const ScalarI32Ptr indptr = (ScalarI32Ptr)a.kv_indptr;
    const int row0 = indptr[t];
    L = indptr[t + 1] - row0;
    part = a.kv_indices + row0;
  }
  const int nparts = partitions_of(L, a.splits, a.split_rows);
  if (c >= nparts) return;  // nothing for this partition

  const int h0 = hg * kHeads + wave * 16;  // first head of this wave
  const int h = h0 + n16;                  // this lane's head
  const bool hvalid = h < a.H;

  if (L <= 0) {
    zero_heads<D>(a.out, a.H, t, h0, a.H - h0 < 16 ? a.H - h0 : 16, lane, 64);
    return;
  }

  const int cb = c * a.split_rows;
  const int nrows = (c == nparts - 1) ? L - cb : a.split_rows;
  if constexpr (!kPaged) part += cb;

  bf16x8 qreg[kKSteps];
  load_q<D>(a.q, (int64_t)t * a.H + (hvalid ? h : 0), g, qreg);
  stage_sinks(a.sink, a.H, hg * kHeads, ssink, wave, lane);

  const TileOffsets<D> off(n16, g);  // rows n16 / rtr, and 16 rows further

  float m = -INFINITY, lpart = 0.f, mtrue = -INFINITY, sink_l2 = -INFINITY;
  f32x4 acc[kDTiles];
  for (int pass = 0; pass < 2; ++pass) {
  bool first = pass == 0;
  if (pass == 1) second_pass_state(sink_l2, mtrue, g, m, lpart);
#pragma unroll
  for (int i = 0; i < kDTiles; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  bool over = false;

  for (int sc = 0; sc < nrows; sc += kIdxCap) {
    const int n = nrows - sc < kIdxCap ? nrows - sc : kIdxCap;
    if (sc > 0 || pass > 0) barrier_lds();  // every wave is done with the stages and indices
    if constexpr (!kPaged) stage_indices(part, sc, n, sidx, wave, W, lane);  // paged: built once
    wait_vmcnt<0>();
    barrier_lds();
    if (pass == 0 && sc == 0)  // the sink belongs to partition 0's state
      sink_l2 = (c == 0 && hvalid) ? ssink[wave * 16 + n16] * kLog2e : -INFINITY;
    const int ntiles = (n + kTile - 1) / kTile;

    auto issue_tile = [&](int tile) {
      issue_rows<kRowBytes, kLoadsPerWave>(a.kv, sidx, n, tile * kTile + wave * (kTile / W),
                                           wave * (kTile / W),
                                           smem + (tile % kStages) * kStageBytes +
                                               wave * kLoadsPerWave * 1024,
                                           lane);
    };

#pragma unroll
    for (int k = 0; k < kAhead; ++k)
      if (k < ntiles) issue_tile(k);

    for (int i = 0; i < ntiles; ++i) {
      // tile i has landed once at most min(kAhead - 1, ntiles - 1 - i) later
      // tiles of this wave are still outstanding
      const int later = ntiles - 1 - i;
      if (later >= kAhead - 1)
        wait_vmcnt<(kAhead - 1) * kLoadsPerWave>();
      else if (kAhead == 3 && later == 1)
        wait_vmcnt<kLoadsPerWave>();
      else
        wait_vmcnt<0>();
      barrier_lds();  // every wave's part of tile i is in LDS; tile i-1's stage is free
      if (i + kAhead < ntiles) issue_tile(i + kAhead);

      const unsigned char* st = smem + (i % kStages) * kStageBytes;
      const int nvalid = n - i * kTile;  // rows of this tile that exist (>= 1)

      // S^T = K Q^T.  The K operands are read in batches of kB k-steps, all
      // reads of a batch issued before its MFMAs (sched_barrier keeps the
      // compiler from interleaving each read with its use).
      constexpr int kB = kKSteps < 8 ? kKSteps : 8;
      f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sa2 = sa;  // two chains per 16-row half
      f32x4 sb = {0.f, 0.f, 0.f, 0.f}, sb2 = sb;
#pragma unroll
      for (int s0 = 0; s0 < kKSteps; s0 += kB) {
        bf16x8 ka[kB], kb[kB];
#pragma unroll
        for (int u = 0; u < kB; ++u) {
          const int o = off.kq(s0 + u);
          ka[u] = *reinterpret_cast<const bf16x8*>(st + o);
          kb[u] = *reinterpret_cast<const bf16x8*>(st + o + 16 * kRowBytes);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < kB; ++u) {
          if (u & 1) {
            sa2 = mfma_k32(ka[u], qreg[s0 + u], sa2);
            sb2 = mfma_k32(kb[u], qreg[s0 + u], sb2);
          } else {
            sa = mfma_k32(ka[u], qreg[s0 + u], sa);
            sb = mfma_k32(kb[u], qreg[s0 + u], sb);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      sa += sa2;
      sb += sb2;

      float x[8];
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        x[i4] = (4 * g + i4 < nvalid) ? sa[i4] * a.qk_scale : -INFINITY;
        x[4 + i4] = (16 + 4 * g + i4 < nvalid) ? sb[i4] * a.qk_scale : -INFINITY;
      }
      __bf16 p[8];
      over |= softmax_tile<8>(x, sink_l2, g, first, m, mtrue, lpart, p);
      bf16x8 pt;
#pragma unroll
      for (int j = 0; j < 8; ++j) pt[j] = p[j];

      // O^T += V^T P^T, V^T operands read in batches of kVB d-tiles.
      constexpr int kVB = kDTiles < 8 ? kDTiles : 8;
#pragma unroll
      for (int d0 = 0; d0 < kDTiles; d0 += kVB) {
        bf16x8 vt[kVB];
#pragma unroll
        for (int u = 0; u < kVB; ++u) {
          const int o = off.vt(d0 + u);
          const bf16x4 vlo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LdsBf16x4*)(st + o));
          const bf16x4 vhi =
              __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LdsBf16x4*)(st + o + 16 * kRowBytes));
          vt[u] = __builtin_shufflevector(vlo, vhi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < kVB; ++u) acc[d0 + u] = mfma_k32(vt[u], pt, acc[d0 + u]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  if (!workgroup_any(over, sflag, wave, W)) break;
  }

  const float l = group_sum4(lpart);

  if (nparts == 1) {
    if (hvalid) {
      const float inv = 1.0f / l;
      uint16_t* op = a.out + ((int64_t)t * a.H + h) * D + 4 * g;
#pragma unroll
      for (int dt = 0; dt < kDTiles; ++dt) store_bf16x4(op + 16 * dt, acc[dt], inv);
    }
  } else {
    float* base = a.ws + (int64_t)item * (kHeads * (D + 2));
    f32x4* po = reinterpret_cast<f32x4*>(base) + wave * kDTiles * 64 + lane;
#pragma unroll
    for (int dt = 0; dt < kDTiles; ++dt) po[dt * 64] = acc[dt];
    if (g == 0) {
      base[kHeads * D + wave * 16 + n16] = m;
      base[kHeads * D + kHeads + wave * 16 + n16] = l;
    }
  }
}

// Merge the partitions of each token with more than one (heads mode):
//   M = max_c m_c,  l = sum_c l_c 2^(m_c - M),  O = sum_c O_c 2^(m_c - M),
//   out = O / l.  Partition 0 already carries the sink.  Workgroup = (token,
// head group, quarter of D), so the grid is four times the token count.
template <int D, int W>
__global__ void __launch_bounds__(64 * W) attn_combine_kernel(AttnArgs a) {
  constexpr int kDTiles = D / 16;
  constexpr int kQ = kDTiles / 4;  // d-tiles per quarter
  constexpr int kHeads = 16 * W;
  const int quarter = blockIdx.x & 3;
  const int th = blockIdx.x >> 2;
  const int hg = th % a.head_groups;
  const int t = th / a.head_groups;
  const ScalarI32Ptr indptr = (ScalarI32Ptr)a.kv_indptr;
  const int L = indptr[t + 1] - indptr[t];
  const int nparts = partitions_of(L, a.splits, a.split_rows);
  if (nparts <= 1) return;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n16 = lane & 15;
  const int g = lane >> 4;
  const int h = hg * kHeads + wave * 16 + n16;
  if (h >= a.H) return;

  const int64_t stride = (int64_t)kHeads * (D + 2);
  const float* base0 = a.ws + (int64_t)th * a.splits * stride;
  const int hi = wave * 16 + n16;

  float M = -INFINITY;
  for (int c = 0; c < nparts; ++c) M = fmaxf(M, base0[c * stride + kHeads * D + hi]);
  float lsum = 0.f;
  f32x4 acc[kQ];
#pragma unroll
  for (int i = 0; i < kQ; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int c = 0; c < nparts; ++c) {
    const float* base = base0 + c * stride;
    const float w = __builtin_amdgcn_exp2f(base[kHeads * D + hi] - M);
    lsum += w * base[kHeads * D + kHeads + hi];
    const f32x4* po =
        reinterpret_cast<const f32x4*>(base) + (wave * kDTiles + quarter * kQ) * 64 + lane;
    f32x4 v[kQ];
#pragma unroll
    for (int i = 0; i < kQ; ++i) v[i] = po[i * 64];
#pragma unroll
    for (int i = 0; i < kQ; ++i) acc[i] += w * v[i];
  }
  const float inv = 1.0f / lsum;
  uint16_t* op = a.out + ((int64_t)t * a.H + h) * D + 4 * g + 16 * quarter * kQ;
#pragma unroll
  for (int i = 0; i < kQ; ++i) store_bf16x4(op + 16 * i, acc[i], inv);
}

// ---------------------------------------------------------------------------
// wide heads mode: workgroup = (token, 32*W heads), W waves of 32 heads each,
// sharing every 32-row tile staged in LDS (no split-L).  A 32-head wave reads
// each K and V^T operand from LDS once for two 16-head MFMA blocks, half the
// LDS bytes per flop of a 16-head wave:
//  * S^T = K Q^T on 16x16x32 MFMAs: the K operand of rows r0..r0+15 (one b128
//    read per k-step) meets the Q^T operands of both head blocks;
//  * O^T += V^T P^T on 32x32x16 MFMAs (M = 32 values of d, N = the 32 heads,
//    K = 16 rows): lane (n, kg) of the B operand must hold P of rows
//    8kg..8kg+7 for head n.  The 16x16 score layout gives lane (h, g) rows
//    4g..4g+3 of head h of each block, so the B operand is the two blocks' P
//    after one v_permlane16_swap per dword (lanes 16..31 of block 0's value
//    trade with lanes 0..15 of block 1's, in each half-wave): the K index of
//    the product is then exactly the row.  The A operand (V^T, lane (d, kg)
//    holding rows 8kg..8kg+7 of column d) is two transposing reads.
// The accumulator of a wave is 32 heads x D fp32 (256 AGPRs at D = 512).

// kWin: 0 = CSR slices; 1 = one token a workgroup whose slice is its window of
// the index stream (no masks); 2 = tokens_per_group tokens share the union of
// their windows, each wave masking the rows outside its token's window.
template <int D, int W, bool kPaged, int kWin = 0>
__global__ void __launch_bounds__(64 * W) attn_wide_kernel(AttnArgs a) {
  constexpr int kTile = 32;
  constexpr int kRowBytes = 2 * D;
  constexpr int kStageBytes = kTile * kRowBytes;
  constexpr int kKSteps = D / 32;
  constexpr int kDT = D / 32;  // 32-wide d-tiles of the PV product
  constexpr int kRowsPerLoad = 1024 / kRowBytes;
  constexpr int kLoadsPerTile = kTile / kRowsPerLoad;
  constexpr int kLoadsPerWave = kLoadsPerTile / W;
  constexpr int kHeads = 32 * W;
  static_assert(D % 64 == 0 && D <= 512, "unsupported D");
  static_assert(kLoadsPerTile % W == 0, "loads must divide among waves");
  // W = 4: one workgroup per CU, two tiles in flight; W = 2: two workgroups
  // per CU (LDS <= 80 KiB each), one tile in flight per workgroup
  constexpr int kAhead = W >= 4 ? 2 : 1;
  constexpr int kStages = kAhead + 1;
  constexpr bool kSpread = W == 4 && kRowsPerLoad == 1 && kLoadsPerWave <= kKSteps;

  __shared__ __attribute__((aligned(1024))) unsigned char smem[kStages * kStageBytes];
  __shared__ __attribute__((aligned(256))) int sidx[kIdxCap];
  __shared__ __attribute__((aligned(256))) float ssink[kHeads];
  __shared__ int sflag[W];
  __shared__ int scount[8 * W];

  const int item = xcd_item(blockIdx.x, gridDim.x);
  const int hg = item % a.head_groups;
  const int t = item / a.head_groups;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n16 = lane & 15;
  const int g = lane >> 4;

  int L;
  const int32_t* part = nullptr;
  int tok = t;                       // this wave's token
  int h0 = hg * kHeads + wave * 32;  // first head of this wave (H % kHeads == 0)
  int lo = 0, hi = 0x7fffffff;       // shared windows: this wave's rows of the slice
  if constexpr (kWin == 1) {
    const ScalarI32Ptr ws = (ScalarI32Ptr)a.win_start, wl = (ScalarI32Ptr)a.win_len;
    const int s0 = ws[t], l0 = wl[t];
    L = (s0 >= 0 && l0 > 0 && (int64_t)s0 + l0 <= a.stream_len) ? l0 : 0;
    part = a.kv_indices + (L > 0 ? s0 : 0);
    if (L <= 0) {
      zero_heads<D>(a.out, a.H, t, h0, 32, lane, 64);
      return;
    }
  } else if constexpr (kWin == 2) {
    // tokens t0 .. t0 + T - 1 share the workgroup; the slice is the union of
    // their windows of the index stream, and wave w serves token
    // t0 + 32 w / H, heads 32 w mod H .. + 31.  A window that is empty or
    // leaves the stream counts as empty.
    const int T = a.tokens_per_group;
    const int t0 = item * T;
    tok = t0 + (wave * 32) / a.H;
    h0 = (wave * 32) % a.H;
    const ScalarI32Ptr ws = (ScalarI32Ptr)a.win_start, wl = (ScalarI32Ptr)a.win_len;
    auto window_ok = [&](int s0, int l0) {
      return s0 >= 0 && l0 > 0 && (int64_t)s0 + l0 <= a.stream_len;
    };
    int u0 = 0x7fffffff, u1 = 0;
    for (int k = 0; k < T; ++k) {
      const int tk = t0 + k;
      if (tk < a.N && window_ok(ws[tk], wl[tk])) {
        u0 = min(u0, ws[tk]);
        u1 = max(u1, ws[tk] + wl[tk]);
      }
    }
    L = u1 > u0 ? u1 - u0 : 0;
    part = a.kv_indices + (L > 0 ? u0 : 0);
    lo = hi = 0;
    if (tok < a.N && window_ok(ws[tok], wl[tok])) {
      lo = ws[tok] - u0;
      hi = lo + wl[tok];
    }
    if (L <= 0) {
      if (tok < a.N) zero_heads<D>(a.out, a.H, tok, h0, 32, lane, 64);
      return;
    }
  } else {
    if constexpr (kPaged) {
      L = stage_paged_list<64 * W>(a, t, sidx, scount);
    } else {
      const ScalarI32Ptr indptr = (ScalarI32Ptr)a.kv_indptr;
      const int row0 = indptr[t];
      L = indptr[t + 1] - row0;
      part = a.kv_indices + row0;
    }
    if (L <= 0) {
      zero_heads<D>(a.out, a.H, t, h0, 32, lane, 64);
      return;
    }
  }

  bf16x8 q0[kKSteps], q1[kKSteps];  // Q^T operands of head blocks 0 and 1
  const int64_t qrow = (int64_t)(kWin == 2 ? (tok < a.N ? tok : a.N - 1) : t) * a.H + h0;
  load_q<D>(a.q, qrow + n16, g, q0);
  load_q<D>(a.q, qrow + 16 + n16, g, q1);
  if (wave == 0) {  // the workgroup's kHeads sinks (kHeads <= 128), one LDS-DMA per 64
#pragma unroll
    for (int c = 0; c < kHeads; c += 64) {
      const int hs = kWin == 2 ? (c + lane) % a.H : hg * kHeads + c + lane;
      dma_4B(a.sink + hs, __builtin_amdgcn_readfirstlane(lds_addr(ssink + c)));
    }
  }

  const TileOffsets<D, 1> off(n16, g);
  const WideVtOffsets<D> voff(lane);

  float m0 = -INFINITY, l0 = 0.f, mt0 = -INFINITY, sk0 = -INFINITY;
  float m1 = -INFINITY, l1 = 0.f, mt1 = -INFINITY, sk1 = -INFINITY;
  f32x16 acc[kDT];
  for (int pass = 0; pass < 2; ++pass) {
    bool first0 = pass == 0, first1 = pass == 0;
    if (pass == 1) {
      second_pass_state(sk0, mt0, g, m0, l0);
      second_pass_state(sk1, mt1, g, m1, l1);
    }
#pragma unroll
    for (int i = 0; i < kDT; ++i) acc[i] = f32x16{};
    bool over = false;

    for (int sc = 0; sc < L; sc += kIdxCap) {
      const int n = L - sc < kIdxCap ? L - sc : kIdxCap;
      if (sc > 0 || pass > 0) barrier_lds();  // every wave is done with the stages and indices
      if constexpr (!kPaged) stage_indices(part, sc, n, sidx, wave, W, lane);
      wait_vmcnt<0>();
      barrier_lds();
      if (pass == 0 && sc == 0) {
        sk0 = ssink[wave * 32 + n16] * kLog2e;
        sk1 = ssink[wave * 32 + 16 + n16] * kLog2e;
      }
      const int ntiles = (n + kTile - 1) / kTile;

      auto issue_tile = [&](int tile) {
        issue_rows<kRowBytes, kLoadsPerWave, 1>(a.kv, sidx, n, tile * kTile + wave * (kTile / W),
                                             wave * (kTile / W),
                                             smem + (tile % kStages) * kStageBytes +
                                                 wave * kLoadsPerWave * 1024,
                                             lane);
      };
#pragma unroll
      for (int k = 0; k < kAhead; ++k)
        if (k < ntiles) issue_tile(k);

      for (int i = 0; i < ntiles; ++i) {
        // tile i has landed once at most min(kAhead - 1, ntiles - 1 - i)
        // later tiles of this wave are still outstanding
        if (kAhead == 2 && i + 1 < ntiles)
          wait_vmcnt<kLoadsPerWave>();
        else
          wait_vmcnt<0>();
        barrier_lds();  // every wave's part of tile i is in LDS; tile i-1's stage is free
        // At D = 512 (one row a load) the wave's loads of tile i + kAhead are
        // spread over the QK k-steps, one after each step's MFMAs, so the
        // address unit takes them while the MFMAs run; the row indices are
        // read here.  Otherwise they are issued now.
        const bool more = i + kAhead < ntiles;
        int nidx = 0;
        if (more) {
          if constexpr (kSpread)
            nidx = sidx[min((i + kAhead) * kTile + wave * (kTile / W) +
                                (lane < kLoadsPerWave ? lane : 0), n - 1)];
          else
            issue_tile(i + kAhead);
        }
        const uint32_t ndst = __builtin_amdgcn_readfirstlane(
            lds_addr(smem + ((i + kAhead) % kStages) * kStageBytes + wave * kLoadsPerWave * 1024));

        // The stage's offset is opaque to the compiler: it would otherwise keep
        // every lane offset precomputed for each stage (registers it lacks).
        int stoff = (i % kStages) * kStageBytes;
        asm volatile("" : "+v"(stoff));
        const unsigned char* st = smem + stoff;
        const int nvalid = n - i * kTile;

        // S^T = K Q^T: rows 0-15 and 16-31 of the tile, head blocks 0 and 1.
        // The K reads run two k-steps ahead of the MFMAs that consume them
        // (sched_group_barrier pins the interleave: four MFMAs per k-step,
        // each pair followed by one of the two reads of k-step s + 2).
        f32x4 s00 = {0.f, 0.f, 0.f, 0.f}, s01 = s00, s10 = s00, s11 = s00;
        if constexpr (kSpread) {
          // per k-step, in program order: the K reads of step u + 2, the four
          // MFMAs of step u, then row load u of the next tile
          bf16x8 ka[kKSteps], kb[kKSteps];
          auto read_k = [&](int u) {
            const int o = off.kq(u);
            ka[u] = *reinterpret_cast<const bf16x8*>(st + o);
            kb[u] = *reinterpret_cast<const bf16x8*>(st + o + 16 * kRowBytes);
          };
          read_k(0);
          read_k(1);
          const unsigned char* kvb = reinterpret_cast<const unsigned char*>(a.kv);
#pragma unroll
          for (int u = 0; u < kKSteps; ++u) {
            if (u + 2 < kKSteps) read_k(u + 2);
            s00 = mfma_k32(ka[u], q0[u], s00);
            s01 = mfma_k32(ka[u], q1[u], s01);
            s10 = mfma_k32(kb[u], q0[u], s10);
            s11 = mfma_k32(kb[u], q1[u], s11);
            if (u < kLoadsPerWave && more) {
              const int grow = __builtin_amdgcn_readlane(nidx, u);
              const int r = wave * (kTile / W) + u;
              const uint32_t lane_off =
                  (uint32_t)((lane ^ (wide_swizzle(r & 15) & (kRowBytes / 16 - 1))) << 4);
              dma_16B_s(lane_off, kvb + (int64_t)grow * kRowBytes, ndst + u * 1024);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        } else {
          bf16x8 ka[kKSteps], kb[kKSteps];
#pragma unroll
          for (int u = 0; u < kKSteps; ++u) {
            const int o = off.kq(u);
            ka[u] = *reinterpret_cast<const bf16x8*>(st + o);
            kb[u] = *reinterpret_cast<const bf16x8*>(st + o + 16 * kRowBytes);
          }
#pragma unroll
          for (int u = 0; u < kKSteps; ++u) {
            s00 = mfma_k32(ka[u], q0[u], s00);
            s01 = mfma_k32(ka[u], q1[u], s01);
            s10 = mfma_k32(kb[u], q0[u], s10);
            s11 = mfma_k32(kb[u], q1[u], s11);
          }
          constexpr int kPre = kKSteps < 2 ? kKSteps : 2;
          __builtin_amdgcn_sched_group_barrier(0x100, 2 * kPre, 0);  // reads of k-steps 0, 1
#pragma unroll
          for (int u = 0; u < kKSteps; ++u) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            if (u + kPre < kKSteps) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            if (u + kPre < kKSteps) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
        }

        float x0[8], x1[8];
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          bool v0 = 4 * g + i4 < nvalid, v1 = 16 + 4 * g + i4 < nvalid;
          if constexpr (kWin == 2) {  // rows of the slice outside this wave's window
            const int j = sc + i * kTile + 4 * g + i4;
            v0 = v0 && j >= lo && j < hi;
            v1 = v1 && j + 16 >= lo && j + 16 < hi;
          }
          x0[i4] = v0 ? s00[i4] * a.qk_scale : -INFINITY;
          x0[4 + i4] = v1 ? s10[i4] * a.qk_scale : -INFINITY;
          x1[i4] = v0 ? s01[i4] * a.qk_scale : -INFINITY;
          x1[4 + i4] = v1 ? s11[i4] * a.qk_scale : -INFINITY;
        }
        __bf16 p0[8], p1[8];
        over |= softmax_tile<8, kWin == 2>(x0, sk0, g, first0, m0, mt0, l0, p0);
        over |= softmax_tile<8, kWin == 2>(x1, sk1, g, first1, m1, mt1, l1, p1);
        bf16x8 pb[2];  // B operands for rows 0-15 and 16-31
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          bf16x4 a0, a1;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            a0[e] = p0[4 * rb + e];
            a1[e] = p1[4 * rb + e];
          }
          pb[rb] = wide_p_operand(a0, a1);
        }

        // O^T += V^T P^T: the four transposing reads of d-tile dt + 2 run
        // under the two MFMAs of d-tile dt (pinned as for S^T above).
        {
          bf16x8 va[kDT], vb[kDT];
#pragma unroll
          for (int u = 0; u < kDT; ++u) {
            const int o0 = voff.at(u, 0), o1 = voff.at(u, 1);
            const bf16x4 a_lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LdsBf16x4*)(st + o0));
            const bf16x4 a_hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LdsBf16x4*)(st + o1));
            const bf16x4 b_lo =
                __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LdsBf16x4*)(st + o0 + 16 * kRowBytes));
            const bf16x4 b_hi =
                __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LdsBf16x4*)(st + o1 + 16 * kRowBytes));
            va[u] = __builtin_shufflevector(a_lo, a_hi, 0, 1, 2, 3, 4, 5, 6, 7);
            vb[u] = __builtin_shufflevector(b_lo, b_hi, 0, 1, 2, 3, 4, 5, 6, 7);
          }
#pragma unroll
          for (int u = 0; u < kDT; ++u) {
            acc[u] = mfma32(va[u], pb[0], acc[u]);
            acc[u] = mfma32(vb[u], pb[1], acc[u]);
          }
          constexpr int kPre = kDT < 2 ? kDT : 2;
          __builtin_amdgcn_sched_group_barrier(0x100, 4 * kPre, 0);  // reads of d-tiles 0, 1
#pragma unroll
          for (int u = 0; u < kDT; ++u) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (u + kPre < kDT) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (u + kPre < kDT) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    if (!workgroup_any(over, sflag, wave, W)) break;
  }

  // lane (n, hf) = lane n + 32 hf holds, for head h0 + n, d = 32 dt + 8 e4 +
  // 4 hf + e as element 4 e4 + e of acc[dt]; its denominator is block n / 16's
  // l of head n % 16, which every lane with lane % 16 == n % 16 holds.
  const float lb0 = group_sum4(l0), lb1 = group_sum4(l1);
  if constexpr (kWin == 2) {
    if (tok >= a.N) return;
    if (hi <= lo) {  // this wave's token has an empty window: zeros
      zero_heads<D>(a.out, a.H, tok, h0, 32, lane, 64);
      return;
    }
  }
  const int n = lane & 31, hf = lane >> 5;
  const float inv = 1.0f / (n < 16 ? lb0 : lb1);
  uint16_t* op = a.out + ((int64_t)tok * a.H + h0 + n) * D + 4 * hf;
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      const f32x4 v = {acc[dt][4 * e4], acc[dt][4 * e4 + 1], acc[dt][4 * e4 + 2], acc[dt][4 * e4 + 3]};
      store_bf16x4(op + 32 * dt + 8 * e4, v, inv);
    }
}

// ---------------------------------------------------------------------------
// rows mode: workgroup = (token, 16 heads); 4 waves split the slice into
// 16-row tiles (wave w takes tiles w, w+4, ...) staged in private LDS, then
// merge their softmax states in LDS.
template <int D, bool kPaged>
__global__ void __launch_bounds__(256) attn_rows_kernel(AttnArgs a) {
  constexpr int kWaves = 4;
  constexpr int kTile = 16;
  constexpr int kRowBytes = 2 * D;
  constexpr int kKSteps = D / 32;
  constexpr int kDTiles = D / 16;
  constexpr int kRowsPerLoad = 1024 / kRowBytes;
  constexpr int kLoads = kTile / kRowsPerLoad;  // DMA ops per wave tile
  constexpr int kStageBytes = kTile * kRowBytes;
  constexpr int kWaveBytes = 2 * kStageBytes;   // == 16 heads * D * 4: room for the partial O
  static_assert(kWaveBytes == 16 * D * 4, "partial O must fit the wave's stages");
  static_assert(kLoads >= 1 && kLoads < 64, "bad load count");

  __shared__ __attribute__((aligned(1024))) unsigned char smem[kWaves * kWaveBytes];
  __shared__ __attribute__((aligned(256))) int sidx[kIdxCap];
  __shared__ __attribute__((aligned(256))) float ssink[64];
  __shared__ float sml[kWaves][2][16];
  __shared__ int sflag[kWaves];
  __shared__ int scount[8 * kWaves];  // page transform: valid entries per (group slot, wave)

  const int item = xcd_item(blockIdx.x, gridDim.x);
  const int hg = item % a.head_groups;
  const int t = item / a.head_groups;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n16 = lane & 15;
  const int g = lane >> 4;

  int L;
  const int32_t* part = nullptr;
  if constexpr (kPaged) {
    L = stage_paged_list<64 * kWaves>(a, t, sidx, scount);
  } else {
    const ScalarI32Ptr indptr = (ScalarI32Ptr)a.kv_indptr;
    const int row0 = indptr[t];
    L = indptr[t + 1] - row0;
    part = a.kv_indices + row0;
  }
  const int h0 = hg * 16;
  const int h = h0 + n16;
  const bool hvalid = h < a.H;
  const int nh = a.H - h0 < 16 ? a.H - h0 : 16;

  if (L <= 0) {
    zero_heads<D>(a.out, a.H, t, h0, nh, threadIdx.x, 64 * kWaves);
    return;
  }

  bf16x8 qreg[kKSteps];
  stage_sinks(a.sink, a.H, h0, ssink, wave, lane);

  unsigned char* mine = smem + wave * kWaveBytes;
  const TileOffsets<D> off(n16, g);

  float m = -INFINITY, lpart = 0.f, mtrue = -INFINITY, sink_l2 = -INFINITY;
  f32x4 acc[kDTiles];
  for (int pass = 0; pass < 2; ++pass) {
    bool first = pass == 0;
    if (pass == 1) second_pass_state(sink_l2, mtrue, g, m, lpart);
#pragma unroll
    for (int i = 0; i < kDTiles; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    bool over = false;

    for (int sc = 0; sc < L; sc += kIdxCap) {
      const int n = L - sc < kIdxCap ? L - sc : kIdxCap;
      const bool restage = sc > 0 || (pass == 1 && L > kIdxCap);
      if (restage) {  // (never with the page transform: its lists fit kIdxCap)
        barrier_lds();  // every wave is done with the indices and its stages
        if constexpr (!kPaged) stage_indices(part, sc, n, sidx, wave, kWaves, lane);
        wait_vmcnt<0>();
        barrier_lds();
      } else if (pass == 0) {
        if constexpr (!kPaged) stage_indices(part, sc, n, sidx, wave, kWaves, lane);
        wait_vmcnt<0>();
        barrier_lds();
        sink_l2 = (wave == 0 && hvalid) ? ssink[n16] * kLog2e : -INFINITY;  // sink in wave 0
      }
      const int ntiles = (n + kTile - 1) / kTile;
      const int my_tiles = ntiles > wave ? (ntiles - wave + kWaves - 1) / kWaves : 0;

      auto issue = [&](int j) {  // this wave's j-th tile = global tile wave + 4j
        issue_rows<kRowBytes, kLoads>(a.kv, sidx, n, (wave + kWaves * j) * kTile, 0,
                                      mine + (j & 1) * kStageBytes, lane);
      };

      // Software pipeline over this wave's tiles, two LDS stages: the V^T
      // reads of tile j run under tile j's QK MFMAs, the K reads of tile j+1
      // run under tile j's PV MFMAs, and the load of tile j+2 goes into tile
      // j's stage as soon as its reads are done.  (sched_group_barrier fixes
      // the interleave: one MFMA per two LDS reads, then two per one.)
      constexpr int kCh = kKSteps < 4 ? kKSteps : 4;  // independent QK chains
      bf16x8 ka[kKSteps];
      if (my_tiles > 0) issue(0);
      if (my_tiles > 1) issue(1);
      // q is loaded once its first two tiles are in flight: the index staging
      // before them then waits for the indices alone
      if (pass == 0 && sc == 0) load_q<D>(a.q, (int64_t)t * a.H + (hvalid ? h : 0), g, qreg);
      if (my_tiles > 0) {
        if (my_tiles > 1)
          wait_vmcnt<kLoads>();
        else
          wait_vmcnt<0>();
        asm volatile("" ::: "memory");
#pragma unroll
        for (int s = 0; s < kKSteps; ++s) ka[s] = *reinterpret_cast<const bf16x8*>(mine + off.kq(s));
      }
      for (int j = 0; j < my_tiles; ++j) {
        const unsigned char* st = mine + (j & 1) * kStageBytes;
        const unsigned char* stn = mine + ((j + 1) & 1) * kStageBytes;
        const int nvalid = n - (wave + kWaves * j) * kTile;

        // S^T = K Q^T (four chains) with the V^T reads of the same tile.
        f32x4 part[kCh];
#pragma unroll
        for (int c = 0; c < kCh; ++c) part[c] = f32x4{0.f, 0.f, 0.f, 0.f};
        bf16x4 vt[kDTiles];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < kKSteps; ++s) {
          part[s % kCh] = mfma_k32(ka[s], qreg[s], part[s % kCh]);
          vt[2 * s] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LdsBf16x4*)(st + off.vt(2 * s)));
          vt[2 * s + 1] =
              __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LdsBf16x4*)(st + off.vt(2 * s + 1)));
        }
#pragma unroll
        for (int s = 0; s < kKSteps; ++s) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS reads
        }
        __builtin_amdgcn_sched_barrier(0);
        f32x4 sa = part[0];
#pragma unroll
        for (int c = 1; c < kCh; ++c) sa += part[c];
        float x[4];
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4)
          x[i4] = (4 * g + i4 < nvalid) ? sa[i4] * a.qk_scale : -INFINITY;
        __bf16 p[4];
        over |= softmax_tile<4>(x, sink_l2, g, first, m, mtrue, lpart, p);
        bf16x4 pt;
#pragma unroll
        for (int j4 = 0; j4 < 4; ++j4) pt[j4] = p[j4];
        // Every read of tile j's stage is complete: it takes the load of tile j+2.
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        asm volatile("" ::: "memory");
        if (j + 2 < my_tiles) issue(j + 2);
        if (j + 1 < my_tiles) {  // tile j+1 has landed once only tile j+2 may be outstanding
          if (j + 2 < my_tiles)
            wait_vmcnt<kLoads>();
          else
            wait_vmcnt<0>();
        }
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        // O^T += V^T P^T, with the K reads of tile j+1 (harmless stale reads
        // after the last tile: the stage is in bounds and the values unused).
#pragma unroll
        for (int dt = 0; dt < kDTiles; ++dt) {
          acc[dt] = mfma_k16(vt[dt], pt, acc[dt]);
          if (dt & 1) ka[dt >> 1] = *reinterpret_cast<const bf16x8*>(stn + off.kq(dt >> 1));
        }
#pragma unroll
        for (int s = 0; s < kKSteps; ++s) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (!workgroup_any(over, sflag, wave, kWaves)) break;
  }

  // Merge the four waves' states.  Wave w's partial O goes to its own stage
  // area as [head][d] fp32 with the 16-byte column index XOR-ed by the head.
  const float l = group_sum4(lpart);
  {
    f32x4* po = reinterpret_cast<f32x4*>(mine);
#pragma unroll
    for (int dt = 0; dt < kDTiles; ++dt) {
      const int col = (4 * dt + g) ^ n16;  // d/4 of this lane's four values, swizzled
      po[n16 * (D / 4) + col] = acc[dt];
    }
    if (g == 0) {
      sml[wave][0][n16] = m;
      sml[wave][1][n16] = l;
    }
  }
  barrier_lds();

  // Wave w produces d in [w*D/4, (w+1)*D/4) for all 16 heads: lane -> (head
  // hh = lane % 16, sub-range of D/16 values).
  const int hh = lane & 15;
  const int sub = lane >> 4;
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sml[w][0][hh]);
  float wgt[kWaves];
  float lsum = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    wgt[w] = __builtin_amdgcn_exp2f(sml[w][0][hh] - M);  // 0 for a wave with no rows
    lsum += wgt[w] * sml[w][1][hh];
  }
  const float inv = 1.0f / lsum;
  constexpr int kPer = D / 64;  // float4 columns per lane
  const int col0 = wave * (D / 16) + sub * kPer;
  if (hh < nh) {
    uint16_t* op = a.out + ((int64_t)t * a.H + h0 + hh) * D + 4 * col0;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const f32x4* po = reinterpret_cast<const f32x4*>(smem + w * kWaveBytes);
        s += wgt[w] * po[hh * (D / 4) + ((col0 + k) ^ hh)];
      }
      store_bf16x4(op + 4 * k, s, inv);
    }
  }
}

template <int D, int W>
hipError_t launch_heads(const AttnArgs& a, hipStream_t stream) {
  const long long items = (long long)a.N * a.head_groups * a.splits;
  if (a.paged)
    hipLaunchKernelGGL((attn_heads_kernel<D, W, true>), dim3((unsigned)items), dim3(64 * W), 0,
                       stream, a);
  else
    hipLaunchKernelGGL((attn_heads_kernel<D, W, false>), dim3((unsigned)items), dim3(64 * W), 0,
                       stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits == 1) return e;
  hipLaunchKernelGGL((attn_combine_kernel<D, W>), dim3((unsigned)(a.N * a.head_groups * 4)),
                     dim3(64 * W), 0, stream, a);
  return hipGetLastError();
}

template <int D, int W>
hipError_t launch_wide(const AttnArgs& a, hipStream_t stream) {
  const unsigned items = (unsigned)((long long)a.N * a.head_groups);
  if (a.paged)
    hipLaunchKernelGGL((attn_wide_kernel<D, W, true>), dim3(items), dim3(64 * W), 0, stream, a);
  else
    hipLaunchKernelGGL((attn_wide_kernel<D, W, false>), dim3(items), dim3(64 * W), 0, stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_prefill_d(const AttnArgs& a, hipStream_t stream) {
  // a workgroup's 32 * W query rows are tokens_per_group tokens x H heads
  const long long groups = ((long long)a.N + a.tokens_per_group - 1) / a.tokens_per_group;
  const int w = a.tokens_per_group * a.H / 32;
  const bool shared = a.tokens_per_group > 1;
  if (w == 4 && shared)
    hipLaunchKernelGGL((attn_wide_kernel<D, 4, false, 2>), dim3((unsigned)groups), dim3(256), 0,
                       stream, a);
  else if (w == 4)
    hipLaunchKernelGGL((attn_wide_kernel<D, 4, false, 1>), dim3((unsigned)groups), dim3(256), 0,
                       stream, a);
  else if (w == 2 && shared)
    hipLaunchKernelGGL((attn_wide_kernel<D, 2, false, 2>), dim3((unsigned)groups), dim3(128), 0,
                       stream, a);
  else if (w == 2)
    hipLaunchKernelGGL((attn_wide_kernel<D, 2, false, 1>), dim3((unsigned)groups), dim3(128), 0,
                       stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const AttnArgs& a, const AttnPlan& plan, hipStream_t stream) {
  if (plan.mode == kModeSplit) return launch_split(a, D, plan, false, stream);
  if (plan.mode == kModeRows) {
    if (a.paged)
      hipLaunchKernelGGL((attn_rows_kernel<D, true>), dim3((unsigned)(a.N * a.head_groups)),
                         dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((attn_rows_kernel<D, false>), dim3((unsigned)(a.N * a.head_groups)),
                         dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  if (plan.wide) {
    if (a.splits != 1) return hipErrorInvalidValue;
    if (plan.waves == 4) return launch_wide<D, 4>(a, stream);
    if (plan.waves == 2) return launch_wide<D, 2>(a, stream);
    return hipErrorInvalidValue;
  }
  switch (plan.waves) {
    case 1: return launch_heads<D, 1>(a, stream);
    case 2: return launch_heads<D, 2>(a, stream);
    case 4: return launch_heads<D, 4>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool attn_supported(int32_t H, int32_t D) {
  return (D == 64 || D == 128 || D == 256 || D == 512) && H >= 1 && H <= 1024;
}

// Split mode: workgroups of 32 HB heads on 4 waves (HB head blocks x P
// parities), slices cut into partitions of split_rows rows (at most
// kSplitMax) so that the batch gives about one workgroup per CU.  Up to 32
// heads (D >= 128) take HB = 1, P = 4; otherwise HB = 2, P = 2, so that a
// token's rows enter one CU per partition for 64 heads.  (HB = 1, P = 4 for
// 64 heads, a token's rows entering two CUs, measured 32.1 us against 28.5
// us for N = 64 tokens of 640 rows, D = 512.)
constexpr int kSplitMax = 32;
// Shortest capacity bound for which the automatic plan of a small batch
// splits the slices: below it the exchange of the partitions' states costs
// more than the rows the head-split workgroups would share (measured at H =
// 64, D = 512: N = 64 tokens of 1280 rows 37.7 us split against 36.0 us in
// rows mode, of 2048 rows 46.4 us against 49.8 us; N = 8 of 8192 rows 58 us
// against 150 us).
constexpr int kSplitAutoLen = 2048;
// Balanced split plans (no split_rows given, a batch of at most kBalancedSlots
// (token, head group) pairs): kBalancedSlots workgroups in all, one per CU of
// the chip, which the kernel deals out as partitions sized from the call's
// slice lengths, so a long slice among short ones takes more of them.  The
// kernel's plan search holds at most kBalancedMaxN tokens.
constexpr int kBalancedSlots = 256;
constexpr int kBalancedMaxN = 512;

static bool make_split_plan(int32_t N, int32_t H, int32_t D, int32_t max_len, int32_t split_rows,
                            AttnPlan* p) {
  const bool hb1 = H <= 32 && D >= 128;
  p->mode = kModeSplit;
  p->wide = 0;
  p->parities = hb1 ? 4 : 2;
  p->heads_per_group = hb1 ? 32 : 64;
  p->waves = 4;
  p->head_groups = (H + p->heads_per_group - 1) / p->heads_per_group;
  p->bal_slots = 0;
  const long long base = (long long)N * p->head_groups;
  const int super_rows = 16 * p->parities;  // rows of the kernel's super-tile
  if (split_rows == 0 && N > 0 && N <= kBalancedMaxN && base <= kBalancedSlots &&
      max_len > super_rows) {
    // balanced: partitions of at least one super-tile, at most kSplitMax a
    // slice (splits reports that bound; the rows are chosen in the kernel)
    const long long tiles = (max_len + super_rows - 1) / super_rows;
    p->splits = (int)(tiles < kSplitMax ? tiles : kSplitMax);
    p->split_rows = 0;
    p->bal_slots = kBalancedSlots / p->head_groups;
    p->workspace_bytes = split_workspace_bytes(N, D, *p);
    return true;
  }
  long long splits = 1, rows = 0;
  if (split_rows > 0) {
    rows = ((long long)split_rows + 31) / 32 * 32;
    splits = max_len > rows ? (max_len + rows - 1) / rows : 1;
  } else if (max_len > 0 && base > 0 && base < 256) {
    // as many partitions as keep the grid within one workgroup per CU: past
    // that the grid runs in rounds, and the mergers cannot wait for partners
    // that are not resident, so every partition publishes every piece (N = 100
    // tokens of 4096 rows: 3 partitions, 300 workgroups, 164 us; 2 partitions
    // 113 us)
    const long long want = 256 / base;
    const long long cap = (max_len + 63) / 64;  // partitions of at least 64 rows
    splits = want < cap ? want : cap;
    if (splits > kSplitMax) splits = kSplitMax;
    if (splits > 1) {
      rows = (max_len + splits - 1) / splits;
      rows = (rows + 31) / 32 * 32;
      splits = (max_len + rows - 1) / rows;
    }
  }
  if (splits > kSplitMax) return false;
  if (splits <= 1) {
    splits = 1;
    rows = 1 << 30;
  }
  if (base * splits > 0x7fffffffLL) return false;
  p->splits = (int)splits;
  p->split_rows = (int)rows;
  p->workspace_bytes = splits > 1 ? split_workspace_bytes(N, D, *p) : 0;
  return true;
}

bool make_attn_plan(int32_t N, int32_t H, int32_t D, int32_t max_len, int32_t split_rows,
                    int32_t mode, AttnPlan* p) {
  if (!attn_supported(H, D) || N < 0 || max_len < 0 || split_rows < 0) return false;
  if (mode != kModeAuto && mode != kModeHeads && mode != kModeRows && mode != kModeWide &&
      mode != kModeSplit)
    return false;
  p->parities = 1;
  p->bal_slots = 0;
  if (mode == kModeSplit) return make_split_plan(N, H, D, max_len, split_rows, p);
  if (mode == kModeWide) {  // 32-head waves, no split-L
    if (H % 64 != 0 || split_rows != 0) return false;
    p->mode = kModeHeads;
    p->wide = 1;
    p->waves = H % 128 == 0 ? 4 : 2;
    p->heads_per_group = 32 * p->waves;
    p->head_groups = H / p->heads_per_group;
    p->splits = 1;
    p->split_rows = 1 << 30;
    p->workspace_bytes = 0;
    return (long long)N * p->head_groups <= 0x7fffffffLL;
  }
  // heads mode: 16 heads per wave, 16*W heads per workgroup
  const int heads_waves = H <= 16 ? 1 : (H <= 32 ? 2 : 4);
  const int heads_per = 16 * heads_waves;
  const long long heads_groups = (H + heads_per - 1) / heads_per;
  // Work items the heads mode provides without split-L; the chip has 256 CUs.
  const long long target = 256;
  if (mode == kModeAuto && split_rows == 0 && (long long)N * heads_groups <= target &&
      max_len >= kSplitAutoLen) {
    // a batch of at most one workgroup per CU with long slices: partitions
    // sized from the lengths, merged in-kernel (the ragged mix of 256 slices:
    // 87.1 us against 101.8 us in heads mode)
    if (make_split_plan(N, H, D, max_len, 0, p) && p->splits > 1) return true;
    p->parities = 1;
    p->bal_slots = 0;
  }
  if (mode == kModeAuto)
    mode = (split_rows == 0 && (long long)N * heads_groups < target) ? kModeRows : kModeHeads;
  if (mode == kModeRows) {
    if (split_rows != 0) return false;  // the rows mode does not split across workgroups
    p->mode = kModeRows;
    p->wide = 0;
    p->waves = 4;
    p->heads_per_group = 16;
    p->head_groups = (H + 15) / 16;
    p->splits = 1;
    p->split_rows = 1 << 30;
    p->workspace_bytes = 0;
    return (long long)N * p->head_groups <= 0x7fffffffLL;
  }
  p->mode = kModeHeads;
  p->waves = heads_waves;
  p->heads_per_group = heads_per;
  p->head_groups = (int)heads_groups;
  long long splits = 1, rows = 0;
  if (split_rows > 0) {
    rows = ((long long)split_rows + 31) / 32 * 32;
    splits = max_len > rows ? (max_len + rows - 1) / rows : 1;
  } else if (max_len > 0 && N > 0) {
    // Aim at about one workgroup per compute unit when the batch alone does
    // not provide that many; keep partitions >= 128 rows.
    const long long base = (long long)N * p->head_groups;
    if (base < target) {
      const long long want = (target + base - 1) / base;
      const long long cap = (max_len + 127) / 128;
      splits = want < cap ? want : cap;
      if (splits > 64) splits = 64;
      if (splits > 1) {
        rows = (max_len + splits - 1) / splits;
        rows = (rows + 31) / 32 * 32;
        splits = (max_len + rows - 1) / rows;
      }
    }
  }
  if (splits <= 1) {
    splits = 1;
    rows = 1 << 30;
  }
  // Without split-L, head counts that are multiples of 64 run on 32-head
  // waves: 128 heads per workgroup (4 waves, one workgroup per CU) when
  // H % 128 == 0, else 64 (2 waves: two workgroups share a CU, so the batch
  // must give at least two per CU to keep every SIMD busy).
  p->wide = 0;
  if (kUseWide && splits == 1 && H % 64 == 0) {
    const int w = H % 128 == 0 ? 4 : 2;
    const long long items = (long long)N * (H / (32 * w));
    if (items >= (w == 4 ? target : 2 * target)) {
      p->wide = 1;
      p->waves = w;
      p->heads_per_group = 32 * w;
      p->head_groups = H / p->heads_per_group;
    }
  }
  if (splits > 4096) return false;
  if ((long long)N * p->head_groups * splits * 4 > 0x7fffffffLL) return false;
  p->splits = (int)splits;
  p->split_rows = (int)rows;
  p->workspace_bytes = splits > 1 ? (size_t)N * p->head_groups * splits * p->heads_per_group *
                                        (size_t)(D + 2) * sizeof(float)
                                  : 0;
  return true;
}

bool make_fp8_plan(int32_t N, int32_t H, int32_t D, int32_t max_len, int32_t split_rows,
                   int32_t mode, AttnPlan* p) {
  if (!attn_supported(H, D) || N < 0 || max_len < 0 || split_rows < 0) return false;
  if (mode != kModeAuto && mode != kModeRows && mode != kModeWide && mode != kModeSplit)
    return false;
  p->parities = 1;
  p->bal_slots = 0;
  // the batch's workgroups without split-L, counted as for the bf16 pool
  const int heads_per = H <= 16 ? 16 : (H <= 32 ? 32 : 64);
  const long long base = (long long)N * ((H + heads_per - 1) / heads_per);
  // split mode when asked for, when the automatic plan is given a partition
  // length, or for a small batch of long slices
  const bool chosen = mode == kModeSplit || (mode == kModeAuto && split_rows > 0);
  if (chosen || (mode == kModeAuto && base <= 256 && max_len >= kSplitAutoLen && D >= 128)) {
    if (D < 128) return false;
    if (make_split_plan(N, H, D, max_len, split_rows, p) && (chosen || p->splits > 1)) return true;
    if (chosen) return false;
    p->parities = 1;
    p->bal_slots = 0;
  }
  if (split_rows != 0) return false;  // only split mode cuts slices
  // 32-head waves (128 heads a workgroup when H % 128 == 0, else 64) once the
  // batch gives every CU a workgroup (two per CU for 64-head workgroups on
  // two waves); 64-head workgroups on four waves (two parities of each head
  // block) when it gives one per CU; 16-head rows workgroups otherwise.
  int wide = 0;
  if (mode == kModeWide) {
    if (D < 128 || H % 64 != 0) return false;
    wide = H % 128 == 0 ? 4 : 2;
  } else if (mode == kModeAuto && D >= 128 && H % 64 == 0) {
    const int w = H % 128 == 0 ? 4 : 2;
    const long long items = (long long)N * (H / (32 * w));
    if (items >= (w == 4 ? 256 : 512))
      wide = w;
    else if (w == 2 && items >= 256)
      wide = 3;
  }
  p->mode = wide ? kModeHeads : kModeRows;
  p->wide = wide;
  p->waves = wide == 2 ? 2 : 4;
  p->heads_per_group = wide == 4 ? 128 : (wide ? 64 : 16);
  p->head_groups = (H + p->heads_per_group - 1) / p->heads_per_group;
  p->splits = 1;
  p->split_rows = 1 << 30;
  p->workspace_bytes = 0;
  return (long long)N * p->head_groups <= 0x7fffffffLL;
}

hipError_t launch_prefill(const AttnArgs& a, int D, hipStream_t stream) {
  switch (D) {
    case 64: return launch_prefill_d<64>(a, stream);
    case 128: return launch_prefill_d<128>(a, stream);
    case 256: return launch_prefill_d<256>(a, stream);
    case 512: return launch_prefill_d<512>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attention(const AttnArgs& a, int D, const AttnPlan& plan, hipStream_t stream) {
  switch (D) {
    case 64: return launch_d<64>(a, plan, stream);
    case 128: return launch_d<128>(a, plan, stream);
    case 256: return launch_d<256>(a, plan, stream);
    case 512: return launch_d<512>(a, plan, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace spd
