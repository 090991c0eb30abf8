// attn_fp8.hip -- sparse decode attention over an FP8 pool, and the
// quantising store that fills such a pool, gfx950.
//
// Pool format (sglang PR #25898 summary page, "key files": its fused
// norm/RoPE/store kernel and its store-cache kernels quantise rows to FP8 as
// they scatter them into the paged caches; "comment highlights" and "risks
// and impact": the conversion is to round to nearest even, not half up): row
// r holds D OCP e4m3 codes (sign, 4 exponent bits with bias 7, 3 mantissa
// bits; no infinities; 0x7f and 0xff are NaN) and one fp32 scale, and its
// value is kv_scale[r] * e4m3(code).  The attention is the one of attn.hip
// (sglang PR #28392 summary page, "key source snippet") with that row as both
// key and value.
//
// Quantiser, per row x[0, D): amax = max |x|; a row with amax < 2^-64 stores
// scale 0 and zero codes; otherwise scale = amax / 448 and inv = 448 / amax
// (fp32, correctly rounded), y = clamp(x * inv, -448, 448) in fp32, and the
// code is y rounded to the nearest e4m3 value, ties to even (v_cvt_pk_fp8_f32).
// 448 is the largest finite e4m3 value, so the largest |x| maps to +-448.
//
// Attention kernel (rows decomposition, as attn_rows_kernel: workgroup =
// token x 16 heads, its 4 waves take every 4th 16-row tile and merge their
// states in LDS at the end):
//   * a tile's rows are gathered as codes (D bytes a row, half a bf16 row) by
//     LDS-DMA loads into one of four FP8 slots of the wave, with the 16 row
//     scales beside them, so three tiles are in flight while one is used;
//   * the MFMAs stay bf16: the K operand of S^T = K Q^T is read from the slot
//     in the MFMA's lane order (ds_read_b64) and the V^T operand of
//     O^T += V^T P^T with the 8-bit transposing read ds_read_b64_tr_b8; both
//     are converted to bf16 in registers by v_cvt_scalef32_pk_bf16_fp8 with
//     scale 1, which is exact (every e4m3 value is a bf16 value).  Each tile
//     costs 16 bytes of LDS reads per code and no LDS writes;
//   * the scale multiplies its row's scores and its softmax weight, which
//     becomes P' = bf16(p * scale); the denominator sums the unscaled p.
#include "attn_device.h"
#include "fp8_device.h"
#include "row_device.h"
#include "store_internal.h"

namespace spd {
namespace {

// Byte offsets of the K-operand read of an FP8 tile (16 rows of D codes; the
// 16-byte chunk c of row r is stored at c ^ (r & 15), within the row's D / 16
// chunks, by issue_rows).  Lane (n16, g) reads codes 32 s + 8 g .. + 7 of row
// n16 for k-step s: half g & 1 of logical chunk 2 s + (g >> 1).  With
// w = swizzle(n16) ^ (g >> 1) that chunk is stored at 2 (s ^ (w >> 1)) + (w & 1),
// i.e. the read is at k[s & 7] + 256 (s >> 3) bytes.  In the first 32 lanes
// the 16 rows then hit 16 different 4-bank groups, at D >= 256.
template <int D>
struct Fp8Offsets {
  static constexpr int kN = D / 32 < 8 ? D / 32 : 8;
  int k[kN];
  __device__ __forceinline__ Fp8Offsets(int n16, int g) {
    constexpr int kChunks = D / 16;
    const int w = (row_swizzle(n16) & (kChunks - 1)) ^ (g >> 1);
#pragma unroll
    for (int u = 0; u < kN; ++u) k[u] = n16 * D + 32 * (u ^ (w >> 1)) + 16 * (w & 1) + 8 * (g & 1);
  }
  __device__ __forceinline__ int kq(int s) const { return k[s & 7] + 256 * (s >> 3); }
};

// Byte offsets of the V^T reads (ds_read_b64_tr_b8) of an FP8 tile.  Within
// each 16-lane group the read gives destination lane i byte e from source
// lane 2e + i/8, byte i % 8.  Source lane (n16, g), with e = n16 / 2 and
// b = n16 % 2, points at row 4g + e % 4, columns 16 c + 8b .. + 7 of logical
// chunk c = dt + kPair * (e / 4): destination lane (i, g) then holds rows
// 4g .. 4g+3 of column 16 dt + i in bytes 0-3 and of column 16 (dt + kPair) + i
// in bytes 4-7, the V^T operands of two 16x16x16 MFMAs (d-tiles dt and
// dt + kPair).  Pair pp covers dt = 2 kPair (pp / kPair) + pp % kPair.  With
// kPair = 8 (D >= 256) the 16 (row, chunk) reads of each half-wave fall on
// distinct 4-bank groups.  With sw = the row's swizzle (< 2 kPair), the read of
// pair pp is at v[pp % kPair] + 32 kPair (pp / kPair) bytes.
template <int D>
struct Fp8VtOffsets {
  static constexpr int kDTiles = D / 16;
  static constexpr int kPair = kDTiles / 2 < 8 ? kDTiles / 2 : 8;
  int v[kPair];
  __device__ __forceinline__ Fp8VtOffsets(int n16, int g) {
    const int e = n16 >> 1, b = n16 & 1;
    const int r = 4 * g + (e & 3), h = e >> 2;
    const int sw = row_swizzle(r) & (kDTiles - 1);
#pragma unroll
    for (int u = 0; u < kPair; ++u)
      v[u] = r * D + 16 * (kPair * (h ^ (sw / kPair)) + (u ^ (sw % kPair))) + 8 * b;
  }
  __device__ __forceinline__ int pair(int pp) const {
    return v[pp % kPair] + 32 * kPair * (pp / kPair);
  }
  static constexpr int first_dtile(int pp) { return 2 * kPair * (pp / kPair) + pp % kPair; }
};

// The scales of the 16 rows of a tile (staged indices from sidx[p0]; positions
// past n repeat the last row) into sc[0, 64): lane l loads the scale of tile
// row l & 15, so lanes 16 .. 63 repeat the first 16.
__device__ __forceinline__ void issue_scales(const float* kv_scale, const int* sidx, int n, int p0,
                                             float* sc, int lane) {
  const int p = p0 + (lane & 15);
  const int grow = sidx[p < n ? p : n - 1];
  dma_4B(kv_scale + grow, __builtin_amdgcn_readfirstlane(lds_addr(sc)));
}

template <int D>
__global__ void __launch_bounds__(256) attn_rows_fp8_kernel(AttnArgs a) {
  constexpr int kWaves = 4;
  constexpr int kTile = 16;
  constexpr int kKSteps = D / 32;             // also the V^T read pairs of a tile
  constexpr int kDTiles = D / 16;
  constexpr int kSlots = 4;                   // FP8 tile slots per wave
  constexpr int kLoads = kTile * D / 1024;    // LDS-DMA ops per FP8 tile
  constexpr int kPerTile = kLoads + 1;        // and the scale load
  constexpr int kSlotBytes = kTile * D;
  constexpr int kWaveBytes = kSlots * kSlotBytes;
  constexpr int kAhead = kKSteps < 4 ? kKSteps : 4;  // LDS reads issued ahead of use
  static_assert(kWaveBytes == 16 * D * 4, "partial O must fit the wave's LDS");
  static_assert(kLoads >= 1 && (kSlots - 1) * kPerTile < 64, "bad load count");
  using Vt = Fp8VtOffsets<D>;

  __shared__ __attribute__((aligned(1024))) unsigned char smem[kWaves * kWaveBytes];
  __shared__ __attribute__((aligned(256))) int sidx[kIdxCap];
  __shared__ __attribute__((aligned(256))) float ssink[64];
  __shared__ __attribute__((aligned(256))) float sscale[kWaves][kSlots][64];
  __shared__ float sml[kWaves][2][16];
  __shared__ int sflag[kWaves];

  const int item = xcd_item(blockIdx.x, gridDim.x);
  const int hg = item % a.head_groups;
  const int t = item / a.head_groups;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n16 = lane & 15;
  const int g = lane >> 4;

  const ScalarI32Ptr indptr = (ScalarI32Ptr)a.kv_indptr;
  const int row0 = indptr[t];
  const int L = indptr[t + 1] - row0;
  const int32_t* part = a.kv_indices + row0;
  const int h0 = hg * 16;
  const int h = h0 + n16;
  const bool hvalid = h < a.H;
  const int nh = a.H - h0 < 16 ? a.H - h0 : 16;

  if (L <= 0) {
    zero_heads<D>(a.out, a.H, t, h0, nh, threadIdx.x, 64 * kWaves);
    return;
  }

  bf16x8 qreg[kKSteps];
  load_q<D>(a.q, (int64_t)t * a.H + (hvalid ? h : 0), g, qreg);
  stage_sinks(a.sink, a.H, h0, ssink, wave, lane);

  unsigned char* mine = smem + wave * kWaveBytes;  // the wave's FP8 slots
  const uint16_t* kv8 = reinterpret_cast<const uint16_t*>(a.kv8);  // rows of D bytes
  const Fp8Offsets<D> off8(n16, g);
  const Vt offv(n16, g);

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
      if (restage) {
        barrier_lds();  // every wave is done with the indices and its slots
        stage_indices(part, sc, n, sidx, wave, kWaves, lane);
        wait_vmcnt<0>();
        barrier_lds();
      } else if (pass == 0) {
        stage_indices(part, sc, n, sidx, wave, kWaves, lane);
        wait_vmcnt<0>();
        barrier_lds();
        sink_l2 = (wave == 0 && hvalid) ? ssink[n16] * kLog2e : -INFINITY;  // sink in wave 0
      }
      const int ntiles = (n + kTile - 1) / kTile;
      const int my_tiles = ntiles > wave ? (ntiles - wave + kWaves - 1) / kWaves : 0;

      auto issue = [&](int j) {  // this wave's j-th tile = global tile wave + 4j, slot j % 4
        const int p0 = (wave + kWaves * j) * kTile;
        issue_rows<D, kLoads>(kv8, sidx, n, p0, 0, mine + (j % kSlots) * kSlotBytes, lane);
        issue_scales(a.kv_scale, sidx, n, p0, sscale[wave][j % kSlots], lane);
      };
      // Wait until tile j has landed.  Every tile up to j + 3 (below my_tiles)
      // has been issued by then, in order, so exactly those after j may stay
      // in flight.
      auto wait_tile = [&](int j) {
        const int later = my_tiles - 1 - j;
        if (later >= 3)
          wait_vmcnt<3 * kPerTile>();
        else if (later == 2)
          wait_vmcnt<2 * kPerTile>();
        else if (later == 1)
          wait_vmcnt<kPerTile>();
        else
          wait_vmcnt<0>();
      };

      // Pipeline over this wave's tiles, four slots: in iteration j, S^T of
      // tile j (K operand in registers) with the V^T reads of tile j; once
      // those reads are done the slot takes the loads of tile j+4; then the PV
      // MFMAs of tile j with the K-operand reads of tile j+1.
      bf16x8 ka[kKSteps];
      f32x4 scl = {0.f, 0.f, 0.f, 0.f};  // scales of rows 4g .. 4g+3 of the current tile
#pragma unroll
      for (int j = 0; j < kSlots; ++j)  // tiles 0 .. 3 fill the four slots
        if (j < my_tiles) issue(j);
      if (my_tiles > 0) {
        wait_tile(0);
        asm volatile("" ::: "memory");
        u32x2 raw[kKSteps];
#pragma unroll
        for (int s = 0; s < kKSteps; ++s) raw[s] = *reinterpret_cast<const u32x2*>(mine + off8.kq(s));
        scl = *reinterpret_cast<const f32x4*>(&sscale[wave][0][4 * g]);
#pragma unroll
        for (int s = 0; s < kKSteps; ++s) ka[s] = e4m3x8_to_bf16(raw[s]);
      }
      for (int j = 0; j < my_tiles; ++j) {
        const unsigned char* st = mine + (j % kSlots) * kSlotBytes;
        const int nvalid = n - (wave + kWaves * j) * kTile;
        constexpr int kCh = kKSteps < 4 ? kKSteps : 4;  // independent QK chains
        f32x4 part_s[kCh];
#pragma unroll
        for (int c = 0; c < kCh; ++c) part_s[c] = f32x4{0.f, 0.f, 0.f, 0.f};
        bf16x4 vt[kDTiles];
        u32x2 vraw[kKSteps];
        __builtin_amdgcn_sched_barrier(0);
        // S^T = K Q^T (four chains) with the V^T reads of the same tile
#pragma unroll
        for (int s = 0; s < kKSteps; ++s) {
          part_s[s % kCh] = mfma_k32(ka[s], qreg[s], part_s[s % kCh]);
          vraw[s] = __builtin_bit_cast(
              u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32((LdsV2i32*)(st + offv.pair(s))));
        }
#pragma unroll
        for (int s = 0; s < kKSteps; ++s) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
        }
        __builtin_amdgcn_sched_barrier(0);
        f32x4 sa = part_s[0];
#pragma unroll
        for (int c = 1; c < kCh; ++c) sa += part_s[c];
        float x[4];
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4)
          x[i4] = (4 * g + i4 < nvalid) ? sa[i4] * (a.qk_scale * scl[i4]) : -INFINITY;
        float pf[4];
        over |= softmax_tile_f32<4>(x, sink_l2, g, first, m, mtrue, lpart, pf);
        bf16x4 pt;
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) pt[i4] = (__bf16)(pf[i4] * scl[i4]);
#pragma unroll
        for (int s = 0; s < kKSteps; ++s) {
          vt[Vt::first_dtile(s)] = e4m3x4_to_bf16(vraw[s][0]);
          vt[Vt::first_dtile(s) + Vt::kPair] = e4m3x4_to_bf16(vraw[s][1]);
        }
        // Every read of tile j's slot is complete: it takes the loads of tile j+4.
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        asm volatile("" ::: "memory");
        if (j + kSlots < my_tiles) issue(j + kSlots);
        if (j + 1 < my_tiles) wait_tile(j + 1);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        // O^T += V^T P^T with the K-operand reads of tile j+1 (after the last
        // tile they read a slot with no load in flight: in bounds, unused).
        const unsigned char* sn = mine + ((j + 1) % kSlots) * kSlotBytes;
        u32x2 kraw[kKSteps];
#pragma unroll
        for (int s = 0; s < kAhead; ++s) kraw[s] = *reinterpret_cast<const u32x2*>(sn + off8.kq(s));
        const f32x4 scn = *reinterpret_cast<const f32x4*>(&sscale[wave][(j + 1) % kSlots][4 * g]);
#pragma unroll
        for (int s = 0; s < kKSteps; ++s) {
          if (s + kAhead < kKSteps)
            kraw[s + kAhead] = *reinterpret_cast<const u32x2*>(sn + off8.kq(s + kAhead));
          const int d0 = Vt::first_dtile(s);
          acc[d0] = mfma_k16(vt[d0], pt, acc[d0]);
          acc[d0 + Vt::kPair] = mfma_k16(vt[d0 + Vt::kPair], pt, acc[d0 + Vt::kPair]);
          ka[s] = e4m3x8_to_bf16(kraw[s]);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, kAhead + 1, 0);  // LDS reads
#pragma unroll
        for (int s = 0; s < kKSteps; ++s) {
          if (s + kAhead < kKSteps) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // VALU: conversion
        }
        __builtin_amdgcn_sched_barrier(0);
        scl = scn;
      }
    }
    if (!workgroup_any(over, sflag, wave, kWaves)) break;
  }

  // Merge the four waves' states (as attn_rows_kernel): wave w's partial O
  // goes to its own LDS area as [head][d] fp32, 16-byte columns XOR-ed by head.
  const float l = group_sum4(lpart);
  {
    f32x4* po = reinterpret_cast<f32x4*>(mine);
#pragma unroll
    for (int dt = 0; dt < kDTiles; ++dt) {
      const int col = (4 * dt + g) ^ n16;
      po[n16 * (D / 4) + col] = acc[dt];
    }
    if (g == 0) {
      sml[wave][0][n16] = m;
      sml[wave][1][n16] = l;
    }
  }
  barrier_lds();

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
  constexpr int kPer = D / 64;
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

// ---------------------------------------------------------------------------
// Wide heads mode over an FP8 pool: workgroup = (token, 32 W heads), W waves
// of 32 heads sharing every 32-row tile of codes (as attn_wide_kernel over
// the bf16 pool; no split-L).  Per wave and tile, S^T = K Q^T on 16x16x32
// MFMAs (K operand: one ds_read_b64 of 8 codes per k-step and 16-row half,
// shared by both head blocks) and O^T += V^T P^T on 32x32x16 MFMAs (V^T
// operand: one ds_read_b64_tr_b8 per d-tile and half, fp8_device.h); codes
// are decoded to bf16 in registers.  Each K and V^T code is read from LDS
// once per 32 heads: a quarter of the LDS bytes per flop of the 16-head FP8
// rows kernel.  The row scales multiply scores and weights as there.

// Weight 2^(m - M) of a state with reference maximum m in a merge whose
// maximum is M >= m; a state that saw no row (m = -inf) weighs exactly 0.
__device__ __forceinline__ float fp8_state_weight(float m, float M) {
  return m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - M);
}

// P = 1: workgroups of 32 W heads, each wave 32 heads over all 32 rows of a
// tile.  P = 2 (W = 4): workgroups of 64 heads, waves (head block hb, parity
// par) = (wave / 2, wave % 2); a wave takes rows [16 par, 16 par + 16) of
// each tile for its 32 heads, so all four SIMDs work when H is 64; at the
// end the two parity states of a head block merge in LDS, each wave keeping
// half of D.
template <int D, int W, int P = 1>
__global__ void __launch_bounds__(64 * W) attn_wide_fp8_kernel(AttnArgs a) {
  constexpr int kTile = 32;
  constexpr int kStageBytes = kTile * D;
  constexpr int kKSteps = D / 32;
  constexpr int kDT = D / 32;                       // 32-wide d-tiles of the PV product
  constexpr int kRowsPerLoad = 1024 / D;            // rows per LDS-DMA op
  constexpr int kLoadsPerWave = kTile / kRowsPerLoad / W;
  constexpr int kRowsPerWave = kTile / W;           // rows (and scales) each wave loads
  constexpr int kPerTile = kLoadsPerWave + 1;       // and the scale load
  constexpr int kHB = W / P;  // 32-head blocks of the workgroup
  constexpr int kHeads = 32 * kHB;
  // W = 4: one workgroup per CU, three tiles in flight; W = 2: two per CU
  constexpr int kAhead = W >= 4 ? 3 : 2;
  constexpr int kStages = kAhead + 1;
  static_assert(P == 1 || (P == 2 && W == 4), "parities: P = 2 with four waves");
  // LDS of the stages, and of the parity merge (each wave hands over half of
  // its accumulators)
  constexpr int kMergeBytes = P > 1 ? W * (kDT / 2) * 64 * 64 : 0;
  constexpr int kSmem = kStages * kStageBytes > kMergeBytes ? kStages * kStageBytes : kMergeBytes;
  static_assert(D >= 128 && D <= 512 && D % 64 == 0, "unsupported D");
  static_assert(kLoadsPerWave >= 1 && kTile % (kRowsPerLoad * W) == 0, "loads must divide");
  static_assert((kAhead - 1) * kPerTile < 64, "vmcnt range");
  using Vt = Fp8WideVtOffsets<D>;

  __shared__ __attribute__((aligned(1024))) unsigned char smem[kSmem];
  __shared__ __attribute__((aligned(256))) int sidx[kIdxCap];
  __shared__ __attribute__((aligned(256))) float ssink[kHeads];
  __shared__ __attribute__((aligned(256))) float sscale[kStages][W][64];
  __shared__ float sml[W][4][16];  // parity merge: m0, m1, l0, l1 of each wave's 32 heads
  __shared__ int sflag[W];

  const int item = xcd_item(blockIdx.x, gridDim.x);
  const int hg = item % a.head_groups;
  const int t = item / a.head_groups;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n16 = lane & 15;
  const int g = lane >> 4;
  const int hb = wave / P;    // head block
  const int par = wave % P;   // parity: rows [16 par, 16 par + 16) of each tile (P = 2)
  const int h0 = hg * kHeads + hb * 32;  // first head of this wave (H % kHeads == 0)

  const ScalarI32Ptr indptr = (ScalarI32Ptr)a.kv_indptr;
  const int row0 = indptr[t];
  const int L = indptr[t + 1] - row0;
  const int32_t* part = a.kv_indices + row0;
  if (L <= 0) {
    if (par == 0) zero_heads<D>(a.out, a.H, t, h0, 32, lane, 64);
    return;
  }

  bf16x8 q0[kKSteps], q1[kKSteps];  // Q^T operands of head blocks 0 and 1
  const int64_t qrow = (int64_t)t * a.H + h0;
  load_q<D>(a.q, qrow + n16, g, q0);
  load_q<D>(a.q, qrow + 16 + n16, g, q1);
  if (wave == 0) {  // the workgroup's kHeads sinks, one LDS-DMA per 64
#pragma unroll
    for (int c = 0; c < kHeads; c += 64)
      dma_4B(a.sink + hg * kHeads + c + lane, __builtin_amdgcn_readfirstlane(lds_addr(ssink + c)));
  }

  const uint16_t* kv8 = reinterpret_cast<const uint16_t*>(a.kv8);  // rows of D bytes
  const Fp8KOffsets<D> off8(n16, g);
  const Vt voff(lane);

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
      stage_indices(part, sc, n, sidx, wave, W, lane);
      wait_vmcnt<0>();
      barrier_lds();
      if (pass == 0 && sc == 0) {  // (with parities, the sink belongs to parity 0)
        sk0 = par == 0 ? ssink[hb * 32 + n16] * kLog2e : -INFINITY;
        sk1 = par == 0 ? ssink[hb * 32 + 16 + n16] * kLog2e : -INFINITY;
      }
      const int ntiles = (n + kTile - 1) / kTile;

      // this wave's rows of a tile (codes, then their scales: lane l loads
      // the scale of row l % kRowsPerWave of its part)
      auto issue_tile = [&](int tile) {
        const int st = tile % kStages;
        const int p0 = tile * kTile + wave * kRowsPerWave;
        // The lane id is made opaque per call: the loads' per-lane chunk
        // addresses are loop-invariant, and hoisting them (two registers a
        // load) would spill the 64-head workgroup's eight loads.
        int ln = lane;
        asm volatile("" : "+v"(ln));
        issue_rows<D, kLoadsPerWave>(kv8, sidx, n, p0, wave * kRowsPerWave,
                                     smem + st * kStageBytes + wave * kRowsPerWave * D, ln);
        const int p = p0 + lane % kRowsPerWave;
        const int grow = sidx[p < n ? p : n - 1];
        dma_4B(a.kv_scale + grow, __builtin_amdgcn_readfirstlane(lds_addr(sscale[st][wave])));
      };
#pragma unroll
      for (int k = 0; k < kAhead; ++k)
        if (k < ntiles) issue_tile(k);

      for (int i = 0; i < ntiles; ++i) {
        // tile i has landed once at most min(kAhead - 1, ntiles - 1 - i) later
        // tiles of this wave are still outstanding
        const int later = ntiles - 1 - i;
        if (later >= 2 && kAhead >= 3)
          wait_vmcnt<(kAhead >= 3 ? 2 : 0) * kPerTile>();
        else if (later >= 1)
          wait_vmcnt<kPerTile>();
        else
          wait_vmcnt<0>();
        barrier_lds();  // every wave's part of tile i is in LDS; tile i-1's stage is free
        if (i + kAhead < ntiles) issue_tile(i + kAhead);

        int stoff = (i % kStages) * kStageBytes;
        asm volatile("" : "+v"(stoff));
        const unsigned char* st = smem + stoff;
        const float* scl = sscale[i % kStages][0];
        const int nvalid = n - i * kTile;

        if constexpr (P == 2) {
          const int nv = nvalid - 16 * par;  // rows of this wave's 16 that exist
          if (nv <= 0) continue;             // (wave-uniform: a ragged tail)
          const unsigned char* sp = st + 16 * D * par;  // the parity's 16 rows
          // S^T = K Q^T over the parity's rows, head blocks 0 and 1
          f32x4 s00 = {0.f, 0.f, 0.f, 0.f}, s01 = s00;
          {
            constexpr int kPre = kKSteps < 2 ? kKSteps : 2;
            u32x2 ra[kKSteps];
#pragma unroll
            for (int u = 0; u < kPre; ++u) ra[u] = *reinterpret_cast<const u32x2*>(sp + off8.kq(u));
#pragma unroll
            for (int u = 0; u < kKSteps; ++u) {
              if (u + kPre < kKSteps) ra[u + kPre] = *reinterpret_cast<const u32x2*>(sp + off8.kq(u + kPre));
              const bf16x8 ka = e4m3x8_to_bf16(ra[u]);
              s00 = mfma_k32(ka, q0[u], s00);
              s01 = mfma_k32(ka, q1[u], s01);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
          const int r0 = 16 * par + 4 * g;
          const f32x4 c0 = *reinterpret_cast<const f32x4*>(
              scl + (r0 / kRowsPerWave) * 64 + r0 % kRowsPerWave);
          float x0[4], x1[4];
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            const bool v = 4 * g + i4 < nv;
            x0[i4] = v ? s00[i4] * (a.qk_scale * c0[i4]) : -INFINITY;
            x1[i4] = v ? s01[i4] * (a.qk_scale * c0[i4]) : -INFINITY;
          }
          float pf0[4], pf1[4];
          over |= softmax_tile_f32<4>(x0, sk0, g, first0, m0, mt0, l0, pf0);
          over |= softmax_tile_f32<4>(x1, sk1, g, first1, m1, mt1, l1, pf1);
          bf16x4 a0, a1;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            a0[e] = (__bf16)(pf0[e] * c0[e]);
            a1[e] = (__bf16)(pf1[e] * c0[e]);
          }
          const bf16x8 pb = wide_p_operand(a0, a1);
          // O^T += V^T P^T over the parity's 16 rows
          {
            constexpr int kPre = kDT < 2 ? kDT : 2;
            u32x2 va[kDT];
            auto read_vt = [&](int u) {
              va[u] = __builtin_bit_cast(
                  u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32((LdsV2i32*)(sp + voff.at(u))));
            };
#pragma unroll
            for (int u = 0; u < kPre; ++u) read_vt(u);
#pragma unroll
            for (int u = 0; u < kDT; ++u) {
              if (u + kPre < kDT) read_vt(u + kPre);
              acc[u] = mfma32(e4m3x8_to_bf16(va[u]), pb, acc[u]);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
        } else {
        // S^T = K Q^T: rows 0-15 and 16-31, head blocks 0 and 1.  Per k-step:
        // the code reads of k-step u + 2, the decode of k-step u, its four
        // MFMAs (the fence keeps each decode next to its MFMAs, so only two
        // k-steps of codes are live).
        f32x4 s00 = {0.f, 0.f, 0.f, 0.f}, s01 = s00, s10 = s00, s11 = s00;
        {
          constexpr int kPre = kKSteps < 2 ? kKSteps : 2;
          u32x2 ra[kKSteps], rb[kKSteps];
#pragma unroll
          for (int u = 0; u < kPre; ++u) {
            ra[u] = *reinterpret_cast<const u32x2*>(st + off8.kq(u));
            rb[u] = *reinterpret_cast<const u32x2*>(st + off8.kq(u) + 16 * D);
          }
#pragma unroll
          for (int u = 0; u < kKSteps; ++u) {
            if (u + kPre < kKSteps) {
              ra[u + kPre] = *reinterpret_cast<const u32x2*>(st + off8.kq(u + kPre));
              rb[u + kPre] = *reinterpret_cast<const u32x2*>(st + off8.kq(u + kPre) + 16 * D);
            }
            const bf16x8 ka = e4m3x8_to_bf16(ra[u]);
            const bf16x8 kb = e4m3x8_to_bf16(rb[u]);
            s00 = mfma_k32(ka, q0[u], s00);
            s01 = mfma_k32(ka, q1[u], s01);
            s10 = mfma_k32(kb, q0[u], s10);
            s11 = mfma_k32(kb, q1[u], s11);
            __builtin_amdgcn_sched_barrier(0);
          }
        }

        // scales of this lane's rows 4g..4g+3 and 16+4g..16+4g+3 (row r was
        // loaded by wave r / kRowsPerWave into entry r % kRowsPerWave)
        const int r0 = 4 * g, r1 = 16 + 4 * g;
        const f32x4 c0 = *reinterpret_cast<const f32x4*>(
            scl + (r0 / kRowsPerWave) * 64 + r0 % kRowsPerWave);
        const f32x4 c1 = *reinterpret_cast<const f32x4*>(
            scl + (r1 / kRowsPerWave) * 64 + r1 % kRowsPerWave);
        float x0[8], x1[8];
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const bool v0 = 4 * g + i4 < nvalid, v1 = 16 + 4 * g + i4 < nvalid;
          x0[i4] = v0 ? s00[i4] * (a.qk_scale * c0[i4]) : -INFINITY;
          x0[4 + i4] = v1 ? s10[i4] * (a.qk_scale * c1[i4]) : -INFINITY;
          x1[i4] = v0 ? s01[i4] * (a.qk_scale * c0[i4]) : -INFINITY;
          x1[4 + i4] = v1 ? s11[i4] * (a.qk_scale * c1[i4]) : -INFINITY;
        }
        float pf0[8], pf1[8];
        over |= softmax_tile_f32<8>(x0, sk0, g, first0, m0, mt0, l0, pf0);
        over |= softmax_tile_f32<8>(x1, sk1, g, first1, m1, mt1, l1, pf1);
        bf16x8 pb[2];  // B operands for rows 0-15 and 16-31
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          const f32x4 c = rb == 0 ? c0 : c1;
          bf16x4 a0, a1;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            a0[e] = (__bf16)(pf0[4 * rb + e] * c[e]);
            a1[e] = (__bf16)(pf1[4 * rb + e] * c[e]);
          }
          pb[rb] = wide_p_operand(a0, a1);
        }

        // O^T += V^T P^T: per d-tile, the transposing reads of d-tile u + 2,
        // the decode of d-tile u and its two MFMAs.
        {
          constexpr int kPre = kDT < 2 ? kDT : 2;
          u32x2 va[kDT], vb[kDT];
          auto read_vt = [&](int u) {
            const int o = voff.at(u);
            va[u] = __builtin_bit_cast(
                u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32((LdsV2i32*)(st + o)));
            vb[u] = __builtin_bit_cast(
                u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32((LdsV2i32*)(st + o + 16 * D)));
          };
#pragma unroll
          for (int u = 0; u < kPre; ++u) read_vt(u);
#pragma unroll
          for (int u = 0; u < kDT; ++u) {
            if (u + kPre < kDT) read_vt(u + kPre);
            acc[u] = mfma32(e4m3x8_to_bf16(va[u]), pb[0], acc[u]);
            acc[u] = mfma32(e4m3x8_to_bf16(vb[u]), pb[1], acc[u]);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        }
      }
    }
    if (!workgroup_any(over, sflag, wave, W)) break;
  }

  // lane (n, hf) = lane n + 32 hf holds, for head h0 + n, d = 32 dt + 8 e4 +
  // 4 hf + e as element 4 e4 + e of acc[dt]; its denominator is block n / 16's
  // l of head n % 16, which every lane with lane % 16 == n % 16 holds.
  float lb0 = group_sum4(l0), lb1 = group_sum4(l1);
  const int nn = lane & 31, hf = lane >> 5;
  // P = 2: the two parity states of the head block merge in LDS; the lower
  // parity keeps d-tiles [0, kDT / 2), the upper one the rest, each combining
  // its own half with the half its partner hands over (the lower parity's
  // state first).  A parity that saw no row has m = -inf and weighs 0.
  int lo = 0;
  if constexpr (P == 2) {
    constexpr int kHalf = kDT / 2;
    const bool upper = par != 0;
    const int partner = hb * P + (par ^ 1);
    barrier_lds();  // the stages are free
    if (g == 0) {
      sml[wave][0][n16] = m0;
      sml[wave][1][n16] = m1;
      sml[wave][2][n16] = lb0;
      sml[wave][3][n16] = lb1;
    }
    f32x4* mine = reinterpret_cast<f32x4*>(smem) + wave * kHalf * 256 + lane;
    if (upper) {
#pragma unroll
      for (int i = 0; i < kHalf; ++i)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4)
          mine[(i * 4 + e4) * 64] = f32x4{acc[i][4 * e4], acc[i][4 * e4 + 1], acc[i][4 * e4 + 2], acc[i][4 * e4 + 3]};
    } else {
#pragma unroll
      for (int i = 0; i < kHalf; ++i)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4)
          mine[(i * 4 + e4) * 64] = f32x4{acc[kHalf + i][4 * e4], acc[kHalf + i][4 * e4 + 1],
                                          acc[kHalf + i][4 * e4 + 2], acc[kHalf + i][4 * e4 + 3]};
    }
    barrier_lds();
    const float pm0 = sml[partner][0][n16], pm1 = sml[partner][1][n16];
    const float pl0 = sml[partner][2][n16], pl1 = sml[partner][3][n16];
    const float M0 = fmaxf(m0, pm0), M1 = fmaxf(m1, pm1);
    const float ws0 = fp8_state_weight(m0, M0), wp0 = fp8_state_weight(pm0, M0);
    const float ws1 = fp8_state_weight(m1, M1), wp1 = fp8_state_weight(pm1, M1);
    const float wself = nn < 16 ? ws0 : ws1, wpart = nn < 16 ? wp0 : wp1;
    const f32x4* tp = reinterpret_cast<const f32x4*>(smem) + partner * kHalf * 256 + lane;
    if (upper) {
#pragma unroll
      for (int i = 0; i < kHalf; ++i) {
        f32x16 other;
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const f32x4 q4 = tp[(i * 4 + e4) * 64];
#pragma unroll
          for (int e = 0; e < 4; ++e) other[4 * e4 + e] = q4[e];
        }
        acc[i] = wpart * other + wself * acc[kHalf + i];
      }
      lb0 = wp0 * pl0 + ws0 * lb0;
      lb1 = wp1 * pl1 + ws1 * lb1;
      lo = kHalf;
    } else {
#pragma unroll
      for (int i = 0; i < kHalf; ++i) {
        f32x16 other;
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const f32x4 q4 = tp[(i * 4 + e4) * 64];
#pragma unroll
          for (int e = 0; e < 4; ++e) other[4 * e4 + e] = q4[e];
        }
        acc[i] = wself * acc[i] + wpart * other;
      }
      lb0 = ws0 * lb0 + wp0 * pl0;
      lb1 = ws1 * lb1 + wp1 * pl1;
    }
  }
  const float inv = 1.0f / (nn < 16 ? lb0 : lb1);
  uint16_t* op = a.out + ((int64_t)t * a.H + h0 + nn) * D + 4 * hf;
#pragma unroll
  for (int dt = 0; dt < kDT / P; ++dt)
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {  // d = 8 e4 + 4 hf + e: chunk half e4 / 2 of d-tile lo + dt
      const f32x4 v = {acc[dt][4 * e4], acc[dt][4 * e4 + 1], acc[dt][4 * e4 + 2], acc[dt][4 * e4 + 3]};
      store_bf16x4(op + 16 * wide_vt_chunk<D>(lo + dt, e4 >> 1) + 8 * (e4 & 1), v, inv);
    }
}

// ---------------------------------------------------------------------------
// Quantising store: one wave per source row, D / 64 values per lane; row i
// goes to pool row slots[i] (i when slots is null); a slot outside
// [0, num_rows) skips the row.
template <int D>
__global__ void __launch_bounds__(256) quantize_fp8_kernel(QuantArgs a) {
  constexpr int E = D / 64;
  const int lane = threadIdx.x & 63;
  const int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (i >= a.n) return;  // wave-uniform
  const int64_t slot = a.slots != nullptr ? (int64_t)a.slots[i] : i;
  if (slot < 0 || slot >= a.num_rows) return;

  float x[E];
  load_bf16_lane<E>(a.src + i * D + lane * E, x);
  store_fp8_lane<E>(x, a.kv8 + slot * D + lane * E, a.kv_scale + slot, lane);
}

template <int D>
hipError_t launch_fp8_d(const AttnArgs& a, int wide_waves, hipStream_t stream) {
  const dim3 grid((unsigned)(a.N * a.head_groups));
  if constexpr (D >= 128) {
    if (wide_waves == 4) {
      hipLaunchKernelGGL((attn_wide_fp8_kernel<D, 4>), grid, dim3(256), 0, stream, a);
      return hipGetLastError();
    }
    if (wide_waves == 2) {
      hipLaunchKernelGGL((attn_wide_fp8_kernel<D, 2>), grid, dim3(128), 0, stream, a);
      return hipGetLastError();
    }
    if (wide_waves == 3) {  // 64 heads on four waves: two head blocks x two parities
      hipLaunchKernelGGL((attn_wide_fp8_kernel<D, 4, 2>), grid, dim3(256), 0, stream, a);
      return hipGetLastError();
    }
  }
  if (wide_waves != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL((attn_rows_fp8_kernel<D>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_quant_d(const QuantArgs& a, hipStream_t stream) {
  const long long blocks = ((long long)a.n + 3) / 4;
  hipLaunchKernelGGL((quantize_fp8_kernel<D>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention_fp8(const AttnArgs& a, int D, const AttnPlan& plan,
                                hipStream_t stream) {
  if (plan.mode == kModeSplit) return launch_split(a, D, plan, true, stream);
  const int wide_waves = plan.wide;
  switch (D) {
    case 64: return launch_fp8_d<64>(a, wide_waves, stream);
    case 128: return launch_fp8_d<128>(a, wide_waves, stream);
    case 256: return launch_fp8_d<256>(a, wide_waves, stream);
    case 512: return launch_fp8_d<512>(a, wide_waves, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_quantize_fp8(const QuantArgs& a, int D, hipStream_t stream) {
  switch (D) {
    case 64: return launch_quant_d<64>(a, stream);
    case 128: return launch_quant_d<128>(a, stream);
    case 256: return launch_quant_d<256>(a, stream);
    case 512: return launch_quant_d<512>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace spd
