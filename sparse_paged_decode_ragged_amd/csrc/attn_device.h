// attn_device.h -- device helpers shared by the attention kernels of libspd
// (bf16 pool: attn.hip; FP8 pool: attn_fp8.hip): LDS-DMA row gathers with the
// XOR-swizzled tile layouts, MFMA wrappers, the XCD-aware work mapping, the
// online-softmax tile step with its fixed reference maximum, and the
// cross-lane reductions.  Everything is in an anonymous namespace: each
// translation unit gets its own copy.
#pragma once

#include <math.h>

#include <type_traits>

#include "spd_internal.h"

namespace spd {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(4))) int32_t* ScalarI32Ptr;
typedef __attribute__((address_space(3))) bf16x4 LdsBf16x4;

constexpr int kIdxCap = 2048;              // row indices staged in LDS at a time
static_assert(kPagedMaxLen <= kIdxCap, "a paged list is built in LDS at once");
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRaise = 64.0f;            // log2 headroom of the fixed reference max
constexpr bool kUseWide = true;            // heads mode on 32-head waves where it applies

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt[3:0] in bits
// 3:0, vmcnt[5:4] in bits 15:14; expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt out of range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Workgroup barrier without a memory fence: the LDS data it publishes was
// written by LDS-DMA loads that each wave has already waited for with
// wait_vmcnt, or by ordinary LDS stores, which lgkmcnt(0) completes before
// the barrier.  The empty asm keeps the compiler from moving memory accesses
// across it.
__device__ __forceinline__ void barrier_lds() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// XOR swizzle of the 16-byte chunks of LDS row r: chunk c is stored at
// c ^ (r & 15).  Rows 0..15 then put any one logical chunk in 16 different
// bank positions; among the layouts measured on gfx950 for the K reads (16
// rows, one 16-byte chunk each) and the transpose reads (4 rows x 32 bytes),
// this one gives the highest K-read rate at a near-equal transpose rate.
__device__ __forceinline__ int row_swizzle(int r) { return r & 15; }

// The swizzle of the 32-head-wave (wide) tiles: chunk c of row r is stored at
// c ^ (4 (r mod 4) + (r / 4) mod 4).  Its transposing reads (four consecutive
// rows per 16-lane group) then spread over every bank, as do the K reads.
__device__ __forceinline__ int wide_swizzle(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

template <int kSwz>
__device__ __forceinline__ int tile_swizzle(int r) {
  return kSwz == 0 ? row_swizzle(r) : wide_swizzle(r & 15);
}

// Per-lane byte offsets, within a tile's LDS stage, of the two read patterns,
// split so that the tile-dependent part is an instruction immediate.
//  * K read (S^T = K Q^T): lane (n16, g) reads logical 16-byte chunk 4s + g
//    of row n16; with sw = swizzle(n16) = 4a + b that chunk is stored at
//    4 (s ^ a) + (g ^ b) = 4 (s & ~3) + 4 ((s & 3) ^ a) + (g ^ b), i.e. at
//    koff[s & 3] + 256 (s >> 2) bytes.
//  * transpose read (V^T operand): lane (n16, g) reads d = 16 dt + 4 (n16 & 3)
//    .. +3 of row rtr = 4g + n16/4; with sw = swizzle(rtr) = 2c + e, the chunk
//    (2 dt + b1) ^ sw (b1 = bit 1 of n16) is 2 (dt ^ c) + (b1 ^ e), i.e. the
//    read is at voff[dt & 7] + 256 (dt >> 3) bytes.
template <int D, int kSwz = 0>
struct TileOffsets {
  static constexpr int kRowBytes = 2 * D;
  static constexpr int kChunks = D / 8;
  int k[4];
  int v[8];
  __device__ __forceinline__ TileOffsets(int n16, int g) {
    const int rtr = 4 * g + (n16 >> 2);
    const int sk = tile_swizzle<kSwz>(n16) & (kChunks - 1);
    const int sv = tile_swizzle<kSwz>(rtr) & (kChunks - 1);
#pragma unroll
    for (int u = 0; u < 4; ++u) k[u] = n16 * kRowBytes + 64 * (u ^ (sk >> 2)) + 16 * (g ^ (sk & 3));
#pragma unroll
    for (int u = 0; u < 8; ++u)
      v[u] = rtr * kRowBytes + 32 * (u ^ (sv >> 1)) + 16 * (((n16 >> 1) & 1) ^ (sv & 1)) +
             8 * (n16 & 1);
  }
  // byte offset of k-step s of the K read, and of d-tile dt of the transpose read
  __device__ __forceinline__ int kq(int s) const { return k[s & 3] + 256 * (s >> 2); }
  __device__ __forceinline__ int vt(int dt) const { return v[dt & 7] + 256 * (dt >> 3); }
};

// Per-lane byte offsets of the 32x32x16 V^T operand reads within a stage:
// lane (G = lane / 16, j = lane % 16) reads row 8 (G / 2) + 4 half + j / 4,
// d = 32 dt + 16 (G % 2) + 4 (j % 4) .. +3, i.e. logical 16-byte chunk
// 4 dt + b (b = 2 (G % 2) + (j / 2) % 2) at byte 8 (j % 2); stored at chunk
// (4 dt + b) ^ sw with sw = wide_swizzle(row) < 16, that is
// 4 ((dt % 4) ^ (sw / 4)) + 16 (dt / 4) ... split as v[half][dt % 4] + 256 (dt / 4).
template <int D>
struct WideVtOffsets {
  static constexpr int kRowBytes = 2 * D;
  static constexpr int kChunks = D / 8;
  int v[2][4];
  __device__ __forceinline__ explicit WideVtOffsets(int lane) {
    const int G = lane >> 4, j = lane & 15;
    const int b = 2 * (G & 1) + ((j >> 1) & 1);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int row = 8 * (G >> 1) + 4 * half + (j >> 2);
      const int sw = wide_swizzle(row) & (kChunks - 1);
#pragma unroll
      for (int u = 0; u < 4; ++u)
        v[half][u] = row * kRowBytes + 64 * (u ^ (sw >> 2)) + 16 * (b ^ (sw & 3)) + 8 * (j & 1);
    }
  }
  __device__ __forceinline__ int at(int dt, int half) const { return v[half][dt & 3] + 256 * (dt >> 2); }
};

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// LDS-DMA loads: lane i copies 4 or 16 bytes from its global address to LDS
// bytes [lds + size*i, lds + size*(i+1)).  Issued through asm so that the
// compiler's wait-count pass does not treat every later LDS read as depending
// on them (it would otherwise drain all prefetched tiles before the transpose
// reads); the kernels wait for these loads themselves with wait_vmcnt.  m0,
// which holds the LDS address, is saved and restored inside the asm since the
// compiler treats it as a reserved register.
__device__ __forceinline__ void dma_16B(const void* gaddr, uint32_t lds_byte_addr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(gaddr), "s"(lds_byte_addr)
      : "memory");
}

// Same as dma_16B with the address split into a wave-uniform base (SGPRs)
// and a per-lane 32-bit offset.
__device__ __forceinline__ void dma_16B_s(uint32_t lane_off, const void* sbase,
                                          uint32_t lds_byte_addr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(lane_off), "s"(sbase), "s"(lds_byte_addr)
      : "memory");
}

__device__ __forceinline__ void dma_4B(const void* gaddr, uint32_t lds_byte_addr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "global_load_lds_dword %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(gaddr), "s"(lds_byte_addr)
      : "memory");
}

__device__ __forceinline__ f32x4 mfma_k32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// B operand of the 32x32x16 PV product (lane (n, kg): P of rows 8kg..8kg+7
// for head n) from the two 16-head blocks' weights of 16 rows in the 16x16
// score layout (p0: block 0, p1: block 1, each this lane's 4 rows 4g..4g+3):
// one v_permlane16_swap per dword, lanes 16..31 of block 0's value trading
// with lanes 0..15 of block 1's in each half-wave.
__device__ __forceinline__ bf16x8 wide_p_operand(bf16x4 p0, bf16x4 p1) {
  const auto x = __builtin_bit_cast(HIP_vector_base<unsigned, 2>::Native_vec_, p0);
  const auto y = __builtin_bit_cast(HIP_vector_base<unsigned, 2>::Native_vec_, p1);
  const auto s0 = __builtin_amdgcn_permlane16_swap(x[0], y[0], false, false);
  const auto s1 = __builtin_amdgcn_permlane16_swap(x[1], y[1], false, false);
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 r = {(unsigned)s0[0], (unsigned)s1[0], (unsigned)s0[1], (unsigned)s1[1]};
  return __builtin_bit_cast(bf16x8, r);
}

__device__ __forceinline__ f32x4 mfma_k16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                   __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}

// Map the linear workgroup id to a work item so that consecutive work items
// (the partitions and head groups of one token) run on the same XCD: the
// dispatcher hands workgroups to the 8 XCDs round-robin.
__device__ __forceinline__ int xcd_item(int wg, int total) {
  const int per = total >> 3, rem = total & 7;
  const int x = wg & 7, k = wg >> 3;
  return x * per + (x < rem ? x : rem) + k;
}

__device__ __forceinline__ int partitions_of(int L, int splits, int split_rows) {
  if (splits == 1 || L <= split_rows) return 1;
  const int n = (L + split_rows - 1) / split_rows;
  return n < splits ? n : splits;
}

// Stage the row indices [base, base + n) of a partition (n <= kIdxCap) into
// sidx[0, n): wave w of nw issues the 64-entry groups w, w + nw, ...; each lane
// clamps its position to the last row, so no load leaves the partition.
__device__ __forceinline__ void stage_indices(const int32_t* part, int base, int n, int* sidx,
                                              int wave, int nw, int lane) {
  for (int g0 = wave * 64; g0 < n; g0 += nw * 64) {
    const int p = g0 + lane < n ? g0 + lane : n - 1;
    dma_4B(part + base + p, __builtin_amdgcn_readfirstlane(lds_addr(sidx + g0)));
  }
}

// The page transform of token t, in the index builder's order: the window
// slots state_slot*win + r for r < clamp(swa_len, 0, win), then each valid
// entry p of the token's comp_pos row (0 <= p < max_blocks*K), in row order,
// as swa_pages + block_table[t][p / K]*K + p mod K (sglang PR #28392 summary
// page, "key source snippet").  All NT threads of the workgroup call it; it
// writes the list into sidx[0, L), returns L and ends with a barrier.  Each
// group of 8*NT comp_pos entries costs two memory round trips (the entries,
// then their block-table lookups); the valid ones are compacted with per-wave
// ballots and a prefix over the per-wave counts in scount[8 * NT / 64].
template <int NT>
__device__ int stage_paged_list(const AttnArgs& a, int t, int* sidx, int* scount) {
  constexpr int kW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t s0 = (int64_t)((ScalarI32Ptr)a.state_slot)[t] * a.win;
  int sl = ((ScalarI32Ptr)a.swa_len)[t];
  sl = sl < 0 ? 0 : (sl > a.win ? a.win : sl);
  const int ntop = a.comp_pos != nullptr ? a.topk : 0;
  const int32_t* row = a.comp_pos + (int64_t)t * a.topk;
  const int32_t* bt = a.block_table + (int64_t)t * a.max_blocks;
  for (int r = tid; r < sl; r += NT) sidx[r] = (int32_t)(s0 + r);
  int total = sl;
  for (int c0 = 0; c0 < ntop; c0 += 8 * NT) {
    int p[8], blk[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int c = c0 + u * NT + tid;
      const int x = row[c < ntop ? c : ntop - 1];
      p[u] = c < ntop ? x : -1;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const bool ok = (unsigned)p[u] < a.comp_limit;  // a negative p compares as >= 2^31
      const int x = bt[ok ? p[u] / a.k_per_block : 0];
      blk[u] = ok ? x : 0;
    }
    unsigned long long mask[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      mask[u] = __ballot((unsigned)p[u] < a.comp_limit);
      if (lane == 0) scount[u * kW + wave] = __popcll(mask[u]);
    }
    barrier_lds();
    int run = total;  // valid entries before group slot (u, wave), in (u, wave) order
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      int before = run;
#pragma unroll
      for (int w = 0; w < kW; ++w) {
        const int v = scount[u * kW + w];
        before += w < wave ? v : 0;
        run += v;
      }
      if ((unsigned)p[u] < a.comp_limit) {
        const int below = __builtin_amdgcn_mbcnt_hi((unsigned)(mask[u] >> 32),
                                                    __builtin_amdgcn_mbcnt_lo((unsigned)mask[u], 0));
        sidx[before + below] = (int32_t)((int64_t)a.swa_pages + (int64_t)blk[u] * a.k_per_block +
                                         p[u] % a.k_per_block);
      }
    }
    total = run;
    barrier_lds();  // scount is reused by the next group
  }
  barrier_lds();
  return total;
}

// Stage attn_sink[h0 .. h0 + nh) into ssink[0, nh) (nh <= 64) with one LDS-DMA
// load issued by wave 0, so that it completes with the index staging instead
// of adding a dependent memory round trip before it.
__device__ __forceinline__ void stage_sinks(const float* sink, int H, int h0, float* ssink,
                                            int wave, int lane) {
  if (wave == 0) {
    const int h = h0 + lane < H ? h0 + lane : H - 1;
    dma_4B(sink + h, __builtin_amdgcn_readfirstlane(lds_addr(ssink)));
  }
}

// Issue the LDS-DMA loads of kRows consecutive rows of a tile: tile rows
// [r0, r0 + kRows) whose staged indices start at sidx[p0] (positions past the
// partition's n rows repeat its last row, so a ragged tail never reads stale
// LDS), into LDS at dst (kLoads * 1024 bytes).  rbase is the first row's index
// within its tile (it selects the XOR swizzle).  At D = 512 a load is one row:
// the wave reads all its indices with one LDS read and broadcasts them with
// v_readlane, instead of one dependent LDS round trip per load.
template <int kRowBytes, int kLoads, int kSwz = 0>
__device__ __forceinline__ void issue_rows(const uint16_t* kv, const int* sidx, int n, int p0,
                                           int rbase, unsigned char* dst, int lane) {
  auto row_swizzle = [](int r) { return tile_swizzle<kSwz>(r); };
  constexpr int kChunks = kRowBytes / 16;
  constexpr int kRowsPerLoad = 1024 / kRowBytes;
  static_assert(kLoads <= 64, "one lane per row index");
  const unsigned char* base = reinterpret_cast<const unsigned char*>(kv);
  if constexpr (kRowsPerLoad == 1) {
    int p = p0 + (lane < kLoads ? lane : 0);
    const int mine = sidx[p < n ? p : n - 1];
    const uint32_t dst0 = __builtin_amdgcn_readfirstlane(lds_addr(dst));
#pragma unroll
    for (int ld = 0; ld < kLoads; ++ld) {
      const int grow = __builtin_amdgcn_readlane(mine, ld);  // row index, wave-uniform
      const unsigned char* rowp = base + (int64_t)grow * kRowBytes;
      const uint32_t lane_off = (uint32_t)((lane ^ (row_swizzle(rbase + ld) & (kChunks - 1))) << 4);
      dma_16B_s(lane_off, rowp, dst0 + ld * 1024);
    }
  } else {
#pragma unroll
    for (int ld = 0; ld < kLoads; ++ld) {
      const int rr = ld * kRowsPerLoad + lane / kChunks;
      const int p = p0 + rr;
      const int grow = sidx[p < n ? p : n - 1];
      const int lchunk = (lane % kChunks) ^ (row_swizzle(rbase + rr) & (kChunks - 1));
      dma_16B(base + (int64_t)grow * kRowBytes + lchunk * 16,
              __builtin_amdgcn_readfirstlane(lds_addr(dst + ld * 1024)));
    }
  }
}

// Q^T operand of S^T = K Q^T: lane (n16, g) holds q[t, h, 32s + 8g .. +7].
// Lanes of padding heads (h >= H) load a valid row instead; their results are
// never stored, and nothing consumes the values here, so the compiler does not
// wait for these loads before the index staging that follows.
template <int D>
__device__ __forceinline__ void load_q(const uint16_t* q, int64_t row, int g,
                                       bf16x8 (&qreg)[D / 32]) {
  const uint16_t* qp = q + row * D + 8 * g;
#pragma unroll
  for (int s = 0; s < D / 32; ++s) qreg[s] = *reinterpret_cast<const bf16x8*>(qp + 32 * s);
}

// Write zeros for heads [h0, h0 + nh) of token t (empty slice).
template <int D>
__device__ __forceinline__ void zero_heads(uint16_t* out, int H, int t, int h0, int nh, int tid,
                                           int nthreads) {
  if (nh <= 0) return;
  uint4* dst = reinterpret_cast<uint4*>(out + ((int64_t)t * H + h0) * D);
  const int n = nh * D / 8;
  for (int i = tid; i < n; i += nthreads) dst[i] = make_uint4(0, 0, 0, 0);
}

__device__ __forceinline__ void store_bf16x4(uint16_t* dst, f32x4 v, float inv) {
  bf16x4 o;
  o[0] = (__bf16)(v[0] * inv);
  o[1] = (__bf16)(v[1] * inv);
  o[2] = (__bf16)(v[2] * inv);
  o[3] = (__bf16)(v[3] * inv);
  *reinterpret_cast<bf16x4*>(dst) = o;
}

// Maximum / sum over the four 16-lane groups (lanes n16, n16+16, n16+32,
// n16+48) with v_permlane32_swap / v_permlane16_swap: pure VALU, so it does not
// wait behind LDS reads still in flight (ds_bpermute would).  Each swap returns
// this lane's value and its partner's (lane ^ 32, then lane ^ 16).
__device__ __forceinline__ float group_max4(float v) {
  const unsigned u = __builtin_bit_cast(unsigned, v);
  auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  v = fmaxf(__builtin_bit_cast(float, (unsigned)a[0]), __builtin_bit_cast(float, (unsigned)a[1]));
  const unsigned w = __builtin_bit_cast(unsigned, v);
  auto b = __builtin_amdgcn_permlane16_swap(w, w, false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)b[0]), __builtin_bit_cast(float, (unsigned)b[1]));
}

__device__ __forceinline__ float group_sum4(float v) {
  const unsigned u = __builtin_bit_cast(unsigned, v);
  auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  v = __builtin_bit_cast(float, (unsigned)a[0]) + __builtin_bit_cast(float, (unsigned)a[1]);
  const unsigned w = __builtin_bit_cast(unsigned, v);
  auto b = __builtin_amdgcn_permlane16_swap(w, w, false, false);
  return __builtin_bit_cast(float, (unsigned)b[0]) + __builtin_bit_cast(float, (unsigned)b[1]);
}

// Weights of one tile.  x[] are the log2-domain scores of this lane's rows
// (-inf for rows past the end), all of head n16.  The reference maximum m of a
// state is fixed at its first tile (max of that tile and the sink) and never
// moves afterwards, so the accumulator is never rescaled inside the loop: a
// later score may exceed m, giving a weight above 1, which bf16 and fp32
// represent exactly as long as it stays below 2^kRaise.  A tile with a score
// beyond m + kRaise sets the returned flag (wave-uniform); the caller then
// recomputes the whole state with m = mtrue, the running maximum tracked
// here, which no score can exceed.  lpart is this lane's share of the
// denominator: it sums the same bf16-rounded weights the PV product uses.
//
// kGuard: the state may see tiles in which every row is masked before its
// first unmasked one (windows that start inside a shared tile range); such a
// tile with no sink leaves m at -inf, so the state stays "first" and its
// weights are 0 instead of exp2(-inf - -inf).
template <int R, bool kGuard = false>
__device__ __forceinline__ bool softmax_tile(const float (&x)[R], float sink_l2, int g,
                                             bool& first, float& m, float& mtrue, float& lpart,
                                             __bf16 (&p)[R]) {
  float mx = x[0];
#pragma unroll
  for (int j = 1; j < R; ++j) mx = fmaxf(mx, x[j]);
  mx = group_max4(mx);
  mtrue = fmaxf(mtrue, mx);
  if (first) {
    m = fmaxf(sink_l2, mx);
    lpart = (g == 0 && sink_l2 > -INFINITY) ? __builtin_amdgcn_exp2f(sink_l2 - m) : 0.f;
    first = kGuard ? m == -INFINITY : false;
  }
  const bool over = __builtin_amdgcn_ballot_w64(mx > m + kRaise) != 0;
  float psum = 0.f;
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const float e = __builtin_amdgcn_exp2f(x[j] - m);
    p[j] = (__bf16)(kGuard && m == -INFINITY ? 0.f : e);
    psum += (float)p[j];
  }
  lpart += psum;
  return over;
}

// State of the second pass: reference max = the true maximum of the first
// pass (and the sink), so every weight is at most 1.
__device__ __forceinline__ void second_pass_state(float sink_l2, float mtrue, int g, float& m,
                                                  float& lpart) {
  m = fmaxf(sink_l2, mtrue);
  lpart = (g == 0 && sink_l2 > -INFINITY) ? __builtin_amdgcn_exp2f(sink_l2 - m) : 0.f;
}

// OR of a wave-uniform flag over the waves of the workgroup (all waves must
// call it; it ends with a barrier).
__device__ __forceinline__ bool workgroup_any(bool flag, int* sflag, int wave, int nw) {
  sflag[wave] = flag ? 1 : 0;
  barrier_lds();
  int any = 0;
  for (int w = 0; w < nw; ++w) any |= sflag[w];
  barrier_lds();  // the flags may be rewritten by a later call
  return any != 0;
}

}  // namespace
}  // namespace spd
