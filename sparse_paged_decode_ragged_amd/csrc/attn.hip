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
//   * one workgroup = (token, group of 16*W heads, partition of the slice);
//     wave w owns heads [16w, 16w+16) of the group, so every gathered row is
//     loaded once per workgroup and shared by all of its heads;
//   * rows are gathered 32 at a time straight into LDS with
//     global_load_lds_dwordx4 (one 1 KiB row per wave instruction at D=512),
//     three stages in flight, XOR-swizzled by row so that both LDS read
//     patterns below are bank-conflict free;
//   * S^T = K Q^T on MFMA 16x16x32 bf16: A = K rows read from LDS, B = Q^T
//     held in VGPRs for the whole slice;
//   * the S^T accumulator layout (lane = head, 4 rows per lane) is exactly the
//     B operand layout of O^T += V^T P^T, so P never leaves registers; V^T is
//     read from the same LDS rows with ds_read_b64_tr_b16 (the 16-lane
//     transpose read of gfx950);
//   * the online softmax statistics live per lane (lane = head), so the
//     rescale of the accumulator needs no cross-lane traffic; only the tile
//     maximum is reduced across the four 16-lane groups;
//   * long slices are split into partitions (split-L); partials (m, l, O) go
//     to a workspace and a combine kernel merges them, counting the sink once.
#include <math.h>

#include "spd_internal.h"

namespace spd {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(4))) int32_t* ScalarI32Ptr;
typedef __attribute__((address_space(3))) bf16x4 LdsBf16x4;

constexpr int kStages = 3;
constexpr float kLog2e = 1.4426950408889634f;

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt[3:0] in bits
// 3:0, vmcnt[5:4] in bits 15:14; expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt out of range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Workgroup barrier without a memory fence: the LDS data it publishes was
// written by this workgroup's own LDS-DMA loads, which each wave has already
// waited for with wait_vmcnt.  The empty asm keeps the compiler from moving
// memory accesses across it.
__device__ __forceinline__ void barrier_no_fence() {
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// XOR swizzle of the 16-byte chunks of LDS row r.  Rows 0..15 map to 16
// distinct chunk positions (QK reads: 16 rows, same logical chunk) and any 4
// consecutive rows map to distinct chunk pairs (transpose reads: 4 rows x 32 B).
__device__ __forceinline__ int row_swizzle(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }

// One 64-lane LDS-DMA load: lane i copies 16 bytes from its global address to
// LDS bytes [lds + 16 i, lds + 16 i + 16).  Issued through asm so that the
// compiler's wait-count pass does not treat every later LDS read as depending
// on it (it would otherwise drain all prefetched tiles before the transpose
// reads); the kernel waits for these loads itself with wait_vmcnt.
// m0 (which the instruction takes the LDS address from) is saved and restored
// inside the asm, since the compiler treats it as a reserved register.
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

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
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

template <int D>
__device__ __forceinline__ void store_bf16_row4(uint16_t* dst, f32x4 v, float inv) {
  bf16x4 o;
  o[0] = (__bf16)(v[0] * inv);
  o[1] = (__bf16)(v[1] * inv);
  o[2] = (__bf16)(v[2] * inv);
  o[3] = (__bf16)(v[3] * inv);
  *reinterpret_cast<bf16x4*>(dst) = o;
}

template <int D, int W>
__global__ void __launch_bounds__(64 * W) attn_main_kernel(AttnArgs a) {
  constexpr int kRowBytes = 2 * D;
  constexpr int kChunks = D / 8;  // 16-byte chunks per row
  constexpr int kStageBytes = kTileRows * kRowBytes;
  constexpr int kKSteps = D / 32;
  constexpr int kDTiles = D / 16;
  constexpr int kRowsPerLoad = 1024 / kRowBytes;  // rows filled by one 64-lane x 16 B load
  constexpr int kLoadsPerTile = kTileRows / kRowsPerLoad;
  constexpr int kLoadsPerWave = kLoadsPerTile / W;
  constexpr int kHeads = 16 * W;
  static_assert(D % 64 == 0 && D <= 512, "unsupported D");
  static_assert(kLoadsPerTile % W == 0, "loads must divide among waves");

  __shared__ __attribute__((aligned(1024))) unsigned char smem[kStages * kStageBytes];

  const int item = xcd_item(blockIdx.x, gridDim.x);
  const int c = item % a.splits;
  const int th = item / a.splits;
  const int hg = th % a.head_groups;
  const int t = th / a.head_groups;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n16 = lane & 15;
  const int g = lane >> 4;

  const ScalarI32Ptr indptr = (ScalarI32Ptr)a.kv_indptr;
  const int row0 = indptr[t];
  const int L = indptr[t + 1] - row0;
  const int nparts = partitions_of(L, a.splits, a.split_rows);
  if (c >= nparts) return;  // nothing for this partition

  const int h0 = hg * kHeads + wave * 16;  // first head of this wave
  const int h = h0 + n16;                  // this lane's head
  const bool hvalid = h < a.H;

  if (L <= 0) {
    // Empty slice: the output is exactly zero.
    const int nh = a.H - h0 < 16 ? a.H - h0 : 16;
    if (nh > 0) {
      uint4* dst = reinterpret_cast<uint4*>(a.out + ((int64_t)t * a.H + h0) * D);
      const int n16b = nh * D / 8;
      for (int i = lane; i < n16b; i += 64) dst[i] = make_uint4(0, 0, 0, 0);
    }
    return;
  }

  const int cb = c * a.split_rows;
  const int nrows = (c == nparts - 1) ? L - cb : a.split_rows;
  const ScalarI32Ptr cidx = (ScalarI32Ptr)(a.kv_indices + row0 + cb);
  const int ntiles = (nrows + kTileRows - 1) / kTileRows;

  // Issue the LDS-DMA loads of tile `tile` (rows clamped to the last row of the
  // partition, so a ragged tail re-reads a valid row instead of stale LDS).
  auto issue_tile = [&](int tile) {
    unsigned char* st = smem + (tile % kStages) * kStageBytes;
    const int rbase = tile * kTileRows;
#pragma unroll
    for (int j = 0; j < kLoadsPerWave; ++j) {
      const int ld = wave * kLoadsPerWave + j;
      const int rfirst = ld * kRowsPerLoad;
      int grow;
      int rr;
      if constexpr (kRowsPerLoad == 1) {
        const int p = rbase + rfirst;
        grow = cidx[p < nrows ? p : nrows - 1];
        rr = rfirst;
      } else {
        const int sub = lane / kChunks;
        rr = rfirst + sub;
        grow = 0;
#pragma unroll
        for (int u = 0; u < kRowsPerLoad; ++u) {
          const int p = rbase + rfirst + u;
          const int v = cidx[p < nrows ? p : nrows - 1];
          if (sub == u) grow = v;
        }
      }
      const int pchunk = lane % kChunks;
      const int lchunk = pchunk ^ (row_swizzle(rr) & (kChunks - 1));
      const unsigned char* src =
          reinterpret_cast<const unsigned char*>(a.kv) + (int64_t)grow * kRowBytes + lchunk * 16;
      dma_16B(src, __builtin_amdgcn_readfirstlane(lds_addr(st + ld * 1024)));
    }
  };

  // Prologue: the first two tiles go out before the query loads, so that the
  // compiler's waits for the queries (it cannot see the asm DMA loads) cost no
  // more than waiting for tile 0, which the first step needs anyway.
  issue_tile(0);
  if (ntiles > 1) issue_tile(1);

  // Q^T operand: lane (n16, g) holds q[t, h, 32s + 8g .. +7] for k-step s.
  bf16x8 qreg[kKSteps];
  {
    const uint16_t* qp = a.q + ((int64_t)t * a.H + (hvalid ? h : 0)) * D + 8 * g;
#pragma unroll
    for (int s = 0; s < kKSteps; ++s) {
      bf16x8 v = *reinterpret_cast<const bf16x8*>(qp + 32 * s);
      if (!hvalid) v = bf16x8{};
      qreg[s] = v;
    }
  }

  // Online-softmax state.  The sink enters once, in partition 0, as a virtual
  // key whose log2 logit is sink*log2(e): m starts there with weight 1.
  // m is the reference maximum the weights are taken against; it is only
  // raised when a score exceeds it by more than kLazy (log2 units), which
  // bounds every weight by 2^kLazy and leaves the result unchanged.
  constexpr float kLazy = 8.0f;
  float m = -INFINITY;
  float lpart = 0.f;  // this lane's share of the denominator
  if (c == 0 && hvalid) {
    const float sk = a.sink[h] * kLog2e;
    m = sk;
    if (g == 0 && sk > -INFINITY) lpart = 1.f;
  }
  f32x4 acc[kDTiles];
#pragma unroll
  for (int i = 0; i < kDTiles; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int sw_qk = row_swizzle(n16) & (kChunks - 1);  // rows n16 and 16+n16
  const int rtr = 4 * g + (n16 >> 2);                    // transpose-read row (and +16)
  const int sw_tr = row_swizzle(rtr) & (kChunks - 1);

  for (int i = 0; i < ntiles; ++i) {
    if (i + 1 < ntiles)
      wait_vmcnt<kLoadsPerWave>();
    else
      wait_vmcnt<0>();
    barrier_no_fence();
    if (i + 2 < ntiles) issue_tile(i + 2);

    const unsigned char* st = smem + (i % kStages) * kStageBytes;
    const int nvalid = nrows - i * kTileRows;  // rows of this tile that exist (>= 1)

    // S^T[32 rows x 16 heads] = K Q^T
    f32x4 sa = {0.f, 0.f, 0.f, 0.f};
    f32x4 sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kKSteps; ++s) {
      const int pc = ((4 * s + g) ^ sw_qk) << 4;
      const bf16x8 ka = *reinterpret_cast<const bf16x8*>(st + n16 * kRowBytes + pc);
      const bf16x8 kb = *reinterpret_cast<const bf16x8*>(st + (16 + n16) * kRowBytes + pc);
      sa = mfma_bf16(ka, qreg[s], sa);
      sb = mfma_bf16(kb, qreg[s], sb);
    }

    // Online softmax, log2 domain.  Lane holds rows 4g+i (sa) and 16+4g+i (sb)
    // of head n16.
    float x[8];
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      x[i4] = (4 * g + i4 < nvalid) ? sa[i4] * a.qk_scale : -INFINITY;
      x[4 + i4] = (16 + 4 * g + i4 < nvalid) ? sb[i4] * a.qk_scale : -INFINITY;
    }
    float mx = x[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) mx = fmaxf(mx, x[j]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const bool raise = mx > m + kLazy;
    if (__builtin_amdgcn_ballot_w64(raise) != 0) {  // some head needs a new reference
      const float mnew = raise ? mx : m;
      const float alpha = __builtin_amdgcn_exp2f(m - mnew);  // 0 when m was -inf
      lpart *= alpha;
#pragma unroll
      for (int dt = 0; dt < kDTiles; ++dt) acc[dt] *= alpha;
      m = mnew;
    }
    bf16x8 pt;
    float psum = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const __bf16 pb = (__bf16)__builtin_amdgcn_exp2f(x[j] - m);
      pt[j] = pb;
      psum += (float)pb;  // the denominator sums the same rounded weights as PV
    }
    lpart += psum;

    // O^T[d x 16 heads] += V^T P^T; V^T via 16-lane transpose reads.
#pragma unroll
    for (int dt = 0; dt < kDTiles; ++dt) {
      const int d = 16 * dt + 4 * (n16 & 3);
      const int off = (((d >> 3) ^ sw_tr) << 4) + (d & 7) * 2;
      const bf16x4 vlo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (LdsBf16x4*)(st + rtr * kRowBytes + off));
      const bf16x4 vhi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (LdsBf16x4*)(st + (16 + rtr) * kRowBytes + off));
      const bf16x8 vt = __builtin_shufflevector(vlo, vhi, 0, 1, 2, 3, 4, 5, 6, 7);
      acc[dt] = mfma_bf16(vt, pt, acc[dt]);
    }
  }

  float l = lpart + __shfl_xor(lpart, 16);
  l += __shfl_xor(l, 32);

  if (nparts == 1) {
    if (hvalid) {
      const float inv = 1.0f / l;
      uint16_t* op = a.out + ((int64_t)t * a.H + h) * D + 4 * g;
#pragma unroll
      for (int dt = 0; dt < kDTiles; ++dt) store_bf16_row4<D>(op + 16 * dt, acc[dt], inv);
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

// Merge the partitions of each token with more than one:
//   M = max_c m_c,  l = sum_c l_c 2^(m_c - M),  O = sum_c O_c 2^(m_c - M),
//   out = O / l.  Partition 0 already carries the sink.
template <int D, int W>
__global__ void __launch_bounds__(64 * W) attn_combine_kernel(AttnArgs a) {
  constexpr int kDTiles = D / 16;
  constexpr int kHeads = 16 * W;
  const int th = blockIdx.x;
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
  f32x4 acc[kDTiles];
#pragma unroll
  for (int i = 0; i < kDTiles; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int c = 0; c < nparts; ++c) {
    const float* base = base0 + c * stride;
    const float w = __builtin_amdgcn_exp2f(base[kHeads * D + hi] - M);
    lsum += w * base[kHeads * D + kHeads + hi];
    const f32x4* po = reinterpret_cast<const f32x4*>(base) + wave * kDTiles * 64 + lane;
#pragma unroll
    for (int dt = 0; dt < kDTiles; ++dt) acc[dt] += w * po[dt * 64];
  }
  const float inv = 1.0f / lsum;
  uint16_t* op = a.out + ((int64_t)t * a.H + h) * D + 4 * g;
#pragma unroll
  for (int dt = 0; dt < kDTiles; ++dt) store_bf16_row4<D>(op + 16 * dt, acc[dt], inv);
}

template <int D, int W>
hipError_t launch_dw(const AttnArgs& a, hipStream_t stream) {
  const long long items = (long long)a.N * a.head_groups * a.splits;
  hipLaunchKernelGGL((attn_main_kernel<D, W>), dim3((unsigned)items), dim3(64 * W), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits == 1) return e;
  hipLaunchKernelGGL((attn_combine_kernel<D, W>), dim3((unsigned)(a.N * a.head_groups)),
                     dim3(64 * W), 0, stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const AttnArgs& a, int waves, hipStream_t stream) {
  switch (waves) {
    case 1: return launch_dw<D, 1>(a, stream);
    case 2: return launch_dw<D, 2>(a, stream);
    case 4: return launch_dw<D, 4>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool attn_supported(int32_t H, int32_t D) {
  return (D == 64 || D == 128 || D == 256 || D == 512) && H >= 1 && H <= 1024;
}

bool make_attn_plan(int32_t N, int32_t H, int32_t D, int32_t max_len, int32_t split_rows,
                    AttnPlan* p) {
  if (!attn_supported(H, D) || N < 0 || max_len < 0 || split_rows < 0) return false;
  p->waves = H <= 16 ? 1 : (H <= 32 ? 2 : 4);
  p->heads_per_group = 16 * p->waves;
  p->head_groups = (H + p->heads_per_group - 1) / p->heads_per_group;
  long long splits = 1, rows = 0;
  if (split_rows > 0) {
    rows = ((long long)split_rows + kTileRows - 1) / kTileRows * kTileRows;
    splits = max_len > rows ? (max_len + rows - 1) / rows : 1;
  } else if (max_len > 0 && N > 0) {
    // Aim at about one workgroup per compute unit (256 on MI355X) when the
    // batch alone does not provide that many; keep partitions >= 128 rows.
    const long long base = (long long)N * p->head_groups;
    const long long target = 256;
    if (base < target) {
      long long want = (target + base - 1) / base;
      const long long cap = (max_len + 127) / 128;
      splits = want < cap ? want : cap;
      if (splits > 64) splits = 64;
      if (splits > 1) {
        rows = (max_len + splits - 1) / splits;
        rows = (rows + kTileRows - 1) / kTileRows * kTileRows;
        splits = (max_len + rows - 1) / rows;
      }
    }
  }
  if (splits <= 1) {
    splits = 1;
    rows = 1 << 30;
  }
  if (splits > 4096) return false;
  if ((long long)N * p->head_groups * splits > 0x7fffffffLL) return false;
  p->splits = (int)splits;
  p->split_rows = (int)rows;
  p->workspace_bytes = splits > 1 ? (size_t)N * p->head_groups * splits * p->heads_per_group *
                                        (size_t)(D + 2) * sizeof(float)
                                  : 0;
  return true;
}

hipError_t launch_attention(const AttnArgs& a, int D, const AttnPlan& plan, hipStream_t stream) {
  switch (D) {
    case 64: return launch_d<64>(a, plan.waves, stream);
    case 128: return launch_d<128>(a, plan.waves, stream);
    case 256: return launch_d<256>(a, plan.waves, stream);
    case 512: return launch_d<512>(a, plan.waves, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace spd
