// indices.hip -- decode index builder (the page's write_v4_paged_decode_indices)
// and a debug validator of the attention call's index preconditions, gfx950.
//
// Builder (sglang PR #28392 summary page, "key source snippet": pool slots
// [0, swa_pages) hold window entries at state_slot*win + ring, slots from
// swa_pages on hold compressed entries at block_id*K_PER_BLOCK + slot_in_block;
// the builder emits ragged-packed indices with no sentinels and a padded
// token gets kv_indptr[t+1] == kv_indptr[t]).
//
// Three graph-safe launches, no workspace:
//   1. count:   one wave per token writes its entry count into kv_indptr[t+1];
//   2. scan:    one 1024-thread workgroup turns kv_indptr[1..N] into inclusive
//               prefix sums in place and sets kv_indptr[0] = 0;
//   3. scatter: one wave per token writes the window slots, then the valid
//               compressed slots compacted in comp_pos order (ballot + mbcnt).
#include "spd_internal.h"

namespace spd {
namespace {

__device__ __forceinline__ int clamp_swa(int v, int win) { return v < 0 ? 0 : (v > win ? win : v); }

__device__ __forceinline__ bool comp_valid(int p, const BuildArgs& a) {
  return p >= 0 && p / a.k_per_block < a.max_blocks;
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

__global__ void __launch_bounds__(256) build_count_kernel(BuildArgs a) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= a.N) return;
  int n = 0;
  if (a.comp_pos != nullptr) {
    const int32_t* row = a.comp_pos + (int64_t)t * a.topk;
    for (int c = lane; c < a.topk; c += 64) n += comp_valid(row[c], a) ? 1 : 0;
    n = wave_sum(n);
  }
  if (lane == 0) a.kv_indptr[t + 1] = clamp_swa(a.swa_len[t], a.win) + n;
}

__global__ void __launch_bounds__(1024) build_scan_kernel(int32_t* indptr, int N) {
  __shared__ int wsum[16];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int carry = 0;
  for (int base = 0; base < N; base += 1024) {
    const int i = base + threadIdx.x;
    int x = i < N ? indptr[i + 1] : 0;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    if (wave == 0) {
      int s = lane < 16 ? wsum[lane] : 0;
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) {
        const int y = __shfl_up(s, off);
        if (lane >= off) s += y;
      }
      if (lane < 16) wsum[lane] = s;
    }
    __syncthreads();
    if (i < N) indptr[i + 1] = carry + (wave > 0 ? wsum[wave - 1] : 0) + x;
    carry += wsum[15];
    __syncthreads();
  }
  if (threadIdx.x == 0) indptr[0] = 0;
}

__global__ void __launch_bounds__(256) build_scatter_kernel(BuildArgs a) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= a.N) return;
  const int base = a.kv_indptr[t];
  const int sl = clamp_swa(a.swa_len[t], a.win);
  const int64_t s0 = (int64_t)a.state_slot[t] * a.win;
  for (int r = lane; r < sl; r += 64) a.kv_indices[base + r] = (int32_t)(s0 + r);
  if (a.comp_pos == nullptr) return;
  const int32_t* row = a.comp_pos + (int64_t)t * a.topk;
  const int32_t* bt = a.block_table + (int64_t)t * a.max_blocks;
  int out = base + sl;
  for (int c0 = 0; c0 < a.topk; c0 += 64) {
    const int c = c0 + lane;
    bool valid = false;
    int64_t slot = 0;
    if (c < a.topk) {
      const int p = row[c];
      if (comp_valid(p, a)) {
        valid = true;
        slot = (int64_t)a.swa_pages + (int64_t)bt[p / a.k_per_block] * a.k_per_block +
               p % a.k_per_block;
      }
    }
    const unsigned long long mask = __ballot(valid);
    const int below = __builtin_amdgcn_mbcnt_hi((unsigned)(mask >> 32),
                                                __builtin_amdgcn_mbcnt_lo((unsigned)mask, 0));
    if (valid) a.kv_indices[out + below] = (int32_t)slot;
    out += __popcll(mask);
  }
}

__global__ void __launch_bounds__(256) validate_kernel(const int32_t* idx, int64_t n_idx,
                                                       const int32_t* indptr, int N,
                                                       int64_t num_rows,
                                                       unsigned long long* first_bad) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t t = tid; t <= N; t += stride) {
    bool bad = (t == 0) ? indptr[0] != 0 : indptr[t] < indptr[t - 1];
    if (t == N && (int64_t)indptr[N] > n_idx) bad = true;
    if (bad) atomicMin(first_bad, (unsigned long long)t);
  }
  int64_t total = indptr[N];
  if (total > n_idx) total = n_idx;
  for (int64_t j = tid; j < total; j += stride) {
    const int32_t v = idx[j];
    if (v < 0 || (int64_t)v >= num_rows) atomicMin(first_bad, (unsigned long long)(N + 1 + j));
  }
}

}  // namespace

hipError_t launch_build_indices(const BuildArgs& a, hipStream_t stream) {
  const unsigned blocks = (unsigned)((a.N + 3) / 4);
  if (a.N > 0) {
    hipLaunchKernelGGL(build_count_kernel, dim3(blocks), dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(build_scan_kernel, dim3(1), dim3(1024), 0, stream, a.kv_indptr, a.N);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.N == 0) return e;
  hipLaunchKernelGGL(build_scatter_kernel, dim3(blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_validate_indices(const int32_t* kv_indices, int64_t num_indices,
                                   const int32_t* kv_indptr, int32_t N, int64_t num_rows,
                                   unsigned long long* first_bad_dev, hipStream_t stream) {
  hipLaunchKernelGGL(validate_kernel, dim3(256), dim3(256), 0, stream, kv_indices, num_indices,
                     kv_indptr, N, num_rows, first_bad_dev);
  return hipGetLastError();
}

}  // namespace spd
