// indices.hip -- decode index builder (the page's write_v4_paged_decode_indices)
// and a debug validator of the attention call's index preconditions, gfx950.
//
// Builder (sglang PR #28392 summary page, "key source snippet": pool slots
// [0, swa_pages) hold window entries at state_slot*win + ring, slots from
// swa_pages on hold compressed entries at block_id*K_PER_BLOCK + slot_in_block;
// the builder emits ragged-packed indices with no sentinels and a padded
// token gets kv_indptr[t+1] == kv_indptr[t]).
//
// Graph-safe launches, no workspace; every kernel issues all its independent
// loads before it consumes any of them, so each costs one or two memory round
// trips however long comp_pos is (a kernel boundary costs a few microseconds,
// so small batches get one launch):
//   batches of one workgroup (N <= 16, N * topk <= 2^16): one launch that
//     counts every token, writes kv_indptr and scatters them;
//   N <= 1024: 1. count (one wave per token, counts stored inverted in
//     kv_indptr), 2. look-back scatter: each token's wave sums the counts
//     below it down to the first entry an earlier wave has already made final,
//     writes its own final entry and scatters its token -- no wave waits;
//   otherwise: 1a. count (one wave per token), 1b. scan (one workgroup, in
//     place), 2. scatter.
//   A scatter writes the window slots, then the valid compressed slots
//   compacted in comp_pos order (ballot + mbcnt).
#include "spd_internal.h"

namespace spd {
namespace {

constexpr int kBatch = 8;           // comp_pos entries per lane in flight (512 per wave)
constexpr int kSmallN = 1024;       // largest batch of the look-back builder
constexpr int kFusedEntries = 1 << 16;  // largest N * topk built by the one-launch kernel
// Largest batch built by the one-launch kernel: one workgroup.  Beyond it each
// workgroup recounts every earlier token and the launch saved no longer pays
// (64 tokens x 512 entries: 10.1 us in one launch, 6.9 us as count and
// look-back scatter).
constexpr int kFusedMaxN = 16;

__device__ __forceinline__ int clamp_swa(int v, int win) { return v < 0 ? 0 : (v > win ? win : v); }

__device__ __forceinline__ bool comp_valid(int p, const BuildArgs& a) {
  // p >= 0 and p / K < max_blocks, i.e. 0 <= p < max_blocks * K (no division;
  // a negative p compares as an unsigned value >= 2^31 >= comp_limit)
  return (unsigned)p < a.comp_limit;
}

// A per-token value read by every lane of the wave with a vector load, so that
// it travels in the same memory round trip as the vector loads issued with it
// (a scalar load would be waited on before the vector loads are issued).
__device__ __forceinline__ int wave_load(const int32_t* p) {
  return __builtin_nontemporal_load(p);
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// Number of valid comp_pos entries of the tokens tok[0..T) (entries >= N are
// skipped), each summed over the wave.  All T tokens' loads of a batch go out
// before any is consumed; with 16-byte aligned rows a lane reads 4 entries per
// load (the per-CU load path is limited by requests more than by bytes).
template <int T>
__device__ __forceinline__ void count_compressed(const BuildArgs& a, const int (&tok)[T], int lane,
                                                 int (&n)[T]) {
#pragma unroll
  for (int i = 0; i < T; ++i) n[i] = 0;
  if (a.comp_pos == nullptr) return;
  if (a.comp_vec4) {
    const int nq = a.topk >> 2;  // int4 per row
    for (int q0 = 0; q0 < nq; q0 += 64 * (kBatch / 4)) {
      int4 v[T][kBatch / 4];
#pragma unroll
      for (int i = 0; i < T; ++i) {
        const int4* row = reinterpret_cast<const int4*>(
            a.comp_pos + (int64_t)(tok[i] < a.N ? tok[i] : a.N - 1) * a.topk);
#pragma unroll
        for (int u = 0; u < kBatch / 4; ++u) {
          const int q = q0 + 64 * u + lane;
          const int4 x = row[q < nq ? q : nq - 1];
          v[i][u] = q < nq ? x : make_int4(-1, -1, -1, -1);
        }
      }
#pragma unroll
      for (int i = 0; i < T; ++i)
#pragma unroll
        for (int u = 0; u < kBatch / 4; ++u)
          n[i] += (comp_valid(v[i][u].x, a) ? 1 : 0) + (comp_valid(v[i][u].y, a) ? 1 : 0) +
                  (comp_valid(v[i][u].z, a) ? 1 : 0) + (comp_valid(v[i][u].w, a) ? 1 : 0);
    }
  } else {
    for (int c0 = 0; c0 < a.topk; c0 += 64 * kBatch) {
      int v[T][kBatch];
#pragma unroll
      for (int i = 0; i < T; ++i) {
        // tokens past the batch read token N-1's row and are not counted
        const int32_t* row = a.comp_pos + (int64_t)(tok[i] < a.N ? tok[i] : a.N - 1) * a.topk;
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int c = c0 + 64 * u + lane;
          const int x = row[c < a.topk ? c : a.topk - 1];  // clamped: no branch around the load
          v[i][u] = c < a.topk ? x : -1;
        }
      }
#pragma unroll
      for (int i = 0; i < T; ++i)
#pragma unroll
        for (int u = 0; u < kBatch; ++u) n[i] += comp_valid(v[i][u], a) ? 1 : 0;
    }
  }
#pragma unroll
  for (int i = 0; i < T; ++i) n[i] = tok[i] < a.N ? wave_sum(n[i]) : 0;
}

// Inclusive scan of v over the 1024 threads of a workgroup (16 waves); *total
// receives the sum over all threads.
__device__ __forceinline__ int block_scan_1024(int v, int* wsum, int lane, int wave, int* total) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(v, off);
    if (lane >= off) v += y;
  }
  if (lane == 63) wsum[wave] = v;
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
  const int r = v + (wave > 0 ? wsum[wave - 1] : 0);
  *total = wsum[15];
  __syncthreads();  // wsum may be rewritten by the next call
  return r;
}

// Counts and prefix sums in one workgroup (used for N == 0, where it writes
// kv_indptr[0]; correct for any N <= kSmallN).  Wave
// w counts the tokens w + 16 i, four at a time; the counts meet in LDS and one
// block scan produces kv_indptr[0..N].
__global__ void __launch_bounds__(1024) build_count_scan_kernel(BuildArgs a) {
  __shared__ int cnt[kSmallN];
  __shared__ int wsum[16];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  for (int t0 = wave; t0 < a.N; t0 += 64) {
    int tok[4], sl[4], n[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      tok[i] = t0 + 16 * i;
      sl[i] = wave_load(a.swa_len + (tok[i] < a.N ? tok[i] : a.N - 1));
    }
    count_compressed<4>(a, tok, lane, n);
    if (lane == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (tok[i] < a.N) cnt[tok[i]] = clamp_swa(sl[i], a.win) + n[i];
    }
  }
  __syncthreads();
  const int i = threadIdx.x;
  int total;
  const int incl = block_scan_1024(i < a.N ? cnt[i] : 0, wsum, lane, wave, &total);
  if (i < a.N) a.kv_indptr[i + 1] = incl;
  if (i == 0) a.kv_indptr[0] = 0;
}

// Large batches, step 1a: one wave per token.  With kFlagged the count is
// stored inverted (~count < 0: "a count, not yet a prefix sum") for the
// look-back scatter, and kv_indptr[0] = 0 is written here.
template <bool kFlagged>
__global__ void __launch_bounds__(256) build_count_kernel(BuildArgs a) {
  const int t = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= a.N) return;
  const int sl = wave_load(a.swa_len + t);
  const int tok[1] = {t};
  int n[1];
  count_compressed<1>(a, tok, lane, n);
  if (lane == 0) {
    const int c = clamp_swa(sl, a.win) + n[0];
    a.kv_indptr[t + 1] = kFlagged ? ~c : c;
    if (kFlagged && t == 0) a.kv_indptr[0] = 0;
  }
}

// Large batches, step 1b: kv_indptr[1..N] (counts) -> inclusive prefix sums,
// kv_indptr[0] = 0.  Reads kScanBatch chunks of 1024 counts before scanning.
__global__ void __launch_bounds__(1024) build_scan_kernel(int32_t* indptr, int N) {
  constexpr int kScanBatch = 8;
  __shared__ int wsum[16];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int carry = 0;
  for (int base = 0; base < N; base += 1024 * kScanBatch) {
    int x[kScanBatch];
#pragma unroll
    for (int u = 0; u < kScanBatch; ++u) {
      const int i = base + 1024 * u + threadIdx.x;
      x[u] = i < N ? indptr[i + 1] : 0;
    }
#pragma unroll
    for (int u = 0; u < kScanBatch; ++u) {
      if (base + 1024 * u >= N) break;  // uniform over the workgroup
      const int i = base + 1024 * u + threadIdx.x;
      int total;
      const int incl = block_scan_1024(x[u], wsum, lane, wave, &total);
      if (i < N) indptr[i + 1] = carry + incl;
      carry += total;
    }
  }
  if (threadIdx.x == 0) indptr[0] = 0;
}

// Window slots, then the valid compressed slots compacted in comp_pos order,
// of token t by one wave, from out position base.  A batch of comp_pos
// entries and then their block-table lookups go out together; the window
// stores overlap the lookups.
__device__ __forceinline__ void scatter_token(const BuildArgs& a, int t, int base, int sl,
                                              int64_t s0, int lane) {
  const int ntop = a.comp_pos != nullptr ? a.topk : 0;
  const int32_t* row = a.comp_pos + (int64_t)t * a.topk;
  const int32_t* bt = a.block_table + (int64_t)t * a.max_blocks;
  bool window_done = false;
  int out = base + sl;
  for (int c0 = 0; c0 < ntop || !window_done; c0 += 64 * kBatch) {
    int p[kBatch], blk[kBatch];
    if (c0 < ntop) {
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int c = c0 + 64 * u + lane;
        const int x = row[c < ntop ? c : ntop - 1];
        p[u] = c < ntop ? x : -1;
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const bool ok = comp_valid(p[u], a);
        const int x = bt[ok ? p[u] / a.k_per_block : 0];
        blk[u] = ok ? x : 0;
      }
    }
    if (!window_done) {
      for (int r = lane; r < sl; r += 64) a.kv_indices[base + r] = (int32_t)(s0 + r);
      window_done = true;
    }
    if (c0 >= ntop) break;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const bool valid = comp_valid(p[u], a);
      const unsigned long long mask = __ballot(valid);
      const int below = __builtin_amdgcn_mbcnt_hi((unsigned)(mask >> 32),
                                                  __builtin_amdgcn_mbcnt_lo((unsigned)mask, 0));
      if (valid)
        a.kv_indices[out + below] =
            (int32_t)((int64_t)a.swa_pages + (int64_t)blk[u] * a.k_per_block + p[u] % a.k_per_block);
      out += __popcll(mask);
    }
  }
}

// Step 2 (large batches): one wave per token; kv_indptr[t], swa_len[t] and
// state_slot[t] arrive in one vector load (lanes 0, 1, 2).
__global__ void __launch_bounds__(256) build_scatter_kernel(BuildArgs a) {
  const int t = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= a.N) return;
  const int32_t* src = lane == 0 ? a.kv_indptr + t : (lane == 1 ? a.swa_len + t : a.state_slot + t);
  const int scal = *src;
  const int base = __builtin_amdgcn_readlane(scal, 0);
  const int sl = clamp_swa(__builtin_amdgcn_readlane(scal, 1), a.win);
  const int64_t s0 = (int64_t)__builtin_amdgcn_readlane(scal, 2) * a.win;
  scatter_token(a, t, base, sl, s0, lane);
}

// Adds n to cnt[tk] for every lane; when the whole wave's entries belong to
// one token (the common case: rows of >= 64 loads) the wave sums first, so one
// LDS atomic replaces 64 colliding ones.
__device__ __forceinline__ void add_counts(int* cnt, int tk, int n) {
  const int lo = __builtin_amdgcn_readfirstlane(tk);
  const int hi = __builtin_amdgcn_readlane(tk, 63);
  if (lo == hi) {
    // n is 0..4: its wave sum from three ballots, with no cross-lane shuffles
    const int sum = __popcll(__ballot(n & 1)) + 2 * __popcll(__ballot(n & 2)) +
                    4 * __popcll(__ballot(n & 4));
    if ((threadIdx.x & 63) == 0 && sum > 0) atomicAdd(&cnt[lo], sum);
  } else if (n > 0) {
    atomicAdd(&cnt[tk], n);
  }
}

// Adds to cnt[t] (LDS) the number of valid comp_pos entries of every token
// t < last.  The rows of tokens [0, last) are one contiguous array; the
// workgroup's threads stride through it kFlat loads at a time (4 entries per
// load with 16-byte aligned rows).
__device__ __forceinline__ void count_flat(const BuildArgs& a, int last, int* cnt, int tid,
                                           int nthreads) {
  constexpr int kFlat = 16;
  if (a.comp_pos == nullptr || last <= 0) return;
  const int per = a.comp_vec4 ? a.topk >> 2 : a.topk;  // loads per token row
  const int total = last * per;
  for (int f0 = 0; f0 < total; f0 += nthreads * kFlat) {
    int n[kFlat];
    if (a.comp_vec4) {
      const int4* base = reinterpret_cast<const int4*>(a.comp_pos);
      int4 v[kFlat];
#pragma unroll
      for (int u = 0; u < kFlat; ++u) {
        const int f = f0 + u * nthreads + tid;
        v[u] = base[f < total ? f : total - 1];
      }
#pragma unroll
      for (int u = 0; u < kFlat; ++u)
        n[u] = (comp_valid(v[u].x, a) ? 1 : 0) + (comp_valid(v[u].y, a) ? 1 : 0) +
               (comp_valid(v[u].z, a) ? 1 : 0) + (comp_valid(v[u].w, a) ? 1 : 0);
    } else {
      int v[kFlat];
#pragma unroll
      for (int u = 0; u < kFlat; ++u) {
        const int f = f0 + u * nthreads + tid;
        v[u] = a.comp_pos[f < total ? f : total - 1];
      }
#pragma unroll
      for (int u = 0; u < kFlat; ++u) n[u] = comp_valid(v[u], a) ? 1 : 0;
    }
#pragma unroll
    for (int u = 0; u < kFlat; ++u) {
      const int f = f0 + u * nthreads + tid;
      if (f0 + u * nthreads >= total) break;  // uniform over the workgroup
      add_counts(cnt, (f < total ? f : total - 1) / per, f < total ? n[u] : 0);
    }
  }
}

// Batches of one workgroup (N <= kFusedMaxN, N * topk <= kFusedEntries; the
// kernel itself is correct for any N <= kSmallN): the whole builder in one
// launch.  Workgroup b (16 waves) owns tokens 16b .. 16b+15, one per wave,
// and counts every token up to its last one itself, so it knows its prefix
// without waiting for any other workgroup; then each wave writes its token's
// kv_indptr entry and scatters the token.
__global__ void __launch_bounds__(1024) build_fused_small_kernel(BuildArgs a) {
  constexpr int kTok = 16;
  __shared__ int cnt[kSmallN];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int last = min(a.N, (int)blockIdx.x * kTok + kTok);  // tokens [0, last) are counted
  const int t = (int)blockIdx.x * kTok + wave;
  for (int i = tid; i < last; i += 1024) cnt[i] = 0;
  // window lengths of the tokens before this wave's token (up to 16 per lane),
  // loaded now so that they travel with the comp_pos loads below
  int wx[kSmallN / 64];
#pragma unroll
  for (int j = 0; j < kSmallN / 64; ++j) {
    const int s = lane + 64 * j;
    wx[j] = a.swa_len[s < t && s < a.N ? s : 0];  // (waves past the batch: in bounds, unused)
  }
  int wl = 0;
#pragma unroll
  for (int j = 0; j < kSmallN / 64; ++j) wl += lane + 64 * j < t ? clamp_swa(wx[j], a.win) : 0;
  __syncthreads();
  count_flat(a, last, cnt, tid, 1024);
  __syncthreads();
  if (t >= a.N) return;
  int pre = wl;
  for (int s = lane; s < t; s += 64) pre += cnt[s];
  pre = wave_sum(pre);
  const int32_t* src = lane == 0 ? a.swa_len + t : a.state_slot + t;
  const int scal = *src;
  const int sl = clamp_swa(__builtin_amdgcn_readlane(scal, 0), a.win);
  const int64_t s0 = (int64_t)__builtin_amdgcn_readlane(scal, 1) * a.win;
  if (lane == 0) {
    a.kv_indptr[t + 1] = pre + sl + cnt[t];
    if (t == 0) a.kv_indptr[0] = 0;
  }
  scatter_token(a, t, pre, sl, s0, lane);
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

// Step 2 of the look-back builder (N <= kSmallN): one wave per token.  On
// entry kv_indptr[s+1] holds, for every token s, either ~count(s) (negative)
// or, once token s's wave has passed this point, the final prefix sum through
// s (>= 0).  Token t's start is kv_indptr[t] once final; the wave reads the
// entries below t+1, 64 at a time from the top, adding counts down to the
// first final entry (kv_indptr[0] = 0 always is one).  Every entry is either
// kind at every moment and both are exact, so no wave ever waits for another
// and any interleaving gives the same result.  The wave then writes its own
// final entry and scatters its token.
__global__ void __launch_bounds__(256) build_scatter_lookback_kernel(BuildArgs a) {
  const int t = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= a.N) return;
  const int32_t* src = lane == 0 ? a.kv_indptr + t + 1 : (lane == 1 ? a.swa_len + t : a.state_slot + t);
  const int scal = __builtin_nontemporal_load(src);
  const int own = ~__builtin_amdgcn_readlane(scal, 0);  // this token's count
  const int sl = clamp_swa(__builtin_amdgcn_readlane(scal, 1), a.win);
  const int64_t s0 = (int64_t)__builtin_amdgcn_readlane(scal, 2) * a.win;
  int base = 0;
  for (int top = t; top >= 0; top -= 64) {  // entries top, top-1, ..., top-63
    const int e = top - lane;
    const int v = e > 0 ? __builtin_nontemporal_load(a.kv_indptr + e) : 0;
    const bool fin = e <= 0 || v >= 0;
    const unsigned long long m = __ballot(fin);
    if (m != 0) {
      const int f = __builtin_ctzll(m);  // highest final entry of this chunk
      base += wave_sum(lane < f ? ~v : (lane == f ? v : 0));
      break;
    }
    base += wave_sum(~v);
  }
  if (lane == 0) a.kv_indptr[t + 1] = base + own;
  scatter_token(a, t, base, sl, s0, lane);
}

}  // namespace

hipError_t launch_build_indices(const BuildArgs& a, hipStream_t stream) {
  const unsigned blocks = (unsigned)((a.N + 3) / 4);
  if (a.N == 0) {
    hipLaunchKernelGGL(build_count_scan_kernel, dim3(1), dim3(1024), 0, stream, a);
    return hipGetLastError();
  }
  if (a.N <= kFusedMaxN && (int64_t)a.N * (a.comp_pos ? a.topk : 0) <= kFusedEntries) {
    hipLaunchKernelGGL(build_fused_small_kernel, dim3((unsigned)((a.N + 15) / 16)), dim3(1024), 0,
                       stream, a);
    return hipGetLastError();
  }
  if (a.N <= kSmallN) {  // parallel counts, then the look-back scatter
    hipLaunchKernelGGL(build_count_kernel<true>, dim3(blocks), dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(build_scatter_lookback_kernel, dim3(blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  {
    hipLaunchKernelGGL(build_count_kernel<false>, dim3(blocks), dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(build_scan_kernel, dim3(1), dim3(1024), 0, stream, a.kv_indptr, a.N);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
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
