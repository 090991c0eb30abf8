// probe.hip -- measurement kernels of libspd_probe.so (include/spd_probe.h):
// the gather of the attention kernels without their arithmetic, an empty
// launch and a whole-grid store.  They bound the attention path's time from
// below; nothing in the attention path calls them.
#include "attn_device.h"
#include "spd_probe.h"

namespace spd {
namespace {

// The rows kernel's gather: workgroup = (token, group, partition), four
// waves taking every fourth 16-row tile of the partition's rows into two
// private LDS stages, two tiles in flight a wave, indices staged in LDS first.
template <int D>
__global__ void __launch_bounds__(256) gather_probe_kernel(const uint16_t* kv,
                                                           const int32_t* kv_indices,
                                                           const int32_t* kv_indptr, int groups,
                                                           int parts, uint32_t* out_words) {
  constexpr int kWaves = 4;
  constexpr int kTile = 16;
  constexpr int kRowBytes = 2 * D;
  constexpr int kRowsPerLoad = 1024 / kRowBytes;
  constexpr int kLoads = kTile / kRowsPerLoad;
  constexpr int kStageBytes = kTile * kRowBytes;
  static_assert(2 * kLoads <= 63, "two tiles of loads must fit vmcnt");

  __shared__ __attribute__((aligned(1024))) unsigned char smem[kWaves * 2 * kStageBytes];
  __shared__ __attribute__((aligned(256))) int sidx[kIdxCap];

  const int item = xcd_item(blockIdx.x, gridDim.x);
  const int c = item % parts;
  const int t = item / parts / groups;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  const ScalarI32Ptr indptr = (ScalarI32Ptr)kv_indptr;
  const int row0 = indptr[t];
  const int L = indptr[t + 1] - row0;
  const int lo = (int)((int64_t)L * c / parts);
  const int hi = (int)((int64_t)L * (c + 1) / parts);
  const int Lp = hi - lo;
  unsigned char* mine = smem + wave * 2 * kStageBytes;
  uint32_t word = 0;
  for (int sc = 0; sc < Lp; sc += kIdxCap) {
    const int n = Lp - sc < kIdxCap ? Lp - sc : kIdxCap;
    if (sc > 0) barrier_lds();  // every wave is done with the previous indices
    stage_indices(kv_indices + row0 + lo, sc, n, sidx, wave, kWaves, lane);
    wait_vmcnt<0>();
    barrier_lds();
    const int ntiles = (n + kTile - 1) / kTile;
    const int my = ntiles > wave ? (ntiles - wave + kWaves - 1) / kWaves : 0;
    auto issue = [&](int j) {
      issue_rows<kRowBytes, kLoads>(kv, sidx, n, (wave + kWaves * j) * kTile, 0,
                                    mine + (j & 1) * kStageBytes, lane);
    };
    if (my > 0) issue(0);
    if (my > 1) issue(1);
    for (int j = 0; j < my; ++j) {
      // tile j has landed once at most the next tile's loads are outstanding
      if (j + 1 < my)
        wait_vmcnt<kLoads>();
      else
        wait_vmcnt<0>();
      asm volatile("" ::: "memory");
      if (j + 2 < my) issue(j + 2);
    }
    wait_vmcnt<0>();
    asm volatile("" ::: "memory");
    if (my > 0) word ^= reinterpret_cast<const uint32_t*>(mine)[lane];
  }
  // one word a workgroup (lane 0 of wave 0), so the loads have a consumer
  if (threadIdx.x == 0) out_words[blockIdx.x] = word;
}

__global__ void __launch_bounds__(256) null_probe_kernel() {}

__global__ void __launch_bounds__(256) store_probe_kernel(uint4* out, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride)
    out[i] = make_uint4(0u, 0u, 0u, 0u);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace
}  // namespace spd

extern "C" {

SPD_PROBE_API int spd_probe_gather(const void* kv, const int32_t* kv_indices,
                                   const int32_t* kv_indptr, int32_t N, int32_t D, int32_t groups,
                                   int32_t parts, uint32_t* out_words, void* stream) {
  if (N < 0 || groups < 1 || parts < 1) return 1;
  if (D != 64 && D != 128 && D != 256 && D != 512) return 1;
  const long long wgs = (long long)N * groups * parts;
  if (wgs > 0x7fffffffLL) return 1;
  if (N == 0) return 0;
  if (!kv || !kv_indices || !kv_indptr || !out_words || !spd::aligned16(kv)) return 1;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)wgs), block(256);
  const uint16_t* k = static_cast<const uint16_t*>(kv);
  switch (D) {
    case 64:
      hipLaunchKernelGGL(spd::gather_probe_kernel<64>, grid, block, 0, s, k, kv_indices, kv_indptr,
                         groups, parts, out_words);
      break;
    case 128:
      hipLaunchKernelGGL(spd::gather_probe_kernel<128>, grid, block, 0, s, k, kv_indices,
                         kv_indptr, groups, parts, out_words);
      break;
    case 256:
      hipLaunchKernelGGL(spd::gather_probe_kernel<256>, grid, block, 0, s, k, kv_indices,
                         kv_indptr, groups, parts, out_words);
      break;
    default:
      hipLaunchKernelGGL(spd::gather_probe_kernel<512>, grid, block, 0, s, k, kv_indices,
                         kv_indptr, groups, parts, out_words);
      break;
  }
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

SPD_PROBE_API int spd_probe_null(int32_t workgroups, void* stream) {
  if (workgroups < 1) return 1;
  hipLaunchKernelGGL(spd::null_probe_kernel, dim3((unsigned)workgroups), dim3(256), 0,
                     static_cast<hipStream_t>(stream));
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

SPD_PROBE_API int spd_probe_store(void* out, int64_t bytes, int32_t workgroups, void* stream) {
  if (workgroups < 1 || bytes < 0 || bytes % 16 != 0) return 1;
  if (bytes == 0) return 0;
  if (!out || !spd::aligned16(out)) return 1;
  hipLaunchKernelGGL(spd::store_probe_kernel, dim3((unsigned)workgroups), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<uint4*>(out), bytes / 16);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // extern "C"
