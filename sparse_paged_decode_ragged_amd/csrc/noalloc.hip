// noalloc.hip -- sparse_decode_attn_ex for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc): the split plans' workspace is a static device array
// of this library instead of a caller buffer.
//
// The array lives in the library's code object, one copy per GPU, held until
// the process ends.  Its address on a GPU is read once per device with
// hipGetSymbolAddress (the array's name in host code is only a host-side
// stand-in) and kept; kernels and the clearing launch take that address.
// Every call on a GPU shares the array: calls that overlap on one GPU (other
// streams, other host threads) race on it.
#include <atomic>
#include <mutex>

#include "api_internal.h"

namespace {

constexpr size_t kScratchBytes = SPD_NOALLOC_WORKSPACE_BYTES;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
std::atomic<void*> g_scratch[kMaxDevices];

// The array's device address on `dev`, which must be the current device.
hipError_t scratch_address(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

// Zero n 32-bit words (a kernel, not a memset node: graph-capturable).
__global__ void __launch_bounds__(256) clear_words_kernel(uint32_t* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0u;
}

}  // namespace

extern "C" {

SPD_API spd_status sparse_decode_attn_noalloc(const void* q, const void* unified_kv,
                                              int64_t num_rows, const int32_t* kv_indices,
                                              const int32_t* kv_indptr, const float* attn_sink,
                                              float softmax_scale, void* out, int32_t N, int32_t H,
                                              int32_t D, int32_t max_len, int32_t split_rows,
                                              int32_t mode, void* stream) {
  spd::AttnArgs a{};
  spd::AttnPlan plan{};
  bool empty = false;
  const spd_status st =
      spd::prepare_attn_ex(q, unified_kv, num_rows, kv_indices, kv_indptr, attn_sink, softmax_scale,
                           out, N, H, D, max_len, split_rows, mode, &a, &plan, &empty);
  if (st != SPD_OK || empty) return st;
  if (plan.workspace_bytes > kScratchBytes) return SPD_ERR_WORKSPACE;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (plan.workspace_bytes > 0) {
    // the array of the GPU the stream runs on, which must be the current one
    int cur = 0, dev = 0;
    if (hipGetDevice(&cur) != hipSuccess) return SPD_ERR_HIP;
    dev = cur;
    if (s != nullptr && hipStreamGetDevice(s, &dev) != hipSuccess) return SPD_ERR_HIP;
    if (dev != cur) return SPD_ERR_INVALID_ARG;
    void* ws = nullptr;
    if (scratch_address(dev, &ws) != hipSuccess) return SPD_ERR_HIP;
    a.ws = static_cast<float*>(ws);
    if (plan.mode == spd::kModeSplit) {
      // the arrival counters must start at zero; an earlier call of another
      // plan may have left partial results where this plan keeps them
      unsigned char* base = static_cast<unsigned char*>(ws);
      const size_t off = spd::split_counters_offset(N, D, plan);
      const int64_t words = (int64_t)(plan.workspace_bytes - off) / 4;
      const unsigned blocks = (unsigned)((words + 255) / 256);
      hipLaunchKernelGGL(clear_words_kernel, dim3(blocks), dim3(256), 0, s,
                         reinterpret_cast<uint32_t*>(base + off), words);
      if (hipGetLastError() != hipSuccess) return SPD_ERR_HIP;
    }
  }
  const hipError_t e = spd::launch_attention(a, D, plan, s);
  return e == hipSuccess ? SPD_OK : SPD_ERR_HIP;
}

}  // extern "C"
