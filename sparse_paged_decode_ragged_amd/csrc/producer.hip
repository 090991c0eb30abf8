// producer.hip -- the decode-step producer, gfx950: per-head RMSNorm of q,
// RMSNorm of each token's new KV row, rotary embedding of both, and the store
// of the KV row into its window-ring slot of the pool (bf16 and/or FP8).
//
// Source: sglang PR #25898 summary page, "key files": one fused kernel does
// the q per-head RMSNorm, the KV RMSNorm, RoPE, the FP8 quantisation and the
// paged sliding-window store (helpers: a batched RMSNorm, a GPT-J rotation, a
// batched RoPE).  The page names the steps, not their formulas; the readings:
//   * RMSNorm of a row x[0, D) with an fp32 weight w: x_d * w_d / sqrt(mean(x^2) + eps);
//   * RoPE with GPT-J (interleaved) pairs on the last rope_dim entries
//     (o = D - rope_dim): for i < rope_dim / 2, with c = cos_sin[p][i] and
//     s = cos_sin[p][rope_dim/2 + i] from the caller's table,
//     (y[o+2i], y[o+2i+1]) <- (y[o+2i] c - y[o+2i+1] s, y[o+2i] s + y[o+2i+1] c);
//   * the KV row of token t at position p goes to pool row
//     state_slot[t] * win + p mod win (the ring keeps positions p-win+1 .. p);
//   * every output is rounded to bf16; the FP8 store quantises that bf16 row
//     exactly as quantize_kv_fp8 would.
//
// Work: one wave per row, D / 64 entries a lane (entries 2i, 2i+1 of a pair
// sit in one lane for D >= 128; at D = 64 the partner comes from lane ^ 1).
// Rows [0, N*H) are q rows (token r / H), rows [N*H, N*H + N) KV rows.  The
// kernel reads and writes each row once; a wave's life is one row load and
// the cross-lane sum, so the row's latency sets its throughput.
#include <math.h>

#include "row_device.h"
#include "store_internal.h"

namespace spd {
namespace {

// Wave-uniform loads from these (the token's position and state slot) go
// through the scalar unit, so they do not queue behind the row's vector load.
typedef const __attribute__((address_space(4))) int32_t* ConstI32Ptr;

// One row's state between its loads and its stores.  issue_row sends the
// row's load first; the position (a scalar load) comes back on its own
// counter, so the rotary factors it selects, and the weights, are loaded
// while the row is still in flight: the row's sum of squares in finish_row is
// the only step that waits for it.
template <int D>
struct RowState {
  static constexpr int E = D / 64;
  static constexpr int kPairs = E >= 2 ? E / 2 : 1;
  int64_t r;
  bool live, is_kv, pos_ok;
  int t, p;
  int64_t ring0;
  float x[E], wt[E], cr[kPairs], sr[kPairs];
};

template <int D>
__device__ __forceinline__ void issue_row(const ProducerArgs& a, int64_t r, int lane, RowState<D>& st) {
  constexpr int E = D / 64;
  const int64_t nq = (int64_t)a.N * a.H;
  st.r = r;
  st.live = r < nq + a.N;
  if (!st.live) return;
  st.is_kv = r >= nq;
  st.t = st.is_kv ? (int)(r - nq) : (int)(r / a.H);
  const uint16_t* src = st.is_kv ? a.kv + (int64_t)st.t * D : a.q + r * D;
  load_bf16_lane<E>(src + lane * E, st.x);
  st.p = ((ConstI32Ptr)a.positions)[st.t];
  st.ring0 = st.is_kv ? (int64_t)((ConstI32Ptr)a.state_slot)[st.t] * a.win : 0;
  const float* w = st.is_kv ? a.kv_weight : a.q_weight;
#pragma unroll
  for (int e = 0; e < E; ++e) st.wt[e] = w[lane * E + e];
  st.pos_ok = st.p >= 0 && (a.rope_dim == 0 || st.p < a.max_pos);
  const int o = D - a.rope_dim, half = a.rope_dim >> 1;
#pragma unroll
  for (int k = 0; k < RowState<D>::kPairs; ++k) {
    st.cr[k] = 1.f;
    st.sr[k] = 0.f;
  }
  if (st.pos_ok && a.rope_dim > 0) {
    const float* cs = a.cos_sin + (int64_t)st.p * a.rope_dim;
#pragma unroll
    for (int k = 0; k < RowState<D>::kPairs; ++k) {
      const int d = E >= 2 ? lane * E + 2 * k : lane;
      if (d >= o) {
        const int i = (d - o) >> 1;
        st.cr[k] = cs[i];
        st.sr[k] = cs[half + i];
      }
    }
  }
}

template <int D>
__device__ __forceinline__ void finish_row(const ProducerArgs& a, int lane, RowState<D>& st) {
  constexpr int E = D / 64;
  if (!st.live) return;
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) ss += st.x[e] * st.x[e];
  ss = wave_reduce<false>(ss);
  if (!st.pos_ok) return;
  int64_t slot = 0;
  if (st.is_kv) {
    slot = st.ring0 + st.p % a.win;
    if (slot < 0 || slot >= a.num_rows) return;
  }
  const float inv = 1.0f / sqrtf(ss / (float)D + a.eps);
  float y[E];
#pragma unroll
  for (int e = 0; e < E; ++e) y[e] = st.x[e] * inv * st.wt[e];
  const int o = D - a.rope_dim;
  if constexpr (E >= 2) {
#pragma unroll
    for (int e = 0; e < E; e += 2) {
      const int d = lane * E + e;
      if (d >= o) {
        const float c = st.cr[e / 2], s = st.sr[e / 2];
        const float y0 = y[e], y1 = y[e + 1];
        y[e] = y0 * c - y1 * s;
        y[e + 1] = y0 * s + y1 * c;
      }
    }
  } else {
    const float partner = __shfl_xor(y[0], 1);
    if (lane >= o) {
      const float c = st.cr[0], s = st.sr[0];
      y[0] = (lane & 1) == 0 ? y[0] * c - partner * s : partner * s + y[0] * c;
    }
  }
  if (!st.is_kv) {
    store_bf16_lane<E>(a.q_out + st.r * D + lane * E, y);
    return;
  }
  if (a.kv_bf16 != nullptr) store_bf16_lane<E>(a.kv_bf16 + slot * D + lane * E, y);
  if (a.kv8 != nullptr) {
    float yb[E];
#pragma unroll
    for (int e = 0; e < E; ++e) yb[e] = __builtin_bit_cast(float, bf16_rne_bits(y[e]) << 16);
    store_fp8_lane<E>(yb, a.kv8 + slot * D + lane * E, a.kv_scale + slot, lane);
  }
}

// kRows consecutive rows a wave, every row's loads issued before the first
// is finished: two rows double the bytes a wave keeps in flight, which large
// batches need; small batches want the waves instead (one row a wave).
template <int D, int kRows>
__global__ void __launch_bounds__(256) qk_norm_rope_store_kernel(ProducerArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t r0 =
      ((int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6)) * kRows;
  RowState<D> st[kRows];
#pragma unroll
  for (int j = 0; j < kRows; ++j) issue_row<D>(a, r0 + j, lane, st[j]);
#pragma unroll
  for (int j = 0; j < kRows; ++j) finish_row<D>(a, lane, st[j]);
}

// Rows from which a wave takes two (measured: N = 1024, H = 128, D = 512 with
// 132k rows 64.4 -> 57.5 us; N = 64, H = 64 with 4160 rows 4.9 -> 5.6 us;
// four rows a wave 76 us).
constexpr long long kTwoRowsFrom = 32768;

template <int D>
hipError_t launch_producer_d(const ProducerArgs& a, hipStream_t stream) {
  const long long rows = (long long)a.N * a.H + a.N;
  if (rows >= kTwoRowsFrom) {
    hipLaunchKernelGGL((qk_norm_rope_store_kernel<D, 2>), dim3((unsigned)((rows + 7) / 8)),
                       dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL((qk_norm_rope_store_kernel<D, 1>), dim3((unsigned)((rows + 3) / 4)),
                       dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_producer(const ProducerArgs& a, int D, hipStream_t stream) {
  switch (D) {
    case 64: return launch_producer_d<64>(a, stream);
    case 128: return launch_producer_d<128>(a, stream);
    case 256: return launch_producer_d<256>(a, stream);
    case 512: return launch_producer_d<512>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace spd
