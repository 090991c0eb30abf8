// row_device.h -- per-wave row helpers shared by the quantising store
// (attn_fp8.hip) and the decode-step producer (producer.hip): a row of
// D = 64 E entries is held by one wave, lane l owning entries E l .. E l + E - 1.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace spd {
namespace {

typedef unsigned rd_u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned rd_u32x4 __attribute__((ext_vector_type(4)));

// The lane's E bf16 entries of a row (src = row start + E * lane) as fp32.
template <int E>
__device__ __forceinline__ void load_bf16_lane(const uint16_t* src, float (&x)[E]) {
  unsigned w[(E + 1) / 2];
  if constexpr (E == 8) {
    const rd_u32x4 v = *reinterpret_cast<const rd_u32x4*>(src);
    w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3];
  } else if constexpr (E == 4) {
    const rd_u32x2 v = *reinterpret_cast<const rd_u32x2*>(src);
    w[0] = v[0]; w[1] = v[1];
  } else if constexpr (E == 2) {
    w[0] = *reinterpret_cast<const unsigned*>(src);
  } else {
    w[0] = src[0];
  }
#pragma unroll
  for (int e = 0; e < E; ++e)
    x[e] = __builtin_bit_cast(float, e % 2 == 0 ? w[e / 2] << 16 : w[e / 2] & 0xffff0000u);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ unsigned bf16_rne_bits(float f) {
  const unsigned u = __builtin_bit_cast(unsigned, f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Store the lane's E values rounded to bf16 (dst = row start + E * lane).
template <int E>
__device__ __forceinline__ void store_bf16_lane(uint16_t* dst, const float (&y)[E]) {
  unsigned w[(E + 1) / 2];
#pragma unroll
  for (int e = 0; e < E; e += 2)
    w[e / 2] = bf16_rne_bits(y[e]) | (e + 1 < E ? bf16_rne_bits(y[e + 1]) << 16 : 0u);
  if constexpr (E == 8) {
    *reinterpret_cast<rd_u32x4*>(dst) = rd_u32x4{w[0], w[1], w[2], w[3]};
  } else if constexpr (E == 4) {
    *reinterpret_cast<rd_u32x2*>(dst) = rd_u32x2{w[0], w[1]};
  } else if constexpr (E == 2) {
    *reinterpret_cast<unsigned*>(dst) = w[0];
  } else {
    dst[0] = (uint16_t)w[0];
  }
}

// Sum and maximum of one value over the wave with VALU cross-lane operations
// only: DPP within each 16-lane row (pairs, quads, then the two mirrors), then
// v_permlane32_swap and v_permlane16_swap across the rows.  No LDS permute
// sits in the row's dependent chain, and every lane gets the same bits (each
// step combines a lane with a partner that combines it back).
template <int kCtrl>
__device__ __forceinline__ float rd_dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, 0xf, 0xf, false));
}

template <bool kMax>
__device__ __forceinline__ float rd_combine(float a, float b) {
  return kMax ? fmaxf(a, b) : a + b;
}

template <bool kMax>
__device__ __forceinline__ float wave_reduce(float v) {
  v = rd_combine<kMax>(v, rd_dpp<0xB1>(v));   // quad_perm [1, 0, 3, 2]
  v = rd_combine<kMax>(v, rd_dpp<0x4E>(v));   // quad_perm [2, 3, 0, 1]
  v = rd_combine<kMax>(v, rd_dpp<0x141>(v));  // row_half_mirror
  v = rd_combine<kMax>(v, rd_dpp<0x140>(v));  // row_mirror
  const unsigned u = __builtin_bit_cast(unsigned, v);
  const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  v = rd_combine<kMax>(__builtin_bit_cast(float, (unsigned)a[0]), __builtin_bit_cast(float, (unsigned)a[1]));
  const unsigned w = __builtin_bit_cast(unsigned, v);
  const auto b = __builtin_amdgcn_permlane16_swap(w, w, false, false);
  return rd_combine<kMax>(__builtin_bit_cast(float, (unsigned)b[0]), __builtin_bit_cast(float, (unsigned)b[1]));
}

// FP8 store of one row held by the wave (x: the lane's E values): amax over
// the wave; a row with amax < 2^-64 stores scale 0 and zero codes; otherwise
// scale = amax / 448, inv = 448 / amax (correctly rounded fp32 divisions),
// y = clamp(x * inv, -448, 448) and the codes are y rounded to the nearest
// e4m3 value, ties to even (v_cvt_pk_fp8_f32).  dst = row start + E * lane;
// lane 0 writes *scale_dst.
template <int E>
__device__ __forceinline__ void store_fp8_lane(const float (&x)[E], uint8_t* dst, float* scale_dst,
                                               int lane) {
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) amax = fmaxf(amax, fabsf(x[e]));
  amax = wave_reduce<true>(amax);
  unsigned code[(E + 3) / 4];
  float scale = 0.f;
#pragma unroll
  for (int c = 0; c < (E + 3) / 4; ++c) code[c] = 0;
  if (amax >= 0x1p-64f) {
    scale = amax / 448.0f;
    const float inv = 448.0f / amax;
    float y[E];
#pragma unroll
    for (int e = 0; e < E; ++e) y[e] = fminf(fmaxf(x[e] * inv, -448.0f), 448.0f);
#pragma unroll
    for (int c = 0; c < (E + 3) / 4; ++c) {
      const float y0 = y[4 * c];
      const float y1 = 4 * c + 1 < E ? y[4 * c + 1] : 0.f;
      unsigned w = (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
      if (4 * c + 2 < E) {
        const float y3 = 4 * c + 3 < E ? y[4 * c + 3] : 0.f;
        w = (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(y[4 * c + 2], y3, (int)w, true);
      }
      code[c] = w;
    }
  }
  if constexpr (E == 8) {
    *reinterpret_cast<rd_u32x2*>(dst) = rd_u32x2{code[0], code[1]};
  } else if constexpr (E == 4) {
    *reinterpret_cast<unsigned*>(dst) = code[0];
  } else if constexpr (E == 2) {
    *reinterpret_cast<uint16_t*>(dst) = (uint16_t)(code[0] & 0xffff);
  } else {
    dst[0] = (uint8_t)(code[0] & 0xff);
  }
  if (lane == 0) *scale_dst = scale;
}

}  // namespace
}  // namespace spd
