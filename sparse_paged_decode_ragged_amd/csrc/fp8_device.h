// fp8_device.h -- device helpers for attention over an FP8 pool (rows of D
// e4m3 codes plus one fp32 scale a row), shared by attn_fp8.hip and the
// split kernel of attn_split.hip: the exact e4m3 -> bf16 operand decode, the
// softmax step with fp32 weights (the row scale multiplies them before they
// are rounded), and the LDS read offsets of the K and V^T operands of a tile
// of codes staged with the row swizzle of issue_rows (chunk c of row r at
// c ^ (r & 15)).  Anonymous namespace: each translation unit gets its own copy.
#pragma once

#include "attn_device.h"

namespace spd {
namespace {

typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 LdsV2i32;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Four e4m3 codes (bytes of raw, in order) -> four bf16 values, exactly
// (v_cvt_scalef32_pk_bf16_fp8 with scale 1 decodes two codes per instruction;
// an e4m3 value has at most 4 significant bits and an exponent well inside
// the bf16 range).
__device__ __forceinline__ bf16x4 e4m3x4_to_bf16(unsigned raw) {
  const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw, 1.0f, false);  // bytes 0, 1
  const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw, 1.0f, true);   // bytes 2, 3
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3);
}

__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(u32x2 raw) {
  return __builtin_shufflevector(e4m3x4_to_bf16(raw[0]), e4m3x4_to_bf16(raw[1]), 0, 1, 2, 3, 4,
                                 5, 6, 7);
}

// softmax_tile with fp32 weights: pf[j] = 2^(x[j] - m), unrounded, for the
// caller to scale by its row's FP8 scale before rounding to bf16; lpart sums
// them.  Reference maximum, its headroom and the second-pass flag as in
// softmax_tile.
template <int R>
__device__ __forceinline__ bool softmax_tile_f32(const float (&x)[R], float sink_l2, int g,
                                                 bool& first, float& m, float& mtrue,
                                                 float& lpart, float (&pf)[R]) {
  float mx = x[0];
#pragma unroll
  for (int j = 1; j < R; ++j) mx = fmaxf(mx, x[j]);
  mx = group_max4(mx);
  mtrue = fmaxf(mtrue, mx);
  if (first) {
    m = fmaxf(sink_l2, mx);
    lpart = (g == 0 && sink_l2 > -INFINITY) ? __builtin_amdgcn_exp2f(sink_l2 - m) : 0.f;
    first = false;
  }
  const bool over = __builtin_amdgcn_ballot_w64(mx > m + kRaise) != 0;
  float psum = 0.f;
#pragma unroll
  for (int j = 0; j < R; ++j) {
    pf[j] = __builtin_amdgcn_exp2f(x[j] - m);
    psum += pf[j];
  }
  lpart += psum;
  return over;
}

// Byte offsets of the 32x32x16 V^T operand reads of an FP8 tile (rows of D
// codes; 16-byte chunk c of row r stored at c ^ (r & 15)).  Within each
// 16-lane group the 8-bit transposing read gives destination lane i byte e
// from source lane 2e + i/8, byte i % 8.  Source lane (G = lane / 16,
// j = lane % 16) points at row 8 (G / 2) + j / 2, byte 8 (j % 2) of chunk
// wide_vt_chunk(dt, G % 2); destination lane (G, i) then holds rows
// 8 (G / 2) .. + 7 of that chunk's column i, the A operand of the product
// (lane (d, kg): rows 8 kg .. 8 kg + 7 of column d of d-tile dt).  At D >= 256
// d-tile dt is chunks a and a ^ 8 with a = dt % 8 + 16 (dt / 8): the 8 rows
// of one group fall on 8 different 16-byte bank groups (the swizzle XORs the
// low bits), and the two groups of a half-wave (chunks a and a ^ 8) on the
// two other octets of the 16, so a half-wave's 256 bytes meet no conflict.
// (Chunks 2 dt and 2 dt + 1, the columns in order, put both groups on the
// same octet: two cycles a half-wave.)  At D = 128 the d-tiles stay 2 dt,
// 2 dt + 1.  The output columns follow the same map.  Rows 16..31 add 16 D.
template <int D>
__device__ __forceinline__ constexpr int wide_vt_chunk(int dt, int half) {
  return D >= 256 ? ((dt & 7) + 16 * (dt >> 3)) + 8 * half : 2 * dt + half;
}

template <int D>
struct Fp8WideVtOffsets {
  int base, x;
  __device__ __forceinline__ explicit Fp8WideVtOffsets(int lane) {
    const int G = lane >> 4, j = lane & 15;
    const int row = 8 * (G >> 1) + (j >> 1);
    const int sw = row_swizzle(row) & (D / 16 - 1);
    base = row * D + 8 * (j & 1);
    x = (wide_vt_chunk<D>(0, G & 1) - wide_vt_chunk<D>(0, 0)) ^ sw;  // chunk (a + h) ^ sw = a ^ x
  }
  __device__ __forceinline__ int at(int dt) const { return base + 16 * (wide_vt_chunk<D>(dt, 0) ^ x); }
};

// Byte offsets of the K-operand reads of an FP8 tile (16-byte chunk c of row r
// stored at c ^ (r & 15)): lane (n16, g) reads codes 32 s + 8 g .. + 7 of row
// n16 for k-step s, half g & 1 of logical chunk 2 s + (g >> 1).  With
// w = swizzle(n16) ^ (g >> 1) that chunk sits at 2 (s ^ (w >> 1)) + (w & 1), so
// the read is at base + 32 (s ^ x), computed per read (two VALU ops, no table
// in registers).  Rows 16..31 add 16 D.
template <int D>
struct Fp8KOffsets {
  int base, x;
  __device__ __forceinline__ Fp8KOffsets(int n16, int g) {
    const int w = (row_swizzle(n16) & (D / 16 - 1)) ^ (g >> 1);
    base = n16 * D + 16 * (w & 1) + 8 * (g & 1);
    x = w >> 1;
  }
  __device__ __forceinline__ int kq(int s) const { return base + 32 * (s ^ x); }
};

}  // namespace
}  // namespace spd
