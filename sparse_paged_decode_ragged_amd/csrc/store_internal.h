// Internal declarations of the row-store kernels of libspd: the quantising
// store into an FP8 pool and the decode-step producer.  Not installed; the
// public ABI is include/spd.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace spd {

struct QuantArgs {
  const uint16_t* src;   // [n][D] bf16 rows
  const int32_t* slots;  // [n] destination rows, or null for 0 .. n-1
  uint8_t* kv8;          // [num_rows][D] e4m3 codes (out)
  float* kv_scale;       // [num_rows] (out)
  int32_t n;
  int64_t num_rows;
};

hipError_t launch_quantize_fp8(const QuantArgs& args, int D, hipStream_t stream);

struct ProducerArgs {
  const uint16_t* q;          // [N][H][D] bf16
  uint16_t* q_out;            // [N][H][D] bf16 (may be q)
  const uint16_t* kv;         // [N][D] bf16, each token's new KV row
  const float* q_weight;      // [D]
  const float* kv_weight;     // [D]
  float eps;
  const int32_t* positions;   // [N]
  const float* cos_sin;       // [max_pos][rope_dim]: cos in [0, rope_dim/2), sin after
  int32_t max_pos, rope_dim;
  const int32_t* state_slot;  // [N]
  int32_t win;
  uint16_t* kv_bf16;          // [num_rows][D] bf16 pool, or null
  uint8_t* kv8;               // [num_rows][D] FP8 pool codes, or null
  float* kv_scale;            // [num_rows] FP8 pool scales (with kv8)
  int64_t num_rows;
  int32_t N, H;
};

hipError_t launch_producer(const ProducerArgs& args, int D, hipStream_t stream);

}  // namespace spd
