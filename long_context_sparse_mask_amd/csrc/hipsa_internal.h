// Internal declarations shared by the HIP kernels and the host entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/hipsa.h"

namespace hipsa {

constexpr int kMaxKb = 512;   // largest K_b = k / block_k the kernels accept
constexpr int kMaxGroup = 16; // largest Hq / Hkv

// Validated shape of one call, in the units the kernels use.
struct Shape {
  int64_t B, Hq, Hkv, Tq, T, T_cap, d;
  int32_t G, Kb, bk, bq, causal, dtype;
  int64_t nqb;     // query blocks per (b, kv head)
  int64_t problems; // B * Hkv * nqb
};

struct MaskArgs {
  const void *q, *K;
  int32_t *indices, *nnz;
  Shape s;
};

struct AttnArgs {
  const void *q, *K, *V;
  const int32_t *indices, *nnz;
  void *out;
  float *ws;
  Shape s;
  int32_t splits;  // decode: key splits per problem
  float scale;     // 1 / sqrt(d)
};

// Decode / per-row problems (block_q == 1).
hipError_t launch_mask_decode(const MaskArgs &a, hipStream_t st);
hipError_t launch_attn_decode(const AttnArgs &a, hipStream_t st);
size_t attn_decode_workspace(const Shape &s);
int32_t attn_decode_splits(const Shape &s);

// Chunked prefill (block_q == 64, bf16).
hipError_t launch_mask_prefill(const MaskArgs &a, hipStream_t st);
hipError_t launch_attn_prefill(const AttnArgs &a, hipStream_t st);

// ------------------------------------------------------------------ device helpers

// 16-byte vector loads widened to fp32.  bf16 widens exactly by a 16-bit shift.
template <typename E> struct Vec;
template <> struct Vec<float> {
  static constexpr int N = 4;
  __device__ static inline void load(const float *p, float (&v)[4]) {
    float4 x = *reinterpret_cast<const float4 *>(p);
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
  }
};
template <> struct Vec<uint16_t> {
  static constexpr int N = 8;
  __device__ static inline void load(const uint16_t *p, float (&v)[8]) {
    uint4 x = *reinterpret_cast<const uint4 *>(p);
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int i = 0; i < 4; i++) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};

// fp32 -> bf16 bits, round to nearest even (inputs here are finite).
__device__ inline uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ inline void store_elem(float *p, float v) { *p = v; }
__device__ inline void store_elem(uint16_t *p, float v) { *p = f32_to_bf16(v); }

// Ranking key of a candidate chunk: larger key = ranked earlier.  Score
// descending first (IEEE order mapped onto unsigned order, -0 folded into +0),
// then chunk start ascending.  0 is below every real key (empty slot).
__device__ inline uint64_t rank_key(float score, int32_t start) {
  float s = score + 0.0f;
  uint32_t u = __float_as_uint(s);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (uint32_t)(0x7fffffff - start);
}

template <int W> __device__ inline float group_sum(float v) {
#pragma unroll
  for (int m = W / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}
__device__ inline float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}
__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

}  // namespace hipsa
