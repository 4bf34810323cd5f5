// Internal definitions shared by the HIP translation units of librlloss.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "../../include/rlloss.h"

typedef uint16_t bf16_t;  // raw IEEE bfloat16 bits
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

#define RL_WAVE 64

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two floats to packed bf16 with v_cvt_pk_bf16_f32 (round to nearest even,
// NaN kept; checked bit for bit against the definition above).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// Element access for the two storage types (bf16 bits or fp32).
template <typename T> struct Elem;
template <> struct Elem<bf16_t> {
  static constexpr int VEC = 8;  // elements per 16-byte vector
  __device__ __forceinline__ static float to_f32(bf16_t x) { return bf16_bits_to_f32(x); }
  __device__ __forceinline__ static bf16_t from_f32(float f) {
    return __builtin_bit_cast(bf16_t, (__bf16)f);
  }
  // Unpack one 16-byte vector to 8 floats.
  __device__ __forceinline__ static void unpack(const u32x4& v, float* out) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(v[i] << 16);
      out[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
  }
  __device__ __forceinline__ static u32x4 pack(const float* in) {
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = pack_bf16x2(in[2 * i], in[2 * i + 1]);
    return v;
  }
};
template <> struct Elem<float> {
  static constexpr int VEC = 4;
  __device__ __forceinline__ static float to_f32(float x) { return x; }
  __device__ __forceinline__ static float from_f32(float f) { return f; }
  __device__ __forceinline__ static void unpack(const u32x4& v, float* out) {
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(v[i]);
  }
  __device__ __forceinline__ static u32x4 pack(const float* in) {
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __float_as_uint(in[i]);
    return v;
  }
};

// Importance weight of the three loss types (prime-rl PR 4233, "What
// changes"): ipo 1(|p-q| <= eps) * min(p/q, max_ratio); icepop
// 1(lo <= p/q <= hi) * p/q; reinforce 1.  Inputs are log-probabilities.
struct WeightParams {
  int type;
  float eps, max_ratio, lo, hi;
};

__device__ __forceinline__ float rl_weight(float lp, float lq, const WeightParams& wp,
                                           bool* keep) {
  if (wp.type == RL_LOSS_REINFORCE) {
    *keep = true;
    return 1.0f;
  }
  float r = expf(lp - lq);
  if (wp.type == RL_LOSS_IPO) {
    float P = expf(lp), Q = expf(lq);
    bool k = fabsf(P - Q) <= wp.eps;
    *keep = k;
    return k ? fminf(r, wp.max_ratio) : 0.0f;
  }
  bool k = (wp.lo <= r) && (r <= wp.hi);
  *keep = k;
  return k ? r : 0.0f;
}

// Wave-level reductions (64 lanes), fixed butterfly order.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_add(float x) {
  // lanes outside ROW_MASK, and lanes whose source falls outside their row,
  // receive 0
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK,
                                                        0xf, true));
}

// Wave totals of NF per-lane float sums, in a fixed order, stored as fp64 to
// dst[0 .. NF).  A transposing butterfly (gfx950 lane swaps):
//  * permlane32_swap of sums x, y gives (x lanes 0-31 | y lanes 0-31) and
//    (x lanes 32-63 | y lanes 32-63); their sum holds 32 partials of x in
//    lanes 0-31 and 32 of y in lanes 32-63 (one add for two sums);
//  * permlane16_swap of two such values swaps 16-lane rows the same way, so
//    their sum holds four sums with 16 partials each, one per row: row r
//    holds sum 4j + (0, 2, 1, 3)[r];
//  * an inclusive scan inside each row (row shifts by 1, 2, 4, 8) leaves the
//    row total in the row's lane 15.
template <int NF>
__device__ __forceinline__ void wave_totals(const float* f, double* dst, int lane) {
  constexpr int NG = (NF + 1) / 2, NH = (NG + 1) / 2;
  float g[2 * NH];
#pragma unroll
  for (int i = 0; i < NG; ++i) {
    const float x = f[2 * i], y = 2 * i + 1 < NF ? f[2 * i + 1] : 0.0f;
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y),
                                                    false, false);
    g[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  if constexpr (NG < 2 * NH) g[NG] = 0.0f;
  const int r = lane >> 4;
  const int off = ((r & 1) << 1) | (r >> 1);
#pragma unroll
  for (int j = 0; j < NH; ++j) {
    const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(g[2 * j]),
                                                    __float_as_uint(g[2 * j + 1]), false, false);
    float h = __uint_as_float(s[0]) + __uint_as_float(s[1]);
    h = dpp_add<0x111, 0xf>(h);  // row_shr:1
    h = dpp_add<0x112, 0xf>(h);  // row_shr:2
    h = dpp_add<0x114, 0xf>(h);  // row_shr:4
    h = dpp_add<0x118, 0xf>(h);  // row_shr:8
    const int id = 4 * j + off;
    if ((lane & 15) == 15 && id < NF) dst[id] = (double)h;
  }
}

__host__ __device__ static inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
__host__ __device__ static inline int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }
