// fr_device.h -- device-side types and helpers shared by the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "fr_internal.h"

namespace fr {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef float float2v __attribute__((ext_vector_type(2)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef uint32_t uint4v __attribute__((ext_vector_type(4)));

constexpr int KB = kKeyBlock;
constexpr float kLog2e = 1.4426950408889634f;


static __device__ __forceinline__ float4v mfma16x16x32(half8 a, half8 b, float4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Row of the instance that unit row rho of KV head kv stands for (see the
// KV-head groups of Problem): rho = t*grp + j  ->  t*n_head + kv*grp + j.
static __device__ __forceinline__ int instance_row(int rho, int kv, int grp, int n_head) {
  if (grp == n_head) return rho;   // one KV head
  const int t = rho / grp;
  return t * n_head + kv * grp + (rho - t * grp);
}

static __device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

static __device__ __forceinline__ _Float16 bits_to_half(uint16_t b) {
  return __builtin_bit_cast(_Float16, b);
}

// Loads 8 query values of row r at d = d0 .. d0+7 and splits them into the
// f16 operand(s) of the score contraction.
template <int QMODE>
static __device__ __forceinline__ void load_q8(const void *qinst, int64_t off, bool valid, half8 &hi,
                                        half8 &lo) {
  if (QMODE == kQF16) {
    uint4v raw = valid ? *(const uint4v *)((const uint16_t *)qinst + off) : uint4v{0, 0, 0, 0};
    hi = __builtin_bit_cast(half8, raw);
    lo = half8{};
    return;
  }
  float4v x0 = {0.f, 0.f, 0.f, 0.f}, x1 = {0.f, 0.f, 0.f, 0.f};
  if (valid) {
    const float *p = (const float *)qinst + off;
    x0 = *(const float4v *)p;
    x1 = *(const float4v *)(p + 4);
  }
  float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    _Float16 h = (_Float16)x[e]; // round to nearest even
    hi[e] = h;
    lo[e] = (QMODE == kQHiLo) ? (_Float16)(x[e] - (float)h) : (_Float16)0.f;
  }
}


}  // namespace fr
