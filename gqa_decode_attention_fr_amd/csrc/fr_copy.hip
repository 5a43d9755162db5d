// fr_copy.hip -- batched f32 -> f16 row copies (round to nearest even).
//
// FlashRT pull request #185 ("feat(structures): ggml host adapter -- llama.cpp
// distribution for pi0.5 on Thor (SM110)"), the commit batching the
// persistent-KV tail copies: the prefill graph ends with one small f32 -> f16
// row copy per layer and KV tensor into the persistent encoder-KV buffers (the
// K and V this decode window later reads), and a run of them becomes one
// launch with the same per-element rounding, so the stored bits are unchanged.
//
// One launch takes up to kCopiesPerLaunch copies, their descriptors passed by
// value in the kernel arguments (no host-to-device copy, so capture-safe).
// Workgroup (x, c) converts groups of 8 elements of copy c, grid-striding over
// x, four groups per thread with their loads issued together: two 16-byte
// loads, eight conversions, one 16-byte store per group where both pointers
// are 16-byte aligned, element by element otherwise (and for the ragged last
// group).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fr_device.h"
#include "fr_internal.h"

namespace fr {
namespace {

struct CopyArgs {
  const float *src[kCopiesPerLaunch];
  uint16_t *dst[kCopiesPerLaunch];
  int64_t n[kCopiesPerLaunch];
};

__device__ __forceinline__ uint16_t to_f16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (_Float16)x);   // v_cvt_f16_f32, nearest even
}

__global__ __launch_bounds__(256) void f16_copy_kernel(CopyArgs a) {
  const int c = blockIdx.y;
  const float *src = a.src[c];
  uint16_t *dst = a.dst[c];
  const int64_t n = a.n[c];
  const bool vec = (((uintptr_t)src | (uintptr_t)dst) & 15) == 0;
  const int64_t groups = (n + 7) / 8;
  constexpr int U = 4;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t g0 = (int64_t)blockIdx.x * 256 + threadIdx.x; g0 < groups; g0 += U * stride) {
    float4v x[U][2];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t e0 = (g0 + u * stride) * 8;
      if (vec && e0 + 8 <= n) {
        x[u][0] = *(const float4v *)(src + e0);
        x[u][1] = *(const float4v *)(src + e0 + 4);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t gi = g0 + u * stride;
      if (gi >= groups) break;
      const int64_t e0 = gi * 8;
      if (vec && e0 + 8 <= n) {
        const uint4v packed = {
            (uint32_t)to_f16_bits(x[u][0].x) | ((uint32_t)to_f16_bits(x[u][0].y) << 16),
            (uint32_t)to_f16_bits(x[u][0].z) | ((uint32_t)to_f16_bits(x[u][0].w) << 16),
            (uint32_t)to_f16_bits(x[u][1].x) | ((uint32_t)to_f16_bits(x[u][1].y) << 16),
            (uint32_t)to_f16_bits(x[u][1].z) | ((uint32_t)to_f16_bits(x[u][1].w) << 16)};
        *(uint4v *)(dst + e0) = packed;
      } else {
        for (int j = 0; j < 8 && e0 + j < n; ++j) dst[e0 + j] = to_f16_bits(src[e0 + j]);
      }
    }
  }
}

}  // namespace

hipError_t launch_f16_copies(const CopyDesc *copies, int n_copies, hipStream_t stream) {
  for (int base = 0; base < n_copies; base += kCopiesPerLaunch) {
    const int cnt = n_copies - base < kCopiesPerLaunch ? n_copies - base : kCopiesPerLaunch;
    CopyArgs a = {};
    int64_t max_groups = 0;
    for (int i = 0; i < cnt; ++i) {
      a.src[i] = copies[base + i].src;
      a.dst[i] = copies[base + i].dst;
      a.n[i] = copies[base + i].n;
      const int64_t gr = (a.n[i] + 7) / 8;
      if (gr > max_groups) max_groups = gr;
    }
    if (max_groups == 0) continue;
    // enough workgroups per copy for the largest one, capped (they grid-stride)
    const int64_t gx = (max_groups + 4 * 256 - 1) / (4 * 256);
    const unsigned gridx = (unsigned)(gx < 1024 ? gx : 1024);
    hipLaunchKernelGGL(f16_copy_kernel, dim3(gridx, (unsigned)cnt), dim3(256), 0, stream, a);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace fr
