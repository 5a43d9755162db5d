// fr_qkv.hip -- the query/KV producer ahead of the decode window ("qkv_post").
//
// FlashRT pull request #185 ("feat(structures): ggml host adapter -- llama.cpp
// distribution for pi0.5 on Thor (SM110)"): the prefix QKV window folds the
// epilogue of the q/k/v projections -- RoPE, the query scale and the f16
// materialisations -- into one pass, and its qkv_post handoff commit stores
// the rope'd, scaled query rows as f16 in exactly the t-major order the
// decomposed decode attention reads, so the window needs no gather launch.
//
// RoPE in its NeoX form: for head vector x of a token at position p and
// i < hd/2, the pair (x_i, x_{i+hd/2}) is rotated by a_i = p * base^(-2i/hd).
// The angles are taken in double precision (an fp32 product p * base^(-2i/hd)
// loses ~p * 2^-24 radians, 2e-3 at p = 32768) and their cosine and sine are
// rounded to fp32; the rotations run in fp32 and round to f16 nearest-even.
//
// One workgroup per (token, instance): the token's hd/2 angles into LDS, then
// every query and key head rotated (query heads also scaled) and the value
// heads copied; query rows go to q16, key and value rows to the caches at row
// pos (rows whose position is outside [0, capacity) are not written).

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "fr_device.h"
#include "fr_internal.h"

namespace fr {
namespace {

__device__ __forceinline__ uint16_t f16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (_Float16)x);   // nearest even
}

__global__ __launch_bounds__(256) void qkv_post_kernel(QkvPostArgs a) {
  __shared__ float s_cos[128], s_sin[128];   // hd <= 256
  const int t = blockIdx.x, inst = blockIdx.y;
  const int hd = a.hd, half = hd / 2;
  const int p = a.pos[(int64_t)inst * a.pos_stride + t];
  for (int i = threadIdx.x; i < half; i += blockDim.x) {
    const double ang = (double)p * exp2(-2.0 * (double)i / (double)hd * a.log2_base);
    double sn, cs;
    sincos(ang, &sn, &cs);
    s_cos[i] = (float)cs;
    s_sin[i] = (float)sn;
  }
  __syncthreads();
  const float *row = a.qkv + (int64_t)inst * a.qkv_stride +
                     (int64_t)t * (a.n_head + 2 * a.n_kvh) * hd;
  const bool store_kv = a.k_cache != nullptr && p >= 0 && p < a.capacity;
  const int64_t cache0 = (int64_t)inst * a.cache_stride + (int64_t)p * hd;
  const int n_rot = (a.n_head + a.n_kvh) * half;
  for (int u = threadIdx.x; u < n_rot; u += blockDim.x) {
    const int h = u / half, i = u - h * half;
    const float x0 = row[h * hd + i], x1 = row[h * hd + i + half];
    const float c = s_cos[i], s = s_sin[i];
    float y0 = x0 * c - x1 * s;
    float y1 = x1 * c + x0 * s;
    if (h < a.n_head) {
      y0 *= a.q_scale;
      y1 *= a.q_scale;
      uint16_t *q = a.q16 + (int64_t)inst * a.q16_stride + ((int64_t)t * a.n_head + h) * hd;
      q[i] = f16_bits(y0);
      q[i + half] = f16_bits(y1);
    } else if (store_kv) {
      uint16_t *k = a.k_cache + cache0 + (int64_t)(h - a.n_head) * a.cache_head_stride;
      k[i] = f16_bits(y0);
      k[i + half] = f16_bits(y1);
    }
  }
  if (!store_kv) return;
  const float *vrow = row + (a.n_head + a.n_kvh) * hd;
  for (int u = threadIdx.x; u < a.n_kvh * hd; u += blockDim.x) {
    const int h = u / hd, d = u - h * hd;
    a.v_cache[cache0 + (int64_t)h * a.cache_head_stride + d] = f16_bits(vrow[u]);
  }
}

}  // namespace

hipError_t launch_qkv_post(const QkvPostArgs &a, int n_tok, int n_inst, hipStream_t stream) {
  hipLaunchKernelGGL(qkv_post_kernel, dim3(n_tok, n_inst), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace fr
