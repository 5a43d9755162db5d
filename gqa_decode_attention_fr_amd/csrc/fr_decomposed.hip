// fr_decomposed.hip -- the three-launch decomposition of decode attention.
//
// FlashRT pull request #185 ("feat(structures): ggml host adapter -- llama.cpp
// distribution for pi0.5 on Thor (SM110)"), decomposed decode attention commit:
// the window runs as a QK^T GEMM, a masked fp32 softmax and a PV GEMM, and the
// GQA-collapse commit turns the per-head GEMMs into single GEMMs over all
// n_head*n_tok t-major query rows.  This file keeps exactly that shape, as
// three kernels with the score and probability matrices in device memory:
//
//   qk_kernel       S[r][j] = scale * q_r . K_j          (fp32, [M][kv_pad])
//   softmax_kernel  P[r][j] = exp(S + mask - max) / sum   (f16, [M][kv_pad]),
//                   one wavefront per row, max and sum by cross-lane shuffles
//   pv_kernel       out[r] = sum_j P[r][j] V_j           (fp32, t-major rows)
//   (sum_kernel     adds the key-split partials of pv_kernel when it is split)
//
// It exists for A/B comparison with the fused split-KV kernel: the S and P
// round trips are exactly the HBM traffic that fusion removes.  Like the fused
// path it works on units (instance, KV head); S, P and the partials are
// indexed by unit and unit row, the inputs and the output by instance and row.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "fr_device.h"
#include "fr_internal.h"

namespace fr {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;

// Keys of instance i that count: the device count clamped to [0, n_kv], or all
// n_kv without counts.  Keys past it are hidden from every token and never read.
__device__ inline int valid_keys(const int32_t *kv_len, int rinst, int n_kv) {
  return kv_len ? min(max(kv_len[rinst], 0), n_kv) : n_kv;
}

struct QkArgs {
  const void *q;
  const uint16_t *k;
  float *s;
  int64_t q_stride, kv_stride, kvh_stride;
  const int32_t *kv_len;   // per-instance valid key counts, or null
  int M, n_kv, kv_pad, n_rowblk, n_kblk;
  int n_kvh, grp, n_head;
  float scale;
};

// HD = 80 runs its contraction over 96 dimensions: K's LDS rows and the query
// fragments are zero past d = 80 (the 16x16x32 MFMA takes 32 at a time).
template <int HD, int TILES, int QMODE>
__global__ __launch_bounds__(kThreads) void qk_kernel(QkArgs a) {
  constexpr int HDP = (HD + 31) / 32 * 32;   // contraction length, padded
  constexpr int KSTR = HDP + 8;
  constexpr int GPR = HDP / 8;
  constexpr int KS = HDP / 32;
  __shared__ __attribute__((aligned(16))) _Float16 sK[KB * KSTR];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  int bid = blockIdx.x;
  const int kblk = bid % a.n_kblk;
  bid /= a.n_kblk;
  const int rowblk = bid % a.n_rowblk;
  const int inst = bid / a.n_rowblk;   // unit
  const int kvh = inst % a.n_kvh, rinst = inst / a.n_kvh;
  const int kb0 = kblk * KB;
  const uint16_t *kbase = a.k + (int64_t)rinst * a.kv_stride + (int64_t)kvh * a.kvh_stride;
  const int n_eff = valid_keys(a.kv_len, rinst, a.n_kv);

  for (int u = tid; u < KB * GPR; u += kThreads) {
    const int row = u / GPR, c = u % GPR;
    uint4v val = {0u, 0u, 0u, 0u};
    if (kb0 + row < n_eff && c * 8 < HD)
      val = *(const uint4v *)(kbase + (int64_t)(kb0 + row) * HD + c * 8);
    *(uint4v *)(sK + row * KSTR + c * 8) = val;
  }
  __syncthreads();

  const int tile0 = rowblk * (kWaves * TILES) + wave * TILES;
  if (tile0 * 16 >= a.M) return;
  const void *qinst = (QMODE == kQF16)
                          ? (const void *)((const uint16_t *)a.q + (int64_t)rinst * a.q_stride)
                          : (const void *)((const float *)a.q + (int64_t)rinst * a.q_stride);
  half8 qh[TILES][KS], ql[TILES][KS];
#pragma unroll
  for (int i = 0; i < TILES; ++i) {
    const int r = (tile0 + i) * 16 + l16;
    const int64_t qrow = r < a.M ? (int64_t)instance_row(r, kvh, a.grp, a.n_head) * HD : 0;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      load_q8<QMODE>(qinst, qrow + ks * 32 + g * 8, r < a.M && ks * 32 + g * 8 < HD, qh[i][ks],
                     ql[i][ks]);
  }
  float4v s[TILES][4];
#pragma unroll
  for (int i = 0; i < TILES; ++i)
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) s[i][kt] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      // lane group g of tile kt holds keys 32*(kt/2) + 8g + 4*(kt%2) + 0..3
      const int krow = (kt >> 1) * 32 + (l16 >> 2) * 8 + (kt & 1) * 4 + (l16 & 3);
      const half8 kf = *(const half8 *)(sK + krow * KSTR + ks * 32 + g * 8);
#pragma unroll
      for (int i = 0; i < TILES; ++i) {
        s[i][kt] = mfma16x16x32(kf, qh[i][ks], s[i][kt]);
        if (QMODE == kQHiLo) s[i][kt] = mfma16x16x32(kf, ql[i][ks], s[i][kt]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < TILES; ++i) {
    const int r = (tile0 + i) * 16 + l16;
    if (r >= a.M) continue;
    float *srow = a.s + ((int64_t)inst * a.M + r) * a.kv_pad + kb0;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      *(float4v *)(srow + 32 * hh + 8 * g) = s[i][2 * hh] * a.scale;
      *(float4v *)(srow + 32 * hh + 8 * g + 4) = s[i][2 * hh + 1] * a.scale;
    }
  }
}

struct SoftmaxArgs {
  const float *s;
  const uint16_t *mask;
  uint16_t *p;
  float *lsum;   // per row: the sum of the row's f16 probabilities as stored
  int64_t mask_stride;
  const int32_t *kv_len;   // per-instance valid key counts, or null
  int M, grp, n_kvh, n_tok, n_kv, kv_pad, rows;   // rows = units * M
};

// One wavefront per query row: the row max (per lane, then a butterfly over
// the 64 lanes), then unnormalised probabilities 2^(x - max) <= 1 as f16, and
// the row sum of exactly those f16 values.  The PV step divides by that sum,
// so numerator and denominator see the same rounded weights: where one key
// dominates a row, the f16 rounding of its weight cancels instead of scaling
// the output.
__global__ __launch_bounds__(kThreads) void softmax_kernel(SoftmaxArgs a) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (row >= a.rows) return;
  // unit row r of unit u = row / M is token r / grp of instance u / n_kvh
  const int inst = row / a.M / a.n_kvh, r = row % a.M, t = r / a.grp;
  const int n_eff = valid_keys(a.kv_len, inst, a.n_kv);
  const float *srow = a.s + (int64_t)row * a.kv_pad;
  const uint16_t *mrow =
      a.mask ? a.mask + (int64_t)inst * a.mask_stride + (int64_t)t * a.n_kv : nullptr;
  auto logit2 = [&](int j) {
    const float mk = mrow ? (float)bits_to_half(mrow[j]) : 0.f;
    return (srow[j] + mk) * kLog2e;
  };
  float m = -INFINITY;
  for (int j = lane; j < n_eff; j += 64) m = fmaxf(m, logit2(j));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  uint16_t *prow = a.p + (int64_t)row * a.kv_pad;
  float l = 0.f;
  for (int j = lane; j < a.kv_pad; j += 64) {
    float pj = 0.f;
    if (j < n_eff && m != -INFINITY) pj = fast_exp2(logit2(j) - m);
    const _Float16 ph = (_Float16)pj;
    l += (float)ph;
    prow[j] = __builtin_bit_cast(uint16_t, ph);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) l += __shfl_xor(l, off);
  if (lane == 0) a.lsum[row] = l;
}

struct PvArgs {
  const uint16_t *p;
  const float *lsum;   // per row: the sum the probabilities are divided by
  const uint16_t *v;
  float *out;
  float *part;
  int64_t kv_stride, kvh_stride, out_stride;
  const int32_t *kv_len;   // per-instance valid key counts, or null
  int M, n_kv, kv_pad, n_rowblk, n_split, chunk;
  int n_kvh, grp, n_head;
};

template <int HD, int TILES>
__global__ __launch_bounds__(kThreads) void pv_kernel(PvArgs a) {
  constexpr int VSTR = KB + 8;
  constexpr int GPR = HD / 8;
  constexpr int DT = HD / 16;
  __shared__ __attribute__((aligned(16))) _Float16 sVt[HD * VSTR];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  int bid = blockIdx.x;
  const int split = bid % a.n_split;
  bid /= a.n_split;
  const int rowblk = bid % a.n_rowblk;
  const int inst = bid / a.n_rowblk;   // unit
  const int kvh = inst % a.n_kvh, rinst = inst / a.n_kvh;
  const uint16_t *vbase = a.v + (int64_t)rinst * a.kv_stride + (int64_t)kvh * a.kvh_stride;
  const int key_begin = split * a.chunk;
  const int key_end = min(key_begin + a.chunk, valid_keys(a.kv_len, rinst, a.n_kv));
  const int tile0 = rowblk * (kWaves * TILES) + wave * TILES;
  const bool active = tile0 * 16 < a.M;

  float4v o[TILES][DT];
#pragma unroll
  for (int i = 0; i < TILES; ++i)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[i][dt] = float4v{0.f, 0.f, 0.f, 0.f};

  for (int kb0 = key_begin; kb0 < key_end; kb0 += KB) {
    __syncthreads();
    for (int u = tid; u < (KB / 4) * GPR; u += kThreads) {
      const int kq = u / GPR, c = u % GPR;
      uint32_t w[4][4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = kb0 + 4 * kq + e;
        uint4v val = {0u, 0u, 0u, 0u};
        if (key < key_end) val = *(const uint4v *)(vbase + (int64_t)key * HD + c * 8);
#pragma unroll
        for (int x = 0; x < 4; ++x) w[e][x] = val[x];
      }
      typedef uint32_t uint2v __attribute__((ext_vector_type(2)));
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        *(uint2v *)(sVt + (8 * c + 2 * x) * VSTR + 4 * kq) =
            uint2v{(w[0][x] & 0xFFFFu) | (w[1][x] << 16), (w[2][x] & 0xFFFFu) | (w[3][x] << 16)};
        *(uint2v *)(sVt + (8 * c + 2 * x + 1) * VSTR + 4 * kq) =
            uint2v{(w[0][x] >> 16) | (w[1][x] & 0xFFFF0000u),
                   (w[2][x] >> 16) | (w[3][x] & 0xFFFF0000u)};
      }
    }
    __syncthreads();
    if (!active) continue;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      half8 pb[TILES];
#pragma unroll
      for (int i = 0; i < TILES; ++i) {
        const int r = (tile0 + i) * 16 + l16;
        uint4v raw = {0u, 0u, 0u, 0u};
        if (r < a.M)
          raw = *(const uint4v *)(a.p + ((int64_t)inst * a.M + r) * a.kv_pad + kb0 + 32 * hh +
                                  8 * g);
        pb[i] = __builtin_bit_cast(half8, raw);
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const half8 vf = *(const half8 *)(sVt + (dt * 16 + l16) * VSTR + 32 * hh + 8 * g);
#pragma unroll
        for (int i = 0; i < TILES; ++i) o[i][dt] = mfma16x16x32(vf, pb[i], o[i][dt]);
      }
    }
  }
  if (!active) return;
#pragma unroll
  for (int i = 0; i < TILES; ++i) {
    const int r = (tile0 + i) * 16 + l16;
    if (r >= a.M) continue;
    if (a.n_split == 1) {
      // (a row with no visible key: sum 0, output 0)
      const float l = a.lsum[(int64_t)inst * a.M + r];
      const float inv = l > 0.f ? 1.f / l : 0.f;
      float *dst = a.out + (int64_t)rinst * a.out_stride +
                   (int64_t)instance_row(r, kvh, a.grp, a.n_head) * HD;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) *(float4v *)(dst + dt * 16 + 4 * g) = o[i][dt] * inv;
    } else {
      float *dst = a.part + (((int64_t)inst * a.n_split + split) * a.M + r) * HD;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) *(float4v *)(dst + dt * 16 + 4 * g) = o[i][dt];
    }
  }
}

struct SumArgs {
  const float *part;
  const float *lsum;
  float *out;
  int64_t out_stride;
  int M, hd, n_split, n_inst;   // n_inst counts units
  int n_kvh, grp, n_head;
};

// out = sum over key splits of the PV partials, in split order, divided by
// the row's probability sum.
__global__ __launch_bounds__(256) void sum_kernel(SumArgs a) {
  const int q4 = a.hd / 4;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)a.n_inst * a.M * q4) return;
  const int d4 = (int)(idx % q4);
  const int64_t rr = idx / q4;
  const int r = (int)(rr % a.M), inst = (int)(rr / a.M);
  float4v acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < a.n_split; ++s)
    acc += *(const float4v *)(a.part + (((int64_t)inst * a.n_split + s) * a.M + r) * a.hd +
                              4 * d4);
  const float l = a.lsum[(int64_t)inst * a.M + r];
  const int64_t orow = (int64_t)(inst / a.n_kvh) * a.out_stride +
                       (int64_t)instance_row(r, inst % a.n_kvh, a.grp, a.n_head) * a.hd;
  *(float4v *)(a.out + orow + 4 * d4) = acc * (l > 0.f ? 1.f / l : 0.f);
}

template <int HD>
void launch_qk(int qmode, dim3 grid, hipStream_t st, const QkArgs &a) {
  constexpr int T = (HD == 256) ? 1 : (HD == 128 ? 2 : 4);   // hd 64 and 80: 4
  switch (qmode) {
    case kQHiLo: hipLaunchKernelGGL((qk_kernel<HD, T, kQHiLo>), grid, dim3(kThreads), 0, st, a); break;
    case kQF16: hipLaunchKernelGGL((qk_kernel<HD, T, kQF16>), grid, dim3(kThreads), 0, st, a); break;
    case kQRound: hipLaunchKernelGGL((qk_kernel<HD, T, kQRound>), grid, dim3(kThreads), 0, st, a); break;
  }
}

template <int HD>
void launch_pv(dim3 grid, hipStream_t st, const PvArgs &a) {
  constexpr int T = (HD == 256) ? 1 : (HD == 128 ? 2 : 4);
  hipLaunchKernelGGL((pv_kernel<HD, T>), grid, dim3(kThreads), 0, st, a);
}

}  // namespace

hipError_t launch_decomposed(const Problem &p, const Plan &plan, void *workspace,
                             hipStream_t stream) {
  const int M = p.unit_rows();
  const int U = p.units();
  const int n_kblk = (p.n_kv + KB - 1) / KB;
  const int kv_pad = n_kblk * KB;
  char *ws = (char *)workspace;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char *ptr = ws + off;
    off += (bytes + 255) & ~(size_t)255;
    return ptr;
  };
  float *part = nullptr;
  if (plan.n_split > 1) part = (float *)take((size_t)U * plan.n_split * M * p.hd * 4);
  float *s = (float *)take((size_t)U * M * kv_pad * 4);
  uint16_t *pm = (uint16_t *)take((size_t)U * M * kv_pad * 2);
  float *lsum = (float *)take((size_t)U * M * 4);
  if (off > plan.ws_bytes) return hipErrorInvalidValue;

  QkArgs qa;
  qa.q = p.q;
  qa.k = p.k;
  qa.s = s;
  qa.q_stride = p.q_stride;
  qa.kv_stride = p.kv_stride;
  qa.kvh_stride = p.kvh_stride;
  qa.n_kvh = p.n_kvh;
  qa.grp = p.grp();
  qa.n_head = p.n_head;
  qa.M = M;
  qa.n_kv = p.n_kv;
  qa.kv_len = p.kv_len;
  qa.kv_pad = kv_pad;
  qa.n_rowblk = plan.n_rowblk;
  qa.n_kblk = n_kblk;
  qa.scale = p.scale;
  hipEvent_t ev0, ev1;
  profile_events(&ev0, &ev1);
  if (ev0 && hipEventRecord(ev0, stream) != hipSuccess) return hipGetLastError();
  const dim3 qgrid(U * plan.n_rowblk * n_kblk);
  switch (p.hd) {
    case 64: launch_qk<64>(p.qmode, qgrid, stream, qa); break;
    case 80: launch_qk<80>(p.qmode, qgrid, stream, qa); break;
    case 128: launch_qk<128>(p.qmode, qgrid, stream, qa); break;
    case 256: launch_qk<256>(p.qmode, qgrid, stream, qa); break;
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;

  SoftmaxArgs sa;
  sa.s = s;
  sa.mask = p.mask;
  sa.p = pm;
  sa.lsum = lsum;
  sa.mask_stride = p.mask_stride;
  sa.M = M;
  sa.grp = p.grp();
  sa.n_kvh = p.n_kvh;
  sa.n_tok = p.n_tok;
  sa.n_kv = p.n_kv;
  sa.kv_len = p.kv_len;
  sa.kv_pad = kv_pad;
  sa.rows = U * M;
  hipLaunchKernelGGL(softmax_kernel, dim3((sa.rows + kWaves - 1) / kWaves), dim3(kThreads), 0,
                     stream, sa);
  err = hipGetLastError();
  if (err != hipSuccess) return err;

  PvArgs pa;
  pa.p = pm;
  pa.lsum = lsum;
  pa.v = p.v;
  pa.out = p.out;
  pa.part = part;
  pa.kv_stride = p.kv_stride;
  pa.kvh_stride = p.kvh_stride;
  pa.out_stride = p.out_stride;
  pa.n_kvh = p.n_kvh;
  pa.grp = p.grp();
  pa.n_head = p.n_head;
  pa.M = M;
  pa.n_kv = p.n_kv;
  pa.kv_len = p.kv_len;
  pa.kv_pad = kv_pad;
  pa.n_rowblk = plan.n_rowblk;
  pa.n_split = plan.n_split;
  pa.chunk = plan.chunk;
  const dim3 pgrid(U * plan.n_rowblk * plan.n_split);
  switch (p.hd) {
    case 64: launch_pv<64>(pgrid, stream, pa); break;
    case 80: launch_pv<80>(pgrid, stream, pa); break;
    case 128: launch_pv<128>(pgrid, stream, pa); break;
    case 256: launch_pv<256>(pgrid, stream, pa); break;
  }
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (plan.n_split == 1) return ev1 ? hipEventRecord(ev1, stream) : hipSuccess;

  SumArgs ua;
  ua.part = part;
  ua.lsum = lsum;
  ua.out = p.out;
  ua.out_stride = p.out_stride;
  ua.M = M;
  ua.hd = p.hd;
  ua.n_split = plan.n_split;
  ua.n_inst = U;
  ua.n_kvh = p.n_kvh;
  ua.grp = p.grp();
  ua.n_head = p.n_head;
  const int64_t threads = (int64_t)U * M * (p.hd / 4);
  hipLaunchKernelGGL(sum_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream,
                     ua);
  err = hipGetLastError();
  if (err == hipSuccess && ev1) err = hipEventRecord(ev1, stream);
  return err;
}

}  // namespace fr
