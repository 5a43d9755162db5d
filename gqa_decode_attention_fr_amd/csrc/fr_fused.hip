// fr_fused.hip -- fused split-KV decode attention for gfx950 (CDNA4).
//
// Operation: FlashRT pull request #185 ("feat(structures): ggml host adapter --
// llama.cpp distribution for pi0.5 on Thor (SM110)"), commit introducing the
// decomposed decode attention: QK^T over one shared f16 KV head, a masked
// softmax accurate to fp32, then PV with an fp32 result in [hd, n_head, n_tok].
// The GQA-collapse commit of the same pull request makes this ONE contraction
// over all n_head*n_tok query rows ordered t-major (row r = t*n_head + h), so
// that row r's output is the contiguous slice out[r*hd .. r*hd + hd).
//
// The pages run the three steps as separate GEMM launches on Thor.  Here the
// three steps run inside one kernel per key split, so the score matrix never
// leaves the chip:
//
//   workgroup = (instance, row block, key split)
//     for each 64-key block of the split:
//       K block  -> LDS as [key][d]           (16-byte coalesced loads)
//       V block  -> LDS transposed [d][key]    (so PV's key-reduction operand is
//                                               contiguous per lane)
//       mask     -> LDS as fp32, pre-multiplied by log2(e); keys past n_kv = -inf
//       each wave, for its 16-row tiles:
//         S^T = K . Q^T        v_mfma_f32_16x16x32_f16, fp32 accumulation
//                              (f32 Q enters as hi + lo f16 halves)
//         online softmax       block max across the 4 lane groups of a row by
//                              cross-lane shuffles, exp2 in fp32
//         O^T += V^T . P^T     v_mfma_f32_16x16x32_f16 with unnormalised f16 P
//     n_split == 1: out = O / l written directly
//     n_split  > 1: (O, m, l) partials; a combine kernel merges them in a fixed
//                   split order (deterministic)
//
// MFMA operand mapping used throughout (16x16 tiles, wave64): the A operand
// lane L supplies row (L % 16), the B operand lane L supplies column (L % 16),
// both with 8 contraction elements per lane indexed by (L / 16, element); the
// accumulator lane L holds rows 4*(L/16) .. +3 of column (L % 16).  Because
// K (or V^T) is the A operand and Q (or P) the B operand, every lane owns one
// query row (L % 16) in both the score and the output accumulators, so the
// softmax statistics and the output rescaling stay lane-local.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "fr_device.h"
#include "fr_internal.h"

namespace fr {
namespace {

struct SplitArgs {
  const void *q;
  const uint16_t *k;
  const uint16_t *v;
  const uint16_t *mask;
  float *out;
  float *part_o;    // [n_inst][n_split][M][hd] unnormalised partial outputs
  float2v *part_ml; // [n_inst][n_split][M] (running max in log2 units, sum)
  int64_t q_stride, kv_stride, mask_stride, out_stride;
  int n_head, n_tok, n_kv, M;
  int n_split, chunk, n_rowblk;
  float scale_log2; // scale * log2(e)
};

template <int HD, int WAVES, int TILES, int QMODE>
__global__ __launch_bounds__(WAVES * 64) void split_kernel(SplitArgs a) {
  constexpr int NT = WAVES * 64;
  constexpr int KSTR = HD + 8;   // halfs per K row in LDS (pad spreads banks)
  constexpr int VSTR = KB + 8;   // halfs per V^T row in LDS
  constexpr int GPR = HD / 8;    // 16-byte granules per K/V row
  constexpr int NK = (KB * GPR + NT - 1) / NT;
  constexpr int NV = ((KB / 4) * GPR + NT - 1) / NT;
  constexpr int NMASK = (kMaxTok * KB + NT - 1) / NT;
  constexpr int KS = HD / 32;    // contraction steps of QK^T
  constexpr int DT = HD / 16;    // 16-wide d tiles of the output

  __shared__ __attribute__((aligned(16))) _Float16 sK[KB * KSTR];
  __shared__ __attribute__((aligned(16))) _Float16 sVt[HD * VSTR];
  __shared__ __attribute__((aligned(16))) float sM[kMaxTok * KB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int g = lane >> 4;

  int bid = blockIdx.x;
  const int split = bid % a.n_split;
  bid /= a.n_split;
  const int rowblk = bid % a.n_rowblk;
  const int inst = bid / a.n_rowblk;

  const uint16_t *kbase = a.k + (int64_t)inst * a.kv_stride;
  const uint16_t *vbase = a.v + (int64_t)inst * a.kv_stride;
  const uint16_t *mbase = a.mask ? a.mask + (int64_t)inst * a.mask_stride : nullptr;
  const int key_begin = split * a.chunk;
  const int key_end = min(key_begin + a.chunk, a.n_kv);
  const int nblk = (key_end - key_begin + KB - 1) / KB;

  // ---- staging registers for the next block (global -> VGPR -> LDS)
  uint4v rk[NK];
  uint4v rv[NV][4];
  uint16_t rm[NMASK];

  auto load_block = [&](int kb0) {
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      const int u = tid + i * NT;
      const int row = u / GPR, c = u % GPR;
      const int key = kb0 + row;
      uint4v val = {0u, 0u, 0u, 0u};
      if (u < KB * GPR && key < key_end)
        val = *(const uint4v *)(kbase + (int64_t)key * HD + c * 8);
      rk[i] = val;
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int u = tid + i * NT;
      const int kq = u / GPR, c = u % GPR;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = kb0 + 4 * kq + e;
        uint4v val = {0u, 0u, 0u, 0u};
        if (u < (KB / 4) * GPR && key < key_end)
          val = *(const uint4v *)(vbase + (int64_t)key * HD + c * 8);
        rv[i][e] = val;
      }
    }
#pragma unroll
    for (int i = 0; i < NMASK; ++i) {
      const int u = tid + i * NT;
      const int t = u / KB, j = u % KB;
      const int key = kb0 + j;
      uint16_t mv = 0xFC00; // -inf: keys outside this split or past n_kv
      if (key < key_end) mv = (mbase && t < a.n_tok) ? mbase[(int64_t)t * a.n_kv + key] : 0;
      rm[i] = mv;
    }
  };

  auto store_block = [&]() {
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      const int u = tid + i * NT;
      if (u < KB * GPR) {
        const int row = u / GPR, c = u % GPR;
        *(uint4v *)(sK + row * KSTR + c * 8) = rk[i];
      }
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int u = tid + i * NT;
      if (u < (KB / 4) * GPR) {
        const int kq = u / GPR, c = u % GPR;
        // rv[i][e] holds V[4kq+e][8c .. 8c+7]; write V^T rows d = 8c+dd with
        // the four keys 4kq .. 4kq+3 packed in one 8-byte store.
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t k0 = rv[i][0][w], k1 = rv[i][1][w];
          const uint32_t k2 = rv[i][2][w], k3 = rv[i][3][w];
          const uint32_t lo01 = (k0 & 0xFFFFu) | (k1 << 16);
          const uint32_t lo23 = (k2 & 0xFFFFu) | (k3 << 16);
          const uint32_t hi01 = (k0 >> 16) | (k1 & 0xFFFF0000u);
          const uint32_t hi23 = (k2 >> 16) | (k3 & 0xFFFF0000u);
          typedef uint32_t uint2v __attribute__((ext_vector_type(2)));
          *(uint2v *)(sVt + (8 * c + 2 * w) * VSTR + 4 * kq) = uint2v{lo01, lo23};
          *(uint2v *)(sVt + (8 * c + 2 * w + 1) * VSTR + 4 * kq) = uint2v{hi01, hi23};
        }
      }
    }
#pragma unroll
    for (int i = 0; i < NMASK; ++i) {
      const int u = tid + i * NT;
      if (u < kMaxTok * KB) sM[u] = (float)bits_to_half(rm[i]) * kLog2e;
    }
  };

  // ---- this wave's query rows: tiles of 16, lane owns row l16 of each tile
  const int tile0 = rowblk * (WAVES * TILES) + wave * TILES;
  const bool wave_active = tile0 * 16 < a.M;

  load_block(key_begin);

  half8 qh[TILES][KS], ql[TILES][KS];
  int tok[TILES];
  const void *qinst = (QMODE == kQF16)
                          ? (const void *)((const uint16_t *)a.q + (int64_t)inst * a.q_stride)
                          : (const void *)((const float *)a.q + (int64_t)inst * a.q_stride);
#pragma unroll
  for (int i = 0; i < TILES; ++i) {
    const int r = (tile0 + i) * 16 + l16;
    const bool rvalid = r < a.M;
    tok[i] = min(r / a.n_head, a.n_tok - 1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      load_q8<QMODE>(qinst, (int64_t)r * HD + ks * 32 + g * 8, rvalid, qh[i][ks], ql[i][ks]);
  }

  float m_run[TILES], l_run[TILES];
  float4v o[TILES][DT];
#pragma unroll
  for (int i = 0; i < TILES; ++i) {
    m_run[i] = -INFINITY;
    l_run[i] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[i][dt] = float4v{0.f, 0.f, 0.f, 0.f};
  }

  for (int b = 0; b < nblk; ++b) {
    if (b > 0) __syncthreads(); // every wave is done reading the previous block
    store_block();
    __syncthreads();
    if (b + 1 < nblk) load_block(key_begin + (b + 1) * KB); // in flight during compute

    if (wave_active) {
      // -- S^T = K . Q^T for the four 16-key tiles kt of this block.  Tile kt
      //    feeds K rows so that lane group g ends up holding keys
      //    32*(kt/2) + 8g + 4*(kt%2) + 0..3: the 8 keys of group g per 32-key
      //    half are then contiguous, matching PV's contraction layout.
      float4v s[TILES][4];
#pragma unroll
      for (int i = 0; i < TILES; ++i)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) s[i][kt] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          const int krow = (kt >> 1) * 32 + (l16 >> 2) * 8 + (kt & 1) * 4 + (l16 & 3);
          const half8 kf = *(const half8 *)(sK + krow * KSTR + ks * 32 + g * 8);
#pragma unroll
          for (int i = 0; i < TILES; ++i) {
            s[i][kt] = mfma16x16x32(kf, qh[i][ks], s[i][kt]);
            if (QMODE == kQHiLo) s[i][kt] = mfma16x16x32(kf, ql[i][ks], s[i][kt]);
          }
        }
      }

      // -- scale, mask, online softmax; pack P^T as the PV B operand
      half8 pb[TILES][2];
#pragma unroll
      for (int i = 0; i < TILES; ++i) {
        const float *mrow = sM + tok[i] * KB;
        float x[16];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const float4v m0 = *(const float4v *)(mrow + 32 * hh + 8 * g);
          const float4v m1 = *(const float4v *)(mrow + 32 * hh + 8 * g + 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x[8 * hh + e] = s[i][2 * hh][e] * a.scale_log2 + m0[e];
            x[8 * hh + 4 + e] = s[i][2 * hh + 1][e] * a.scale_log2 + m1[e];
          }
        }
        float bm = x[0];
#pragma unroll
        for (int e = 1; e < 16; ++e) bm = fmaxf(bm, x[e]);
        bm = fmaxf(bm, __shfl_xor(bm, 16));
        bm = fmaxf(bm, __shfl_xor(bm, 32));
        const float m_new = fmaxf(m_run[i], bm);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = fast_exp2(m_run[i] - m_use);
        m_run[i] = m_new;
        float psum = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = fast_exp2(x[e] - m_use);
          psum += p;
          pb[i][e >> 3][e & 7] = (_Float16)p;
        }
        l_run[i] = l_run[i] * alpha + psum;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[i][dt] *= alpha;
      }

      // -- O^T += V^T . P^T over the two 32-key halves of the block
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const half8 vf = *(const half8 *)(sVt + (dt * 16 + l16) * VSTR + 32 * hh + 8 * g);
#pragma unroll
          for (int i = 0; i < TILES; ++i) o[i][dt] = mfma16x16x32(vf, pb[i][hh], o[i][dt]);
        }
      }
    }
  }

  if (!wave_active) return;

  // ---- finish: full row sums, then either the final output or a partial
#pragma unroll
  for (int i = 0; i < TILES; ++i) {
    float l = l_run[i];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const int r = (tile0 + i) * 16 + l16;
    if (r >= a.M) continue;
    if (a.n_split == 1) {
      const float inv = (l > 0.f) ? 1.f / l : 0.f;
      float *orow = a.out + (int64_t)inst * a.out_stride + (int64_t)r * HD;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) *(float4v *)(orow + dt * 16 + 4 * g) = o[i][dt] * inv;
    } else {
      const int64_t prow = ((int64_t)inst * a.n_split + split) * a.M + r;
      float *po = a.part_o + prow * HD;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) *(float4v *)(po + dt * 16 + 4 * g) = o[i][dt];
      if (g == 0) a.part_ml[prow] = float2v{m_run[i], l};
    }
  }
}

struct CombineArgs {
  const float *part_o;
  const float2v *part_ml;
  float *out;
  int64_t out_stride;
  int M, n_split, n_inst;
};

// One thread per (instance, row, 4 consecutive d): merges the split partials in
// split order.  out = sum_s 2^(m_s - m) O_s / sum_s 2^(m_s - m) l_s, where m is
// the largest m_s; a row with no visible key (m = -inf) is written as zeros.
template <int HD>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  constexpr int Q4 = HD / 4;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)a.n_inst * a.M * Q4;
  if (idx >= total) return;
  const int d4 = (int)(idx % Q4);
  const int64_t rr = idx / Q4;
  const int r = (int)(rr % a.M);
  const int inst = (int)(rr / a.M);
  const int64_t base = (int64_t)inst * a.n_split;

  float m = -INFINITY;
  for (int s = 0; s < a.n_split; ++s) m = fmaxf(m, a.part_ml[(base + s) * a.M + r].x);
  float4v acc = {0.f, 0.f, 0.f, 0.f};
  if (m != -INFINITY) {
    float l = 0.f;
    for (int s = 0; s < a.n_split; ++s) {
      const int64_t prow = (base + s) * a.M + r;
      const float2v ml = a.part_ml[prow];
      const float w = fast_exp2(ml.x - m);
      l += w * ml.y;
      acc += w * *(const float4v *)(a.part_o + prow * HD + 4 * d4);
    }
    acc *= 1.f / l;
  }
  *(float4v *)(a.out + (int64_t)inst * a.out_stride + (int64_t)r * HD + 4 * d4) = acc;
}

typedef void (*SplitFn)(SplitArgs);

template <int HD, int QMODE>
SplitFn pick_split(int waves) {
  constexpr int T = (HD == 256) ? 1 : (HD == 128 ? 2 : 4);
  switch (waves) {
    case 4: return split_kernel<HD, 4, T, QMODE>;
    case 5: return split_kernel<HD, 5, T, QMODE>;
    case 6: return split_kernel<HD, 6, T, QMODE>;
    case 7: return split_kernel<HD, 7, T, QMODE>;
    case 8: return split_kernel<HD, 8, T, QMODE>;
    default: return nullptr;
  }
}

template <int HD>
SplitFn pick_split_q(int qmode, int waves) {
  switch (qmode) {
    case kQHiLo: return pick_split<HD, kQHiLo>(waves);
    case kQF16: return pick_split<HD, kQF16>(waves);
    case kQRound: return pick_split<HD, kQRound>(waves);
    default: return nullptr;
  }
}

}  // namespace

int tiles_per_wave(int hd) { return hd == 256 ? 1 : (hd == 128 ? 2 : 4); }

hipError_t launch_fused(const Problem &p, const Plan &plan, void *workspace, hipStream_t stream) {
  SplitFn fn = nullptr;
  switch (p.hd) {
    case 64: fn = pick_split_q<64>(p.qmode, plan.waves); break;
    case 128: fn = pick_split_q<128>(p.qmode, plan.waves); break;
    case 256: fn = pick_split_q<256>(p.qmode, plan.waves); break;
  }
  if (!fn || plan.tiles != tiles_per_wave(p.hd)) return hipErrorInvalidValue;

  const int M = p.n_head * p.n_tok;
  SplitArgs a;
  a.q = p.q;
  a.k = p.k;
  a.v = p.v;
  a.mask = p.mask;
  a.out = p.out;
  a.q_stride = p.q_stride;
  a.kv_stride = p.kv_stride;
  a.mask_stride = p.mask_stride;
  a.out_stride = p.out_stride;
  a.n_head = p.n_head;
  a.n_tok = p.n_tok;
  a.n_kv = p.n_kv;
  a.M = M;
  a.n_split = plan.n_split;
  a.chunk = plan.chunk;
  a.n_rowblk = plan.n_rowblk;
  a.scale_log2 = (float)((double)p.scale * 1.4426950408889634);
  const size_t part_o_bytes = (size_t)p.n_inst * plan.n_split * M * p.hd * sizeof(float);
  a.part_o = plan.n_split > 1 ? (float *)workspace : nullptr;
  a.part_ml = plan.n_split > 1 ? (float2v *)((char *)workspace + part_o_bytes) : nullptr;

  hipLaunchKernelGGL(fn, dim3(plan.grid), dim3(plan.waves * 64), 0, stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || plan.n_split == 1) return err;

  CombineArgs c;
  c.part_o = a.part_o;
  c.part_ml = a.part_ml;
  c.out = p.out;
  c.out_stride = p.out_stride;
  c.M = M;
  c.n_split = plan.n_split;
  c.n_inst = p.n_inst;
  const int64_t threads = (int64_t)p.n_inst * M * (p.hd / 4);
  const int blocks = (int)((threads + 255) / 256);
  switch (p.hd) {
    case 64: hipLaunchKernelGGL(combine_kernel<64>, dim3(blocks), dim3(256), 0, stream, c); break;
    case 128: hipLaunchKernelGGL(combine_kernel<128>, dim3(blocks), dim3(256), 0, stream, c); break;
    case 256: hipLaunchKernelGGL(combine_kernel<256>, dim3(blocks), dim3(256), 0, stream, c); break;
  }
  return hipGetLastError();
}

}  // namespace fr
