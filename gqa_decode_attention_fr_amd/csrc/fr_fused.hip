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
// The pages run the three steps as separate GEMM launches on Thor.  Here they
// run inside one kernel per key split, so scores and probabilities never
// leave the chip:
//
//   workgroup = 4 or 8 waves = (unit, row block, key split); one 16-row query
//   tile per wave.  A unit is one instance's KV head with its group of query
//   heads (with one KV head, the instance); keys past an instance's valid
//   count, when one is given, are neither loaded nor weighed
//   K, V and mask blocks of 64 keys stream global -> LDS with gfx950's 16-byte
//   direct-to-LDS loads (no register staging) into a two-stage ring, so block
//   b+1 is in flight while block b is computed.  Waits are explicit vmcnt
//   counts ahead of a plain s_barrier.
//   each wave, for its tile:
//     S^T = K . Q^T + C   v_mfma_f32_16x16x32_f16, fp32 accumulation; an f32 Q
//                         enters as hi + lo f16 halves (two MFMAs) carrying
//                         scale*log2(e); the accumulator starts from the mask
//                         and minus the row's reference max, so the scores
//                         leave the matrix core as base-2 logits
//     online softmax      a lazy reference max (moved rarely, by a threshold
//                         test and two shuffles), exp2, f16 probabilities
//     O^T += V^T . P^T    V^T operand read with ds_read_b64_tr_b16 straight
//                         from V's natural [key][d] layout; P is unnormalised f16
//   n_split == 1: out = O / l;  n_split > 1: (O, m, l) partials merged by the
//   combine kernel in split order (deterministic).
//
// MFMA operand mapping (16x16 tiles, wave64): A-operand lane L supplies row
// L%16, B-operand lane L column L%16, each with 8 contraction elements indexed
// by (L/16, element); accumulator lane L holds rows 4*(L/16)..+3 of column
// L%16.  K (or V^T) is the A operand and Q (or P) the B operand, so a lane owns
// one query row in both accumulators and the softmax state stays lane-local.
//
// LDS layouts are unpadded and XOR-swizzled at 16-byte granularity: granule c
// of row r sits in slot c ^ swz(r).  The K swizzle makes the 16 rows of one
// score-tile read hit distinct banks; the V swizzle does the same for the four
// rows each 16-lane group touches in a transposing read.

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <utility>

#include "fr_device.h"
#include "fr_internal.h"

namespace fr {
namespace {

// How the mask reaches LDS: not at all (no mask), by 16-byte direct loads
// (rows 16-byte aligned), or through registers two bytes at a time, for up to
// 16 token rows (kMaskReg) or, in the 8-wave shape, 64 (kMaskReg64, which
// needs four times the staging registers).
enum MaskMode { kMaskNone = 0, kMaskDma = 1, kMaskReg = 2, kMaskReg64 = 3 };

// First work item of XCD x when W items are dealt to the 8 XCDs in
// contiguous, balanced ranges (XCDs below W % 8 take one more).
__host__ __device__ __forceinline__ int xcd_item_start(int x, int W) {
  return x * (W >> 3) + min(x, W & 7);
}

// The XCD holding most of the items [k0, k0 + n) (the lowest on a tie).
int xcd_majority(int k0, int n, int W) {
  int best = 0, best_n = -1;
  for (int x = 0; x < 8; ++x) {
    const int lo = std::max(k0, xcd_item_start(x, W));
    const int hi = std::min(k0 + n, xcd_item_start(x + 1, W));
    if (hi - lo > best_n) {
      best_n = hi - lo;
      best = x;
    }
  }
  return best;
}

struct SplitArgs {
  const void *q;
  const uint16_t *k;
  const uint16_t *v;
  const uint16_t *mask;
  const int32_t *kv_len;  // per instance valid key count (device), or null
  float *out;
  float *part_o;    // [units][n_split][M][hd] unnormalised partial outputs
  float2v *part_ml; // [units][n_split][M] (running max in log2 units, sum)
  int64_t q_stride, kv_stride, mask_stride, out_stride;
  int64_t kvh_stride; // elements between the KV heads of one instance
  int n_head, n_tok, n_kv, M;   // n_head: all query heads; M: rows of one unit
  int n_kvh, grp;     // KV heads per instance, query heads per KV head
  int n_split, chunk, n_rowblk;
  int tpr;          // 16-row tiles per row block (<= NW * TPW)
  float scale;      // applied to q.k before the mask
};

typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void global_cvoid;

__device__ __forceinline__ int swz_k(int r, int gpr) {
  return ((r & 3) | (((r >> 3) & 3) << 2)) & (gpr - 1);
}
__device__ __forceinline__ int swz_v(int r, int gpr) {
  return ((2 * (r & 3)) | (((r >> 3) & 1) << 3)) & (gpr - 1);
}
__device__ __forceinline__ int swz_m(int t) { return t & 7; }

// Keeps a computed value where it is: the empty volatile statement cannot move,
// so the arithmetic producing x stays ahead of it instead of being sunk to its
// first use (the softmax steps are placed between MFMA steps on purpose).
template <typename T>
__device__ __forceinline__ void pin(T &x) {
  asm volatile("" : "+v"(x));
}

// 16-byte global -> LDS copy: lane l's bytes land at lds_base + 16*l.
__device__ __forceinline__ void dma16(const void *g, void *lds_base) {
  __builtin_amdgcn_global_load_lds((global_cvoid *)g, (lds_void *)lds_base, 16, 0, 0);
}
// The same from a uniform base plus a 32-bit lane offset, as one load with a
// scalar base register.  The offset passes through an empty statement so the
// compiler cannot hoist a 64-bit per-lane sum out of the loop instead.
__device__ __forceinline__ void dma16(const char *base, uint32_t off, void *lds_base) {
  asm volatile("" : "+v"(off));
  dma16(base + off, lds_base);
}

// 16-byte global load issued as inline assembly: the compiler then inserts no
// wait of its own for the result (it would wait for every outstanding load,
// including the block loads issued after it).  The caller waits with
// wait_vm_tie before anything reads the value.
__device__ __forceinline__ float4v gload16(const void *p) {
  float4v r;
  asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(r) : "v"(p) : "memory");
  return r;
}

// 2-byte global load (zero-extended), inline assembly for the same reason.
__device__ __forceinline__ uint32_t gload_u16(const void *p) {
  uint32_t r;
  asm volatile("global_load_ushort %0, %1, off" : "=v"(r) : "v"(p) : "memory");
  return r;
}

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
// The same, tied to values loaded with gload16 (they cannot be read before it).
template <int N>
__device__ __forceinline__ void wait_vm_tie(float4v &x, float4v &y) {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%2)" : "+v"(x), "+v"(y) : "i"(N));
}

// Workgroup barrier that orders LDS accesses in the compiler without waiting
// on outstanding direct-to-LDS loads (the waits above cover those).
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

__device__ __forceinline__ half4 lds_tr16(const _Float16 *p) {
  typedef __attribute__((__vector_size__(4 * sizeof(__fp16)))) __fp16 fp16x4;
  fp16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4f16(
      (__attribute__((address_space(3))) fp16x4 *)(p));
  return __builtin_bit_cast(half4, v);
}

// Lazy softmax reference: the running max moves only when a block's logits
// exceed it by more than 8 (base-2 units), so unnormalised probabilities stay
// <= 2^8.
constexpr float kLazy2 = 8.f;

// Reductions over the four lanes l, l^16, l^32, l^48 (the four lane groups
// that share one query row) with gfx950's VALU row swaps, no LDS traffic:
// after a self-swap, the two results of a lane hold its own value and its
// partner's (partner = l^32, then l^16).
__device__ __forceinline__ float group_max(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float group_sum(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---- LDS reads of the compute phase, issued as inline assembly.  The
// compiler would otherwise wait for every outstanding direct-to-LDS load
// (including the next block's prefetch) before the first read of a block; the
// explicit vmcnt waits ahead of each barrier already order those loads.  The
// reads complete in issue order, and every consumer waits with lgkmcnt(N) on
// the fragments it uses (tied through the wait, so it cannot move above it).
typedef uint32_t uint2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char *)p;
}
template <int OFF>
__device__ __forceinline__ half8 lds_b128(uint32_t a) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset");
  half8 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(a), "i"(OFF));
  return r;
}
template <int OFF>
__device__ __forceinline__ uint2v lds_tr_b64(uint32_t a) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset");
  uint2v r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(a), "i"(OFF));
  return r;
}
template <int N>
__device__ __forceinline__ void wait_lgkm() {
  asm volatile("s_waitcnt lgkmcnt(%0)" ::"i"(N));
}
template <int N, typename T>
__device__ __forceinline__ void wait_lgkm_tie(T &x) {
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(x) : "i"(N));
}
template <int N, typename T>
__device__ __forceinline__ void wait_lgkm_tie(T &x, T &y) {
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(x), "+v"(y) : "i"(N));
}
template <int N, typename T>
__device__ __forceinline__ void wait_lgkm_tie(T &x, T &y, T &z, T &w) {
  asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(x), "+v"(y), "+v"(z), "+v"(w) : "i"(N));
}

template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
// f(std::integral_constant<int, i>) for i = 0 .. N-1, unrolled at compile time
template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

template <int HD, int NW>
struct Stage {
  _Float16 k[KB * HD];
  _Float16 v[KB * HD];
  uint16_t m[NW * 64 * 8];  // one 16-byte granule per lane: NW*8 token rows of 64 keys
};

// NW waves per workgroup (4 or 8), TPW 16-row tiles per wave.  HD is the
// head size of the LDS layout and the contractions, HDD that of the data in
// memory: hd 80 runs in the hd-128 layout (HDD = 80 < HD = 128).  The granules
// of a K/V row past HDD repeat in-row granules: in the scores they meet the
// query's zero columns (exact zeros), and the output columns past HDD they
// produce are never stored.
template <int HD, int NW, int TPW, int QMODE, int MASKMODE, int HDD = HD>
__global__ __launch_bounds__(NW * 64, 8 / NW) void split_kernel(SplitArgs a) {
  constexpr int kWaves = NW;
  constexpr int kThreads = NW * 64;
  constexpr int GPR = HD / 8;                 // 16-byte granules per K/V row
  constexpr int NJ = GPR / NW;                // K (and V) DMA instructions per wave per block
  constexpr bool kReg = MASKMODE == kMaskReg || MASKMODE == kMaskReg64;
  constexpr int kTok = MASKMODE == kMaskReg ? kMaxTok4 : max_tokens(NW); // token rows staged
  static_assert(MASKMODE != kMaskReg64 || NW == 8, "64 register-staged rows need 8 waves");
  static_assert(kTok * 8 <= NW * 64, "mask stage holds one granule per lane");
  constexpr int NMR = (kTok * KB) / kThreads; // register-path mask loads per thread
  constexpr int NJM = MASKMODE == kMaskDma ? 1 : (kReg ? NMR : 0);
  static_assert(NJ >= 1 && NJ * NW == GPR, "K/V rows split evenly over the waves");
  constexpr int J = 2 * NJ + NJM;             // vector-memory ops per wave per block
  constexpr int KS = HD / 32;
  constexpr int DT = HD / 16;
  constexpr int GPRD = HDD / 8;               // granules of a row in memory
  constexpr int DTD = HDD / 16;               // output tiles of 16 columns stored
  static_assert(HDD <= HD && HDD % 16 == 0 && 2 * GPRD >= GPR, "data row within the layout");

  __shared__ __attribute__((aligned(16))) Stage<HD, NW> stg[2];
  Stage<HD, NW> &st0 = stg[0];
  Stage<HD, NW> &st1 = stg[1];
  // Stage 1 sits a fixed distance after stage 0; where that distance fits the
  // 16-bit immediate offset of an LDS read (hd <= 128), stage-1 reads reuse
  // the stage-0 lane addresses with a larger immediate.
  constexpr int kStageBytes = (int)sizeof(Stage<HD, NW>);
  constexpr bool kImmStage = HD <= 128;
  constexpr int NAS = kImmStage ? 1 : 2;   // lane address sets kept

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform
  const int l16 = lane & 15;
  const int g = lane >> 4;

  // Workgroup -> (unit, key split, row block).  Workgroup b runs on XCD
  // b % 8, and each XCD has its own L2.  Work items k = pair*n_rowblk + rowblk
  // (pair = unit*n_split + split) are dealt to the XCDs in contiguous,
  // balanced ranges (xcd_item_start): the row blocks of a pair, which read the
  // same K/V chunk, and the key splits of a unit, which read the same queries,
  // share an L2 (a unit spans at most two XCDs when it has fewer items than
  // an XCD), and where the combine kernel merges a unit on the XCD that wrote
  // most of its partials, it finds them in that L2.
  const int xcd = blockIdx.x & 7;
  const int item = xcd_item_start(xcd, gridDim.x) + (blockIdx.x >> 3);
  // (integer division runs on the vector unit; the results are uniform and
  // are moved back to scalar registers, so addresses built from them are too)
  const int rowblk = __builtin_amdgcn_readfirstlane(item % a.n_rowblk);
  const int pair = __builtin_amdgcn_readfirstlane(item / a.n_rowblk);
  const int split = __builtin_amdgcn_readfirstlane(pair % a.n_split);
  // the unit (instance, KV head) of this workgroup; its partials are indexed
  // by the unit, its inputs and output by the instance and the KV head
  const int inst = __builtin_amdgcn_readfirstlane(pair / a.n_split);
  const int kvh = __builtin_amdgcn_readfirstlane(inst % a.n_kvh);
  const int rinst = __builtin_amdgcn_readfirstlane(inst / a.n_kvh);

  const int64_t kv_off = (int64_t)rinst * a.kv_stride + (int64_t)kvh * a.kvh_stride;
  const uint16_t *kbase = a.k + kv_off;
  const uint16_t *vbase = a.v + kv_off;
  const uint16_t *mbase = a.mask ? a.mask + (int64_t)rinst * a.mask_stride : nullptr;
  // keys past the instance's valid count (read from device memory, so a
  // replayed graph sees the current value) are hidden and never loaded; n_kv
  // stays the mask's row stride
  const int n_eff = a.kv_len ? __builtin_amdgcn_readfirstlane(
                                   min(max(a.kv_len[rinst], 0), a.n_kv))
                             : a.n_kv;
  const int key_begin = split * a.chunk;
  const int key_end = min(key_begin + a.chunk, n_eff);
  const int nblk = key_end > key_begin ? (key_end - key_begin + KB - 1) / KB : 0;

  if (nblk == 0) {
    // (uniform) no valid key in this split: a zero output (every key of the
    // rows is hidden) or an empty partial that the combine weighs 0
    for (int i = 0; i < TPW; ++i) {
      const int r = (rowblk * a.tpr + wave + kWaves * i) * 16 + l16;
      if (wave + kWaves * i >= a.tpr || r >= a.M) continue;
      const float4v zero = {0.f, 0.f, 0.f, 0.f};
      if (a.n_split == 1) {
        float *orow = a.out + (int64_t)rinst * a.out_stride +
                      (int64_t)instance_row(r, kvh, a.grp, a.n_head) * HDD;
        for (int dt = 0; dt < DTD; ++dt) *(float4v *)(orow + dt * 16 + 4 * g) = zero;
      } else {
        const int64_t prow = ((int64_t)inst * a.n_split + split) * a.M + r;
        for (int dt = 0; dt < DTD; ++dt)
          *(float4v *)(a.part_o + prow * HDD + dt * 16 + 4 * g) = zero;
        if (g == 0) a.part_ml[prow] = float2v{-INFINITY, 0.f};
      }
    }
    return;
  }

  // register-staged mask values (kMaskReg, kMaskReg64), loaded by inline assembly
  // and read only after the wait for their block
  uint32_t rm[2][NMR];

  // Per-lane DMA source byte offsets from the block's first K (V) row, fixed
  // for the whole kernel.  Granule lin = (wave*NJ + j)*64 + lane of a block is
  // K/V row r = lin / GPR, 16-byte slot lin % GPR = lane % GPR; it lands at
  // LDS slot slot ^ swz(r).  Only the block's first key moves between blocks,
  // and it is uniform: each load is a scalar base plus a 32-bit lane offset.
  constexpr int RPI = 64 / GPR;                       // rows per DMA instruction
  uint32_t dma_kofs[NJ], dma_vofs[NJ];
  int dma_row[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int r = (wave * NJ + j) * RPI + lane / GPR;
    const int slot = lane % GPR;
    dma_row[j] = r;
    const int ck = slot ^ swz_k(r, GPR), cv = slot ^ swz_v(r, GPR);   // row granules
    dma_kofs[j] = 2u * (uint32_t)(r * HDD + 8 * (ck < GPRD ? ck : ck - GPRD));
    dma_vofs[j] = 2u * (uint32_t)(r * HDD + 8 * (cv < GPRD ? cv : cv - GPRD));
  }
  // mask granule of this lane: token t = lin / 8, key group (lin % 8) ^ swz_m(t);
  // byte offset < 2^31 (n_tok * n_kv <= 2^30 is checked by the host)
  const int m_lin = wave * 64 + lane;
  const int m_tok = m_lin >> 3;
  const int m_gr = (m_lin & 7) ^ swz_m(m_lin >> 3);
  const uint32_t m_ofs = m_tok < a.n_tok ? 2u * (uint32_t)(m_tok * a.n_kv + 8 * m_gr) : 0u;

  // Issue every load of one 64-key block into stage `s`, in the order K,
  // mask, V: the last NJ vector-memory operations of a wave are its V loads,
  // so a wait for at most NJ outstanding operations has K and the mask.
  // Blocks that reach past the valid keys (at most the last) clamp their rows
  // to a valid one and read the mask granules past them from a valid address
  // (those keys are dropped by the ragged-block handling of the softmax).
  auto issue = [&](Stage<HD, NW> &s, int kb0, uint32_t (&rmr)[NMR]) __attribute__((always_inline)) {
    const bool full = kb0 + KB <= n_eff;
    const char *kb = (const char *)(kbase + (int64_t)kb0 * HDD);   // uniform
    const char *vb = (const char *)(vbase + (int64_t)kb0 * HDD);
    const int last = n_eff - 1 - kb0;                               // last valid row
    uint32_t back[NJ];   // bytes from rows past the valid keys back to the last one
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      back[j] = full ? 0u : 2u * (uint32_t)(max(dma_row[j] - last, 0) * HDD);
      dma16(kb, dma_kofs[j] - back[j], (char *)s.k + (wave * NJ + j) * 1024);
    }
    if (MASKMODE == kMaskDma) {
      const bool ok = m_tok < a.n_tok && (full || kb0 + 8 * m_gr < n_eff);
      dma16((const char *)mbase, ok ? 2u * (uint32_t)kb0 + m_ofs : 0u, (char *)s.m + wave * 1024);
    } else if (kReg) {
#pragma unroll
      for (int i = 0; i < NMR; ++i) {
        const int u = tid + i * kThreads;            // kTok tokens x 64 keys
        const int t = u >> 6, j = u & 63;
        const bool ok = t < a.n_tok && kb0 + j < n_eff;
        rmr[i] = gload_u16(mbase + (ok ? (int64_t)t * a.n_kv + kb0 + j : 0));
      }
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      dma16(vb, dma_vofs[j] - back[j], (char *)s.v + (wave * NJ + j) * 1024);
  };

  // kMaskReg, kMaskReg64: place the register-staged values (after they have arrived).
  // (called after the wait for the block; the empty statements keep every read
  // of the loaded registers after it)
  auto place_mask = [&](Stage<HD, NW> &s, uint32_t (&rmr)[NMR]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NMR; ++i) asm volatile("" : "+v"(rmr[i]));
#pragma unroll
    for (int i = 0; i < NMR; ++i) {
      const int u = tid + i * kThreads;
      const int t = u >> 6, j = u & 63;
      s.m[(t * 8 + ((j >> 3) ^ swz_m(t))) * 8 + (j & 7)] = (uint16_t)rmr[i];
    }
  };

  // ---- query rows of this wave: tile i is tile (wave + kWaves*i) of the row
  // block, which holds tiles rowblk*tpr .. rowblk*tpr + tpr - 1 (the planner
  // balances the row blocks, so tpr may be below NW*TPW)
  const int tile_base = rowblk * a.tpr + wave;
  // a wave with no tile in the block or no row in range skips the arithmetic
  // (it still loads and joins every barrier); inside a wave all TPW tiles are
  // computed, rows past M or past the row block are never stored
  const bool wave_on = wave < a.tpr && tile_base * 16 < a.M;
  // raw query values first; they are split into f16 operands only after the
  // first block has landed, so waiting on them never waits on the prefetch
  float4v qraw[TPW][KS][2];
  bool q_on[TPW];
  const void *qinst = (QMODE == kQF16)
                          ? (const void *)((const uint16_t *)a.q + (int64_t)rinst * a.q_stride)
                          : (const void *)((const float *)a.q + (int64_t)rinst * a.q_stride);
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int tile = tile_base + kWaves * i;
    const int r = tile * 16 + l16;
    const bool in_blk = wave + kWaves * i < a.tpr;   // tile belongs to this row block
    q_on[i] = r < a.M && in_blk;
    // every lane loads (rows out of range read row 0 and are zeroed after the wait)
    const int64_t rbase = q_on[i] ? (int64_t)instance_row(r, kvh, a.grp, a.n_head) * HDD : 0;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      // columns past HDD read the row's start and are zeroed after the wait
      const int64_t off = rbase + (ks * 32 + g * 8 < HDD ? ks * 32 + g * 8 : 0);
      if (QMODE == kQF16) {
        qraw[i][ks][0] = gload16((const uint16_t *)qinst + off);
        qraw[i][ks][1] = float4v{0.f, 0.f, 0.f, 0.f};
      } else {
        qraw[i][ks][0] = gload16((const float *)qinst + off);
        qraw[i][ks][1] = gload16((const float *)qinst + off + 4);
      }
    }
  }
  asm volatile("" ::: "memory"); // query loads are issued before the block loads

  // The queries and block 0 first, alone: every workgroup starts at once, so
  // requesting block 1 as well would make block 0 (and the start of the
  // arithmetic) wait behind the whole machine's block-1 traffic.  The queries
  // land first (they were requested first) and are split into f16 operands
  // while block 0 is still arriving; the scores of block 0 start once K and
  // the mask have landed; its V is waited for between the score and the PV
  // stages, and block 1 is requested then (it loads while block 0 is
  // computed).
  issue(st0, key_begin, rm[0]);
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) wait_vm_tie<J>(qraw[i][ks][0], qraw[i][ks][1]);
  }

  half8 qh[TPW][KS], ql[TPW][KS];
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      // Lanes of rows past the tile's valid rows hold row 0's (finite) values:
      // their scores and outputs are computed and never stored.  Only the
      // columns past HDD (hd 80 in the hd-128 layout) must be zero, as they
      // meet K granules in the scores.
      const float4v zero = {0.f, 0.f, 0.f, 0.f};
      const bool on = q_on[i] && ks * 32 + g * 8 < HDD;
      const float4v x0 = (HDD < HD && !on) ? zero : qraw[i][ks][0];
      const float4v x1 = (HDD < HD && !on) ? zero : qraw[i][ks][1];
      if (QMODE == kQF16) {
        qh[i][ks] = __builtin_bit_cast(half8, x0);
        ql[i][ks] = half8{};
      } else {
        // pairs: hi = f16(x) (round to nearest even, packed), lo = f16(x - hi)
        // with the difference taken exactly in one mixed-precision fma.  The
        // split queries carry scale*log2(e), so the scores come out of the
        // matrix core as base-2 logits; a single rounding (kQRound) stays
        // unscaled, so that it equals the pre-rounded f16 input bit for bit.
        const float qs = QMODE == kQHiLo ? a.scale * kLog2e : 1.f;
        const float x[8] = {x0.x * qs, x0.y * qs, x0.z * qs, x0.w * qs,
                            x1.x * qs, x1.y * qs, x1.z * qs, x1.w * qs};
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const half2v h = __builtin_convertvector(float2v{x[e], x[e + 1]}, half2v);
          qh[i][ks][e] = h.x;
          qh[i][ks][e + 1] = h.y;
          if (QMODE == kQHiLo) {
            // x - hi in one mixed-precision fma per element, hi read as f16
            // from its half of the packed pair (exact: one rounding of an
            // exactly representable difference)
            const uint32_t hp = __builtin_bit_cast(uint32_t, h);
            float2v r;
            asm("v_fma_mix_f32 %0, %1, -1.0, %2 op_sel_hi:[1,0,0]"
                : "=v"(r.x) : "v"(hp), "v"(x[e]));
            asm("v_fma_mix_f32 %0, %1, -1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
                : "=v"(r.y) : "v"(hp), "v"(x[e + 1]));
            const half2v lo = __builtin_convertvector(r, half2v);
            ql[i][ks][e] = lo.x;
            ql[i][ks][e + 1] = lo.y;
          } else {
            ql[i][ks][e] = (_Float16)0.f;
            ql[i][ks][e + 1] = (_Float16)0.f;
          }
        }
      }
    }
  }

  // Online-softmax state of each tile row, in "score units" u: the scores the
  // matrix core produces are base-2 logits times 1/su, where su = 1 for split
  // queries (they carry scale*log2(e)) and su = scale*log2(e) for f16 queries
  // (given as f16, or f32 rounded once).
  //   ref: the reference max (base-2 logit units), 0 until the row has seen a
  //        key (ref_set false), then moved up only by more than kLazy2
  //   cb:  -ref/su, the reference as it enters the score accumulator; cq is
  //        cb in all four elements (the accumulator start of unmasked calls)
  //   thr: a half's logits above it move the reference: kLazy2/su once set,
  //        -inf before (the row's first visible key sets it)
  //   adj: what half 0 moved the reference by, for half 1 of the same block
  //        (its accumulators started from the old reference)
  // lacc: running row sums (all four elements equal); o: unnormalised output
  constexpr bool kScaledQ = QMODE == kQHiLo;
  const float su = kScaledQ ? 1.f : a.scale * kLog2e;
  const float inv_su = kScaledQ ? 1.f : 1.f / su;
  const float mmul = kLog2e * inv_su;    // mask (natural-log units) into score units
  float ref[TPW], cb[TPW], thr[TPW], adj[TPW], alpha[TPW];
  bool ref_set[TPW];
  float4v cq[TPW];
  float4v lacc[TPW];
  float4v o[TPW][DT];
  const half8 kOnes = {(_Float16)1.f, (_Float16)1.f, (_Float16)1.f, (_Float16)1.f,
                       (_Float16)1.f, (_Float16)1.f, (_Float16)1.f, (_Float16)1.f};
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    ref[i] = 0.f;
    cb[i] = 0.f;
    thr[i] = -INFINITY;
    adj[i] = 0.f;
    alpha[i] = 1.f;
    ref_set[i] = false;
    cq[i] = float4v{0.f, 0.f, 0.f, 0.f};
    lacc[i] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[i][dt] = float4v{0.f, 0.f, 0.f, 0.f};
  }

  constexpr int NKO = KS < 4 ? KS : 4;
  constexpr int NVO = DT < 8 ? DT : 8;

  // ---- per-lane LDS byte addresses of the compute phase, for both stages.
  // With the swizzles above, the XOR term of a K read depends on the lane and
  // on ks mod 4 only, and that of a V read on the lane and dt mod 8 only;
  // everything else is a compile-time immediate.
  //   K row of score tile kt, lane q = l16:  32*(kt/2) + 4*(kt%2) + [8*(q/4) + q%4]
  //   K slot of step ks: (4*ks + g) ^ swz_k(row) = 16*(ks/4) + ((4*(ks%4) + g) ^ (q % GPR))
  //   V rows of a transposing read: 32*hh + 4*e + [8*g + q/4]
  //   V slot of tile dt: 16*(dt/8) + ((2*(dt%8) + (q%4)/2) ^ swz_v(row)), swz_v lane-constant
  //   mask granule of token t, half hh: t*8 + ((4*hh + g) ^ swz_m(t))
  uint32_t kaddr_s[NAS][NKO], vaddr_s[NAS][NVO], maddr_s[NAS][TPW][2];
  {
    const int krl = 8 * (l16 >> 2) + (l16 & 3);
    const int qk = l16 & (GPR - 1);
    const int vrl = 8 * g + (l16 >> 2);
    const int sv = swz_v(vrl, GPR);
    const float inv_nh = 1.f / (float)a.grp;
#pragma unroll
    for (int si = 0; si < NAS; ++si) {
      Stage<HD, NW> &st = si ? st1 : st0;
      const uint32_t kb = lds_addr(st.k) + krl * HD * 2;
#pragma unroll
      for (int j = 0; j < NKO; ++j) kaddr_s[si][j] = kb + 16 * ((4 * j + g) ^ qk);
      const uint32_t vb = lds_addr(st.v) + vrl * HD * 2 + 8 * (l16 & 1);
#pragma unroll
      for (int j = 0; j < NVO; ++j) vaddr_s[si][j] = vb + 16 * ((2 * j + ((l16 & 3) >> 1)) ^ sv);
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
        // token of this lane's unit row r = tile*16 + l16: t = r / grp through a
        // float reciprocal (exact: r < 2^15 and the rounding margin is 0.5/grp)
        const int r = (tile_base + kWaves * i) * 16 + l16;
        const int t = min((int)(((float)r + 0.5f) * inv_nh), a.n_tok - 1);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
          maddr_s[si][i][hh] = lds_addr(st.m) + 16 * (t * 8 + ((4 * hh + g) ^ swz_m(t)));
      }
    }
  }

  // block 0's K and mask (its V may still be in flight)
  wait_vm<NJ>();

  // ---- one 64-key block, as a software pipeline over its two 32-key halves.
  // The MFMA work of one half runs while the softmax (VALU) of the other half
  // is issued between its steps, so the two units overlap inside a wave:
  //   A: S^T(h0) = K(h0).Q^T + C(h0)
  //   B: S^T(h1) = K(h1).Q^T + C(h1)   with softmax(h0) steps in between
  //   C: O^T += V^T(h0).P^T(h0)        with softmax(h1) steps in between
  //   D: O^T += V^T(h1).P^T(h1)
  // The score accumulators start from C = mask*log2(e)/su - ref/su (keys past
  // the split's end: -inf), so the matrix core delivers each logit already
  // masked and relative to the reference: the softmax of a half is a
  // threshold test, exp2 and a conversion (the f16-query modes multiply by su
  // first).  Each half updates the state on its own; a rescale of the output
  // (rare: the reference moves only by more than kLazy2) is applied between
  // stages, before the PV of the half that moved it.
  float yv[TPW][8];   // probabilities of the half in flight
  float bmv[TPW];     // largest logit of this lane in the half in flight
  bool moved = false;
  bool pend = false;  // half 0 moved a reference after half 1's accumulators started
  half8 pb[TPW][2];   // P^T of the two halves, the PV B operand

  // Step ST (0..7) of the softmax of half HH for every tile of the wave.
  auto sm_step = [&](auto STEP, auto HH, float4v (&sc)[TPW][4]) __attribute__((always_inline)) {
    constexpr int st = decltype(STEP)::value;
    constexpr int hh = decltype(HH)::value;
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      if constexpr (st == 0) {
        if (hh == 1 && pend) {   // (uniform, rare) half 0 moved the reference
#pragma unroll
          for (int j = 0; j < 2; ++j) sc[i][2 + j] -= adj[i];
        }
      } else if constexpr (st == 1) {
        // keys of tile kt = 2hh+j are 32hh + 8g + 4j + e for e < 4
        const float4v &s0 = sc[i][2 * hh], &s1 = sc[i][2 * hh + 1];
        bmv[i] = fmaxf(fmaxf(fmaxf(s0[0], s0[1]), fmaxf(s0[2], s0[3])),
                       fmaxf(fmaxf(s1[0], s1[1]), fmaxf(s1[2], s1[3])));
        pin(bmv[i]);
      } else if constexpr (st == 2) {
        // The common case costs one compare and a uniform branch.  A move
        // takes the row's largest logit over its four lane groups as the new
        // reference (relative: d); before the row has seen a key its logits
        // are relative to 0 and o, lacc are still zero.
        const bool mv = bmv[i] > thr[i];
        if (__any(mv)) {
          const float rm = group_max(bmv[i]);
          const bool mvr = rm > thr[i];
          const float d = mvr ? rm : 0.f;
#pragma unroll
          for (int j = 0; j < 2; ++j) sc[i][2 * hh + j] -= d;
          alpha[i] = (mvr && ref_set[i]) ? fast_exp2(-d * su) : 1.f;
          ref[i] += d * su;
          ref_set[i] = ref_set[i] || mvr;
          thr[i] = ref_set[i] ? kLazy2 * inv_su : -INFINITY;
          cb[i] = -ref[i] * inv_su;
          cq[i] = float4v{cb[i], cb[i], cb[i], cb[i]};
          if (hh == 0) {
            adj[i] = d;
            pend = true;
          }
          moved = true;
        }
      } else if constexpr (st <= 5) {
        // exp2 of the 8 logits over three steps (3, 3, 2)
        constexpr int e0 = 3 * (st - 3), e1 = e0 + 3 < 8 ? e0 + 3 : 8;
#pragma unroll
        for (int e = e0; e < e1; ++e) {
          const float x = sc[i][2 * hh + e / 4][e % 4];
          yv[i][e] = fast_exp2(kScaledQ ? x : x * su);
          pin(yv[i][e]);
        }
      } else {
        constexpr int e0 = 4 * (st - 6);
#pragma unroll
        for (int e = e0; e < e0 + 4; ++e) pb[i][hh][e] = (_Float16)yv[i][e];
        if constexpr (st == 7) pin(pb[i][hh]);
      }
    }
  };

  // Output rescale after a half that moved some reference max.
  auto rescale = [&]() __attribute__((always_inline)) {
    if (moved) {   // wave-uniform
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[i][dt] *= alpha[i];
        lacc[i] *= alpha[i];
        alpha[i] = 1.f;
      }
    }
    moved = false;
  };

  // Called by every wave (a wave without rows skips the arithmetic but joins
  // the barrier of the first block).
  auto compute = [&](auto SI, int kb0, bool first) __attribute__((always_inline)) {
    constexpr int si = decltype(SI)::value;
    const bool ragged = kb0 + KB > key_end;
    constexpr int asi = kImmStage ? 0 : si;              // lane address set
    constexpr int SOFF = kImmStage ? si * kStageBytes : 0; // extra immediate offset
    const uint32_t(&kaddr)[NKO] = kaddr_s[asi];
    const uint32_t(&vaddr)[NVO] = vaddr_s[asi];

    // mask values of half HH: read ahead of the stage whose first LDS wait
    // covers them (half 0 before stage A, half 1 before stage B); they are
    // consumed by that stage's accumulator start
    half8 mh[TPW][2];
    auto mread = [&](auto HH) __attribute__((always_inline)) {
      constexpr int hh = decltype(HH)::value;
      if (MASKMODE != kMaskNone) {
#pragma unroll
        for (int i = 0; i < TPW; ++i) mh[i][hh] = lds_b128<SOFF>(maddr_s[asi][i][hh]);
      }
    };
    mread(std::integral_constant<int, 0>{});
    pend = false;
#pragma unroll
    for (int i = 0; i < TPW; ++i) adj[i] = 0.f;

    // Score accumulators and their start for half HH: the mask term and minus
    // the reference, in score units; keys past the split's end start at -inf.
    // Called after the wait that covers the half's mask read (the empty
    // statement keeps every read of the mask registers after that wait).
    float4v sc[TPW][4];
    auto cinit = [&](auto HH) __attribute__((always_inline)) {
      constexpr int hh = decltype(HH)::value;
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
        if constexpr (MASKMODE != kMaskNone) asm volatile("" : "+v"(mh[i][hh]));
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          float4v c = cq[i];
          if constexpr (MASKMODE != kMaskNone) {
#pragma unroll
            for (int e = 0; e < 4; ++e) c[e] = fmaf((float)mh[i][hh][4 * j + e], mmul, cb[i]);
          }
          if (ragged) {   // uniform: only the block holding the split's end
            const int k0 = kb0 + 32 * hh + 8 * g + 4 * j;
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (k0 + e >= key_end) c[e] = -INFINITY;
          }
          sc[i][2 * hh + j] = c;
        }
      }
    };

    // LDS prefetch distance (steps ahead) of the K and V fragment reads:
    // deeper where the register budget allows (one tile per wave; at hd 256
    // only with one wave per SIMD).  Measured: 2 beats 1 at hd 256 (one wave
    // per SIMD waits on each step's reads otherwise); 3 does not beat 2.
    constexpr int PD = (TPW == 1 && (HD <= 128 || NW == 4)) ? 2 : 1;

    // S^T for half HH: K tiles kt = 2HH, 2HH+1 (keys 32HH + 8g + 4(kt%2) + 0..3
    // in lane group g), fragments read PD steps ahead of their MFMAs; the
    // accumulators start after the first wait.  after(ks) runs after the
    // MFMAs of step ks.
    auto qk_half = [&](auto HH, auto after) __attribute__((always_inline)) {
      constexpr int hh = decltype(HH)::value;
      half8 kb[PD + 1][2];
      auto kread = [&](auto KSI) __attribute__((always_inline)) {
        constexpr int ks = decltype(KSI)::value;
        kb[ks % (PD + 1)][0] = lds_b128<SOFF + 256 * (ks >> 2) + (32 * hh) * HD * 2>(kaddr[ks & 3]);
        kb[ks % (PD + 1)][1] =
            lds_b128<SOFF + 256 * (ks >> 2) + (32 * hh + 4) * HD * 2>(kaddr[ks & 3]);
      };
      static_for<(PD < KS ? PD : KS)>([&](auto KSI) __attribute__((always_inline)) { kread(KSI); });
      static_for<KS>([&](auto KSI) __attribute__((always_inline)) {
        constexpr int ks = decltype(KSI)::value;
        if constexpr (ks + PD < KS) kread(std::integral_constant<int, ks + PD>{});
        // reads issued after those of step ks: 2 per later step in flight
        constexpr int later = (KS - 1 - ks < PD ? KS - 1 - ks : PD);
        wait_lgkm_tie<2 * later>(kb[ks % (PD + 1)][0], kb[ks % (PD + 1)][1]);
        if constexpr (ks == 0) cinit(HH);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
#pragma unroll
          for (int i = 0; i < TPW; ++i) {
            const half8 kf = kb[ks % (PD + 1)][j];
            sc[i][2 * hh + j] = mfma16x16x32(kf, qh[i][ks], sc[i][2 * hh + j]);
            if (QMODE == kQHiLo) sc[i][2 * hh + j] = mfma16x16x32(kf, ql[i][ks], sc[i][2 * hh + j]);
          }
        }
        after(KSI);
      });
    };

    // O^T += V^T . P^T for half HH; each transposing read gives lane (q, g) the
    // keys 32HH + 8g + 4e + 0..3 of column d = 16dt + q, the key order of P.
    auto pv_half = [&](auto HH, auto after) __attribute__((always_inline)) {
      constexpr int hh = decltype(HH)::value;
      uint2v vr[PD + 1][2];
      auto vread = [&](auto DTI) __attribute__((always_inline)) {
        constexpr int dt = decltype(DTI)::value;
        constexpr int off = SOFF + 256 * (dt >> 3) + 32 * hh * HD * 2;
        vr[dt % (PD + 1)][0] = lds_tr_b64<off>(vaddr[dt & 7]);
        vr[dt % (PD + 1)][1] = lds_tr_b64<off + 4 * HD * 2>(vaddr[dt & 7]);
      };
      static_for<(PD < DT ? PD : DT)>([&](auto DTI) __attribute__((always_inline)) { vread(DTI); });
      static_for<DT>([&](auto DTI) __attribute__((always_inline)) {
        constexpr int dt = decltype(DTI)::value;
        if constexpr (dt + PD < DT) vread(std::integral_constant<int, dt + PD>{});
        constexpr int later = (DT - 1 - dt < PD ? DT - 1 - dt : PD);
        wait_lgkm_tie<2 * later>(vr[dt % (PD + 1)][0], vr[dt % (PD + 1)][1]);
        const half4 v0 = __builtin_bit_cast(half4, vr[dt % (PD + 1)][0]);
        const half4 v1 = __builtin_bit_cast(half4, vr[dt % (PD + 1)][1]);
        const half8 vf = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
#pragma unroll
        for (int i = 0; i < TPW; ++i) o[i][dt] = mfma16x16x32(vf, pb[i][hh], o[i][dt]);
        if constexpr (dt == 0) {
          // row sums of the f16 probabilities on the matrix core: an all-ones
          // A operand puts sum_k P[k][row] in every element of lacc
#pragma unroll
          for (int i = 0; i < TPW; ++i) lacc[i] = mfma16x16x32(kOnes, pb[i][hh], lacc[i]);
        }
        after(DTI);
      });
    };

    using H0 = std::integral_constant<int, 0>;
    using H1 = std::integral_constant<int, 1>;
    if (wave_on) {
    // A
    qk_half(H0{}, [&](auto) __attribute__((always_inline)) {});
    mread(std::integral_constant<int, 1>{});
    // B: softmax steps [8ks/KS, 8(ks+1)/KS) of half 0 after QK step ks of half 1
    qk_half(H1{}, [&](auto KSI) __attribute__((always_inline)) {
      constexpr int ks = decltype(KSI)::value;
      static_for<8>([&](auto STI) __attribute__((always_inline)) {
        constexpr int stp = decltype(STI)::value;
        if constexpr (stp * KS >= 8 * ks && stp * KS < 8 * (ks + 1))
          sm_step(STI, H0{}, sc);
      });
    });
    rescale();
    }
    if (first) {   // uniform: block 0's V, then the request for block 1
      wait_vm<0>();
      barrier();
      if (nblk > 1) issue(st1, key_begin + KB, rm[1]);
    }
    if (wave_on) {
    // C: softmax steps of half 1 after PV step dt of half 0
    pv_half(H0{}, [&](auto DTI) __attribute__((always_inline)) {
      constexpr int dt = decltype(DTI)::value;
      static_for<8>([&](auto STI) __attribute__((always_inline)) {
        constexpr int stp = decltype(STI)::value;
        if constexpr (stp * DT >= 8 * dt && stp * DT < 8 * (dt + 1))
          sm_step(STI, H1{}, sc);
      });
    });
    rescale();
    // D
    pv_half(H1{}, [&](auto) __attribute__((always_inline)) {});
    }
  };


  // ---- main loop: two blocks per trip, st0 then st1.  Invariant at the top
  // of a trip: block b is complete in st0 (for b = 0: all but its V) and only
  // block b+1 (into st1) may still be in flight, so reads of st0 never wait on
  // the prefetch; the wait for the next block is taken at the point it is
  // needed.
  for (int b = 0; b < nblk; b += 2) {
    if (kReg) {
      place_mask(st0, rm[0]);
      wait_lgkm<0>();
    }
    barrier();
    compute(std::integral_constant<int, 0>{}, key_begin + b * KB, b == 0);
    barrier();
    if (b + 2 < nblk) issue(st0, key_begin + (b + 2) * KB, rm[0]);
    if (b + 1 >= nblk) break;
    if (b + 2 < nblk) wait_vm<J>(); else wait_vm<0>();   // block b+1 landed
    if (kReg) {
      place_mask(st1, rm[1]);
      wait_lgkm<0>();
    }
    barrier();
    compute(std::integral_constant<int, 1>{}, key_begin + (b + 1) * KB, false);
    barrier();
    if (b + 3 < nblk) {
      issue(st1, key_begin + (b + 3) * KB, rm[1]);
      wait_vm<J>();                                       // block b+2 landed
    } else {
      wait_vm<0>();
    }
  }

  // ---- finish.  n_split == 1: out = O / l.  n_split > 1: the unnormalised
  // partial and its (max, sum).  Stored straight from the accumulators, a
  // wave's store covers 16 rows x 64 bytes (a lane holds 4 columns of one
  // row); partials instead leave through LDS, so that every store writes
  // whole rows (pi0.5 step -0.4 us per call, causal tail -0.7, long context
  // -1.0).  The stages are free: every wave has passed the barrier after its
  // last block, and no load is in flight.  (The register-staged mask kernels,
  // for unaligned masks only, keep the direct stores.)
  if (a.n_split == 1 || kReg) {
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      if (!wave_on) break;
      const float l = lacc[i][0];
      const int r = (tile_base + kWaves * i) * 16 + l16;
      if (r >= a.M || wave + kWaves * i >= a.tpr) continue;
      if (a.n_split == 1) {
        const float inv = (l > 0.f) ? 1.f / l : 0.f;   // (a row with no key: 0)
        float *orow = a.out + (int64_t)rinst * a.out_stride +
                      (int64_t)instance_row(r, kvh, a.grp, a.n_head) * HDD;
#pragma unroll
        for (int dt = 0; dt < DTD; ++dt) *(float4v *)(orow + dt * 16 + 4 * g) = o[i][dt] * inv;
      } else {
        const int64_t prow = ((int64_t)inst * a.n_split + split) * a.M + r;
        float *po = a.part_o + prow * HDD;
#pragma unroll
        for (int dt = 0; dt < DTD; ++dt)
          __builtin_nontemporal_store(o[i][dt], (float4v *)(po + dt * 16 + 4 * g));
        if (g == 0) a.part_ml[prow] = float2v{ref_set[i] ? ref[i] : -INFINITY, l};
      }
    }
    return;
  }
  constexpr int OS = HD + 4;              // padded row: a wave's 16 rows hit different banks
  static_assert(NW * TPW * 16 * OS * 4 <= (int)sizeof(stg), "the tiles fit the stages");
  float *tiles = reinterpret_cast<float *>(&stg[0]);
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    if (!wave_on) break;
    float *t = tiles + (wave * TPW + i) * 16 * OS;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) *(float4v *)(t + l16 * OS + dt * 16 + 4 * g) = o[i][dt];
  }
  // each wave reads back only its own tiles
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    if (!wave_on) break;
    if (wave + kWaves * i >= a.tpr) continue;
    const int tile = tile_base + kWaves * i;
    const float *t = tiles + (wave * TPW + i) * 16 * OS;
    constexpr int C4 = HD / 4;            // float4 per row
    constexpr int PER = 16 * C4 / 64;     // float4 per lane per tile
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int e = k * 64 + lane;
      const int q = e / C4, c = e % C4;
      const int r = tile * 16 + q;
      if (r >= a.M || 4 * c >= HDD) continue;
      const int64_t prow = ((int64_t)inst * a.n_split + split) * a.M + r;
      // streaming stores: the partials are read once, by the combine kernel
      __builtin_nontemporal_store(*(const float4v *)(t + q * OS + 4 * c),
                                  (float4v *)(a.part_o + prow * HDD + 4 * c));
    }
    const int r = tile * 16 + l16;
    if (g == 0 && r < a.M) {
      const int64_t prow = ((int64_t)inst * a.n_split + split) * a.M + r;
      // reference in base-2 units (-inf: the row saw no key, weight 0)
      a.part_ml[prow] = float2v{ref_set[i] ? ref[i] : -INFINITY, lacc[i][0]};
    }
  }
}

struct CombineArgs {
  const float *part_o;
  const float2v *part_ml;
  float *out;
  int64_t out_stride;
  int M, n_split, n_inst;   // n_inst counts units (instance, KV head)
  int n_kvh, grp, n_head;
  // XCD-local merging (the kernel's LOCAL instance): the workgroups on XCD x
  // (workgroup b runs on XCD b % 8) merge units [ub[x], ub[x+1]), wpu
  // workgroups per unit; else the rows of all units are dealt out in order.
  int xcd_local, wpu;
  int ub[9];
};

// NT threads = RW rows x G split groups x (HD/4) columns of 4 consecutive d,
// with G * RW * HD/4 = NT (128 or 256).  Thread (row, g, c) merges splits g, g+G, g+2G, ...
// (R of its loads in flight together); with G > 1 the G group results of a row
// are then merged in group order through LDS.  Few splits take G = 1 and several
// rows per workgroup, so every load of a row is in flight at once and no LDS
// merge is needed.  With m the running max (log2 units):
//   out = sum_s 2^(m_s - m) O_s / sum_s 2^(m_s - m) l_s
// A split with no visible key has m_s = -inf and weight 0; a row with no
// visible key at all is written as zeros.  The merge order is fixed, so the
// result does not depend on timing.
template <int HD, int G, int NT, bool LOCAL>
__global__ __launch_bounds__(NT) void combine_kernel(CombineArgs a) {
  constexpr int C = HD / 4;          // float4 columns per row
  constexpr int RW = NT / (C * G);   // rows per workgroup
  static_assert(RW >= 1 && RW * G * C == NT, "thread layout");
  constexpr int R = 8;               // loads in flight per thread per round
  __shared__ float4v s_acc[G > 1 ? RW : 1][G][C];
  __shared__ float s_m[G > 1 ? RW : 1][G][C], s_l[G > 1 ? RW : 1][G][C];

  const int c = threadIdx.x % C;
  const int g = (threadIdx.x / C) % G;
  const int rw = threadIdx.x / (C * G);
  bool on;
  int r, inst;
  if (LOCAL) {
    const int xcd = blockIdx.x & 7, jx = blockIdx.x >> 3;
    const int unit = a.ub[xcd] + jx / a.wpu;
    const int row = (jx % a.wpu) * RW + rw;        // row of the unit
    on = unit < a.ub[xcd + 1] && row < a.M;
    r = on ? row : 0;
    inst = on ? unit : 0;
  } else {
    const int row = blockIdx.x * RW + rw;          // over units * M
    on = row < a.n_inst * a.M;
    r = on ? row % a.M : 0;
    inst = on ? row / a.M : 0;
  }
  const int64_t base = (int64_t)inst * a.n_split;

  float m = -INFINITY, l = 0.f;
  float4v acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = g; on && s0 < a.n_split; s0 += G * R) {
    float2v ml[R];
    float4v po[R];
#pragma unroll
    for (int j = 0; j < R; ++j) {
      ml[j] = float2v{-INFINITY, 0.f};
      po[j] = float4v{0.f, 0.f, 0.f, 0.f};
      const int sp = s0 + j * G;
      if (sp < a.n_split) {
        const int64_t prow = (base + sp) * a.M + r;
        ml[j] = a.part_ml[prow];
        // each partial is read once: merged on the XCD that wrote it, an
        // ordinary load finds it in that L2; otherwise a streaming load
        // (measured: pi0.5 step -0.5 us with ordinary loads XCD-locally;
        // long context +2.2 us and the prefill +2.9 with them elsewhere)
        const float4v *src = (const float4v *)(a.part_o + prow * HD + 4 * c);
        if constexpr (LOCAL)
          po[j] = *src;
        else
          po[j] = __builtin_nontemporal_load(src);
      }
    }
    float mc = m;
#pragma unroll
    for (int j = 0; j < R; ++j) mc = fmaxf(mc, ml[j].x);
    if (mc == -INFINITY) continue;
    const float k = fast_exp2(m - mc);   // 0 while m = -inf
    l *= k;
    acc *= k;
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const float w = fast_exp2(ml[j].x - mc);   // 0 for a split with no visible key
      l += w * ml[j].y;
      acc += w * po[j];
    }
    m = mc;
  }
  if constexpr (G > 1) {
    s_acc[rw][g][c] = acc;
    s_m[rw][g][c] = m;
    s_l[rw][g][c] = l;
    __syncthreads();
    if (g != 0) return;
    float mm = -INFINITY;
#pragma unroll
    for (int j = 0; j < G; ++j) mm = fmaxf(mm, s_m[rw][j][c]);
    acc = float4v{0.f, 0.f, 0.f, 0.f};
    l = 0.f;
    if (mm != -INFINITY) {
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const float w = fast_exp2(s_m[rw][j][c] - mm);
        l += w * s_l[rw][j][c];
        acc += w * s_acc[rw][j][c];
      }
    }
  }
  if (!on) return;
  const float4v out = (l > 0.f) ? acc * (1.f / l) : float4v{0.f, 0.f, 0.f, 0.f};
  // streaming store: the output is not read again by this call
  const int kvh = inst % a.n_kvh;
  const int64_t orow = (int64_t)(inst / a.n_kvh) * a.out_stride +
                       (int64_t)instance_row(r, kvh, a.grp, a.n_head) * HD;
  __builtin_nontemporal_store(out, (float4v *)(a.out + orow + 4 * c));
}

// Split groups of the combine: enough that each thread has at most R = 8 splits
// to load, and no more (more groups mean fewer rows per workgroup).  Where the
// groups of one row fit in 128 threads and that gives fewer than 1024
// workgroups, workgroups of 128 threads (twice as many: pi0.5 step -0.22 us
// per call, f16-Q -0.38); else 256 (larger grids, such as a prefill's, were
// slower with 128).
template <int HD>
hipError_t launch_combine(CombineArgs c, hipStream_t stream) {
  constexpr int C = HD / 4;
  const int rows = c.n_inst * c.M;
  // workgroups for RW rows each: one per RW rows in order, or, XCD-local,
  // 8 x (most units on one XCD) x (workgroups per unit), some of them idle
  auto grid = [&](int RW) {
    if (!c.xcd_local) return (rows + RW - 1) / RW;
    c.wpu = (c.M + RW - 1) / RW;
    int most = 0;
    for (int x = 0; x < 8; ++x) most = std::max(most, c.ub[x + 1] - c.ub[x]);
    return 8 * most * c.wpu;
  };
  auto go = [&](auto GI) {
    constexpr int GN = decltype(GI)::value;   // split groups wanted
    if constexpr ((C & (C - 1)) != 0) {
      // hd 80: 20 columns; workgroups of 160 threads (320 for 16 groups)
      constexpr int NT = GN * C <= 160 ? 160 : 320;
      constexpr int RW = NT / (C * GN);
      const int wgs = grid(RW);
      if (c.xcd_local)
        hipLaunchKernelGGL((combine_kernel<HD, GN, NT, true>), dim3(wgs), dim3(NT), 0, stream, c);
      else
        hipLaunchKernelGGL((combine_kernel<HD, GN, NT, false>), dim3(wgs), dim3(NT), 0, stream, c);
      return hipGetLastError();
    } else {
      if constexpr (GN * C <= 128) {
        constexpr int RW = 128 / (C * GN);
        if ((rows + RW - 1) / RW < 1024) {
          const int wgs = grid(RW);
          if (c.xcd_local)
            hipLaunchKernelGGL((combine_kernel<HD, GN, 128, true>), dim3(wgs), dim3(128), 0, stream, c);
          else
            hipLaunchKernelGGL((combine_kernel<HD, GN, 128, false>), dim3(wgs), dim3(128), 0, stream, c);
          return hipGetLastError();
        }
      }
      constexpr int G = GN < 256 / C ? GN : 256 / C;
      constexpr int RW = 256 / (C * G);
      const int wgs = grid(RW);
      if (c.xcd_local)
        hipLaunchKernelGGL((combine_kernel<HD, G, 256, true>), dim3(wgs), dim3(256), 0, stream, c);
      else
        hipLaunchKernelGGL((combine_kernel<HD, G, 256, false>), dim3(wgs), dim3(256), 0, stream, c);
      return hipGetLastError();
    }
  };
  const int need = (c.n_split + 7) / 8;   // groups that give each thread <= 8 splits
  if (need <= 1) return go(std::integral_constant<int, 1>{});
  if (need <= 2) return go(std::integral_constant<int, 2>{});
  if (need <= 4) return go(std::integral_constant<int, 4>{});
  if (need <= 8) return go(std::integral_constant<int, 8>{});
  return go(std::integral_constant<int, 16>{});
}

typedef void (*SplitFn)(SplitArgs);

template <int HD, int NW, int TPW, int QMODE, int HDD>
SplitFn pick_mask(int mm) {
  switch (mm) {
    case kMaskNone: return split_kernel<HD, NW, TPW, QMODE, kMaskNone, HDD>;
    case kMaskDma: return split_kernel<HD, NW, TPW, QMODE, kMaskDma, HDD>;
    case kMaskReg: return split_kernel<HD, NW, TPW, QMODE, kMaskReg, HDD>;
    case kMaskReg64:
      if constexpr (NW == 8) return split_kernel<HD, NW, TPW, QMODE, kMaskReg64, HDD>;
      return nullptr;
    default: return nullptr;
  }
}

template <int HD, int NW, int TPW, int HDD>
SplitFn pick_q(int qmode, int mm) {
  switch (qmode) {
    case kQHiLo: return pick_mask<HD, NW, TPW, kQHiLo, HDD>(mm);
    case kQF16: return pick_mask<HD, NW, TPW, kQF16, HDD>(mm);
    case kQRound: return pick_mask<HD, NW, TPW, kQRound, HDD>(mm);
    default: return nullptr;
  }
}

// Instantiated shapes: 4 or 8 waves, one 16-row tile per wave.
template <int HD, int HDD = HD>
SplitFn pick_shape(int nw, int tpw, int qmode, int mm) {
  if (nw == 4 && tpw == 1) return pick_q<HD, 4, 1, HDD>(qmode, mm);
  if (nw == 8 && tpw == 1) return pick_q<HD, 8, 1, HDD>(qmode, mm);
  return nullptr;
}

}  // namespace

hipError_t launch_fused(const Problem &p, const Plan &plan, void *workspace, hipStream_t stream) {
  int mm = kMaskNone;
  if (p.mask) {
    const bool vec = (p.n_kv % 8 == 0) && ((uintptr_t)p.mask % 16 == 0) &&
                     (p.n_inst == 1 || p.mask_stride % 8 == 0);
    mm = vec ? kMaskDma : (p.n_tok > kMaxTok4 ? kMaskReg64 : kMaskReg);
  }
  SplitFn fn = nullptr;
  switch (p.hd) {
    case 64: fn = pick_shape<64>(plan.waves, plan.tiles, p.qmode, mm); break;
    case 80: fn = pick_shape<128, 80>(plan.waves, plan.tiles, p.qmode, mm); break;
    case 128: fn = pick_shape<128>(plan.waves, plan.tiles, p.qmode, mm); break;
    case 256: fn = pick_shape<256>(plan.waves, plan.tiles, p.qmode, mm); break;
  }
  if (!fn || (p.mask && p.n_tok > max_tokens(plan.waves))) return hipErrorInvalidValue;
  if (mm == kMaskReg && p.n_tok > kMaxTok4) return hipErrorInvalidValue;

  const int M = p.unit_rows();
  SplitArgs a;
  a.q = p.q;
  a.k = p.k;
  a.v = p.v;
  a.mask = p.mask;
  a.kv_len = p.kv_len;
  a.out = p.out;
  a.q_stride = p.q_stride;
  a.kv_stride = p.kv_stride;
  a.mask_stride = p.mask_stride;
  a.out_stride = p.out_stride;
  a.kvh_stride = p.kvh_stride;
  a.n_head = p.n_head;
  a.n_tok = p.n_tok;
  a.n_kv = p.n_kv;
  a.M = M;
  a.n_kvh = p.n_kvh;
  a.grp = p.grp();
  a.n_split = plan.n_split;
  a.chunk = plan.chunk;
  a.n_rowblk = plan.n_rowblk;
  a.tpr = plan.tpr;
  a.scale = p.scale;
  const size_t part_o_bytes = (size_t)p.units() * plan.n_split * M * p.hd * sizeof(float);
  a.part_o = plan.n_split > 1 ? (float *)workspace : nullptr;
  a.part_ml = plan.n_split > 1 ? (float2v *)((char *)workspace + part_o_bytes) : nullptr;

  // With profiling events installed, the launch carries them, so they take the
  // split kernel's own start and end timestamps (no event-packet overhead).
  hipEvent_t ev0, ev1;
  profile_events(&ev0, &ev1);
  if (ev0 || ev1)
    hipExtLaunchKernelGGL(fn, dim3(plan.grid), dim3(plan.waves * 64), 0, stream, ev0, ev1, 0, a);
  else
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
  c.n_inst = p.units();
  c.n_kvh = p.n_kvh;
  c.grp = p.grp();
  c.n_head = p.n_head;
  // XCD-local merging where each unit's work items fit in one XCD's share of
  // the split kernel's grid (so each unit's partials lie on one or two XCDs);
  // a unit is merged on the XCD holding most of its items
  const int ipu = plan.n_split * plan.n_rowblk;
  c.xcd_local = ipu <= plan.grid / 8 ? 1 : 0;
  c.wpu = 0;
  c.ub[0] = 0;
  if (c.xcd_local) {
    int x_prev = 0, u = 0;
    for (; u < p.units(); ++u) {
      const int x = xcd_majority(u * ipu, ipu, plan.grid);
      for (; x_prev < x; ++x_prev) c.ub[x_prev + 1] = u;
    }
    for (; x_prev < 8; ++x_prev) c.ub[x_prev + 1] = u;
  }
  switch (p.hd) {
    case 64: return launch_combine<64>(c, stream);
    case 80: return launch_combine<80>(c, stream);
    case 128: return launch_combine<128>(c, stream);
    case 256: return launch_combine<256>(c, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace fr
