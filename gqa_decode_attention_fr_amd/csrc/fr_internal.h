// fr_internal.h -- launch plan and kernel launchers shared by the host API and
// the kernel translation unit.  Not part of the public C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fr {

// Keys staged through LDS per block iteration of the split kernel.
constexpr int kKeyBlock = 64;
// Query tokens one split-kernel workgroup stages mask rows for: 16 (the
// pages' window, q_tokens <= 16) in the 4-wave shape, 64 in the 8-wave shape,
// which therefore takes every call with more than 16 tokens.
constexpr int kMaxTok4 = 16;
constexpr int kMaxTok8 = 64;
constexpr int max_tokens(int waves) { return waves == 8 ? kMaxTok8 : kMaxTok4; }

enum Variant { kFused = 1, kDecomposed = 2 };
enum QMode { kQHiLo = 0, kQF16 = 1, kQRound = 2 };

struct Plan {
  int variant = kFused;
  int n_split = 1;     // key splits per instance
  int chunk = 0;       // keys per split (multiple of kKeyBlock)
  int waves = 4;       // waves per workgroup of the split kernel
  int tiles = 1;       // 16-row tiles per wave
  int n_rowblk = 1;    // row blocks per instance
  int tpr = 1;         // 16-row tiles per row block (balanced; <= waves * tiles)
  int grid = 0;        // workgroups of the split kernel
  int launches = 1;    // kernel launches per call
  size_t ws_bytes = 0; // device workspace bytes
};

// Everything one launch sequence needs.  Strides count elements.
//
// KV-head groups: each instance has n_kvh KV heads, and query head h reads KV
// head h / (n_head / n_kvh) (consecutive query heads share one).  The kernels
// work on units u = inst * n_kvh + kv, one per (instance, KV head), each with
// grp = n_head / n_kvh query heads and grp * n_tok rows ordered t-major inside
// the unit; unit row rho = t*grp + j is row t*n_head + kv*grp + j of the
// instance.  With one KV head a unit is an instance and the rows coincide.
struct Problem {
  const void *q;
  const uint16_t *k;
  const uint16_t *v;
  const uint16_t *mask;
  const int32_t *kv_len;   // per instance valid key count (device), or null
  float *out;
  int n_inst;
  int64_t q_stride, kv_stride, mask_stride, out_stride;
  int n_head, n_tok, n_kv, hd;
  int n_kvh;            // KV heads per instance (divides n_head)
  int64_t kvh_stride;   // elements between consecutive KV heads of K (and V)
  float scale;
  int qmode;
  int grp() const { return n_head / n_kvh; }
  int units() const { return n_inst * n_kvh; }
  int unit_rows() const { return grp() * n_tok; }
};

// Integer environment override (developer knobs; fallback when unset).
int env_int(const char *name, int fallback);

// Caller events recorded around the main kernel (null when timing is off).
void profile_events(hipEvent_t *start, hipEvent_t *stop);

// Chooses the variant and the work decomposition (pure host logic; the same
// for every query format).
int make_plan(int n_inst, int n_head, int n_tok, int n_kv, int hd, unsigned flags,
              Plan *plan);

// Enqueue the fused split-KV path (split kernel, plus the combine kernel when
// n_split > 1).  Returns hipSuccess or the launch error.
hipError_t launch_fused(const Problem &p, const Plan &plan, void *workspace, hipStream_t stream);

// One f32 -> f16 row copy of a batch (n elements, src to dst).
struct CopyDesc {
  const float *src;
  uint16_t *dst;
  int64_t n;
};
// Copies whose descriptors one launch carries in its kernel arguments.
constexpr int kCopiesPerLaunch = 64;

// Enqueue a run of f32 -> f16 (nearest-even) copies, kCopiesPerLaunch per launch.
hipError_t launch_f16_copies(const CopyDesc *copies, int n_copies, hipStream_t stream);

// The query/KV producer (RoPE, query scale, f16 rows).  Strides in elements.
struct QkvPostArgs {
  const float *qkv;       // [n_inst][n_tok][(n_head + 2*n_kvh) * hd]
  const int32_t *pos;     // [n_inst][n_tok] positions
  uint16_t *q16;          // [n_inst][n_tok][n_head][hd]
  uint16_t *k_cache;      // [n_inst][n_kvh][capacity][hd], or null (no K/V store)
  uint16_t *v_cache;
  int64_t qkv_stride, pos_stride, q16_stride, cache_stride, cache_head_stride;
  int n_head, n_kvh, hd, capacity;
  double log2_base;       // log2 of the RoPE base
  float q_scale;
};
hipError_t launch_qkv_post(const QkvPostArgs &a, int n_tok, int n_inst, hipStream_t stream);

// Enqueue the three-launch decomposition: QK^T, masked softmax, PV.
hipError_t launch_decomposed(const Problem &p, const Plan &plan, void *workspace,
                             hipStream_t stream);

}  // namespace fr
