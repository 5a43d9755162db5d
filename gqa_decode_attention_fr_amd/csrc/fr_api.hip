// fr_api.hip -- the exported C ABI (include/fr_decode_attn.h): argument checks,
// the grow-only device workspace, and dispatch (the planner is fr_plan.hip).
//
// Argument checks play the role of the window predicate in the FlashRT-llama.cpp
// development guide (section "Adding a fusion window"): every assumption the
// kernels make -- dtypes, shapes, element strides, alignment, the absence of
// aliasing -- is pinned here, and anything else is declined with a status code
// before any HIP call is made.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <vector>

#include "fr_decode_attn.h"
#include "fr_internal.h"

namespace fr {


int env_int(const char *name, int fallback) {
  const char *s = std::getenv(name);
  if (!s || !*s) return fallback;
  return std::atoi(s);
}

bool debug_on() { return env_int("FR_DEBUG", 0) != 0; }

static std::atomic<hipEvent_t> g_prof_start{nullptr};
static std::atomic<hipEvent_t> g_prof_stop{nullptr};

void profile_events(hipEvent_t *start, hipEvent_t *stop) {
  *start = g_prof_start.load();
  *stop = g_prof_stop.load();
  if (!*start || !*stop) *start = *stop = nullptr;
}

}  // namespace fr

using fr::Plan;
using fr::Problem;

namespace {

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

struct Range {
  uintptr_t lo, hi; // [lo, hi)
};

bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

Range span(const void *base, int n_inst, int64_t stride, int64_t elems, size_t esize) {
  const uintptr_t lo = (uintptr_t)base;
  const int64_t last = (int64_t)(n_inst - 1) * stride + elems;
  return Range{lo, lo + (uintptr_t)(last * (int64_t)esize)};
}

// has_mask: the token limit of a masked call (mask rows are staged per token);
// without a mask (and for the plan helpers) the unmasked limit applies
int check_sizes(int n_inst, int n_head, int n_tok, int n_kv, int hd, bool has_mask = false) {
  if (n_inst < 1 || n_head < 1 || n_tok < 1 || n_kv < 1 || hd < 1) return FR_ERR_INVALID;
  if (n_tok > (has_mask ? FR_MAX_TOKENS : FR_MAX_TOKENS_UNMASKED) || n_head > FR_MAX_HEADS)
    return FR_ERR_UNSUPPORTED;
  if (hd != 64 && hd != 80 && hd != 128 && hd != 256) return FR_ERR_UNSUPPORTED;
  if (n_kv > (1 << 26)) return FR_ERR_UNSUPPORTED;
  // the kernels' 32-bit mask offsets
  if (has_mask && (int64_t)n_tok * n_kv > (1 << 30)) return FR_ERR_UNSUPPORTED;
  if ((int64_t)n_inst * n_head * n_tok > (1 << 24)) return FR_ERR_UNSUPPORTED;
  return FR_OK;
}

int check_flags(int q_format, unsigned flags) {
  const unsigned known =
      FR_Q_ROUND_F16 | FR_VARIANT_FUSED | FR_VARIANT_DECOMPOSED | FR_PLAN_UNMASKED;
  if (flags & ~known) return FR_ERR_INVALID;
  if ((flags & FR_VARIANT_FUSED) && (flags & FR_VARIANT_DECOMPOSED)) return FR_ERR_INVALID;
  if (q_format != FR_Q_F32 && q_format != FR_Q_F16) return FR_ERR_INVALID;
  if (q_format == FR_Q_F16 && (flags & FR_Q_ROUND_F16)) return FR_ERR_INVALID;
  return FR_OK;
}

int validate(const void *q, int q_format, const uint16_t *k, const uint16_t *v,
             const uint16_t *mask, const float *out, int n_inst, int64_t q_stride,
             int64_t kv_stride, int64_t mask_stride, int64_t out_stride, int n_head,
             int n_kvh, int64_t kvh_stride, int n_tok, int n_kv, int hd, float scale,
             unsigned flags) {
  if (!q || !k || !v || !out) return FR_ERR_INVALID;
  int st = check_sizes(n_inst, n_head, n_tok, n_kv, hd, mask != nullptr);
  if (st != FR_OK) return st;
  // KV heads: a divisor of n_head, each a 16-byte aligned [n_kv][hd] block
  if (n_kvh < 1 || n_head % n_kvh != 0) return FR_ERR_INVALID;
  if (n_kvh > 1 && (kvh_stride < (int64_t)n_kv * hd || (kvh_stride * 2) % 16))
    return FR_ERR_INVALID;
  const int64_t kv_elems = (int64_t)(n_kvh - 1) * (n_kvh > 1 ? kvh_stride : 0) +
                           (int64_t)n_kv * hd;   // one instance's K (or V)
  st = check_flags(q_format, flags);
  if (st != FR_OK) return st;
  if (!std::isfinite(scale)) return FR_ERR_INVALID;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
    return FR_ERR_INVALID;
  if (mask && !aligned(mask, 2)) return FR_ERR_INVALID;
  const int64_t M = (int64_t)n_head * n_tok;
  const size_t qsize = q_format == FR_Q_F16 ? 2 : 4;
  if (n_inst > 1) {
    if (q_stride < 0 || (q_stride != 0 && q_stride < M * hd)) return FR_ERR_INVALID;
    if ((q_stride * (int64_t)qsize) % 16) return FR_ERR_INVALID;
    if (kv_stride < 0 || (kv_stride != 0 && kv_stride < kv_elems)) return FR_ERR_INVALID;
    if ((kv_stride * 2) % 16) return FR_ERR_INVALID;
    if (mask_stride < 0 || (mask_stride != 0 && mask_stride < (int64_t)n_tok * n_kv))
      return FR_ERR_INVALID;
    if (out_stride < M * hd || (out_stride * 4) % 16) return FR_ERR_INVALID;
  } else {
    q_stride = kv_stride = mask_stride = out_stride = 0;
  }
  const Range ro = span(out, n_inst, out_stride, M * hd, 4);
  if (overlaps(ro, span(q, n_inst, q_stride, M * hd, qsize))) return FR_ERR_INVALID;
  if (overlaps(ro, span(k, n_inst, kv_stride, kv_elems, 2))) return FR_ERR_INVALID;
  if (overlaps(ro, span(v, n_inst, kv_stride, kv_elems, 2))) return FR_ERR_INVALID;
  if (mask && overlaps(ro, span(mask, n_inst, mask_stride, (int64_t)n_tok * n_kv, 2)))
    return FR_ERR_INVALID;
  return FR_OK;
}

// ---- library-owned, per-device, grow-only workspace.  A buffer that is
// replaced by a larger one is retired, never freed while the process runs: a
// graph captured earlier keeps its address in its kernel arguments and may be
// replayed at any time (the grow-only, address-stable slots that the
// FlashRT-llama.cpp development guide asks of caches, section "Caches (all
// capture-safe)").  Only fr_decode_attn_workspace_release frees them.
struct DeviceWs {
  void *ptr = nullptr;
  size_t bytes = 0;
  std::vector<void *> retired;   // earlier, smaller buffers (still valid memory)
};
std::mutex g_ws_mu;
std::vector<DeviceWs> g_ws;

size_t round_ws(size_t need) {
  const size_t mb = (size_t)1 << 20;
  return (need + mb - 1) / mb * mb;
}

// Returns a workspace of at least `need` bytes on the current device.  Grows
// only outside graph capture (FR_ERR_CAPTURE otherwise).  A new buffer is
// zero-filled before it is handed out (synchronously, outside any capture).
int library_ws(size_t need, hipStream_t stream, bool check_capture, void **out) {
  *out = nullptr;
  if (need == 0) return FR_OK;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FR_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_ws_mu);
  if ((int)g_ws.size() <= dev) g_ws.resize(dev + 1);
  DeviceWs &w = g_ws[dev];
  if (w.bytes >= need) {
    *out = w.ptr;
    return FR_OK;
  }
  if (check_capture) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) != hipSuccess) return FR_ERR_HIP;
    if (cs != hipStreamCaptureStatusNone) return FR_ERR_CAPTURE;
  }
  const size_t bytes = round_ws(need);
  void *p = nullptr;
  if (hipMalloc(&p, bytes) != hipSuccess) return FR_ERR_HIP;
  if (hipMemset(p, 0, bytes) != hipSuccess) {
    (void)hipFree(p);
    return FR_ERR_HIP;
  }
  if (w.ptr) w.retired.push_back(w.ptr);   // earlier calls and graphs may still use it
  w.ptr = p;
  w.bytes = bytes;
  *out = p;
  return FR_OK;
}

// Frees every library workspace buffer of the current device (current and
// retired) after a device synchronisation.
int release_library_ws() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FR_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_ws_mu);
  if ((int)g_ws.size() <= dev) return FR_OK;
  DeviceWs &w = g_ws[dev];
  if (!w.ptr && w.retired.empty()) return FR_OK;
  if (hipDeviceSynchronize() != hipSuccess) return FR_ERR_HIP;
  int st = FR_OK;
  for (void *p : w.retired)
    if (hipFree(p) != hipSuccess) st = FR_ERR_HIP;
  if (w.ptr && hipFree(w.ptr) != hipSuccess) st = FR_ERR_HIP;
  w = DeviceWs{};
  return st;
}

// ---- the fixed scratch array of fr_decode_attn_gqa_noalloc.  In host code
// `scratch` names a host-side stand-in, not device memory: kernels get the
// per-device address that hipGetSymbolAddress reports, never the name itself.
static __device__ __align__(256) unsigned char scratch[FR_NOALLOC_SCRATCH_BYTES];
std::mutex g_scratch_mu;
std::vector<void *> g_scratch_ptr;   // per device; null until looked up

// The current device's address of `scratch` (looked up once per device, with
// that device current).  FR_ERR_HIP if the lookup fails.
int scratch_address(void **out) {
  *out = nullptr;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FR_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if ((int)g_scratch_ptr.size() <= dev) g_scratch_ptr.resize(dev + 1, nullptr);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FR_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FR_OK;
}

int run(const void *q, int q_format, const uint16_t *k, const uint16_t *v, const uint16_t *mask,
        const int32_t *kv_len, float *out, int n_inst, int64_t q_stride, int64_t kv_stride, int64_t mask_stride,
        int64_t out_stride, int n_head, int n_kvh, int64_t kvh_stride, int n_tok, int n_kv,
        int hd, float scale, unsigned flags, void *workspace, size_t workspace_bytes,
        bool caller_ws, void *stream) {
  int st = validate(q, q_format, k, v, mask, out, n_inst, q_stride, kv_stride, mask_stride,
                    out_stride, n_head, n_kvh, kvh_stride, n_tok, n_kv, hd, scale, flags);
  if (st != FR_OK) return st;
  if (kv_len && !aligned(kv_len, 4)) return FR_ERR_INVALID;
  if (n_inst == 1) q_stride = kv_stride = mask_stride = out_stride = 0;
  if (n_kvh == 1) kvh_stride = 0;
  // the plan knows whether the call has a mask (the caller's bit is replaced)
  flags = (flags & ~FR_PLAN_UNMASKED) | (mask ? 0u : FR_PLAN_UNMASKED);
  // the kernels run on units (instance, KV head) of n_head / n_kvh query heads
  Plan plan;
  st = fr::make_plan(n_inst * n_kvh, n_head / n_kvh, n_tok, n_kv, hd, flags, &plan);
  if (st != FR_OK) return st;
  // Memory the kernels write (out, and a caller workspace) must not overlap
  // anything they read: q, k, v, the mask and the valid key counts (the
  // library's own workspace is disjoint from every caller buffer).
  const int64_t M = (int64_t)n_head * n_tok;
  const int64_t kv_elems = (int64_t)(n_kvh - 1) * kvh_stride + (int64_t)n_kv * hd;
  const Range r_out = span(out, n_inst, out_stride, M * hd, 4);
  const Range r_len = kv_len ? span(kv_len, 1, 0, n_inst, 4) : Range{0, 0};
  if (kv_len && overlaps(r_len, r_out)) return FR_ERR_INVALID;
  if (caller_ws) {
    if (plan.ws_bytes > 0 && (!workspace || workspace_bytes < plan.ws_bytes))
      return FR_ERR_WORKSPACE;
    if (workspace && !aligned(workspace, 256)) return FR_ERR_INVALID;
    if (plan.ws_bytes > 0) {
      const Range r_ws = span(workspace, 1, 0, (int64_t)plan.ws_bytes, 1);
      const size_t qsize = q_format == FR_Q_F16 ? 2 : 4;
      if (overlaps(r_ws, r_out) || overlaps(r_ws, span(q, n_inst, q_stride, M * hd, qsize)) ||
          overlaps(r_ws, span(k, n_inst, kv_stride, kv_elems, 2)) ||
          overlaps(r_ws, span(v, n_inst, kv_stride, kv_elems, 2)) ||
          (mask && overlaps(r_ws, span(mask, n_inst, mask_stride, (int64_t)n_tok * n_kv, 2))) ||
          (kv_len && overlaps(r_ws, r_len)))
        return FR_ERR_INVALID;
    }
  } else {
    st = library_ws(plan.ws_bytes, (hipStream_t)stream, true, &workspace);
    if (st != FR_OK) return st;
  }
  Problem p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.mask = mask;
  p.kv_len = kv_len;
  p.out = out;
  p.n_inst = n_inst;
  p.q_stride = q_stride;
  p.kv_stride = kv_stride;
  p.mask_stride = mask_stride;
  p.out_stride = out_stride == 0 ? (int64_t)n_head * n_tok * hd : out_stride;
  p.n_head = n_head;
  p.n_tok = n_tok;
  p.n_kv = n_kv;
  p.hd = hd;
  p.n_kvh = n_kvh;
  p.kvh_stride = kvh_stride;
  p.scale = scale;
  p.qmode = q_format == FR_Q_F16 ? fr::kQF16 : ((flags & FR_Q_ROUND_F16) ? fr::kQRound : fr::kQHiLo);
  if (fr::debug_on())
    std::fprintf(stderr,
                 "[fr_decode_attn] variant=%d n_inst=%d kv_heads=%d M=%d n_kv=%d hd=%d qmode=%d "
                 "splits=%d chunk=%d waves=%d tiles=%d rowblk=%d grid=%d ws=%zu\n",
                 plan.variant, n_inst, n_kvh, n_head * n_tok, n_kv, hd, p.qmode, plan.n_split,
                 plan.chunk, plan.waves, plan.tiles, plan.n_rowblk, plan.grid, plan.ws_bytes);
  hipError_t err = plan.variant == fr::kDecomposed
                       ? fr::launch_decomposed(p, plan, workspace, (hipStream_t)stream)
                       : fr::launch_fused(p, plan, workspace, (hipStream_t)stream);
  return err == hipSuccess ? FR_OK : FR_ERR_HIP;
}

}  // namespace

extern "C" {

int fr_decode_attn(const float *q, const uint16_t *k, const uint16_t *v, const uint16_t *mask,
                   float *out, int n_head, int n_tok, int n_kv, int hd, float scale,
                   void *stream) {
  return run(q, FR_Q_F32, k, v, mask, nullptr, out, 1, 0, 0, 0, 0, n_head, 1, 0, n_tok, n_kv, hd, scale,
             0u, nullptr, 0, false, stream);
}

int fr_decode_attn_q16(const uint16_t *q16, const uint16_t *k, const uint16_t *v,
                       const uint16_t *mask, float *out, int n_head, int n_tok, int n_kv, int hd,
                       float scale, void *stream) {
  return run(q16, FR_Q_F16, k, v, mask, nullptr, out, 1, 0, 0, 0, 0, n_head, 1, 0, n_tok, n_kv, hd,
             scale, 0u, nullptr, 0, false, stream);
}

int fr_decode_attn_batched(const void *q, int q_format, const uint16_t *k, const uint16_t *v,
                           const uint16_t *mask, float *out, int n_inst, int64_t q_stride,
                           int64_t kv_stride, int64_t mask_stride, int64_t out_stride,
                           int n_head, int n_tok, int n_kv, int hd, float scale, void *stream) {
  return run(q, q_format, k, v, mask, nullptr, out, n_inst, q_stride, kv_stride, mask_stride,
             out_stride, n_head, 1, 0, n_tok, n_kv, hd, scale, 0u, nullptr, 0, false, stream);
}

int fr_decode_attn_ex(const void *q, int q_format, const uint16_t *k, const uint16_t *v,
                      const uint16_t *mask, float *out, int n_inst, int64_t q_stride,
                      int64_t kv_stride, int64_t mask_stride, int64_t out_stride, int n_head,
                      int n_tok, int n_kv, int hd, float scale, unsigned flags, void *workspace,
                      size_t workspace_bytes, void *stream) {
  return run(q, q_format, k, v, mask, nullptr, out, n_inst, q_stride, kv_stride, mask_stride,
             out_stride, n_head, 1, 0, n_tok, n_kv, hd, scale, flags, workspace,
             workspace_bytes, workspace != nullptr, stream);
}

int fr_decode_attn_gqa(const void *q, int q_format, const uint16_t *k, const uint16_t *v,
                       const uint16_t *mask, const int32_t *kv_len, float *out, int n_inst,
                       int64_t q_stride,
                       int64_t kv_stride, int64_t mask_stride, int64_t out_stride, int n_head,
                       int n_kv_head, int64_t kv_head_stride, int n_tok, int n_kv, int hd,
                       float scale, unsigned flags, void *workspace, size_t workspace_bytes,
                       void *stream) {
  return run(q, q_format, k, v, mask, kv_len, out, n_inst, q_stride, kv_stride, mask_stride,
             out_stride, n_head, n_kv_head, kv_head_stride, n_tok, n_kv, hd, scale, flags, workspace,
             workspace_bytes, workspace != nullptr, stream);
}

int fr_decode_attn_gqa_noalloc(const void *q, int q_format, const uint16_t *k, const uint16_t *v,
                               const uint16_t *mask, const int32_t *kv_len, float *out,
                               int n_inst, int64_t q_stride, int64_t kv_stride,
                               int64_t mask_stride, int64_t out_stride, int n_head,
                               int n_kv_head, int64_t kv_head_stride, int n_tok, int n_kv,
                               int hd, float scale, unsigned flags, void *stream) {
  // The plan's workspace must fit the fixed array: checked here (after the
  // same argument checks the other entry points make) so that the address
  // lookup below is the only HIP call before the launch.
  int st = validate(q, q_format, k, v, mask, out, n_inst, q_stride, kv_stride, mask_stride,
                    out_stride, n_head, n_kv_head, kv_head_stride, n_tok, n_kv, hd, scale, flags);
  if (st != FR_OK) return st;
  if (kv_len) {
    if (!aligned(kv_len, 4)) return FR_ERR_INVALID;
    const int64_t os = n_inst > 1 ? out_stride : 0;
    if (overlaps(span(kv_len, 1, 0, n_inst, 4),
                 span(out, n_inst, os, (int64_t)n_head * n_tok * hd, 4)))
      return FR_ERR_INVALID;
  }
  const unsigned pflags = (flags & ~FR_PLAN_UNMASKED) | (mask ? 0u : FR_PLAN_UNMASKED);
  Plan plan;
  st = fr::make_plan(n_inst * n_kv_head, n_head / n_kv_head, n_tok, n_kv, hd, pflags, &plan);
  if (st != FR_OK) return st;
  if (plan.ws_bytes > (size_t)FR_NOALLOC_SCRATCH_BYTES) return FR_ERR_WORKSPACE;
  void *ws = nullptr;
  st = scratch_address(&ws);
  if (st != FR_OK) return st;
  return run(q, q_format, k, v, mask, kv_len, out, n_inst, q_stride, kv_stride, mask_stride,
             out_stride, n_head, n_kv_head, kv_head_stride, n_tok, n_kv, hd, scale, flags, ws,
             (size_t)FR_NOALLOC_SCRATCH_BYTES, true, stream);
}

size_t fr_decode_attn_workspace_size(int n_inst, int n_head, int n_tok, int n_kv, int hd,
                                     unsigned flags, int *status) {
  int st = check_sizes(n_inst, n_head, n_tok, n_kv, hd);
  if (st == FR_OK) st = check_flags(FR_Q_F32, flags);
  size_t need = 0;
  if (st == FR_OK) {
    Plan a;
    st = fr::make_plan(n_inst, n_head, n_tok, n_kv, hd, flags, &a);
    need = a.ws_bytes;
    if (st == FR_OK && !(flags & FR_PLAN_UNMASKED)) {
      // without the bit the size covers calls with and without a mask
      Plan b;
      st = fr::make_plan(n_inst, n_head, n_tok, n_kv, hd, flags | FR_PLAN_UNMASKED, &b);
      need = std::max(need, b.ws_bytes);
    }
  }
  if (status) *status = st;
  return st == FR_OK ? need : 0;
}

int fr_decode_attn_reserve(int n_inst, int n_head, int n_tok, int n_kv, int hd,
                           unsigned flags) {
  int st = FR_OK;
  const size_t need = fr_decode_attn_workspace_size(n_inst, n_head, n_tok, n_kv, hd, flags, &st);
  if (st != FR_OK) return st;
  void *p = nullptr;
  return library_ws(need, nullptr, false, &p);
}

int fr_decode_attn_workspace_query(void **ptr, size_t *bytes, int *n_retired) {
  if (ptr) *ptr = nullptr;
  if (bytes) *bytes = 0;
  if (n_retired) *n_retired = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FR_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_ws_mu);
  if ((int)g_ws.size() <= dev) return FR_OK;
  if (ptr) *ptr = g_ws[dev].ptr;
  if (bytes) *bytes = g_ws[dev].bytes;
  if (n_retired) *n_retired = (int)g_ws[dev].retired.size();
  return FR_OK;
}

int fr_decode_attn_workspace_release(void) { return release_library_ws(); }

int fr_decode_attn_plan(int n_inst, int n_head, int n_tok, int n_kv, int hd, unsigned flags,
                        int *info, int n_info) {
  if (!info || n_info < 0) return FR_ERR_INVALID;
  int st = check_sizes(n_inst, n_head, n_tok, n_kv, hd);
  if (st == FR_OK) st = check_flags(FR_Q_F32, flags);
  if (st != FR_OK) return st;
  Plan p;
  st = fr::make_plan(n_inst, n_head, n_tok, n_kv, hd, flags, &p);
  if (st != FR_OK) return st;
  const int vals[8] = {p.variant, p.n_split, p.chunk, p.waves,
                       p.tiles,   p.n_rowblk, p.grid, p.launches};
  for (int i = 0; i < n_info && i < 8; ++i) info[i] = vals[i];
  return FR_OK;
}

int fr_qkv_post(const float *qkv, const int32_t *pos, uint16_t *q16, uint16_t *k_cache,
                uint16_t *v_cache, int n_inst, int64_t qkv_stride, int64_t pos_stride,
                int64_t q16_stride, int64_t cache_stride, int64_t cache_head_stride,
                int n_head, int n_kv_head, int n_tok, int hd, int capacity, float rope_base,
                float q_scale, void *stream) {
  if (!qkv || !pos || !q16 || (!k_cache) != (!v_cache)) return FR_ERR_INVALID;
  if (n_inst < 1 || n_head < 1 || n_kv_head < 1 || n_tok < 1) return FR_ERR_INVALID;
  if (n_tok > FR_MAX_TOKENS_UNMASKED || n_head > FR_MAX_HEADS || n_kv_head > FR_MAX_HEADS)
    return FR_ERR_UNSUPPORTED;
  if (hd != 64 && hd != 80 && hd != 128 && hd != 256) return FR_ERR_UNSUPPORTED;
  if (!std::isfinite(rope_base) || !(rope_base > 0.f) || !std::isfinite(q_scale))
    return FR_ERR_INVALID;
  if (!aligned(qkv, 4) || !aligned(pos, 4) || !aligned(q16, 2)) return FR_ERR_INVALID;
  const int64_t width = (int64_t)(n_head + 2 * n_kv_head) * hd;
  const int64_t qkv_elems = (int64_t)n_tok * width, q_elems = (int64_t)n_tok * n_head * hd;
  int64_t cache_elems = 0;
  if (k_cache) {
    if (!aligned(k_cache, 2) || !aligned(v_cache, 2) || capacity < 1) return FR_ERR_INVALID;
    if (n_kv_head > 1 && cache_head_stride < (int64_t)capacity * hd) return FR_ERR_INVALID;
    cache_elems = (int64_t)(n_kv_head - 1) * (n_kv_head > 1 ? cache_head_stride : 0) +
                  (int64_t)capacity * hd;
  }
  if (n_inst > 1) {
    if (qkv_stride < qkv_elems || q16_stride < q_elems) return FR_ERR_INVALID;
    if (pos_stride < 0 || (pos_stride != 0 && pos_stride < n_tok)) return FR_ERR_INVALID;
    if (k_cache && cache_stride < cache_elems) return FR_ERR_INVALID;
  } else {
    qkv_stride = pos_stride = q16_stride = cache_stride = 0;
  }
  if (n_kv_head == 1) cache_head_stride = 0;
  const Range rq = span(q16, n_inst, q16_stride, q_elems, 2);
  const Range rin = span(qkv, n_inst, qkv_stride, qkv_elems, 4);
  const Range rpos = span(pos, n_inst, pos_stride, n_tok, 4);
  if (overlaps(rq, rin) || overlaps(rq, rpos)) return FR_ERR_INVALID;
  if (k_cache) {
    const Range rk = span(k_cache, n_inst, cache_stride, cache_elems, 2);
    const Range rv = span(v_cache, n_inst, cache_stride, cache_elems, 2);
    if (overlaps(rk, rv) || overlaps(rk, rq) || overlaps(rv, rq) || overlaps(rk, rin) ||
        overlaps(rv, rin) || overlaps(rk, rpos) || overlaps(rv, rpos))
      return FR_ERR_INVALID;
  }
  fr::QkvPostArgs a;
  a.qkv = qkv;
  a.pos = pos;
  a.q16 = q16;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.qkv_stride = qkv_stride;
  a.pos_stride = pos_stride;
  a.q16_stride = q16_stride;
  a.cache_stride = cache_stride;
  a.cache_head_stride = cache_head_stride;
  a.n_head = n_head;
  a.n_kvh = n_kv_head;
  a.hd = hd;
  a.capacity = capacity;
  a.log2_base = std::log2((double)rope_base);
  a.q_scale = q_scale;
  const hipError_t err = fr::launch_qkv_post(a, n_tok, n_inst, (hipStream_t)stream);
  return err == hipSuccess ? FR_OK : FR_ERR_HIP;
}

int fr_f16_copy_batch(const fr_f16_copy *copies, int n_copies, void *stream) {
  if (n_copies < 0 || n_copies > FR_MAX_COPIES || (n_copies > 0 && !copies))
    return FR_ERR_INVALID;
  std::vector<fr::CopyDesc> run;
  run.reserve(n_copies);
  struct Tagged {
    Range r;
    bool dst;
  };
  std::vector<Tagged> ranges;
  ranges.reserve(2 * (size_t)n_copies);
  for (int i = 0; i < n_copies; ++i) {
    const fr_f16_copy &c = copies[i];
    if (c.n < 0) return FR_ERR_INVALID;
    if (c.n == 0) continue;
    if (!c.src || !c.dst || !aligned(c.src, 4) || !aligned(c.dst, 2)) return FR_ERR_INVALID;
    ranges.push_back(Tagged{span(c.src, 1, 0, c.n, 4), false});
    ranges.push_back(Tagged{span(c.dst, 1, 0, c.n, 2), true});
    run.push_back(fr::CopyDesc{c.src, c.dst, c.n});
  }
  // No destination may overlap a source or another destination (sources may
  // overlap each other).  Sorted by start, a range overlaps an earlier one
  // exactly when it starts below the largest earlier end.
  std::sort(ranges.begin(), ranges.end(),
            [](const Tagged &a, const Tagged &b) { return a.r.lo < b.r.lo; });
  uintptr_t end_any = 0, end_dst = 0;
  for (const Tagged &t : ranges) {
    if (t.r.lo < (t.dst ? end_any : end_dst)) return FR_ERR_INVALID;
    end_any = std::max(end_any, t.r.hi);
    if (t.dst) end_dst = std::max(end_dst, t.r.hi);
  }
  if (run.empty()) return FR_OK;
  const hipError_t err = fr::launch_f16_copies(run.data(), (int)run.size(), (hipStream_t)stream);
  return err == hipSuccess ? FR_OK : FR_ERR_HIP;
}

int fr_decode_attn_profile_events(void *start, void *stop) {
  if ((start == nullptr) != (stop == nullptr)) return FR_ERR_INVALID;
  fr::g_prof_start.store((hipEvent_t)start);
  fr::g_prof_stop.store((hipEvent_t)stop);
  return FR_OK;
}

const char *fr_status_str(int status) {
  switch (status) {
    case FR_OK: return "FR_OK";
    case FR_ERR_INVALID: return "FR_ERR_INVALID: bad pointer, size, stride, alignment or aliasing";
    case FR_ERR_UNSUPPORTED: return "FR_ERR_UNSUPPORTED: shape outside the supported window";
    case FR_ERR_CAPTURE: return "FR_ERR_CAPTURE: workspace must grow while the stream is captured";
    case FR_ERR_HIP: return "FR_ERR_HIP: HIP runtime or launch failure";
    case FR_ERR_WORKSPACE: return "FR_ERR_WORKSPACE: caller workspace too small";
    default: return "unknown fr_status";
  }
}

int fr_abi_version(void) { return FR_DECODE_ATTN_ABI_VERSION; }

}  // extern "C"
