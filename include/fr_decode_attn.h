/*
 * fr_decode_attn.h -- C ABI of the MI355X (gfx950) small-q GQA decode attention.
 *
 * The operation.  FlashRT pull request #185, "feat(structures): ggml host
 * adapter -- llama.cpp distribution for pi0.5 on Thor (SM110)", in the commit
 * that introduces the decomposed decode attention: FLASH_ATTN_EXT with at
 * most 16 query tokens over a single padded f16 KV head is computed as a
 * QK^T contraction, a masked softmax accurate to fp32, and a PV contraction
 * whose fp32 result lands in the node's [hd, n_head, n_tok] destination.
 * For every query token t < n_tok, head h < n_head and d < hd:
 *
 *     s_j           = scale * sum_e q[t][h][e] * K[j][e] + mask[t][j]   (j < n_kv)
 *     out[t][h][d]  = sum_j exp(s_j - max s) * V[j][d] / sum_j exp(s_j - max s)
 *
 * Layouts (element offsets, fastest index last, all dense):
 *   q    [n_tok][n_head][hd]  -- "t-major" rows r = t*n_head + h.  The same
 *                                pull request's GQA-collapse commit orders the
 *                                n_head*n_tok query rows this way so that one
 *                                contraction covers every head; its qkv_post
 *                                handoff commit stores Q in exactly this order.
 *   k, v [n_kv][hd]           -- IEEE binary16 bits, the one KV head that all
 *                                query heads share (GQA with one KV group).
 *                                Pad rows (keys the mask hides for every token)
 *                                may hold any finite values; zero is usual.
 *   mask [n_tok][n_kv]        -- IEEE binary16 bits, additive, one row per query
 *                                token, shared by every head: 0 keeps a key,
 *                                -inf hides it; other finite values are added
 *                                to the logit.  NULL means all zero.
 *   out  [n_tok][n_head][hd]  -- fp32; this is ggml's [hd, n_head, n_tok]
 *                                (fastest first), written contiguously.
 *
 * Readings the pages leave open, fixed by this library:
 *   - scale multiplies q.K before the mask is added;
 *   - a row whose keys are all hidden gets an all-zero output row;
 *   - f32 queries are used at fp32 accuracy: each q is split into two f16
 *     parts (hi = f16(q), lo = f16(q - hi)) that both enter the f16 matrix
 *     cores, so q.K carries ~22 significand bits.  FR_Q_ROUND_F16 instead
 *     rounds q to f16 once, the way the pages' gather kernel does.
 *   - |q| must stay below 65504 (the f16 range); inputs holding NaN or inf
 *     give unspecified output.
 *
 * Pointers.  Every tensor pointer is a DEVICE pointer owned by the caller; the
 * library never frees or retains it past the call.  q, k, v and out must be
 * 16-byte aligned; mask needs 2-byte alignment.  Inputs are never written.
 * out must not overlap any input.
 *
 * Streams.  `stream` is a hipStream_t passed as void* (NULL: the null stream).
 * Every entry point only enqueues work on that stream: it does not
 * synchronise and returns before the result exists.  Entry points never abort
 * the process; failures come back as an fr_status code.  Argument checks run
 * before any HIP call, so a rejected call launches nothing.
 *
 * Beyond the pages' window (which fixes one KV head, at most 16 query tokens
 * and a mask): fr_decode_attn_gqa takes several KV heads and device-side
 * valid key counts; masked calls take up to 64 query tokens and unmasked ones
 * (the prefix-LM prefill) up to 16384; head size 80 is taken as well.
 * fr_qkv_post (the query/KV producer ahead of the window) and
 * fr_f16_copy_batch (the batched f32 -> f16 KV tail copies after it) are the
 * neighbouring steps of the same pull request.
 *
 * Workspace.  Shapes that split the key range across workgroups keep partial
 * results in a device workspace.  With workspace == NULL (every entry point
 * without a workspace argument, and fr_decode_attn_ex / fr_decode_attn_gqa
 * when they get NULL) the library uses its own per-device buffer, which only
 * grows and is never allocated while `stream` is being captured into a graph
 * (the capture-safety rule of the FlashRT-llama.cpp development guide,
 * section "Caches (all capture-safe)"): a call that would need to grow it
 * during capture returns FR_ERR_CAPTURE; call fr_decode_attn_reserve before
 * capturing.  A buffer outgrown by a later call is kept, not freed, so graphs
 * captured with it stay valid; fr_decode_attn_workspace_release frees them
 * all.  Calls that share the library workspace must be ordered on one
 * stream (or otherwise serialised); concurrent calls on different streams of
 * one device must each pass their own workspace to fr_decode_attn_ex (or
 * fr_decode_attn_gqa).
 */
#ifndef FR_DECODE_ATTN_H
#define FR_DECODE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
typedef enum fr_status {
    FR_OK = 0,
    FR_ERR_INVALID = -1,     /* null/misaligned pointer, bad size, stride or KV-head count, out overlaps an input */
    FR_ERR_UNSUPPORTED = -2, /* n_tok above 64 with a mask (16384 without), hd not 64/80/128/256,
                                n_head above 1024, n_kv above 2^26 or n_tok*n_kv above 2^30 */
    FR_ERR_CAPTURE = -3,     /* the library workspace would have to grow while the stream is captured */
    FR_ERR_HIP = -4,         /* a HIP runtime call or kernel launch failed */
    FR_ERR_WORKSPACE = -5    /* the caller's workspace is smaller than fr_decode_attn_workspace_size
                                (fr_decode_attn_gqa_noalloc: its fixed array is) */
} fr_status;

/* Query formats for fr_decode_attn_batched / fr_decode_attn_ex. */
#define FR_Q_F32 0 /* q is float32 */
#define FR_Q_F16 1 /* q is binary16 bits, already rounded (the qkv_post f16 handoff) */

/* Flags for fr_decode_attn_ex. */
#define FR_Q_ROUND_F16 0x1u        /* f32 q: round to f16 once, as the pages' gather does */
#define FR_VARIANT_FUSED 0x2u      /* force the fused single-pass split-KV variant */
#define FR_VARIANT_DECOMPOSED 0x4u /* force the three-launch QK^T -> softmax -> PV variant */
#define FR_PLAN_UNMASKED 0x8u      /* plan/workspace helpers: for calls with mask == NULL
                                      (calls themselves set or clear it from their mask) */

/* Limits checked by every entry point. */
#define FR_MAX_TOKENS 64    /* the pages' window covers q_tokens <= 16; up to 64 (a
                               speculative-verify window) are taken with a mask */
#define FR_MAX_TOKENS_UNMASKED 16384 /* without a mask (mask == NULL): every query
                               row sees the same keys, the prefix-LM prefill of
                               the pages (its padded tail excluded by n_kv or
                               by fr_decode_attn_gqa's kv_len) */
#define FR_MAX_HEADS 1024
/* Head sizes: 64, 80 (a vision-encoder size), 128 and 256, on both variants;
 * the fused kernel runs hd 80 in its hd-128 layout. */

/*
 * f32 queries.  q: float32 [n_tok][n_head][hd]; k, v, mask, out as above.
 * The decomposed decode attention commit of FlashRT PR #185 defines the
 * operation; q is used at fp32 accuracy (hi/lo f16 split).
 * Returns FR_OK or a negative fr_status.
 */
int fr_decode_attn(const float *q, const uint16_t *k, const uint16_t *v,
                   const uint16_t *mask, float *out, int n_head, int n_tok,
                   int n_kv, int hd, float scale, void *stream);

/*
 * Pre-rounded f16 queries: the qkv_post handoff commit of FlashRT PR #185,
 * where the producer stores the rope'd and scaled Q rows as f16 in the t-major
 * order this window reads, so no gather step runs.  q16: binary16 bits
 * [n_tok][n_head][hd].  fr_decode_attn_q16(f16_rne(q)) equals
 * fr_decode_attn_ex(q, FR_Q_F32, ..., FR_Q_ROUND_F16, ...) bit for bit.
 */
int fr_decode_attn_q16(const uint16_t *q16, const uint16_t *k, const uint16_t *v,
                       const uint16_t *mask, float *out, int n_head, int n_tok,
                       int n_kv, int hd, float scale, void *stream);

/*
 * n_inst independent instances (e.g. the layers of one model step) in one
 * launch sequence.  The pages run the window once per layer inside the model
 * graph and define no batched call; it is this library's, for the pi0.5
 * action step of 18 layer instances (one launch sequence instead of 18, each
 * instance computed exactly as fr_decode_attn would).  Instance i reads q + i*q_stride, k + i*kv_stride,
 * v + i*kv_stride, mask + i*mask_stride and writes out + i*out_stride; strides
 * count ELEMENTS of each tensor's type.  q_stride and kv_stride may be 0
 * (shared input); mask_stride may be 0 (one mask for all); out_stride must be
 * at least n_tok*n_head*hd.  Non-zero strides must keep 16-byte alignment
 * (mask: any).  q_format is FR_Q_F32 or FR_Q_F16.
 */
int fr_decode_attn_batched(const void *q, int q_format, const uint16_t *k,
                           const uint16_t *v, const uint16_t *mask, float *out,
                           int n_inst, int64_t q_stride, int64_t kv_stride,
                           int64_t mask_stride, int64_t out_stride, int n_head,
                           int n_tok, int n_kv, int hd, float scale, void *stream);

/*
 * Everything: batched instances, flags (FR_Q_ROUND_F16, FR_VARIANT_*), and an
 * optional caller-owned device workspace.  The pages define no such call; its
 * options come from them: FR_Q_ROUND_F16 is the single f16 rounding of the
 * gather that the qkv_post handoff commit of FlashRT PR #185 replaces,
 * FR_VARIANT_DECOMPOSED the separate QK^T, softmax and PV launches of its
 * decomposed decode attention commit, and the caller workspace serves the
 * development guide's "Caches (all capture-safe)" rule for callers that own
 * their memory.  workspace == NULL uses the library
 * workspace (grow-only, see above); otherwise it must be 256-byte aligned and
 * at least fr_decode_attn_workspace_size(...) bytes, else FR_ERR_WORKSPACE.
 * The library keeps no reference to a caller workspace after the call's
 * kernels finish.
 */
int fr_decode_attn_ex(const void *q, int q_format, const uint16_t *k,
                      const uint16_t *v, const uint16_t *mask, float *out,
                      int n_inst, int64_t q_stride, int64_t kv_stride,
                      int64_t mask_stride, int64_t out_stride, int n_head,
                      int n_tok, int n_kv, int hd, float scale, unsigned flags,
                      void *workspace, size_t workspace_bytes, void *stream);

/*
 * Several KV heads (grouped-query attention with n_kv_head groups) and an
 * optional device-side valid key count.  The pages fix one KV head shared by
 * every query head; this entry point widens the same window to n_kv_head KV
 * heads, with query head h attending over KV head
 * h / (n_head / n_kv_head) (consecutive query heads share a KV head, the
 * flash-attention node's broadcast of KV heads over query heads):
 *
 *     s_j           = scale * sum_e q[t][h][e] * K[h/G][j][e] + mask[t][j]
 *     out[t][h][d]  = softmax_j(s)_j-weighted sum of V[h/G][j][d],   G = n_head/n_kv_head
 *
 * q, mask and out keep the layouts above (t-major rows over all n_head heads,
 * one mask row per token shared by every head).  k and v of one instance are
 * n_kv_head blocks of [n_kv][hd], block kh at k + kh*kv_head_stride (ELEMENTS;
 * at least n_kv*hd and a multiple of 8 when n_kv_head > 1, ignored when it is
 * 1).  kv_stride between instances, when not 0, must cover all n_kv_head
 * blocks.  n_kv_head must divide n_head, else FR_ERR_INVALID.  Every other
 * argument, flag and rule is that of fr_decode_attn_ex, which is this call
 * with n_kv_head = 1.
 *
 * Planning: the call runs as n_inst*n_kv_head units of n_head/n_kv_head query
 * heads each, so fr_decode_attn_workspace_size, fr_decode_attn_reserve and
 * fr_decode_attn_plan take (n_inst*n_kv_head, n_head/n_kv_head, n_tok, n_kv,
 * hd, flags) for it.
 *
 * kv_len: NULL, or a DEVICE array of n_inst int32 valid key counts (4-byte
 * aligned).  Instance i then behaves as if keys j >= kv_len[i] were hidden
 * from every token (values below 0 count as 0, above n_kv as n_kv); their
 * K, V and mask entries are never read.  The kernels read the array when
 * they run, so a graph captured once replays with the counts the array holds
 * at replay time, while n_kv (the padded capacity, the mask's row stride)
 * stays fixed.  The key splits are planned for n_kv; splits past the valid
 * count finish at once.  A row whose keys are all hidden is zero.  Both
 * variants take it.
 */
int fr_decode_attn_gqa(const void *q, int q_format, const uint16_t *k,
                       const uint16_t *v, const uint16_t *mask,
                       const int32_t *kv_len, float *out,
                       int n_inst, int64_t q_stride, int64_t kv_stride,
                       int64_t mask_stride, int64_t out_stride, int n_head,
                       int n_kv_head, int64_t kv_head_stride, int n_tok, int n_kv,
                       int hd, float scale, unsigned flags, void *workspace,
                       size_t workspace_bytes, void *stream);

/*
 * fr_decode_attn_gqa for callers that cannot allocate device memory (code
 * under graph capture without a prior reserve, tight serving loops, harnesses
 * that forbid hipMalloc): the same arguments without a workspace.  The split
 * partials go to a fixed device array inside the library of
 * FR_NOALLOC_SCRATCH_BYTES bytes (one per GPU the library runs on, held until
 * the process ends); the call makes no allocation of any kind.  A call whose
 * plan needs more than that (fr_decode_attn_workspace_size) returns
 * FR_ERR_WORKSPACE and launches nothing.  Every call on one GPU shares that
 * GPU's array, which keeps the last call's contents: calls that overlap in
 * time on one GPU (different streams, or host threads racing) corrupt each
 * other's partials, so they must be ordered.  No part of the array needs to
 * start at zero: each call writes every partial it reads.  Otherwise as
 * fr_decode_attn_gqa.
 */
#define FR_NOALLOC_SCRATCH_BYTES 33554432u /* 32 MiB */
int fr_decode_attn_gqa_noalloc(const void *q, int q_format, const uint16_t *k,
                               const uint16_t *v, const uint16_t *mask,
                               const int32_t *kv_len, float *out,
                               int n_inst, int64_t q_stride, int64_t kv_stride,
                               int64_t mask_stride, int64_t out_stride, int n_head,
                               int n_kv_head, int64_t kv_head_stride, int n_tok,
                               int n_kv, int hd, float scale, unsigned flags,
                               void *stream);

/* Device workspace bytes a call with these sizes and flags needs (0 if none),
 * or 0 with *status set when the sizes are rejected (status may be NULL).
 * Not defined by the pages: it lets a caller size a workspace before capture,
 * as the development guide's "Caches (all capture-safe)" section requires of
 * anything allocated for a captured window.
 * The size does not depend on the query format, so it also suits
 * fr_decode_attn_q16 and FR_Q_F16 calls.  Without FR_PLAN_UNMASKED it covers
 * calls with and without a mask (the plan of an unmasked call with many rows
 * differs); with it, unmasked calls only. */
size_t fr_decode_attn_workspace_size(int n_inst, int n_head, int n_tok, int n_kv,
                                     int hd, unsigned flags, int *status);

/* Grow the library workspace of the CURRENT device so that calls up to these
 * sizes never allocate.  Synchronous; must not be called during capture.
 * A buffer replaced by a larger one is retired, not freed: graphs captured
 * with it keep working until fr_decode_attn_workspace_release.  The pages
 * define no such call; it serves the capture-safety rule above (the
 * development guide's "Caches (all capture-safe)": reserve before capture).
 * Returns FR_OK or a negative fr_status. */
int fr_decode_attn_reserve(int n_inst, int n_head, int n_tok, int n_kv, int hd,
                           unsigned flags);

/* The library workspace of the CURRENT device: its address (NULL if none yet),
 * its size in bytes and how many smaller, retired buffers the library still
 * holds for graphs captured with them.  Any output pointer may be NULL.  A
 * diagnostic the pages do not define (it lets a caller check that a captured
 * graph's workspace is still allocated).  Returns FR_OK or FR_ERR_HIP. */
int fr_decode_attn_workspace_query(void **ptr, size_t *bytes, int *n_retired);

/* Frees every library workspace buffer of the CURRENT device, current and
 * retired, after synchronising the device.  Graphs captured with any of them
 * must not be replayed afterwards; the next call allocates afresh.  Not during
 * capture.  Not defined by the pages (the counterpart of the grow-only rule
 * above, for a caller that is done with the library).  Returns FR_OK or
 * FR_ERR_HIP. */
int fr_decode_attn_workspace_release(void);

/*
 * The launch plan a call with these sizes and flags would use (the same for
 * every query format; pass FR_PLAN_UNMASKED for a call with mask == NULL),
 * for tests and benchmarks.  Not defined by the pages (a diagnostic of how
 * this library splits the work).  Fills up to n_info ints of
 * info[]:
 *   [0] variant (1 fused, 2 decomposed)  [1] key splits per instance
 *   [2] keys per split                   [3] waves per workgroup
 *   [4] 16-row tiles per wave            [5] row blocks per instance
 *   [6] workgroups of the main kernel    [7] kernel launches per call
 * Returns FR_OK or a negative fr_status.
 */
int fr_decode_attn_plan(int n_inst, int n_head, int n_tok, int n_kv, int hd,
                        unsigned flags, int *info, int n_info);

/*
 * Optional kernel timing (not defined by the pages: a measurement aid for the
 * per-call device time and HBM rate of each workload).  When start and stop
 * are both non-NULL (caller-owned hipEvent_t handles passed as void*), every
 * later call on this process records `start` on its stream immediately
 * before its main kernel and `stop` immediately after it: the split kernel of
 * the fused variant, or the whole three- or four-launch sequence of the
 * decomposed one.  hipEventElapsedTime
 * on the pair then gives that kernel's device time.  Pass NULL, NULL to stop.
 * The setting is process-wide; calls on several host threads share it.
 * Returns FR_OK, or FR_ERR_INVALID if exactly one event is NULL.
 */
int fr_decode_attn_profile_events(void *start, void *stop);

/*
 * The step before the window: the query/KV producer ("qkv_post").  FlashRT
 * PR #185 folds the epilogue of the q/k/v projections -- RoPE, the query
 * scale and the f16 materialisations -- into one pass, and its qkv_post
 * handoff commit stores the rope'd, scaled query rows as f16 in exactly the
 * t-major order this window reads (fr_decode_attn_q16 / FR_Q_F16), so no
 * gather runs.  Per instance, token t (position pos[t]) and head:
 *
 *   RoPE, NeoX form: for i < hd/2 the pair (x_i, x_{i+hd/2}) is rotated by
 *   a_i = pos * rope_base^(-2i/hd):  y_i = x_i cos a_i - x_{i+hd/2} sin a_i,
 *   y_{i+hd/2} = x_{i+hd/2} cos a_i + x_i sin a_i.
 *   q16[t][h]           = f16(rope(q) * q_scale)           (query heads)
 *   k_cache[kh][pos[t]] = f16(rope(k)), v_cache[kh][pos[t]] = f16(v)
 *
 * qkv   float32 [n_tok][(n_head + 2*n_kv_head) * hd]: each token's query
 *       heads, then key heads, then value heads (a fused QKV projection row).
 * pos   DEVICE int32 [n_tok] positions (read when the kernel runs, so a
 *       captured graph replays with the current values).
 * q16   binary16 bits [n_tok][n_head][hd].
 * k_cache, v_cache  binary16 bits [n_kv_head][capacity][hd], KV head kh at
 *       + kh*cache_head_stride (>= capacity*hd when n_kv_head > 1); both NULL
 *       to produce q16 only.  Token t's key and value rows go to row pos[t];
 *       positions outside [0, capacity) are not stored.
 * Instance i reads qkv + i*qkv_stride and pos + i*pos_stride (0: shared) and
 * writes q16 + i*q16_stride and the caches + i*cache_stride (ELEMENTS).
 * hd is 64, 80, 128 or 256; 1 <= n_tok <= FR_MAX_TOKENS_UNMASKED; rope_base > 0.
 * Angles are computed in double precision, the rotations in fp32, each output
 * rounded to f16 nearest-even.  No output may overlap an input or another
 * output.  Returns FR_OK or a negative fr_status.
 */
int fr_qkv_post(const float *qkv, const int32_t *pos, uint16_t *q16,
                uint16_t *k_cache, uint16_t *v_cache, int n_inst,
                int64_t qkv_stride, int64_t pos_stride, int64_t q16_stride,
                int64_t cache_stride, int64_t cache_head_stride, int n_head,
                int n_kv_head, int n_tok, int hd, int capacity, float rope_base,
                float q_scale, void *stream);

/*
 * Batched f32 -> f16 row copies (the step after the window's K/V producer).
 * FlashRT PR #185, the commit batching the persistent-KV tail copies: the
 * prefill graph ends with one small f32 -> f16 row copy per layer and KV
 * tensor into the persistent encoder-KV buffers, which this window then reads
 * as K and V; a run of them is one launch, with the same rounding per element.
 *
 * Copy i converts copies[i].n float32 values at copies[i].src to IEEE binary16
 * bits at copies[i].dst, rounding to nearest, ties to even (magnitudes from
 * 65520 up become infinity; NaN inputs give an unspecified NaN).  `copies` is
 * a HOST array of n_copies descriptors (0 <= n_copies <= FR_MAX_COPIES), read
 * during the call only; src and dst are DEVICE pointers (src 4-byte, dst
 * 2-byte aligned; 16-byte alignment of both takes the vector path).  No
 * destination may overlap a source or another destination (FR_ERR_INVALID).
 * Copies with n = 0 are skipped.  Up to 64 copies go in one launch, their
 * descriptors in the kernel arguments, so the call is capture-safe.
 * Returns FR_OK or a negative fr_status.
 */
typedef struct fr_f16_copy {
    const float *src;
    uint16_t *dst;
    int64_t n;
} fr_f16_copy;
#define FR_MAX_COPIES 4096
int fr_f16_copy_batch(const fr_f16_copy *copies, int n_copies, void *stream);

/* Static, human-readable name of a status code.  Not defined by the pages; it
 * names why a call was declined (the development guide's "Adding a fusion
 * window" predicate declines shapes it does not pin, and the caller falls back). */
const char *fr_status_str(int status);

/* ABI version of this header (bumped on incompatible changes).  Not defined by
 * the pages. */
#define FR_DECODE_ATTN_ABI_VERSION 1
int fr_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* FR_DECODE_ATTN_H */
