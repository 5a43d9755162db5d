// fr_probe.hip -- measurement probes for the benchmark, built as libfrprobe.so
// apart from the attention library: the launch floor of an empty kernel, the
// HBM read rate one compute unit and the whole chip reach, LDS read rates, how
// matrix-core and vector-ALU work share a SIMD, and the cost of merging
// key-split partials inside one kernel against a second launch.  None of it is
// on the attention path; bench.py reports what it measures.
//
// Every launch has a fixed, host-checked grid.  The split workgroups never
// wait; the one-launch merges count arrivals and let the last arriver merge,
// except merge_wait_kernel, whose combine workgroups wait for their group's
// count at most 2 ms (every workgroup of its grid fits on the chip at once, so
// the counts arrive long before that).  Every wave finishes on its own.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float float4v __attribute__((ext_vector_type(4)));
typedef uint32_t uint2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint64_t clock100() { return __builtin_amdgcn_s_memrealtime(); }

__global__ void empty_kernel() {}

// Workgroup b reads n16 16-byte granules at src + b*n16 with UNR granules per
// lane in flight (256 lanes: 4 KiB x UNR per workgroup), and records the start
// and end of its reads (100 MHz ticks) in times[2b], times[2b+1].
template <int UNR>
__global__ __launch_bounds__(256) void read_kernel(const float4v *src, int64_t n16,
                                                   uint64_t *times, float *sink) {
  const float4v *p = src + (int64_t)blockIdx.x * n16;
  float acc = 0.f;
  __syncthreads();
  const uint64_t t0 = clock100();
  for (int64_t i = threadIdx.x; i < n16; i += 256 * UNR) {
    float4v v[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int64_t j = i + u * 256;
      v[u] = j < n16 ? p[j] : float4v{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) acc += (v[u].x + v[u].y) + (v[u].z + v[u].w);
  }
  __syncthreads();
  const uint64_t t1 = clock100();
  if (threadIdx.x == 0) {
    times[2 * blockIdx.x] = t0;
    times[2 * blockIdx.x + 1] = t1;
  }
  if (acc == -1.f) sink[blockIdx.x] = acc;   // keeps the loads (the data is never -1 in sum)
}

// Workgroup b reads n16 granules at src + (b % n_region)*n16 twice (the
// workgroups of one region share it, in L2 where they run on one XCD; workgroup
// b runs on XCD b % 8); times[3b .. 3b+2] = start, end of pass 1, end of pass 2.
__global__ __launch_bounds__(512) void shared_read_kernel(const float4v *src, int64_t n16,
                                                          int n_region, uint64_t *times,
                                                          float *sink) {
  const float4v *p = src + (int64_t)(blockIdx.x % n_region) * n16;
  float acc = 0.f;
  uint64_t t[3];
  __syncthreads();
  t[0] = clock100();
  for (int ps = 0; ps < 2; ++ps) {
    for (int64_t i = threadIdx.x; i < n16; i += 512 * 8) {
      float4v v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t j = i + u * 512;
        v[u] = j < n16 ? p[j] : float4v{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) acc += (v[u].x + v[u].y) + (v[u].z + v[u].w);
    }
    __syncthreads();
    t[ps + 1] = clock100();
  }
  if (threadIdx.x == 0) {
    times[3 * blockIdx.x] = t[0];
    times[3 * blockIdx.x + 1] = t[1];
    times[3 * blockIdx.x + 2] = t[2];
  }
  if (acc == -1.f) sink[blockIdx.x] = acc;
}

// LDS read rate of one workgroup of NT lanes: each lane reads 16 bytes per
// ds_read_b128 (KIND 0) or 8 per ds_read_b64_tr_b16 (KIND 1), 16 reads issued
// back to back per trip (the compiler waits for them as their results are
// used), iters trips; times[0], times[1] bracket the reads.
typedef uint32_t uint4v __attribute__((ext_vector_type(4)));
template <int KIND, int NT>
__global__ __launch_bounds__(NT) void lds_read_kernel(uint64_t *times, uint32_t *sink,
                                                      int iters) {
  __shared__ __attribute__((aligned(16))) uint32_t lds[16384];   // 64 KiB
  for (int i = threadIdx.x; i < 16384; i += NT) lds[i] = (uint32_t)i;
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int base = (wave * 256 + lane * 4) & 1023;   // 16-byte slots, uint32 index
  uint32_t acc = 0;
  __syncthreads();
  const uint64_t t0 = clock100();
  for (int it = 0; it < iters; ++it) {
    if (KIND == 0) {
      uint4v r[16];
#pragma unroll
      for (int u = 0; u < 16; ++u)
        r[u] = *(const uint4v *)&lds[(base + u * 1024 + it) & 16380];
#pragma unroll
      for (int u = 0; u < 16; ++u) acc ^= r[u].x ^ r[u].w;
    } else {
      typedef __attribute__((__vector_size__(4 * sizeof(__fp16)))) __fp16 fp16x4;
      fp16x4 r[16];
#pragma unroll
      for (int u = 0; u < 16; ++u)
        r[u] = __builtin_amdgcn_ds_read_tr16_b64_v4f16(
            (__attribute__((address_space(3))) fp16x4 *)&lds[(base + u * 1024 + 2 * it) & 16382]);
#pragma unroll
      for (int u = 0; u < 16; ++u) acc ^= __builtin_bit_cast(uint2v, r[u]).x;
    }
  }
  __syncthreads();
  const uint64_t t1 = clock100();
  if (threadIdx.x == 0) {
    times[0] = t0;
    times[1] = t1;
  }
  if (acc == 0xdeadbeefu) sink[0] = acc;
}

// ---- issue probe: how matrix-core (MFMA) and vector-ALU work share a SIMD.
// One workgroup of NT lanes (one or two waves per SIMD); each trip of a wave:
//   MODE 0: 8 v_mfma_f32_16x16x32_f16 (four accumulation chains)
//   MODE 1: 32 independent fp32 fma
//   MODE 2: both, interleaved in the same wave
//   MODE 3: (two waves per SIMD) waves 0-3 the 32 fma, waves 4-7 the 8 MFMAs
// times[0], times[1] bracket `iters` trips (100 MHz counter).
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
template <int MODE, int NT>
__global__ __launch_bounds__(NT) void issue_kernel(uint64_t *times, float *sink, int iters) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const half8 a = {(_Float16)(lane * 1e-3f), 0, 0, 0, 0, 0, 0, (_Float16)1};
  const half8 b = {(_Float16)1, 0, 0, 0, 0, 0, 0, (_Float16)(lane * 1e-3f)};
  float4v c[4] = {};
  float x[32];
  for (int i = 0; i < 32; ++i) x[i] = lane * 1e-3f + i;
  const bool do_m = MODE == 0 || MODE == 2 || (MODE == 3 && wave >= 4);
  const bool do_v = MODE == 1 || MODE == 2 || (MODE == 3 && wave < 4);
  __syncthreads();
  const uint64_t t0 = clock100();
  if (do_m && do_v) {
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        c[k & 3] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c[k & 3], 0, 0, 0);
#pragma unroll
        for (int i = 4 * k; i < 4 * k + 4; ++i) x[i] = __builtin_fmaf(x[i], 0.999f, 0.5f);
      }
    }
  } else if (do_m) {
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int k = 0; k < 8; ++k)
        c[k & 3] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c[k & 3], 0, 0, 0);
    }
  } else if (do_v) {
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int i = 0; i < 32; ++i) x[i] = __builtin_fmaf(x[i], 0.999f, 0.5f);
    }
  }
  __syncthreads();
  const uint64_t t1 = clock100();
  if (threadIdx.x == 0) {
    times[0] = t0;
    times[1] = t1;
  }
  float acc = c[0][0] + c[1][1] + c[2][2] + c[3][3];
  for (int i = 0; i < 32; ++i) acc += x[i];
  if (acc == 1234.5f) sink[0] = acc;
}

// ---- merge probe.  kMergeGrid workgroups of 256 lanes form groups of n_split
// (a key split's workgroups of one row block).  Each reads its own 64 KiB of
// work input, then writes a partial of kPartFloats floats (48 KiB: the partial
// of a 48-row, hd-256 row block) with value(c) = (iter*131 + s*7 + c) % 1021.
// The merged output of group g is the sum over its splits.
//   MODE 0: nothing more; merge_combine_kernel runs as a second launch
//   MODE 1: one launch; an agent-scope acquire-release arrival count (the
//           compiler's fences: L2 write-back before, invalidate after), the
//           last arriver reads the partials with ordinary loads
//   MODE 2: one launch; partials stored and read back at device coherence
//           (sc1, no write-back or invalidate of the whole L2), relaxed count
//   MODE 3: one launch; the partial is cut into n_split column slices, each
//           with its own arrival count; split s publishes slices s, s+1, ...
//           (mod n_split) one by one, and the last publisher of a slice
//           merges that slice (the merge spread over the group, no waiting)
//   (merge_wait_kernel: one launch with extra combine workgroups after the
//   split workgroups, each waiting -- bounded -- for its group's count)
constexpr int kMergeGrid = 256;
constexpr int kPartFloats = 12288;
constexpr int kWorkGranules = 4096;   // 64 KiB per workgroup

template <int MODE>
__global__ __launch_bounds__(256) void merge_kernel(const float4v *work, float *part, int *cnt,
                                                    float *out, int n_split, int iter) {
  const int g = blockIdx.x / n_split, s = blockIdx.x % n_split;
  const int tid = threadIdx.x;
  const float4v *wp = work + (int64_t)blockIdx.x * kWorkGranules;
  float4v v[16];
#pragma unroll
  for (int u = 0; u < 16; ++u) v[u] = wp[u * 256 + tid];
  float acc = 0.f;
#pragma unroll
  for (int u = 0; u < 16; ++u) acc += (v[u].x + v[u].y) + (v[u].z + v[u].w);
  acc *= 0.f;   // the work input is zero; the value still depends on the loads
  float *pp = part + ((int64_t)g * n_split + s) * kPartFloats;
  const __amdgpu_buffer_rsrc_t rp =
      __builtin_amdgcn_make_buffer_rsrc(pp, 0, kPartFloats * 4, 0x00020000);
#pragma unroll
  for (int u = 0; u < (MODE == 3 ? 0 : kPartFloats / 4 / 256); ++u) {
    const int c4 = u * 256 + tid;
    float4v x;
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = (float)((iter * 131 + s * 7 + 4 * c4 + e) % 1021) + acc;
    if (MODE == 2)
      __builtin_amdgcn_raw_buffer_store_b128(x, rp, c4 * 16, 0, 16 /* sc1 */);
    else
      *(float4v *)(pp + 4 * c4) = x;
  }
  if (MODE == 0) return;
  __shared__ int s_old;
  if (MODE == 3) {
    // slices of w floats; counts cnt[g * n_split + slice]
    const int w = kPartFloats / n_split;
    for (int k = 0; k < n_split; ++k) {
      const int sl = (s + k) % n_split;
      for (int c = tid; c < w / 4; c += 256) {
        const int c4 = sl * (w / 4) + c;
        float4v x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = (float)((iter * 131 + s * 7 + 4 * c4 + e) % 1021) + acc;
        __builtin_amdgcn_raw_buffer_store_b128(x, rp, c4 * 16, 0, 16 /* sc1 */);
      }
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (tid == 0)
        s_old = __hip_atomic_fetch_add(cnt + g * n_split + sl, 1, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
      if (s_old == n_split - 1) {   // the last publisher merges the slice
        for (int c = tid; c < w / 4; c += 256) {
          const int c4 = sl * (w / 4) + c;
          float4v sum = {0.f, 0.f, 0.f, 0.f};
          for (int j = 0; j < n_split; ++j) {
            const float *src = part + ((int64_t)g * n_split + j) * kPartFloats;
            const __amdgpu_buffer_rsrc_t r =
                __builtin_amdgcn_make_buffer_rsrc((void *)src, 0, kPartFloats * 4, 0x00020000);
            sum += __builtin_amdgcn_raw_buffer_load_b128(r, c4 * 16, 0, 16 /* sc1 */);
          }
          *(float4v *)(out + (int64_t)g * kPartFloats + 4 * c4) = sum;
        }
        if (tid == 0) cnt[g * n_split + sl] = 0;
      }
      __syncthreads();
    }
    return;
  }
  if (MODE == 1) {
    __syncthreads();
    if (tid == 0)
      s_old = __hip_atomic_fetch_add(cnt + g, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
  } else {
    __builtin_amdgcn_s_waitcnt(0);   // this lane's partial stores have completed
    __syncthreads();
    if (tid == 0)
      s_old = __hip_atomic_fetch_add(cnt + g, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
  }
  if (s_old != n_split - 1) return;
  // the last arriver: every column of the group, 8 splits' loads in flight
  for (int u = 0; u < kPartFloats / 4 / 256; ++u) {
    const int c4 = u * 256 + tid;
    float4v sum = {0.f, 0.f, 0.f, 0.f};
    for (int j0 = 0; j0 < n_split; j0 += 8) {
      float4v x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        x[j] = float4v{0.f, 0.f, 0.f, 0.f};
        if (j0 + j < n_split) {
          const float *src = part + ((int64_t)g * n_split + j0 + j) * kPartFloats;
          if (MODE == 1) {
            x[j] = *(const float4v *)(src + 4 * c4);
          } else {
            const __amdgpu_buffer_rsrc_t r =
                __builtin_amdgcn_make_buffer_rsrc((void *)src, 0, kPartFloats * 4, 0x00020000);
            x[j] = __builtin_amdgcn_raw_buffer_load_b128(r, c4 * 16, 0, 16 /* sc1 */);
          }
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) sum += x[j];
    }
    *(float4v *)(out + (int64_t)g * kPartFloats + 4 * c4) = sum;
  }
  if (tid == 0) cnt[g] = 0;   // ready for the next launch
}

// One launch: kMergeGrid split workgroups (partials stored sc1, one count per
// group) followed by (groups x 12) combine workgroups, each waiting for its
// group's count -- at most 2 ms, then it gives up and merges what is there --
// before merging 1024 columns with sc1 loads.  The split workgroups never
// wait, and every workgroup of the grid fits on the chip at once, so each wait
// ends when the counts arrive.  The group's last combine workgroup resets its
// counts (cnt[kMergeGrid + g] counts finished combine workgroups).
__global__ __launch_bounds__(256) void merge_wait_kernel(const float4v *work, float *part,
                                                         int *cnt, float *out, int n_split,
                                                         int iter) {
  const int tid = threadIdx.x;
  constexpr int kCb = kPartFloats / 1024;
  if ((int)blockIdx.x < kMergeGrid) {
    const int g = blockIdx.x / n_split, s = blockIdx.x % n_split;
    const float4v *wp = work + (int64_t)blockIdx.x * kWorkGranules;
    float4v v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) v[u] = wp[u * 256 + tid];
    float acc = 0.f;
#pragma unroll
    for (int u = 0; u < 16; ++u) acc += (v[u].x + v[u].y) + (v[u].z + v[u].w);
    acc *= 0.f;
    float *pp = part + ((int64_t)g * n_split + s) * kPartFloats;
    const __amdgpu_buffer_rsrc_t rp =
        __builtin_amdgcn_make_buffer_rsrc(pp, 0, kPartFloats * 4, 0x00020000);
#pragma unroll
    for (int u = 0; u < kPartFloats / 4 / 256; ++u) {
      const int c4 = u * 256 + tid;
      float4v x;
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = (float)((iter * 131 + s * 7 + 4 * c4 + e) % 1021) + acc;
      __builtin_amdgcn_raw_buffer_store_b128(x, rp, c4 * 16, 0, 16 /* sc1 */);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) __hip_atomic_fetch_add(cnt + g, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  const int c = blockIdx.x - kMergeGrid, g = c / kCb, cb = c % kCb;
  if (tid == 0) {
    const uint64_t t0 = clock100();
    while (__hip_atomic_load(cnt + g, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < n_split &&
           clock100() - t0 < 200000)
      __builtin_amdgcn_s_sleep(60);
  }
  __syncthreads();
  const int c4 = cb * 256 + tid;
  float4v sum = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < n_split; ++j) {
    const float *src = part + ((int64_t)g * n_split + j) * kPartFloats;
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc((void *)src, 0, kPartFloats * 4, 0x00020000);
    sum += __builtin_amdgcn_raw_buffer_load_b128(r, c4 * 16, 0, 16 /* sc1 */);
  }
  *(float4v *)(out + (int64_t)g * kPartFloats + 4 * c4) = sum;
  __syncthreads();
  if (tid == 0) {
    const int f = __hip_atomic_fetch_add(cnt + kMergeGrid + g, 1, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    if (f == kCb - 1) {
      cnt[g] = 0;
      cnt[kMergeGrid + g] = 0;
    }
  }
}

// the second launch of MODE 0: one workgroup per (group, 1024 columns)
__global__ __launch_bounds__(256) void merge_combine_kernel(const float *part, float *out,
                                                            int n_split) {
  const int g = blockIdx.x / (kPartFloats / 1024), cb = blockIdx.x % (kPartFloats / 1024);
  const int c4 = cb * 256 + threadIdx.x;
  float4v sum = {0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 < n_split; j0 += 8) {
    float4v x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      x[j] = j0 + j < n_split
                 ? *(const float4v *)(part + ((int64_t)g * n_split + j0 + j) * kPartFloats + 4 * c4)
                 : float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 8; ++j) sum += x[j];
  }
  *(float4v *)(out + (int64_t)g * kPartFloats + 4 * c4) = sum;
}

}  // namespace

extern "C" {

// n back-to-back launches of an empty kernel of `grid` workgroups of 64 lanes.
int frp_empty(int grid, int n, void *stream) {
  if (grid < 1 || grid > 65536 || n < 0) return -1;
  for (int i = 0; i < n; ++i)
    hipLaunchKernelGGL(empty_kernel, dim3(grid), dim3(64), 0, (hipStream_t)stream);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

// n_wg workgroups, each reading bytes_per_wg bytes (a multiple of 16) of src
// from src + b*bytes_per_wg with 8 or 32 granules per lane in flight; times
// receives 2*n_wg start/end ticks (100 MHz).  The caller's buffers must hold
// n_wg*bytes_per_wg bytes (src), 2*n_wg uint64 (times) and n_wg floats (sink).
int frp_read(const void *src, int64_t bytes_per_wg, int n_wg, int unroll, uint64_t *times,
             float *sink, void *stream) {
  if (!src || !times || !sink || n_wg < 1 || n_wg > 65536 || bytes_per_wg < 16 ||
      bytes_per_wg % 16 || ((uintptr_t)src % 16))
    return -1;
  const int64_t n16 = bytes_per_wg / 16;
  if (unroll == 8)
    hipLaunchKernelGGL(read_kernel<8>, dim3(n_wg), dim3(256), 0, (hipStream_t)stream,
                       (const float4v *)src, n16, times, sink);
  else if (unroll == 32)
    hipLaunchKernelGGL(read_kernel<32>, dim3(n_wg), dim3(256), 0, (hipStream_t)stream,
                       (const float4v *)src, n16, times, sink);
  else
    return -1;
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

// n_wg workgroups of 512 lanes, workgroup b reading (twice) the bytes_per_wg
// bytes at src + (b % n_region)*bytes_per_wg; src must hold
// n_region*bytes_per_wg bytes, times 3*n_wg uint64, sink n_wg floats.
int frp_read_shared(const void *src, int64_t bytes_per_wg, int n_wg, int n_region,
                    uint64_t *times, float *sink, void *stream) {
  if (!src || !times || !sink || n_wg < 1 || n_wg > 65536 || n_region < 1 ||
      bytes_per_wg < 16 || bytes_per_wg % 16 || ((uintptr_t)src % 16))
    return -1;
  hipLaunchKernelGGL(shared_read_kernel, dim3(n_wg), dim3(512), 0, (hipStream_t)stream,
                     (const float4v *)src, bytes_per_wg / 16, n_region, times, sink);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

// One workgroup reading LDS: kind 0 = ds_read_b128, 1 = ds_read_b64_tr_b16;
// 256 or 512 lanes (one or two waves per SIMD); times 2 uint64, sink 1 uint32.
int frp_lds(int kind, int lanes, int iters, uint64_t *times, uint32_t *sink, void *stream) {
  if (!times || !sink || iters < 1 || (kind != 0 && kind != 1) || (lanes != 256 && lanes != 512))
    return -1;
  hipStream_t s = (hipStream_t)stream;
  if (kind == 0 && lanes == 256)
    hipLaunchKernelGGL((lds_read_kernel<0, 256>), dim3(1), dim3(256), 0, s, times, sink, iters);
  else if (kind == 0)
    hipLaunchKernelGGL((lds_read_kernel<0, 512>), dim3(1), dim3(512), 0, s, times, sink, iters);
  else if (lanes == 256)
    hipLaunchKernelGGL((lds_read_kernel<1, 256>), dim3(1), dim3(256), 0, s, times, sink, iters);
  else
    hipLaunchKernelGGL((lds_read_kernel<1, 512>), dim3(1), dim3(512), 0, s, times, sink, iters);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

// One workgroup of the issue probe: mode 0..2 with 256 or 512 lanes, mode 3
// with 512; times 2 uint64, sink 1 float.
int frp_issue(int mode, int lanes, int iters, uint64_t *times, float *sink, void *stream) {
  if (!times || !sink || iters < 1 || mode < 0 || mode > 3 || (lanes != 256 && lanes != 512) ||
      (mode == 3 && lanes != 512))
    return -1;
  hipStream_t s = (hipStream_t)stream;
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(1), dim3(lanes), 0, s, times, sink, iters);
  };
  if (lanes == 256) {
    if (mode == 0) go(issue_kernel<0, 256>);
    if (mode == 1) go(issue_kernel<1, 256>);
    if (mode == 2) go(issue_kernel<2, 256>);
  } else {
    if (mode == 0) go(issue_kernel<0, 512>);
    if (mode == 1) go(issue_kernel<1, 512>);
    if (mode == 2) go(issue_kernel<2, 512>);
    if (mode == 3) go(issue_kernel<3, 512>);
  }
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

// Sizes the merge probe needs: grid, floats per partial, work bytes per workgroup.
void frp_merge_sizes(int *grid, int *partial_floats, int *work_bytes_per_wg) {
  *grid = kMergeGrid;
  *partial_floats = kPartFloats;
  *work_bytes_per_wg = kWorkGranules * 16;
}

// One merge-probe call (mode 0: two launches; 1, 2, 3: one launch, the last
// arriver merges; 4: one launch with waiting combine workgroups).  Buffers:
// work kMergeGrid*64 KiB (zero), part and out kMergeGrid*kPartFloats floats,
// cnt 2*kMergeGrid ints (zero before the first call; every call leaves them zero).
int frp_merge(int mode, const void *work, float *part, int *cnt, float *out, int n_split,
              int iter, void *stream) {
  if (!work || !part || !cnt || !out || n_split < 1 || n_split > 64 ||
      kMergeGrid % n_split || iter < 0)
    return -1;
  hipStream_t s = (hipStream_t)stream;
  const float4v *w = (const float4v *)work;
  switch (mode) {
    case 0:
      hipLaunchKernelGGL(merge_kernel<0>, dim3(kMergeGrid), dim3(256), 0, s, w, part, cnt, out,
                         n_split, iter);
      hipLaunchKernelGGL(merge_combine_kernel, dim3(kMergeGrid / n_split * (kPartFloats / 1024)),
                         dim3(256), 0, s, part, out, n_split);
      break;
    case 1:
      hipLaunchKernelGGL(merge_kernel<1>, dim3(kMergeGrid), dim3(256), 0, s, w, part, cnt, out,
                         n_split, iter);
      break;
    case 2:
      hipLaunchKernelGGL(merge_kernel<2>, dim3(kMergeGrid), dim3(256), 0, s, w, part, cnt, out,
                         n_split, iter);
      break;
    case 3:
      if (kPartFloats % (4 * n_split)) return -1;   // whole float4 slices
      hipLaunchKernelGGL(merge_kernel<3>, dim3(kMergeGrid), dim3(256), 0, s, w, part, cnt, out,
                         n_split, iter);
      break;
    case 4:
      hipLaunchKernelGGL(merge_wait_kernel,
                         dim3(kMergeGrid + kMergeGrid / n_split * (kPartFloats / 1024)),
                         dim3(256), 0, s, w, part, cnt, out, n_split, iter);
      break;
    default:
      return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
