// Per-tensor current scaling into OCP E4M3.
//
//   amax = max |v|;  scale = 448 / amax (float32; 1 when amax is 0 or so
//   small that the quotient overflows);
//   code = E4M3(clamp(fl32(v * scale), -448, 448)), round to nearest even;
//   scale_inv = 1 / scale (float32).
//
// Two passes without atomics, so the result is independent of scheduling:
// amax_partial_kernel writes one maximum per workgroup; quantize_kernel has
// every workgroup reduce those partials in the same order (every workgroup
// obtains the same amax and scale), then converts its share of the tensor.
// The fp8 forward's fc1 epilogue writes the partials itself, so only the
// second pass runs there. Divisions are IEEE (correctly rounded) float32.
#pragma once

#include "common.h"

namespace tpmlp {

constexpr int kQuantThreads = 256;
constexpr int kQuantMaxParts = 1024;
constexpr int kQuantVec = 8;  // elements per thread per iteration

template <typename SrcT>
__device__ __forceinline__ void load8(const SrcT* src, int64_t i, int64_t n, float (&v)[8]) {
  if (i + 8 <= n) {
    if constexpr (sizeof(SrcT) == 2) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(src + i);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[2 * q] = bf2f((bf16_t)(w[q] & 0xffffu));
        v[2 * q + 1] = bf2f((bf16_t)(w[q] >> 16));
      }
    } else {
      const f32x4 a = *reinterpret_cast<const f32x4*>(src + i);
      const f32x4 b = *reinterpret_cast<const f32x4*>(src + i + 4);
#pragma unroll
      for (int q = 0; q < 4; ++q) { v[q] = a[q]; v[q + 4] = b[q]; }
    }
  } else {
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = (i + q < n) ? Elem<SrcT>::load(src, i + q) : 0.f;
  }
}

template <typename SrcT>
__global__ void __launch_bounds__(kQuantThreads) amax_partial_kernel(const SrcT* src, int64_t n,
                                                                     float* partial) {
  float m = 0.f;
  const int64_t stride = (int64_t)gridDim.x * kQuantThreads * kQuantVec;
  for (int64_t i = ((int64_t)blockIdx.x * kQuantThreads + threadIdx.x) * kQuantVec; i < n;
       i += stride) {
    float v[8];
    load8(src, i, n, v);
#pragma unroll
    for (int q = 0; q < 8; ++q) m = __builtin_fmaxf(m, __builtin_fabsf(v[q]));
  }
  m = wave_max(m);
  __shared__ float wm[kQuantThreads / 64];
  if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float r = 0.f;
    for (int w = 0; w < kQuantThreads / 64; ++w) r = __builtin_fmaxf(r, wm[w]);
    partial[blockIdx.x] = r;
  }
}

// E5: quantise to OCP E5M2 (largest finite 57344) instead of E4M3 (448).
template <typename SrcT, bool E5>
__global__ void __launch_bounds__(kQuantThreads) quantize_kernel(const SrcT* src, int64_t n,
                                                                 uint8_t* dst, const float* partial,
                                                                 int nparts, float* amax_out,
                                                                 float* scale_inv_out) {
  constexpr float kFmax = E5 ? 57344.0f : 448.0f;
  // every workgroup reduces the partials identically
  float m = 0.f;
  for (int p = threadIdx.x; p < nparts; p += kQuantThreads) m = __builtin_fmaxf(m, partial[p]);
  m = wave_max(m);
  __shared__ float wm[kQuantThreads / 64];
  if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = m;
  __syncthreads();
  float amax = 0.f;
  for (int w = 0; w < kQuantThreads / 64; ++w) amax = __builtin_fmaxf(amax, wm[w]);
  // 1 for an amax of 0 or infinity, and for one so small that kFmax / amax
  // overflows (a factor of infinity would make zeros NaN and scale_inv 0)
  float scale = (amax > 0.f && amax <= 3.4028234663852886e38f) ? kFmax / amax : 1.0f;
  if (!(scale <= 3.4028234663852886e38f)) scale = 1.0f;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    *amax_out = amax;
    *scale_inv_out = 1.0f / scale;
  }
  const int64_t stride = (int64_t)gridDim.x * kQuantThreads * kQuantVec;
  for (int64_t i = ((int64_t)blockIdx.x * kQuantThreads + threadIdx.x) * kQuantVec; i < n;
       i += stride) {
    float v[8];
    load8(src, i, n, v);
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] *= scale;
    const u32x2 w = pack_fp8x8<E5>(v);
    const uint32_t lo = w[0], hi = w[1];
    if (i + 8 <= n) {
      *reinterpret_cast<u32x2*>(dst + i) = u32x2{lo, hi};
    } else {
      for (int q = 0; q < 8 && i + q < n; ++q)
        dst[i + q] = (uint8_t)(((q < 4 ? lo : hi) >> (8 * (q & 3))) & 0xffu);
    }
  }
}

// One step of delayed scaling of a tensor whose per-workgroup amaxes are in
// partial[0 .. nparts): amax = their maximum; history <- [amax, history[0 ..
// len-2]] (newest first); *scale_inv = 1 / *scale (the factor the tensor was
// quantised with); *scale <- fmax / max(history), kept while that maximum is
// 0 or not finite, or so small that the quotient overflows. One workgroup,
// all float32; max is exact, so the result does not depend on the order of
// the partials.
constexpr int kMaxHistory = 4096;
__global__ void __launch_bounds__(kQuantThreads) delayed_update_kernel(const float* partial,
                                                                       int nparts, float* history,
                                                                       int len, float* scale,
                                                                       float* scale_inv,
                                                                       float fmax) {
  __shared__ float old[kMaxHistory];
  __shared__ float wm[kQuantThreads / 64];
  float m = 0.f;
  for (int p = threadIdx.x; p < nparts; p += kQuantThreads) m = __builtin_fmaxf(m, partial[p]);
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = m;
  for (int i = threadIdx.x; i < len; i += kQuantThreads) old[i] = history[i];
  __syncthreads();
  float amax = 0.f;
  for (int w = 0; w < kQuantThreads / 64; ++w) amax = __builtin_fmaxf(amax, wm[w]);
  __syncthreads();  // every wave has read wm
  float hm = 0.f;
  for (int i = threadIdx.x; i < len; i += kQuantThreads) {
    const float v = i == 0 ? amax : old[i - 1];
    history[i] = v;
    hm = __builtin_fmaxf(hm, v);
  }
  // max |.| of a history that may hold infinities: fmax ignores NaN only
  hm = wave_max(hm);
  if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = hm;
  __syncthreads();
  if (threadIdx.x == 0) {
    float hmax = 0.f;
    for (int w = 0; w < kQuantThreads / 64; ++w) hmax = __builtin_fmaxf(hmax, wm[w]);
    const float used = *scale;
    *scale_inv = 1.0f / used;
    // kept while the maximum is 0 or infinite, or so small that the next
    // factor would overflow
    const float next = (hmax > 0.f && hmax <= 3.4028234663852886e38f) ? fmax / hmax : used;
    *scale = (next <= 3.4028234663852886e38f) ? next : used;
  }
}

}  // namespace tpmlp
