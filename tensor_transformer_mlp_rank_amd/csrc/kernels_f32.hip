// Instantiations and launchers of the fp32 (VALU) tile kernel, of the
// E4M3 quantiser, of the reduction of the MFMA kernel's column-sum partials
// and of the activation's recomputation from the saved pre-activation.
#include "gemm_f32.h"
#include "launch.h"
#include "quant.h"

namespace tpmlp {

namespace {

template <bool A_K, bool B_K, int EPI, bool COLSUM>
hipError_t launch_f32(const GemmArgs& g, const EpiArgs& e, hipStream_t s) {
  const int nb = g.tiles_m * g.tiles_n;
  hipLaunchKernelGGL((gemm_f32_kernel<A_K, B_K, EPI, COLSUM>), dim3(nb), dim3(kF32Threads), 0, s,
                     g, e);
  return hipGetLastError();
}

// out[m] = (out[m] if accumulate) + sum over r of part[r][m]. A workgroup
// takes 64 columns; its four waves each add every fourth row (r = w, w + 4,
// ...), loads issued eight at a time, and wave 0 adds the four sums in wave
// order: a fixed order, so the result is reproducible bit for bit.
// Groups (blockIdx.y) are independent: group y reads part + y * nparts * M
// and writes out + y * M.
__global__ void __launch_bounds__(256) colsum_reduce_kernel(const float* __restrict__ part,
                                                            int nparts, int M,
                                                            float* __restrict__ out,
                                                            int accumulate) {
  __shared__ float red[4][64];
  part += (int64_t)blockIdx.y * nparts * M;
  out += (int64_t)blockIdx.y * M;
  const int c = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int m = blockIdx.x * 64 + c;
  float s = 0.f;
  if (m < M) {
    int r = w;
    for (; r + 28 < nparts; r += 32) {
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = part[(int64_t)(r + 4 * i) * M + m];
#pragma unroll
      for (int i = 0; i < 8; ++i) s += v[i];
    }
    for (; r < nparts; r += 4) s += part[(int64_t)r * M + m];
  }
  red[w][c] = s;
  __syncthreads();
  if (w == 0 && m < M) {
    const float t = ((red[0][c] + red[1][c]) + red[2][c]) + red[3][c];
    out[m] = accumulate ? out[m] + t : t;
  }
}

// Split-K: the sum of the fp32 partial planes part[s][M][N] in split order,
// then the product's own epilogue: bf16 out = sum (+ bias[col]), or fp32 out
// = sum (+ the old out when accumulating). Eight consecutive elements per
// thread (N is a multiple of 16).
__global__ void __launch_bounds__(256) splitk_reduce_kernel(const float* __restrict__ part,
                                                            int splits, int64_t plane, int N,
                                                            void* __restrict__ out, int out_bf16,
                                                            const bf16_t* __restrict__ bias,
                                                            int accumulate) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (i >= plane) return;
  float v[8];
  Elem<float>::load8(part, i, v);
  for (int s = 1; s < splits; ++s) {
    float w[8];
    Elem<float>::load8(part + (int64_t)s * plane, i, w);
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] += w[u];
  }
  if (out_bf16) {
    if (bias) {
      const int col = (int)(i % N);
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] += bf2f(bias[col + u]);
    }
    Elem<bf16_t>::store8(out, i, v);
  } else {
    if (accumulate) {
      float o[8];
      Elem<float>::load8(out, i, o);
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] += o[u];
    }
    Elem<float>::store8(out, i, v);
  }
}

// a = act(h) for the weight gradients' recomputation: h is the saved
// pre-activation [rows][G fs] (G = 2 for SwiGLU, gate then up), a goes to
// [rows][fs] as bf16 or fp32 (OUT_E4M3 false: the type of h), or as E4M3
// codes at the factor 1 / *scale_inv (OUT_E4M3). The activation is the
// forward epilogue's own function of h as stored (gelu_f; silu_f(gate) * up),
// so bf16 and fp32 results equal the forward's a bit for bit. Eight
// consecutive elements per thread, grid-stride.
template <typename T, bool SWIGLU, bool OUT_E4M3>
__global__ void __launch_bounds__(256) act_recompute_kernel(const T* __restrict__ h, int64_t rows,
                                                            int64_t fs, void* __restrict__ a,
                                                            const float* __restrict__ scale_inv) {
  const int64_t per_row = fs / 8;
  const int64_t groups = rows * per_row;
  const int64_t ldh = SWIGLU ? 2 * fs : fs;
  float qs = 1.0f;
  if constexpr (OUT_E4M3) qs = 1.0f / *scale_inv;
  for (int64_t gi = (int64_t)blockIdx.x * 256 + threadIdx.x; gi < groups;
       gi += (int64_t)gridDim.x * 256) {
    const int64_t r = gi / per_row, c = (gi - r * per_row) * 8;
    const int64_t hi = r * ldh + c;
    float v[8];
    Elem<T>::load8(h, hi, v);
    if constexpr (SWIGLU) {
      float up[8];
      Elem<T>::load8(h, hi + fs, up);
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = silu_f(v[u]) * up[u];
    } else {
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = gelu_f(v[u]);
    }
    const int64_t ai = r * fs + c;
    if constexpr (OUT_E4M3) {
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] *= qs;
      *reinterpret_cast<u32x2*>(static_cast<uint8_t*>(a) + ai) = pack_fp8x8<false>(v);
    } else {
      Elem<T>::store8(a, ai, v);
    }
  }
}

__global__ void __launch_bounds__(256) fill_zero_i32_kernel(int* __restrict__ p, int n) {
  for (int i = (int)(blockIdx.x * 256 + threadIdx.x); i < n; i += (int)(gridDim.x * 256)) p[i] = 0;
}

// Byte transpose: dst[c][r] = src[r][c] for src [rows][cols] (cols a
// multiple of 16), dst [cols][ld] (ld a multiple of 16, at least rows), the
// columns r in [rows, ld) of dst zero. One 64 x 64 tile per block: each
// thread loads 16 bytes of a source row into LDS, then gathers 16 bytes of
// one source column (a destination row) and stores them with one 16-byte
// store.
__global__ void __launch_bounds__(256) transpose_u8_kernel(const uint8_t* __restrict__ src,
                                                           int64_t rows, int64_t cols,
                                                           uint8_t* __restrict__ dst, int64_t ld) {
  __shared__ uint8_t tile[64][64 + 4];
  const int t = threadIdx.x, q = t >> 2, k = t & 3;
  const int64_t r0 = (int64_t)blockIdx.x * 64, c0 = (int64_t)blockIdx.y * 64;
  {
    const int64_t r = r0 + q, c = c0 + 16 * k;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r < rows && c < cols) v = *reinterpret_cast<const u32x4*>(src + r * cols + c);
#pragma unroll
    for (int j = 0; j < 4; ++j) *reinterpret_cast<uint32_t*>(&tile[q][16 * k + 4 * j]) = v[j];
  }
  __syncthreads();
  const int64_t c = c0 + q, r = r0 + 16 * k;  // destination row c, bytes r .. r+15
  if (c < cols && r < ld) {
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t w = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) w |= (uint32_t)tile[16 * k + 4 * j + b][q] << (8 * b);
      o[j] = w;
    }
    *reinterpret_cast<u32x4*>(dst + c * ld + r) = o;
  }
}

// db1 from a token-contiguous E5M2 dH^T [rows][ld]: out[f] (+)= scale_inv *
// sum over t < n of decode(dH^T[f][t]); one block per row, a fixed order of
// the partial sums (reproducible bit for bit).
__global__ void __launch_bounds__(256) rowsum_e5m2_kernel(const uint8_t* __restrict__ src,
                                                          int64_t n, int64_t ld,
                                                          const float* __restrict__ scale_inv,
                                                          float* __restrict__ out, int accumulate) {
  const uint8_t* row = src + (int64_t)blockIdx.x * ld;
  float s = 0.f;
  for (int64_t i = 16 * (int64_t)threadIdx.x; i < n; i += 16 * 256) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(row + i);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const auto lo = __builtin_amdgcn_cvt_pk_f32_bf8((int)v[j], false);
      const auto hi = __builtin_amdgcn_cvt_pk_f32_bf8((int)v[j], true);
      const float e[4] = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
      for (int b = 0; b < 4; ++b)
        if (i + 4 * j + b < n) s += e[b];
    }
  }
  __shared__ float red[256];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const float v = red[0] * *scale_inv;
    out[blockIdx.x] = accumulate ? out[blockIdx.x] + v : v;
  }
}

}  // namespace

hipError_t transpose_u8_launch(const void* src, int64_t rows, int64_t cols, void* dst, int64_t ld,
                               hipStream_t s) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  const int64_t gx = (rows + 63) / 64, gy = (cols + 63) / 64;
  if (gx > 0x7fffffff || gy > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(transpose_u8_kernel, dim3((unsigned)gx, (unsigned)gy), dim3(256), 0, s,
                     static_cast<const uint8_t*>(src), rows, cols, static_cast<uint8_t*>(dst), ld);
  return hipGetLastError();
}

hipError_t rowsum_e5m2_launch(const void* src, int64_t rows, int64_t n, int64_t ld,
                              const float* scale_inv, float* out, int accumulate, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(rowsum_e5m2_kernel, dim3((unsigned)rows), dim3(256), 0, s,
                     static_cast<const uint8_t*>(src), n, ld, scale_inv, out, accumulate);
  return hipGetLastError();
}

hipError_t fill_zero_i32_launch(int* p, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int nb = (n + 255) / 256 > 64 ? 64 : (n + 255) / 256;
  hipLaunchKernelGGL(fill_zero_i32_kernel, dim3(nb), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t act_recompute_launch(Kind kind, bool swiglu, const void* h, int64_t rows, int64_t fs,
                                void* a, const float* scale_inv, hipStream_t s) {
  const int64_t groups = rows * (fs / 8);
  if (groups <= 0) return hipSuccess;
  const int64_t want = (groups + 255) / 256;
  const unsigned nb = (unsigned)(want > 4096 ? 4096 : want);
  auto go = [&](auto kernel, const auto* hp) {
    hipLaunchKernelGGL(kernel, dim3(nb), dim3(256), 0, s, hp, rows, fs, a, scale_inv);
  };
  if (kind == KIND_F32) {
    const float* hp = static_cast<const float*>(h);
    if (swiglu) go(act_recompute_kernel<float, true, false>, hp);
    else go(act_recompute_kernel<float, false, false>, hp);
  } else {
    const bf16_t* hp = static_cast<const bf16_t*>(h);
    if (kind == KIND_E4M3) {
      if (swiglu) go(act_recompute_kernel<bf16_t, true, true>, hp);
      else go(act_recompute_kernel<bf16_t, false, true>, hp);
    } else if (swiglu) {
      go(act_recompute_kernel<bf16_t, true, false>, hp);
    } else {
      go(act_recompute_kernel<bf16_t, false, false>, hp);
    }
  }
  return hipGetLastError();
}

hipError_t splitk_reduce_launch(const float* part, int splits, int64_t M, int64_t N, void* out,
                                bool out_bf16, const void* bias, int accumulate, hipStream_t s) {
  const int64_t plane = M * N;
  if (plane <= 0) return hipSuccess;
  const int64_t blocks = (plane / 8 + 255) / 256;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, s, part, splits,
                     plane, (int)N, out, out_bf16 ? 1 : 0, static_cast<const bf16_t*>(bias),
                     accumulate);
  return hipGetLastError();
}

hipError_t colsum_reduce_launch(const float* part, int nparts, int M, float* out, int accumulate,
                                hipStream_t s, int groups) {
  if (M <= 0 || groups <= 0) return hipSuccess;
  hipLaunchKernelGGL(colsum_reduce_kernel, dim3((M + 63) / 64, groups), dim3(256), 0, s, part,
                     nparts, M, out, accumulate);
  return hipGetLastError();
}

int f32_grid(Step step, GemmArgs& g) {
  const bool pair = (step == FC1_FWD_SWIGLU);
  g.tiles_m = (g.M + kF32Tile - 1) / kF32Tile;
  const int bn = pair ? kF32Tile / 2 : kF32Tile;
  g.tiles_n = (g.N + bn - 1) / bn;
  g.group_m = 1;
  if (g.M <= 0 || g.N <= 0) return 0;
  return g.tiles_m * g.tiles_n;
}

hipError_t f32_launch(Step step, const GemmArgs& g, const EpiArgs& e, hipStream_t s) {
  switch (step) {
    case FC1_FWD_GELU: return launch_f32<true, true, EPI_BIAS_GELU, false>(g, e, s);
    case FC1_FWD_SWIGLU: return launch_f32<true, true, EPI_SWIGLU, false>(g, e, s);
    case FC2_FWD: return launch_f32<true, true, EPI_STORE, false>(g, e, s);
    case FC2_DGRAD_GELU: return launch_f32<true, false, EPI_DGELU, false>(g, e, s);
    case FC2_DGRAD_SWIGLU: return launch_f32<true, false, EPI_DSWIGLU, false>(g, e, s);
    case FC1_DGRAD: return launch_f32<true, false, EPI_STORE, false>(g, e, s);
    case WGRAD: return launch_f32<false, false, EPI_F32, false>(g, e, s);
    case WGRAD_COLSUM: return launch_f32<false, false, EPI_F32, true>(g, e, s);
    case QKV_FWD_BIAS: return launch_f32<true, true, EPI_BIAS, false>(g, e, s);
    default: return hipErrorInvalidValue;
  }
}

int quant_parts(int64_t n) {
  int64_t per = (int64_t)kQuantThreads * kQuantVec * 4;  // ~4 iterations per thread
  int64_t p = (n + per - 1) / per;
  if (p < 1) p = 1;
  if (p > kQuantMaxParts) p = kQuantMaxParts;
  return (int)p;
}

hipError_t amax_partial_launch(bool src_bf16, const void* src, int64_t n, float* partial,
                               int nparts, hipStream_t s) {
  if (src_bf16)
    hipLaunchKernelGGL(amax_partial_kernel<bf16_t>, dim3(nparts), dim3(kQuantThreads), 0, s,
                       static_cast<const bf16_t*>(src), n, partial);
  else
    hipLaunchKernelGGL(amax_partial_kernel<float>, dim3(nparts), dim3(kQuantThreads), 0, s,
                       static_cast<const float*>(src), n, partial);
  return hipGetLastError();
}

hipError_t quantize_launch(bool src_bf16, const void* src, int64_t n, uint8_t* dst,
                           const float* partial, int nparts, float* amax_out,
                           float* scale_inv_out, hipStream_t s, bool e5m2) {
  const int nb = quant_parts(n) * 4 > 4096 ? 4096 : quant_parts(n) * 4;
  auto go = [&](auto kernel, const auto* p) {
    hipLaunchKernelGGL(kernel, dim3(nb), dim3(kQuantThreads), 0, s, p, n, dst, partial, nparts,
                       amax_out, scale_inv_out);
  };
  if (src_bf16) {
    const bf16_t* p = static_cast<const bf16_t*>(src);
    if (e5m2) go(quantize_kernel<bf16_t, true>, p); else go(quantize_kernel<bf16_t, false>, p);
  } else {
    const float* p = static_cast<const float*>(src);
    if (e5m2) go(quantize_kernel<float, true>, p); else go(quantize_kernel<float, false>, p);
  }
  return hipGetLastError();
}

hipError_t delayed_update_launch(const float* partial, int nparts, float* history, int len,
                                 float* scale, float* scale_inv, bool e5m2, hipStream_t s) {
  hipLaunchKernelGGL(delayed_update_kernel, dim3(1), dim3(kQuantThreads), 0, s, partial, nparts,
                     history, len, scale, scale_inv, e5m2 ? 57344.0f : 448.0f);
  return hipGetLastError();
}

}  // namespace tpmlp
