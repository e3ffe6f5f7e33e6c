// fp32 tile kernel on the vector ALUs, for float32 blocks.
//
// Same problem statement, operand layouts and epilogues as the MFMA kernel
// (C[m][n] = sum_k A(m,k) B(n,k); A and B K-major or MN-major; the gated fc1
// pairs gate and up columns), computed with exact fp32 fused multiply-adds:
// no reduced-precision matrix instructions are used for fp32 data.
//
// 256 threads compute a 64 x 64 tile (a 64 x 32 pair tile for the gated fc1);
// thread (tx, ty) = (t % 16, t / 16) owns rows ty + 16i and columns tx + 16j
// (i, j < 4). K advances 16 per step through LDS tiles stored [k][m] with one
// word of padding. Loads are bounds-checked element by element, so any M, N,
// K work. For the gated fc1, tile columns [0, 32) are gate features and
// [32, 64) the matching up features, so thread columns j and j + 2 pair up.
#pragma once

#include "epilogue.h"

namespace tpmlp {

constexpr int kF32Tile = 64, kF32BK = 16, kF32Threads = 256;
constexpr int kF32Fold = 256;  // k values per block of the two-level summation

template <bool A_K, bool B_K, int EPI, bool COLSUM>
__global__ void __launch_bounds__(kF32Threads) gemm_f32_kernel(const GemmArgs g, const EpiArgs e) {
  static_assert(!COLSUM || !A_K, "the fused column sum reads an MN-major A tile");
  constexpr bool kPair = (EPI == EPI_SWIGLU);
  __shared__ float As[kF32BK][kF32Tile + 1];
  __shared__ float Bs[kF32BK][kF32Tile + 1];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int bm = blockIdx.x % g.tiles_m, bn = blockIdx.x / g.tiles_m;
  const int m0 = bm * kF32Tile;
  const int n0 = bn * (kPair ? kF32Tile / 2 : kF32Tile);
  const float* A = static_cast<const float*>(g.A);
  const float* B = static_cast<const float*>(g.B);
  const bool do_colsum = COLSUM && bn == 0 && e.colsum != nullptr;
  float csum = 0.f;

  // Two-level summation: each block of kF32Fold k values is summed on its
  // own, then folded into the running total, so the rounding error grows
  // with K / kF32Fold + kF32Fold rather than with K (long token sums of the
  // weight gradients).
  float acc[4][4], blk[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = blk[i][j] = 0.f;
  float cblk = 0.f;

  for (int k0 = 0; k0 < g.K; k0 += kF32BK) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = tid + kF32Threads * i;
      // A tile element (m, k): consecutive threads walk the contiguous dimension
      int m, k;
      if constexpr (A_K) { m = q >> 4; k = q & 15; } else { k = q >> 6; m = q & 63; }
      const int gm = m0 + m, gk = k0 + k;
      float va = 0.f;
      if (gm < g.M && gk < g.K)
        va = A_K ? A[(int64_t)gm * g.lda + gk] : A[(int64_t)gk * g.lda + gm];
      As[k][m] = va;
      // B tile element (n, k); for pair tiles n maps to a gate or an up row
      int n, kb;
      if constexpr (B_K) { n = q >> 4; kb = q & 15; } else { kb = q >> 6; n = q & 63; }
      int gn = n0 + n;
      bool nok = gn < g.N;
      if constexpr (kPair) {
        const int p = n0 + (n & 31);
        nok = p < g.N;
        gn = (n >= 32 ? g.pair_off : 0) + p;
      }
      const int gkb = k0 + kb;
      float vb = 0.f;
      if (nok && gkb < g.K)
        vb = B_K ? B[(int64_t)gn * g.ldb + gkb] : B[(int64_t)gkb * g.ldb + gn];
      Bs[kb][n] = vb;
    }
    __syncthreads();
    if constexpr (COLSUM) {
      if (do_colsum && tid < kF32Tile) {
#pragma unroll
        for (int k = 0; k < kF32BK; ++k) cblk += As[k][tid];
      }
    }
#pragma unroll
    for (int k = 0; k < kF32BK; ++k) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[k][ty + 16 * i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[k][tx + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) blk[i][j] = __builtin_fmaf(a[i], b[j], blk[i][j]);
    }
    __syncthreads();
    if ((k0 + kF32BK) % kF32Fold == 0 || k0 + kF32BK >= g.K) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[i][j] += blk[i][j];
          blk[i][j] = 0.f;
        }
      csum += cblk;
      cblk = 0.f;
    }
  }

  if constexpr (COLSUM) {
    if (do_colsum && tid < kF32Tile && m0 + tid < g.M) {
      const int m = m0 + tid;
      e.colsum[m] = e.accumulate ? e.colsum[m] + csum : csum;
    }
  }

  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = m0 + ty + 16 * i;
    if (row >= g.M) continue;
    if constexpr (kPair) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = n0 + tx + 16 * j;
        if (col < g.N) epi_pair<float>(e, g.pair_off, row, col, acc[i][j], acc[i][j + 2]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = n0 + tx + 16 * j;
        if (col >= g.N) continue;
        float bias = 0.f;
        if constexpr (EPI == EPI_BIAS_GELU || EPI == EPI_BIAS) {
          if (e.bias) bias = static_cast<const float*>(e.bias)[col];
        }
        epi_one<EPI, float, false>(e, g.pair_off, row, col, acc[i][j], 1.0f, bias, amax);
      }
    }
  }
}

}  // namespace tpmlp
