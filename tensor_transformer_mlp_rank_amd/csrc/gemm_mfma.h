// MFMA GEMM tile kernel for gfx950 with the MLP block's fused epilogues.
//
// Computes C[m][n] = sum_k A(m,k) * B(n,k) for one 256 x 256 output tile per
// workgroup (a 256 x 128 "pair" tile for the gated fc1, see below), then
// applies an epilogue in registers and stores to HBM.
//
//   A(m,k): K-major  -> A[m*lda + k]   (rows of a row-major [M,K] matrix)
//           MN-major -> A[k*lda + m]   (a row-major [K,M] matrix read transposed)
//   B(n,k): K-major  -> B[n*ldb + k];  MN-major -> B[k*ldb + n]
//
// Which of the block's six products uses which layout:
//   fc1 fwd   x[T,H]  . W1[GFs,H]^T   A K-major,  B K-major
//   fc2 fwd   a[T,Fs] . W2[H,Fs]^T    A K-major,  B K-major
//   fc2 dgrad dy[T,H] . W2[H,Fs]      A K-major,  B MN-major
//   fc1 dgrad dH[T,GFs] . W1[GFs,H]   A K-major,  B MN-major
//   fc2 wgrad dy^T . a                A MN-major, B MN-major (K = T)
//   fc1 wgrad dH^T . x                A MN-major, B MN-major (K = T)
//
// Work decomposition (512 threads = 8 waves of 64 lanes):
//   * workgroup tile 256 (M) x 256 (N), K step of 128 bytes per row
//     (64 bf16 or 128 e4m3 elements), two LDS stages of 2 x 32 KiB;
//   * waves in a 2 x 4 grid, each owning a 128 x 64 sub-tile held as 4 x 2
//     accumulators of the 32x32 MFMA (v_mfma_f32_32x32x16_bf16, or
//     v_mfma_f32_32x32x64_f8f6f4 for e4m3): 128 fp32 registers per lane;
//   * global -> registers -> LDS with 16-byte loads coalesced along the
//     contiguous dimension; loads for step k+1 are in flight while step k's
//     MFMAs run; one barrier per step.
//
// LDS layouts (bank-conflict-free for the access patterns used):
//   * K-major operand: [256 rows][128 B]; 16-byte chunk c of row r is stored at
//     chunk c ^ (r & 7). Fragment reads are ds_read_b128 (one 32x32x16 bf16
//     operand = 8 consecutive k of one row).
//   * MN-major operand: [64 k-rows][256 elements] (512 B); chunk c of k-row r
//     is stored at chunk c ^ 2(r & 3). Fragment reads use the CDNA4 transpose
//     read ds_read_b64_tr_b16: in each group of 16 lanes, lane j receives
//     element j%4 of the 8-byte chunks addressed by lanes 4q + j/4 (q = 0..3),
//     so pointing lane i at k-row k0 + i/4, elements m0 + 4(i%4) .. +3 hands
//     lane j the four k values k0..k0+3 of element m0 + j -- the MFMA operand
//     layout, read straight from the un-transposed tile.
//
// Gated fc1 (SwiGLU): the B tile holds 128 gate rows and the 128 matching up
// rows of W1, interleaved in blocks of 32 so that each wave's two N
// accumulators are a (gate, up) pair for the same 32 output features; the
// epilogue then forms silu(gate) * up in registers.
//
// Workgroup order: blockIdx.x is first remapped so that the workgroups the
// hardware places on one XCD (ids congruent mod 8) get consecutive tile ids,
// then tiles are walked in groups of `group_m` M-tiles, so the workgroups
// resident on an XCD share A and B tiles in that XCD's L2.
#pragma once

#include "epilogue.h"

namespace tpmlp {

constexpr int kBM = 256, kBN = 256, kBKB = 128;  // tile rows, cols, K bytes per step
constexpr int kThreads = 512;
constexpr int kTileBytes = 256 * kBKB;             // 32 KiB per operand per stage
constexpr int kSmemBytes = 2 * 2 * kTileBytes;     // 128 KiB

__device__ __forceinline__ void tile_coords(const GemmArgs& g, int bid, int& bm, int& bn) {
  const int nb = g.tiles_m * g.tiles_n;
  // XCD remap: hardware sends workgroup b to XCD b % 8.
  const int xcd = bid & 7, local = bid >> 3;
  const int q = nb >> 3, r = nb & 7;
  const int id = xcd * q + (xcd < r ? xcd : r) + local;
  // grouped walk over M-tiles
  const int per_group = g.group_m * g.tiles_n;
  const int grp = id / per_group;
  const int first_m = grp * g.group_m;
  int gsz = g.tiles_m - first_m;
  if (gsz > g.group_m) gsz = g.group_m;
  const int in = id - grp * per_group;
  bm = first_m + in % gsz;
  bn = in / gsz;
}

// --------------------------------------------------------------- tile loaders
// K-major: 256 rows x 8 chunks; thread t loads chunk t&7 of rows (t>>3) + 64i.
// row_map gives each tile row's rsrc (0: rs0, 1: rs1) and local row index.
struct KMajorLoader {
  __amdgpu_buffer_rsrc_t rs0, rs1;
  int64_t ld_bytes;
  uint32_t kbytes;       // K * element size (row length in bytes)
  uint32_t row_off[4];   // byte offset of the row start within its rsrc (or kOOB)
  bool use1[4];

  __device__ __forceinline__ void load(u32x4 (&r)[4], int tid, uint32_t k0b) const {
    const uint32_t cb = k0b + (uint32_t)((tid & 7) << 4);
    const bool kin = cb < kbytes;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t off = (kin && row_off[i] != kOOB) ? row_off[i] + cb : kOOB;
      r[i] = use1[i] ? buf_load16(rs1, off) : buf_load16(rs0, off);
    }
  }
  __device__ __forceinline__ static void store(char* lds, const u32x4 (&r)[4], int tid) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = (tid >> 3) + 64 * i;
      const int c = (tid & 7) ^ (row & 7);
      *reinterpret_cast<u32x4*>(lds + row * kBKB + (c << 4)) = r[i];
    }
  }
};

// MN-major (bf16 only): 64 k-rows x 32 chunks; thread t loads chunk t&31 of
// k-rows (t>>5) + 16i. The resource is rebased to k-row k0 each step.
struct MNMajorLoader {
  const char* base;      // element (k=0, m=tile start)
  int64_t ld_bytes;
  int64_t total_bytes;   // bytes from `base` to the end of the tensor
  uint32_t col_ok;       // chunk t&31 lies inside the M (or N) extent

  __device__ __forceinline__ void load(u32x4 (&r)[4], int tid, int k0) const {
    const int64_t kofs = (int64_t)k0 * ld_bytes;
    __amdgpu_buffer_rsrc_t rs = make_rsrc(base + kofs, total_bytes - kofs);
    const uint32_t cb = (uint32_t)((tid & 31) << 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kr = (tid >> 5) + 16 * i;
      uint32_t off = col_ok ? (uint32_t)(kr * ld_bytes) + cb : kOOB;
      r[i] = buf_load16(rs, off);
    }
  }
  __device__ __forceinline__ static void store(char* lds, const u32x4 (&r)[4], int tid) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kr = (tid >> 5) + 16 * i;
      const int c = (tid & 31) ^ ((kr & 3) << 1);
      *reinterpret_cast<u32x4*>(lds + kr * 512 + (c << 4)) = r[i];
    }
  }
};

// --------------------------------------------------------------- fragment reads
// bf16, K-major tile: lane l takes row (l&31) of the 32-row block starting at
// `row0`, k elements 16*ks + 8*(l>>5) .. +7.
__device__ __forceinline__ bf16x8 frag_k_bf16(const char* lds, int row0, int ks, int lane) {
  const int row = row0 + (lane & 31);
  const int c = ((ks << 1) | (lane >> 5)) ^ (row & 7);
  return *reinterpret_cast<const bf16x8*>(lds + row * kBKB + (c << 4));
}
// bf16, MN-major tile: same operand through two transpose reads.
__device__ __forceinline__ bf16x8 frag_mn_bf16(const char* lds, int col0, int ks, int lane) {
  const int g = lane >> 4, i = lane & 15;
  const int m = col0 + ((g & 1) << 4) + ((i & 3) << 2);
  const int kb = (ks << 4) + ((g >> 1) << 3) + (i >> 2);
  bf16x4 v[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int kr = kb + 4 * r;
    const int c = (m >> 3) ^ ((kr & 3) << 1);
    const char* p = lds + kr * 512 + (c << 4) + ((m & 7) << 1);
    i16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16((TPMLP_LDS i16x4*)(p));
    v[r] = __builtin_bit_cast(bf16x4, t);
  }
  return __builtin_shufflevector(v[0], v[1], 0, 1, 2, 3, 4, 5, 6, 7);
}
// e4m3, K-major tile: lane l takes row (l&31), bytes 64*ks + 32*(l>>5) .. +31.
__device__ __forceinline__ i32x8 frag_k_e4m3(const char* lds, int row0, int ks, int lane) {
  const int row = row0 + (lane & 31);
  const int c0 = ((ks << 2) | ((lane >> 5) << 1));
  const u32x4 lo = *reinterpret_cast<const u32x4*>(lds + row * kBKB + (((c0) ^ (row & 7)) << 4));
  const u32x4 hi = *reinterpret_cast<const u32x4*>(lds + row * kBKB + (((c0 + 1) ^ (row & 7)) << 4));
  i32x8 r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  return r;
}

// --------------------------------------------------------------- the kernel
// IS_FP8: operands are e4m3 (both K-major). A_K / B_K: operand layouts.
// EPI: epilogue kind. OutT: element type of EPI_STORE's output and of the
// activation tensors (h, a, dH). COLSUM: also reduce A over k into e.colsum
// (workgroups with tile column 0 only).
template <bool IS_FP8, bool A_K, bool B_K, int EPI, typename OutT, bool COLSUM>
__global__ void __launch_bounds__(kThreads, 1) gemm_mfma_kernel(const GemmArgs g, const EpiArgs e) {
  static_assert(!COLSUM || !A_K, "the fused column sum reads an MN-major A tile");
  static_assert(!IS_FP8 || (A_K && B_K), "e4m3 operands are K-major");
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr bool kPair = (EPI == EPI_SWIGLU);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  int bm, bn;
  tile_coords(g, blockIdx.x, bm, bn);
  const int m0 = bm * kBM;
  const int n0 = bn * (kPair ? kBN / 2 : kBN);
  constexpr int esz = IS_FP8 ? 1 : 2;
  const int kelems_per_step = kBKB / esz;
  const int nk = (g.K + kelems_per_step - 1) / kelems_per_step;

  // ---- operand A loader
  KMajorLoader la{};
  MNMajorLoader lma{};
  if constexpr (A_K) {
    const char* base = static_cast<const char*>(g.A) + (int64_t)m0 * g.lda * esz;
    la.rs0 = make_rsrc(base, (int64_t)(g.M - m0) * g.lda * esz);
    la.rs1 = la.rs0;
    la.ld_bytes = g.lda * esz;
    la.kbytes = (uint32_t)(g.K * esz);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = (tid >> 3) + 64 * i;
      la.row_off[i] = (m0 + row < g.M) ? (uint32_t)(row * la.ld_bytes) : kOOB;
      la.use1[i] = false;
    }
  } else {
    lma.base = static_cast<const char*>(g.A) + (int64_t)m0 * esz;
    lma.ld_bytes = g.lda * esz;
    lma.total_bytes = (int64_t)g.K * g.lda * esz - (int64_t)m0 * esz;
    lma.col_ok = (m0 + ((tid & 31) << 3)) < g.M;
  }
  // ---- operand B loader
  KMajorLoader lb{};
  MNMajorLoader lmb{};
  if constexpr (B_K) {
    lb.ld_bytes = g.ldb * esz;
    lb.kbytes = (uint32_t)(g.K * esz);
    if constexpr (kPair) {
      // rows 64w + 32f + i  ->  gate (f = 0) or up (f = 1) row n0 + 32w + i
      const char* gate = static_cast<const char*>(g.B) + (int64_t)n0 * g.ldb * esz;
      const char* up = static_cast<const char*>(g.B) + (int64_t)(g.pair_off + n0) * g.ldb * esz;
      const int64_t rem = (int64_t)(g.pair_off - n0) * g.ldb * esz;
      lb.rs0 = make_rsrc(gate, rem);
      lb.rs1 = make_rsrc(up, rem);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = (tid >> 3) + 64 * i;
        const int lr = ((row >> 6) << 5) + (row & 31);
        lb.row_off[i] = (n0 + lr < g.N) ? (uint32_t)(lr * lb.ld_bytes) : kOOB;
        lb.use1[i] = (row >> 5) & 1;
      }
    } else {
      const char* base = static_cast<const char*>(g.B) + (int64_t)n0 * g.ldb * esz;
      lb.rs0 = make_rsrc(base, (int64_t)(g.N - n0) * g.ldb * esz);
      lb.rs1 = lb.rs0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = (tid >> 3) + 64 * i;
        lb.row_off[i] = (n0 + row < g.N) ? (uint32_t)(row * lb.ld_bytes) : kOOB;
        lb.use1[i] = false;
      }
    }
  } else {
    lmb.base = static_cast<const char*>(g.B) + (int64_t)n0 * esz;
    lmb.ld_bytes = g.ldb * esz;
    lmb.total_bytes = (int64_t)g.K * g.ldb * esz - (int64_t)n0 * esz;
    lmb.col_ok = (n0 + ((tid & 31) << 3)) < g.N;
  }

  const bool do_colsum = COLSUM && (bn == 0) && (e.colsum != nullptr);
  float csum[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) csum[j] = 0.f;

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  u32x4 ra[4], rb[4];
  auto gload = [&](int kt) {
    if constexpr (A_K) la.load(ra, tid, (uint32_t)(kt * kBKB));
    else lma.load(ra, tid, kt * kelems_per_step);
    if constexpr (B_K) lb.load(rb, tid, (uint32_t)(kt * kBKB));
    else lmb.load(rb, tid, kt * kelems_per_step);
  };
  auto sstore = [&](int stage) {
    char* sa = smem + stage * (2 * kTileBytes);
    char* sb = sa + kTileBytes;
    if constexpr (A_K) KMajorLoader::store(sa, ra, tid);
    else MNMajorLoader::store(sa, ra, tid);
    if constexpr (B_K) KMajorLoader::store(sb, rb, tid);
    else MNMajorLoader::store(sb, rb, tid);
    if constexpr (COLSUM) {
      if (do_colsum) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            csum[2 * w] += bf2f((bf16_t)(ra[i][w] & 0xffffu));
            csum[2 * w + 1] += bf2f((bf16_t)(ra[i][w] >> 16));
          }
      }
    }
  };

  gload(0);
  sstore(0);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int stage = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    const char* sa = smem + stage * (2 * kTileBytes);
    const char* sb = sa + kTileBytes;
    if constexpr (!IS_FP8) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        bf16x8 af[4], bfr[2];
#pragma unroll
        for (int fm = 0; fm < 4; ++fm) {
          if constexpr (A_K) af[fm] = frag_k_bf16(sa, 128 * wm + 32 * fm, ks, lane);
          else af[fm] = frag_mn_bf16(sa, 128 * wm + 32 * fm, ks, lane);
        }
#pragma unroll
        for (int fn = 0; fn < 2; ++fn) {
          if constexpr (B_K) bfr[fn] = frag_k_bf16(sb, 64 * wn + 32 * fn, ks, lane);
          else bfr[fn] = frag_mn_bf16(sb, 64 * wn + 32 * fn, ks, lane);
        }
#pragma unroll
        for (int fm = 0; fm < 4; ++fm)
#pragma unroll
          for (int fn = 0; fn < 2; ++fn)
            acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[fm], bfr[fn], acc[fm][fn], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        i32x8 af[4], bfr[2];
#pragma unroll
        for (int fm = 0; fm < 4; ++fm) af[fm] = frag_k_e4m3(sa, 128 * wm + 32 * fm, ks, lane);
#pragma unroll
        for (int fn = 0; fn < 2; ++fn) bfr[fn] = frag_k_e4m3(sb, 64 * wn + 32 * fn, ks, lane);
#pragma unroll
        for (int fm = 0; fm < 4; ++fm)
#pragma unroll
          for (int fn = 0; fn < 2; ++fn)
            acc[fm][fn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                af[fm], bfr[fn], acc[fm][fn], 0, 0, 0, 0, 0, 0);
      }
    }
    if (kt + 1 < nk) sstore(stage ^ 1);
    __syncthreads();
  }

  // ---- fused column sum of A (db1 = sum over tokens of dH)
  if constexpr (COLSUM) {
    if (do_colsum) {
      // threads t and t + 32j (j = 0..15) hold the same 8 columns
      float* red = reinterpret_cast<float*>(smem);  // 16 x 256 floats
#pragma unroll
      for (int j = 0; j < 8; ++j) red[(tid >> 5) * 256 + ((tid & 31) << 3) + j] = csum[j];
      __syncthreads();
      if (tid < 256) {
        float s = 0.f;
        for (int q = 0; q < 16; ++q) s += red[q * 256 + tid];
        const int m = m0 + tid;
        if (m < g.M) e.colsum[m] = e.accumulate ? e.colsum[m] + s : s;
      }
    }
  }

  // ---- epilogue. acc[fm][fn][j] is C at
  //   row m0 + 128 wm + 32 fm + 8 (j/4) + 4 (lane/32) + j%4,
  //   col n0 + 64 wn + 32 fn + lane%32          (pair tiles: see below)
  float alpha = 1.0f;
  if constexpr (IS_FP8) alpha = (*e.scale_a) * (*e.scale_b);
  float amax = 0.f;
  const int rbase = m0 + 128 * wm + 4 * (lane >> 5);
  if constexpr (kPair) {
    const int col = n0 + 32 * wn + (lane & 31);
    if (col < g.N) {
#pragma unroll
      for (int fm = 0; fm < 4; ++fm)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int row = rbase + 32 * fm + 8 * (j >> 2) + (j & 3);
          if (row < g.M)
            epi_pair<OutT>(e, g.pair_off, row, col, acc[fm][0][j] * alpha, acc[fm][1][j] * alpha);
        }
    }
  } else {
#pragma unroll
    for (int fn = 0; fn < 2; ++fn) {
      const int col = n0 + 64 * wn + 32 * fn + (lane & 31);
      if (col >= g.N) continue;
      float bias = 0.f;
      if constexpr (EPI == EPI_BIAS_GELU) {
        if (e.bias) bias = Elem<OutT>::load(e.bias, col);
      }
#pragma unroll
      for (int fm = 0; fm < 4; ++fm)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int row = rbase + 32 * fm + 8 * (j >> 2) + (j & 3);
          if (row < g.M)
            epi_one<EPI, OutT, IS_FP8>(e, g.pair_off, row, col, acc[fm][fn][j], alpha, bias, amax);
        }
    }
  }
  if constexpr (IS_FP8 && EPI == EPI_BIAS_GELU) {
    amax = wave_max(amax);
    __shared__ float wmax[8];
    if (lane == 0) wmax[wave] = amax;
    __syncthreads();
    if (tid == 0) {
      float m = 0.f;
      for (int w = 0; w < 8; ++w) m = __builtin_fmaxf(m, wmax[w]);
      e.amax_part[blockIdx.x] = m;
    }
  }
}

}  // namespace tpmlp
