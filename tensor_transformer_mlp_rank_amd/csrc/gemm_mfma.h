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
// Work decomposition: 256 threads = 4 waves in a 2 x 2 grid, one wave per
// SIMD. Each wave owns a 128 x 128 sub-tile: for bf16, 8 x 8 accumulator
// blocks of the 16x16x32 MFMA (v_mfma_f32_16x16x32_bf16); for FP8 with two
// K-major operands (the forward products), 8 x 8 blocks of the 16x16x128
// one (v_mfma_f32_16x16x128_f8f6f4, E4M3 x E4M3); for the other FP8
// products, 4 x 4 blocks of the 32x32x64 one (v_mfma_scale_f32_32x32x64_f8f6f4
// with unit scales, its format bits choosing E4M3 or E5M2 per operand).
// Either way 256 fp32 accumulator registers per lane (AGPRs). Per FLOP this
// reads half the LDS bytes of a 128 x 64 wave tile. Under the chip's power
// limit the 16x16 MFMAs sustain a higher clock than the 32x32 ones (MFMA-only
// loops with random operands: bf16 1.97 against 1.76 GHz, 8% more FLOP/s;
// FP8 2.18 against 2.01 GHz, 8% more).
//
// Pipeline: K advances 128 bytes per row per stage (64 bf16 / 128 e4m3
// elements, whole cache lines per request); a stage holds a 32 KiB A tile and
// a 32 KiB B tile; two stages (128 KiB of the 160 KiB LDS, laid out A0 A1 B0
// B1) alternate, and the main loop runs them in pairs so that a read's stage
// offset is an immediate (see main_loop). Tiles go from HBM straight into LDS
// with buffer_load_dwordx4 ... lds (no staging registers, no LDS store
// instructions); the buffer resource's range check turns reads past a
// tensor's end into zeros. Within a stage (see stage_iter16 for bf16,
// stage_f16 and stage_iter_rolling for FP8) the MFMAs run from registers
// while the LDS reads for the next k-steps and the loads of stage k+2 are
// interleaved between them; barriers inside the stage hand the buffers over
// (bf16: one when A is free, one when the next stage has landed). Each is a
// plain s_barrier preceded by an explicit wait (vmcnt for this wave's loads,
// lgkmcnt for its LDS reads): a full __syncthreads would drain all loads in
// flight and serialise the pipeline.
//
// Tile mappings besides the plain grid: grouped products (the experts of a
// mixture-of-experts layer, see find_group) and split-K (GemmArgs::k_splits),
// where the workgroups of a tile take consecutive K ranges and write fp32
// partial planes that a reduce pass adds up.
//
// LDS layouts (direct-to-LDS loads write 64 lanes x 16 B = 1 KiB linearly per
// instruction, so swizzles are applied by choosing which global chunk each
// lane fetches):
//   * K-major tile: [256 rows][128 B]; 16-byte chunk c of row r lives at
//     chunk c ^ ((r >> 1) & 7). Any 16 consecutive rows then put a given chunk
//     in 16 distinct 16-byte slots of a 256-byte bank window, so the fragment
//     reads (ds_read_b128, 8 consecutive k of one row per lane) are
//     conflict-free.
//   * MN-major tile: [64 k-rows][256 elements = 512 B]; chunk c of k-row r
//     lives at chunk c ^ ({0, 4, 10, 14}[r % 4] ^ 2 (r / 8 % 2)). A
//     transpose read of the 16x16x32 operand takes k-rows k0..k0+3 in lanes
//     0-15 and k0+8..k0+11 in lanes 16-31, two chunks each: the swizzle puts
//     these 16 (k-row, chunk) pairs in 16 distinct 16-byte slots of a
//     256-byte bank window. Fragments are read with the CDNA4 transpose
//     read ds_read_b64_tr_b16: in each group of 16 lanes, lane j receives
//     element j%4 of the 8-byte chunks addressed by lanes 4q + j/4 (q = 0..3),
//     so pointing lane i at k-row k0 + i/4, elements m0 + 4(i%4) .. +3 hands
//     lane j the four k values k0..k0+3 of element m0 + j -- the MFMA operand
//     layout, read straight from the untransposed tile.
//
// Gated fc1 (SwiGLU): the first half of each wave's 128 accumulator columns
// holds gate features and the second half the matching up features of the
// same 64 output features, so the epilogue forms silu(gate) * up in
// registers.
//
// Workgroup order: blockIdx.x is first remapped so that the workgroups the
// hardware places on one XCD (ids congruent mod 8) get consecutive tile ids,
// then tiles are walked in groups of `group_m` M-tiles, so the workgroups
// resident on an XCD share A and B tiles in that XCD's L2.
#pragma once

#include <type_traits>
#include <utility>

#include "epilogue.h"

namespace tpmlp {

// Compile-time loops: f(IC<i>{}) for i = 0 .. N-1. The index is a constant
// expression inside f, so it can pick registers and instruction offsets.
template <int V>
using IC = std::integral_constant<int, V>;
template <typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F& f, std::integer_sequence<int, Is...>) {
  (f(IC<Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

constexpr int kBM = 256, kBN = 256;
constexpr int kThreads = 256;
constexpr int kRowBytes = 128;                     // per tile row per stage
constexpr int kStages = 2;
constexpr int kTileBytes = 256 * kRowBytes;        // 32 KiB
constexpr int kStageBytes = 2 * kTileBytes;        // A + B
constexpr int kSmemBytes = kStages * kStageBytes;  // 128 KiB
// LDS: A of stages 0, 1, then B of stages 0, 1 (32 KiB each). A fragment read
// adds its stage's offset (0 or 32 KiB) in the instruction's offset field,
// and the main loop runs two stages per iteration, so the per-lane read
// addresses stay the same from stage to stage.
constexpr int kTileB0 = kStages * kTileBytes;      // first B tile
// A stage's buffer parity is a compile-time IC<0>/IC<1>: the buffer's offset
// goes into the reads' offset field.
template <typename P>
struct ParityOffset;
template <int P>
struct ParityOffset<std::integral_constant<int, P>> {
  static constexpr int value = P * kTileBytes;
};

// XCD remap: hardware sends workgroup b to XCD b % 8; this gives the
// workgroups of one XCD consecutive ids out of nb.
__device__ __forceinline__ int xcd_remap(int bid, int nb) {
  const int xcd = bid & 7, local = bid >> 3;
  const int q = nb >> 3, r = nb & 7;
  return xcd * q + (xcd < r ? xcd : r) + local;
}
// Walk over the tiles in groups of group_m M-tiles (all N-tiles of a group
// before the next), so consecutive ids share A and B panels in L2.
__device__ __forceinline__ void tile_walk(int id, int tiles_m, int tiles_n, int group_m, int& bm,
                                          int& bn) {
  const int per_group = group_m * tiles_n;
  const int grp = id / per_group;
  const int first_m = grp * group_m;
  int gsz = tiles_m - first_m;
  if (gsz > group_m) gsz = group_m;
  const int in = id - grp * per_group;
  bm = first_m + in % gsz;
  bn = in / gsz;
}

// Grouped products. Each wave scans the group counts 64 groups per pass with
// a saturating prefix sum (every wave of a workgroup gets the same, uniform
// results). GROUP_M: group e has ceil(c_e / 256) M-tiles times tiles_n;
// GROUP_K: every group has tiles_m x tiles_n tiles.
// group_scan returns the total number of tiles; with target >= 0 it also
// fills `hit` with the group holding tile `target`, its first row, its row
// count and the tile's index within the group (hit.e = -1: none).
struct GroupHit {
  int e, local, off, cnt;
};
template <int GROUP>
__device__ __forceinline__ int group_scan(const GemmArgs& g, int target, int lane, GroupHit& hit) {
  const uint32_t R = (uint32_t)g.rows;
  const int per = g.tiles_m * g.tiles_n;
  const int want = (GROUP == GROUP_K && target >= 0) ? target / per : -1;
  hit.e = -1;
  uint32_t row_base = 0;
  int tile_base = 0;
  for (int p0 = 0; p0 < g.groups; p0 += 64) {
    const int j = p0 + lane;
    const int c = (j < g.groups) ? g.counts[j] : 0;
    uint32_t cu = c > 0 ? (uint32_t)c : 0u;
    if (cu > R) cu = R;
    uint32_t incl = cu;  // saturating inclusive prefix within the pass
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const uint32_t o = (uint32_t)__shfl_up((int)incl, d, 64);
      if (lane >= d) incl = (incl + o > R) ? R : incl + o;
    }
    uint32_t excl = (uint32_t)__shfl_up((int)incl, 1, 64);
    if (lane == 0) excl = 0;
    uint32_t start = row_base + excl, end = row_base + incl;
    if (start > R) start = R;
    if (end > R) end = R;
    const int cnt = (int)(end - start);
    int tiles = 0, t_incl = 0;
    if constexpr (GROUP == GROUP_M) {
      tiles = (j < g.groups) ? ((cnt + kBM - 1) / kBM) * g.tiles_n : 0;
      t_incl = tiles;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(t_incl, d, 64);
        if (lane >= d) t_incl += o;
      }
    }
    const int t_start = tile_base + t_incl - tiles;
    if (target >= 0 && hit.e < 0) {
      const bool mine = (GROUP == GROUP_M)
                            ? (tiles > 0 && target >= t_start && target < t_start + tiles)
                            : (j == want);
      const uint64_t bal = __ballot(mine);
      if (bal) {
        const int src = __builtin_ctzll(bal);
        hit.e = p0 + src;
        hit.off = __builtin_amdgcn_readlane((int)start, src);
        hit.cnt = __builtin_amdgcn_readlane(cnt, src);
        hit.local = (GROUP == GROUP_M) ? target - __builtin_amdgcn_readlane(t_start, src)
                                       : target % per;
        if (GROUP == GROUP_K) return g.groups * per;
      }
    }
    row_base += (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
    if (row_base > R) row_base = R;
    tile_base += __builtin_amdgcn_readlane(t_incl, 63);
  }
  return (GROUP == GROUP_K) ? g.groups * per : tile_base;
}
// The tile of workgroup `bid`.
// GROUP_M: the launch has an upper bound of workgroups; ids past the real total
// exit. The XCD remap runs over the real total, so each XCD gets a contiguous
// run of tiles (all of equal work) and the surplus workgroups are spread over
// all XCDs.
// GROUP_K: exactly the tiles are launched, every group with the same tile
// grid but its own K. A contiguous run per XCD would hand whole groups to
// single XCDs, and group sizes vary by orders of magnitude. So ids stay in
// hardware order, round-robin over the XCDs: each XCD gets every eighth tile
// of every group (within a group, its tiles of one M-tile row and thus that
// row's A panel).
template <int GROUP>
__device__ __forceinline__ bool find_group(const GemmArgs& g, int bid, int lane, GroupHit& hit) {
  if constexpr (GROUP == GROUP_K) {
    group_scan<GROUP>(g, bid, lane, hit);
    return hit.e >= 0;
  }
  const int total = group_scan<GROUP>(g, -1, lane, hit);
  if (bid >= total) return false;
  group_scan<GROUP>(g, xcd_remap(bid, total), lane, hit);
  return hit.e >= 0;
}

__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rs, char* lds_wave_base,
                                          uint32_t voff, uint32_t soff = 0) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (TPMLP_LDS void*)lds_wave_base, 16, voff, soff, 0,
                                           0);
}

// --------------------------------------------------------------- tile loaders
// A tile is filled by 32 load instructions of 1 KiB; instruction ii fills LDS
// bytes [ii KiB, +1 KiB). Wave w issues instructions 8w .. 8w+7 of each tile.
//
// K-major: instruction ii covers rows 8 ii .. +7 (a full 128-byte row each, so
// every request is a whole cache line); lane l fetches row 8 ii + l/8,
// logical chunk (l%8) ^ kswz(row) (kswz16(row) in the FP8 products of two
// K-major operands).
// For the gated fc1 the rows of one instruction all come from one half of W1
// (gate: rs0, up: base1); which one depends on the instruction only, so the
// choice is wave-uniform and the resource stays in scalar registers.
template <bool PAIR>
struct KMajorLoader {
  __amdgpu_buffer_rsrc_t rs0;
  const char* base1;              // gated fc1: start of the up half's rows
  int64_t bytes1;
  uint32_t voff[8];               // row*ld + chunk*16 within its resource
  uint32_t klim[8];               // the chunk is inside K for stage offsets below this
                                  // (0 for rows past the tensor's end)
  uint32_t kbytes;                // row length K * element size

  __device__ __forceinline__ static uint32_t k_limit(bool row_ok, uint32_t kbytes,
                                                     uint32_t chunk_b) {
    return (row_ok && kbytes > chunk_b) ? kbytes - chunk_b : 0u;
  }

  __device__ __forceinline__ static bool up_half(int ii) {
    return ((ii >> 2) & 3) >= 2;  // fragment (row / 32) % 4 of these rows
  }
  // For a K that is a whole number of stages, the K-range test only tells
  // rows past the tensor's end apart: fold that into the offsets once
  // (kOOB for such rows), and the loads of issue_one<true> need no
  // per-lane instruction at all. Their stages past the end of K then read
  // whatever lies behind (the next row, or zeros past the resource), into
  // stage buffers that no MFMA reads.
  __device__ __forceinline__ void fold_rows() {
#pragma unroll
    for (int i = 0; i < 8; ++i) voff[i] = klim[i] ? voff[i] : kOOB;
  }
  template <bool FAST>
  __device__ __forceinline__ void issue_one(char* tile, int wave, uint32_t k0b, int i) const {
    const int ii = 8 * wave + i;
    // one compare and one select, no per-lane branch; the stage's k offset
    // is the instruction's scalar offset (a lane past the end keeps an
    // offset of at least kOOB, beyond any resource)
    const uint32_t off = FAST ? voff[i] : (k0b < klim[i]) ? voff[i] : kOOB;
    if constexpr (PAIR) {
      if (up_half(ii))
        lds_dma16(make_rsrc(base1, bytes1), tile + (ii << 10), off, k0b);
      else
        lds_dma16(rs0, tile + (ii << 10), off, k0b);
    } else {
      lds_dma16(rs0, tile + (ii << 10), off, k0b);
    }
  }
};

// MN-major: bf16 instruction ii covers k-rows 2 ii, +1 (512 bytes each); lane
// l fetches k-row 2 ii + l/32, logical chunk (l%32) ^ mnswz(krow). FP8
// instruction ii covers k-rows 4 ii .. +3 (256 bytes each); lane l fetches
// k-row 4 ii + l/16, logical chunk (l%16) ^ mnswz8(krow). The resource is
// rebased to the stage's first k-row.
struct MNMajorLoader {
  const char* base;      // element (k=0, m=tile start)
  int64_t ld_bytes;
  int64_t total_bytes;   // bytes from `base` to the end of the tensor
  uint32_t voff[8];

  __device__ __forceinline__ void issue_one(char* tile, int wave, int k0, int i) const {
    const int64_t kofs = (int64_t)k0 * ld_bytes;
    lds_dma16(make_rsrc(base + kofs, total_bytes - kofs), tile + ((8 * wave + i) << 10), voff[i]);
  }
};

// --------------------------------------------------------------- fragment reads
// Swizzles (gfx950's LDS serves 256 bytes per cycle): K-major 128-byte rows
// put chunk c at c ^ ((row >> 1) & 7), so 16 consecutive rows put a given
// chunk in 16 distinct 16-byte slots of a 256-byte window; MN-major k-rows put
// chunk c at c ^ mnswz(krow), mnswz = 0, 4, 10, 14 for krow % 4 = 0..3 (the
// part measured conflict-free for the 32x32 operand's reads), XOR 2 when
// krow / 8 is odd (for the 16x16 operand's, which pair k-rows 8 apart).
__device__ __forceinline__ int kswz(int row) { return (row >> 1) & 7; }
// FP8 K-major tiles of the 16x16x128 products: a lane reads chunks 2g, 2g+1
// (g = lane / 16) of row lane % 16, and with kswz two of the four 16-lane
// groups meet in the same 16-byte slots of a 256-byte window (2-way
// conflicts, measured: half of all LDS cycles of these reads). Chunk c goes to
// c ^ 2 ((row >> 1) & 3) ^ ((row >> 3) & 1), measured conflict-free.
__device__ __forceinline__ int kswz16(int row) {
  return (((row >> 1) & 3) << 1) ^ ((row >> 3) & 1);
}
template <bool F16>
__device__ __forceinline__ int kswz_of(int row) { return F16 ? kswz16(row) : kswz(row); }
__device__ __forceinline__ int mnswz(int kr) {
  return ((0xEA40 >> ((kr & 3) << 2)) & 15) ^ ((kr >> 2) & 2);
}
// FP8 MN-major k-rows (256 bytes) put chunk c at c ^ 2 (krow % 8): a transpose
// read takes one 16-byte chunk pair (c, c+1), c even, from 8 consecutive
// k-rows per half-wave, which land in 16 distinct 16-byte slots.
__device__ __forceinline__ int mnswz8(int kr) { return (kr & 7) << 1; }

// bf16, K-major tile: lane l takes row row0 + (l&31), k elements
// 16*ks + 8*(l>>5) .. +7 of the stage.
// bf16, K-major tile, operand of the 16x16x32 MFMA: lane l takes row
// wrow + 16 R + (l & 15), k elements 32 KS + 8 (l >> 4) .. +7 (16 bytes,
// chunk 4 KS + l / 16). Issued through inline asm like the transpose reads
// below (its result is untracked: the stage barrier and the wait at the top
// of a stage cover it). The swizzle depends on (l & 15) only, since wrow and
// 16 R are multiples of 16 rows, so the tile T and the row block R go into
// the offset field.
template <int T, int KS, int R>
__device__ __forceinline__ bf16x8 frag_k_bf16(const char* stage, int wrow, int lane) {
  const int row = wrow + (lane & 15);
  const int c = ((KS << 2) | (lane >> 4)) ^ kswz(row);
  const uint32_t a = (uint32_t)(uintptr_t)(const TPMLP_LDS char*)stage + row * kRowBytes + (c << 4);
  constexpr int kOff = T + R * 16 * kRowBytes;
  static_assert(kOff >= 0 && kOff < 65536, "DS offset field");
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(a), "i"(kOff));
  return __builtin_bit_cast(bf16x8, r);
}
// The transpose reads (ds_read_tr16_at, ds_read_tr8_at below) are issued
// through inline asm: the compiler's builtin for them carries no
// memory-operand information, so the compiler would make them wait for every
// LDS-bound global load in flight (vmcnt(0)) and drain the pipeline. The asm
// results are not tracked by the compiler's wait counters: every use of them
// follows an explicit lgkmcnt wait (the stage barrier, or wait_lds at the
// top of a stage).
// A 16-byte LDS read whose result the compiler does not wait for: the
// caller waits (lgkmcnt) before using it.
__device__ __forceinline__ u32x4 ds_read_b128_async(const char* p) {
  u32x4 r;
  const uint32_t a = (uint32_t)(uintptr_t)(const TPMLP_LDS char*)p;
  asm volatile("ds_read_b128 %0, %1" : "=v"(r) : "v"(a));
  return r;
}
// Wait until at most N of this wave's LDS reads are in flight (they
// complete in order).
template <int N = 0>
__device__ __forceinline__ void wait_lds() {
  static_assert(N >= 0 && N <= 15, "lgkmcnt range");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (N << 8) | (3 << 14));  // lgkmcnt(N) only
  __builtin_amdgcn_sched_barrier(0);
}
// Transpose reads at a constant byte offset from a per-lane base address:
// the offset goes into the instruction's 16-bit offset field, so the k-step,
// the part of the fragment and the tile (A or B) cost no address arithmetic.
template <int OFF>
__device__ __forceinline__ i16x4 ds_read_tr16_at(uint32_t a) {
  static_assert(OFF >= 0 && OFF < 65536, "DS offset field");
  i16x4 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(a), "i"(OFF));
  return r;
}
template <int OFF>
__device__ __forceinline__ u32x2 ds_read_tr8_at(uint32_t a) {
  static_assert(OFF >= 0 && OFF < 65536, "DS offset field");
  u32x2 r;
  asm volatile("ds_read_b64_tr_b8 %0, %1 offset:%2" : "=v"(r) : "v"(a), "i"(OFF));
  return r;
}

// bf16, MN-major tile, operand of the 16x16x32 MFMA through two transpose
// reads. `stage` is the stage buffer and T the tile's offset in it (0: A,
// kTileBytes: B). In 16-lane group g (k 8g .. 8g+7 of the k-step), lane i
// points at k-row 32 KS + 8 g + i/4 (+4 for the second read), elements
// col0 + 4 (i%4) .. +3, so lane j of the group receives the k values of
// element col0 + j. The swizzle depends on k-row bits 0, 1 and 3 only, which
// neither KS nor the +4 changes, so KS * 16384 + r * 2048 goes into the
// offset field.
template <int T, int KS>
__device__ __forceinline__ bf16x8 frag_mn_bf16(const char* stage, int col0, int lane) {
  const int g = lane >> 4, i = lane & 15;
  const int m = col0 + ((i & 3) << 2);
  const int kr0 = (g << 3) + (i >> 2);
  const int c = (m >> 3) ^ mnswz(kr0);
  const uint32_t a = (uint32_t)(uintptr_t)(const TPMLP_LDS char*)stage + kr0 * 512 + (c << 4) +
                     ((m & 7) << 1);
  const bf16x4 v0 = __builtin_bit_cast(bf16x4, ds_read_tr16_at<T + KS * 16384>(a));
  const bf16x4 v1 = __builtin_bit_cast(bf16x4, ds_read_tr16_at<T + KS * 16384 + 2048>(a));
  return __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
}
// e4m3, K-major tile: lane l takes row (l&31), bytes 64*ks + 32*(l>>5) .. +31.
template <int T, int KS, int F>
__device__ __forceinline__ i32x8 frag_k_e4m3(const char* stage, int wrow, int lane) {
  // as frag_k_bf16: asm reads, the tile and 32-row block in the offset field
  const int row = wrow + (lane & 31);
  const int c0 = (KS << 2) | ((lane >> 5) << 1);
  const uint32_t base = (uint32_t)(uintptr_t)(const TPMLP_LDS char*)stage + row * kRowBytes;
  const uint32_t a0 = base + ((c0 ^ kswz(row)) << 4), a1 = base + (((c0 + 1) ^ kswz(row)) << 4);
  constexpr int kOff = T + F * 32 * kRowBytes;
  static_assert(kOff >= 0 && kOff < 65536, "DS offset field");
  u32x4 lo, hi;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(lo) : "v"(a0), "i"(kOff));
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(hi) : "v"(a1), "i"(kOff));
  i32x8 r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  return r;
}

// e4m3, K-major tile, operand of the 16x16x128 MFMA: lane l takes row
// wrow + 16 R + (l & 15), bytes 32 (l >> 4) .. +31 of the stage's 128
// (chunks 2 (l >> 4) and 2 (l >> 4) + 1). As frag_k_bf16, the swizzle
// depends on (l & 15) only, so the tile T and the row block R go into the
// offset field.
template <int T, int R>
__device__ __forceinline__ i32x8 frag_k_e4m3_16(const char* stage, int wrow, int lane) {
  const int row = wrow + (lane & 15);
  const int c0 = (lane >> 4) << 1;
  const uint32_t base = (uint32_t)(uintptr_t)(const TPMLP_LDS char*)stage + row * kRowBytes;
  const uint32_t a0 = base + ((c0 ^ kswz16(row)) << 4), a1 = base + (((c0 + 1) ^ kswz16(row)) << 4);
  constexpr int kOff = T + R * 16 * kRowBytes;
  static_assert(kOff >= 0 && kOff < 65536, "DS offset field");
  u32x4 lo, hi;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(lo) : "v"(a0), "i"(kOff));
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(hi) : "v"(a1), "i"(kOff));
  i32x8 r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  return r;
}

// FP8 (either format), MN-major tile [128 k-rows][256 bytes]: the operand
// of frag_k_e4m3 (lane l: column col0 + l%32, k 64 ks + 32 (l/32) .. +31)
// through four 8-bit transpose reads. ds_read_b64_tr_b8 gives lane j of each
// 16-lane group byte j%8 of the 8-byte chunks addressed by lanes 2q + j/8
// (q = 0..7, output byte q), so pointing lane i at k-row kb + i/2, bytes
// col + 8 (i%2) .. +7 hands lane j the 8 k values kb .. kb+7 of column
// col + j.
// Read q takes k-row kr = 64 ks + 32 (g/2) + 8 q + i/2; the swizzle depends
// on kr % 8 = (i/2) % 8 only, so the address is a per-lane part plus
// ks * 16384 + q * 2048, which goes into the offset field.
template <int T, int KS>
__device__ __forceinline__ i32x8 frag_mn_fp8(const char* stage, int col0, int lane) {
  const int g = lane >> 4, i = lane & 15;
  const int m = col0 + ((g & 1) << 4);  // 16-byte aligned column of the group
  const int kr0 = ((g >> 1) << 5) + (i >> 1);
  const int c = (m >> 4) ^ mnswz8(kr0);
  const uint32_t a = (uint32_t)(uintptr_t)(const TPMLP_LDS char*)stage + kr0 * 256 + (c << 4) +
                     ((i & 1) << 3);
  i32x8 r;
  static_for<4>([&](auto Q) {
    constexpr int q = decltype(Q)::value;
    const u32x2 v = ds_read_tr8_at<T + KS * 16384 + q * 2048>(a);
    r[2 * q] = (int)v[0];
    r[2 * q + 1] = (int)v[1];
  });
  return r;
}

// Wait until at most N of this wave's vector-memory loads are in flight and
// all its LDS reads are done, then barrier. The wait is the s_waitcnt builtin
// (so the compiler's own wait tracking knows about it) with vmcnt = N,
// expcnt and lgkmcnt = 0 (gfx9 encoding: vmcnt[3:0], expcnt[6:4],
// lgkmcnt[11:8], vmcnt[5:4] at bits 15:14). The empty asm statements keep
// the compiler from moving memory accesses across the barrier, the
// scheduling barriers keep the instruction scheduler from moving anything
// (MFMAs included) across it.
template <int N>
__device__ __forceinline__ void wait_and_barrier() {
  static_assert(N >= 0 && N <= 63, "vmcnt range (63: no wait on loads)");
  constexpr int imm = (N & 15) | (7 << 4) | ((N >> 4) << 14);
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(imm);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// --------------------------------------------------------------- epilogue
// acc[fm][fn][j] is C at
//   row 128 wm + 32 fm + 8 (j/4) + 4 (lane/32) + j%4 of the tile,
//   col 128 wn + 32 fn + lane%32                  (pair tiles: see above).
// Each wave stages one 32-row slab (fm) at a time through its own 17 KiB of
// LDS as fp32 [32][132] (4 floats of padding: measured conflict-free for both
// the scattered writes and the row-segment reads). Then every lane takes 8
// consecutive columns (group cg) of the rows rl, rl + kRowStep, ... of the
// slab, so each row segment is covered by consecutive lanes with 16-byte
// accesses. Global accesses are buffer loads and stores on a resource per
// slab: the range check drops the rows past the tensor's end, and column
// groups past N get an offset outside the resource. No branches, so all
// loads of a slab can be in flight together.
//
// LOADS: the epilogue reads global memory per element (h for the activation
// derivative, the old dW when accumulating). Those loads are issued for two
// slabs at a time, before the slabs are staged, and waited for once: one
// counter tracks both loads and stores, so a wait for a load issued after a
// store also waits for the store, and per-group load/use pairs would
// serialise the epilogue on memory latency.
//
// tail_other: the other half's accumulator dump of a split tile (register r
// of this lane at float (r / 4) * 256 + r % 4 from it), added to the
// accumulators as they are staged; null otherwise.
template <bool IS_FP8, int EPI, typename OutT, bool LOADS, typename Acc>
__device__ __forceinline__ void store_tile(const GemmArgs& g, const EpiArgs& e, Acc& acc,
                                           char* smem, int wave, int lane, int m0, int n0,
                                           float& amax, const float* tail_other) {
  static_assert(std::is_same<OutT, bf16_t>::value, "MFMA activations and outputs are bf16");
  constexpr bool kPair = (EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_Q);
  constexpr int kLd = 132;
  constexpr int kT = kPair ? 4 : 8;         // row groups per lane and slab
  constexpr int kRowStep = kPair ? 8 : 4;   // rows between them
  constexpr bool kDSw = (EPI == EPI_DSWIGLU || EPI == EPI_DSWIGLU_Q);
  constexpr int kPre = (EPI == EPI_F32 || kDSw) ? 2 : 1;  // 16 B loads per group
  constexpr bool kQ8 = (EPI == EPI_BIAS_GELU_Q || EPI == EPI_DGELU_Q || EPI == EPI_SWIGLU_Q ||
                        EPI == EPI_DSWIGLU_Q);  // FP8 codes out
  constexpr int kOes = (EPI == EPI_F32) ? 4 : kQ8 ? 1 : 2;  // primary output element bytes
  constexpr uint32_t kBf = 2;
  const int wm = wave >> 1, wn = wave & 1;
  float* wl = reinterpret_cast<float*>(smem + wave * 32768);
  const int cg = kPair ? (lane & 7) : (lane & 15);
  const int rl = kPair ? (lane >> 3) : (lane >> 4);
  const int wrow = m0 + 128 * wm;
  const int wcol = kPair ? n0 + 64 * wn : n0 + 128 * wn;
  // or-ed into every offset of a column group past N: puts it outside any
  // resource (offsets inside a slab stay below 2^31)
  const uint32_t oob = (wcol + 8 * cg < g.N) ? 0u : kOOB;
  float alpha = 1.0f;
  if constexpr (IS_FP8) alpha = (*e.scale_a) * (*e.scale_b);
  float qs = 1.0f;
  if constexpr (kQ8) qs = *e.q_scale;

  // byte offset of group t in a slab resource with `ld` elements of `es` bytes per row
  auto goff = [&](int64_t ld, uint32_t es, int t) __attribute__((always_inline)) -> uint32_t {
    return ((uint32_t)(rl + kRowStep * t) * (uint32_t)(ld * es) + (uint32_t)(8 * cg) * es) | oob;
  };
  // rows [row0, M) of a row-major tensor, from column wcol of slab fm's first
  // row; an empty range for a null tensor (its stores are dropped)
  auto slab_rsrc = [&](const void* p, int64_t ld, int64_t es, int fm)
      __attribute__((always_inline)) {
    const int row0 = wrow + 32 * fm;
    const int64_t bytes = p ? ((int64_t)(g.M - row0) * ld - wcol) * es : 0;
    return make_rsrc(static_cast<const char*>(p) + ((int64_t)row0 * ld + wcol) * es, bytes);
  };

  u32x4 pre[2][kT][kPre];
  auto load_slabs = [&](int fm0) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if constexpr (EPI == EPI_F32) {
        const auto rs = slab_rsrc(e.out, e.ldo, 4, fm0 + s);
#pragma unroll
        for (int t = 0; t < kT; ++t) {
          const uint32_t o = goff(e.ldo, 4, t);
          pre[s][t][0] = buf_load16(rs, o);
          pre[s][t][kPre - 1] = buf_load16(rs, o + 16);
        }
      } else {
        const auto rs = slab_rsrc(e.aux, e.ldaux, 2, fm0 + s);
#pragma unroll
        for (int t = 0; t < kT; ++t) {
          const uint32_t o = goff(e.ldaux, kBf, t);
          pre[s][t][0] = buf_load16(rs, o);
          if constexpr (kDSw)
            pre[s][t][kPre - 1] = buf_load16(rs, o + (uint32_t)g.pair_off * kBf);
        }
      }
    }
  };

  float bias[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) bias[q] = 0.f;
  if constexpr (EPI == EPI_BIAS_GELU || EPI == EPI_BIAS_GELU_Q || EPI == EPI_BIAS) {
    if (e.bias) {
      const auto rb = make_rsrc(e.bias, (int64_t)g.N * 2);
      unpack_bf16x8(buf_load16(rb, ((uint32_t)(wcol + 8 * cg) * kBf) | oob), bias);
    }
  }

#pragma unroll
  for (int fm = 0; fm < 4; ++fm) {
    if constexpr (LOADS) {
      if ((fm & 1) == 0) load_slabs(fm);
    }
    // the slab's accumulators, in quarters of four dump chunks (chunks
    // fm 16 + 4 qt .. +3; with tail_other their dump values are added)
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) {
      f32x4 t[4];
      if (tail_other) {
#pragma unroll
        for (int k = 0; k < 4; ++k)
          t[k] = *reinterpret_cast<const f32x4*>(tail_other + (fm * 16 + qt * 4 + k) * 256);
      }
      if constexpr (sizeof(acc[0][0]) == 64) {
        // 32x32 blocks: register j of block (fm, fn) is row 8 (j/4) + 4 (l/32)
        // + j%4, column 32 fn + l%32; its dump chunk (fm 4 + fn) 4 + j/4
        const int fn = qt;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float v = acc[fm][fn][j];
          wl[(8 * (j >> 2) + 4 * (lane >> 5) + (j & 3)) * kLd + 32 * fn + (lane & 31)] =
              tail_other ? v + t[j >> 2][j & 3] : v;
        }
      } else {
        // 16x16 blocks: register q of block (2 fm + h, c) is row 16 h + 4 (l/16)
        // + q, column 16 c + l%16; its dump chunk (2 fm + h) 8 + c
        const int h = qt >> 1;
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
          const int c = 4 * (qt & 1) + c4;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float v = acc[2 * fm + h][c][q];
            wl[(16 * h + 4 * (lane >> 4) + q) * kLd + 16 * c + (lane & 15)] =
                tail_other ? v + t[c4][q] : v;
          }
        }
      }
    }
    if constexpr (LOADS) {
      if ((fm & 1) == 0) {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt((0) | (7 << 4) | (15 << 8));  // vmcnt(0)
      }
    }
    const int s = fm & 1;
    const auto ro = slab_rsrc(e.out, e.ldo, kOes, fm);
#pragma unroll
    for (int t = 0; t < kT; ++t) {
      const float* src = wl + (rl + kRowStep * t) * kLd + 8 * cg;
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = src[u] * alpha;
      if constexpr (EPI == EPI_STORE) {
        buf_store16(ro, goff(e.ldo, kOes, t), pack_bf16x8(v));
      } else if constexpr (EPI == EPI_BIAS) {
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] += bias[u];
        buf_store16(ro, goff(e.ldo, kOes, t), pack_bf16x8(v));
      } else if constexpr (EPI == EPI_F32) {
        if constexpr (LOADS) {
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            v[u] += __uint_as_float(pre[s][t][0][u]);
            v[u + 4] += __uint_as_float(pre[s][t][1][u]);
          }
        }
        const uint32_t o = goff(e.ldo, kOes, t);
        buf_store16(ro, o, u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]),
                                 __float_as_uint(v[2]), __float_as_uint(v[3])});
        buf_store16(ro, o + 16, u32x4{__float_as_uint(v[4]), __float_as_uint(v[5]),
                                      __float_as_uint(v[6]), __float_as_uint(v[7])});
      } else if constexpr (EPI == EPI_BIAS_GELU || EPI == EPI_BIAS_GELU_Q) {
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] += bias[u];
        const u32x4 hw = pack_bf16x8(v);
        buf_store16(slab_rsrc(e.out2, e.ldo2, 2, fm), goff(e.ldo2, kBf, t), hw);  // h, if saved
        unpack_bf16x8(hw, v);  // the activation is taken of h as stored
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = gelu_f(v[u]);
        // rows past M hold gelu(b1), not activations: the amax leaves them out
        const bool row_ok = oob == 0u && wrow + 32 * fm + rl + kRowStep * t < g.M;
        if constexpr (kQ8) {
          // codes straight from the fp32 activation, amax of the same values
          if (row_ok) {
#pragma unroll
            for (int u = 0; u < 8; ++u) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[u]));
          }
#pragma unroll
          for (int u = 0; u < 8; ++u) v[u] *= qs;
          buf_store8(ro, goff(e.ldo, 1, t), pack_fp8x8<false>(v));
        } else {
          const u32x4 aw = pack_bf16x8(v);
          if constexpr (IS_FP8) {
            // amax of a as stored in bf16, the values the quantiser reads
            float ar[8];
            unpack_bf16x8(aw, ar);
            if (row_ok) {
#pragma unroll
              for (int u = 0; u < 8; ++u) amax = __builtin_fmaxf(amax, __builtin_fabsf(ar[u]));
            }
          }
          buf_store16(ro, goff(e.ldo, kBf, t), aw);
        }
      } else if constexpr (kPair) {
        float up[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) up[u] = src[64 + u] * alpha;
        const u32x4 gw = pack_bf16x8(v), uw = pack_bf16x8(up);
        const auto r2 = slab_rsrc(e.out2, e.ldo2, 2, fm);  // h, if saved
        const uint32_t o2 = goff(e.ldo2, kBf, t);
        buf_store16(r2, o2, gw);
        buf_store16(r2, o2 + (uint32_t)g.pair_off * kBf, uw);
        unpack_bf16x8(gw, v);
        unpack_bf16x8(uw, up);
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = silu_f(v[u]) * up[u];
        // rows past M and columns past N leave the amax out
        const bool row_ok = oob == 0u && wrow + 32 * fm + rl + kRowStep * t < g.M;
        if constexpr (kQ8) {
          // codes straight from the fp32 activation, amax of the same values
          if (row_ok) {
#pragma unroll
            for (int u = 0; u < 8; ++u) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[u]));
          }
#pragma unroll
          for (int u = 0; u < 8; ++u) v[u] *= qs;
          buf_store8(ro, goff(e.ldo, 1, t), pack_fp8x8<false>(v));
        } else {
          const u32x4 aw = pack_bf16x8(v);
          if constexpr (IS_FP8) {
            // amax of a as stored in bf16, the values the quantiser reads
            float ar[8];
            unpack_bf16x8(aw, ar);
            if (row_ok) {
#pragma unroll
              for (int u = 0; u < 8; ++u) amax = __builtin_fmaxf(amax, __builtin_fabsf(ar[u]));
            }
          }
          buf_store16(ro, goff(e.ldo, kBf, t), aw);
        }
      } else if constexpr (EPI == EPI_DGELU || EPI == EPI_DGELU_Q) {
        float h[8];
        unpack_bf16x8(pre[s][t][0], h);
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] *= gelu_grad_f(h[u]);
        if constexpr (kQ8) {
          if (oob == 0u && wrow + 32 * fm + rl + kRowStep * t < g.M) {
#pragma unroll
            for (int u = 0; u < 8; ++u) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[u]));
          }
#pragma unroll
          for (int u = 0; u < 8; ++u) v[u] *= qs;
          buf_store8(ro, goff(e.ldo, 1, t), pack_fp8x8<true>(v));
        } else {
          buf_store16(ro, goff(e.ldo, kBf, t), pack_bf16x8(v));
        }
      } else if constexpr (kDSw) {
        float gt[8], up[8], dg[8];
        unpack_bf16x8(pre[s][t][0], gt);
        unpack_bf16x8(pre[s][t][1], up);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          dg[u] = v[u] * up[u] * silu_grad_f(gt[u]);
          v[u] = v[u] * silu_f(gt[u]);
        }
        if constexpr (kQ8) {
          // both halves at the one scale of dH, amax over both
          if (oob == 0u && wrow + 32 * fm + rl + kRowStep * t < g.M) {
#pragma unroll
            for (int u = 0; u < 8; ++u)
              amax = __builtin_fmaxf(amax, __builtin_fmaxf(__builtin_fabsf(dg[u]),
                                                           __builtin_fabsf(v[u])));
          }
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            dg[u] *= qs;
            v[u] *= qs;
          }
          const uint32_t o = goff(e.ldo, 1, t);
          buf_store8(ro, o, pack_fp8x8<true>(dg));
          buf_store8(ro, o + (uint32_t)g.pair_off, pack_fp8x8<true>(v));
        } else {
          const uint32_t o = goff(e.ldo, kBf, t);
          buf_store16(ro, o, pack_bf16x8(dg));
          buf_store16(ro, o + (uint32_t)g.pair_off * kBf, pack_bf16x8(v));
        }
      }
    }
  }
}

// --------------------------------------------------------------- the kernel
// IS_FP8: FP8 operands, A in E5M2 if FMT & 1 else E4M3, B in E5M2 if FMT & 2
// else E4M3. A_K / B_K: operand layouts. EPI: epilogue kind. OutT: element
// type of EPI_STORE's output and of the activation tensors (h, a, dH).
// COLSUM: also reduce A over k into the per-tile-column partial sums
// e.colsum (A must be MN-major; FP8 sums are scaled by *e.scale_a).
template <bool IS_FP8, bool A_K, bool B_K, int EPI, typename OutT, bool COLSUM, int FMT = 0,
          int GROUP = GROUP_NONE>
__global__ void __launch_bounds__(kThreads, 1) gemm_mfma_kernel(const GemmArgs g_in,
                                                                const EpiArgs e_in) {
  static_assert(!COLSUM || !A_K, "the fused column sum reads an MN-major A tile");
  static_assert(IS_FP8 || FMT == 0, "formats select FP8 encodings");
  static_assert(GROUP == GROUP_NONE || !IS_FP8, "grouped products are bf16");
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  constexpr bool kPair = (EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_Q);
  constexpr bool kF16 = IS_FP8 && A_K && B_K;  // FP8 on the 16x16x128 MFMA
  constexpr int esz = IS_FP8 ? 1 : 2;
  constexpr int kStep = kRowBytes / esz;  // k elements per stage
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  GemmArgs g = g_in;
  EpiArgs e = e_in;
  // clock capture: stored at once (nothing held in registers across the loop)
  const bool clk_on = g.clk != nullptr && (int)blockIdx.x < g.clk_slots;
  if (clk_on && tid == 0) {
    g.clk[4 * blockIdx.x] = __builtin_amdgcn_s_memtime();
    g.clk[4 * blockIdx.x + 1] = __builtin_amdgcn_s_memrealtime();
  }
  int bm, bn;
  int kt0 = 0;                              // first stage of this workgroup's K range
  int nk = (g.K + kStep - 1) / kStep;       // its number of stages
  int split = 0;
  // the products whose partial last round the host may split: the weight
  // gradients without a fused column sum (in the other kernels the code
  // would cost registers their main loops do not have)
  constexpr bool kTail = GROUP == GROUP_NONE && !COLSUM && !A_K && !B_K && EPI == EPI_F32;
  int tail_p = -1, tail_h = 0;  // split tile of a partial last round, and its half
  if constexpr (GROUP == GROUP_NONE) {
    const int full = g.tiles_m * g.tiles_n - (kTail ? g.tail_tiles : 0);
    if (kTail && g.tail_tiles > 0 && (int)blockIdx.x >= full) {
      // workgroup u of the tail runs on XCD x = blockIdx.x % 8: it takes half
      // (u / 8) % 2 of tail tile x * (tail_tiles / 8) + u / 16, so both halves
      // of a tile share an XCD (and its L2) and each XCD a run of the walk
      const int u = (int)blockIdx.x - full;
      tail_h = (u >> 3) & 1;
      tail_p = ((int)blockIdx.x & 7) * (g.tail_tiles >> 3) + (u >> 4);
      tile_walk(full + tail_p, g.tiles_m, g.tiles_n, g.group_m, bm, bn);
      // the first half an even number of stages (see split-K)
      const int half = (((nk + 1) >> 1) + 1) & ~1;
      kt0 = tail_h ? half : 0;
      nk = tail_h ? nk - half : (half < nk ? half : nk);
    } else if (g.k_splits > 1) {
      // ids split-major: the workgroups of one XCD share a split's panels
      const int tiles = g.tiles_m * g.tiles_n;
      const int id = xcd_remap(blockIdx.x, tiles * g.k_splits);
      split = id / tiles;
      tile_walk(id - split * tiles, g.tiles_m, g.tiles_n, g.group_m, bm, bn);
      kt0 = split * g.split_stages;
      nk = nk - kt0 < g.split_stages ? nk - kt0 : g.split_stages;
      e.out = static_cast<char*>(e.out) + (int64_t)split * g.M * e.ldo * 4;
    } else {
      tile_walk(xcd_remap(blockIdx.x, full), g.tiles_m, g.tiles_n, g.group_m, bm, bn);
    }
  } else {
    GroupHit hit;
    if (!find_group<GROUP>(g, blockIdx.x, lane, hit)) return;
    // rebase every tensor on the group's rows or on its own block
    constexpr int64_t kOut = (EPI == EPI_F32) ? 4 : 2;  // output element bytes
    g.A = static_cast<const char*>(g.A) + (int64_t)hit.off * g.lda * esz;
    if constexpr (GROUP == GROUP_M) {
      g.M = hit.cnt;
      g.tiles_m = (hit.cnt + kBM - 1) / kBM;
      g.B = static_cast<const char*>(g.B) + (int64_t)hit.e * g.b_gstride * esz;
      e.out = static_cast<char*>(e.out) + (int64_t)hit.off * e.ldo * kOut;
      if (e.out2) e.out2 = static_cast<char*>(e.out2) + (int64_t)hit.off * e.ldo2 * 2;
      if (e.aux) e.aux = static_cast<const char*>(e.aux) + (int64_t)hit.off * e.ldaux * 2;
      if (e.bias) e.bias = static_cast<const char*>(e.bias) + (int64_t)hit.e * g.bias_gstride * 2;
    } else {
      g.K = hit.cnt;
      g.B = static_cast<const char*>(g.B) + (int64_t)hit.off * g.ldb * esz;
      e.out = static_cast<char*>(e.out) + (int64_t)hit.e * g.out_gstride * kOut;
      if (e.colsum) e.colsum += (int64_t)hit.e * g.tiles_n * g.M;
    }
    tile_walk(hit.local, g.tiles_m, g.tiles_n, g.group_m, bm, bn);
  }
  const int m0 = bm * kBM;
  const int n0 = bn * (kPair ? kBN / 2 : kBN);
  if constexpr (GROUP != GROUP_NONE) nk = (g.K + kStep - 1) / kStep;
  // The main loop runs stages in pairs. An odd count is padded at the front:
  // loop stage 0 is then a stage of zeros written to LDS by the prologue
  // (no loads), and loop stage j holds K stage kt0 + j - pad.
  const int pad = nk & 1;
  const int kbase = kt0 - pad;  // K stage of loop stage 0

  // ---- operand A loader
  KMajorLoader<false> la{};
  MNMajorLoader lma{};
  if constexpr (A_K) {
    const int64_t ldb_ = g.lda * esz;
    la.rs0 = make_rsrc(static_cast<const char*>(g.A) + (int64_t)m0 * ldb_,
                       (int64_t)(g.M - m0) * ldb_);
    la.kbytes = (uint32_t)(g.K * esz);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = 8 * (wave * 8 + i) + (lane >> 3);
      const int c = (lane & 7) ^ kswz_of<kF16>(row);
      la.klim[i] = la.k_limit(m0 + row < g.M, la.kbytes, (uint32_t)(c << 4));
      la.voff[i] = (uint32_t)(row * ldb_) + (uint32_t)(c << 4);
    }
  } else {
    lma.base = static_cast<const char*>(g.A) + (int64_t)m0 * esz;
    lma.ld_bytes = g.lda * esz;
    lma.total_bytes = (int64_t)g.K * g.lda * esz - (int64_t)m0 * esz;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // chunk c holds 16 bytes: columns 8c .. (bf16) or 16c .. (FP8)
      const int kr = IS_FP8 ? 4 * (wave * 8 + i) + (lane >> 4) : 2 * (wave * 8 + i) + (lane >> 5);
      const int c = IS_FP8 ? (lane & 15) ^ mnswz8(kr) : (lane & 31) ^ mnswz(kr);
      lma.voff[i] = (m0 + (c << (IS_FP8 ? 4 : 3)) < g.M)
                        ? (uint32_t)(kr * lma.ld_bytes) + (uint32_t)(c << 4) : kOOB;
    }
  }
  // ---- operand B loader
  KMajorLoader<kPair> lb{};
  MNMajorLoader lmb{};
  if constexpr (B_K) {
    const int64_t ldb_ = g.ldb * esz;
    lb.kbytes = (uint32_t)(g.K * esz);
    if constexpr (kPair) {
      // tile row r: wave half wn = r/128, fragment f = (r/32)%4; f < 2 gate,
      // f >= 2 up; feature n0 + 64 wn + 32 (f%2) + r%32
      const int64_t rem = (int64_t)(g.pair_off - n0) * ldb_;
      lb.rs0 = make_rsrc(static_cast<const char*>(g.B) + (int64_t)n0 * ldb_, rem);
      lb.base1 = static_cast<const char*>(g.B) + (int64_t)(g.pair_off + n0) * ldb_;
      lb.bytes1 = rem;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = 8 * (wave * 8 + i) + (lane >> 3);
        const int c = (lane & 7) ^ kswz_of<kF16>(row);
        const int f = (row >> 5) & 3;
        const int lr = ((row >> 7) << 6) + ((f & 1) << 5) + (row & 31);
        lb.klim[i] = lb.k_limit(n0 + lr < g.N, lb.kbytes, (uint32_t)(c << 4));
        lb.voff[i] = (uint32_t)(lr * ldb_) + (uint32_t)(c << 4);
      }
    } else {
      lb.rs0 = make_rsrc(static_cast<const char*>(g.B) + (int64_t)n0 * ldb_,
                         (int64_t)(g.N - n0) * ldb_);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = 8 * (wave * 8 + i) + (lane >> 3);
        const int c = (lane & 7) ^ kswz_of<kF16>(row);
        lb.klim[i] = lb.k_limit(n0 + row < g.N, lb.kbytes, (uint32_t)(c << 4));
        lb.voff[i] = (uint32_t)(row * ldb_) + (uint32_t)(c << 4);
      }
    }
  } else {
    lmb.base = static_cast<const char*>(g.B) + (int64_t)n0 * esz;
    lmb.ld_bytes = g.ldb * esz;
    lmb.total_bytes = (int64_t)g.K * g.ldb * esz - (int64_t)n0 * esz;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int kr = IS_FP8 ? 4 * (wave * 8 + i) + (lane >> 4) : 2 * (wave * 8 + i) + (lane >> 5);
      const int c = IS_FP8 ? (lane & 15) ^ mnswz8(kr) : (lane & 31) ^ mnswz(kr);
      lmb.voff[i] = (n0 + (c << (IS_FP8 ? 4 : 3)) < g.N)
                        ? (uint32_t)(kr * lmb.ld_bytes) + (uint32_t)(c << 4) : kOOB;
    }
  }

  // This wave's load instruction j of stage kt: j = 0..7 fill its part of
  // the A tile, 8..15 of the B tile.
  // FAST (std::true_type): K-major loaders folded (fold_rows), no K-range test
  auto issue_one = [&](int kt, int j, auto FAST) __attribute__((always_inline)) {
    constexpr bool fast = decltype(FAST)::value;
    char* sa = smem + (kt & (kStages - 1)) * kTileBytes;
    char* sb = smem + kTileB0 + (kt & (kStages - 1)) * kTileBytes;
    if (j < 8) {
      if constexpr (A_K) la.template issue_one<fast>(sa, wave, (uint32_t)((kbase + kt) * kRowBytes), j);
      else lma.issue_one(sa, wave, (kbase + kt) * kStep, j);
    } else {
      if constexpr (B_K) lb.template issue_one<fast>(sb, wave, (uint32_t)((kbase + kt) * kRowBytes), j - 8);
      else lmb.issue_one(sb, wave, (kbase + kt) * kStep, j - 8);
    }
  };
  auto issue = [&](int kt) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 16; ++j) issue_one(kt, j, std::false_type{});
  };

  // accumulators: bf16, 8 x 8 blocks of the 16x16x32 MFMA (4 registers
  // each); FP8, 4 x 4 blocks of the 32x32x64 one (16 registers each)
  // FP8 with two K-major operands runs the 16x16x128 MFMA (k-step = stage):
  // bf16-like 8 x 8 blocks of 16x16; other FP8 products the 32x32x64 one
  constexpr bool kAcc32 = IS_FP8 && !kF16;
  constexpr int kAb = kAcc32 ? 4 : 8;
  using AccV = typename std::conditional<kAcc32, f32x16, f32x4>::type;
  AccV acc[kAb][kAb];
#pragma unroll
  for (int i = 0; i < kAb; ++i)
#pragma unroll
    for (int j = 0; j < kAb; ++j)
#pragma unroll
      for (int r = 0; r < (kAcc32 ? 16 : 4); ++r) acc[i][j][r] = 0.f;

  // fused column sum: thread t owns 8 columns (chunk t%32) of k-rows t/32 + 8j.
  // The k-stages are shared out over the tile columns: the workgroup in tile
  // column bn sums stages bn, bn + tiles_n, ... and writes its partial sums to
  // row bn of e.colsum ([tiles_n][M]); a second pass adds up the rows.
  // Under split-K the share is taken within the split's own stages (global
  // stage index congruent to bn modulo tiles_n) and written to partial row
  // split * tiles_n + bn.
  const bool do_colsum = COLSUM && (e.colsum != nullptr);
  // next loop stage summed (K stages kt0 + local; the front pad shifts them)
  int cs_next = ((bn - kt0) % g.tiles_n + g.tiles_n) % g.tiles_n + pad;
  const int cs_row = split * g.tiles_n + bn;
  constexpr int kCs = IS_FP8 ? 16 : 8;  // columns per thread
  float csum[kCs];
#pragma unroll
  for (int j = 0; j < kCs; ++j) csum[j] = 0.f;

  // A stage has two MFMA k-steps (bf16: 32 elements each, 64 MFMAs of
  // 16x16x32; FP8 with an MN-major operand: 64 each, 16 MFMAs of 32x32x64;
  // the 16x16x128 schedule keeps its own fragments). The fragments of k-step
  // ks live in register slot ks: kFr per operand (bf16: A rows 128 wm + 16 f,
  // B rows 128 wn + 16 f, f = 0..7; FP8: 32-row blocks, f = 0..3).
  constexpr int kKs = 2;
  constexpr int kFr = IS_FP8 ? 4 : 8;
  using Frag = typename std::conditional<IS_FP8, i32x8, bf16x8>::type;
  Frag fa[kKs][kFr], fb[kKs][kFr];
  // fragment J of k-step KS of stage kt: A0..A(kFr-1), then B0.. (KS and J
  // are compile-time constants: they select registers and offsets)
  auto read_one = [&](auto PAR, auto KS, auto J) __attribute__((always_inline)) {
    constexpr int ks = decltype(KS)::value, j = decltype(J)::value, f = j % kFr;
    constexpr int po = ParityOffset<decltype(PAR)>::value;  // the stage buffer's offset
    const char* ta = smem;            // A tiles
    const char* tb = smem + kTileB0;  // B tiles
    if constexpr (j < kFr) {
      if constexpr (IS_FP8 && A_K) fa[ks][f] = frag_k_e4m3<po, ks, f>(ta, 128 * wm, lane);
      else if constexpr (IS_FP8) fa[ks][f] = frag_mn_fp8<po, ks>(ta, 128 * wm + 32 * f, lane);
      else if constexpr (A_K) fa[ks][f] = frag_k_bf16<po, ks, f>(ta, 128 * wm, lane);
      else fa[ks][f] = frag_mn_bf16<po, ks>(ta, 128 * wm + 16 * f, lane);
    } else {
      if constexpr (IS_FP8 && B_K) fb[ks][f] = frag_k_e4m3<po, ks, f>(tb, 128 * wn, lane);
      else if constexpr (IS_FP8) fb[ks][f] = frag_mn_fp8<po, ks>(tb, 128 * wn + 32 * f, lane);
      else if constexpr (B_K) fb[ks][f] = frag_k_bf16<po, ks, f>(tb, 128 * wn, lane);
      else fb[ks][f] = frag_mn_bf16<po, ks>(tb, 128 * wn + 16 * f, lane);
    }
  };
  // the parity of the stage after one of parity P
  auto next_parity = [](auto P) __attribute__((always_inline)) {
    return IC<1 - decltype(P)::value>{};
  };


  // (the 16x16x128 schedule issues its own MFMAs)
  auto mma = [&](int i) __attribute__((always_inline)) {
    if constexpr (kF16) {
    } else if constexpr (IS_FP8) {
      // MFMA i of a stage: k-step i/16, row block (i/4)%4, column block i%4
      const int ks = i >> 4, fm = (i >> 2) & 3, fn = i & 3;
      acc[fm][fn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          fa[ks][fm], fb[ks][fn], acc[fm][fn], FMT & 1, (FMT >> 1) & 1, 0, 0, 0, 0);
    } else {
      // MFMA i of a stage: k-step i/64, row block (i/8)%8, column block i%8.
      // Inline asm with the accumulator tied in place: with the builtin the
      // register allocator parked accumulators in VGPRs and moved them
      // around the loop. An accumulator is reused 64 MFMAs later, far past
      // the instruction's latency; the wait after the main loop covers the
      // epilogue's first reads of the results.
      const int ks = i >> 6, r = (i >> 3) & 7, c = i & 7;
      asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0"
                   : "+a"(acc[r][c])
                   : "v"(fa[ks][r]), "v"(fb[ks][c]));
    }
  };
  // column sums of the A tile of stage kt: bf16, thread t adds chunk t%32 (8
  // columns) of k-rows t/32 + 8j; FP8, chunk t%16 (16 columns) of k-rows
  // t/16 + 16j (j = 0..7); FP8 codes are decoded to floats exactly.
  // colsum_issue reads part j without waiting for it; colsum_add adds it
  // once a wait has covered the read.
  auto colsum_issue = [&](int kt, int j) __attribute__((always_inline)) -> u32x4 {
    const char* sa = smem + (kt & (kStages - 1)) * kTileBytes;
    if constexpr (IS_FP8) {
      const int c = tid & 15;
      const int kr = (tid >> 4) + 16 * j;
      return ds_read_b128_async(sa + kr * 256 + ((c ^ mnswz8(kr)) << 4));
    } else {
      const int c = tid & 31;
      const int kr = (tid >> 5) + 8 * j;
      return ds_read_b128_async(sa + kr * 512 + ((c ^ mnswz(kr)) << 4));
    }
  };
  auto colsum_add = [&](u32x4 v) __attribute__((always_inline)) {
    asm volatile("" : "+v"(v));  // keeps the adds after the wait before them
    if constexpr (IS_FP8) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const auto lo = (FMT & 1) ? __builtin_amdgcn_cvt_pk_f32_bf8((int)v[w], false)
                                  : __builtin_amdgcn_cvt_pk_f32_fp8((int)v[w], false);
        const auto hi = (FMT & 1) ? __builtin_amdgcn_cvt_pk_f32_bf8((int)v[w], true)
                                  : __builtin_amdgcn_cvt_pk_f32_fp8((int)v[w], true);
        csum[4 * w] += lo[0];
        csum[4 * w + 1] += lo[1];
        csum[4 * w + 2] += hi[0];
        csum[4 * w + 3] += hi[1];
      }
    } else {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        csum[2 * w] += bf2f((bf16_t)(v[w] & 0xffffu));
        csum[2 * w + 1] += bf2f((bf16_t)(v[w] >> 16));
      }
    }
  };
  // Every stage's loads are issued, also those of the two stages past the end
  // of the loop (into buffers no MFMA and no column sum reads): the number of
  // loads in flight stays uniform, one wait count and no branches. Their
  // offsets fall outside the resources (no memory traffic), except for
  // folded K-major loaders, which read whatever lies behind the rows.
  constexpr int kMma = 16 * kKs;  // MFMAs per stage (FP8, 32x32x64)

  // FP8 stage kt with an MN-major operand (32 slots in two groups of 16,
  // group q issuing the MFMAs of k-step q): the 8 fragments of a k-step are
  // read right after the previous stage's MFMAs of that k-step have released
  // their registers, one every two slots, so the LDS reads are spread over
  // the stage instead of coming in bursts:
  //   group 0   reads of stage kt's k-step 1 (and of its column-sum parts)
  //   barrier   every wave has finished reading stage kt, and stage kt+1
  //             has landed (vmcnt(0))
  //   group 1   reads of stage kt+1's k-step 0; the 16 loads of stage kt+2;
  //             the column-sum parts are added
  constexpr int kDmaStride = 1;  // slots per load from slot 16 on
  // Column sums: in a stage whose sums are this workgroup's share, slot 1
  // reads the eight parts, and the slot after the stage's first barrier (whose
  // wait covers the reads) adds them. The parts live within one stage: the
  // reads are asm, so the compiler takes their registers as written at once,
  // and a value it kept across stages could be spilled before its data
  // arrived. One uniform branch at each of the two slots, laid out for the
  // common case of no column sums.
  auto stage_iter_rolling = [&](int kt, auto FAST, auto PAR) __attribute__((always_inline)) {
    const auto PAR1 = next_parity(PAR);  // stage kt+1
    // fragment reads (asm, not tracked by the compiler) of the previous
    // stage must have landed before their first use here
    wait_lds();
    int cs_mode = 0;  // this stage's column sums are this workgroup's share
    u32x4 cs_buf[8];
    if constexpr (COLSUM) {
      const int on = (do_colsum && kt == cs_next) ? 1 : 0;
      cs_next += on * g.tiles_n;
      cs_mode = __builtin_amdgcn_readfirstlane(on);
    }
    static_for<kMma>([&](auto I) {
      constexpr int i = decltype(I)::value;
      mma(i);
      constexpr int grp = i >> 4, r = i & 15;
      if constexpr ((r & 1) == 0) {
        if constexpr (grp == 0) read_one(PAR, IC<kKs - 1>{}, IC<(r >> 1)>{});
        else read_one(PAR1, IC<grp - 1>{}, IC<(r >> 1)>{});
      }
      if constexpr (COLSUM && i == 1) {
        if (__builtin_expect(cs_mode != 0, 0)) {
#pragma unroll
          for (int j = 0; j < 8; ++j) cs_buf[j] = colsum_issue(kt, j);
        }
      }
      if constexpr (COLSUM && i == 16) {
        if (__builtin_expect(cs_mode != 0, 0)) {
#pragma unroll
          for (int j = 0; j < 8; ++j) colsum_add(cs_buf[j]);
        }
      }
      if constexpr (i >= 16 && i < 16 + 16 * kDmaStride && (i - 16) % kDmaStride == kDmaStride - 1)
        issue_one(kt + kStages, (i - 16) / kDmaStride, FAST);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (i == 15) wait_and_barrier<0>();
    });
  };

  // bf16 stage kt (128 slots of one 16x16x32 MFMA each, k-step 0 in slots
  // 0..63, k-step 1 in 64..127), any operand layouts:
  //   slots 0..47     read this stage's k-step 1 (16 fragments, one every
  //                   third slot) into the registers k-step 1 of the last
  //                   stage has released
  //   slot 63         the stage's one barrier: every wave has read all of
  //                   stage kt (its buffer is free) and stage kt+1 has landed
  //                   (this wave's loads: vmcnt(0))
  //   slots 64..111   read stage kt+1's k-step 0 into the registers k-step 0
  //                   of this stage has released
  //   slots 64..127   the 16 loads of stage kt+2, one every fourth slot
  // A load has a whole stage to land, and every read has 16 slots before the
  // wait that covers it (the barrier, or the top of the next stage).
  auto stage_iter16 = [&](int kt, auto FAST, auto PAR) __attribute__((always_inline)) {
    const auto PAR1 = next_parity(PAR);  // stage kt+1
    wait_lds();  // this stage's k-step 0 (read in slots 64..111 of the last)
    // Two wait states before the first MFMA. The MFMAs are asm, so the
    // compiler's hazard checks do not see their operands; where a kernel has
    // two loop forms it may move fragments into the registers one loop
    // expects with VALU copies just before it, and an MFMA may not read a
    // VGPR that a VALU instruction wrote fewer than two wait states earlier.
    asm volatile("s_nop 1");
    int cs_mode = 0;  // this stage's column sums are this workgroup's share
    u32x4 cs_buf[8];
    if constexpr (COLSUM) {
      const int on = (do_colsum && kt == cs_next) ? 1 : 0;
      cs_next += on * g.tiles_n;
      cs_mode = __builtin_amdgcn_readfirstlane(on);
    }
    static_for<128>([&](auto I) {
      constexpr int i = decltype(I)::value;
      constexpr int h = i >> 6, sl = i & 63;
      mma(i);
      if constexpr (sl % 3 == 0 && sl / 3 < 2 * kFr) {
        if constexpr (h == 0) read_one(PAR, IC<1>{}, IC<sl / 3>{});
        else read_one(PAR1, IC<0>{}, IC<sl / 3>{});
      }
      if constexpr (COLSUM && i == 1) {
        if (__builtin_expect(cs_mode != 0, 0)) {
#pragma unroll
          for (int j = 0; j < 8; ++j) cs_buf[j] = colsum_issue(kt, j);
        }
      }
      if constexpr (COLSUM && i == 24) {
        if (__builtin_expect(cs_mode != 0, 0)) {
#pragma unroll
          for (int j = 0; j < 8; ++j) colsum_add(cs_buf[j]);
        }
      }
      // loads of stage kt+2: the A tile's eight once every wave has read A of
      // stage kt (the barrier after slot 23), one every fifth slot; the B
      // tile's eight after the stage's main barrier, one every eighth slot
      if constexpr (i >= 25 && i < 25 + 5 * 8 && (i - 25) % 5 == 0) issue_one(kt + kStages, (i - 25) / 5, FAST);
      if constexpr (h == 1 && (sl & 7) == 3) issue_one(kt + kStages, 8 + (sl >> 3), FAST);
      __builtin_amdgcn_sched_barrier(0);
      // A's fragments of k-step 1 are read in slots 0..21 (and the column-sum
      // parts at slot 1): after this barrier A of stage kt is free
      if constexpr (i == 23) wait_and_barrier<63>();
      // stage kt+1 has landed: all but this stage's eight A loads are done
      if constexpr (i == 63) wait_and_barrier<8>();
    });
  };

  // FP8 stage kt with two K-major operands: 64 slots of one 16x16x128 MFMA
  // (a stage is one k-step; row block r = i / 8, column block c = i % 8 of
  // the wave tile). The B fragments of a stage are read during the stage
  // before (gb[PAR]); the A fragments roll through three register sets (A_r
  // in ga[r % 3]), each read seven slots before its row's first MFMA.
  //   slots 0, 2, 4, 6       A loads 4..7 of stage kt+1
  //   slot 8r + 1            A_{r+1} read (r = 0..6)
  //   barrier before slot 8  every wave is done with stage kt-1 (the B tile of
  //                          this buffer is free) and has stage kt+1's B tile
  //                          (all but its eight A loads done)
  //   slots 9, 11, .., 23    B loads of stage kt+2
  //   slots 10, 16, .., 52   reads of stage kt+1's B fragments
  //   barrier before slot 56 every wave has read A_7 (the A tile is free) and
  //                          has stage kt+1's A tile (all but the B loads)
  //   slot 57                A_0 of stage kt+1 read
  //   slots 58..61           A loads 0..3 of stage kt+2
  // A load has at least 48 slots to land; the waits before rows 2..6 let the
  // one B fragment read issued since A_{r+1} stay in flight.
  i32x8 ga[3], gb[2][8];
  auto read16 = [&](auto PR, auto IS_B, auto IDX) __attribute__((always_inline)) {
    constexpr int po = ParityOffset<decltype(PR)>::value;
    constexpr int idx = decltype(IDX)::value;
    if constexpr (decltype(IS_B)::value)
      gb[decltype(PR)::value][idx] = frag_k_e4m3_16<po, idx>(smem + kTileB0, 128 * wn, lane);
    else
      ga[idx % 3] = frag_k_e4m3_16<po, idx>(smem, 128 * wm, lane);
  };
  auto stage_f16 = [&](int kt, auto FAST, auto PAR) __attribute__((always_inline)) {
    const auto PAR1 = next_parity(PAR);  // stage kt+1
    constexpr int par = decltype(PAR)::value;
    wait_lds();  // this stage's B fragments and A_0 (read in the last)
    asm volatile("s_nop 1");  // as in stage_iter16
    static_for<64>([&](auto I) {
      constexpr int i = decltype(I)::value, r = i >> 3, c = i & 7;
      if constexpr (i == 8 || i == 56) wait_and_barrier<8>();
      if constexpr (i > 8 && i < 56 && c == 0) wait_lds<2>();
      {
        auto& d = acc[r][c];
        auto& a = ga[r % 3];
        auto& b = gb[par][c];
        // operand formats: cbsz / blgp 1 = E5M2 (A / B), 0 = E4M3
        if constexpr ((FMT & 3) == 1)
          asm volatile("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, %0 cbsz:1" : "+a"(d) : "v"(a), "v"(b));
        else if constexpr ((FMT & 3) == 2)
          asm volatile("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, %0 blgp:1" : "+a"(d) : "v"(a), "v"(b));
        else if constexpr ((FMT & 3) == 3)
          asm volatile("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, %0 cbsz:1 blgp:1" : "+a"(d)
                       : "v"(a), "v"(b));
        else
          asm volatile("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, %0" : "+a"(d) : "v"(a), "v"(b));
      }
      if constexpr (c == 1 && r < 7) read16(PAR, std::false_type{}, IC<r + 1>{});
      if constexpr (i >= 10 && i <= 52 && (i - 10) % 6 == 0) read16(PAR1, std::true_type{}, IC<(i - 10) / 6>{});
      if constexpr (i == 57) read16(PAR1, std::false_type{}, IC<0>{});
      if constexpr (i < 8 && (i & 1) == 0) issue_one(kt + 1, 4 + (i >> 1), FAST);
      if constexpr (i >= 9 && i <= 23 && (i & 1) == 1) issue_one(kt + 2, 8 + ((i - 9) >> 1), FAST);
      if constexpr (i >= 58 && i <= 61) issue_one(kt + 2, i - 58, FAST);
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // prologue: stages 0 and 1 in flight; stage 0's first k-steps in registers.
  // A front pad stage is zeros written here with LDS stores (its A and B
  // tiles in buffer 0, 256 bytes per thread): no load of it is issued, and
  // its MFMAs add exact zeros. The barrier's wait covers the stores.
  if (pad) {
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int off = (i < 8 ? 0 : kTileB0) + ((i & 7) * kThreads + tid) * 16;
      *reinterpret_cast<u32x4*>(smem + off) = z;
    }
  } else {
    issue(0);
  }
  if constexpr (kF16) {
    // stage 1: its B tile, then A loads 0..3 (the first stage issues 4..7)
#pragma unroll
    for (int j = 8; j < 16; ++j) issue_one(1, j, std::false_type{});
#pragma unroll
    for (int j = 0; j < 4; ++j) issue_one(1, j, std::false_type{});
    wait_and_barrier<12>();
  } else {
    issue(1);
    wait_and_barrier<16>();
  }
  // The main loop runs two stages per iteration, even ones in buffer 0 and odd
  // ones in buffer 1, so each read's stage offset is an immediate and the
  // per-lane read addresses stay the same from stage to stage. An odd count
  // of stages starts with the zero stage of the prologue (pad). When K is a
  // whole number of stages (every product at the benchmark shapes; split-K
  // gives every split whole stages), the K-major loaders are folded (no
  // per-lane K test: the K-range test only separates rows past the tensor's
  // end, which get an out-of-range offset once). A ragged K keeps the test on
  // every K-major load; products with both operands MN-major need none (their
  // resource is rebased on each stage's first k-row and ends at the tensor's
  // last one).
  // (A conditional stage inside or after the paired loop made the compiler
  // move the accumulators between registers; with a second loop form in the
  // column-sum kernels it spilled an asm read's destination before the read
  // landed: those kernels have one loop.)
  auto pair_loop = [&](auto stage, auto FAST, int n) __attribute__((always_inline)) {
    for (int kt = 0; kt < n; kt += 2) {
      stage(kt, FAST, IC<0>{});
      stage(kt + 1, FAST, IC<1>{});
    }
  };
  // `after`: the fence after the loop, inside each loop form, so that no
  // read is in flight where the two forms' paths meet
  auto main_loop = [&](auto stage, auto after) __attribute__((always_inline)) {
    if constexpr (!A_K && !B_K) {
      pair_loop(stage, std::false_type{}, nk + pad);
      after();
    } else {
      static_assert(!COLSUM, "the fused column sum reads an MN-major A tile");
      if (g.K % kStep == 0) {
        if constexpr (A_K) la.fold_rows();
        if constexpr (B_K) lb.fold_rows();
        pair_loop(stage, std::true_type{}, nk + pad);
        after();
      } else {
        pair_loop(stage, std::false_type{}, nk + pad);
        after();
      }
    }
  };
  // Fragment reads are asm: the compiler takes their results as written when
  // the read is issued, not when it lands. Outside the loop's own schedule
  // (whose waits cover every use) two places need a fence, a wait for all LDS
  // reads followed by an empty asm that takes every fragment register as
  // read and rewritten, so that the compiler neither copies a fragment nor
  // reuses its register before the data has landed:
  //  * after the prologue's reads: where a kernel has two loop forms it may
  //    copy the fragments into the registers one of them expects (a build
  //    without the fence did, before the reads landed, and gave NaN);
  //  * after the loop: the last stage's reads ahead are still in flight, and
  //    their registers are free for the code that follows (a build without
  //    the fence set up an epilogue address in one of them).
  // Both places have reads of k-step 0 fragments only in flight.
  auto frag_keep = [&](auto I) __attribute__((always_inline)) {
    constexpr int i = decltype(I)::value;
    auto& ra = fa[0][i];  // named first: an asm operand alone does not make
    auto& rb = fb[0][i];  // the lambda capture the array
    asm volatile("" : "+v"(ra), "+v"(rb));
  };
  auto frag_fence = [&]() __attribute__((always_inline)) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    static_for<kFr>(frag_keep);
  };
  // the 16x16x128 schedule's reads in flight at its fences: stage 0's (or
  // the stage past the end's) B fragments and A_0
  auto frag_fence16 = [&]() __attribute__((always_inline)) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    static_for<8>([&](auto I) {
      auto& rb = gb[0][decltype(I)::value];
      asm volatile("" : "+v"(rb));
    });
    auto& ra = ga[0];
    asm volatile("" : "+v"(ra));
  };
  if constexpr (kF16) {
    static_for<8>([&](auto J) { read16(IC<0>{}, std::true_type{}, J); });
    read16(IC<0>{}, std::false_type{}, IC<0>{});
    frag_fence16();
    main_loop(stage_f16, frag_fence16);
  } else if constexpr (!IS_FP8) {
    static_for<2 * kFr>([&](auto J) { read_one(IC<0>{}, IC<0>{}, J); });
    frag_fence();
    main_loop(stage_iter16, frag_fence);
  } else {
    static_for<8 * (kKs - 1)>([&](auto J) {
      constexpr int j = decltype(J)::value;
      read_one(IC<0>{}, IC<j / 8>{}, IC<j & 7>{});
    });
    frag_fence();
    main_loop(stage_iter_rolling, frag_fence);
  }
  if constexpr (!kAcc32) {
    // the last MFMAs (asm, unseen by the compiler's hazard checks) complete
    // before any instruction reads their accumulators
    asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15\n\ts_nop 15" ::: "memory");
  }
  // ---- fused column sum of A: this workgroup's share of the k-stages
  if constexpr (COLSUM) {
    if (do_colsum) {
      __syncthreads();  // all waves are done with the stage buffers
      // 8 (bf16) or 16 (FP8) groups of 256 column sums
      constexpr int kGroups = IS_FP8 ? 16 : 8;
      float* red = reinterpret_cast<float*>(smem);
#pragma unroll
      for (int j = 0; j < kCs; ++j)
        red[(tid / (256 / kGroups)) * 256 + (tid % (256 / kGroups)) * kCs + j] = csum[j];
      __syncthreads();
      const int m = m0 + tid;
      float s = 0.f;
#pragma unroll
      for (int q = 0; q < kGroups; ++q) s += red[q * 256 + tid];
      if constexpr (IS_FP8) s *= *e.scale_a;
      if (m < g.M) e.colsum[(int64_t)cs_row * g.M + m] = s;
    }
  }

  // ---- a split tile of a partial last round: the two halves meet here
  const float* tail_other = nullptr;
  if constexpr (kTail) {
    if (tail_p >= 0) {
      // accumulator register r of lane l of wave w in 16-byte chunks: chunk
      // c = r / 4 at floats (w * 64 + c) * 256 + 4 l of the half's 256 KiB
      constexpr int kChunks = (int)(sizeof(AccV) / 16);  // per block
      const int64_t half_floats = (int64_t)kBM * kBN;
      // the lane's offset as a fresh value: not one the compiler would keep
      // live across the main loop from the prologue's address arithmetic
      int lane4 = 4 * (int)(threadIdx.x & 63);
      asm volatile("" : "+v"(lane4));
      float* mine = g.tail_ws + ((int64_t)tail_p * 2 + tail_h) * half_floats + wave * 16384 + lane4;
      // Stored from the accumulator registers (asm with AGPR operands: with
      // plain stores the compiler copies every accumulator to VGPRs first
      // and spills); 1 KiB per wave and chunk, 16 bytes per lane. The
      // compiler's hazard checks do not see asm stores: a VALU write to the
      // data registers of a store of more than 8 bytes needs a wait state,
      // and the compiler may stage the next chunk in the same registers, so
      // each store is followed by two.
      static_for<kAb * kAb>([&](auto B) {
        constexpr int b = decltype(B)::value;
        auto& v = acc[b / kAb][b % kAb];
        float* p = mine + b * kChunks * 256;
        if constexpr (kChunks == 1) {
          asm volatile("global_store_dwordx4 %0, %1, off\n\ts_nop 1" : : "v"(p), "a"(v) : "memory");
        } else {
          asm volatile(
              "global_store_dwordx4 %0, %1, off\n\t"
              "global_store_dwordx4 %0, %2, off offset:1024\n\t"
              "global_store_dwordx4 %0, %3, off offset:2048\n\t"
              "global_store_dwordx4 %0, %4, off offset:3072\n\t"
              "s_nop 1"
              :
              : "v"(p), "a"(__builtin_shufflevector(v, v, 0, 1, 2, 3)),
                "a"(__builtin_shufflevector(v, v, 4, 5, 6, 7)),
                "a"(__builtin_shufflevector(v, v, 8, 9, 10, 11)),
                "a"(__builtin_shufflevector(v, v, 12, 13, 14, 15))
              : "memory");
        }
      });
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();  // every wave's dump has reached the L2
      __shared__ int tail_seen;
      if (tid == 0)
        tail_seen = __hip_atomic_fetch_add(g.tail_cnt + tail_p, 1, __ATOMIC_ACQ_REL,
                                           __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
      if (tail_seen == 0) {
        // the other half, still running, finishes the tile: this one runs
        // the epilogue with no tensors (every access out of range, no memory
        // traffic), the same code either way
        e.out = nullptr;
        e.out2 = nullptr;
        e.aux = nullptr;
      } else {
        // the epilogue adds the other half's dump (its release, this
        // atomic's acquire) as it stages the accumulators
        tail_other =
            g.tail_ws + ((int64_t)tail_p * 2 + (1 - tail_h)) * half_floats + wave * 16384 + lane4;
        if (tid == 0) g.tail_cnt[tail_p] = 0;  // for the next launch
      }
    }
  }

  __syncthreads();  // every wave is done reading the stage buffers
  float amax = 0.f;
  if constexpr (EPI == EPI_F32) {
    if (e.accumulate)
      store_tile<IS_FP8, EPI, OutT, true>(g, e, acc, smem, wave, lane, m0, n0, amax, tail_other);
    else
      store_tile<IS_FP8, EPI, OutT, false>(g, e, acc, smem, wave, lane, m0, n0, amax, tail_other);
  } else {
    constexpr bool kLoads = (EPI == EPI_DGELU || EPI == EPI_DSWIGLU || EPI == EPI_DGELU_Q ||
                             EPI == EPI_DSWIGLU_Q);
    store_tile<IS_FP8, EPI, OutT, kLoads>(g, e, acc, smem, wave, lane, m0, n0, amax, tail_other);
  }
  if constexpr (IS_FP8 && (EPI == EPI_BIAS_GELU || EPI == EPI_BIAS_GELU_Q || EPI == EPI_DGELU_Q ||
                          EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_Q || EPI == EPI_DSWIGLU_Q)) {
    amax = wave_max(amax);
    __shared__ float wmax[4];
    if (lane == 0) wmax[wave] = amax;
    __syncthreads();
    if (tid == 0) {
      float m = 0.f;
      for (int w = 0; w < 4; ++w) m = __builtin_fmaxf(m, wmax[w]);
      e.amax_part[blockIdx.x] = m;
    }
  }
  if (clk_on && tid == 0) {
    g_in.clk[4 * blockIdx.x + 2] = __builtin_amdgcn_s_memtime();
    g_in.clk[4 * blockIdx.x + 3] = __builtin_amdgcn_s_memrealtime();
  }
}

}  // namespace tpmlp
