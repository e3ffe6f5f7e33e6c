// Epilogues of the MLP block's GEMMs. The per-element forms below serve the
// VALU (fp32) tile kernel; the MFMA kernel applies the same formulas to eight
// consecutive columns at a time. Each takes the fp32 accumulator value of C
// at (row, col) and writes the block's tensors:
//
//   EPI_STORE     out = alpha * acc                   (y_partial, dx_partial)
//   EPI_F32       out = acc (+ out if accumulate)     (dW1, dW2, fp32)
//   EPI_BIAS_GELU h = alpha * acc + b1[col]; out2 = h; out = gelu(h)
//   EPI_SWIGLU    (gate, up) pair: out2 = [g | u]; out = silu(g) * u
//   EPI_DGELU     out = acc * gelu'(h[row, col])      (dH)
//   EPI_DSWIGLU   out[col] = acc * u * silu'(g); out[col + Fs] = acc * silu(g)
//   EPI_BIAS_GELU_Q  as EPI_BIAS_GELU; out = E4M3 codes of a * q_scale (a in fp32)
//   EPI_DGELU_Q   as EPI_DGELU; out = E5M2 codes of dH * q_scale
//   EPI_SWIGLU_Q  as EPI_SWIGLU; out = E4M3 codes of a * q_scale (a in fp32)
//   EPI_DSWIGLU_Q as EPI_DSWIGLU; both halves E5M2 codes of dH * q_scale
//   EPI_BIAS      out = alpha * acc + bias[col]        (packed q, k, v)
// (FP8 codes saturate at the format's largest finite value; the quantising
// epilogues also fold max |value| into a per-workgroup amax.)
//
// The activation is evaluated on h as stored (rounded to the activation type),
// so the backward pass, which reads the stored h, differentiates exactly the
// function whose value the forward produced.
#pragma once

#include "common.h"

namespace tpmlp {

enum EpiKind : int {
  EPI_STORE = 0,
  EPI_F32 = 1,
  EPI_BIAS_GELU = 2,
  EPI_SWIGLU = 3,
  EPI_DGELU = 4,
  EPI_DSWIGLU = 5,
  EPI_BIAS_GELU_Q = 6,  // EPI_BIAS_GELU, a quantised to E4M3 at *q_scale
  EPI_DGELU_Q = 7,      // EPI_DGELU, dH quantised to E5M2 at *q_scale
  EPI_BIAS = 8,         // bias added, no activation (attention's QKV projection)
  EPI_SWIGLU_Q = 9,     // EPI_SWIGLU, a quantised to E4M3 at *q_scale
  EPI_DSWIGLU_Q = 10,   // EPI_DSWIGLU, dH quantised to E5M2 at *q_scale
};

// Grouped products (the expert MLPs of a mixture-of-experts layer): group e
// owns the rows [off_e, off_e + c_e) of the token-major tensors, off_e the
// sum of the counts before it, and its own block of each per-group tensor.
//   GROUP_M: the tokens are M (forward, data gradients): A and the outputs
//            are token-major; B (the weight) and the bias are per group.
//   GROUP_K: the tokens are K (weight gradients): A and B are token-major;
//            the output and the column-sum partials are per group.
// Counts are read on the device and clamped (negative as 0, prefix sums
// saturated at `rows`), so no row outside [0, rows) is touched.
enum GroupKind : int { GROUP_NONE = 0, GROUP_M = 1, GROUP_K = 2 };

struct GemmArgs {
  const void* A;
  const void* B;
  int64_t lda, ldb;
  int M, N, K;     // N: output columns (for the gated fc1: the Fs pair columns)
  int pair_off;    // gated blocks: Fs (offset between gate and up rows/columns)
  int tiles_m, tiles_n, group_m;
  // grouped products only
  const int* counts;       // [groups] rows per group (device)
  int groups;
  int rows;                // rows of the token-major tensors
  int64_t b_gstride;       // GROUP_M: elements between groups' B blocks
  int64_t out_gstride;     // GROUP_K: elements between groups' output blocks
  int64_t bias_gstride;    // GROUP_M: elements between groups' biases
  // split-K (ungrouped products only): k_splits > 1 workgroups share a tile,
  // split s taking stages [s * split_stages, (s + 1) * split_stages) and
  // writing an fp32 partial plane at out + s * M * ldo (EPI_F32, no
  // accumulate); a reduce pass forms the result
  int k_splits;
  int split_stages;
  // a partial last round (ungrouped, unsplit products): the last tail_tiles
  // tiles of the walk (a multiple of 8; the others a multiple of 8 too) are
  // each taken by two workgroups, one per half of the K stages, placed on the
  // same XCD; each dumps its accumulators to its half's 256 KiB of tail_ws
  // ([tail_tiles][2][256 x 256] floats, in register order), then adds one to
  // the tile's counter in tail_cnt ([tail_tiles], zero at the launch); the
  // one that finds the other's count adds the other's dump to its own
  // accumulators, runs the epilogue and sets the counter back to zero
  int tail_tiles;
  float* tail_ws;
  int* tail_cnt;
  // clock capture (the timing facility), or null: each workgroup writes
  // (shader clock, real-time counter) at its start and end to
  // clk[4 * blockIdx.x .. +3] while blockIdx.x < clk_slots
  unsigned long long* clk;
  int clk_slots;
};

struct EpiArgs {
  void* out;          int64_t ldo;    // primary output
  void* out2;         int64_t ldo2;   // saved pre-activation h (may be null)
  const void* bias;                   // b1, or the QKV bias (may be null)
  const void* aux;    int64_t ldaux;  // saved h read by the dgrad epilogues
  const float* scale_a;               // e4m3: dequantisation factors (device)
  const float* scale_b;
  float* amax_part;                   // e4m3 fc1 (a) / fc2 dgrad (dH): per-workgroup amax
  const float* q_scale;               // quantising epilogues: the factor codes are taken at
  float* colsum;                      // fc1 wgrad: column sums of A over k, or null:
                                      //   VALU kernel: db1 itself (written by tile
                                      //   column 0); MFMA kernel: a [tiles_n][M]
                                      //   array of per-tile-column partial sums
  int accumulate;                     // EPI_F32 and colsum: add into outputs
};

// Non-paired kinds. `bias` is b1[col] (0 when absent). For IS_FP8 the
// activation is written as bf16 and its rounded magnitude folded into amax.
template <int EPI, typename OutT, bool IS_FP8>
__device__ __forceinline__ void epi_one(const EpiArgs& e, int pair_off, int row, int col,
                                        float v, float alpha, float bias, float& amax) {
  const int64_t o = (int64_t)row * e.ldo + col;
  if constexpr (EPI == EPI_STORE) {
    Elem<OutT>::store(e.out, o, v * alpha);
  } else if constexpr (EPI == EPI_BIAS) {
    Elem<OutT>::store(e.out, o, v * alpha + bias);
  } else if constexpr (EPI == EPI_F32) {
    float* out = static_cast<float*>(e.out);
    out[o] = e.accumulate ? out[o] + v : v;
  } else if constexpr (EPI == EPI_BIAS_GELU) {
    const float h = v * alpha + bias;
    if (e.out2) Elem<OutT>::store(e.out2, (int64_t)row * e.ldo2 + col, h);
    const float a = gelu_f(Elem<OutT>::round(h));
    if constexpr (IS_FP8) amax = __builtin_fmaxf(amax, __builtin_fabsf(round_bf16(a)));
    Elem<OutT>::store(e.out, o, a);
  } else if constexpr (EPI == EPI_DGELU) {
    const float h = Elem<OutT>::load(e.aux, (int64_t)row * e.ldaux + col);
    Elem<OutT>::store(e.out, o, v * gelu_grad_f(h));
  } else if constexpr (EPI == EPI_DSWIGLU) {
    const int64_t ho = (int64_t)row * e.ldaux + col;
    const float gt = Elem<OutT>::load(e.aux, ho);
    const float up = Elem<OutT>::load(e.aux, ho + pair_off);
    Elem<OutT>::store(e.out, o, v * up * silu_grad_f(gt));
    Elem<OutT>::store(e.out, o + pair_off, v * silu_f(gt));
  }
}

// Gated fc1: gate and up accumulators of pair column `col`.
template <typename OutT>
__device__ __forceinline__ void epi_pair(const EpiArgs& e, int pair_off, int row, int col,
                                         float gt, float up) {
  if (e.out2) {
    Elem<OutT>::store(e.out2, (int64_t)row * e.ldo2 + col, gt);
    Elem<OutT>::store(e.out2, (int64_t)row * e.ldo2 + pair_off + col, up);
  }
  const float gr = Elem<OutT>::round(gt), ur = Elem<OutT>::round(up);
  Elem<OutT>::store(e.out, (int64_t)row * e.ldo + col, silu_f(gr) * ur);
}

}  // namespace tpmlp
