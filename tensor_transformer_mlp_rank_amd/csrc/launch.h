// Host-side launchers of the libtpmlp kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>

#include "epilogue.h"

namespace tpmlp {

// The GEMM steps of the block; each maps to one kernel instantiation per
// element type.
enum Step : int {
  FC1_FWD_GELU = 0,   // x . W1^T, bias + GELU, saves h, writes a (e4m3: bf16 a + amax)
  FC1_FWD_SWIGLU,     // x . W1^T (gate/up pairs), SiLU(g) * u, saves h, writes a
  FC2_FWD,            // a . W2^T -> y_partial
  FC2_DGRAD_GELU,     // dy . W2, times gelu'(h) -> dH
  FC2_DGRAD_SWIGLU,   // dy . W2, SwiGLU derivative -> dH (both halves)
  FC1_DGRAD,          // dH . W1 -> dx_partial
  WGRAD,              // A^T . B over tokens -> fp32 (dW2, or dW1 without bias)
  WGRAD_COLSUM,       // same, plus column sums of A (dW1 and db1)
  FC1_FWD_GELU_Q,     // e4m3: as FC1_FWD_GELU, a quantised to e4m3 in the epilogue
  FC2_DGRAD_GELU_Q,   // e4m3 weights, e5m2 dy: dH quantised to e5m2 in the epilogue
  QKV_FWD_BIAS,       // attention: x . Wqkv^T + bias -> packed q, k, v
  FC1_FWD_SWIGLU_Q,   // e4m3: as FC1_FWD_SWIGLU, a quantised to e4m3 in the epilogue
  FC2_DGRAD_SWIGLU_Q, // e4m3 weights, e5m2 dy: both halves of dH quantised to e5m2
  WGRAD_T,            // e4m3: A^T . B over tokens from token-contiguous copies of both
                      // operands (A e5m2) -> fp32
  kNumSteps
};

enum Kind : int { KIND_F32 = 0, KIND_BF16 = 1, KIND_E4M3 = 2 };

// Fill the grid fields of `g` (tiles_m, tiles_n, group_m) for the step and
// return the number of workgroups (0: nothing to launch).
int mfma_grid(Step step, GemmArgs& g);
int f32_grid(Step step, GemmArgs& g);

// Enqueue one GEMM step; `g` must have its grid fields filled.
hipError_t mfma_launch(bool fp8, Step step, const GemmArgs& g, const EpiArgs& e,
                       hipStream_t stream);

// Grouped (bf16) GEMM steps. `g` carries the per-group tile grid (tiles_m,
// tiles_n of one group; for GROUP_M tiles_m is that of the largest possible
// group) and the group fields; the launch covers every group's tiles.
// Returns the number of workgroups launched (0: nothing to launch).
int64_t mfma_group_grid(Step step, int group, GemmArgs& g);

// Split-K form of a bf16 step whose epilogue is a plain store, a bias, or an
// fp32 store/accumulate (FC2_FWD, QKV_FWD_BIAS, FC1_DGRAD, WGRAD,
// WGRAD_COLSUM): g.k_splits workgroups per tile write fp32 partial planes to
// e.out (k_splits x M x N floats); splitk_reduce_launch then forms the output.
hipError_t mfma_split_launch(Step step, const GemmArgs& g, const EpiArgs& e, hipStream_t stream);
hipError_t splitk_reduce_launch(const float* part, int splits, int64_t M, int64_t N, void* out,
                                bool out_bf16, const void* bias, int accumulate,
                                hipStream_t stream);
hipError_t mfma_group_launch(Step step, int group, const GemmArgs& g, const EpiArgs& e,
                             hipStream_t stream);
hipError_t f32_launch(Step step, const GemmArgs& g, const EpiArgs& e, hipStream_t stream);

// db1 from the MFMA kernel's [nparts][M] column-sum partials ([groups] of
// them, one output row of M each).
hipError_t colsum_reduce_launch(const float* part, int nparts, int M, float* out, int accumulate,
                                hipStream_t stream, int groups = 1);

// a = act(h) from the saved pre-activation h ([rows][G fs], bf16 for
// KIND_BF16 and KIND_E4M3, fp32 for KIND_F32) into a ([rows][fs]: bf16,
// fp32, or E4M3 codes at the factor 1 / *scale_inv for KIND_E4M3, GELU
// only).
hipError_t act_recompute_launch(Kind kind, bool swiglu, const void* h, int64_t rows, int64_t fs,
                                void* a, const float* scale_inv, hipStream_t stream);

// n ints at p set to zero (a kernel, so that the call can be captured into a
// graph).
hipError_t fill_zero_i32_launch(int* p, int n, hipStream_t stream);
// dst [cols][ld] = transpose of the byte array src [rows][cols] (cols and ld
// multiples of 16, ld >= rows; dst's columns [rows, ld) zero)
hipError_t transpose_u8_launch(const void* src, int64_t rows, int64_t cols, void* dst, int64_t ld,
                               hipStream_t stream);
// out[f] (+)= *scale_inv * sum over t < n of E5M2 src[f][t] (rows rows of ld bytes)
hipError_t rowsum_e5m2_launch(const void* src, int64_t rows, int64_t n, int64_t ld,
                              const float* scale_inv, float* out, int accumulate, hipStream_t stream);

// Quantiser passes. src_bf16 selects the source type (bf16 or f32).
int quant_parts(int64_t n);
hipError_t amax_partial_launch(bool src_bf16, const void* src, int64_t n, float* partial,
                               int nparts, hipStream_t stream);
hipError_t quantize_launch(bool src_bf16, const void* src, int64_t n, uint8_t* dst,
                           const float* partial, int nparts, float* amax_out,
                           float* scale_inv_out, hipStream_t stream, bool e5m2 = false);
// One step of delayed scaling from per-workgroup amax partials (E4M3 or E5M2
// largest finite value); history has len entries, newest first.
constexpr int kMaxHistoryLen = 4096;
hipError_t delayed_update_launch(const float* partial, int nparts, float* history, int len,
                                 float* scale, float* scale_inv, bool e5m2, hipStream_t stream);

}  // namespace tpmlp
