// Instantiations and launchers of the MFMA tile kernel (bf16 and e4m3).
#include <mutex>

#include "gemm_mfma.h"
#include "launch.h"

namespace tpmlp {

namespace {

template <bool IS_FP8, bool A_K, bool B_K, int EPI, bool COLSUM, int FMT = 0,
          int GROUP = GROUP_NONE>
hipError_t launch_one(const GemmArgs& g, const EpiArgs& e, hipStream_t s, int64_t nb = -1) {
  auto* k = &gemm_mfma_kernel<IS_FP8, A_K, B_K, EPI, bf16_t, COLSUM, FMT, GROUP>;
  // the LDS allowance is raised once per instantiation and device; call_once
  // makes that safe when several host threads launch at once (its result,
  // success or error, is kept)
  static std::once_flag once[64];
  static hipError_t attr_err[64];
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::call_once(once[dev], [&]() {
    attr_err[dev] = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                        hipFuncAttributeMaxDynamicSharedMemorySize, kSmemBytes);
  });
  if (attr_err[dev] != hipSuccess) return attr_err[dev];
  if (nb < 0) nb = (int64_t)g.tiles_m * g.tiles_n + g.tail_tiles;
  hipLaunchKernelGGL(k, dim3((unsigned)nb), dim3(kThreads), kSmemBytes, s, g, e);
  return hipGetLastError();
}

}  // namespace

int mfma_grid(Step step, GemmArgs& g) {
  const bool pair = (step == FC1_FWD_SWIGLU || step == FC1_FWD_SWIGLU_Q);
  g.tiles_m = (g.M + kBM - 1) / kBM;
  const int bn = pair ? kBN / 2 : kBN;
  g.tiles_n = (g.N + bn - 1) / bn;
  g.group_m = 8;
  if (g.M <= 0 || g.N <= 0) return 0;
  return g.tiles_m * g.tiles_n;
}

int64_t mfma_group_grid(Step step, int group, GemmArgs& g) {
  mfma_grid(step, g);  // tiles_n (and tiles_m of one group for GROUP_K)
  if (g.groups <= 0 || g.N <= 0) return 0;
  if (group == GROUP_M) {
    // at most ceil(rows / 256) + groups M-tiles over all groups
    if (g.rows <= 0) return 0;
    return ((int64_t)(g.rows + kBM - 1) / kBM + g.groups) * g.tiles_n;
  }
  if (g.M <= 0) return 0;
  return (int64_t)g.groups * g.tiles_m * g.tiles_n;
}

hipError_t mfma_group_launch(Step step, int group, const GemmArgs& g0, const EpiArgs& e,
                             hipStream_t s) {
  GemmArgs g = g0;
  const int64_t nb = mfma_group_grid(step, group, g);
  if (nb <= 0) return hipSuccess;
  if (group == GROUP_M) {
    switch (step) {
      case FC1_FWD_GELU:
        return launch_one<false, true, true, EPI_BIAS_GELU, false, 0, GROUP_M>(g, e, s, nb);
      case FC1_FWD_SWIGLU:
        return launch_one<false, true, true, EPI_SWIGLU, false, 0, GROUP_M>(g, e, s, nb);
      case FC2_FWD: return launch_one<false, true, true, EPI_STORE, false, 0, GROUP_M>(g, e, s, nb);
      case FC2_DGRAD_GELU:
        return launch_one<false, true, false, EPI_DGELU, false, 0, GROUP_M>(g, e, s, nb);
      case FC2_DGRAD_SWIGLU:
        return launch_one<false, true, false, EPI_DSWIGLU, false, 0, GROUP_M>(g, e, s, nb);
      case FC1_DGRAD:
        return launch_one<false, true, false, EPI_STORE, false, 0, GROUP_M>(g, e, s, nb);
      default: return hipErrorInvalidValue;
    }
  }
  if (group == GROUP_K) {
    switch (step) {
      case WGRAD: return launch_one<false, false, false, EPI_F32, false, 0, GROUP_K>(g, e, s, nb);
      case WGRAD_COLSUM:
        return launch_one<false, false, false, EPI_F32, true, 0, GROUP_K>(g, e, s, nb);
      default: return hipErrorInvalidValue;
    }
  }
  return hipErrorInvalidValue;
}

hipError_t mfma_split_launch(Step step, const GemmArgs& g, const EpiArgs& e, hipStream_t s) {
  if (g.k_splits < 2) return hipErrorInvalidValue;
  const int64_t nb = (int64_t)g.tiles_m * g.tiles_n * g.k_splits;
  switch (step) {
    case FC2_FWD:
    case QKV_FWD_BIAS: return launch_one<false, true, true, EPI_F32, false>(g, e, s, nb);
    case FC1_DGRAD: return launch_one<false, true, false, EPI_F32, false>(g, e, s, nb);
    case WGRAD: return launch_one<false, false, false, EPI_F32, false>(g, e, s, nb);
    case WGRAD_COLSUM: return launch_one<false, false, false, EPI_F32, true>(g, e, s, nb);
    default: return hipErrorInvalidValue;
  }
}

hipError_t mfma_launch(bool fp8, Step step, const GemmArgs& g, const EpiArgs& e, hipStream_t s) {
  if (fp8) {
    // forward: e4m3 x e4m3; backward: e5m2 gradient (A) x e4m3 (B)
    constexpr int kA5 = 1;
    switch (step) {
      case FC1_FWD_GELU: return launch_one<true, true, true, EPI_BIAS_GELU, false>(g, e, s);
      case FC1_FWD_GELU_Q: return launch_one<true, true, true, EPI_BIAS_GELU_Q, false>(g, e, s);
      case FC1_FWD_SWIGLU: return launch_one<true, true, true, EPI_SWIGLU, false>(g, e, s);
      case FC1_FWD_SWIGLU_Q: return launch_one<true, true, true, EPI_SWIGLU_Q, false>(g, e, s);
      case FC2_FWD: return launch_one<true, true, true, EPI_STORE, false>(g, e, s);
      case FC2_DGRAD_GELU_Q:
        return launch_one<true, true, false, EPI_DGELU_Q, false, kA5>(g, e, s);
      case FC2_DGRAD_SWIGLU_Q:
        return launch_one<true, true, false, EPI_DSWIGLU_Q, false, kA5>(g, e, s);
      case FC1_DGRAD: return launch_one<true, true, false, EPI_STORE, false, kA5>(g, e, s);
      case WGRAD: return launch_one<true, false, false, EPI_F32, false, kA5>(g, e, s);
      case WGRAD_COLSUM: return launch_one<true, false, false, EPI_F32, true, kA5>(g, e, s);
      case WGRAD_T: return launch_one<true, true, true, EPI_F32, false, kA5>(g, e, s);
      default: return hipErrorInvalidValue;
    }
  }
  switch (step) {
    case FC1_FWD_GELU: return launch_one<false, true, true, EPI_BIAS_GELU, false>(g, e, s);
    case FC1_FWD_SWIGLU: return launch_one<false, true, true, EPI_SWIGLU, false>(g, e, s);
    case FC2_FWD: return launch_one<false, true, true, EPI_STORE, false>(g, e, s);
    case FC2_DGRAD_GELU: return launch_one<false, true, false, EPI_DGELU, false>(g, e, s);
    case FC2_DGRAD_SWIGLU: return launch_one<false, true, false, EPI_DSWIGLU, false>(g, e, s);
    case FC1_DGRAD: return launch_one<false, true, false, EPI_STORE, false>(g, e, s);
    case WGRAD: return launch_one<false, false, false, EPI_F32, false>(g, e, s);
    case WGRAD_COLSUM: return launch_one<false, false, false, EPI_F32, true>(g, e, s);
    case QKV_FWD_BIAS: return launch_one<false, true, true, EPI_BIAS, false>(g, e, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tpmlp
