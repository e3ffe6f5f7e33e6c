// libtpmlp C ABI: argument validation, kernel selection and launch, and the
// kernel timing facility. The interface is documented in include/tpmlp.h.
#include <math.h>
#include <string.h>

#include <cmath>
#include <initializer_list>
#include <mutex>

#include <string>
#include <vector>

#include "../../include/tpmlp.h"
#include "launch.h"

using namespace tpmlp;

namespace {

thread_local std::string g_last_hip_error;

tpmlp_status hip_fail(hipError_t err) {
  g_last_hip_error = hipGetErrorString(err);
  return TPMLP_E_HIP;
}

// ---------------------------------------------------------------- timing
struct TimingRec {
  const char* name;
  hipEvent_t start, stop;
};
bool g_timing = false;
std::string g_filter;
std::vector<TimingRec> g_recs;
std::vector<hipEvent_t> g_pool;
std::vector<std::string> g_names_out;

hipError_t take_event(hipEvent_t* ev) {
  if (!g_pool.empty()) {
    *ev = g_pool.back();
    g_pool.pop_back();
    return hipSuccess;
  }
  return hipEventCreate(ev);
}

// Clock capture of the MFMA GEMM launches while the facility is enabled
// (every such launch, whatever the name filter selects for events): each
// workgroup writes (shader clock counter, real-time counter) at its start and
// end into 4 slots of this array (one range of workgroups per launch, handed
// out in launch order until the array is full). tpmlp_timing_collect turns
// them into each kernel's mean shader clock: the sum of its workgroups'
// cycles over the sum of their real-time ticks, at the counter's 100 MHz.
constexpr int kClockSlots = 131072;
__device__ __align__(256) unsigned long long clock_slots[4 * kClockSlots];
struct ClockRec {
  const char* name;
  int off, n;
};
unsigned long long* g_clk_dev = nullptr;  // the current device's array, while timing
int g_clk_used = 0;
std::vector<ClockRec> g_clk_recs;
std::vector<std::pair<std::string, double>> g_clk_mhz;  // from the last collect


// Points the launch's clock capture at the next free slots (or leaves it off).
void clock_attach(const char* name, GemmArgs& g, int64_t nb) {
  g.clk = nullptr;
  g.clk_slots = 0;
  if (!g_timing || !g_clk_dev || nb <= 0 || g_clk_used + nb > kClockSlots) return;
  g.clk = g_clk_dev + 4 * (int64_t)g_clk_used;
  g.clk_slots = (int)nb;
  g_clk_recs.push_back({name, g_clk_used, (int)nb});
  g_clk_used += (int)nb;
}

template <class F>
hipError_t timed(const char* name, hipStream_t s, F&& launch) {
  if (!g_timing || (!g_filter.empty() && strstr(name, g_filter.c_str()) == nullptr))
    return launch();
  TimingRec r{name, nullptr, nullptr};
  hipError_t err = take_event(&r.start);
  if (err == hipSuccess) err = take_event(&r.stop);
  if (err == hipSuccess) err = hipEventRecord(r.start, s);
  if (err != hipSuccess) return err;
  err = launch();
  if (err != hipSuccess) return err;
  err = hipEventRecord(r.stop, s);
  if (err != hipSuccess) return err;
  g_recs.push_back(r);
  return hipSuccess;
}

// ---------------------------------------------------------------- validation
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Row length bound for H, G*Fs and the attention widths: 256 rows of a
// K-major tile stay within one buffer resource's 2 GiB range.
constexpr int64_t kMaxDim = int64_t(1) << 21;
constexpr int64_t kMaxTokens = int64_t(1) << 30;

// Every product of a call launches at most ceil(T / 64) x ceil(widest / 64)
// workgroups (the fp32 kernel's 64 x 64 tiles; the MFMA kernel's are larger):
// tile ids must stay below 2^31.
bool grid_fits(int64_t tokens, int64_t widest) {
  return ((tokens + 63) / 64 + 1) * ((widest + 63) / 64 + 1) < (int64_t(1) << 31);
}

tpmlp_status check_desc(const tpmlp_desc* d) {
  if (!d) return TPMLP_E_NULL;
  if (d->reserved != 0) return TPMLP_E_DTYPE;
  if (d->dtype < TPMLP_F32 || d->dtype > TPMLP_E4M3) return TPMLP_E_DTYPE;
  if (d->act != TPMLP_ACT_GELU_TANH && d->act != TPMLP_ACT_SWIGLU) return TPMLP_E_DTYPE;
  if (d->has_bias != 0 && d->has_bias != 1) return TPMLP_E_DTYPE;
  if (d->tokens < 0 || d->hidden <= 0 || d->ffn_shard <= 0) return TPMLP_E_SHAPE;
  if (d->hidden % 16 != 0 || d->ffn_shard % 16 != 0) return TPMLP_E_SHAPE;
  const int64_t g = d->act == TPMLP_ACT_SWIGLU ? 2 : 1;
  if (d->hidden > kMaxDim || g * d->ffn_shard > kMaxDim || d->tokens > kMaxTokens)
    return TPMLP_E_SHAPE;
  if (!grid_fits(d->tokens, d->hidden > g * d->ffn_shard ? d->hidden : g * d->ffn_shard))
    return TPMLP_E_SHAPE;
  if (d->act == TPMLP_ACT_SWIGLU && d->has_bias) return TPMLP_E_UNSUPPORTED;
  return TPMLP_OK;
}

// Pointers that must be present and 16-byte aligned.
tpmlp_status check_ptrs(std::initializer_list<const void*> req) {
  for (const void* p : req)
    if (!p) return TPMLP_E_NULL;
  for (const void* p : req)
    if (!aligned16(p)) return TPMLP_E_ALIGN;
  return TPMLP_OK;
}

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// ---------------------------------------------------------------- split-K
// Splits of K for a bf16 product whose tile grid leaves CUs idle (1 = none).
// The estimate of s splits: rounds of tiles over the 256 CUs times one tile's
// share of K (at an assumed 4.7 TFLOP/s per CU), plus writing and reading the
// s fp32 partial planes (at an assumed 4 TB/s). The best s in 2..4 is taken
// if it saves at least 10% and every split keeps 8 stages or more.
int plan_splits(Kind kind, Step step, int64_t M, int64_t N, int64_t K) {
  if (kind != KIND_BF16) return 1;
  if (step != FC2_FWD && step != QKV_FWD_BIAS && step != FC1_DGRAD && step != WGRAD &&
      step != WGRAD_COLSUM)
    return 1;
  if (M <= 0 || N <= 0 || K <= 0) return 1;
  const double tiles = (double)((M + 255) / 256) * (double)((N + 255) / 256);
  const int64_t stages = (K + 63) / 64;
  auto est = [&](int sp) {
    const double rounds = std::ceil(tiles * sp / 256.0);
    const double t_tile = 2.0 * 256 * 256 * 64.0 * (double)((stages + sp - 1) / sp) / 4.7e12;
    const double t_red = sp > 1 ? 2.0 * sp * (double)M * (double)N * 4 / 4e12 : 0.0;
    return rounds * t_tile + t_red;
  };
  const double t1 = est(1);
  int best = 1;
  double tb = 0.9 * t1;
  for (int sp = 2; sp <= 4; ++sp) {
    if (stages < 8 * sp) break;
    const double t = est(sp);
    if (t < tb) {
      tb = t;
      best = sp;
    }
  }
  return best;
}
size_t split_bytes(int sp, int64_t M, int64_t N) {
  return sp > 1 ? align_up((size_t)sp * (size_t)M * (size_t)N * 4, 256) : 0;
}


// workgroups of the MFMA kernel for an M x N product (one per 256 x 256 tile)
int gemm_tiles(int64_t M, int64_t N) {
  GemmArgs g{};
  g.M = (int)M;
  g.N = (int)N;
  return mfma_grid(FC2_FWD, g);
}

// e4m3 forward: fc1's workgroups, one amax partial each (the gated fc1 runs
// 256 x 128 pair tiles)
int fp8_fc1_parts(const tpmlp_desc* d) {
  GemmArgs g{};
  g.M = (int)d->tokens;
  g.N = (int)d->ffn_shard;
  return mfma_grid(d->act == TPMLP_ACT_SWIGLU ? FC1_FWD_SWIGLU_Q : FC1_FWD_GELU_Q, g);
}
// e4m3 dgrad: fc2 dgrad's workgroups (M = T, N = Fs), one amax partial of dH each
int fp8_dgrad_parts(const tpmlp_desc* d) { return gemm_tiles(d->tokens, d->ffn_shard); }

// ---------------------------------------------------------------- partial last rounds
// A weight gradient whose tiles leave a last round of r workgroups (8 <= r
// <= 128) on the 256 compute units runs r rounded down to a multiple of 8 of
// its tiles as two workgroups each, one per half of the K stages, so that the
// last round fills the chip and takes half a tile's time. The halves meet in
// the workspace (kernel: GemmArgs::tail_tiles). Only for unsplit MFMA
// products without the fused column sum, of at least 16 stages.
constexpr int kTailCUs = 256;
int tail_plan(Kind kind, Step step, int64_t M, int64_t N, int64_t K) {
  if (kind == KIND_F32 || step != WGRAD) return 0;
  if (M <= 0 || N <= 0 || M > INT32_MAX || N > INT32_MAX) return 0;
  GemmArgs g{};
  g.M = (int)M;
  g.N = (int)N;
  const int tiles = mfma_grid(step, g);
  const int64_t stages = (K + (kind == KIND_E4M3 ? 127 : 63)) / (kind == KIND_E4M3 ? 128 : 64);
  if (stages < 16) return 0;
  const int r = tiles % kTailCUs;
  if (r < 8 || r > kTailCUs / 2) return 0;
  return r & ~7;
}
size_t tail_count_bytes(int tail) { return align_up((size_t)tail * 4, 256); }
// counters, then two 256 x 256 fp32 dumps per split tile
size_t tail_bytes(int tail) {
  return tail > 0 ? tail_count_bytes(tail) + (size_t)tail * 2 * 256 * 256 * 4 : 0;
}

// fc1 wgrad with bias: tile columns of dW1 = dH^T . x (N = H), each of which
// writes one row of db1 partial sums
int colsum_parts(const tpmlp_desc* d) {
  GemmArgs g{};
  g.M = (int)(d->act == TPMLP_ACT_SWIGLU ? 2 * d->ffn_shard : d->ffn_shard);
  g.N = (int)d->hidden;
  mfma_grid(WGRAD_COLSUM, g);
  return g.tiles_n;
}

// The MLP wgrad's split plans (fc2's dW2, fc1's dW1) and its workspace: the
// db1 partial rows of the column sums (sp1 * tiles_n of them), then one
// region for the partial planes of the larger split product or the halves of
// an unsplit product's partial last round (the products run one after the
// other).
struct WgradPlan {
  int sp2, sp1;
  int tail2, tail1;
  size_t colsum, planes;  // planes: the shared region
};
WgradPlan wgrad_plan(const tpmlp_desc* d, bool split_ok) {
  const Kind kind = d->dtype == TPMLP_F32 ? KIND_F32 : d->dtype == TPMLP_BF16 ? KIND_BF16 : KIND_E4M3;
  const int64_t gfs = (d->act == TPMLP_ACT_SWIGLU ? 2 : 1) * d->ffn_shard;
  WgradPlan p{1, 1, 0, 0, 0, 0};
  if (split_ok) {
    p.sp2 = plan_splits(kind, WGRAD, d->hidden, d->ffn_shard, d->tokens);
    p.sp1 = plan_splits(kind, d->has_bias ? WGRAD_COLSUM : WGRAD, gfs, d->hidden, d->tokens);
    if (p.sp2 < 2) p.tail2 = tail_plan(kind, WGRAD, d->hidden, d->ffn_shard, d->tokens);
    if (p.sp1 < 2 && !d->has_bias) p.tail1 = tail_plan(kind, WGRAD, gfs, d->hidden, d->tokens);
  }
  if (d->has_bias && kind != KIND_F32)
    p.colsum = align_up((size_t)p.sp1 * (size_t)colsum_parts(d) * (size_t)gfs * 4, 256);
  const size_t sizes[4] = {split_bytes(p.sp2, d->hidden, d->ffn_shard),
                           split_bytes(p.sp1, gfs, d->hidden), tail_bytes(p.tail2),
                           tail_bytes(p.tail1)};
  for (size_t v : sizes) p.planes = v > p.planes ? v : p.planes;
  return p;
}

// The recomputed activation a at the front of the recomputing weight-gradient
// call's workspace: [T][Fs] of bf16, fp32 or E4M3 codes.
size_t recompute_a_bytes(const tpmlp_desc* d) {
  const size_t es = d->dtype == TPMLP_F32 ? 4 : d->dtype == TPMLP_BF16 ? 2 : 1;
  return align_up((size_t)d->tokens * (size_t)d->ffn_shard * es, 256);
}

size_t workspace_bytes(const tpmlp_desc* d, int32_t call) {
  const bool fp8 = d->dtype == TPMLP_E4M3;
  if (call == TPMLP_CALL_WGRAD_RECOMPUTE)
    return recompute_a_bytes(d) + workspace_bytes(d, TPMLP_CALL_WGRAD);
  if (call == TPMLP_CALL_FWD && fp8) {
    // current scaling: bf16 a, then the partials; delayed scaling: partials only
    const size_t a_bytes = align_up((size_t)d->tokens * (size_t)d->ffn_shard * 2, 256);
    const size_t parts = align_up((size_t)fp8_fc1_parts(d) * 4 + 4, 256);
    return a_bytes + parts;
  }
  if (call == TPMLP_CALL_DGRAD && fp8) return align_up((size_t)fp8_dgrad_parts(d) * 4 + 4, 256);
  if (call == TPMLP_CALL_WGRAD) {
    const WgradPlan p = wgrad_plan(d, true);
    return p.colsum + p.planes;
  }
  return 0;
}
// The part of the workspace a call cannot run without (the rest only enables
// split-K).
size_t workspace_min_bytes(const tpmlp_desc* d, int32_t call) {
  if (call == TPMLP_CALL_WGRAD) return wgrad_plan(d, false).colsum;
  if (call == TPMLP_CALL_WGRAD_RECOMPUTE)
    return recompute_a_bytes(d) + workspace_min_bytes(d, TPMLP_CALL_WGRAD);
  return workspace_bytes(d, call);
}

// A delayed-scaling state: pointers present, length in range.
tpmlp_status check_history(const tpmlp_fp8_history* h) {
  if (!h || !h->amax_history || !h->scale || !h->scale_inv) return TPMLP_E_NULL;
  if (h->reserved != 0 || h->len < 1 || h->len > kMaxHistoryLen) return TPMLP_E_SHAPE;
  return TPMLP_OK;
}

tpmlp_status check_workspace(const tpmlp_desc* d, int32_t call, void* ws, size_t ws_bytes) {
  const size_t need = workspace_min_bytes(d, call);
  if (need == 0) return TPMLP_OK;
  if (!ws || ws_bytes < need) return TPMLP_E_WORKSPACE;
  if (!aligned16(ws)) return TPMLP_E_ALIGN;
  return TPMLP_OK;
}

// ---------------------------------------------------------------- GEMM step dispatch
// `label` names the launch for the timing facility (e.g. "fc1_fwd.bf16").
// `tail` > 0: that many tiles of a partial last round run as two half-K
// workgroups each, with tail_ws holding tail_bytes(tail) (see tail_plan).
hipError_t run_step(Kind kind, Step step, const char* label, GemmArgs g, const EpiArgs& e,
                    hipStream_t s, int tail = 0, void* tail_ws = nullptr) {
  const int nb = (kind == KIND_F32) ? f32_grid(step, g) : mfma_grid(step, g);
  if (nb == 0) return hipSuccess;
  if (kind != KIND_F32 && tail > 0) {
    g.tail_tiles = tail;
    g.tail_cnt = static_cast<int*>(tail_ws);
    g.tail_ws = reinterpret_cast<float*>(static_cast<char*>(tail_ws) + tail_count_bytes(tail));
  }
  if (kind != KIND_F32) clock_attach(label, g, (int64_t)nb + g.tail_tiles);
  return timed(label, s, [&]() {
    if (kind == KIND_F32) return f32_launch(step, g, e, s);
    if (g.tail_tiles > 0) {
      const hipError_t err = fill_zero_i32_launch(g.tail_cnt, g.tail_tiles, s);
      if (err != hipSuccess) return err;
    }
    return mfma_launch(kind == KIND_E4M3, step, g, e, s);
  });
}

// One product: split-K when `sp` > 1 (the caller checked that `part` holds
// the sp partial planes), else the plain kernel. The timing facility brackets
// the product and its reduce together under `label`. A fused column sum then
// writes sp * tiles_n partial rows.
hipError_t run_gemm(Kind kind, Step step, const char* label, GemmArgs g, const EpiArgs& e,
                    hipStream_t s, int sp, float* part, int tail = 0, void* tail_ws = nullptr) {
  if (sp < 2) return run_step(kind, step, label, g, e, s, tail, tail_ws);
  if (mfma_grid(step, g) == 0) return hipSuccess;
  g.k_splits = sp;
  g.split_stages = (int)(((g.K + 63) / 64 + sp - 1) / sp);
  // even, so that every split but the last can take the kernel's loop for
  // K-major operands without a per-lane K-range test
  g.split_stages += g.split_stages & 1;
  clock_attach(label, g, (int64_t)g.tiles_m * g.tiles_n * sp);
  EpiArgs ep = e;
  ep.out = part;
  ep.ldo = g.N;
  ep.accumulate = 0;
  const bool out_bf16 = step != WGRAD && step != WGRAD_COLSUM;
  return timed(label, s, [&]() {
    hipError_t err = mfma_split_launch(step, g, ep, s);
    if (err != hipSuccess) return err;
    return splitk_reduce_launch(part, sp, g.M, g.N, e.out, out_bf16,
                                step == QKV_FWD_BIAS ? e.bias : nullptr, e.accumulate, s);
  });
}

const char* label(Kind kind, int which) {
  // which: 0 fc1_fwd, 1 fc2_fwd, 2 fc2_dgrad, 3 fc1_dgrad, 4 fc2_wgrad, 5 fc1_wgrad
  static const char* names[3][6] = {
      {"fc1_fwd.f32", "fc2_fwd.f32", "fc2_dgrad.f32", "fc1_dgrad.f32", "fc2_wgrad.f32", "fc1_wgrad.f32"},
      {"fc1_fwd.bf16", "fc2_fwd.bf16", "fc2_dgrad.bf16", "fc1_dgrad.bf16", "fc2_wgrad.bf16",
       "fc1_wgrad.bf16"},
      {"fc1_fwd.e4m3", "fc2_fwd.e4m3", "fc2_dgrad.e4m3", "fc1_dgrad.e4m3", "fc2_wgrad.e4m3",
       "fc1_wgrad.e4m3"}};
  return names[kind][which];
}

// ---------------------------------------------------------------- attention
tpmlp_status check_attn_desc(const tpmlp_attn_desc* d) {
  if (!d) return TPMLP_E_NULL;
  if (d->reserved != 0) return TPMLP_E_DTYPE;
  if (d->dtype == TPMLP_E4M3) return TPMLP_E_UNSUPPORTED;
  if (d->dtype != TPMLP_F32 && d->dtype != TPMLP_BF16) return TPMLP_E_DTYPE;
  if (d->has_bias != 0 && d->has_bias != 1) return TPMLP_E_DTYPE;
  if (d->tokens < 0 || d->hidden <= 0 || d->q_heads <= 0 || d->kv_heads <= 0 ||
      d->head_dim <= 0)
    return TPMLP_E_SHAPE;
  if (d->hidden % 16 != 0 || d->head_dim % 16 != 0 || d->q_heads % d->kv_heads != 0)
    return TPMLP_E_SHAPE;
  const int64_t nqkv = ((int64_t)d->q_heads + 2 * (int64_t)d->kv_heads) * d->head_dim;
  if (d->hidden > kMaxDim || nqkv > kMaxDim || d->tokens > kMaxTokens) return TPMLP_E_SHAPE;
  if (!grid_fits(d->tokens, d->hidden > nqkv ? d->hidden : nqkv)) return TPMLP_E_SHAPE;
  return TPMLP_OK;
}
int64_t attn_nqkv(const tpmlp_attn_desc* d) {
  return ((int64_t)d->q_heads + 2 * (int64_t)d->kv_heads) * d->head_dim;
}
int64_t attn_d(const tpmlp_attn_desc* d) { return (int64_t)d->q_heads * d->head_dim; }
Kind attn_kind(const tpmlp_attn_desc* d) { return d->dtype == TPMLP_F32 ? KIND_F32 : KIND_BF16; }

// which: 0 qkv_fwd, 1 out_fwd, 2 out_dgrad, 3 out_wgrad, 4 qkv_dgrad, 5 qkv_wgrad, 6 dbqkv_reduce
const char* attn_label(Kind kind, int which) {
  static const char* names[2][7] = {
      {"qkv_fwd.f32", "out_fwd.f32", "out_dgrad.f32", "out_wgrad.f32", "qkv_dgrad.f32",
       "qkv_wgrad.f32", "dbqkv_reduce.f32"},
      {"qkv_fwd.bf16", "out_fwd.bf16", "out_dgrad.bf16", "out_wgrad.bf16", "qkv_dgrad.bf16",
       "qkv_wgrad.bf16", "dbqkv_reduce.bf16"}};
  return names[kind == KIND_F32 ? 0 : 1][which];
}

// qkv wgrad with bias on the MFMA kernel: one row of dbqkv partials per tile
// column of dWqkv = dqkv^T . x (N = H)
int attn_colsum_parts(const tpmlp_attn_desc* d) {
  GemmArgs g{};
  g.M = (int)attn_nqkv(d);
  g.N = (int)d->hidden;
  mfma_grid(WGRAD_COLSUM, g);
  return g.tiles_n;
}
// Split plans of the attention backward's products and the workspace each
// call needs: the qkv wgrad's dbqkv partial rows first, then partial planes.
struct AttnPlan {
  int sp_od, sp_ow, sp_qw;
  size_t colsum;  // qkv wgrad's dbqkv partial rows
};
AttnPlan attn_plan(const tpmlp_attn_desc* d, bool split_ok) {
  const Kind kind = attn_kind(d);
  AttnPlan p{1, 1, 1, 0};
  if (split_ok) {
    p.sp_od = plan_splits(kind, FC1_DGRAD, d->tokens, attn_d(d), d->hidden);
    p.sp_ow = plan_splits(kind, WGRAD, d->hidden, attn_d(d), d->tokens);
    p.sp_qw = plan_splits(kind, d->has_bias ? WGRAD_COLSUM : WGRAD, attn_nqkv(d), d->hidden,
                          d->tokens);
  }
  if (d->has_bias && kind != KIND_F32)
    p.colsum = align_up((size_t)p.sp_qw * (size_t)attn_colsum_parts(d) * (size_t)attn_nqkv(d) * 4,
                        256);
  return p;
}
// which: 0 out dgrad, 1 out wgrad, 2 qkv wgrad
size_t attn_call_bytes(const tpmlp_attn_desc* d, const AttnPlan& p, int which) {
  if (which == 0) return split_bytes(p.sp_od, d->tokens, attn_d(d));
  if (which == 1) return split_bytes(p.sp_ow, d->hidden, attn_d(d));
  return p.colsum + split_bytes(p.sp_qw, attn_nqkv(d), d->hidden);
}
size_t attn_workspace_bytes(const tpmlp_attn_desc* d) {
  const AttnPlan p = attn_plan(d, true);
  size_t m = 0;
  for (int w = 0; w < 3; ++w) {
    const size_t b = attn_call_bytes(d, p, w);
    if (b > m) m = b;
  }
  return m;
}
// the plan a call runs with: split-K if the workspace holds the full plan's
// bytes for this call, else none (which needs only the column-sum rows)
AttnPlan attn_plan_for(const tpmlp_attn_desc* d, int which, const void* ws, size_t ws_bytes) {
  const AttnPlan full = attn_plan(d, true);
  if (ws && ws_bytes >= attn_call_bytes(d, full, which)) return full;
  return attn_plan(d, false);
}

// ---------------------------------------------------------------- mixture of experts
constexpr int32_t kMaxExperts = 1024;

tpmlp_status check_moe_desc(const tpmlp_moe_desc* d) {
  if (!d) return TPMLP_E_NULL;
  if (d->reserved0 != 0 || d->reserved1 != 0) return TPMLP_E_DTYPE;
  if (d->dtype < TPMLP_F32 || d->dtype > TPMLP_E4M3) return TPMLP_E_DTYPE;
  if (d->act != TPMLP_ACT_GELU_TANH && d->act != TPMLP_ACT_SWIGLU) return TPMLP_E_DTYPE;
  if (d->has_bias != 0 && d->has_bias != 1) return TPMLP_E_DTYPE;
  if (d->tokens < 0 || d->hidden <= 0 || d->ffn_shard <= 0 || d->experts <= 0) return TPMLP_E_SHAPE;
  if (d->hidden % 16 != 0 || d->ffn_shard % 16 != 0 || d->experts > kMaxExperts)
    return TPMLP_E_SHAPE;
  const int64_t g = d->act == TPMLP_ACT_SWIGLU ? 2 : 1;
  if (d->hidden > kMaxDim || g * d->ffn_shard > kMaxDim || d->tokens > kMaxTokens)
    return TPMLP_E_SHAPE;
  // the grouped grid, (ceil(tokens / 256) + E) M-tiles by the widest N, fits one launch
  const int64_t widest = d->hidden > g * d->ffn_shard ? d->hidden : g * d->ffn_shard;
  if (((d->tokens + 255) / 256 + d->experts) * ((widest + 255) / 256) >= (int64_t(1) << 31))
    return TPMLP_E_SHAPE;
  if ((int64_t)d->experts * ((widest + 255) / 256) * ((widest + 255) / 256) >= (int64_t(1) << 31))
    return TPMLP_E_SHAPE;
  if (d->dtype != TPMLP_BF16) return TPMLP_E_UNSUPPORTED;
  if (d->act == TPMLP_ACT_SWIGLU && d->has_bias) return TPMLP_E_UNSUPPORTED;
  return TPMLP_OK;
}

const char* moe_label(int which) {
  static const char* names[7] = {"moe_fc1_fwd.bf16",   "moe_fc2_fwd.bf16",   "moe_fc2_dgrad.bf16",
                                 "moe_fc1_dgrad.bf16", "moe_fc2_wgrad.bf16", "moe_fc1_wgrad.bf16",
                                 "moe_db1_reduce.bf16"};
  return names[which];
}

// fc1 wgrad with bias: tile columns of each expert's dW1 (N = H); every
// expert writes that many rows of db1 partial sums
int moe_colsum_parts(const tpmlp_moe_desc* d) {
  GemmArgs g{};
  g.M = (int)((d->act == TPMLP_ACT_SWIGLU ? 2 : 1) * d->ffn_shard);
  g.N = (int)d->hidden;
  mfma_grid(WGRAD_COLSUM, g);
  return g.tiles_n;
}
size_t moe_workspace_bytes(const tpmlp_moe_desc* d) {
  if (!d->has_bias) return 0;
  const size_t gfs = (size_t)(d->act == TPMLP_ACT_SWIGLU ? 2 : 1) * (size_t)d->ffn_shard;
  return align_up((size_t)d->experts * (size_t)moe_colsum_parts(d) * gfs * 4, 256);
}

hipError_t run_group_step(Step step, int group, const char* label, const GemmArgs& g,
                          const EpiArgs& e, hipStream_t s) {
  GemmArgs gg = g;
  const int64_t nb = mfma_group_grid(step, group, gg);
  if (nb <= 0) return hipSuccess;
  GemmArgs ga = g;
  clock_attach(label, ga, nb);
  return timed(label, s, [&]() { return mfma_group_launch(step, group, ga, e, s); });
}

GemmArgs make_gemm(const void* A, int64_t lda, const void* B, int64_t ldb, int64_t M, int64_t N,
                   int64_t K, int64_t pair_off) {
  GemmArgs g{};
  g.A = A;
  g.B = B;
  g.lda = lda;
  g.ldb = ldb;
  g.M = (int)M;
  g.N = (int)N;
  g.K = (int)K;
  g.pair_off = (int)pair_off;
  return g;
}


// ---------------------------------------------------------------- weight gradients
// The weight-gradient call's checks that do not involve the workspace.
tpmlp_status check_wgrad(const tpmlp_desc* d, const void* dy, const void* x, const void* a_saved,
                         const void* dH, float* dW1, float* db1, float* dW2, int32_t accumulate,
                         const tpmlp_fp8_scales* fp8) {
  tpmlp_status st = check_desc(d);
  if (st != TPMLP_OK) return st;
  if (accumulate != 0 && accumulate != 1) return TPMLP_E_DTYPE;
  if ((st = check_ptrs({dy, x, a_saved, dH, dW1, dW2})) != TPMLP_OK) return st;
  if (d->has_bias && (st = check_ptrs({db1})) != TPMLP_OK) return st;
  const bool is_fp8 = d->dtype == TPMLP_E4M3;
  if (is_fp8 != (fp8 != nullptr)) return is_fp8 ? TPMLP_E_NULL : TPMLP_E_DTYPE;
  if (is_fp8 && (!fp8->dy_scale_inv || !fp8->x_scale_inv || !fp8->a_scale_inv ||
                 !fp8->dH_scale_inv))
    return TPMLP_E_NULL;
  return TPMLP_OK;
}

// dW2 = dy^T . a, dW1 = dH^T . x, db1; arguments already checked. The
// products are split along K where the workspace holds the full plan's bytes.
tpmlp_status run_wgrad(const tpmlp_desc* d, const void* dy, const void* x, const void* a_saved,
                       const void* dH, float* dW1, float* db1, float* dW2, int32_t accumulate,
                       const tpmlp_fp8_scales* fp8, void* ws, size_t ws_bytes, hipStream_t s) {
  const int64_t T = d->tokens, H = d->hidden, Fs = d->ffn_shard;
  if (T == 0 && accumulate) return TPMLP_OK;  // adding nothing
  const bool is_fp8 = d->dtype == TPMLP_E4M3;
  const bool swiglu = d->act == TPMLP_ACT_SWIGLU;
  const int64_t GFs = swiglu ? 2 * Fs : Fs;
  const Kind kind = d->dtype == TPMLP_F32 ? KIND_F32 : d->dtype == TPMLP_BF16 ? KIND_BF16 : KIND_E4M3;
  // split-K for grids that leave CUs idle, when the workspace has room for it
  const WgradPlan full = wgrad_plan(d, true);
  const WgradPlan p = (ws && ws_bytes >= full.colsum + full.planes) ? full : wgrad_plan(d, false);
  float* planes = reinterpret_cast<float*>(static_cast<char*>(ws) + p.colsum);
  // dW2 [H, Fs] = dy^T . a : A = dy as [K=T][M=H], B = a as [K=T][N=Fs]
  EpiArgs e1{};
  e1.out = dW2; e1.ldo = Fs; e1.accumulate = accumulate;
  if (is_fp8) { e1.scale_a = fp8->dy_scale_inv; e1.scale_b = fp8->a_scale_inv; }
  GemmArgs g1 = make_gemm(dy, H, a_saved, Fs, H, Fs, T, 0);
  hipError_t err = run_gemm(kind, WGRAD, label(kind, 4), g1, e1, s, p.sp2, planes, p.tail2, planes);
  if (err != hipSuccess) return hip_fail(err);
  // dW1 [GFs, H] = dH^T . x (+ db1 = column sums of dH). The fp32 kernel
  // writes db1 itself; the MFMA kernel writes per-tile-column partial sums
  // (per split and tile column) into the workspace, which a second pass adds
  // up into db1.
  const bool parts = d->has_bias && kind != KIND_F32;
  EpiArgs e2{};
  e2.out = dW1; e2.ldo = H; e2.accumulate = accumulate;
  e2.colsum = d->has_bias ? (parts ? static_cast<float*>(ws) : db1) : nullptr;
  if (is_fp8) { e2.scale_a = fp8->dH_scale_inv; e2.scale_b = fp8->x_scale_inv; }
  GemmArgs g2 = make_gemm(dH, GFs, x, H, GFs, H, T, 0);
  err = run_gemm(kind, d->has_bias ? WGRAD_COLSUM : WGRAD, label(kind, 5), g2, e2, s, p.sp1,
                 planes, p.tail1, planes);
  if (err != hipSuccess) return hip_fail(err);
  if (parts) {
    err = timed(is_fp8 ? "db1_reduce.e4m3" : "db1_reduce.bf16", s, [&]() {
      return colsum_reduce_launch(static_cast<const float*>(ws), p.sp1 * colsum_parts(d),
                                  (int)GFs, db1, accumulate, s);
    });
    if (err != hipSuccess) return hip_fail(err);
  }
  return TPMLP_OK;
}

// ---------------------------------------------------------------- fixed scratch
// Device memory of the allocation-free weight-gradient call: a fixed array
// that every GPU the library runs on holds until the process ends. In host
// code the array's name is a stand-in, not a device address, so the address
// of each device's copy is looked up once per device, with that device
// current, and kept; kernels and copies get that address. Every such call on
// one GPU shares the array, so calls that overlap on one GPU race.
constexpr size_t kScratchBytes = TPMLP_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

hipError_t scratch_address(void** out) {
  int dev = 0;
  const hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev]() {
    g_scratch_err[dev] = hipGetSymbolAddress(&g_scratch_ptr[dev], HIP_SYMBOL(scratch));
  });
  if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

const char* tpmlp_strerror(tpmlp_status s) {
  switch (s) {
    case TPMLP_OK: return "success";
    case TPMLP_E_NULL: return "a required pointer is NULL";
    case TPMLP_E_SHAPE:
      return "invalid sizes (T >= 0; H, Fs, head size > 0 and multiples of 16; kv heads divide "
             "query heads; within limits)";
    case TPMLP_E_DTYPE: return "unknown dtype, activation or flag value";
    case TPMLP_E_ALIGN: return "a pointer is not 16-byte aligned";
    case TPMLP_E_UNSUPPORTED:
      return "combination not provided (SwiGLU bias, E4M3 attention projections, expert MLPs "
             "other than BF16)";
    case TPMLP_E_WORKSPACE: return "workspace missing or too small";
    case TPMLP_E_HIP: return "HIP runtime error while enqueuing (see tpmlp_last_hip_error)";
    case TPMLP_E_SCRATCH:
      return "problem too large for the fixed scratch of the allocation-free call "
             "(TPMLP_SCRATCH_BYTES)";
  }
  return "unknown status";
}

int32_t tpmlp_abi_version(void) { return TPMLP_ABI_VERSION; }

const char* tpmlp_last_hip_error(void) { return g_last_hip_error.c_str(); }

size_t tpmlp_workspace_size(const tpmlp_desc* desc, int32_t call) {
  if (check_desc(desc) != TPMLP_OK) return 0;
  if (call < TPMLP_CALL_FWD || call > TPMLP_CALL_WGRAD_RECOMPUTE) return 0;
  return workspace_bytes(desc, call);
}

tpmlp_status tpmlp_fwd(const tpmlp_desc* d, const void* x, const void* W1, const void* b1,
                       const void* W2, void* y, void* h_saved, void* a_saved,
                       const tpmlp_fp8_scales* fp8, void* ws, size_t ws_bytes,
                       hipStream_t s) {
  tpmlp_status st = check_desc(d);
  if (st != TPMLP_OK) return st;
  if ((st = check_ptrs({x, W1, W2, y, a_saved})) != TPMLP_OK) return st;
  if (d->has_bias && (st = check_ptrs({b1})) != TPMLP_OK) return st;
  if (h_saved && !aligned16(h_saved)) return TPMLP_E_ALIGN;
  const bool is_fp8 = d->dtype == TPMLP_E4M3;
  if (is_fp8 != (fp8 != nullptr)) return is_fp8 ? TPMLP_E_NULL : TPMLP_E_DTYPE;
  const bool delayed = is_fp8 && fp8->a_history != nullptr;
  if (is_fp8 && (!fp8->x_scale_inv || !fp8->w1_scale_inv || !fp8->w2_scale_inv))
    return TPMLP_E_NULL;
  if (is_fp8 && !delayed && (!fp8->a_amax || !fp8->a_scale_inv)) return TPMLP_E_NULL;
  if (delayed && (st = check_history(fp8->a_history)) != TPMLP_OK) return st;
  if ((st = check_workspace(d, TPMLP_CALL_FWD, ws, ws_bytes)) != TPMLP_OK) return st;

  const int64_t T = d->tokens, H = d->hidden, Fs = d->ffn_shard;
  const bool swiglu = d->act == TPMLP_ACT_SWIGLU;
  const int64_t GFs = swiglu ? 2 * Fs : Fs;
  const Kind kind = d->dtype == TPMLP_F32 ? KIND_F32 : d->dtype == TPMLP_BF16 ? KIND_BF16 : KIND_E4M3;
  hipError_t err;

  if (!is_fp8) {
    if (T == 0) return TPMLP_OK;
    EpiArgs e1{};
    e1.out = a_saved; e1.ldo = Fs;
    e1.out2 = h_saved; e1.ldo2 = GFs;
    e1.bias = d->has_bias ? b1 : nullptr;
    GemmArgs g1 = make_gemm(x, H, W1, H, T, Fs, H, Fs);
    err = run_step(kind, swiglu ? FC1_FWD_SWIGLU : FC1_FWD_GELU, label(kind, 0), g1, e1, s);
    if (err != hipSuccess) return hip_fail(err);
    EpiArgs e2{};
    e2.out = y; e2.ldo = H;
    GemmArgs g2 = make_gemm(a_saved, Fs, W2, Fs, T, H, Fs, 0);
    err = run_step(kind, FC2_FWD, label(kind, 1), g2, e2, s);
    if (err != hipSuccess) return hip_fail(err);
    return TPMLP_OK;
  }

  if (delayed) {
    // e4m3, delayed scaling: fc1 quantises a at a_history->scale in its
    // epilogue (+ per-workgroup amax) -> history update -> fc2
    // (no tokens: no products; the call still enters an amax of 0 and rolls
    // the history, one entry per call)
    const tpmlp_fp8_history* ah = fp8->a_history;
    float* parts = static_cast<float*>(ws);
    const int nparts = T > 0 ? fp8_fc1_parts(d) : 0;
    if (T > 0) {
      EpiArgs e1{};
      e1.out = a_saved; e1.ldo = Fs;
      e1.out2 = h_saved; e1.ldo2 = GFs;
      e1.bias = d->has_bias ? b1 : nullptr;
      e1.scale_a = fp8->x_scale_inv; e1.scale_b = fp8->w1_scale_inv;
      e1.q_scale = ah->scale;
      e1.amax_part = parts;
      GemmArgs g1 = make_gemm(x, H, W1, H, T, Fs, H, Fs);
      err = run_step(kind, swiglu ? FC1_FWD_SWIGLU_Q : FC1_FWD_GELU_Q, label(kind, 0), g1, e1, s);
      if (err != hipSuccess) return hip_fail(err);
    }
    err = timed("a_scale_update.e4m3", s, [&]() {
      return delayed_update_launch(parts, nparts, ah->amax_history, ah->len, ah->scale,
                                   ah->scale_inv, false, s);
    });
    if (err != hipSuccess) return hip_fail(err);
    if (T == 0) return TPMLP_OK;
    EpiArgs e2{};
    e2.out = y; e2.ldo = H;
    e2.scale_a = ah->scale_inv; e2.scale_b = fp8->w2_scale_inv;
    GemmArgs g2 = make_gemm(a_saved, Fs, W2, Fs, T, H, Fs, 0);
    err = run_step(kind, FC2_FWD, label(kind, 1), g2, e2, s);
    if (err != hipSuccess) return hip_fail(err);
    return TPMLP_OK;
  }

  // e4m3, current scaling: fc1 (bf16 a + per-workgroup amax) -> quantise a -> fc2
  char* wsb = static_cast<char*>(ws);
  void* a_bf16 = wsb;
  float* parts = reinterpret_cast<float*>(wsb + align_up((size_t)T * (size_t)Fs * 2, 256));
  const int nparts = fp8_fc1_parts(d);
  if (T > 0) {
    EpiArgs e1{};
    e1.out = a_bf16; e1.ldo = Fs;
    e1.out2 = h_saved; e1.ldo2 = GFs;
    e1.bias = d->has_bias ? b1 : nullptr;
    e1.scale_a = fp8->x_scale_inv; e1.scale_b = fp8->w1_scale_inv;
    e1.amax_part = parts;
    GemmArgs g1 = make_gemm(x, H, W1, H, T, Fs, H, Fs);
    err = run_step(kind, swiglu ? FC1_FWD_SWIGLU : FC1_FWD_GELU, label(kind, 0), g1, e1, s);
    if (err != hipSuccess) return hip_fail(err);
  }
  err = timed("quantize_a.e4m3", s, [&]() {
    return quantize_launch(true, a_bf16, T * Fs, static_cast<uint8_t*>(a_saved), parts, nparts,
                           fp8->a_amax, fp8->a_scale_inv, s);
  });
  if (err != hipSuccess) return hip_fail(err);
  if (T > 0) {
    EpiArgs e2{};
    e2.out = y; e2.ldo = H;
    e2.scale_a = fp8->a_scale_inv; e2.scale_b = fp8->w2_scale_inv;
    GemmArgs g2 = make_gemm(a_saved, Fs, W2, Fs, T, H, Fs, 0);
    err = run_step(kind, FC2_FWD, label(kind, 1), g2, e2, s);
    if (err != hipSuccess) return hip_fail(err);
  }
  return TPMLP_OK;
}

tpmlp_status tpmlp_bwd_dgrad(const tpmlp_desc* d, const void* dy, const void* W1,
                             const void* W2, const void* h_saved, void* dH, void* dx,
                             const tpmlp_fp8_scales* fp8, void* ws, size_t ws_bytes,
                             hipStream_t s) {
  tpmlp_status st = check_desc(d);
  if (st != TPMLP_OK) return st;
  if ((st = check_ptrs({dy, W1, W2, h_saved, dH, dx})) != TPMLP_OK) return st;
  const bool is_fp8 = d->dtype == TPMLP_E4M3;
  if (is_fp8 != (fp8 != nullptr)) return is_fp8 ? TPMLP_E_NULL : TPMLP_E_DTYPE;
  if (is_fp8) {
    if (!fp8->dy_scale_inv || !fp8->w1_scale_inv || !fp8->w2_scale_inv) return TPMLP_E_NULL;
    if ((st = check_history(fp8->dH_history)) != TPMLP_OK) return st;
  }
  if ((st = check_workspace(d, TPMLP_CALL_DGRAD, ws, ws_bytes)) != TPMLP_OK) return st;
  const int64_t T = d->tokens, H = d->hidden, Fs = d->ffn_shard;
  if (T == 0) {
    // no products; with FP8 the call still enters an amax of 0 into dH's history
    if (!is_fp8) return TPMLP_OK;
    const tpmlp_fp8_history* hh = fp8->dH_history;
    hipError_t err = timed("dH_scale_update.e4m3", s, [&]() {
      return delayed_update_launch(static_cast<float*>(ws), 0, hh->amax_history, hh->len,
                                   hh->scale, hh->scale_inv, true, s);
    });
    return err == hipSuccess ? TPMLP_OK : hip_fail(err);
  }
  const bool swiglu = d->act == TPMLP_ACT_SWIGLU;
  const int64_t GFs = swiglu ? 2 * Fs : Fs;
  const Kind kind = d->dtype == TPMLP_F32 ? KIND_F32 : d->dtype == TPMLP_BF16 ? KIND_BF16 : KIND_E4M3;
  hipError_t err;
  // fc2 dgrad: dA = dy . W2 (W2 [H, Fs] read as [K=H][N=Fs]), activation derivative fused
  EpiArgs e1{};
  e1.out = dH; e1.ldo = GFs;
  e1.aux = h_saved; e1.ldaux = GFs;
  GemmArgs g1 = make_gemm(dy, H, W2, Fs, T, Fs, H, Fs);
  if (!is_fp8) {
    err = run_step(kind, swiglu ? FC2_DGRAD_SWIGLU : FC2_DGRAD_GELU, label(kind, 2), g1, e1, s);
    if (err != hipSuccess) return hip_fail(err);
  } else {
    // dH quantised to e5m2 at dH_history->scale in the epilogue, then the
    // history update (which also writes the factor fc1 dgrad dequantises with)
    const tpmlp_fp8_history* hh = fp8->dH_history;
    float* parts = static_cast<float*>(ws);
    e1.scale_a = fp8->dy_scale_inv; e1.scale_b = fp8->w2_scale_inv;
    e1.q_scale = hh->scale;
    e1.amax_part = parts;
    err = run_step(kind, swiglu ? FC2_DGRAD_SWIGLU_Q : FC2_DGRAD_GELU_Q, label(kind, 2), g1, e1, s);
    if (err != hipSuccess) return hip_fail(err);
    err = timed("dH_scale_update.e4m3", s, [&]() {
      return delayed_update_launch(parts, fp8_dgrad_parts(d), hh->amax_history, hh->len,
                                   hh->scale, hh->scale_inv, true, s);
    });
    if (err != hipSuccess) return hip_fail(err);
  }
  // fc1 dgrad: dx = dH . W1 (W1 [GFs, H] read as [K=GFs][N=H])
  EpiArgs e2{};
  e2.out = dx; e2.ldo = H;
  if (is_fp8) { e2.scale_a = fp8->dH_history->scale_inv; e2.scale_b = fp8->w1_scale_inv; }
  GemmArgs g2 = make_gemm(dH, GFs, W1, H, T, H, GFs, 0);
  err = run_step(kind, FC1_DGRAD, label(kind, 3), g2, e2, s);
  if (err != hipSuccess) return hip_fail(err);
  return TPMLP_OK;
}

tpmlp_status tpmlp_bwd_wgrad(const tpmlp_desc* d, const void* dy, const void* x,
                             const void* a_saved, const void* dH, float* dW1, float* db1,
                             float* dW2, int32_t accumulate, const tpmlp_fp8_scales* fp8,
                             void* ws, size_t ws_bytes, hipStream_t s) {
  tpmlp_status st = check_wgrad(d, dy, x, a_saved, dH, dW1, db1, dW2, accumulate, fp8);
  if (st != TPMLP_OK) return st;
  if ((st = check_workspace(d, TPMLP_CALL_WGRAD, ws, ws_bytes)) != TPMLP_OK) return st;
  return run_wgrad(d, dy, x, a_saved, dH, dW1, db1, dW2, accumulate, fp8, ws, ws_bytes, s);
}

tpmlp_status tpmlp_bwd_wgrad_recompute(const tpmlp_desc* d, const void* dy, const void* x,
                                       const void* h_saved, const void* dH, float* dW1,
                                       float* db1, float* dW2, int32_t accumulate,
                                       const tpmlp_fp8_scales* fp8, void* ws, size_t ws_bytes,
                                       hipStream_t s) {
  tpmlp_status st = check_wgrad(d, dy, x, h_saved, dH, dW1, db1, dW2, accumulate, fp8);
  if (st != TPMLP_OK) return st;
  if ((st = check_workspace(d, TPMLP_CALL_WGRAD_RECOMPUTE, ws, ws_bytes)) != TPMLP_OK) return st;
  // a = act(h) into the front of the workspace; the weight gradients use the rest
  const size_t ab = recompute_a_bytes(d);
  const Kind kind = d->dtype == TPMLP_F32 ? KIND_F32 : d->dtype == TPMLP_BF16 ? KIND_BF16 : KIND_E4M3;
  const hipError_t err = timed(d->dtype == TPMLP_F32 ? "a_recompute.f32"
                               : d->dtype == TPMLP_BF16 ? "a_recompute.bf16" : "a_recompute.e4m3",
                               s, [&]() {
    return act_recompute_launch(kind, d->act == TPMLP_ACT_SWIGLU, h_saved, d->tokens,
                                d->ffn_shard, ws, kind == KIND_E4M3 ? fp8->a_scale_inv : nullptr,
                                s);
  });
  if (err != hipSuccess) return hip_fail(err);
  return run_wgrad(d, dy, x, ws, dH, dW1, db1, dW2, accumulate, fp8,
                   static_cast<char*>(ws) + ab, ws_bytes - ab, s);
}

// Row stride of a token-contiguous copy: T rounded up to 16 bytes.
int64_t token_ld(int64_t T) { return (T + 15) / 16 * 16; }
constexpr int64_t kMaxTokenLdT = (int64_t(1) << 23) - 256;

tpmlp_status tpmlp_transpose_u8(const void* src, int64_t rows, int64_t cols, void* dst,
                                hipStream_t s) {
  if (rows < 0 || cols < 0 || cols % 16 != 0 || rows > kMaxTokens || cols > kMaxDim)
    return TPMLP_E_SHAPE;
  if (rows == 0 || cols == 0) return TPMLP_OK;
  tpmlp_status st = check_ptrs({src, dst});
  if (st != TPMLP_OK) return st;
  const hipError_t err = timed("transpose_u8", s, [&]() {
    return transpose_u8_launch(src, rows, cols, dst, token_ld(rows), s);
  });
  return err == hipSuccess ? TPMLP_OK : hip_fail(err);
}

tpmlp_status tpmlp_bwd_wgrad_t(const tpmlp_desc* d, const void* dy_t, const void* x_t,
                               const void* a_t, const void* dH_t, float* dW1, float* db1,
                               float* dW2, int32_t accumulate, const tpmlp_fp8_scales* fp8,
                               hipStream_t s) {
  tpmlp_status st = check_wgrad(d, dy_t, x_t, a_t, dH_t, dW1, db1, dW2, accumulate, fp8);
  if (st != TPMLP_OK) return st;
  if (d->dtype != TPMLP_E4M3) return TPMLP_E_UNSUPPORTED;
  const int64_t T = d->tokens, H = d->hidden, Fs = d->ffn_shard;
  const int64_t GFs = d->act == TPMLP_ACT_SWIGLU ? 2 * Fs : Fs;
  // a 256-row tile of a token-contiguous operand is addressed with 32-bit
  // offsets from its first row: 256 rows of Tp bytes must stay below 2^31
  if (token_ld(T) > kMaxTokenLdT) return TPMLP_E_SHAPE;
  hipError_t err;
  // no tokens: accumulating adds nothing; otherwise the products of K = 0
  // write zeros (every operand range empty) and db1 sums nothing
  if (T == 0 && accumulate) return TPMLP_OK;
  const int64_t ld = token_ld(T);
  // dW2 [H, Fs] = dy^T . a: A = dy_t [M=H][K=T], B = a_t [N=Fs][K=T], both K-major
  EpiArgs e1{};
  e1.out = dW2; e1.ldo = Fs; e1.accumulate = accumulate;
  e1.scale_a = fp8->dy_scale_inv; e1.scale_b = fp8->a_scale_inv;
  GemmArgs g1 = make_gemm(dy_t, ld, a_t, ld, H, Fs, T, 0);
  err = run_step(KIND_E4M3, WGRAD_T, label(KIND_E4M3, 4), g1, e1, s);
  if (err != hipSuccess) return hip_fail(err);
  // dW1 [GFs, H] = dH^T . x: A = dH_t [M=GFs][K=T], B = x_t [N=H][K=T]
  EpiArgs e2{};
  e2.out = dW1; e2.ldo = H; e2.accumulate = accumulate;
  e2.scale_a = fp8->dH_scale_inv; e2.scale_b = fp8->x_scale_inv;
  GemmArgs g2 = make_gemm(dH_t, ld, x_t, ld, GFs, H, T, 0);
  err = run_step(KIND_E4M3, WGRAD_T, label(KIND_E4M3, 5), g2, e2, s);
  if (err != hipSuccess) return hip_fail(err);
  if (d->has_bias) {
    // db1 = the rows of dH_t summed, dequantised
    err = timed("db1_rowsum.e4m3", s, [&]() {
      return rowsum_e5m2_launch(dH_t, GFs, T, ld, fp8->dH_scale_inv, db1, accumulate, s);
    });
    if (err != hipSuccess) return hip_fail(err);
  }
  return TPMLP_OK;
}

tpmlp_status tpmlp_bwd_wgrad_noalloc(const tpmlp_desc* d, const void* dy, const void* x,
                                     const void* a_saved, const void* dH, float* dW1,
                                     float* db1, float* dW2, int32_t accumulate,
                                     const tpmlp_fp8_scales* fp8, hipStream_t s) {
  tpmlp_status st = check_wgrad(d, dy, x, a_saved, dH, dW1, db1, dW2, accumulate, fp8);
  if (st != TPMLP_OK) return st;
  // the part of the workspace the call cannot run without (the db1 partial
  // sums); split-K is left out, so nothing else is needed
  const size_t need = workspace_min_bytes(d, TPMLP_CALL_WGRAD);
  if (need > kScratchBytes) return TPMLP_E_SCRATCH;
  void* ws = nullptr;
  if (need > 0) {
    const hipError_t err = scratch_address(&ws);
    if (err != hipSuccess) return hip_fail(err);
  }
  return run_wgrad(d, dy, x, a_saved, dH, dW1, db1, dW2, accumulate, fp8, ws, need, s);
}

// ---------------------------------------------------------------- attention
size_t tpmlp_attn_workspace_size(const tpmlp_attn_desc* d) {
  if (check_attn_desc(d) != TPMLP_OK) return 0;
  return attn_workspace_bytes(d);
}

tpmlp_status tpmlp_attn_qkv_fwd(const tpmlp_attn_desc* d, const void* x, const void* Wqkv,
                                const void* bqkv, void* qkv, hipStream_t s) {
  tpmlp_status st = check_attn_desc(d);
  if (st != TPMLP_OK) return st;
  if ((st = check_ptrs({x, Wqkv, qkv})) != TPMLP_OK) return st;
  if (d->has_bias && (st = check_ptrs({bqkv})) != TPMLP_OK) return st;
  const int64_t T = d->tokens, H = d->hidden, N = attn_nqkv(d);
  if (T == 0) return TPMLP_OK;
  const Kind kind = attn_kind(d);
  EpiArgs e{};
  e.out = qkv; e.ldo = N;
  e.bias = d->has_bias ? bqkv : nullptr;
  GemmArgs g = make_gemm(x, H, Wqkv, H, T, N, H, 0);
  // without a bias the plain store epilogue serves
  hipError_t err = run_step(kind, d->has_bias ? QKV_FWD_BIAS : FC2_FWD, attn_label(kind, 0), g,
                            e, s);
  return err == hipSuccess ? TPMLP_OK : hip_fail(err);
}

tpmlp_status tpmlp_attn_out_fwd(const tpmlp_attn_desc* d, const void* ctx, const void* Wo,
                                void* y, hipStream_t s) {
  tpmlp_status st = check_attn_desc(d);
  if (st != TPMLP_OK) return st;
  if ((st = check_ptrs({ctx, Wo, y})) != TPMLP_OK) return st;
  const int64_t T = d->tokens, H = d->hidden, D = attn_d(d);
  if (T == 0) return TPMLP_OK;
  const Kind kind = attn_kind(d);
  EpiArgs e{};
  e.out = y; e.ldo = H;
  GemmArgs g = make_gemm(ctx, D, Wo, D, T, H, D, 0);
  hipError_t err = run_step(kind, FC2_FWD, attn_label(kind, 1), g, e, s);
  return err == hipSuccess ? TPMLP_OK : hip_fail(err);
}

tpmlp_status tpmlp_attn_out_bwd_dgrad(const tpmlp_attn_desc* d, const void* dy, const void* Wo,
                                      void* dctx, void* ws, size_t ws_bytes, hipStream_t s) {
  tpmlp_status st = check_attn_desc(d);
  if (st != TPMLP_OK) return st;
  if ((st = check_ptrs({dy, Wo, dctx})) != TPMLP_OK) return st;
  if (ws && !aligned16(ws)) return TPMLP_E_ALIGN;
  const int64_t T = d->tokens, H = d->hidden, D = attn_d(d);
  if (T == 0) return TPMLP_OK;
  const Kind kind = attn_kind(d);
  const AttnPlan p = attn_plan_for(d, 0, ws, ws_bytes);
  // dctx = dy . Wo: A = dy [T, H] K-major, B = Wo [H, D] read as [K=H][N=D]
  EpiArgs e{};
  e.out = dctx; e.ldo = D;
  GemmArgs g = make_gemm(dy, H, Wo, D, T, D, H, 0);
  hipError_t err = run_gemm(kind, FC1_DGRAD, attn_label(kind, 2), g, e, s, p.sp_od,
                            static_cast<float*>(ws));
  return err == hipSuccess ? TPMLP_OK : hip_fail(err);
}

tpmlp_status tpmlp_attn_out_bwd_wgrad(const tpmlp_attn_desc* d, const void* dy, const void* ctx,
                                      float* dWo, int32_t accumulate, void* ws, size_t ws_bytes,
                                      hipStream_t s) {
  tpmlp_status st = check_attn_desc(d);
  if (st != TPMLP_OK) return st;
  if (accumulate != 0 && accumulate != 1) return TPMLP_E_DTYPE;
  if ((st = check_ptrs({dy, ctx, dWo})) != TPMLP_OK) return st;
  if (ws && !aligned16(ws)) return TPMLP_E_ALIGN;
  const int64_t T = d->tokens, H = d->hidden, D = attn_d(d);
  if (T == 0 && accumulate) return TPMLP_OK;  // adding nothing
  const Kind kind = attn_kind(d);
  const AttnPlan p = attn_plan_for(d, 1, ws, ws_bytes);
  // dWo [H, D] = dy^T . ctx: A = dy as [K=T][M=H], B = ctx as [K=T][N=D]
  EpiArgs e{};
  e.out = dWo; e.ldo = D; e.accumulate = accumulate;
  GemmArgs g = make_gemm(dy, H, ctx, D, H, D, T, 0);
  hipError_t err = run_gemm(kind, WGRAD, attn_label(kind, 3), g, e, s, p.sp_ow,
                            static_cast<float*>(ws));
  return err == hipSuccess ? TPMLP_OK : hip_fail(err);
}

tpmlp_status tpmlp_attn_qkv_bwd_dgrad(const tpmlp_attn_desc* d, const void* dqkv,
                                      const void* Wqkv, void* dx, hipStream_t s) {
  tpmlp_status st = check_attn_desc(d);
  if (st != TPMLP_OK) return st;
  if ((st = check_ptrs({dqkv, Wqkv, dx})) != TPMLP_OK) return st;
  const int64_t T = d->tokens, H = d->hidden, N = attn_nqkv(d);
  if (T == 0) return TPMLP_OK;
  const Kind kind = attn_kind(d);
  // dx = dqkv . Wqkv: A = dqkv [T, Nqkv] K-major, B = Wqkv [Nqkv, H] read as [K=Nqkv][N=H]
  EpiArgs e{};
  e.out = dx; e.ldo = H;
  GemmArgs g = make_gemm(dqkv, N, Wqkv, H, T, H, N, 0);
  hipError_t err = run_step(kind, FC1_DGRAD, attn_label(kind, 4), g, e, s);
  return err == hipSuccess ? TPMLP_OK : hip_fail(err);
}

tpmlp_status tpmlp_attn_qkv_bwd_wgrad(const tpmlp_attn_desc* d, const void* dqkv, const void* x,
                                      float* dWqkv, float* dbqkv, int32_t accumulate, void* ws,
                                      size_t ws_bytes, hipStream_t s) {
  tpmlp_status st = check_attn_desc(d);
  if (st != TPMLP_OK) return st;
  if (accumulate != 0 && accumulate != 1) return TPMLP_E_DTYPE;
  if ((st = check_ptrs({dqkv, x, dWqkv})) != TPMLP_OK) return st;
  if (d->has_bias && (st = check_ptrs({dbqkv})) != TPMLP_OK) return st;
  const size_t need = attn_plan(d, false).colsum;
  if (need && (!ws || ws_bytes < need)) return TPMLP_E_WORKSPACE;
  if (ws && !aligned16(ws)) return TPMLP_E_ALIGN;
  const int64_t T = d->tokens, H = d->hidden, N = attn_nqkv(d);
  if (T == 0 && accumulate) return TPMLP_OK;
  const Kind kind = attn_kind(d);
  const AttnPlan p = attn_plan_for(d, 2, ws, ws_bytes);
  float* planes = reinterpret_cast<float*>(static_cast<char*>(ws) + p.colsum);
  // dWqkv [Nqkv, H] = dqkv^T . x (+ dbqkv = column sums of dqkv), as fc1's wgrad
  const bool parts = d->has_bias && kind != KIND_F32;
  EpiArgs e{};
  e.out = dWqkv; e.ldo = H; e.accumulate = accumulate;
  e.colsum = d->has_bias ? (parts ? static_cast<float*>(ws) : dbqkv) : nullptr;
  GemmArgs g = make_gemm(dqkv, N, x, H, N, H, T, 0);
  hipError_t err = run_gemm(kind, d->has_bias ? WGRAD_COLSUM : WGRAD, attn_label(kind, 5), g, e,
                            s, p.sp_qw, planes);
  if (err != hipSuccess) return hip_fail(err);
  if (parts) {
    err = timed(attn_label(kind, 6), s, [&]() {
      return colsum_reduce_launch(static_cast<const float*>(ws), p.sp_qw * attn_colsum_parts(d),
                                  (int)N, dbqkv, accumulate, s);
    });
    if (err != hipSuccess) return hip_fail(err);
  }
  return TPMLP_OK;
}

// ---------------------------------------------------------------- mixture of experts
size_t tpmlp_moe_workspace_size(const tpmlp_moe_desc* d) {
  if (check_moe_desc(d) != TPMLP_OK) return 0;
  return moe_workspace_bytes(d);
}

namespace {
void set_groups(GemmArgs& g, const tpmlp_moe_desc* d, const int32_t* counts) {
  g.counts = counts;
  g.groups = d->experts;
  g.rows = (int)d->tokens;
}
}  // namespace

tpmlp_status tpmlp_moe_fwd(const tpmlp_moe_desc* d, const int32_t* counts, const void* x,
                           const void* W1, const void* b1, const void* W2, void* y,
                           void* h_saved, void* a_saved, hipStream_t s) {
  tpmlp_status st = check_moe_desc(d);
  if (st != TPMLP_OK) return st;
  if ((st = check_ptrs({counts, x, W1, W2, y, a_saved})) != TPMLP_OK) return st;
  if (d->has_bias && (st = check_ptrs({b1})) != TPMLP_OK) return st;
  if (h_saved && !aligned16(h_saved)) return TPMLP_E_ALIGN;
  const int64_t T = d->tokens, H = d->hidden, Fs = d->ffn_shard;
  if (T == 0) return TPMLP_OK;
  const bool swiglu = d->act == TPMLP_ACT_SWIGLU;
  const int64_t GFs = swiglu ? 2 * Fs : Fs;
  EpiArgs e1{};
  e1.out = a_saved; e1.ldo = Fs;
  e1.out2 = h_saved; e1.ldo2 = GFs;
  e1.bias = d->has_bias ? b1 : nullptr;
  GemmArgs g1 = make_gemm(x, H, W1, H, T, Fs, H, Fs);
  set_groups(g1, d, counts);
  g1.b_gstride = GFs * H;
  g1.bias_gstride = GFs;
  hipError_t err = run_group_step(swiglu ? FC1_FWD_SWIGLU : FC1_FWD_GELU, GROUP_M, moe_label(0),
                                  g1, e1, s);
  if (err != hipSuccess) return hip_fail(err);
  EpiArgs e2{};
  e2.out = y; e2.ldo = H;
  GemmArgs g2 = make_gemm(a_saved, Fs, W2, Fs, T, H, Fs, 0);
  set_groups(g2, d, counts);
  g2.b_gstride = H * Fs;
  err = run_group_step(FC2_FWD, GROUP_M, moe_label(1), g2, e2, s);
  return err == hipSuccess ? TPMLP_OK : hip_fail(err);
}

tpmlp_status tpmlp_moe_bwd_dgrad(const tpmlp_moe_desc* d, const int32_t* counts, const void* dy,
                                 const void* W1, const void* W2, const void* h_saved, void* dH,
                                 void* dx, hipStream_t s) {
  tpmlp_status st = check_moe_desc(d);
  if (st != TPMLP_OK) return st;
  if ((st = check_ptrs({counts, dy, W1, W2, h_saved, dH, dx})) != TPMLP_OK) return st;
  const int64_t T = d->tokens, H = d->hidden, Fs = d->ffn_shard;
  if (T == 0) return TPMLP_OK;
  const bool swiglu = d->act == TPMLP_ACT_SWIGLU;
  const int64_t GFs = swiglu ? 2 * Fs : Fs;
  // fc2 dgrad per expert: dA = dy . W2[e], activation derivative fused
  EpiArgs e1{};
  e1.out = dH; e1.ldo = GFs;
  e1.aux = h_saved; e1.ldaux = GFs;
  GemmArgs g1 = make_gemm(dy, H, W2, Fs, T, Fs, H, Fs);
  set_groups(g1, d, counts);
  g1.b_gstride = H * Fs;
  hipError_t err = run_group_step(swiglu ? FC2_DGRAD_SWIGLU : FC2_DGRAD_GELU, GROUP_M,
                                  moe_label(2), g1, e1, s);
  if (err != hipSuccess) return hip_fail(err);
  // fc1 dgrad per expert: dx = dH . W1[e]
  EpiArgs e2{};
  e2.out = dx; e2.ldo = H;
  GemmArgs g2 = make_gemm(dH, GFs, W1, H, T, H, GFs, 0);
  set_groups(g2, d, counts);
  g2.b_gstride = GFs * H;
  err = run_group_step(FC1_DGRAD, GROUP_M, moe_label(3), g2, e2, s);
  return err == hipSuccess ? TPMLP_OK : hip_fail(err);
}

tpmlp_status tpmlp_moe_bwd_wgrad(const tpmlp_moe_desc* d, const int32_t* counts, const void* dy,
                                 const void* x, const void* a_saved, const void* dH, float* dW1,
                                 float* db1, float* dW2, int32_t accumulate, void* ws,
                                 size_t ws_bytes, hipStream_t s) {
  tpmlp_status st = check_moe_desc(d);
  if (st != TPMLP_OK) return st;
  if (accumulate != 0 && accumulate != 1) return TPMLP_E_DTYPE;
  if ((st = check_ptrs({counts, dy, x, a_saved, dH, dW1, dW2})) != TPMLP_OK) return st;
  if (d->has_bias && (st = check_ptrs({db1})) != TPMLP_OK) return st;
  const size_t need = moe_workspace_bytes(d);
  if (need && (!ws || ws_bytes < need)) return TPMLP_E_WORKSPACE;
  if (need && !aligned16(ws)) return TPMLP_E_ALIGN;
  const int64_t T = d->tokens, H = d->hidden, Fs = d->ffn_shard;
  if (T == 0 && accumulate) return TPMLP_OK;  // adding nothing
  const bool swiglu = d->act == TPMLP_ACT_SWIGLU;
  const int64_t GFs = swiglu ? 2 * Fs : Fs;
  // dW2[e] [H, Fs] = dy_e^T . a_e over expert e's rows
  EpiArgs e1{};
  e1.out = dW2; e1.ldo = Fs; e1.accumulate = accumulate;
  GemmArgs g1 = make_gemm(dy, H, a_saved, Fs, H, Fs, T, 0);
  set_groups(g1, d, counts);
  g1.out_gstride = H * Fs;
  hipError_t err = run_group_step(WGRAD, GROUP_K, moe_label(4), g1, e1, s);
  if (err != hipSuccess) return hip_fail(err);
  // dW1[e] [GFs, H] = dH_e^T . x_e (+ per-expert column-sum partials of dH_e)
  EpiArgs e2{};
  e2.out = dW1; e2.ldo = H; e2.accumulate = accumulate;
  e2.colsum = d->has_bias ? static_cast<float*>(ws) : nullptr;
  GemmArgs g2 = make_gemm(dH, GFs, x, H, GFs, H, T, 0);
  set_groups(g2, d, counts);
  g2.out_gstride = GFs * H;
  err = run_group_step(d->has_bias ? WGRAD_COLSUM : WGRAD, GROUP_K, moe_label(5), g2, e2, s);
  if (err != hipSuccess) return hip_fail(err);
  if (d->has_bias) {
    err = timed(moe_label(6), s, [&]() {
      return colsum_reduce_launch(static_cast<const float*>(ws), moe_colsum_parts(d), (int)GFs,
                                  db1, accumulate, s, d->experts);
    });
    if (err != hipSuccess) return hip_fail(err);
  }
  return TPMLP_OK;
}

size_t tpmlp_quantize_workspace_size(int64_t n) {
  if (n < 0) return 0;
  return align_up((size_t)quant_parts(n) * 4, 256);
}

}  // extern "C"

namespace {
tpmlp_status quantize_fp8(int32_t src_dtype, const void* src, int64_t n, uint8_t* dst,
                          float* amax_out, float* scale_inv_out, void* ws, size_t ws_bytes,
                          hipStream_t s, bool e5m2) {
  if (src_dtype != TPMLP_F32 && src_dtype != TPMLP_BF16) return TPMLP_E_DTYPE;
  if (n < 0) return TPMLP_E_SHAPE;
  if (!amax_out || !scale_inv_out) return TPMLP_E_NULL;
  if (n > 0) {
    tpmlp_status st = check_ptrs({src, dst});
    if (st != TPMLP_OK) return st;
  }
  if (!ws || ws_bytes < tpmlp_quantize_workspace_size(n)) return TPMLP_E_WORKSPACE;
  if (!aligned16(ws)) return TPMLP_E_ALIGN;
  const bool bf = src_dtype == TPMLP_BF16;
  const int nparts = quant_parts(n);
  float* parts = static_cast<float*>(ws);
  hipError_t err = timed("amax_partial", s, [&]() {
    return amax_partial_launch(bf, src, n, parts, nparts, s);
  });
  if (err != hipSuccess) return hip_fail(err);
  err = timed("quantize", s, [&]() {
    return quantize_launch(bf, src, n, dst, parts, nparts, amax_out, scale_inv_out, s, e5m2);
  });
  if (err != hipSuccess) return hip_fail(err);
  return TPMLP_OK;
}
}  // namespace

extern "C" {

tpmlp_status tpmlp_quantize_e4m3(int32_t src_dtype, const void* src, int64_t n, uint8_t* dst,
                                 float* amax_out, float* scale_inv_out, void* ws,
                                 size_t ws_bytes, hipStream_t s) {
  return quantize_fp8(src_dtype, src, n, dst, amax_out, scale_inv_out, ws, ws_bytes, s, false);
}

tpmlp_status tpmlp_quantize_e5m2(int32_t src_dtype, const void* src, int64_t n, uint8_t* dst,
                                 float* amax_out, float* scale_inv_out, void* ws,
                                 size_t ws_bytes, hipStream_t s) {
  return quantize_fp8(src_dtype, src, n, dst, amax_out, scale_inv_out, ws, ws_bytes, s, true);
}

tpmlp_status tpmlp_timing_enable(int32_t enable, const char* name_filter) {
  for (auto& r : g_recs) {
    g_pool.push_back(r.start);
    g_pool.push_back(r.stop);
  }
  g_recs.clear();
  g_clk_recs.clear();
  g_clk_used = 0;
  g_clk_dev = nullptr;
  g_timing = enable != 0;
  g_filter = (enable && name_filter) ? name_filter : "";
  if (g_timing) {
    // the clock slots of the current device, cleared (unwritten slots read
    // 0); without a device the facility times with events only
    void* p = nullptr;
    hipError_t err = hipGetSymbolAddress(&p, HIP_SYMBOL(clock_slots));
    if (err == hipSuccess) err = hipMemset(p, 0, sizeof(unsigned long long) * 4 * kClockSlots);
    if (err == hipSuccess) g_clk_dev = static_cast<unsigned long long*>(p);
    else (void)hipGetLastError();
  }
  return TPMLP_OK;
}

double tpmlp_timing_clock_mhz(const char* name) {
  for (auto& kv : g_clk_mhz)
    if (name && kv.first == name) return kv.second;
  return 0.0;
}

int32_t tpmlp_timing_collect(const char** names, int64_t* counts, double* total_ms, int32_t cap) {
  std::vector<const char*> keys;
  std::vector<int64_t> cnt;
  std::vector<double> tot;
  for (auto& r : g_recs) {
    if (hipEventSynchronize(r.stop) != hipSuccess) return -1;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) return -1;
    size_t i = 0;
    while (i < keys.size() && strcmp(keys[i], r.name) != 0) ++i;
    if (i == keys.size()) {
      keys.push_back(r.name);
      cnt.push_back(0);
      tot.push_back(0.0);
    }
    cnt[i] += 1;
    tot[i] += ms;
  }
  for (size_t i = 0; i < keys.size() && (int32_t)i < cap; ++i) {
    if (names) names[i] = keys[i];
    if (counts) counts[i] = cnt[i];
    if (total_ms) total_ms[i] = tot[i];
  }
  // mean shader clock per kernel name from the workgroups' counters (the
  // events above have completed, so have the launches)
  g_clk_mhz.clear();
  if (g_clk_dev && g_clk_used > 0) {
    std::vector<unsigned long long> h((size_t)4 * g_clk_used);
    if (hipMemcpy(h.data(), g_clk_dev, h.size() * sizeof(unsigned long long),
                  hipMemcpyDeviceToHost) != hipSuccess)
      return -1;
    std::vector<std::pair<std::string, std::pair<double, double>>> acc;
    for (auto& r : g_clk_recs) {
      double cyc = 0, tick = 0;
      for (int i = r.off; i < r.off + r.n; ++i) {
        const unsigned long long* q = &h[(size_t)4 * i];
        // a workgroup that exited early (surplus ids of a grouped launch) has no end
        if (q[2] > q[0] && q[3] > q[1]) {
          cyc += (double)(q[2] - q[0]);
          tick += (double)(q[3] - q[1]);
        }
      }
      size_t j = 0;
      while (j < acc.size() && acc[j].first != r.name) ++j;
      if (j == acc.size()) acc.push_back({r.name, {0.0, 0.0}});
      acc[j].second.first += cyc;
      acc[j].second.second += tick;
    }
    for (auto& a : acc)
      if (a.second.second > 0) g_clk_mhz.push_back({a.first, 100.0 * a.second.first / a.second.second});
  }
  return (int32_t)keys.size();
}

}  // extern "C"
