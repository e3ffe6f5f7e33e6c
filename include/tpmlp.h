/*
 * libtpmlp -- one tensor-parallel rank's share of a column->row transformer MLP
 * block on AMD Instinct MI355X (gfx950), forward and backward.
 *
 * The block (Megatron-LM code tour, pyshine.com, sections "The Tensor-Parallel
 * Primitives" and "The Transformer Stack"):
 *   fc1  column-parallel linear: its weight is split along the output features,
 *        so this rank computes a slice of fc1's outputs from the full input;
 *   act  a fused bias + GELU (tanh form), or the gated SwiGLU variant
 *        a = silu(gate) * up;
 *   fc2  row-parallel linear: its weight is split along the input features, so
 *        this rank produces a partial sum of the block output that the caller
 *        all-reduces across ranks.
 * The conjugate operators of the concept note "Megatron-LM / Megatron-Core"
 * (section "Key math / How it works") fix the boundary: the input x and the
 * output gradient dy are replicated on every rank and used as given; the
 * outputs y_partial and dx_partial are partial sums whose all-reduce is the
 * caller's job. No call communicates.
 *
 * Notation and layouts (all row-major, contiguous, 16-byte aligned):
 *   T tokens, H hidden, Fs intermediate features of this shard, G = 2 for
 *   SwiGLU (gate and up halves), 1 for GELU.
 *   x, dy, y_partial, dx_partial : [T, H]
 *   W1_shard : [G*Fs, H]  ([out, in]; for SwiGLU rows [0,Fs) gate, [Fs,2Fs) up)
 *   b1_shard : [G*Fs]     (GELU only)
 *   W2_shard : [H, Fs]
 *   h_saved  : [T, G*Fs]  pre-activation including the bias (saved for backward)
 *   a_saved  : [T, Fs]    activation output (fc2's input)
 *   dH       : [T, G*Fs]  gradient at the pre-activation
 *   dW1 [G*Fs, H], db1 [G*Fs], dW2 [H, Fs] : float32 always.
 *
 * Element types by tpmlp_desc.dtype:
 *   TPMLP_F32  : everything float32.
 *   TPMLP_BF16 : x, W1, b1, W2, dy, h, a, dH, y_partial, dx_partial bfloat16;
 *                products accumulate in float32.
 *   TPMLP_E4M3 : GELU or SwiGLU. FP8 with per-tensor float32 dequantisation
 *                factors (scale_inv): forward tensors in OCP E4M3, gradients
 *                in OCP E5M2 (Transformer Engine's default "hybrid" format;
 *                the pages name FP8 through Transformer Engine, code tour
 *                "Honest Limits", concept note "Key math / How it works").
 *                x, W1, W2, a_saved: E4M3 codes. dy, dH: E5M2 codes.
 *                b1, h_saved, y_partial, dx_partial: bfloat16. dW1, db1,
 *                dW2: float32. The block quantises the two tensors it
 *                produces and reuses: a (E4M3, forward) with current scaling
 *                (scale = 448 / amax(a); 1 when amax is 0 or the quotient
 *                overflows) or delayed
 *                scaling (tpmlp_fp8_history), and dH (E5M2, dgrad) with
 *                delayed scaling; for SwiGLU both halves of dH take the one
 *                scale and amax. Codes saturate at the largest finite value
 *                (448, 57344) and are rounded to nearest even.
 *
 * Ownership: the caller allocates and frees every buffer, the workspace too
 * (size from tpmlp_workspace_size). Pointers are device pointers unless noted.
 * The library keeps no per-call state. Its only global state is the timing
 * facility at the end of this header.
 *
 * Asynchrony: compute calls validate their arguments on the host, then only
 * enqueue kernels on `stream` (NULL = the default stream) and return. On a
 * validation error nothing is enqueued. Device faults surface at the caller's
 * next synchronisation.
 *
 * Aliasing: no output may overlap any input or another output.
 */
#ifndef TPMLP_H
#define TPMLP_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TPMLP_ABI_VERSION 9

typedef enum {
  TPMLP_OK = 0,
  TPMLP_E_NULL = 1,        /* a required pointer is NULL */
  TPMLP_E_SHAPE = 2,       /* T < 0, H <= 0, Fs <= 0, H or Fs not a multiple of 16, or too large */
  TPMLP_E_DTYPE = 3,       /* unknown dtype or activation code */
  TPMLP_E_ALIGN = 4,       /* a pointer is not 16-byte aligned */
  TPMLP_E_UNSUPPORTED = 5, /* valid but not provided (SwiGLU bias; E4M3 attention; MoE not BF16) */
  TPMLP_E_WORKSPACE = 6,   /* workspace NULL or smaller than tpmlp_workspace_size */
  TPMLP_E_HIP = 7,         /* a HIP runtime call failed while enqueuing */
  TPMLP_E_SCRATCH = 8      /* too large for the fixed scratch of tpmlp_bwd_wgrad_noalloc */
} tpmlp_status;

typedef enum { TPMLP_F32 = 0, TPMLP_BF16 = 1, TPMLP_E4M3 = 2 } tpmlp_dtype;
typedef enum { TPMLP_ACT_GELU_TANH = 0, TPMLP_ACT_SWIGLU = 1 } tpmlp_act;
typedef enum {
  TPMLP_CALL_FWD = 0,
  TPMLP_CALL_DGRAD = 1,
  TPMLP_CALL_WGRAD = 2,
  TPMLP_CALL_WGRAD_RECOMPUTE = 3
} tpmlp_call;

/* Problem description (host memory). */
typedef struct tpmlp_desc {
  int64_t tokens;     /* T >= 0 (0: calls are valid and enqueue nothing, except
                         wgrad with accumulate = 0, which zero-fills its outputs) */
  int64_t hidden;     /* H > 0, multiple of 16 */
  int64_t ffn_shard;  /* Fs > 0, multiple of 16 */
  int32_t act;        /* tpmlp_act */
  int32_t dtype;      /* tpmlp_dtype */
  int32_t has_bias;   /* 1: b1_shard is used (GELU only); 0: no bias */
  int32_t reserved;   /* must be 0 */
} tpmlp_desc;

/*
 * Delayed scaling state of one tensor that the block quantises itself (a in
 * the forward, dH in dgrad): a host struct holding device pointers, owned by
 * the caller and updated by each call (Transformer Engine's delayed scaling
 * with margin 0). The call quantises with *scale; afterwards the tensor's
 * amax (max |value| over the tensor) enters the history, newest first, the
 * oldest entry dropping out; *scale_inv = 1 / (the factor the call used),
 * which is what consumers of the codes dequantise with; and *scale =
 * fmax / max(history) for the next call (fmax 448 for E4M3, 57344 for E5M2),
 * unchanged while that maximum is 0 or not finite, or so small that the
 * quotient overflows float32. All float32. The amax is taken over the
 * tensor's float32 values before scaling (NaN elements, which finite inputs
 * do not produce, are left out). A call with no tokens still
 * updates the state, with an amax of 0. Calls that share one state must be
 * ordered on one stream.
 */
typedef struct tpmlp_fp8_history {
  float* amax_history;  /* [len] device floats, newest first (start with zeros) */
  float* scale;         /* device float: in, the factor this call uses; out, the next one */
  float* scale_inv;     /* device float: out, 1 / (the factor this call used) */
  int32_t len;          /* 1 .. 4096 */
  int32_t reserved;     /* must be 0 */
} tpmlp_fp8_history;

/* FP8 scales (host struct holding device pointers to single floats); the
   fields a call does not use are ignored. */
typedef struct tpmlp_fp8_scales {
  const float* x_scale_inv;   /* fwd, wgrad: dequantisation factor of x (E4M3) */
  const float* w1_scale_inv;  /* fwd, dgrad: of W1_shard (E4M3) */
  const float* w2_scale_inv;  /* fwd, dgrad: of W2_shard (E4M3) */
  float* a_amax;              /* fwd with current scaling: out, max |a| of the bfloat16-rounded a */
  float* a_scale_inv;         /* fwd with current scaling: out, 1 / (448 / a_amax), as used by fc2;
                                 wgrad: in, the factor of a_saved (with delayed scaling: the
                                 a_history->scale_inv the forward wrote) */
  const tpmlp_fp8_history* a_history;   /* fwd: delayed scaling of a; NULL: current scaling */
  const float* dy_scale_inv;  /* dgrad, wgrad: of dy (E5M2) */
  const tpmlp_fp8_history* dH_history;  /* dgrad: delayed scaling of dH (E5M2), required */
  const float* dH_scale_inv;  /* wgrad: of dH (the dH_history->scale_inv dgrad wrote) */
} tpmlp_fp8_scales;

/*
 * Bytes of workspace for the call (0 if none). Returns 0 for an invalid desc.
 * Non-zero for: the E4M3 forward (per-workgroup amax partials of a and,
 * with current scaling, the bfloat16 activation before quantisation; the
 * size covers both modes), the E4M3 dgrad (amax partials of dH), and the
 * weight gradient: with bias, per-tile-column partial sums of db1 (needed),
 * and for products whose tile grid would leave compute units idle, the
 * fp32 partial sums of a split along K: for BF16 grids of few tiles, every
 * tile split; for BF16 and E4M3 grids whose last round of tiles is a partial
 * one (8 to 128 workgroups left over on the 256 compute units; products
 * without the fused db1 column sums, of at least 16 K-stages), those last
 * tiles split in two halves along K, each tile's halves added by whichever
 * of its two workgroups ends second, plus one counter per such tile. This
 * part is optional: with fewer bytes the products run unsplit, and the call
 * needs only the db1 partials. Split products are summed in a fixed order,
 * so results stay reproducible, but differ in rounding from unsplit ones.
 * TPMLP_CALL_WGRAD_RECOMPUTE: the
 * recomputed activation (T * Fs elements, rounded up to 256 bytes) plus the
 * weight gradient's workspace. Returns 0 for an unknown call.
 */
size_t tpmlp_workspace_size(const tpmlp_desc* desc, int32_t call);

/*
 * Forward (fc1 -> activation -> fc2), enqueued on `stream`:
 *   h = x . W1_shard^T (+ b1_shard);  a = act(h);  y_partial = a . W2_shard^T.
 * For E4M3 the fc1 accumulator is multiplied by x_scale_inv * w1_scale_inv
 * before the bias, and h is stored in bfloat16; a = gelu(h as stored) is
 * quantised to E4M3 into a_saved. With current scaling (fp8->a_history
 * NULL) it goes through a bfloat16 copy of a in the workspace, and the scale
 * comes from that copy's amax (a second pass). With delayed scaling it is
 * quantised from its fp32 value directly in fc1's epilogue at
 * a_history->scale, after which the history is updated. fc2's accumulator is
 * multiplied by (1 / a's scale) * w2_scale_inv. h_saved may be NULL (inference: nothing saved for backward).
 * a_saved is required. b1_shard is required iff desc->has_bias. fp8 must be
 * non-NULL iff dtype is E4M3.
 */
tpmlp_status tpmlp_fwd(const tpmlp_desc* desc, const void* x, const void* W1_shard,
                       const void* b1_shard, const void* W2_shard, void* y_partial,
                       void* h_saved, void* a_saved, const tpmlp_fp8_scales* fp8,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Data gradient (fc2 dgrad with the activation derivative fused, then fc1 dgrad):
 *   dA = dy . W2_shard;
 *   GELU:   dH = dA * gelu'(h)
 *   SwiGLU: dH = [dA * up * silu'(gate) | dA * silu(gate)]  (gate, up = halves of h)
 *   dx_partial = dH . W1_shard.
 * dH is written (the caller keeps it for tpmlp_bwd_wgrad). For E4M3:
 * dy is E5M2 codes; dA is the accumulator times dy_scale_inv * w2_scale_inv;
 * dH is quantised to E5M2 in the epilogue at fp8->dH_history->scale and the
 * history updated; dx_partial = dH_codes . W1_codes times
 * dH_history->scale_inv * w1_scale_inv. fp8 must be non-NULL iff dtype is
 * E4M3. Workspace: tpmlp_workspace_size(desc, TPMLP_CALL_DGRAD) bytes.
 */
tpmlp_status tpmlp_bwd_dgrad(const tpmlp_desc* desc, const void* dy, const void* W1_shard,
                             const void* W2_shard, const void* h_saved, void* dH,
                             void* dx_partial, const tpmlp_fp8_scales* fp8, void* workspace,
                             size_t workspace_bytes, hipStream_t stream);

/*
 * Weight gradients, float32 results:
 *   dW2 = dy^T . a_saved;  dW1 = dH^T . x;  db1 = column sums of dH (if has_bias).
 * accumulate = 0 overwrites the outputs; accumulate = 1 adds into them
 * (gradient accumulation across micro-batches). db1 may be NULL only when
 * has_bias = 0. For E4M3 the operands are FP8 codes (dy, dH: E5M2; x, a: E4M3)
 * and each product is scaled by its two operands' dequantisation factors
 * from fp8 (dy_scale_inv, a_scale_inv, dH_scale_inv, x_scale_inv); db1 is
 * the column sums of the dequantised dH. fp8 must be non-NULL iff dtype is
 * E4M3. Workspace: tpmlp_workspace_size(desc, TPMLP_CALL_WGRAD) bytes (the
 * db1 partials are required with bias; the split-K part is optional).
 * Results are reproducible bit for bit: every sum is taken in a fixed order
 * (the two halves of a tile split in two are added in one fp32 addition,
 * whose result does not depend on which half ends first); no sum goes
 * through atomics.
 */
tpmlp_status tpmlp_bwd_wgrad(const tpmlp_desc* desc, const void* dy, const void* x,
                             const void* a_saved, const void* dH, float* dW1, float* db1,
                             float* dW2, int32_t accumulate, const tpmlp_fp8_scales* fp8,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Weight gradients with the activation recomputed instead of saved: the
 * selective activation recomputation of the concept note "Megatron-LM /
 * Megatron-Core" (section "Key math / How it works"), which trades a little
 * compute for the memory of a_saved between the forward and the backward.
 * Same arguments, results and errors as tpmlp_bwd_wgrad, with the saved
 * pre-activation h_saved ([T, G*Fs], as tpmlp_fwd wrote it) in place of
 * a_saved: the call first forms a = act(h_saved) in the workspace, with the
 * forward epilogue's own function of h as stored, then runs the products of
 * tpmlp_bwd_wgrad on it.
 *   BF16, F32: a equals the forward's a_saved bit for bit, and so do the
 *     results those of tpmlp_bwd_wgrad.
 *   E4M3: a's codes are E4M3(act(h) * (1 / fp8->a_scale_inv)), the
 *     float32 factor recomputed from the dequantisation factor that the wgrad
 *     call already takes; they match the forward's codes wherever that
 *     factor equals the forward's (with delayed scaling the forward quantised
 *     the float32 act(h) at a_history->scale, of which a_scale_inv is the
 *     inverse).
 * Workspace: tpmlp_workspace_size(desc, TPMLP_CALL_WGRAD_RECOMPUTE) bytes, the
 * recomputed a (T * Fs elements, rounded up to 256 bytes) followed by
 * tpmlp_bwd_wgrad's workspace (its split-K part optional as there).
 */
tpmlp_status tpmlp_bwd_wgrad_recompute(const tpmlp_desc* desc, const void* dy, const void* x,
                                       const void* h_saved, const void* dH, float* dW1,
                                       float* db1, float* dW2, int32_t accumulate,
                                       const tpmlp_fp8_scales* fp8, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream);

/*
 * Byte transpose into the token-contiguous layout of tpmlp_bwd_wgrad_t:
 * dst[c][r] = src[r][c] for the row-major src [rows][cols] (1-byte codes,
 * cols a multiple of 16), dst [cols][Tp] with Tp = rows rounded up to a
 * multiple of 16 and dst's columns [rows, Tp) zero (the cast-transpose
 * layout in which FP8 training keeps the operands it reads along the tokens).
 * src and dst are device pointers, 16-byte aligned, not overlapping.
 * TPMLP_E_SHAPE for negative sizes or cols not a multiple of 16.
 */
tpmlp_status tpmlp_transpose_u8(const void* src, int64_t rows, int64_t cols, void* dst,
                                hipStream_t stream);

/*
 * tpmlp_bwd_wgrad for E4M3 from token-contiguous copies of its four operands
 * (the tokens are the products' K): dy_t [H][Tp] (E5M2), x_t [H][Tp] (E4M3),
 * a_t [Fs][Tp] (E4M3), dH_t [G*Fs][Tp] (E5M2), Tp = T rounded up to a multiple
 * of 16, columns [T, Tp) zero, as tpmlp_transpose_u8 writes them. With both
 * operands of each product contiguous along K, the products run the forward's
 * FP8 schedule instead of reading 8-bit data through LDS transposes.
 * Same arguments otherwise, and the same results up to the float32 rounding
 * of the sums (a different MFMA shape): dW2 = dy^T . a, dW1 = dH^T . x, each
 * times its operands' dequantisation factors, db1 = the dequantised dH
 * summed over the tokens (has_bias); accumulate as tpmlp_bwd_wgrad.
 * Reproducible bit for bit. No workspace. TPMLP_E_UNSUPPORTED unless dtype
 * is E4M3; TPMLP_E_SHAPE for Tp above 2^23 - 256 (a tile's 256 rows of Tp
 * bytes are addressed with 32-bit offsets). The products and the pages'
 * weight-gradient step: code tour "The Tensor-Parallel Primitives"; FP8
 * through Transformer Engine: concept note "Key math / How it works".
 */
tpmlp_status tpmlp_bwd_wgrad_t(const tpmlp_desc* desc, const void* dy_t, const void* x_t,
                               const void* a_t, const void* dH_t, float* dW1, float* db1,
                               float* dW2, int32_t accumulate, const tpmlp_fp8_scales* fp8,
                               hipStream_t stream);

/*
 * tpmlp_bwd_wgrad without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc). Same arguments, results and errors as
 * tpmlp_bwd_wgrad given only the workspace it cannot run without: the
 * products are never split along K, so the results are bit for bit those of
 * tpmlp_bwd_wgrad with tpmlp_workspace_size(desc, TPMLP_CALL_WGRAD) bytes
 * whenever that size plans no split. The db1 partial sums (bias, bf16 or
 * E4M3) go to a fixed device array of TPMLP_SCRATCH_BYTES bytes that every
 * GPU the library runs on holds until the process ends; its address is
 * looked up on the call's first use on a device. A problem whose partial sums
 * need more, (ceil(H / 256) * G * Fs * 4 bytes), returns TPMLP_E_SCRATCH
 * before anything is enqueued. The call allocates and frees nothing. Every
 * call on one GPU shares that GPU's array: calls that overlap on one GPU (on
 * different streams, or from different host threads) race.
 */
#define TPMLP_SCRATCH_BYTES ((size_t)8 << 20)
tpmlp_status tpmlp_bwd_wgrad_noalloc(const tpmlp_desc* desc, const void* dy, const void* x,
                                     const void* a_saved, const void* dH, float* dW1,
                                     float* db1, float* dW2, int32_t accumulate,
                                     const tpmlp_fp8_scales* fp8, hipStream_t stream);

/*
 * Per-tensor current-scaling quantiser (the FP8 recipe used for `a` inside
 * tpmlp_fwd, exported so callers can produce E4M3 inputs on the device):
 *   amax = max |src|; scale = 448 / amax in float32 (1 if amax is 0, or so
 *   small that 448 / amax overflows float32: below about 1.3e-36);
 *   dst[i] = E4M3(clamp(fl32(src[i] * scale), -448, 448)), round to nearest even;
 *   *amax_out = amax; *scale_inv_out = 1 / scale in float32.
 * src_dtype is TPMLP_F32 or TPMLP_BF16; n >= 0 elements; dst n bytes.
 * Workspace: tpmlp_quantize_workspace_size(n) bytes.
 */
size_t tpmlp_quantize_workspace_size(int64_t n);
tpmlp_status tpmlp_quantize_e4m3(int32_t src_dtype, const void* src, int64_t n, uint8_t* dst,
                                 float* amax_out, float* scale_inv_out, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream);
/* The same recipe into OCP E5M2 (for gradients such as dy): scale = 57344 /
   amax, codes saturate at +-57344. Same arguments and workspace. */
tpmlp_status tpmlp_quantize_e5m2(int32_t src_dtype, const void* src, int64_t n, uint8_t* dst,
                                 float* amax_out, float* scale_inv_out, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream);

/*
 * ---------------------------------------------------------------- attention
 * One rank's share of the attention block's two projections, on the same
 * kernels as the MLP (code tour, "The Transformer Stack" and its SelfAttention
 * entry: one packed QKV projection, column-parallel, and the output
 * projection, row-parallel; concept note, "Key math / How it works": heads are
 * split over the TP ranks). The core attention between them (softmax over
 * q k^T, times v) is not part of the library; as for the MLP, the caller
 * all-reduces y_partial and dx_partial.
 *
 * Notation and layouts (row-major, contiguous, 16-byte aligned):
 *   nq query heads and nkv key/value heads on this rank (nkv divides nq;
 *   query head j uses key/value head j / (nq / nkv)), hn the head size,
 *   Nqkv = (nq + 2 nkv) hn, D = nq hn.
 *   x, dy, y_partial, dx_partial : [T, H]
 *   Wqkv : [Nqkv, H]  this rank's rows stacked [Wq (nq hn rows); Wk (nkv hn);
 *                     Wv (nkv hn)], each head's rows contiguous ([out, in])
 *   bqkv : [Nqkv]     the same order (when has_bias)
 *   qkv, dqkv : [T, Nqkv]  per token [q heads | k heads | v heads]: q is
 *                     columns [0, D), k [D, D + nkv hn), v the rest, each a
 *                     [T, heads, hn] view with row stride Nqkv
 *   ctx, dctx : [T, D]  the core attention's output, heads concatenated
 *   Wo : [H, D]
 *   dWqkv [Nqkv, H], dbqkv [Nqkv], dWo [H, D] : float32 always.
 * Element types: TPMLP_F32 (all float32) or TPMLP_BF16 (everything but the
 * weight gradients bfloat16, float32 accumulation); E4M3 is not provided
 * (TPMLP_E_UNSUPPORTED). The output projection's bias is not in the partial
 * sum: it is added once after the all-reduce. Errors, ownership, asynchrony
 * and aliasing as for the MLP calls; accumulate as in tpmlp_bwd_wgrad.
 */
typedef struct tpmlp_attn_desc {
  int64_t tokens;     /* T >= 0 */
  int64_t hidden;     /* H > 0, multiple of 16 */
  int32_t q_heads;    /* nq > 0 */
  int32_t kv_heads;   /* nkv > 0, divides nq */
  int32_t head_dim;   /* hn > 0, multiple of 16 */
  int32_t dtype;      /* TPMLP_F32 or TPMLP_BF16 */
  int32_t has_bias;   /* 1: the QKV projection has a bias; 0: none */
  int32_t reserved;   /* must be 0 */
} tpmlp_attn_desc;

/* qkv = x . Wqkv^T (+ bqkv). bqkv is required iff has_bias. */
tpmlp_status tpmlp_attn_qkv_fwd(const tpmlp_attn_desc* desc, const void* x, const void* Wqkv,
                                const void* bqkv, void* qkv, hipStream_t stream);
/* y_partial = ctx . Wo^T. */
tpmlp_status tpmlp_attn_out_fwd(const tpmlp_attn_desc* desc, const void* ctx, const void* Wo,
                                void* y_partial, hipStream_t stream);
/* dctx = dy . Wo (dy replicated on every rank). The workspace (may be NULL)
   enables split-K, see tpmlp_attn_workspace_size. */
tpmlp_status tpmlp_attn_out_bwd_dgrad(const tpmlp_attn_desc* desc, const void* dy,
                                      const void* Wo, void* dctx, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream);
/* dWo (+)= dy^T . ctx, float32. Workspace as for tpmlp_attn_out_bwd_dgrad. */
tpmlp_status tpmlp_attn_out_bwd_wgrad(const tpmlp_attn_desc* desc, const void* dy,
                                      const void* ctx, float* dWo, int32_t accumulate,
                                      void* workspace, size_t workspace_bytes,
                                      hipStream_t stream);
/* dx_partial = dqkv . Wqkv. */
tpmlp_status tpmlp_attn_qkv_bwd_dgrad(const tpmlp_attn_desc* desc, const void* dqkv,
                                      const void* Wqkv, void* dx_partial, hipStream_t stream);
/* dWqkv (+)= dqkv^T . x and, when has_bias, dbqkv (+)= column sums of dqkv
   (dbqkv required iff has_bias); float32.
   Workspace of the three backward calls that take one: with
   tpmlp_attn_workspace_size(desc) bytes (the same buffer serves all three,
   one call at a time) a bf16 product whose tile grid would leave compute
   units idle is split along K into fp32 partial sums that a second pass adds
   up in a fixed order (results do not depend on timing, but differ in
   rounding from the unsplit product). A smaller workspace (or NULL) runs
   unsplit; the qkv wgrad with bias in bf16 still needs the bytes of its
   column-sum partials (TPMLP_E_WORKSPACE otherwise). */
size_t tpmlp_attn_workspace_size(const tpmlp_attn_desc* desc);
tpmlp_status tpmlp_attn_qkv_bwd_wgrad(const tpmlp_attn_desc* desc, const void* dqkv,
                                      const void* x, float* dWqkv, float* dbqkv,
                                      int32_t accumulate, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream);

/*
 * ---------------------------------------------------------------- mixture of experts
 * The expert MLPs of a mixture-of-experts layer: this rank's E local experts,
 * each the per-rank block above with its own weights, over the token rows
 * already grouped by expert (onegen.ai overview, "Key Features"; concept
 * note, "Key math / How it works": expert parallelism, whose all-to-all
 * dispatch and combine, routing and permutation stay with the caller). Each
 * call is one launch per product covering every expert (grouped GEMM).
 *
 *   counts : [E] int32, device: rows of each expert in expert order; expert e
 *            owns rows [off_e, off_e + counts[e]) of x, y, h, a, dy, dH, dx,
 *            off_e = counts[0] + ... + counts[e-1]. The kernels read them on
 *            the device (no host copy needed). Negative counts count as 0 and
 *            the running total is capped at `tokens`, so no row outside
 *            [0, tokens) is read or written; rows past the sum of the counts
 *            are left as they are (and add nothing to the weight gradients).
 *   x, dy, y, dx : [tokens, H]; h, dH : [tokens, G*Fs]; a : [tokens, Fs]
 *   W1 : [E, G*Fs, H]; b1 : [E, G*Fs] (GELU only); W2 : [E, H, Fs]
 *   dW1 [E, G*Fs, H], db1 [E, G*Fs], dW2 [E, H, Fs] : float32.
 * dtype TPMLP_BF16 only (other dtypes: TPMLP_E_UNSUPPORTED). Layouts,
 * ownership, errors, asynchrony, aliasing and accumulate as for the
 * per-rank block; counts must stay unchanged until the calls reading them
 * have run.
 */
typedef struct tpmlp_moe_desc {
  int64_t tokens;     /* rows of the grouped tensors, >= 0 */
  int64_t hidden;     /* H > 0, multiple of 16 */
  int64_t ffn_shard;  /* Fs per expert > 0, multiple of 16 */
  int32_t experts;    /* E, 1 .. 1024 */
  int32_t act;        /* tpmlp_act */
  int32_t dtype;      /* TPMLP_BF16 */
  int32_t has_bias;   /* GELU only */
  int32_t reserved0;  /* must be 0 */
  int32_t reserved1;  /* must be 0 */
} tpmlp_moe_desc;

tpmlp_status tpmlp_moe_fwd(const tpmlp_moe_desc* desc, const int32_t* counts, const void* x,
                           const void* W1, const void* b1, const void* W2, void* y,
                           void* h_saved, void* a_saved, hipStream_t stream);
tpmlp_status tpmlp_moe_bwd_dgrad(const tpmlp_moe_desc* desc, const int32_t* counts,
                                 const void* dy, const void* W1, const void* W2,
                                 const void* h_saved, void* dH, void* dx, hipStream_t stream);
/* Workspace: tpmlp_moe_workspace_size(desc) bytes (0 without bias). */
size_t tpmlp_moe_workspace_size(const tpmlp_moe_desc* desc);
tpmlp_status tpmlp_moe_bwd_wgrad(const tpmlp_moe_desc* desc, const int32_t* counts,
                                 const void* dy, const void* x, const void* a_saved,
                                 const void* dH, float* dW1, float* db1, float* dW2,
                                 int32_t accumulate, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream);

const char* tpmlp_strerror(tpmlp_status status);
int32_t tpmlp_abi_version(void);
/* Text of the last HIP error seen by the library on this thread ("" if none). */
const char* tpmlp_last_hip_error(void);

/*
 * Kernel timing (host-side facility; not thread-safe, one stream at a time).
 * While enabled, every kernel the library launches whose name contains
 * `name_filter` (NULL or "" = all) is bracketed by two HIP events recorded on
 * its launch stream. tpmlp_timing_collect synchronises on those events and
 * returns, per kernel name, the launch count and total milliseconds.
 * tpmlp_timing_enable(0, NULL) disables and discards records.
 */
tpmlp_status tpmlp_timing_enable(int32_t enable, const char* name_filter);
/* Fills up to `cap` entries; returns the number of distinct kernel names (or -1 on error). */
int32_t tpmlp_timing_collect(const char** names, int64_t* counts, double* total_ms, int32_t cap);
/*
 * Mean shader clock in MHz of the bf16/FP8 GEMM launches named `name` made
 * while the facility was enabled, up to the last tpmlp_timing_collect (0 if
 * none; every such launch counts, whatever the name filter selects for
 * events): each of their workgroups reads the shader clock counter and the
 * 100 MHz real-time counter at its start and end into a fixed device array
 * of 131072 workgroup entries, 4 MiB (launches past that go without); the
 * clock is the sum of cycles over the sum of real-time ticks.
 * tpmlp_timing_enable clears the array (a blocking memset; where that fails
 * the facility times with events only), so the facility is not for use
 * under graph capture.
 */
double tpmlp_timing_clock_mhz(const char* name);

#ifdef __cplusplus
}
#endif

#endif /* TPMLP_H */
