// Device-side building blocks shared by the libtpmlp kernels (gfx950 / CDNA4).
//
// * vector types for MFMA operands and accumulators;
// * buffer-resource loads: the hardware range check turns every access past a
//   tensor's end into a zero, which gives ragged tiles for free;
// * fp32 <-> bf16 and fp32 -> OCP E4M3 conversions (round to nearest even);
// * the activation functions of the MLP block and their derivatives in fp32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tpmlp {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef uint16_t bf16_t;  // bfloat16 storage
typedef uint8_t e4m3_t;   // OCP E4M3 storage

#define TPMLP_LDS __attribute__((address_space(3)))

// ---------------------------------------------------------------- buffer loads
// Resource word 3 for gfx9-family raw buffers (32-bit data format, no swizzle).
constexpr int kBufferFlags = 0x00020000;
// Offsets at or beyond this value are always outside a resource (records are
// capped below it), so loads from them return zero.
constexpr uint32_t kOOB = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  if (bytes < 0) bytes = 0;
  if (bytes > 0x7fffffffLL) bytes = 0x7fffffffLL;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kBufferFlags);
}

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

// ---------------------------------------------------------------- conversions
__device__ __forceinline__ float bf2f(bf16_t u) {
  return __uint_as_float(((uint32_t)u) << 16);
}
__device__ __forceinline__ bf16_t f2bf(float f) {
  __bf16 h = (__bf16)f;  // round to nearest even (hardware cvt on gfx950)
  return __builtin_bit_cast(bf16_t, h);
}
__device__ __forceinline__ float round_bf16(float f) { return bf2f(f2bf(f)); }

// Two floats to two E4M3 codes (low byte = a). Inputs are clamped to +-448
// first: the conversion instruction rounds to nearest even in OCP E4M3 but
// yields NaN (not the largest finite value) above 448.
__device__ __forceinline__ uint32_t f2e4m3x2(float a, float b) {
  a = __builtin_fminf(__builtin_fmaxf(a, -448.0f), 448.0f);
  b = __builtin_fminf(__builtin_fmaxf(b, -448.0f), 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xffffu;
}

// Floats to OCP E5M2 codes, as f2e4m3x2: clamped to +-57344 first (the
// conversion rounds to nearest even but gives infinity past the largest
// finite value).
__device__ __forceinline__ uint32_t f2e5m2x2(float a, float b) {
  a = __builtin_fminf(__builtin_fmaxf(a, -57344.0f), 57344.0f);
  b = __builtin_fminf(__builtin_fmaxf(b, -57344.0f), 57344.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false) & 0xffffu;
}
// 8 floats to 8 FP8 codes (E4M3, or E5M2 if E5), byte u = code of v[u]
template <bool E5>
__device__ __forceinline__ u32x2 pack_fp8x8(const float (&v)[8]) {
  u32x2 w;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const uint32_t lo = E5 ? f2e5m2x2(v[4 * q], v[4 * q + 1]) : f2e4m3x2(v[4 * q], v[4 * q + 1]);
    const uint32_t hi = E5 ? f2e5m2x2(v[4 * q + 2], v[4 * q + 3]) : f2e4m3x2(v[4 * q + 2], v[4 * q + 3]);
    w[q] = lo | (hi << 16);
  }
  return w;
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int kBytes = 4;
  // 8 consecutive elements at index i (i a multiple of 8, 32-byte aligned)
  __device__ __forceinline__ static void load8(const void* p, int64_t i, float (&v)[8]) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(static_cast<const float*>(p) + i);
    const f32x4 b = *reinterpret_cast<const f32x4*>(static_cast<const float*>(p) + i + 4);
#pragma unroll
    for (int q = 0; q < 4; ++q) { v[q] = a[q]; v[q + 4] = b[q]; }
  }
  __device__ __forceinline__ static void store8(void* p, int64_t i, const float (&v)[8]) {
    *reinterpret_cast<f32x4*>(static_cast<float*>(p) + i) = f32x4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4*>(static_cast<float*>(p) + i + 4) = f32x4{v[4], v[5], v[6], v[7]};
  }
  __device__ __forceinline__ static float load(const void* p, int64_t i) {
    return static_cast<const float*>(p)[i];
  }
  __device__ __forceinline__ static void store(void* p, int64_t i, float v) {
    static_cast<float*>(p)[i] = v;
  }
  __device__ __forceinline__ static float round(float v) { return v; }
};
template <> struct Elem<bf16_t> {
  static constexpr int kBytes = 2;
  __device__ __forceinline__ static void load8(const void* p, int64_t i, float (&v)[8]) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(static_cast<const bf16_t*>(p) + i);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q] = __uint_as_float(w[q] << 16);
      v[2 * q + 1] = __uint_as_float(w[q] & 0xffff0000u);
    }
  }
  __device__ __forceinline__ static void store8(void* p, int64_t i, const float (&v)[8]) {
    u32x4 w;
#pragma unroll
    for (int q = 0; q < 4; ++q) w[q] = (uint32_t)f2bf(v[2 * q]) | ((uint32_t)f2bf(v[2 * q + 1]) << 16);
    *reinterpret_cast<u32x4*>(static_cast<bf16_t*>(p) + i) = w;
  }
  __device__ __forceinline__ static float load(const void* p, int64_t i) {
    return bf2f(static_cast<const bf16_t*>(p)[i]);
  }
  __device__ __forceinline__ static void store(void* p, int64_t i, float v) {
    static_cast<bf16_t*>(p)[i] = f2bf(v);
  }
  __device__ __forceinline__ static float round(float v) { return round_bf16(v); }
};

// 8 consecutive elements as 16 (bf16) or 32 (fp32) bytes <-> 8 floats.
__device__ __forceinline__ void unpack_bf16x8(const u32x4 w, float (&v)[8]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    v[2 * q] = __uint_as_float(w[q] << 16);
    v[2 * q + 1] = __uint_as_float(w[q] & 0xffff0000u);
  }
}
// two floats -> two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __attribute__((ext_vector_type(2))) float f32x2;
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), bf16x2));
}
__device__ __forceinline__ u32x4 pack_bf16x8(const float (&v)[8]) {
  u32x4 w;
#pragma unroll
  for (int q = 0; q < 4; ++q) w[q] = pack_bf16x2(v[2 * q], v[2 * q + 1]);
  return w;
}
__device__ __forceinline__ void buf_store16(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0);
}
__device__ __forceinline__ void buf_store8(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, 0);
}

// ---------------------------------------------------------------- activations
// GELU, tanh form: gelu(z) = z/2 (1 + tanh u), u = sqrt(2/pi)(z + 0.044715 z^3).
// Since (1 + tanh u)/2 = sigmoid(2u), gelu(z) = z * s with s = sigmoid(2u),
// and gelu'(z) = s + 2 z s (1 - s) u'(z), u'(z) = sqrt(2/pi)(1 + 3 * 0.044715 z^2).
// sigmoid(2u) = 1 / (1 + 2^(-2u log2 e)) from the hardware exp2 and
// reciprocal, with -2u log2 e = z (k0 + k1 z^2) folded into two constants.
constexpr double kSqrt2OverPi = 0.7978845608028654;
constexpr double kGeluCubic = 0.044715;
constexpr double kLog2eD = 1.4426950408889634;
constexpr float kLog2e = (float)kLog2eD;
constexpr float kGeluK0 = (float)(-2.0 * kSqrt2OverPi * kLog2eD);
constexpr float kGeluK1 = (float)(-2.0 * kSqrt2OverPi * kLog2eD * kGeluCubic);
// 2 u'(z) = m0 + m1 z^2
constexpr float kGeluM0 = (float)(2.0 * kSqrt2OverPi);
constexpr float kGeluM1 = (float)(6.0 * kSqrt2OverPi * kGeluCubic);

__device__ __forceinline__ float sigmoid_f(float t) {
  float e = __builtin_amdgcn_exp2f(-t * kLog2e);  // +inf for very negative t
  return __builtin_amdgcn_rcpf(1.0f + e);          // rcp(+inf) = 0
}
// sigmoid(2u(z)) for GELU
__device__ __forceinline__ float gelu_sig_f(float z, float z2) {
  const float e = __builtin_amdgcn_exp2f(z * __builtin_fmaf(kGeluK1, z2, kGeluK0));
  return __builtin_amdgcn_rcpf(1.0f + e);
}
__device__ __forceinline__ float gelu_f(float z) { return z * gelu_sig_f(z, z * z); }
__device__ __forceinline__ float gelu_grad_f(float z) {
  const float z2 = z * z;
  const float s = gelu_sig_f(z, z2);
  const float q = __builtin_fmaf(kGeluM1, z2, kGeluM0);  // 2 u'(z)
  // s + z s (1 - s) 2u', grouped so that s = 0 gives 0 for any finite z
  return __builtin_fmaf(s * z, (1.0f - s) * q, s);
}
// SiLU: silu(g) = g sigmoid(g); silu'(g) = sigmoid(g) (1 + g (1 - sigmoid(g))).
__device__ __forceinline__ float silu_f(float g) { return g * sigmoid_f(g); }
__device__ __forceinline__ float silu_grad_f(float g) {
  float s = sigmoid_f(g);
  return s * (1.0f + g * (1.0f - s));
}

// ---------------------------------------------------------------- reductions
__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

}  // namespace tpmlp
