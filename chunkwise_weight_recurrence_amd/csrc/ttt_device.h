// Device-side helpers shared by the HIP kernels of libttt (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ttt {

// bfloat16 is carried as its raw 16-bit pattern.
typedef uint16_t bf16_t;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even; NaN stays NaN.  gfx950 converts in hardware
// (v_cvt_pk_bf16_f32, two values an instruction, no branch for the NaN case).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
// bf16(a) in the low half, bf16(b) in the high half
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}

// Element load / store of the I/O tensors (q, k, v, o and their gradients).
template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float ld(const float* p, int64_t i) { return p[i]; }
  static __device__ __forceinline__ void st(float* p, int64_t i, float x) { p[i] = x; }
};
template <> struct Elem<bf16_t> {
  static __device__ __forceinline__ float ld(const bf16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
  static __device__ __forceinline__ void st(bf16_t* p, int64_t i, float x) { p[i] = f32_to_bf16(x); }
};

// Logistic function on the hardware exp2 / reciprocal (v_exp_f32, v_rcp_f32: about
// 1 ulp each); saturates to 0 / 1 for large |x|.
__device__ __forceinline__ float sigmoidf_(float x) { return __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

// The single nonlinearity after the fast Linear, and its first two derivatives.
// ACT 0 = identity, 1 = SiLU(z) = z * sigmoid(z), 2 = GELU(z) = z * Phi(z) with
// Phi the standard normal distribution function (exact form, through erf):
// GELU' = Phi + z phi, GELU'' = phi (2 - z^2), phi(z) = exp(-z^2 / 2) / sqrt(2 pi).
__device__ __forceinline__ float normal_cdf_(float z) { return 0.5f + 0.5f * erff(z * 0.70710678118654752f); }
__device__ __forceinline__ float normal_pdf_(float z) { return 0.39894228040143268f * __expf(-0.5f * z * z); }
template <int ACT> __device__ __forceinline__ float act_f(float z) {
  if constexpr (ACT == 1) return z * sigmoidf_(z);
  if constexpr (ACT == 2) return z * normal_cdf_(z);
  return z;
}
template <int ACT> __device__ __forceinline__ float act_df(float z) {
  if constexpr (ACT == 1) {
    float s = sigmoidf_(z);
    return s * (1.0f + z * (1.0f - s));
  }
  if constexpr (ACT == 2) return normal_cdf_(z) + z * normal_pdf_(z);
  return 1.0f;
}
template <int ACT> __device__ __forceinline__ float act_d2f(float z) {
  if constexpr (ACT == 1) {
    float s = sigmoidf_(z);
    return s * (1.0f - s) * (2.0f + z * (1.0f - 2.0f * s));
  }
  if constexpr (ACT == 2) return normal_pdf_(z) * (2.0f - z * z);
  return 0.0f;
}

// The inner loss's signal at the train-view output V_hat = f(z), per feature:
// LOSS 0 = MSE (V_hat - v), 1 = inner product (-v), 2 = L1 (sign(V_hat - v), 0 at
// a tie).  Its derivative in v is -1 for MSE and IP and 0 for L1 (away from ties).
template <int LOSS, int ACT> __device__ __forceinline__ float loss_signal(float z, float v) {
  if constexpr (LOSS == 1) {
    return -v;
  } else {
    const float d = act_f<ACT>(z) - v;
    if constexpr (LOSS == 2) return static_cast<float>((d > 0.0f) - (d < 0.0f));
    return d;
  }
}
template <int LOSS> __device__ __forceinline__ float loss_dsignal_dv() { return LOSS == 2 ? 0.0f : -1.0f; }

// eta_t = 2 * Sigmoid(beta_t + b).
__device__ __forceinline__ float lr_gate(float beta, float b) { return 2.0f * sigmoidf_(beta + b); }

}  // namespace ttt
