// Device helpers shared by the bridge's HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vlb {

// bf16 is carried as its 16-bit pattern.
__device__ __forceinline__ float bf2f(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// fp32 -> bf16, round to nearest even (the hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f2bf(float f) {
  __bf16 h = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, h);
}

// Activation between the two Linears (vlb_act): exact GELU x*Phi(x) through
// the device erff, the tanh approximation, or none.
__device__ __forceinline__ float activate(float x, int act) {
  if (act == 0) return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f));
  if (act == 1) {
    const float u = 0.79788456080286536f * (x + 0.044715f * x * x * x);
    return 0.5f * x * (1.0f + tanhf(u));
  }
  return x;
}

// Branch-free activations for the GEMM epilogue (one straight-line copy per
// output element, so no branches and little code per element).
//   GELU(x) = x * Phi(x) = 0.5 x (1 + erf(x / sqrt 2)), with erf from
//   Abramowitz & Stegun, Handbook of Mathematical Functions, formula 7.1.26
//   (|error| <= 1.5e-7): erf(z) = 1 - t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) e^{-z^2},
//   t = 1 / (1 + p z), z >= 0, odd extension for z < 0.
//   tanh form: 0.5 x (1 + tanh(u)), u = sqrt(2/pi) (x + 0.044715 x^3), with
//   tanh(u) = 1 - 2 / (e^{2u} + 1).
template <int ACT>
__device__ __forceinline__ float act_fn(float x) {
  if constexpr (ACT == 0) {
    const float z = fabsf(x) * 0.70710678118654752f;
    const float t = __builtin_amdgcn_rcpf(1.0f + 0.3275911f * z);
    const float poly =
        t * (0.254829592f +
             t * (-0.284496736f + t * (1.421413741f + t * (-1.453152027f + t * 1.061405429f))));
    const float e = exp2f(-z * z * 1.4426950408889634f);
    const float erf_abs = 1.0f - poly * e;
    return 0.5f * x * (1.0f + copysignf(erf_abs, x));
  } else if constexpr (ACT == 1) {
    const float u = 0.79788456080286536f * (x + 0.044715f * x * x * x);
    const float th = 1.0f - 2.0f * __builtin_amdgcn_rcpf(exp2f(2.0f * 1.4426950408889634f * u) + 1.0f);
    return 0.5f * x * (1.0f + th);
  } else {
    return x;
  }
}

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static __device__ __forceinline__ float load(float v) { return v; }
  static __device__ __forceinline__ float store(float v) { return v; }
};
template <>
struct Elem<uint16_t> {
  static __device__ __forceinline__ float load(uint16_t v) { return bf2f(v); }
  static __device__ __forceinline__ uint16_t store(float v) { return f2bf(v); }
};

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

}  // namespace vlb
