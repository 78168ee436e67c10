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
