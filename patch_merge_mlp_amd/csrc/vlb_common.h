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

// Two fp32 values -> one dword of two bf16 (a in the low half), round to
// nearest even: one packed hardware conversion.
__device__ __forceinline__ uint32_t f2bf2(float a, float b) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const f32x2 t = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(t, bf16x2));
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
//   GELU(x) = x * Phi(x) = max(x, 0) - |x| * Phi(-|x|), with the Gaussian tail
//   Phi(-a) = erfc(a / sqrt 2) / 2 evaluated as 2^(-h(a)), h a degree-4
//   polynomial fitted as accurately as the bf16 output needs
//   (fit_gelu_poly.py beside this file: near-minimax in the relative error
//   where |GELU| > 1e-3, in the absolute error past that; a is clamped to 5.5,
//   where Phi(-5.5) ~ 2e-8).  Evaluated in fp32 the result is within 2.8e-4
//   relatively of x * Phi(x) wherever |GELU(x)| > 1e-3 (bf16 rounds to 2^-9
//   relatively) and 4.1e-5 absolutely on [-12, 12]: one exp2, no division.
//   tanh form: 0.5 x (1 + tanh(u)), u = sqrt(2/pi) (x + 0.044715 x^3), with
//   tanh(u) = 1 - 2 / (e^{2u} + 1).
// Phi(-|x|) = 2^(-h(|x|)) (no denormal range here).
__device__ __forceinline__ float gauss_tail(float x) {
  const float a = fminf(fabsf(x), 5.5f);
  float h = -0.00311285374f;
  h = fmaf(h, a, 0.0401906446f);
  h = fmaf(h, a, 0.473863691f);
  h = fmaf(h, a, 1.14503634f);
  h = fmaf(h, a, 1.00040841f);
  return __builtin_amdgcn_exp2f(-h);
}

template <int ACT>
__device__ __forceinline__ float act_fn(float x) {
  if constexpr (ACT == 0) {
    return fmaf(-fabsf(x), gauss_tail(x), fmaxf(x, 0.0f));
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

// 16-byte store marked non-temporal (streamed: the data is not read again
// soon, so it need not stay in the caches).
__device__ __forceinline__ void store_nt(uint4 *p, uint4 v) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 t = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(t, reinterpret_cast<u32x4 *>(p));
}

// 16-byte load marked non-temporal (data read once: it need not displace
// what the caches hold for the kernels that follow).
__device__ __forceinline__ uint4 load_nt(const uint4 *p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}
__device__ __forceinline__ uint32_t load_nt(const uint32_t *p) {
  return __builtin_nontemporal_load(p);
}

// Lane exchange inside rows of 16 lanes (DPP control CTRL).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, true));
}

// Sum over the 64 lanes of a wave, the same value in every lane.  The whole
// wave must be active.  Inside each row of 16 lanes: lane ^ 1, lane ^ 2 (quad
// permutes), then the mirrored 8-lane halves and the mirrored rows; every
// lane of a row then holds the row's sum (each step adds the same two values
// in both partners), and the four row sums are added in a fixed order.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f<0x141>(v);  // row_half_mirror
  v += dpp_f<0x140>(v);  // row_mirror
  const int b = __float_as_int(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(b, 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(b, 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(b, 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(b, 48));
  return (r0 + r1) + (r2 + r3);
}

}  // namespace vlb
