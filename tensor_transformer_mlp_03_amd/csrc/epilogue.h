// Element-wise epilogue arithmetic shared by the GEMM kernel and the split-K
// reduction, so that a product finished in either place rounds the same way.
//
// GeLU(p) = p Phi(p) with Phi the standard normal CDF written with erf; its
// derivative is Phi(p) + p phi(p), phi the standard normal density (GeLU between
// the MLP's two GEMMs: QLM page §2.1.2.2 part 3, "大模型训练" notes §3.1; the exact
// erf form is the reading taken of a formula the pages do not print).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tpmlp {

__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  // Round to nearest even (v_cvt_pk_bf16_f32).
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __builtin_bit_cast(float, static_cast<uint32_t>(b) << 16);
}

__device__ __forceinline__ float phi_cdf(float p) { return 0.5f + 0.5f * erff(p * 0.70710678118654752f); }

// G = GeLU(acc) -> bf16
__device__ __forceinline__ uint16_t epi_gelu(float acc) { return f32_to_bf16(acc * phi_cdf(acc)); }

// From the stored bf16 pre-activation p and the accumulated dG: dP = dG GeLU'(p)
// and G = GeLU(p), both bf16.
struct DGelu {
  uint16_t dp, g;
};
__device__ __forceinline__ DGelu epi_dgelu(float dg, uint16_t p_bits) {
  const float p = bf16_to_f32(p_bits);
  const float cdf = phi_cdf(p);
  const float pdf = 0.39894228040143268f * __expf(-0.5f * p * p);
  return DGelu{f32_to_bf16(dg * (cdf + p * pdf)), f32_to_bf16(p * cdf)};
}

}  // namespace tpmlp
