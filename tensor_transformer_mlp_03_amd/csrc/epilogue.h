// Element-wise epilogue arithmetic shared by the GEMM kernel and the split-K
// reduction, so that a product finished in either place rounds the same way.
//
// GeLU(p) = p Phi(p) with Phi the standard normal CDF; its derivative is
// Phi(p) + p phi(p), phi the standard normal density (GeLU between the MLP's two
// GEMMs: QLM page §2.1.2.2 part 3, "大模型训练" notes §3.1; the exact form
// p Phi(p) is the reading taken of a formula the pages do not print).
//
// Phi is evaluated through erfc with the rational-times-Gaussian approximation
// of Abramowitz and Stegun, Handbook of Mathematical Functions, formula 7.1.26
// (C. Hastings' fit): for z >= 0,
//   erfc(z) = (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-z^2),  t = 1/(1 + p z),
// with |error| <= 1.5e-7 in erf.  Phi(x) = 1 - erfc(x/sqrt 2)/2 for x >= 0 and
// erfc(|x|/sqrt 2)/2 for x < 0.  exp(-x^2/2) is shared with phi(x).  The error
// is far below the bf16 rounding (2^-9 relative) that every epilogue output
// receives; the tests pin it against float64 erf.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace tpmlp {

__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  // Round to nearest even (v_cvt_pk_bf16_f32).
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __builtin_bit_cast(float, static_cast<uint32_t>(b) << 16);
}

// The Gaussian tail of x: he = erfc(|x|/sqrt 2)/2, i.e. Phi(-|x|), and
// e = exp(-x^2/2).  The fit's coefficients enter halved, so that the product
// of the polynomial and e is he itself; exp(-x^2/2) is computed as
// exp2(x^2 * (-log2(e)/2)) with the hardware exp2.
struct NormalTail {
  float he;  // Phi(-|x|)
  float e;   // exp(-x^2/2) = sqrt(2 pi) phi(x)
};

__device__ __forceinline__ NormalTail normal_tail(float x) {
  constexpr float P = 0.3275911f;
  constexpr float A1 = 0.254829592f, A2 = -0.284496736f, A3 = 1.421413741f, A4 = -1.453152027f,
                  A5 = 1.061405429f;
  constexpr float INV_SQRT2 = 0.70710678118654752f, LOG2E = 1.4426950408889634f;
  const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(fabsf(x), P * INV_SQRT2, 1.0f));
  const float e = __builtin_amdgcn_exp2f((x * x) * (-0.5f * LOG2E));
  const float q = t * (0.5f * A1 + t * (0.5f * A2 + t * (0.5f * A3 + t * (0.5f * A4 + t * (0.5f * A5)))));
  return NormalTail{q * e, e};
}

// The same tail with the density itself: he = Phi(-|x|) and f = phi(x) =
// exp(-x^2/2) / sqrt(2 pi).  log2(1/sqrt(2 pi)) enters the exponent and the
// fit's coefficients carry sqrt(2 pi)/2 instead of 1/2, so that the polynomial
// times f is he; GeLU' then takes p phi(p) in one fused multiply-add.
struct NormalTailDensity {
  float he;  // Phi(-|x|)
  float f;   // phi(x)
};

__device__ __forceinline__ NormalTailDensity normal_tail_density(float x) {
  constexpr float P = 0.3275911f;
  constexpr double C = 1.2533141373155003;  // sqrt(2 pi) / 2
  constexpr float A1 = (float)(C * 0.254829592), A2 = (float)(C * -0.284496736), A3 = (float)(C * 1.421413741),
                  A4 = (float)(C * -1.453152027), A5 = (float)(C * 1.061405429);
  constexpr float INV_SQRT2 = 0.70710678118654752f, LOG2E = 1.4426950408889634f;
  constexpr float LOG2_INV_SQRT_2PI = -1.3257480647361594f;  // -log2(2 pi) / 2
  const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(fabsf(x), P * INV_SQRT2, 1.0f));
  const float f = __builtin_amdgcn_exp2f(__builtin_fmaf(x * x, -0.5f * LOG2E, LOG2_INV_SQRT_2PI));
  const float q = t * (A1 + t * (A2 + t * (A3 + t * (A4 + t * A5))));
  return NormalTailDensity{q * f, f};
}

// max(x, 0) as a signed-integer max of the bits: a float with the sign bit clear
// orders as a non-negative integer, one with it set as a negative integer (and
// maps to +0).  Unlike fmaxf it needs no canonicalizing of x first.
__device__ __forceinline__ float relu_bits(float x) {
  return __builtin_bit_cast(float, max(__builtin_bit_cast(int, x), 0));
}

// GeLU(x) in float32, as x Phi(x) = max(x, 0) - |x| Phi(-|x|), which holds for
// either sign of x.
__device__ __forceinline__ float gelu_f32(float x) {
  const NormalTail n = normal_tail(x);
  return __builtin_fmaf(-fabsf(x), n.he, relu_bits(x));
}

// G = GeLU(acc) -> bf16.
__device__ __forceinline__ uint16_t epi_gelu(float acc) { return f32_to_bf16(gelu_f32(acc)); }

// From the stored bf16 pre-activation p and the accumulated dG: dP = dG GeLU'(p)
// and G = GeLU(p), both bf16.
struct DGelu {
  uint16_t dp, g;
};
__device__ __forceinline__ DGelu epi_dgelu(float dg, uint16_t p_bits) {
  const float p = bf16_to_f32(p_bits);
  const NormalTailDensity n = normal_tail_density(p);
  const float cdf = p >= 0.0f ? 1.0f - n.he : n.he;  // Phi(p)
  const float grad = __builtin_fmaf(p, n.f, cdf);    // Phi(p) + p phi(p)
  return DGelu{f32_to_bf16(dg * grad), f32_to_bf16(p * cdf)};
}

// dP = dG GeLU'(p) in float32 (the FP8 path's dGeLU, which needs no G).
__device__ __forceinline__ float dgelu_f32(float dg, uint16_t p_bits) {
  const float p = bf16_to_f32(p_bits);
  const NormalTailDensity n = normal_tail_density(p);
  const float cdf = p >= 0.0f ? 1.0f - n.he : n.he;
  return dg * __builtin_fmaf(p, n.f, cdf);
}

// ---------------------------------------------------------------------------
// FP8 operands ("大模型训练" notes §6.1: E4M3, 4 exponent and 3 mantissa bits,
// range +-448; E5M2, 5 and 2 bits, range +-57344) under per-tensor scaling: a
// tensor's scale is s = amax / FMAX (1 for an all-zero tensor), its codes are
// fp8(x * (1 / s)) with the product in float32, saturated to +-FMAX and rounded
// to nearest even by the conversion instruction; in a product each code stands
// for code * s.  Every consumer of a tensor derives s and 1/s from the same
// amax bits with the same two correctly rounded divisions, so the scales agree
// bit for bit across kernels.
// ---------------------------------------------------------------------------
constexpr float FP8_E4M3_MAX = 448.0f;
constexpr float FP8_E5M2_MAX = 57344.0f;

__device__ __forceinline__ float fp8_fmax(int fmt) { return fmt ? FP8_E5M2_MAX : FP8_E4M3_MAX; }

// Max over the 64 lanes of a wave.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// An amax slot (AMAX_SUB etc. in common.h) is `nsub` 32-bit words of float
// bits; the values are >= 0, so unsigned order is float order.

// Max over a wave of per-lane values (all >= 0), added to one word of the slot
// by lane 0 (nsub a power of two).
__device__ __forceinline__ void slot_max(uint32_t* slot, int nsub, float lane_max) {
  const float m = wave_max(lane_max);
  if ((threadIdx.x & 63) == 0) {
    const int sub = (int)(blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)) & (nsub - 1);
    atomicMax(slot + sub * AMAX_SUB_STRIDE, __builtin_bit_cast(uint32_t, m));
  }
}

// Running extremes of values v, for max|v| or max|GeLU(v)| without a GeLU per
// value: GeLU rises on v >= 0, so there the largest v gives the max; on v < 0,
// |GeLU| rises towards its one maximum at v = -GELU_MODE from either side, so the
// largest v below the mode and the smallest v between it and 0 hold the max
// there.  Branch-free; a value of 0 moves nothing (an invalid element enters as
// 0).  The initial -1e30 has GeLU 0.
struct AmaxTrack {
  static constexpr float GELU_MODE = 0.7517915f;
  float v_max = 0.0f, v_min = 0.0f, g_left = -1e30f, g_right = 0.0f;
  __device__ __forceinline__ void add(float v) {
    v_max = fmaxf(v_max, v);
    v_min = fminf(v_min, v);
    g_left = v < -GELU_MODE ? fmaxf(g_left, v) : g_left;
    g_right = (v >= -GELU_MODE && v < 0.0f) ? fminf(g_right, v) : g_right;
  }
  __device__ __forceinline__ float result(bool of_gelu) const {
    return of_gelu ? fmaxf(gelu_f32(v_max), fmaxf(fabsf(gelu_f32(g_left)), fabsf(gelu_f32(g_right))))
                   : fmaxf(v_max, -v_min);
  }
};

__device__ __forceinline__ float slot_read(const uint32_t* slot, int nsub) {
  uint32_t m = 0;
  if (nsub == AMAX_SUB) {  // the workspace slots: all loads issued before the first wait
#pragma unroll
    for (int i = 0; i < AMAX_SUB; ++i) m = max(m, slot[i * AMAX_SUB_STRIDE]);
  } else {
    for (int i = 0; i < nsub; ++i) m = max(m, slot[i * AMAX_SUB_STRIDE]);
  }
  return __builtin_bit_cast(float, m);
}

// Scale of a tensor from its amax, and from its amax slot.
__device__ __forceinline__ float fp8_scale_of(float amax, float fmax) { return amax == 0.0f ? 1.0f : amax / fmax; }

__device__ __forceinline__ float fp8_scale(const uint32_t* slot, int nsub, float fmax) {
  return fp8_scale_of(slot_read(slot, nsub), fmax);
}

// Four float32 values, already multiplied by 1/s, to four FP8 codes (byte e of
// the result holds value e): clamped to +-FMAX, then converted (nearest, ties to
// even).  fmt 0: E4M3, 1: E5M2.
__device__ __forceinline__ uint32_t fp8_pack4(float a, float b, float c, float d, int fmt) {
  const float m = fp8_fmax(fmt);
  a = fminf(fmaxf(a, -m), m);
  b = fminf(fmaxf(b, -m), m);
  c = fminf(fmaxf(c, -m), m);
  d = fminf(fmaxf(d, -m), m);
  int v;
  if (fmt == 0) {
    v = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    v = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, v, true);
  } else {
    v = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
    v = __builtin_amdgcn_cvt_pk_bf8_f32(c, d, v, true);
  }
  return (uint32_t)v;
}

}  // namespace tpmlp
