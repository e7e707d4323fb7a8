// Element-wise kernels of the FP8 path: per-tensor amax and the quantization of
// bf16 tensors (or of the GeLU of a bf16 pre-activation) to FP8 codes, row-major
// or transposed.
//
// The scaling is per tensor ("大模型训练" notes §6.1 gives the two formats, E4M3
// and E5M2, and no recipe; the one taken is current scaling): a tensor's amax is
// collected into a 32-bit slot (float bits; amax >= 0, so unsigned order is float
// order) by one atomic max per wave, and every kernel that quantizes or consumes
// the tensor derives the scale from that slot with fp8_scale (epilogue.h).
// All loads and stores are 16-byte vectors; buffers are 16-byte aligned and rows
// hold multiples of 16 elements.

#include <algorithm>

#include "common.h"
#include "epilogue.h"

namespace tpmlp {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

}  // namespace

namespace kern {

__global__ void __launch_bounds__(256) fp8_zero_kernel(Fp8ZeroArgs a) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < a.n; i += gridDim.x * 256) a.p[i] = 0u;
}

// max |x| over a bf16 [R][C] tensor with rows of ld elements.
// Each workgroup reduces its lanes' maxima through LDS and adds one atomic max
// to a word of the slot: atomics on one address serialize, so their count (the
// grid size, at most AMAX_BLOCKS) is kept small and spread over the slot's words.
constexpr int AMAX_BLOCKS = 1024;

__device__ __forceinline__ float amax8(const u32x4_t x, float m) {
#pragma unroll
  for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(bf16_to_f32((uint16_t)(x[e / 2] >> (16 * (e % 2))))));
  return m;
}

__global__ void __launch_bounds__(256) fp8_amax_kernel(Fp8AmaxArgs a) {
  __shared__ float red[4];
  float m = 0.0f;
  const int64_t stride = (int64_t)gridDim.x * 256;
  if (a.ld == a.C) {  // contiguous rows: one flat range of 16-byte vectors
    const int64_t nv = a.R * a.C / 8;
    const u32x4_t* in = reinterpret_cast<const u32x4_t*>(a.in);
    int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x;
    for (; v + stride < nv; v += 2 * stride) {  // two loads in flight per lane
      const u32x4_t x0 = in[v], x1 = in[v + stride];
      m = amax8(x1, amax8(x0, m));
    }
    if (v < nv) m = amax8(in[v], m);
  } else {
    const int64_t vpr = a.C / 8;  // 16-byte vectors per row
    const int64_t nv = a.R * vpr;
    for (int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x; v < nv; v += stride) {
      const int64_t r = v / vpr, c = (v - r * vpr) * 8;
      m = amax8(*reinterpret_cast<const u32x4_t*>(a.in + r * a.ld + c), m);
    }
  }
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0)
    atomicMax(a.slot + (blockIdx.x & (a.nsub - 1)) * AMAX_SUB_STRIDE,
              __builtin_bit_cast(uint32_t, fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]))));
}

// out[r][c] = fp8(x[r][c] / s) (x = in, or GeLU(in)); 16 elements per thread.
__global__ void __launch_bounds__(256) fp8_quant_kernel(Fp8QuantArgs a) {
  const float inv = 1.0f / fp8_scale(a.slot, a.nsub, fp8_fmax(a.fmt));
  const int64_t vpr = a.C / 16;
  const int64_t nv = a.R * vpr;
  for (int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x; v < nv; v += (int64_t)gridDim.x * 256) {
    const int64_t r = v / vpr, c = (v - r * vpr) * 16;
    const u32x4_t x0 = *reinterpret_cast<const u32x4_t*>(a.in + r * a.ld_in + c);
    const u32x4_t x1 = *reinterpret_cast<const u32x4_t*>(a.in + r * a.ld_in + c + 8);
    float f[16];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      f[e] = bf16_to_f32((uint16_t)(x0[e / 2] >> (16 * (e % 2))));
      f[8 + e] = bf16_to_f32((uint16_t)(x1[e / 2] >> (16 * (e % 2))));
    }
    u32x4_t o;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      float g[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) g[e] = (a.gelu ? gelu_f32(f[4 * w + e]) : f[4 * w + e]) * inv;
      o[w] = fp8_pack4(g[0], g[1], g[2], g[3], a.fmt);
    }
    *reinterpret_cast<u32x4_t*>(a.out + r * a.ld_out + c) = o;
  }
}

// out[c][r] = fp8(x[r][c] / s): one 64 x 64 tile per workgroup, staged in LDS as
// bytes at a 80-byte pitch (16-byte aligned rows for the 16-byte reads).  With
// out2 set, the same codes also go to out2[r][c] (row-major), from the one read.
__global__ void __launch_bounds__(256) fp8_quant_t_kernel(Fp8QuantArgs a) {
  constexpr int PITCH = 80;
  __shared__ __attribute__((aligned(16))) uint8_t tile[64 * PITCH];
  const float inv = 1.0f / fp8_scale(a.slot, a.nsub, fp8_fmax(a.fmt));
  const int64_t r0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * 64;
  const int t = threadIdx.x;
  {
    const int r = t >> 2, cs = 16 * (t & 3);  // row r, columns cs .. cs+15 of the tile
    float f[16];
    if (r0 + r < a.R && c0 + cs < a.C) {
      const uint16_t* p = a.in + (r0 + r) * a.ld_in + c0 + cs;
      const u32x4_t x0 = *reinterpret_cast<const u32x4_t*>(p);
      const u32x4_t x1 = *reinterpret_cast<const u32x4_t*>(p + 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        f[e] = bf16_to_f32((uint16_t)(x0[e / 2] >> (16 * (e % 2))));
        f[8 + e] = bf16_to_f32((uint16_t)(x1[e / 2] >> (16 * (e % 2))));
      }
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) f[e] = 0.0f;
    }
    u32x4_t o;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      float g[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) g[e] = (a.gelu ? gelu_f32(f[4 * w + e]) : f[4 * w + e]) * inv;
      const uint32_t q = fp8_pack4(g[0], g[1], g[2], g[3], a.fmt);
      o[w] = q;
#pragma unroll
      for (int e = 0; e < 4; ++e) tile[(cs + 4 * w + e) * PITCH + r] = (uint8_t)(q >> (8 * e));
    }
    if (a.out2 && r0 + r < a.R && c0 + cs < a.C)
      *reinterpret_cast<u32x4_t*>(a.out2 + (r0 + r) * a.ld_out2 + c0 + cs) = o;
  }
  __syncthreads();
  {
    const int c = t >> 2, rs = 16 * (t & 3);  // output row c (input column), input rows rs .. rs+15
    if (c0 + c < a.C && r0 + rs < a.R)
      *reinterpret_cast<u32x4_t*>(a.out + (c0 + c) * a.ld_out + r0 + rs) =
          *reinterpret_cast<const u32x4_t*>(tile + c * PITCH + rs);
  }
}

}  // namespace kern

hipError_t launch_fp8_zero(uint32_t* p, int n, hipStream_t s) {
  const int blocks = std::max(1, std::min(64, (n + 255) / 256));
  return launch_kernel(kern::fp8_zero_kernel, dim3(blocks), dim3(256), s, Fp8ZeroArgs{p, n});
}

hipError_t launch_fp8_amax(const uint16_t* in, int64_t R, int64_t C, int64_t ld, uint32_t* slot, int nsub,
                           hipStream_t s) {
  const int64_t nv = R * (C / 8);
  const int blocks = (int)std::min<int64_t>(kern::AMAX_BLOCKS, std::max<int64_t>(1, (nv + 511) / 512));
  return launch_kernel(kern::fp8_amax_kernel, dim3(blocks), dim3(256), s, Fp8AmaxArgs{in, R, C, ld, slot, nsub});
}

hipError_t launch_fp8_quant(const uint16_t* in, int64_t R, int64_t C, int64_t ld_in, bool gelu, int fmt,
                            const uint32_t* slot, int nsub, uint8_t* out, int64_t ld_out, bool transpose, hipStream_t s,
                            uint8_t* out_rows, int64_t ld_rows) {
  const Fp8QuantArgs a{in, out, R, C, ld_in, ld_out, gelu ? 1 : 0, fmt, slot, nsub, transpose ? out_rows : nullptr,
                       ld_rows};
  if (transpose)
    return launch_kernel(kern::fp8_quant_t_kernel, dim3((unsigned)((C + 63) / 64), (unsigned)((R + 63) / 64)),
                         dim3(256), s, a);
  const int64_t nv = R * (C / 16);
  const int blocks = (int)std::min<int64_t>(8192, std::max<int64_t>(1, (nv + 255) / 256));
  return launch_kernel(kern::fp8_quant_kernel, dim3(blocks), dim3(256), s, a);
}

}  // namespace tpmlp
