// Ordered float32 sums of equally shaped buffers.
//
//  * sum_kernel: out = p_0 + p_1 + ... + p_{t-1}, the local stand-in for the
//    tensor-parallel all-reduce (the ranks' partial outputs are added,
//    "大模型训练" notes §3.1).
//  * splitk_kernel: the sum of the split-K slices of one product, finished with
//    that product's epilogue (float32 store, GeLU, bf16 store or dGeLU), so that
//    a product split along K ends exactly like an unsplit one.
//
// Both are HBM-bound: each lane moves 16-byte vectors of float32 (4 elements),
// and parts are added left to right so that the result does not depend on the
// launch shape.

#include "../../include/tpmlp.h"
#include "common.h"
#include "epilogue.h"

namespace tpmlp {
namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint16_t u16x4_t __attribute__((ext_vector_type(4)));

struct SumArgs {
  const float* parts[TPMLP_MAX_SHARDS];
  int n_parts;
  int64_t n4;  // number of float4 vectors
  float* out;
};

__global__ void __launch_bounds__(256) sum_kernel(SumArgs a) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < a.n4; j += stride) {
    f32x4_t s = reinterpret_cast<const f32x4_t*>(a.parts[0])[j];
    for (int i = 1; i < a.n_parts; ++i) s += reinterpret_cast<const f32x4_t*>(a.parts[i])[j];
    __builtin_nontemporal_store(s, reinterpret_cast<f32x4_t*>(a.out) + j);
  }
}

struct SplitArgs {
  const float* part;  // splits x n float32, slice i at part + i * n
  int splits;
  int64_t n;          // elements per slice (multiple of 4)
  void* out;          // float* (EPI_F32) or uint16_t*
  uint16_t* out2;     // second bf16 output or null
  const uint16_t* aux;
};

template <int EPI>
__global__ void __launch_bounds__(256) splitk_kernel(SplitArgs a) {
  const int64_t n4 = a.n / 4;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n4; j += stride) {
    f32x4_t s = reinterpret_cast<const f32x4_t*>(a.part)[j];
    for (int i = 1; i < a.splits; ++i) s += reinterpret_cast<const f32x4_t*>(a.part + i * a.n)[j];
    if (EPI == EPI_F32) {
      reinterpret_cast<f32x4_t*>(a.out)[j] = s;
    } else if (EPI == EPI_GELU) {
      u16x4_t g, p;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        g[e] = epi_gelu(s[e]);
        p[e] = f32_to_bf16(s[e]);
      }
      reinterpret_cast<u16x4_t*>(a.out)[j] = g;
      if (a.out2) reinterpret_cast<u16x4_t*>(a.out2)[j] = p;
    } else if (EPI == EPI_BF16) {
      u16x4_t p;
#pragma unroll
      for (int e = 0; e < 4; ++e) p[e] = f32_to_bf16(s[e]);
      reinterpret_cast<u16x4_t*>(a.out)[j] = p;
    } else {  // EPI_DGELU
      const u16x4_t pb = reinterpret_cast<const u16x4_t*>(a.aux)[j];
      u16x4_t dp, g;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const DGelu r = epi_dgelu(s[e], pb[e]);
        dp[e] = r.dp;
        g[e] = r.g;
      }
      reinterpret_cast<u16x4_t*>(a.out)[j] = dp;
      reinterpret_cast<u16x4_t*>(a.out2)[j] = g;
    }
  }
}

int grid_for(int64_t n4) {
  const int64_t want = (n4 + 255) / 256;
  return (int)(want < 4096 ? (want > 0 ? want : 1) : 4096);
}

}  // namespace

hipError_t launch_sum(const float* const* parts, int n_parts, float* out, int64_t n, hipStream_t stream) {
  if (!parts || n_parts < 1 || n_parts > TPMLP_MAX_SHARDS || (n & 3)) return hipErrorInvalidValue;
  SumArgs a;
  for (int i = 0; i < n_parts; ++i) a.parts[i] = parts[i];
  a.n_parts = n_parts;
  a.n4 = n / 4;
  a.out = out;
  hipLaunchKernelGGL(sum_kernel, dim3(grid_for(a.n4)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_splitk_epilogue(Epi epi, const float* part, int splits, int64_t n, void* out, uint16_t* out2,
                                  const uint16_t* aux, hipStream_t stream) {
  if (!part || splits < 1 || (n & 3)) return hipErrorInvalidValue;
  SplitArgs a{part, splits, n, out, out2, aux};
  const dim3 grid(grid_for(n / 4)), block(256);
  switch (epi) {
    case EPI_F32: hipLaunchKernelGGL(splitk_kernel<EPI_F32>, grid, block, 0, stream, a); break;
    case EPI_GELU: hipLaunchKernelGGL(splitk_kernel<EPI_GELU>, grid, block, 0, stream, a); break;
    case EPI_BF16: hipLaunchKernelGGL(splitk_kernel<EPI_BF16>, grid, block, 0, stream, a); break;
    case EPI_DGELU: hipLaunchKernelGGL(splitk_kernel<EPI_DGELU>, grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace tpmlp
