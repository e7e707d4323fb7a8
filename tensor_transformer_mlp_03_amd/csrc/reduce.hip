// Ordered float32 sums of equally shaped buffers: the local stand-in for the
// tensor-parallel all-reduce (the ranks' partial outputs are added, "大模型训练"
// notes §3.1) and the reduction of split-K partials.  HBM-bound: each lane moves
// 16-byte vectors, parts are added left to right so the result does not depend
// on the launch shape.

#include "../../include/tpmlp.h"
#include "common.h"

namespace tpmlp {
namespace {

struct SumArgs {
  const float* parts[TPMLP_MAX_SHARDS];
  int n_parts;
  int64_t n4;  // number of float4 vectors
  float* out;
};

__global__ void __launch_bounds__(256) sum_kernel(SumArgs a) {
  typedef float f32x4_t __attribute__((ext_vector_type(4)));
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < a.n4; j += stride) {
    f32x4_t s = reinterpret_cast<const f32x4_t*>(a.parts[0])[j];
    for (int i = 1; i < a.n_parts; ++i) s += reinterpret_cast<const f32x4_t*>(a.parts[i])[j];
    __builtin_nontemporal_store(s, reinterpret_cast<f32x4_t*>(a.out) + j);
  }
}

}  // namespace

hipError_t launch_sum(const float* const* parts, int n_parts, float* out, int64_t n,
                      hipStream_t stream) {
  if (!parts || n_parts < 1 || n_parts > TPMLP_MAX_SHARDS || (n & 3)) return hipErrorInvalidValue;
  SumArgs a;
  for (int i = 0; i < n_parts; ++i) a.parts[i] = parts[i];
  a.n_parts = n_parts;
  a.n4 = n / 4;
  a.out = out;
  const int64_t want = (a.n4 + 255) / 256;
  const int blocks = (int)(want < 4096 ? (want > 0 ? want : 1) : 4096);
  hipLaunchKernelGGL(sum_kernel, dim3(blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace tpmlp
