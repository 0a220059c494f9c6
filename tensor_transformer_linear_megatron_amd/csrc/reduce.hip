// Sum of the t row-parallel partials on one GPU, in place of the cross-GPU
// all-reduce ("Tensor Parallelism" glossary, "Full definition": partial
// outputs are summed; "Tensor vs Pipeline Parallelism", "Tensor parallelism:
// split inside each layer": the partial results are combined by an
// all-reduce). Pure HBM streaming: (t + 1) M N 4 bytes.
//
// Each thread owns 4 consecutive fp32 columns of one row and adds the ranks
// in order 0, 1, ..., t-1 with 128-bit loads, so the result does not depend
// on the launch shape. Y may alias P_0: every element is read before it is
// written, by the same thread.
#include "tp_internal.h"

namespace tpk {
namespace {

__global__ __launch_bounds__(256) void reduce_kernel(const float* P, int64_t stride, int32_t t,
                                                     int64_t M, int64_t n4, int64_t ldp, float* Y,
                                                     int64_t ldy) {
  const int64_t total = M * n4;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = idx / n4, c = (idx - m * n4) * 4;
    const float* p = P + m * ldp + c;
    float4 s = *reinterpret_cast<const float4*>(p);
    for (int32_t r = 1; r < t; ++r) {
      const float4 v = *reinterpret_cast<const float4*>(p + (int64_t)r * stride);
      s.x += v.x;
      s.y += v.y;
      s.z += v.z;
      s.w += v.w;
    }
    *reinterpret_cast<float4*>(Y + m * ldy + c) = s;
  }
}

}  // namespace

hipError_t launch_reduce(const float* P, int64_t stride, int32_t t, int64_t M, int64_t N,
                         int64_t ldp, float* Y, int64_t ldy, hipStream_t s) {
  const int64_t n4 = N / 4, total = M * n4;
  if (total == 0) return hipSuccess;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, s, P, stride, t, M, n4,
                     ldp, Y, ldy);
  return hipGetLastError();
}

}  // namespace tpk
