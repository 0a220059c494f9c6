// Sum of the t row-parallel partials on one GPU, in place of the cross-GPU
// all-reduce ("Tensor Parallelism" glossary, "Full definition": partial
// outputs are summed; "Tensor vs Pipeline Parallelism", "Tensor parallelism:
// split inside each layer": the partial results are combined by an
// all-reduce). Pure HBM streaming: (t + 1) M N 4 bytes.
//
// Each thread owns 4 consecutive fp32 columns of one row and adds the ranks
// in order 0, 1, ..., t-1 with 128-bit loads, so the result does not depend
// on the launch shape. Y may alias P_0: every element is read before it is
// written, by the same thread. The sequence-parallel form runs the same
// kernel on one rank's block of token rows.
//
// The row gather ("AI Infrastructure series, Part 5", "What about MoE models
// and very long prompts?": sequence parallelism splits the parts of a layer
// that tensor parallelism leaves whole along the sequence) stacks the ranks'
// bf16 row blocks in rank order with 128-bit copies: 2 M N 2 bytes.
#include "tp_internal.h"

namespace tpk {
namespace {

typedef float f32x4v_t __attribute__((ext_vector_type(4)));

// One partial's 4 columns, read once: non-temporal.
__device__ __forceinline__ f32x4v_t load_part(const float* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const f32x4v_t*>(p));
}

// The loads of up to 8 ranks are issued before their sum, so a thread keeps
// that many 16-byte reads in flight; the additions still run in rank order.
__global__ __launch_bounds__(256) void reduce_kernel(const float* P, int64_t stride, int32_t t,
                                                     int64_t M, int64_t n4, int64_t ldp, float* Y,
                                                     int64_t ldy) {
  const int64_t total = M * n4;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = idx / n4, c = (idx - m * n4) * 4;
    const float* p = P + m * ldp + c;
    f32x4v_t s = load_part(p);
    for (int32_t r0 = 1; r0 < t; r0 += 8) {
      const int32_t n = t - r0 < 8 ? t - r0 : 8;
      f32x4v_t v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j < n) v[j] = load_part(p + (int64_t)(r0 + j) * stride);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j < n) s += v[j];
    }
    *reinterpret_cast<f32x4v_t*>(Y + m * ldy + c) = s;
  }
}

// Row gather of bf16 activations: thread idx copies 16 bytes (8 values) of
// output row m = s Mt + i from row i of block s.
__global__ __launch_bounds__(256) void gather_kernel(const uint16_t* Xs, int64_t stride, int64_t Mt,
                                                     int64_t rows, int64_t n8, int64_t ldb,
                                                     uint16_t* X, int64_t ldx) {
  const int64_t total = rows * n8;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = idx / n8, c = (idx - m * n8) * 8;
    const int64_t s = m / Mt, i = m - s * Mt;
    *reinterpret_cast<uint4*>(X + m * ldx + c) =
        *reinterpret_cast<const uint4*>(Xs + s * stride + i * ldb + c);
  }
}

}  // namespace

hipError_t launch_gather(const uint16_t* Xs, int64_t stride, int32_t t, int64_t Mt, int64_t N,
                         int64_t ldb, uint16_t* X, int64_t ldx, hipStream_t s) {
  const int64_t n8 = N / 8, rows = (int64_t)t * Mt, total = rows * n8;
  if (total == 0) return hipSuccess;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)blocks), dim3(256), 0, s, Xs, stride, Mt, rows,
                     n8, ldb, X, ldx);
  return hipGetLastError();
}

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
