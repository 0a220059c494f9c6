// Decode path (M <= 64 tokens): Y = X W_shard streams every weight byte once
// and is bound by HBM bandwidth ("AI Infrastructure series, Part 5",
// "Reason 2": in decode every token needs a read of every weight; a rank of t
// reads 1/t of them).
//
// Design for gfx950:
//  * The weight is the MFMA A operand (16 output columns x 32 k per packed
//    1 KiB tile), the tokens are the B operand (32 k x 16 tokens, zero rows
//    past M). One MFMA per tile and 16-token block, so the matrix cores have
//    ample headroom even at M = 64 where a VALU dot product would not keep up
//    with HBM.
//  * Every weight load is one wavefront-wide 1 KiB contiguous dwordx4 load.
//  * A workgroup owns T adjacent packed tiles (T = 2 pairs gate and up) for
//    the whole K; its S wavefronts split K (step ks goes to wave ks mod S),
//    keep fp32 accumulators in registers and are reduced through LDS in wave
//    order -- deterministic, no atomics, no second pass.
//  * The epilogue (bf16 rounding, SwiGLU, or fp32 partial) runs once the full
//    K sum is known, in registers.
#include "tp_internal.h"

namespace tpk {
namespace {

template <int MB, int T, int EPI, int U>
__global__ __launch_bounds__(1024) void gemv_kernel(LinearArgs a) {
  extern __shared__ f32x4_t red[];  // [S][T][MB][64]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, S = blockDim.x >> 6;
  const int g = lane >> 4, i = lane & 15;
  const int64_t tile0 = (int64_t)blockIdx.x * T;
  const int64_t ksteps = a.ksteps;
  const uint4* wp = a.W + tile0 * ksteps * kTileU4 + lane;

  const uint16_t* xrow[MB];
  bool mvalid[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int64_t m = mb * 16 + i;
    mvalid[mb] = m < a.M;
    xrow[mb] = a.X + (mvalid[mb] ? m : 0) * a.ldx + g * 8;
  }

  f32x4_t acc[T][MB];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[t][mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const uint4 zero = {0u, 0u, 0u, 0u};
  int64_t ks = wave;
  for (; ks + (int64_t)(U - 1) * S < ksteps; ks += (int64_t)U * S) {
    uint4 w[U][T], x[U][MB];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int t = 0; t < T; ++t) w[u][t] = wp[((int64_t)t * ksteps + ks + u * S) * kTileU4];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int64_t k = (ks + u * S) * kTileK;
        uint4 v = zero;
        if (mvalid[mb] && k + g * 8 < a.K) v = *reinterpret_cast<const uint4*>(xrow[mb] + k);
        x[u][mb] = v;
      }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[t][mb] = mfma_16x16x32(w[u][t], x[u][mb], acc[t][mb]);
  }
  for (; ks < ksteps; ks += S) {
    uint4 w[T], x[MB];
#pragma unroll
    for (int t = 0; t < T; ++t) w[t] = wp[((int64_t)t * ksteps + ks) * kTileU4];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int64_t k = ks * kTileK;
      uint4 v = zero;
      if (mvalid[mb] && k + g * 8 < a.K) v = *reinterpret_cast<const uint4*>(xrow[mb] + k);
      x[mb] = v;
    }
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[t][mb] = mfma_16x16x32(w[t], x[mb], acc[t][mb]);
  }

  // Cross-wave reduction of the split-K partial sums, in wave order.
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) red[((wave * T + t) * MB + mb) * 64 + lane] = acc[t][mb];
  __syncthreads();
  for (int mb = wave; mb < MB; mb += S) {
    f32x4_t v[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      v[t] = red[(t * MB + mb) * 64 + lane];
      for (int s = 1; s < S; ++s) v[t] += red[((s * T + t) * MB + mb) * 64 + lane];
    }
    const int64_t m = mb * 16 + i;
    if (m >= a.M) continue;

    // Lane owns output row m and the 4 consecutive columns 4g .. 4g+3 of each tile.
    if constexpr (EPI == kEpiSwiglu) {
      const int64_t n = (int64_t)blockIdx.x * kTileN + g * 4;
      if (n < a.out_n) {
        uint16_t* o = static_cast<uint16_t*>(a.out) + m * a.ldo + n;
        store_bf16x4(o, swiglu(v[0][0], v[1][0]), swiglu(v[0][1], v[1][1]),
                     swiglu(v[0][2], v[1][2]), swiglu(v[0][3], v[1][3]));
      }
    } else {
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const int64_t n = (tile0 + t) * kTileN + g * 4;
        if (n >= a.out_n) continue;
        if constexpr (EPI == kEpiBf16) {
          store_bf16x4(static_cast<uint16_t*>(a.out) + m * a.ldo + n, v[t][0], v[t][1], v[t][2], v[t][3]);
        } else {
          *reinterpret_cast<float4*>(static_cast<float*>(a.out) + m * a.ldo + n) =
              make_float4(v[t][0], v[t][1], v[t][2], v[t][3]);
        }
      }
    }
  }
}

template <int MB, int T, int EPI>
hipError_t launch_mb(const LinearArgs& a, hipStream_t s) {
  constexpr int U = MB * T <= 2 ? 4 : 2;  // keeps every variant within 128 VGPRs
  // Waves per workgroup: split K as far as the LDS reduction buffer (64 KiB)
  // and the K extent allow.
  int S = 64 / (T * MB);
  if (S > 16) S = 16;
  if (S > a.ksteps) S = (int)a.ksteps;
  if (S < 1) S = 1;
  const int64_t groups = a.ntiles / T;
  const size_t lds = (size_t)S * T * MB * 64 * sizeof(f32x4_t);
  hipLaunchKernelGGL((gemv_kernel<MB, T, EPI, U>), dim3((unsigned)groups), dim3(64 * S), lds, s, a);
  return hipGetLastError();
}

template <int T, int EPI>
hipError_t launch_t(const LinearArgs& a, hipStream_t s) {
  switch ((a.M + 15) / 16) {
    case 1: return launch_mb<1, T, EPI>(a, s);
    case 2: return launch_mb<2, T, EPI>(a, s);
    case 3: return launch_mb<3, T, EPI>(a, s);
    case 4: return launch_mb<4, T, EPI>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_gemv(const LinearArgs& a, Epilogue epi, hipStream_t s) {
  if (a.M <= 0 || a.ntiles == 0) return hipSuccess;
  switch (epi) {
    case kEpiSwiglu: return launch_t<2, kEpiSwiglu>(a, s);
    case kEpiBf16: return launch_t<1, kEpiBf16>(a, s);
    case kEpiF32: return launch_t<1, kEpiF32>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace tpk
