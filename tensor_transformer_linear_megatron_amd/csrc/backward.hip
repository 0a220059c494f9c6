// Backward of a rank's linear ("Tensor vs Pipeline Parallelism", "Tensor
// parallelism: split inside each layer": training adds two all-reduces per
// layer in the backward pass; "AI Infrastructure series, Part 5", "Why are 8
// GPUs not 8 times faster?": the backward costs twice the forward). The input
// gradient runs on the forward kernels with a transposed shard (TP_DGRAD);
// this file holds the two kernels that have no forward counterpart.
//
// wgrad_kernel: dW [K x N] fp32 = A^T dC, contraction over the M tokens.
//  * Workgroup tile 128 k x 128 n, four wavefronts of 64 x 64 (4 x 4
//    accumulators of v_mfma_f32_16x16x32_bf16). The MFMA's 32-deep
//    contraction is 32 tokens: A operand lane (g, i) = A[m0 + 8g + e][k_i],
//    B operand lane (g, i) = dC[m0 + 8g + e][n_i].
//  * Both inputs are token-major, so each 32-token chunk is staged in LDS
//    transposed, [k][m] and [n][m]: a thread loads two token rows' 16 bytes
//    (8 k) and stores 8 dwords holding the two tokens' values side by side.
//    Rows are 36 bf16 (72 bytes): the 4-byte stores of a wavefront hit 64
//    distinct banks, and fragment reads are two 8-byte reads per lane.
//  * The next chunk's global loads are in flight while the current one is
//    multiplied; two LDS buffers, one barrier per chunk.
//  * Tokens past M, and k or n past the shard, read as zero; M == 0 writes
//    zeros.
//
// swiglu_bwd_kernel: elementwise, one thread per 4 columns of a row.
#include "tp_internal.h"

namespace tpk {
namespace {

constexpr int WG_T = 128;   // k (and n) per workgroup tile
constexpr int WG_M = 32;    // tokens per chunk
constexpr int WG_RS = 36;   // LDS row stride in bf16 (32 tokens + 4 pad)

// Global -> registers: thread t loads tokens 2 mp and 2 mp + 1 (mp = t % 16)
// at k-octet kq = t / 16 (0..15) of the 128-wide tile.
__device__ __forceinline__ void wg_load(uint4 (&r)[2], const uint16_t* __restrict__ P, int64_t ld,
                                        int64_t M, int64_t W, int64_t m0, int64_t c0, int tid) {
  const int mp = tid & 15, kq = tid >> 4;
  const int64_t col = c0 + 8 * kq;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t m = m0 + 2 * mp + j;
    r[j] = (m < M && col < W) ? *reinterpret_cast<const uint4*>(P + m * ld + col) : make_uint4(0, 0, 0, 0);
  }
}

// Registers -> LDS, transposed: S[8 kq + e][2 mp .. 2 mp + 1] = (r0[e], r1[e]).
__device__ __forceinline__ void wg_store(uint32_t* S, const uint4 (&r)[2], int tid) {
  const int mp = tid & 15, kq = tid >> 4;
  const uint32_t a[4] = {r[0].x, r[0].y, r[0].z, r[0].w}, b[4] = {r[1].x, r[1].y, r[1].z, r[1].w};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t lo = (e & 1) ? (a[e >> 1] >> 16) : (a[e >> 1] & 0xFFFFu);
    const uint32_t hi = (e & 1) ? (b[e >> 1] >> 16) : (b[e >> 1] & 0xFFFFu);
    S[((8 * kq + e) * WG_RS) / 2 + mp] = lo | (hi << 16);
  }
}

// Fragment of rows [row0, row0 + 16): lane (g, i) reads row row0 + i, tokens 8g .. 8g + 7.
__device__ __forceinline__ uint4 wg_frag(const uint32_t* S, int row0, int g, int i) {
  const uint2* p = reinterpret_cast<const uint2*>(S + ((row0 + i) * WG_RS) / 2 + 4 * g);
  const uint2 x = p[0], y = p[1];
  return make_uint4(x.x, x.y, y.x, y.y);
}

__global__ __launch_bounds__(256) void wgrad_kernel(const uint16_t* __restrict__ A, int64_t lda,
                                                    const uint16_t* __restrict__ dC, int64_t lddc,
                                                    int64_t M, int64_t K, int64_t N, float* dW,
                                                    int64_t lddw) {
  __shared__ uint32_t SA[2][WG_T * WG_RS / 2], SC[2][WG_T * WG_RS / 2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, i = lane & 15;
  const int wk = wave >> 1, wn = wave & 1;
  const int64_t k0 = (int64_t)blockIdx.y * WG_T, n0 = (int64_t)blockIdx.x * WG_T;
  const int64_t nch = (M + WG_M - 1) / WG_M;

  f32x4_t acc[4][4];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) acc[x][y] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  uint4 ra[2], rc[2];
  if (nch > 0) {
    wg_load(ra, A, lda, M, K, 0, k0, tid);
    wg_load(rc, dC, lddc, M, N, 0, n0, tid);
    wg_store(SA[0], ra, tid);
    wg_store(SC[0], rc, tid);
  }
  __syncthreads();
  for (int64_t ch = 0; ch < nch; ++ch) {
    const int buf = (int)(ch & 1);
    if (ch + 1 < nch) {
      wg_load(ra, A, lda, M, K, (ch + 1) * WG_M, k0, tid);
      wg_load(rc, dC, lddc, M, N, (ch + 1) * WG_M, n0, tid);
    }
    uint4 fa[4], fc[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) fa[x] = wg_frag(SA[buf], wk * 64 + x * 16, g, i);
#pragma unroll
    for (int y = 0; y < 4; ++y) fc[y] = wg_frag(SC[buf], wn * 64 + y * 16, g, i);
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int y = 0; y < 4; ++y) acc[x][y] = mfma_16x16x32(fa[x], fc[y], acc[x][y]);
    if (ch + 1 < nch) {
      wg_store(SA[buf ^ 1], ra, tid);
      wg_store(SC[buf ^ 1], rc, tid);
    }
    __syncthreads();
  }

  // Lane (g, i) of block (x, y) holds dW[k0 + 64 wk + 16 x + 4 g + r][n0 + 64 wn + 16 y + i].
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) {
      const int64_t n = n0 + wn * 64 + y * 16 + i;
      if (n >= N) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t k = k0 + wk * 64 + x * 16 + 4 * g + r;
        if (k < K) dW[k * lddw + n] = acc[x][y][r];
      }
    }
}

__device__ __forceinline__ float bf16f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// dG = dH U s (1 + G (1 - s)), dU = dH G s, s = 1 / (1 + e^-G); finite for
// finite inputs (e^-G = inf gives s = 0).
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const uint16_t* GU, int64_t ldgu, const float* dH,
                                                         int64_t lddh, int64_t M, int64_t w, uint16_t* dGU,
                                                         int64_t lddgu) {
  const int64_t w4 = w / 4, total = M * w4;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = idx / w4, c = (idx - m * w4) * 4;
    const uint2 gb = *reinterpret_cast<const uint2*>(GU + m * ldgu + c);
    const uint2 ub = *reinterpret_cast<const uint2*>(GU + m * ldgu + w + c);
    const float4 dh = *reinterpret_cast<const float4*>(dH + m * lddh + c);
    const uint16_t gs[4] = {(uint16_t)gb.x, (uint16_t)(gb.x >> 16), (uint16_t)gb.y, (uint16_t)(gb.y >> 16)};
    const uint16_t us[4] = {(uint16_t)ub.x, (uint16_t)(ub.x >> 16), (uint16_t)ub.y, (uint16_t)(ub.y >> 16)};
    const float dhs[4] = {dh.x, dh.y, dh.z, dh.w};
    float dg[4], du[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float gv = bf16f(gs[e]), uv = bf16f(us[e]);
      const float s = 1.0f / (1.0f + expf(-gv));
      dg[e] = dhs[e] * uv * s * (1.0f + gv * (1.0f - s));
      du[e] = dhs[e] * gv * s;
    }
    store_bf16x4(dGU + m * lddgu + c, dg[0], dg[1], dg[2], dg[3]);
    store_bf16x4(dGU + m * lddgu + w + c, du[0], du[1], du[2], du[3]);
  }
}

}  // namespace

hipError_t launch_wgrad(const uint16_t* A, int64_t lda, const uint16_t* dC, int64_t lddc, int64_t M,
                        int64_t K, int64_t N, float* dW, int64_t lddw, hipStream_t s) {
  if (K <= 0 || N <= 0) return hipSuccess;
  const dim3 grid((unsigned)((N + WG_T - 1) / WG_T), (unsigned)((K + WG_T - 1) / WG_T));
  hipLaunchKernelGGL(wgrad_kernel, grid, dim3(256), 0, s, A, lda, dC, lddc, M, K, N, dW, lddw);
  return hipGetLastError();
}

hipError_t launch_swiglu_bwd(const uint16_t* GU, int64_t ldgu, const float* dH, int64_t lddh,
                             int64_t M, int64_t w, uint16_t* dGU, int64_t lddgu, hipStream_t s) {
  const int64_t total = M * (w / 4);
  if (total == 0) return hipSuccess;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(swiglu_bwd_kernel, dim3((unsigned)blocks), dim3(256), 0, s, GU, ldgu, dH, lddh, M,
                     w, dGU, lddgu);
  return hipGetLastError();
}

}  // namespace tpk
