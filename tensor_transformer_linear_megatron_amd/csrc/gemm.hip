// Prefill path (M > 64 tokens): the shard is a dense contraction bound by the
// matrix cores ("Tensor vs Pipeline Parallelism", "A worked communication
// estimate": prompt compute is about 2 x parameters x tokens operations).
//
// Design for gfx950:
//  * Workgroup tile: BN = 128 output columns (8 packed tiles) x BM = 128
//    tokens, k in stages of BK = 64 (two MFMA k-steps). Four wavefronts in a
//    2 x 2 grid, each owning 64 columns x 64 tokens = 4 x 4 MFMA 16x16x32
//    accumulators (64 fp32 registers per lane).
//  * Weight stage: 8 tiles x 2 k-steps = 16 KiB copied straight from the
//    packed layout (contiguous 2 KiB runs) into LDS; a wave's A operand is
//    then one conflict-free ds_read_b128 per tile.
//  * Token stage: 128 rows x 64 k read with 16-byte loads into LDS rows of
//    144 bytes (16 bytes of padding), which makes the B-operand reads of 16
//    rows by one k octet hit 16 distinct 4-bank groups.
//  * Two LDS buffers: the global loads of stage s+1 are in flight while stage
//    s is multiplied; one barrier per stage.
//  * Epilogue in registers: bf16 rounding, SwiGLU (gate/up tiles are adjacent
//    in the packed layout, so a wave's tiles 0/1 and 2/3 pair up) or fp32.
#include "tp_internal.h"

namespace tpk {
namespace {

constexpr int BN_T = 8;    // packed tiles per workgroup (128 columns)
constexpr int BM = 128;    // tokens per workgroup
constexpr int KS = 2;      // MFMA k-steps per stage (BK = 64)
constexpr int XROW = 9;    // uint4 per LDS token row: 8 octets + 1 pad

// Global -> registers for one stage: 4 weight uint4 and 4 token uint4 per thread.
__device__ __forceinline__ void load_stage(uint4 (&rw)[4], uint4 (&rx)[4], const uint4* __restrict__ W,
                                           const uint16_t* __restrict__ X, int64_t ldx, int64_t M,
                                           int64_t K, int64_t ksteps, int64_t ntiles, int64_t nt0,
                                           int64_t m0, int64_t st, int tid) {
  const uint4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = tid + j * 256;        // 0..1023
    const int tl = c >> 6, l = c & 63;  // local tile index (nt_l * KS + ks_l), lane
    const int64_t nt = nt0 + (tl >> 1), ks = st * KS + (tl & 1);
    uint4 v = zero;
    if (nt < ntiles && ks < ksteps) v = W[(nt * ksteps + ks) * kTileU4 + l];
    rw[j] = v;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = tid + j * 256;
    const int row = c >> 3, oct = c & 7;
    const int64_t m = m0 + row, k = st * (KS * kTileK) + oct * 8;
    uint4 v = zero;
    if (m < M && k < K) v = *reinterpret_cast<const uint4*>(X + m * ldx + k);
    rx[j] = v;
  }
}

__device__ __forceinline__ void store_stage(uint4* sW, uint4* sX, const uint4 (&rw)[4],
                                            const uint4 (&rx)[4], int tid) {
#pragma unroll
  for (int j = 0; j < 4; ++j) sW[tid + j * 256] = rw[j];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = tid + j * 256;
    sX[(c >> 3) * XROW + (c & 7)] = rx[j];
  }
}

template <int EPI>
__global__ __launch_bounds__(256) void gemm_kernel(LinearArgs a) {
  __shared__ uint4 sW[2][BN_T * KS * 64];  // 2 x 16 KiB
  __shared__ uint4 sX[2][BM * XROW];       // 2 x 18 KiB
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, i = lane & 15;
  const int wn = wave & 1, wm = wave >> 1;
  const int64_t nt0 = (int64_t)blockIdx.x * BN_T;
  const int64_t m0 = (int64_t)blockIdx.y * BM;
  const uint4* __restrict__ W = a.W;
  const uint16_t* __restrict__ X = a.X;
  const int64_t ldx = a.ldx, M = a.M, K = a.K, ksteps = a.ksteps, ntiles = a.ntiles;
  const int64_t nstages = (ksteps + KS - 1) / KS;

  uint4 rw[4], rx[4];
  f32x4_t acc[4][4];
#pragma unroll
  for (int jn = 0; jn < 4; ++jn)
#pragma unroll
    for (int jm = 0; jm < 4; ++jm) acc[jn][jm] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  load_stage(rw, rx, W, X, ldx, M, K, ksteps, ntiles, nt0, m0, 0, tid);
  store_stage(sW[0], sX[0], rw, rx, tid);
  __syncthreads();
  for (int64_t st = 0; st < nstages; ++st) {
    const int buf = (int)(st & 1);
    if (st + 1 < nstages) load_stage(rw, rx, W, X, ldx, M, K, ksteps, ntiles, nt0, m0, st + 1, tid);
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      uint4 A[4], B[4];
#pragma unroll
      for (int jn = 0; jn < 4; ++jn) A[jn] = sW[buf][((wn * 4 + jn) * KS + kk) * 64 + lane];
#pragma unroll
      for (int jm = 0; jm < 4; ++jm) B[jm] = sX[buf][((wm * 4 + jm) * 16 + i) * XROW + kk * 4 + g];
#pragma unroll
      for (int jn = 0; jn < 4; ++jn)
#pragma unroll
        for (int jm = 0; jm < 4; ++jm) acc[jn][jm] = mfma_16x16x32(A[jn], B[jm], acc[jn][jm]);
    }
    if (st + 1 < nstages) store_stage(sW[buf ^ 1], sX[buf ^ 1], rw, rx, tid);
    __syncthreads();
  }

  // Lane owns rows m = m0 + (wm*4 + jm)*16 + i and columns 4g..4g+3 of each tile.
#pragma unroll
  for (int jm = 0; jm < 4; ++jm) {
    const int64_t m = m0 + (wm * 4 + jm) * 16 + i;
    if (m >= M) continue;
    if constexpr (EPI == kEpiSwiglu) {
#pragma unroll
      for (int jp = 0; jp < 2; ++jp) {
        const int64_t nt = nt0 + wn * 4 + jp * 2;  // gate tile; nt + 1 is its up tile
        const int64_t n = (nt >> 1) * kTileN + g * 4;
        if (nt >= ntiles || n >= a.out_n) continue;
        const f32x4_t gt = acc[jp * 2][jm], up = acc[jp * 2 + 1][jm];
        store_bf16x4(static_cast<uint16_t*>(a.out) + m * a.ldo + n, swiglu(gt[0], up[0]),
                     swiglu(gt[1], up[1]), swiglu(gt[2], up[2]), swiglu(gt[3], up[3]));
      }
    } else {
#pragma unroll
      for (int jn = 0; jn < 4; ++jn) {
        const int64_t n = (nt0 + wn * 4 + jn) * kTileN + g * 4;
        if (n >= a.out_n) continue;
        const f32x4_t v = acc[jn][jm];
        if constexpr (EPI == kEpiBf16) {
          store_bf16x4(static_cast<uint16_t*>(a.out) + m * a.ldo + n, v[0], v[1], v[2], v[3]);
        } else {
          *reinterpret_cast<float4*>(static_cast<float*>(a.out) + m * a.ldo + n) =
              make_float4(v[0], v[1], v[2], v[3]);
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm(const LinearArgs& a, Epilogue epi, hipStream_t s) {
  if (a.M <= 0 || a.ntiles == 0) return hipSuccess;
  const dim3 grid((unsigned)((a.ntiles + BN_T - 1) / BN_T), (unsigned)((a.M + BM - 1) / BM));
  switch (epi) {
    case kEpiSwiglu: hipLaunchKernelGGL(gemm_kernel<kEpiSwiglu>, grid, dim3(256), 0, s, a); break;
    case kEpiBf16: hipLaunchKernelGGL(gemm_kernel<kEpiBf16>, grid, dim3(256), 0, s, a); break;
    case kEpiF32: hipLaunchKernelGGL(gemm_kernel<kEpiF32>, grid, dim3(256), 0, s, a); break;
  }
  return hipGetLastError();
}

}  // namespace tpk
