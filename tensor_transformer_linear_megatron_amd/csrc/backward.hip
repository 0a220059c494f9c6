// Backward of a rank's linear ("Tensor vs Pipeline Parallelism", "Tensor
// parallelism: split inside each layer": training adds two all-reduces per
// layer in the backward pass; "AI Infrastructure series, Part 5", "Why are 8
// GPUs not 8 times faster?": the backward costs twice the forward). The input
// gradient runs on the forward kernels with a transposed shard (TP_DGRAD);
// this file holds the two kernels that have no forward counterpart.
//
// wgrad_kernel: dW [K x N] fp32 = A^T dC, contraction over the M tokens, for
// shards with too few 256 x 256 tiles to fill the GPU (wgrad_big below).
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

// wgrad_big: 256 k x 256 n per workgroup of 8 wavefronts; wavefront (wk, wn)
// owns 128 k x 64 n, 4 x 2 accumulators of v_mfma_f32_32x32x16_bf16.
//  * A stage is 64 tokens: 64 rows of A's 256 columns, then 64 rows of dC's,
//    512 bytes each, landed by buffer-load-to-LDS DMA (no staging registers).
//    Rows are 36 16-byte slots apart; a DMA instruction fills 64 consecutive
//    slots, and the lanes that land on a row's 4 padding slots load zeros.
//  * Operands come out of LDS with the gfx950 transpose read: within each
//    16-lane group, output lane j, element q of ds_read_b64_tr_b16 is element
//    j % 4 of the 8 bytes addressed by lane 4q + j / 4. Lane (h, j) of a
//    32x32x16 operand needs tokens 8h .. 8h + 7 of column j: two reads,
//    tokens 8h + 4hh + 0..3 (hh = 0, 1), where the lane addresses row
//    8h + 4hh + (j % 16) / 4 at columns 16 (j / 16) + 4 (j % 4) .. + 3. Half
//    a wavefront reads 4 rows x 64 bytes, which the 576-byte row pitch puts
//    on 16 distinct 16-byte bank groups.
//  * Pipeline as in the forward's large-tile GEMM: two 72 KiB buffers, one
//    barrier per stage, the DMA of stage s + 2 issued into the buffer that
//    stage s has just left, interleaved with the first MFMAs; the registers
//    hold stage s's fragments while stage s + 1's are read.
//  * Each stage gets its own buffer resource based at its first row, whose
//    range ends at column K (resp. N) of its last valid row: rows past M and
//    the padding stage read as zeros, and 32-bit offsets suffice at any M.
//    Columns past K (N) inside a valid row only feed outputs that are not
//    stored.
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4_t* lds_i16x4_p;

__device__ __forceinline__ f32x16_t mfma_32x32x16(uint4 a, uint4 b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

constexpr int WB_T = 256;                        // k and n per workgroup
constexpr int WB_ST = 64;                        // tokens per stage
constexpr int WB_PITCH = 36;                     // 16-byte slots per LDS row (32 + 4 padding)
constexpr int WB_REGION = WB_ST * WB_PITCH;      // slots of one operand's 64 rows
constexpr int WB_STAGE_U4 = 2 * WB_REGION;       // 72 KiB
constexpr int WB_DMA = WB_STAGE_U4 / 64 / 8;     // DMA instructions per wave and stage (9)
constexpr int kWaitVm0 = 0x0F70;                 // s_waitcnt vmcnt(0)
constexpr int kWaitLgkm0 = 0xC07F;               // s_waitcnt lgkmcnt(0)
constexpr int kWaitStage0 = 0x0F70 | WB_DMA;     // vmcnt(9): the first of two stages has landed
static_assert(WB_REGION % (64 * WB_DMA) == 0, "a wave's DMA stays within one operand");

// The stage's resource; every input is the same on all lanes, which
// readfirstlane makes explicit so that the resource lives in scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t wb_rsrc(const uint16_t* P, int64_t ld, int64_t M, int64_t W,
                                                          int64_t c0, int64_t s) {
  const int64_t m0 = s * WB_ST, left = M - m0;
  const int64_t rows = left < WB_ST ? left : WB_ST;
  const int bytes = rows > 0 ? (int)(((rows - 1) * ld + (W - c0)) * 2) : 0;
  const uint64_t base = (uint64_t)(P + m0 * ld + c0);
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)base);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(base >> 32));
  return __builtin_amdgcn_make_buffer_rsrc((void*)(lo | (hi << 32)), (short)0,
                                           __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

__device__ __forceinline__ uint4 wb_frag(const char* p, int o0, int o1) {
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_p)(p + o0));
  const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_p)(p + o1));
  const uint2 l = __builtin_bit_cast(uint2, lo), h = __builtin_bit_cast(uint2, hi);
  return make_uint4(l.x, l.y, h.x, h.y);
}

__global__ __launch_bounds__(512) void wgrad_big(const uint16_t* __restrict__ A, int64_t lda,
                                                 const uint16_t* __restrict__ C, int64_t ldc, int64_t M,
                                                 int64_t K, int64_t N, float* dW, int64_t lddw, int ntk,
                                                 int ntn) {
  __shared__ uint4 L0[WB_STAGE_U4], L1[WB_STAGE_U4];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wk = wave & 1, wn = wave >> 1;

  // Tile: ids that share an XCD (id mod 8) get consecutive tiles, grouped 8
  // k-tiles deep, so an XCD's L2 serves each column block several times.
  int bid = (int)blockIdx.x;
  {
    const int per = (int)gridDim.x / 8;
    if (bid < per * 8) bid = (bid % 8) * per + bid / 8;
  }
  constexpr int GK = 8;
  const int first_k = bid / (GK * ntn) * GK;
  const int gsize = ntk - first_k < GK ? ntk - first_k : GK;
  const int tk = first_k + (bid % (GK * ntn)) % gsize;
  const int tn = (bid % (GK * ntn)) / gsize;
  const int64_t k0 = (int64_t)tk * WB_T, n0 = (int64_t)tn * WB_T;
  const int64_t nst = (M + WB_ST - 1) / WB_ST;

  // DMA: this wave's instruction u fills slots 64 (WB_DMA wave + u) + lane of
  // the stage: waves 0..3 the A rows, waves 4..7 the dC rows.
  const bool opc = wave >= 4;
  const uint16_t* P = opc ? C : A;
  const int64_t ld = opc ? ldc : lda, W = opc ? N : K, c0 = opc ? n0 : k0;
  unsigned off[WB_DMA];
#pragma unroll
  for (int u = 0; u < WB_DMA; ++u) {
    const int q = (wave * WB_DMA + u) * 64 + lane - (opc ? WB_REGION : 0);
    const int r = q / WB_PITCH, c = q % WB_PITCH;
    off[u] = c < 32 ? (unsigned)((r * ld + 8 * c) * 2) : 0x80000000u;
  }
#define WB_ISSUE(LB, S)                                                                            \
  {                                                                                                \
    const __amdgpu_buffer_rsrc_t rs_ = wb_rsrc(P, ld, M, W, c0, (S));                             \
    _Pragma("unroll") for (int u = 0; u < WB_DMA; ++u) __builtin_amdgcn_raw_ptr_buffer_load_lds(   \
        rs_, (lds_void_t*)&LB[(wave * WB_DMA + u) * 64], 16, off[u], 0, 0, 0);                     \
  }
  // Fragment byte offset of this lane at k-step 0, hh = 0, block 0 of A; the
  // rest are constants: k-step kh adds 16 rows, hh 4 rows, block x 4 slots,
  // dC's block y sits at slot WB_REGION + 8 wn + 4 y.
  const int h = lane >> 5, j = lane & 31;
  const int fbase = ((8 * h + ((j & 15) >> 2)) * WB_PITCH + 2 * (j >> 4) + ((j & 3) >> 1)) * 16 + 8 * (j & 1);
  const char* F0 = (const char*)L0 + fbase;
  const char* F1 = (const char*)L1 + fbase;
  uint4 FA[4][4], FB[4][2];
#define WB_RO(KH, HH) (((KH) * 16 + (HH) * 4) * WB_PITCH * 16)
#define WB_READ(F, KH)                                                                             \
  _Pragma("unroll") for (int x = 0; x < 4; ++x) FA[KH][x] =                                        \
      wb_frag(F, WB_RO(KH, 0) + (wk * 16 + 4 * x) * 16, WB_RO(KH, 1) + (wk * 16 + 4 * x) * 16);    \
  _Pragma("unroll") for (int y = 0; y < 2; ++y) FB[KH][y] =                                        \
      wb_frag(F, WB_RO(KH, 0) + (WB_REGION + wn * 8 + 4 * y) * 16,                                 \
              WB_RO(KH, 1) + (WB_REGION + wn * 8 + 4 * y) * 16);
#define WB_MMA(KH)                                                                                 \
  _Pragma("unroll") for (int x = 0; x < 4; ++x) _Pragma("unroll") for (int y = 0; y < 2; ++y)     \
      acc[x][y] = mfma_32x32x16(FA[KH][x], FB[KH][y], acc[x][y]);
#define WB_SB __builtin_amdgcn_sched_barrier(0);
#define WB_INTERLEAVE                                             \
  _Pragma("unroll") for (int q = 0; q < 8; ++q) {                 \
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0); /* MFMA */ \
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0); /* VMEM */ \
  }
#define WB_STAGE(F)                                                                                \
  WB_MMA(0) WB_INTERLEAVE WB_SB WB_READ(F, 0) WB_SB WB_MMA(1) WB_SB WB_READ(F, 1) WB_SB            \
  WB_MMA(2) WB_SB WB_READ(F, 2) WB_SB WB_MMA(3) WB_SB WB_READ(F, 3)
#define WB_SYNC()                         \
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0); \
  __builtin_amdgcn_s_waitcnt(kWaitVm0);   \
  __builtin_amdgcn_s_barrier();

  f32x16_t acc[4][2];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y) acc[x][y] = f32x16_t{};

  WB_ISSUE(L0, 0)
  WB_ISSUE(L1, 1)
  __builtin_amdgcn_s_waitcnt(kWaitStage0);
  __builtin_amdgcn_s_barrier();
  WB_READ(F0, 0) WB_READ(F0, 1) WB_READ(F0, 2) WB_READ(F0, 3)
  // Whole stage pairs; with an odd count the last stage is all zeros.
  for (int64_t s = 0; s < nst; s += 2) {
    WB_SYNC()
    WB_ISSUE(L0, s + 2)
    WB_STAGE(F1)
    WB_SYNC()
    WB_ISSUE(L1, s + 3)
    WB_STAGE(F0)
  }
  // No DMA may still be landing in LDS when the workgroup ends.
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
#undef WB_ISSUE
#undef WB_RO
#undef WB_READ
#undef WB_MMA
#undef WB_SB
#undef WB_INTERLEAVE
#undef WB_STAGE
#undef WB_SYNC

  // Lane (h, j), accumulator element 4q + r of block (x, y):
  // dW[k0 + 128 wk + 32 x + 8 q + 4 h + r][n0 + 64 wn + 32 y + j].
#pragma unroll
  for (int y = 0; y < 2; ++y) {
    const int64_t n = n0 + wn * 64 + y * 32 + j;
    if (n >= N) continue;
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t k = k0 + wk * 128 + x * 32 + 8 * q + 4 * h + r;
          if (k < K) dW[k * lddw + n] = acc[x][y][4 * q + r];
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
  const int64_t ntk = (K + WB_T - 1) / WB_T, ntn = (N + WB_T - 1) / WB_T;
  if (ntk * ntn >= 256) {  // enough 256 x 256 tiles to fill the GPU
    hipLaunchKernelGGL(wgrad_big, dim3((unsigned)(ntk * ntn)), dim3(512), 0, s, A, lda, dC, lddc, M, K, N, dW,
                       lddw, (int)ntk, (int)ntn);
    return hipGetLastError();
  }
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
