// Prefill path (M > 64 tokens): the shard is a dense contraction bound by the
// matrix cores ("Tensor vs Pipeline Parallelism", "A worked communication
// estimate": prompt compute is about 2 x parameters x tokens operations).
//
// Three kernels. gemm_big (256 x 256 tiles, 8 wavefronts, 32x32x16 MFMA,
// stages landed in LDS by DMA) runs whenever the grid fills the GPU;
// gemm_mid (128 x 256 tiles, three LDS stage buffers) runs prefills of up to
// 512 tokens, where the weights stream from HBM and need more DMA lead, and
// grids of big tiles that neither fill a round nor split K; gemm_kernel
// (128 x 128 tiles, 16x16x32 MFMA, register-staged) covers the rest. On
// gfx950 the 32x32x16 bf16 MFMA sustains about 1.5x the rate of the 16x16x32
// one when fed from LDS.
//
// gemm_kernel, for gfx950:
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
    if (nt < ntiles && ks < ksteps) v = W[tile_index(nt, ks, ksteps) * kTileU4 + l];
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


// ---------------------------------------------------------------------------
// gemm_big: 256 output columns x 256 tokens per workgroup of 8 wavefronts
// (2 per SIMD, so one wavefront's MFMAs cover the other's waits). Wavefront
// (wn, wm) owns 128 columns x 64 tokens: 4 x 2 accumulators of
// v_mfma_f32_32x32x16_bf16.
//
//  * A stage is 64 k (two packed k-steps): 32 weight chunks of 1 KiB (tile t,
//    k-step h at chunk 2t + h, copied verbatim from the packed layout, where
//    a tile pair's two stage k-steps are 4 contiguous KiB) and
//    256 token rows of 128 bytes. Stages land in LDS by buffer-load-to-LDS
//    DMA: no staging registers and no LDS store instructions. Each token row
//    is read as a whole 128-byte line; its octet o is stored at position
//    o ^ ((row >> 1) & 7), which keeps both the DMA writes and the fragment
//    reads free of bank conflicts.
//  * Two 64 KiB LDS buffers and one barrier per stage. The barrier both
//    publishes stage s + 1 (every wave has waited for its own DMA) and frees
//    the buffer of stage s (every wave has read it), after which the DMA of
//    stage s + 2 goes into that buffer, its instructions interleaved with the
//    first MFMAs.
//  * A wave keeps the whole stage's fragments in registers (4 k-halves x
//    (4 weight + 2 token) x 16 bytes). While it multiplies stage s it reads
//    stage s + 1: each k-half's registers are refilled right after their
//    MFMAs have been issued.
//  * Rows and tiles past the end fall outside the buffer resource's range
//    and land as zeros; so does a ragged last k-step (an out-of-range offset),
//    and so does the padding stage when the stage count is odd.
//  * Workgroup ids are spread so that the 32 workgroups an XCD runs together
//    cover 8 token tiles x 4 column tiles (shared through that XCD's L2).
//  * Epilogue: lane (h, j) owns token j of each 32-token block and, for
//    q = 0..3, output columns 8q + 4h .. +3 of each 32-column block
//    (accumulator elements 4q .. 4q+3), so a direct store writes 32 rows x
//    32 (fp32) or 16 (bf16) bytes per instruction. Each wave instead passes
//    its results through its own 4 KiB of LDS beside the stage buffers and
//    writes whole 128-byte lines, with no barrier (store_block_lines).
//    Against direct stores: the 405B down projection 1.48-1.52 -> 1.43-1.45
//    ms, the 70B O slice 84-89 -> 73-76 us; SwiGLU and bf16 outputs
//    unchanged.
// ---------------------------------------------------------------------------

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ f32x16_t mfma_32x32x16(uint4 a, uint4 b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

constexpr int BIG_T = 16;                        // packed tiles per workgroup
constexpr int BIG_MT = 16;                       // 16-token tiles per full-height workgroup
constexpr int BIG_WCH = 2 * BIG_T;               // weight chunks per stage
constexpr int BIG_THREADS = 512;

// s_waitcnt immediates (vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
constexpr int kWaitVm0 = 0x0F70;    // vmcnt(0)
constexpr int kWaitLgkm0 = 0xC07F;  // lgkmcnt(0)

// fp32 epilogue of one wavefront's 32-token x 128-column block: accumulators
// v0..v3 (32-column blocks x = 0..3 in the 32x32x16 MFMA layout: lane (h, j)
// holds token j, columns 8q + 4h .. +3 as elements 4q .. 4q+3), first token
// row m_first, first packed tile nt_first. In that layout a row's 512 bytes
// sit in two lanes, so a direct store writes 32 rows x 32 bytes per
// instruction; the block is transposed in the wave's 16 KiB of LDS T
// instead (16-byte piece P of row r at slot 32 r + (P ^ r)), and each store
// instruction writes two rows x 512 contiguous bytes. The caller has made T
// free for the wave.
__device__ __forceinline__ void store_block_f32(const LinearArgs& a, const f32x16_t& v0, const f32x16_t& v1,
                                                const f32x16_t& v2, const f32x16_t& v3, uint4* T, int lane,
                                                int64_t m_first, int64_t nt_first) {
  const int fh = lane >> 5, fj = lane & 31;
  const f32x16_t* v[4] = {&v0, &v1, &v2, &v3};
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      T[fj * 32 + ((8 * x + 2 * q + fh) ^ fj)] =
          make_uint4(__float_as_uint((*v[x])[4 * q]), __float_as_uint((*v[x])[4 * q + 1]),
                     __float_as_uint((*v[x])[4 * q + 2]), __float_as_uint((*v[x])[4 * q + 3]));
  const int64_t n = nt_first * kTileN + (lane & 31) * 4;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int r = 2 * k + (lane >> 5);
    const uint4 w = T[r * 32 + ((lane & 31) ^ r)];
    const int64_t m = m_first + r;
    if (m < a.M && n < a.out_n) *reinterpret_cast<uint4*>(static_cast<float*>(a.out) + m * a.ldo + n) = w;
  }
}

// gemm_big's epilogue of one wave's 32-token x 128-column block (arguments
// as for store_block_f32) through the wave's own 4 KiB E of LDS, beside the
// stage buffers, so no wave waits for another: rows of 128 bytes, 16-byte
// piece P of row r at slot 8 r + (P ^ ((r >> 1) & 7)), and each store
// instruction writes 8 rows x 128 contiguous bytes. SwiGLU: the block's 64
// output columns at once (a 32-column block is one gate tile, elements 0..7
// of each 16, and its up tile, 8..15); fp32: one 32-column block at a time;
// bf16: 64 columns (two blocks) at a time.
template <int EPI>
__device__ __forceinline__ void store_block_lines(const LinearArgs& a, const f32x16_t& v0, const f32x16_t& v1,
                                                const f32x16_t& v2, const f32x16_t& v3, uint4* E, int lane,
                                                int64_t m_first, int64_t nt_first) {
  const int fh = lane >> 5, fj = lane & 31;
  const f32x16_t* v[4] = {&v0, &v1, &v2, &v3};
  const int sw = (fj >> 1) & 7;
  const int rr = lane >> 3, p = lane & 7;
  if constexpr (EPI == kEpiF32) {
#pragma unroll
    for (int x = 0; x < 4; ++x) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        E[fj * 8 + ((2 * q + fh) ^ sw)] =
            make_uint4(__float_as_uint((*v[x])[4 * q]), __float_as_uint((*v[x])[4 * q + 1]),
                       __float_as_uint((*v[x])[4 * q + 2]), __float_as_uint((*v[x])[4 * q + 3]));
      const int64_t n = (nt_first + 2 * x) * kTileN + p * 4;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int r = 8 * k + rr;
        const uint4 w = E[r * 8 + (p ^ ((r >> 1) & 7))];
        const int64_t m = m_first + r;
        if (m < a.M && n < a.out_n) *reinterpret_cast<uint4*>(static_cast<float*>(a.out) + m * a.ldo + n) = w;
      }
    }
  } else {
    uint2* E2 = reinterpret_cast<uint2*>(E);
    constexpr int NPASS = EPI == kEpiSwiglu ? 1 : 2;  // 64 output columns per pass
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
#pragma unroll
      for (int xx = 0; xx < 4 / NPASS; ++xx) {
        const int x = ps * (4 / NPASS) + xx;
        const f32x16_t& w = *v[x];
        if constexpr (EPI == kEpiSwiglu) {
#pragma unroll
          for (int q = 0; q < 2; ++q)
            E2[(fj * 8 + ((2 * x + q) ^ sw)) * 2 + fh] =
                bf16x4(swiglu(w[4 * q], w[4 * q + 8]), swiglu(w[4 * q + 1], w[4 * q + 9]),
                       swiglu(w[4 * q + 2], w[4 * q + 10]), swiglu(w[4 * q + 3], w[4 * q + 11]));
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            E2[(fj * 8 + ((4 * xx + q) ^ sw)) * 2 + fh] = bf16x4(w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]);
        }
      }
      const int64_t n = (EPI == kEpiSwiglu ? (nt_first >> 1) * kTileN : (nt_first + 4 * ps) * kTileN) + p * 8;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int r = 8 * k + rr;
        const uint4 w = E[r * 8 + (p ^ ((r >> 1) & 7))];
        const int64_t m = m_first + r;
        if (m < a.M && n < a.out_n) *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.out) + m * a.ldo + n) = w;
      }
    }
  }
}

// 256 x 256 tiles: workgroup x takes tile x of the launch (its 128-token
// halves, for a grid's partial last round, run on gemm_mid). TB counts the
// 128-token halves of the tile.
template <int EPI, bool SPLIT>
__global__ __launch_bounds__(BIG_THREADS) void gemm_big(LinearArgs a, int ntn, int ntm, int64_t kper, float* part) {
  constexpr int TB = 2;
  constexpr int ROWS = 128 * TB;                       // tokens per workgroup
  constexpr int XI = 2 * TB;                           // token DMA instructions per wave and stage
  constexpr int STAGE_U4 = BIG_WCH * 64 + ROWS * 8;    // 64 KiB per stage
  __shared__ uint4 L0[STAGE_U4], L1[STAGE_U4];
  __shared__ uint4 EP[8 * 256];  // the epilogue's 4 KiB per wave
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = wave & 1, wm = wave >> 1;  // column half, token quarter

  // Tile of this workgroup: ids that share an XCD (id mod 8) get consecutive
  // tiles, grouped 8 token tiles deep.
  int bid = (int)blockIdx.x;
  {
    const int per = (int)gridDim.x / 8;
    if (bid < per * 8) bid = (bid % 8) * per + bid / 8;
  }
  constexpr int GM = 8;
  const int first_m = bid / (GM * ntn) * GM;
  const int gsize = ntm - first_m < GM ? ntm - first_m : GM;
  const int tm = first_m + (bid % (GM * ntn)) % gsize;
  const int tn = (bid % (GM * ntn)) / gsize;
  const int64_t nt0 = (int64_t)tn * BIG_T;
  const int64_t m0 = (int64_t)tm * (BIG_MT * 16);
  // ksteps is the packed layout's pair stride; kcnt the k-steps this
  // workgroup multiplies. A split takes k-steps [y kper, y kper + kcnt) and
  // writes its fp32 sum to part[y] ([M x ntiles 16], split order y).
  const int64_t ksteps = a.ksteps;
  int64_t kcnt = ksteps;
  if constexpr (SPLIT) {
    const int64_t k0 = (int64_t)blockIdx.y * kper;
    kcnt = ksteps - k0 < kper ? ksteps - k0 : kper;
    a.W += k0 * 2 * kTileU4;  // pair p, k-step ks sits at 1 KiB index (p ksteps + ks) 2 + t
    a.X += k0 * kTileK;
    a.K = a.K - k0 * kTileK < kcnt * kTileK ? a.K - k0 * kTileK : kcnt * kTileK;
    a.out = part + (int64_t)blockIdx.y * a.M * (a.ntiles * kTileN);
    a.ldo = a.ntiles * kTileN;
    a.out_n = a.ldo;
  }
  const int64_t nst = (kcnt + 1) / 2;

  const int64_t wt = a.ntiles - nt0 < BIG_T ? a.ntiles - nt0 : BIG_T;
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.W + nt0 * ksteps * kTileU4), (short)0, (int)(wt * ksteps * 1024), 0x00020000);
  const int64_t rows = a.M - m0 < ROWS ? (a.M > m0 ? a.M - m0 : 0) : ROWS;
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.X + m0 * a.ldx), (short)0, (int)(rows * a.ldx * 2), 0x00020000);

  // DMA sources of this wave: weight chunks c = 4 wave + j and token row
  // blocks XI wave + j (8 rows x 128 bytes each, one per instruction).
  unsigned woff[4], xoff[4], kx[4];  // the token arrays use their first XI entries
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = wave * 4 + j;
    // tile tt = c >> 1 of the workgroup (nt0 is even), k-step h = c & 1 of the stage
    woff[j] = (unsigned)(tile_index(c >> 1, c & 1, ksteps) * 1024 + lane * 16);
  }
#pragma unroll
  for (int j = 0; j < XI; ++j) {
    const int r = (wave * XI + j) * 8 + (lane >> 3);
    const int o = (lane & 7) ^ ((r >> 1) & 7);  // logical octet landing in this lane's slot
    xoff[j] = (unsigned)(((int64_t)r * a.ldx + 8 * o) * 2);
    kx[j] = a.K > 8 * o ? (unsigned)(a.K - 8 * o) : 0u;  // octet inside K while 64 s < kx
  }
#define TP_ISSUE(LB, S)                                                                          \
  {                                                                                              \
    const unsigned s_ = (unsigned)(S);                                                           \
    _Pragma("unroll") for (int j = 0; j < 4; ++j) __builtin_amdgcn_raw_ptr_buffer_load_lds(      \
        rw, (lds_void_t*)&LB[(wave * 4 + j) * 64], 16,                                           \
        2 * s_ + (j & 1) < (unsigned)kcnt ? woff[j] + s_ * 4096u : 0x80000000u, 0, 0, 0);        \
    _Pragma("unroll") for (int j = 0; j < XI; ++j) __builtin_amdgcn_raw_ptr_buffer_load_lds(     \
        rx, (lds_void_t*)&LB[BIG_WCH * 64 + (wave * XI + j) * 64], 16,                           \
        64u * s_ < kx[j] ? xoff[j] + s_ * 128u : 0x80000000u, 0, 0, 0);                          \
  }
  // Fragment addresses. 32x32x16 A operand (weights) of block x, k-half kh:
  // lane (h, j) takes tile 2 (4 wn + x) + j / 16, k-step kh / 2, octet
  // 2 (kh % 2) + h, column j % 16. B operand (tokens): row 32 (TB wm + y) + j,
  // octet 2 kh + h, stored at octet position (2 kh + h) ^ ((j >> 1) & 7).
  const int fh = lane >> 5, fj = lane & 31;
  const int fa = (fj >> 4) * 128 + fh * 16 + (fj & 15);
  const int swz = fh ^ ((fj >> 1) & 7);
  const int fb = BIG_WCH * 64 + (wm * 32 * TB + fj) * 8;
  uint4 FA[4][4], FB[4][TB];
#define TP_READ(LB, KH)                                                                          \
  _Pragma("unroll") for (int x = 0; x < 4; ++x)                                                  \
      FA[KH][x] = LB[(wn * 4 + x) * 256 + ((KH) >> 1) * 64 + ((KH) & 1) * 32 + fa];              \
  _Pragma("unroll") for (int y = 0; y < TB; ++y) FB[KH][y] = LB[fb + y * 256 + ((2 * (KH)) ^ swz)];
#define TP_MMA(KH)                                                                               \
  _Pragma("unroll") for (int x = 0; x < 4; ++x) _Pragma("unroll") for (int y = 0; y < TB; ++y)  \
      acc[x][y] = mfma_32x32x16(FA[KH][x], FB[KH][y], acc[x][y]);
#define TP_SB __builtin_amdgcn_sched_barrier(0);
  // The DMA instructions alternate with the first k-half's MFMAs.
#define TP_INTERLEAVE                                             \
  _Pragma("unroll") for (int q = 0; q < 8; ++q) {                 \
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0); /* MFMA */ \
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0); /* VMEM */ \
  }
  // Multiply the registers' stage while reading the next one from LB.
#define TP_STAGE(LB)                                                                             \
  TP_MMA(0) TP_INTERLEAVE TP_SB TP_READ(LB, 0) TP_SB TP_MMA(1) TP_SB TP_READ(LB, 1) TP_SB        \
  TP_MMA(2) TP_SB TP_READ(LB, 2) TP_SB TP_MMA(3) TP_SB TP_READ(LB, 3)
  // Every wave has finished its LDS reads and its DMA has landed; then the barrier.
#define TP_SYNC()                                    \
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);            \
  __builtin_amdgcn_s_waitcnt(kWaitVm0);              \
  __builtin_amdgcn_s_barrier();

  f32x16_t acc[4][TB];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < TB; ++y) acc[x][y] = f32x16_t{};

  TP_ISSUE(L0, 0)
  TP_ISSUE(L1, 1)
  constexpr int kWaitStage0 = 0x0F70 | ((4 + XI) & 15);  // vmcnt(4 + XI): stage 0 has landed
  __builtin_amdgcn_s_waitcnt(kWaitStage0);
  __builtin_amdgcn_s_barrier();
  TP_READ(L0, 0) TP_READ(L0, 1) TP_READ(L0, 2) TP_READ(L0, 3)
  // The loop runs a whole number of stage pairs; with an odd stage count the
  // last one is the all-zero padding stage.
  for (int64_t s = 0; s < nst; s += 2) {
    // registers: stage s; in flight: s + 1 (L1)
    TP_SYNC()
    TP_ISSUE(L0, s + 2)
    TP_STAGE(L1)
    // registers: stage s + 1; in flight: s + 2 (L0)
    TP_SYNC()
    TP_ISSUE(L1, s + 3)
    TP_STAGE(L0)
  }
  // No DMA may still be landing in LDS when the workgroup ends.
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
#undef TP_ISSUE
#undef TP_READ
#undef TP_MMA
#undef TP_SB
#undef TP_INTERLEAVE
#undef TP_STAGE
#undef TP_SYNC

#pragma unroll
  for (int y = 0; y < TB; ++y)
    store_block_lines<EPI>(a, acc[0][y], acc[1][y], acc[2][y], acc[3][y], &EP[wave * 256], lane,
                           m0 + (wm * TB + y) * 32, nt0 + wn * 8);
}

// gemm_mid: prefills of at most a few hundred tokens, where every weight byte
// comes from HBM once and the big tile's one stage of DMA lead (about 1.2 us)
// is shorter than the HBM latency under a full streaming load. 128-token x
// 256-column tiles (gemm_big's half-height form, 48 KiB stages), three LDS
// stage buffers instead of two: a stage's DMA goes out two stages before its
// fragments are read. Token tiles of 128 rows, grouped as gemm_big groups its
// tiles, so the token tiles of one weight column block share an XCD's L2.
// The stage, fragment and epilogue layouts are gemm_big's at half height.
template <int EPI, bool SPLIT>
__global__ __launch_bounds__(BIG_THREADS) void gemm_mid(LinearArgs a, int ntn, int ntm, int tail_base, int64_t kper,
                                                         float* part) {
  constexpr int ROWS = 128;
  constexpr int XI = 2;                              // token DMA instructions per wave and stage
  constexpr int STAGE_U4 = BIG_WCH * 64 + ROWS * 8;  // 48 KiB per stage
  __shared__ uint4 L0[STAGE_U4], L1[STAGE_U4], L2[STAGE_U4];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = wave & 1, wm = wave >> 1;  // column half, token quarter

  // tail_base < 0: 128-token tiles in gemm_big's grouped order (ntm counts
  // 128-token tiles). tail_base >= 0: the halves of gemm_big's 256-token
  // tiles tail_base + x / 2 (ntm counts 256-token tiles), for the last,
  // partial round of a big-tile grid.
  const bool tail = tail_base >= 0;
  int bid = tail ? tail_base + (int)(blockIdx.x >> 1) : (int)blockIdx.x;
  if (!tail) {
    const int per = (int)gridDim.x / 8;
    if (bid < per * 8) bid = (bid % 8) * per + bid / 8;
  }
  constexpr int GM = 8;
  const int first_m = bid / (GM * ntn) * GM;
  const int gsize = ntm - first_m < GM ? ntm - first_m : GM;
  const int tm = first_m + (bid % (GM * ntn)) % gsize;
  const int tn = (bid % (GM * ntn)) / gsize;
  const int64_t nt0 = (int64_t)tn * BIG_T;
  const int64_t m0 = tail ? (int64_t)tm * (2 * ROWS) + (int64_t)(blockIdx.x & 1) * ROWS : (int64_t)tm * ROWS;
  const int64_t ksteps = a.ksteps;
  int64_t kcnt = ksteps;
  if constexpr (SPLIT) {
    const int64_t k0 = (int64_t)blockIdx.y * kper;
    kcnt = ksteps - k0 < kper ? ksteps - k0 : kper;
    a.W += k0 * 2 * kTileU4;
    a.X += k0 * kTileK;
    a.K = a.K - k0 * kTileK < kcnt * kTileK ? a.K - k0 * kTileK : kcnt * kTileK;
    a.out = part + (int64_t)blockIdx.y * a.M * (a.ntiles * kTileN);
    a.ldo = a.ntiles * kTileN;
    a.out_n = a.ldo;
  }
  const int64_t nst = (kcnt + 1) / 2;

  const int64_t wt = a.ntiles - nt0 < BIG_T ? a.ntiles - nt0 : BIG_T;
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.W + nt0 * ksteps * kTileU4), (short)0, (int)(wt * ksteps * 1024), 0x00020000);
  const int64_t rows = a.M - m0 < ROWS ? (a.M > m0 ? a.M - m0 : 0) : ROWS;
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.X + m0 * a.ldx), (short)0, (int)(rows * a.ldx * 2), 0x00020000);

  unsigned woff[4], xoff[XI], kx[XI];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = wave * 4 + j;
    woff[j] = (unsigned)(tile_index(c >> 1, c & 1, ksteps) * 1024 + lane * 16);
  }
#pragma unroll
  for (int j = 0; j < XI; ++j) {
    const int r = (wave * XI + j) * 8 + (lane >> 3);
    const int o = (lane & 7) ^ ((r >> 1) & 7);
    xoff[j] = (unsigned)(((int64_t)r * a.ldx + 8 * o) * 2);
    kx[j] = a.K > 8 * o ? (unsigned)(a.K - 8 * o) : 0u;
  }
#define TP_ISSUE(LB, S)                                                                          \
  {                                                                                              \
    const unsigned s_ = (unsigned)(S);                                                           \
    _Pragma("unroll") for (int j = 0; j < 4; ++j) __builtin_amdgcn_raw_ptr_buffer_load_lds(      \
        rw, (lds_void_t*)&LB[(wave * 4 + j) * 64], 16,                                           \
        2 * s_ + (j & 1) < (unsigned)kcnt ? woff[j] + s_ * 4096u : 0x80000000u, 0, 0, 0);        \
    _Pragma("unroll") for (int j = 0; j < XI; ++j) __builtin_amdgcn_raw_ptr_buffer_load_lds(     \
        rx, (lds_void_t*)&LB[BIG_WCH * 64 + (wave * XI + j) * 64], 16,                           \
        64u * s_ < kx[j] ? xoff[j] + s_ * 128u : 0x80000000u, 0, 0, 0);                          \
  }
  const int fh = lane >> 5, fj = lane & 31;
  const int fa = (fj >> 4) * 128 + fh * 16 + (fj & 15);
  const int swz = fh ^ ((fj >> 1) & 7);
  const int fb = BIG_WCH * 64 + (wm * 32 + fj) * 8;
  uint4 FA[4][4], FB[4];
#define TP_READ(LB, KH)                                                                          \
  _Pragma("unroll") for (int x = 0; x < 4; ++x)                                                  \
      FA[KH][x] = LB[(wn * 4 + x) * 256 + ((KH) >> 1) * 64 + ((KH) & 1) * 32 + fa];              \
  FB[KH] = LB[fb + ((2 * (KH)) ^ swz)];
#define TP_MMA(KH) _Pragma("unroll") for (int x = 0; x < 4; ++x) acc[x] = mfma_32x32x16(FA[KH][x], FB[KH], acc[x]);
#define TP_SB __builtin_amdgcn_sched_barrier(0);
#define TP_INTERLEAVE                                             \
  _Pragma("unroll") for (int q = 0; q < 4 + XI; ++q) {            \
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0); /* MFMA */ \
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0); /* VMEM */ \
  }
#define TP_STAGE(LB)                                                                             \
  TP_MMA(0) TP_INTERLEAVE TP_SB TP_READ(LB, 0) TP_SB TP_MMA(1) TP_SB TP_READ(LB, 1) TP_SB        \
  TP_MMA(2) TP_SB TP_READ(LB, 2) TP_SB TP_MMA(3) TP_SB TP_READ(LB, 3)
  // The next stage has landed (only the one after it may still be in flight),
  // and every wave has finished reading the buffer that the new DMA refills.
  constexpr int kWaitNext = 0x0F70 | (4 + XI);
#define TP_SYNC()                                    \
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);            \
  __builtin_amdgcn_s_waitcnt(kWaitNext);             \
  __builtin_amdgcn_s_barrier();

  f32x16_t acc[4];
#pragma unroll
  for (int x = 0; x < 4; ++x) acc[x] = f32x16_t{};

  TP_ISSUE(L0, 0)
  TP_ISSUE(L1, 1)
  TP_ISSUE(L2, 2)
  __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * (4 + XI)));  // stage 0 has landed
  __builtin_amdgcn_s_barrier();
  TP_READ(L0, 0) TP_READ(L0, 1) TP_READ(L0, 2) TP_READ(L0, 3)
  // Distinct markers keep the prologue's reads and the loop's last reads
  // from being merged into one block at the loop's head, where the wait
  // insertion could no longer tell which buffer each pending DMA fills.
  asm volatile(";; prologue reads");
  // Whole groups of three stages; the stages past K are all-zero padding.
  for (int64_t s = 0; s < nst; s += 3) {
    TP_SYNC()
    TP_ISSUE(L0, s + 3)
    TP_STAGE(L1)
    TP_SYNC()
    TP_ISSUE(L1, s + 4)
    TP_STAGE(L2)
    TP_SYNC()
    TP_ISSUE(L2, s + 5)
    TP_STAGE(L0)
    asm volatile(";; stage group end");
  }
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
#undef TP_ISSUE
#undef TP_READ
#undef TP_MMA
#undef TP_SB
#undef TP_INTERLEAVE
#undef TP_STAGE
#undef TP_SYNC

  if constexpr (EPI == kEpiF32) {
    __syncthreads();
    uint4* T = wave < 3 ? &L0[wave * 1024] : (wave < 6 ? &L1[(wave - 3) * 1024] : &L2[(wave - 6) * 1024]);
    store_block_f32(a, acc[0], acc[1], acc[2], acc[3], T, lane, m0 + wm * 32, nt0 + wn * 8);
    return;
  }
  const int64_t m = m0 + wm * 32 + fj;
  if (m >= a.M) return;
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const int64_t ntb = nt0 + wn * 8 + 2 * x;
    const f32x16_t& v = acc[x];
    if constexpr (EPI == kEpiSwiglu) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int64_t n = (ntb >> 1) * kTileN + 8 * q + 4 * fh;
        if (ntb >= a.ntiles || n >= a.out_n) continue;
        store_bf16x4(static_cast<uint16_t*>(a.out) + m * a.ldo + n, swiglu(v[4 * q], v[4 * q + 8]),
                     swiglu(v[4 * q + 1], v[4 * q + 9]), swiglu(v[4 * q + 2], v[4 * q + 10]),
                     swiglu(v[4 * q + 3], v[4 * q + 11]));
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t n = ntb * kTileN + 8 * q + 4 * fh;
        if (n >= a.out_n) continue;
        store_bf16x4(static_cast<uint16_t*>(a.out) + m * a.ldo + n, v[4 * q], v[4 * q + 1], v[4 * q + 2],
                     v[4 * q + 3]);
      }
    }
  }
}

// How a prefill linear is launched. The big tile needs buffer offsets below
// 2^31. When its tiles alone cannot fill the 256 CUs (one workgroup per CU),
// K is split G ways, G = the whole number of tile sets that fit in one round
// (each split keeping at least 16 k-steps); the splits write fp32 partials and
// the split fix-up adds them in split order and applies the epilogue.
struct GemmPlan {
  bool big;
  int G;         // K splits of the big tile (1: none)
  int64_t kper;  // k-steps per split (even: whole stages)
};

GemmPlan plan_gemm(int64_t M, int64_t ldx, int64_t ksteps, int64_t ntiles) {
  GemmPlan p{false, 1, ksteps};
  const int64_t ntn = (ntiles + BIG_T - 1) / BIG_T, ntm = (M + BIG_MT * 16 - 1) / (BIG_MT * 16);
  p.big = (int64_t)BIG_MT * 16 * ldx * 2 < (1LL << 31) && BIG_T * ksteps * 1024 < (1LL << 31);
  if (!p.big) return p;
  const int64_t tiles = ntn * ntm;
  if (tiles >= 256) return p;
  int64_t G = 256 / tiles;
  if (G > ksteps / 16) G = ksteps / 16;
  if (G < 2) {
    p.big = false;  // neither whole tiles nor splits fill the GPU: 128 x 128 tiles
    return p;
  }
  p.kper = ((ksteps + G - 1) / G + 1) / 2 * 2;
  p.G = (int)((ksteps + p.kper - 1) / p.kper);
  return p;
}

// The last round of big tiles, when it would run at most half full. If its
// tiles (ids [full, nb) of gemm_big's grouped order) form a rectangle of
// token tiles x column tiles, it runs as a sub-GEMM with K split G = 256 /
// tiles ways (fp32 partials, then the split fix-up applies the epilogue), so
// that whole 256 x 256 tiles fill the GPU; otherwise as 128-token half tiles
// on gemm_mid.
struct TailPlan {
  bool split = false;
  int64_t m0 = 0, rows = 0, nt0 = 0, nt = 0;  // token rows and packed tiles of the sub-GEMM
  int G = 1;
  int64_t kper = 0;
};

TailPlan plan_tail(int64_t M, int64_t ksteps, int64_t ntiles) {
  TailPlan t;
  const int64_t ntn = (ntiles + BIG_T - 1) / BIG_T, ntm = (M + BIG_MT * 16 - 1) / (BIG_MT * 16);
  const int64_t nb = ntn * ntm, full = nb / 256 * 256, left = nb - full;
  if (left == 0 || left > 128) return t;
  int64_t G = 256 / left;
  if (G > ksteps / 16) G = ksteps / 16;
  if (G < 2) return t;
  // gemm_big's tile of id b: groups of GM = 8 token tiles, column-major inside
  constexpr int64_t GM = 8;
  int64_t tm0 = ntm, tm1 = 0, tn0 = ntn, tn1 = 0;
  for (int64_t b = full; b < nb; ++b) {
    const int64_t first_m = b / (GM * ntn) * GM;
    const int64_t gsize = ntm - first_m < GM ? ntm - first_m : GM;
    const int64_t tm = first_m + (b % (GM * ntn)) % gsize, tn = (b % (GM * ntn)) / gsize;
    tm0 = tm < tm0 ? tm : tm0;
    tm1 = tm + 1 > tm1 ? tm + 1 : tm1;
    tn0 = tn < tn0 ? tn : tn0;
    tn1 = tn + 1 > tn1 ? tn + 1 : tn1;
  }
  if ((tm1 - tm0) * (tn1 - tn0) != left) return t;  // not a rectangle
  t.m0 = tm0 * BIG_MT * 16;
  t.rows = (tm1 * BIG_MT * 16 < M ? tm1 * BIG_MT * 16 : M) - t.m0;
  t.nt0 = tn0 * BIG_T;
  t.nt = (tn1 * BIG_T < ntiles ? tn1 * BIG_T : ntiles) - t.nt0;
  t.kper = ((ksteps + G - 1) / G + 1) / 2 * 2;
  t.G = (int)((ksteps + t.kper - 1) / t.kper);
  t.split = t.G > 1;
  return t;
}

// When gemm_mid runs instead of gemm_big: prefills of at most 512 tokens
// (every weight byte comes from HBM, and the big tile's single stage of DMA
// lead stalls on it), and grids of 129-255 big tiles, which neither fill a
// round nor split K (those would otherwise fall back to gemm_kernel). K is
// split G ways (whole stages) when the 128-token tiles alone cannot fill the
// GPU.
constexpr int64_t kMidMaxM = 512;
struct MidPlan {
  bool use;
  int G;
  int64_t kper;
};

MidPlan plan_mid(int64_t M, int64_t ldx, int64_t ksteps, int64_t ntiles) {
  MidPlan p{false, 1, ksteps};
  if ((int64_t)128 * ldx * 2 >= (1LL << 31) || (int64_t)BIG_T * ksteps * 1024 >= (1LL << 31)) return p;
  const int64_t ntn = (ntiles + BIG_T - 1) / BIG_T;
  const int64_t big_tiles = ntn * ((M + BIG_MT * 16 - 1) / (BIG_MT * 16));
  const bool small = M <= kMidMaxM;
  const bool unfilled = big_tiles > 128 && big_tiles < 256 && ksteps >= 32;
  if (!small && !unfilled) return p;
  const int64_t tiles = ntn * ((M + 127) / 128);
  int64_t G = 1;
  if (tiles < 256) {
    G = 256 / tiles;
    if (G > ksteps / 16) G = ksteps / 16;
    if (G < 1) G = 1;
  }
  if (tiles * G < 64) return p;  // too few workgroups either way: the other plans
  p.use = true;
  if (G >= 2) {
    p.kper = ((ksteps + G - 1) / G + 1) / 2 * 2;
    p.G = (int)((ksteps + p.kper - 1) / p.kper);
  }
  return p;
}

}  // namespace

size_t gemm_workspace_bytes(int64_t M, int64_t ldx, int64_t ksteps, int64_t ntiles) {
  if (M <= 0) return 0;
  const MidPlan mp = plan_mid(M, ldx, ksteps, ntiles);
  if (mp.use) return mp.G > 1 ? (size_t)mp.G * M * ntiles * kTileN * sizeof(float) : 0;
  const GemmPlan p = plan_gemm(M, ldx, ksteps, ntiles);
  if (!p.big) return 0;
  if (p.G > 1) return (size_t)p.G * M * ntiles * kTileN * sizeof(float);
  const TailPlan t = plan_tail(M, ksteps, ntiles);
  return t.split ? (size_t)t.G * t.rows * t.nt * kTileN * sizeof(float) : 0;
}

hipError_t launch_gemm(const LinearArgs& a, Epilogue epi, float* ws, hipStream_t s) {
  if (a.M <= 0 || a.ntiles == 0) return hipSuccess;
  const int64_t ntn = (a.ntiles + BIG_T - 1) / BIG_T, ntm = (a.M + BIG_MT * 16 - 1) / (BIG_MT * 16);
  const MidPlan mp = plan_mid(a.M, a.ldx, a.ksteps, a.ntiles);
  if (mp.use) {
    const int64_t ntm128 = (a.M + 127) / 128;
    const dim3 grid((unsigned)(ntn * ntm128), (unsigned)mp.G);
    if (mp.G > 1) {
      if (ws == nullptr) return hipErrorInvalidValue;
      hipLaunchKernelGGL((gemm_mid<kEpiF32, true>), grid, dim3(BIG_THREADS), 0, s, a, (int)ntn, (int)ntm128, -1, mp.kper, ws);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      return launch_split_fixup(a, epi, ws, mp.G, s);
    }
    switch (epi) {
      case kEpiSwiglu: hipLaunchKernelGGL((gemm_mid<kEpiSwiglu, false>), grid, dim3(BIG_THREADS), 0, s, a, (int)ntn, (int)ntm128, -1, (int64_t)0, nullptr); break;
      case kEpiBf16: hipLaunchKernelGGL((gemm_mid<kEpiBf16, false>), grid, dim3(BIG_THREADS), 0, s, a, (int)ntn, (int)ntm128, -1, (int64_t)0, nullptr); break;
      case kEpiF32: hipLaunchKernelGGL((gemm_mid<kEpiF32, false>), grid, dim3(BIG_THREADS), 0, s, a, (int)ntn, (int)ntm128, -1, (int64_t)0, nullptr); break;
    }
    return hipGetLastError();
  }
  const GemmPlan p = plan_gemm(a.M, a.ldx, a.ksteps, a.ntiles);
  if (p.big && p.G > 1) {
    if (ws == nullptr) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemm_big<kEpiF32, true>), dim3((unsigned)(ntn * ntm), (unsigned)p.G),
                       dim3(BIG_THREADS), 0, s, a, (int)ntn, (int)ntm, p.kper, ws);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_split_fixup(a, epi, ws, p.G, s);
  }
  if (p.big) {
    // One workgroup per CU at a time (128 KiB of LDS each). When the last
    // round would run at most half full, it runs as a second launch that
    // fills the GPU: a split-K sub-GEMM of whole tiles (plan_tail), or its
    // tiles split into 128-token halves.
    const int64_t nb = ntn * ntm, full = nb / 256 * 256, left = nb - full;
    const bool split = left > 0 && left <= 128;
    const unsigned n1 = (unsigned)(split ? full : nb);
    const TailPlan tp = plan_tail(a.M, a.ksteps, a.ntiles);
    if (tp.split && ws == nullptr) return hipErrorInvalidValue;
    switch (epi) {
      case kEpiSwiglu: hipLaunchKernelGGL((gemm_big<kEpiSwiglu, false>), dim3(n1), dim3(BIG_THREADS), 0, s, a, (int)ntn, (int)ntm, (int64_t)0, nullptr); break;
      case kEpiBf16: hipLaunchKernelGGL((gemm_big<kEpiBf16, false>), dim3(n1), dim3(BIG_THREADS), 0, s, a, (int)ntn, (int)ntm, (int64_t)0, nullptr); break;
      case kEpiF32: hipLaunchKernelGGL((gemm_big<kEpiF32, false>), dim3(n1), dim3(BIG_THREADS), 0, s, a, (int)ntn, (int)ntm, (int64_t)0, nullptr); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !split) return e;
    if (tp.split) {
      LinearArgs b = a;
      b.X = a.X + tp.m0 * a.ldx;
      b.M = tp.rows;
      b.W = a.W + tp.nt0 * a.ksteps * kTileU4;
      b.ntiles = tp.nt;
      const int64_t col0 = epi == kEpiSwiglu ? tp.nt0 * kTileN / 2 : tp.nt0 * kTileN;
      const int64_t width = epi == kEpiSwiglu ? tp.nt * kTileN / 2 : tp.nt * kTileN;
      const size_t es = epi == kEpiF32 ? sizeof(float) : sizeof(uint16_t);
      b.out = static_cast<char*>(a.out) + (size_t)(tp.m0 * a.ldo + col0) * es;
      b.out_n = a.out_n - col0 < width ? a.out_n - col0 : width;
      if (a.wscale != nullptr) b.wscale = a.wscale + tp.nt0 * kTileN;
      const int64_t bn = (b.ntiles + BIG_T - 1) / BIG_T, bm = (b.M + BIG_MT * 16 - 1) / (BIG_MT * 16);
      hipLaunchKernelGGL((gemm_big<kEpiF32, true>), dim3((unsigned)(bn * bm), (unsigned)tp.G),
                         dim3(BIG_THREADS), 0, s, b, (int)bn, (int)bm, tp.kper, ws);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
      return launch_split_fixup(b, epi, ws, tp.G, s);
    }
    // Otherwise as 128-token halves of its tiles, on gemm_mid's three stages.
    const dim3 g2((unsigned)(2 * left));
    switch (epi) {
      case kEpiSwiglu: hipLaunchKernelGGL((gemm_mid<kEpiSwiglu, false>), g2, dim3(BIG_THREADS), 0, s, a, (int)ntn, (int)ntm, (int)full, (int64_t)0, nullptr); break;
      case kEpiBf16: hipLaunchKernelGGL((gemm_mid<kEpiBf16, false>), g2, dim3(BIG_THREADS), 0, s, a, (int)ntn, (int)ntm, (int)full, (int64_t)0, nullptr); break;
      case kEpiF32: hipLaunchKernelGGL((gemm_mid<kEpiF32, false>), g2, dim3(BIG_THREADS), 0, s, a, (int)ntn, (int)ntm, (int)full, (int64_t)0, nullptr); break;
    }
    return hipGetLastError();
  }

  const dim3 grid((unsigned)((a.ntiles + BN_T - 1) / BN_T), (unsigned)((a.M + BM - 1) / BM));
  switch (epi) {
    case kEpiSwiglu: hipLaunchKernelGGL(gemm_kernel<kEpiSwiglu>, grid, dim3(256), 0, s, a); break;
    case kEpiBf16: hipLaunchKernelGGL(gemm_kernel<kEpiBf16>, grid, dim3(256), 0, s, a); break;
    case kEpiF32: hipLaunchKernelGGL(gemm_kernel<kEpiF32>, grid, dim3(256), 0, s, a); break;
  }
  return hipGetLastError();
}

}  // namespace tpk
