// Decode path (M <= 64 tokens): Y = X W_shard streams every weight byte once
// and is bound by HBM bandwidth ("AI Infrastructure series, Part 5",
// "Reason 2": each decoded token streams the whole weight set once, and a
// rank of t streams its 1/t share).
//
// Both kernels multiply on the matrix cores: the weight tile is the A operand
// of v_mfma_f32_16x16x32_bf16 (16 output columns x 32 k, one packed 1 KiB
// tile, one wavefront-wide coalesced dwordx4 load) and 16 tokens are the B
// operand (zero rows past M). The matrix cores have ample headroom at every M;
// the work is in keeping enough weight bytes in flight.
//
//  * gemv_stream (M <= 16): a workgroup owns T adjacent packed tiles (T = 2
//    pairs gate and up for SwiGLU) for the whole K; its S wavefronts take
//    contiguous k-ranges. Each wavefront keeps a ring of U steps of weight
//    and token loads in flight: the steady-state loop has no branches, so the
//    compiler's wait counts track the ring exactly and never drain it. Token
//    rows past M are read from a clamped address and zeroed by a lane mask.
//    The S partial sums are reduced through LDS in wave order (deterministic)
//    and the epilogue (bf16 rounding, SwiGLU or fp32) runs in registers.
//    It also serves 17 to 32 tokens (two token blocks per wavefront) when
//    the tile pairs fill the GPU and K is short, instead of a split.
//  * gemv_shared (16 < M <= 64): at larger M every wavefront would re-read
//    all the token fragments from L2 for its own tiles, which caps the rate.
//    Here SN wavefronts of a workgroup own different 32-column blocks over
//    the same k-range and share each chunk of C token k-steps through LDS
//    (double buffered, one barrier per chunk; the weight ring stays in flight
//    across it). They multiply on v_mfma_f32_32x32x16_bf16, so a token
//    fragment serves 32 columns and the LDS traffic per weight byte halves.
//    When the column count is too small to fill the GPU, the k-range is also
//    split over G workgroups; each writes an fp32 partial and gemv_fixup
//    adds them in split order and applies the epilogue.
#include "tp_internal.h"

namespace tpk {
namespace {

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

// Rotated starts for the streaming kernels when a tile pair's k-range is a
// power of two of k-steps (so every pair, and every wave's share, starts at a
// power-of-two byte offset). Measured on the 70B TP = 8 gate/up share (256
// k-steps): 22.6 -> 21.4 us; on the 8B shares (448 k-steps) it cost 1-3 %.
bool rotate_starts(int64_t ksteps) { return ksteps > 0 && (ksteps & (ksteps - 1)) == 0; }

// Streamed, read-once weight tile: non-temporal load.
__device__ __forceinline__ uint4 load_w(const uint4* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// One token fragment row (16 bytes = 8 k of one token) without branches. The
// load address is clamped into the row (always in bounds); the value is
// masked when it is consumed, so the load's latency stays hidden: rows past M
// and octets past K become zero.
struct TokenRow {
  const uint16_t* row;  // start of the (clamped) token row plus the lane's k octet
  int64_t kmax;         // largest valid k offset relative to row
  unsigned mask;        // 0 for rows past M
  __device__ __forceinline__ uint4 load(int64_t koff) const {
    return *reinterpret_cast<const uint4*>(row + (koff <= kmax ? koff : kmax));
  }
  __device__ __forceinline__ uint4 use(uint4 v, int64_t koff) const {
    const unsigned m = koff <= kmax ? mask : 0u;
    v.x &= m;
    v.y &= m;
    v.z &= m;
    v.w &= m;
    return v;
  }
  __device__ __forceinline__ uint4 get(int64_t koff) const { return use(load(koff), koff); }
};

__device__ __forceinline__ TokenRow token_row(const LinearArgs& a, int64_t m, int g) {
  TokenRow r;
  const bool ok = m < a.M;
  r.row = a.X + (ok ? m : a.M - 1) * a.ldx + g * 8;
  r.kmax = a.K - 8 - g * 8;
  r.mask = ok ? 0xffffffffu : 0u;
  return r;
}

// The wavefront index as a scalar. Every loop bound and guard derived from it
// is then a scalar branch: an MFMA must never sit under a lane mask, because
// the matrix cores execute it even when EXEC is zero.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Epilogue of one output fragment group: lane (g, i) owns token row m and
// output columns 4g .. 4g+3 of each tile.
template <int EPI, int T>
__device__ __forceinline__ void epilogue(const LinearArgs& a, const f32x4_t (&v)[T], int64_t m,
                                         int64_t first_tile, int g) {
  if (m >= a.M) return;
  if constexpr (EPI == kEpiSwiglu) {
    const int64_t n = (first_tile >> 1) * kTileN + g * 4;
    if (n < a.out_n)
      store_bf16x4(static_cast<uint16_t*>(a.out) + m * a.ldo + n, swiglu(v[0][0], v[1][0]),
                   swiglu(v[0][1], v[1][1]), swiglu(v[0][2], v[1][2]), swiglu(v[0][3], v[1][3]));
  } else {
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int64_t n = (first_tile + t) * kTileN + g * 4;
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

// ---------------------------------------------------------------------------
// gemv_stream
// ---------------------------------------------------------------------------

template <int MB, int T, int U, int EPI, int LB>
__global__ __launch_bounds__(LB) void gemv_stream(LinearArgs a, int64_t chunk, bool rotate) {
  static_assert(T == 1 || T == 2, "one tile or one tile pair per workgroup");
  extern __shared__ f32x4_t red[];  // [S][T][MB][64]
  const int lane = threadIdx.x & 63, wave = wave_id(), S = blockDim.x >> 6;
  const int g = lane >> 4, i = lane & 15;
  const int64_t tile0 = (int64_t)blockIdx.x * T;
  const int64_t ksteps = a.ksteps;
  const int64_t k0 = (int64_t)wave * chunk;
  const int64_t k1 = k0 + chunk < ksteps ? k0 + chunk : ksteps;
  const int64_t n = k1 > k0 ? k1 - k0 : 0;
  // A pair's k-steps alternate between its two tiles: with T = 2 the wave
  // reads one contiguous stream, with T = 1 every other KiB of it.
  const uint4* wp = a.W + tile_index(tile0, n > 0 ? k0 : 0, ksteps) * kTileU4 + lane;
  TokenRow xr[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) xr[mb] = token_row(a, mb * 16 + i, g);
  const int64_t xk0 = k0 * kTileK;

  f32x4_t acc[T][MB];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[t][mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  uint4 wb[U][T], xb[U][MB];
  // With `rotate` (set when the pairs' k-ranges lie at power-of-two
  // strides) the wave walks its k-range from a rotated start, step s being
  // k-step k0 + (s + rot) mod n: waves whose ranges begin at power-of-two
  // offsets would otherwise all read the same HBM channels at the same time.
  const int64_t rot = rotate && n > 0 ? ((int64_t)blockIdx.x * S + wave) * 37 % n : 0;
#define TP_RS(STEP) ((STEP) + rot < n ? (STEP) + rot : (STEP) + rot - n)
#define TP_FILL(SLOT, STEP)                                                                \
  {                                                                                        \
    const int64_t rs_ = TP_RS(STEP);                                                       \
    _Pragma("unroll") for (int t = 0; t < T; ++t)                                          \
        wb[SLOT][t] = load_w(wp + (rs_ * 2 + t) * kTileU4);                                \
    _Pragma("unroll") for (int mb = 0; mb < MB; ++mb)                                      \
        xb[SLOT][mb] = xr[mb].load(xk0 + rs_ * kTileK);                                    \
  }
#define TP_MMA(SLOT, STEP)                                                                 \
  {                                                                                        \
    const int64_t rs_ = TP_RS(STEP);                                                       \
    _Pragma("unroll") for (int mb = 0; mb < MB; ++mb) {                                    \
      const uint4 xv = xr[mb].use(xb[SLOT][mb], xk0 + rs_ * kTileK);                       \
      _Pragma("unroll") for (int t = 0; t < T; ++t)                                        \
          acc[t][mb] = mfma_16x16x32(wb[SLOT][t], xv, acc[t][mb]);                         \
    }                                                                                      \
  }
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (u < n) TP_FILL(u, u)
  const int64_t full = n / U;
  // Steady state: every refill target exists, no branches.
  for (int64_t r = 0; r + 1 < full; ++r) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      TP_MMA(u, r * U + u)
      TP_FILL(u, (r + 1) * U + u)
    }
  }
  // Last full group (refills only for the steps that exist) and the tail.
  if (full >= 1) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      TP_MMA(u, (full - 1) * U + u)
      if (full * U + u < n) TP_FILL(u, full * U + u)
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (full * U + u < n) TP_MMA(u, full * U + u)
#undef TP_FILL
#undef TP_MMA
#undef TP_RS

  // Cross-wave reduction in wave order, then the epilogue (one wave per m-block).
  if (S > 1) {
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
      epilogue<EPI, T>(a, v, mb * 16 + i, tile0, g);
    }
  } else {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      f32x4_t v[T];
#pragma unroll
      for (int t = 0; t < T; ++t) v[t] = acc[t][mb];
      epilogue<EPI, T>(a, v, mb * 16 + i, tile0, g);
    }
  }
}

// ---------------------------------------------------------------------------
// gemv8_stream: 8-bit shards (TP_W_FP8_E4M3), 1 <= M <= 64
// ---------------------------------------------------------------------------

typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two E4M3 codes (word `hi` of d) -> their bf16 values decode * 2^e, packed.
// The hardware conversion scales exactly by the power of two; the results
// have at most 4 significant bits, so their upper halves are the bf16 bits.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_bf16x2(uint32_t d, float scale) {
  const f32x2_t f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(d, scale, HI);
  return __builtin_amdgcn_perm(__float_as_uint(f[1]), __float_as_uint(f[0]), 0x07060302u);
}

// A lane's 16 codes -> the A operands of the step's two bf16 k-steps.
__device__ __forceinline__ void decode_fp8_tile(uint4 w, float sc, uint4& a0, uint4& a1) {
  a0 = make_uint4(fp8x2_bf16x2<false>(w.x, sc), fp8x2_bf16x2<true>(w.x, sc),
                  fp8x2_bf16x2<false>(w.y, sc), fp8x2_bf16x2<true>(w.y, sc));
  a1 = make_uint4(fp8x2_bf16x2<false>(w.z, sc), fp8x2_bf16x2<true>(w.z, sc),
                  fp8x2_bf16x2<false>(w.w, sc), fp8x2_bf16x2<true>(w.w, sc));
}

// As gemv_stream, over steps of 64 k: a workgroup owns T adjacent tiles for
// the whole K, its S wavefronts take contiguous step ranges, and each keeps a
// ring of U steps of code and token loads in flight. A step is one 16-byte
// code load per lane and tile (half the bytes of the bf16 path for the same
// k) and 2 MB token fragments (MB blocks of 16 tokens); the codes are decoded
// in registers with the lane's column scale and multiplied on the bf16 MFMA.
template <int MB, int T, int U, int EPI, int LB>
__global__ __launch_bounds__(LB) void gemv8_stream(LinearArgs a, int64_t chunk, bool rotate) {
  static_assert(T == 1 || T == 2, "one tile or one tile pair per workgroup");
  extern __shared__ f32x4_t red[];  // [S][T][MB][64]
  const int lane = threadIdx.x & 63, wave = wave_id(), S = blockDim.x >> 6;
  const int g = lane >> 4, i = lane & 15;
  const int64_t tile0 = (int64_t)blockIdx.x * T;
  const int64_t ksteps = a.ksteps;  // steps of 64 k
  const int64_t k0 = (int64_t)wave * chunk;
  const int64_t k1 = k0 + chunk < ksteps ? k0 + chunk : ksteps;
  const int64_t n = k1 > k0 ? k1 - k0 : 0;
  const uint4* wp = a.W + tile_index(tile0, n > 0 ? k0 : 0, ksteps) * kTileU4 + lane;
  float sc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) sc[t] = a.wscale[(tile0 + t) * kTileN + i];
  TokenRow xr[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) xr[mb] = token_row(a, mb * 16 + i, g);
  const int64_t xk0 = k0 * kTileK8;

  f32x4_t acc[T][MB];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[t][mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  uint4 wb[U][T], xb[U][MB][2];
  // Rotated start of the wave's k-range, as in gemv_stream.
  const int64_t rot = rotate && n > 0 ? ((int64_t)blockIdx.x * S + wave) * 37 % n : 0;
#define TP_RS(STEP) ((STEP) + rot < n ? (STEP) + rot : (STEP) + rot - n)
#define TP_FILL(SLOT, STEP)                                                                \
  {                                                                                        \
    const int64_t rs_ = TP_RS(STEP);                                                       \
    _Pragma("unroll") for (int t = 0; t < T; ++t)                                          \
        wb[SLOT][t] = load_w(wp + (rs_ * 2 + t) * kTileU4);                                \
    _Pragma("unroll") for (int mb = 0; mb < MB; ++mb) _Pragma("unroll") for (int h = 0; h < 2; ++h) \
        xb[SLOT][mb][h] = xr[mb].load(xk0 + rs_ * kTileK8 + h * kTileK);                   \
  }
#define TP_MMA(SLOT, STEP)                                                                 \
  {                                                                                        \
    _Pragma("unroll") for (int t = 0; t < T; ++t) {                                        \
      uint4 a0, a1;                                                                        \
      decode_fp8_tile(wb[SLOT][t], sc[t], a0, a1);                                         \
      _Pragma("unroll") for (int mb = 0; mb < MB; ++mb) {                                  \
        const int64_t ko = xk0 + TP_RS(STEP) * kTileK8;                                    \
        acc[t][mb] = mfma_16x16x32(a0, xr[mb].use(xb[SLOT][mb][0], ko), acc[t][mb]);      \
        acc[t][mb] = mfma_16x16x32(a1, xr[mb].use(xb[SLOT][mb][1], ko + kTileK), acc[t][mb]); \
      }                                                                                    \
    }                                                                                      \
  }
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (u < n) TP_FILL(u, u)
  const int64_t full = n / U;
  for (int64_t r = 0; r + 1 < full; ++r) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      TP_MMA(u, r * U + u)
      TP_FILL(u, (r + 1) * U + u)
    }
  }
  if (full >= 1) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      TP_MMA(u, (full - 1) * U + u)
      if (full * U + u < n) TP_FILL(u, full * U + u)
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (full * U + u < n) TP_MMA(u, full * U + u)
#undef TP_FILL
#undef TP_MMA
#undef TP_RS

  if (S > 1) {
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
        for (int s2 = 1; s2 < S; ++s2) v[t] += red[((s2 * T + t) * MB + mb) * 64 + lane];
      }
      epilogue<EPI, T>(a, v, mb * 16 + i, tile0, g);
    }
  } else {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      f32x4_t v[T];
#pragma unroll
      for (int t = 0; t < T; ++t) v[t] = acc[t][mb];
      epilogue<EPI, T>(a, v, mb * 16 + i, tile0, g);
    }
  }
}

// ---------------------------------------------------------------------------
// gemv_shared
// ---------------------------------------------------------------------------

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x16_t mfma_32x32x16(uint4 a, uint4 b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// 16 < M <= 64 on v_mfma_f32_32x32x16_bf16: a 32-column block (two adjacent
// packed tiles; for SwiGLU one gate tile and its up tile) times 32 tokens, so
// each token fragment read from LDS serves 32 output columns.
//  * Wave w of workgroup x owns block SN x + w for the workgroup's k-range
//    (split y of G). Its weights stream through a ring of U k-steps of buffer
//    loads; the A operand of k-half kh is lane (h, j) -> tile 2b + j / 16,
//    octet 2 kh + h, column j % 16: two contiguous 512-byte runs per load.
//    Loads past the split or the shard fall outside the buffer range and
//    read as zero, so the loop has no branches around loads.
//  * Token fragments (16 tokens x 32 k, the B layout of the 16x16x32 MFMA)
//    are staged per chunk of C k-steps in LDS, double buffered, loaded two
//    chunks ahead from clamped addresses and masked when stored (rows past M,
//    octets past K). The 32x32x16 B operand of 32-token block t, k-half kh is
//    lane (h, j) -> fragment 2t + j / 16, slot (2 kh + h) * 16 + j % 16.
//  * Accumulator element r = 4q + e of lane (h, j) is output column
//    8q + 4h + e of the block for token j: gate column 8q + 4h + e pairs with
//    up element r + 8.
//  * With G > 1 each split writes an fp32 partial part[y][m][n] and
//    gemv_fixup adds them in split order.
//  * F8: 8-bit shards. A weight step is 64 k (two bf16 k-steps of tokens).
//    The same two 16-byte loads per lane and step bring, for lane (h, j),
//    the codes of column j of the pair at k-octets h and 4 + h (first load,
//    lane h 16 + j % 16 of the 8-bit tile) and 2 + h and 6 + h (second load):
//    exactly its A operands of the step's four 16-k blocks, decoded in
//    registers with the column scale. U and per count weight steps; C counts
//    the bf16 k-steps of a token chunk.
template <int MB32, int U, int C, int SN, int EPI, bool F8 = false>
__global__ __launch_bounds__(64 * SN) void gemv_shared(LinearArgs a, int64_t per, float* part) {
  constexpr int KX = F8 ? 2 : 1;  // bf16 k-steps of tokens per weight step
  static_assert(C % KX == 0 && (C / KX) % U == 0, "the ring must divide the chunk");
  constexpr int MB16 = 2 * MB32;  // 16-token fragments per k-step
  constexpr int F = C * MB16;     // token fragments per chunk
  static_assert(F % SN == 0, "staged fragments divide over the waves");
  constexpr int FPW = F / SN;
  __shared__ uint4 xs[2 * F * 64];
  const int lane = threadIdx.x & 63, nw = wave_id();
  const int g = lane >> 4, i = lane & 15, fh = lane >> 5, fj = lane & 31;
  const int64_t ksteps = a.ksteps;  // weight steps
  const int64_t blk = (int64_t)blockIdx.x * SN + nw;  // this wave's 32-column block
  const int64_t kbeg = (int64_t)blockIdx.y * per;
  const int64_t kend = kbeg + per < ksteps ? kbeg + per : ksteps;
  const int64_t n = kend > kbeg ? kend - kbeg : 0;  // weight steps, uniform over the workgroup
  const int64_t nch = (n * KX + C - 1) / C;
  const int64_t nblk = (a.ntiles + 1) / 2;
  float sc = 1.0f;  // the lane's column scale (8-bit shards)
  if (F8 && blk < nblk) sc = a.wscale[blk * 2 * kTileN + fj];

  // Weights of this workgroup's 2 SN tiles.
  const int64_t t0 = (int64_t)blockIdx.x * SN * 2;
  const int64_t wt = a.ntiles - t0 < 2 * SN ? a.ntiles - t0 : 2 * SN;
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.W + t0 * ksteps * kTileU4), (short)0, (int)(wt * ksteps * 1024), 0x00020000);
  // Pair nw of the workgroup, tile (fj >> 4) of the pair: k-step s at 1 KiB
  // index (nw ksteps + s) 2 + (fj >> 4).
  const unsigned wl =
      (unsigned)((((int64_t)nw * ksteps + kbeg) * 2 + (fj >> 4)) * 1024 + (fh * 16 + (fj & 15)) * 16);
  // Weights are read once per call: non-temporal loads (cache policy bit nt),
  // which on MI355X streams them about 10% faster than default-policy loads.
  uint4 wb[U][2];
#define TP_WLOAD(SLOT, KS)                                                                     \
  _Pragma("unroll") for (int kh = 0; kh < 2; ++kh) wb[SLOT][kh] = __builtin_bit_cast(         \
      uint4, __builtin_amdgcn_raw_buffer_load_b128(                                            \
                 rw, (KS) < n ? wl + (unsigned)(KS) * 2048u + kh * 512u : 0x80000000u, 0, 2));

  // Staging: fragment f = c MB16 + mb of a chunk is loaded by wave f % SN.
  TokenRow sr[FPW];
#pragma unroll
  for (int j = 0; j < FPW; ++j) sr[j] = token_row(a, ((nw + j * SN) % MB16) * 16 + i, g);
  const int64_t xk0 = kbeg * KX * kTileK;
  uint4 st[FPW];
#define TP_KOFF(CH, J) (xk0 + ((int64_t)(CH) * C + (nw + (J) * SN) / MB16) * kTileK)
#define TP_SLOAD(CH) _Pragma("unroll") for (int j = 0; j < FPW; ++j) st[j] = sr[j].load(TP_KOFF(CH, j));
#define TP_SSTORE(BUF, CH)                             \
  _Pragma("unroll") for (int j = 0; j < FPW; ++j)      \
      xs[((BUF) * F + nw + j * SN) * 64 + lane] = sr[j].use(st[j], TP_KOFF(CH, j));

  f32x16_t acc[MB32];
#pragma unroll
  for (int t = 0; t < MB32; ++t) acc[t] = f32x16_t{};
#pragma unroll
  for (int u = 0; u < U; ++u) { TP_WLOAD(u, u) }
  TP_SLOAD(0)
  TP_SSTORE(0, 0)
  if (nch > 1) { TP_SLOAD(1) }
  __syncthreads();

  const int xsl = (fj >> 4) * 64 + fh * 16 + (fj & 15);
  for (int64_t ch = 0; ch < nch; ++ch) {
    const int buf = (int)(ch & 1);
    const int64_t c0 = ch * (C / KX);  // first weight step of the chunk
#pragma unroll
    for (int cw = 0; cw < C / KX; ++cw) {
      if constexpr (F8) {
        // 16-k block q of the step: bf16 k-step 2 cw + q / 2, k-half q % 2
        const uint4 w0 = wb[cw % U][0], w1 = wb[cw % U][1];
        const uint4 A[4] = {make_uint4(fp8x2_bf16x2<false>(w0.x, sc), fp8x2_bf16x2<true>(w0.x, sc),
                                       fp8x2_bf16x2<false>(w0.y, sc), fp8x2_bf16x2<true>(w0.y, sc)),
                            make_uint4(fp8x2_bf16x2<false>(w1.x, sc), fp8x2_bf16x2<true>(w1.x, sc),
                                       fp8x2_bf16x2<false>(w1.y, sc), fp8x2_bf16x2<true>(w1.y, sc)),
                            make_uint4(fp8x2_bf16x2<false>(w0.z, sc), fp8x2_bf16x2<true>(w0.z, sc),
                                       fp8x2_bf16x2<false>(w0.w, sc), fp8x2_bf16x2<true>(w0.w, sc)),
                            make_uint4(fp8x2_bf16x2<false>(w1.z, sc), fp8x2_bf16x2<true>(w1.z, sc),
                                       fp8x2_bf16x2<false>(w1.w, sc), fp8x2_bf16x2<true>(w1.w, sc))};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = 2 * cw + (q >> 1), kh = q & 1;
          uint4 xf[MB32];
#pragma unroll
          for (int t = 0; t < MB32; ++t) xf[t] = xs[((buf * C + c) * MB16 + 2 * t) * 64 + kh * 32 + xsl];
#pragma unroll
          for (int t = 0; t < MB32; ++t) acc[t] = mfma_32x32x16(A[q], xf[t], acc[t]);
        }
      } else {
        const int c = cw;
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          uint4 xf[MB32];
#pragma unroll
          for (int t = 0; t < MB32; ++t) xf[t] = xs[((buf * C + c) * MB16 + 2 * t) * 64 + kh * 32 + xsl];
#pragma unroll
          for (int t = 0; t < MB32; ++t) acc[t] = mfma_32x32x16(wb[c % U][kh], xf[t], acc[t]);
        }
      }
      TP_WLOAD(cw % U, c0 + cw + U)
    }
    if (ch + 1 < nch) {
      TP_SSTORE(buf ^ 1, ch + 1)
      if (ch + 2 < nch) { TP_SLOAD(ch + 2) }
    }
    __syncthreads();
  }
#undef TP_WLOAD
#undef TP_KOFF
#undef TP_SLOAD
#undef TP_SSTORE

  if (blk >= nblk) return;
  if (part == nullptr) {
#pragma unroll
    for (int t = 0; t < MB32; ++t) {
      const int64_t m = t * 32 + fj;
      if (m >= a.M) continue;
      const f32x16_t& v = acc[t];
      if constexpr (EPI == kEpiSwiglu) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int64_t col = blk * kTileN + 8 * q + 4 * fh;
          if (col < a.out_n)
            store_bf16x4(static_cast<uint16_t*>(a.out) + m * a.ldo + col, swiglu(v[4 * q], v[4 * q + 8]),
                         swiglu(v[4 * q + 1], v[4 * q + 9]), swiglu(v[4 * q + 2], v[4 * q + 10]),
                         swiglu(v[4 * q + 3], v[4 * q + 11]));
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t col = blk * 2 * kTileN + 8 * q + 4 * fh;
          if (col >= a.out_n) continue;
          if constexpr (EPI == kEpiBf16) {
            store_bf16x4(static_cast<uint16_t*>(a.out) + m * a.ldo + col, v[4 * q], v[4 * q + 1],
                         v[4 * q + 2], v[4 * q + 3]);
          } else {
            *reinterpret_cast<float4*>(static_cast<float*>(a.out) + m * a.ldo + col) =
                make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
          }
        }
      }
    }
  } else {
    const int64_t pld = a.ntiles * kTileN;
    float* p = part + (int64_t)blockIdx.y * a.M * pld;
#pragma unroll
    for (int t = 0; t < MB32; ++t) {
      const int64_t m = t * 32 + fj;
      if (m >= a.M) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t col = blk * 2 * kTileN + 8 * q + 4 * fh;
        if (col < pld)
          *reinterpret_cast<float4*>(p + m * pld + col) =
              make_float4(acc[t][4 * q], acc[t][4 * q + 1], acc[t][4 * q + 2], acc[t][4 * q + 3]);
      }
    }
  }
}

constexpr int FIX_U = 8;  // split partials loaded together by the fix-up

__device__ __forceinline__ void add4(float4& a, const float4& b) {
  a.x += b.x;
  a.y += b.y;
  a.z += b.z;
  a.w += b.w;
}

// Adds the G split partials in split order and applies the epilogue. One
// thread per 4 output columns of one token row.
template <int EPI>
__global__ __launch_bounds__(256) void gemv_fixup(LinearArgs a, const float* part, int G) {
  const int64_t pld = a.ntiles * kTileN;
  const int64_t ncol4 = (EPI == kEpiSwiglu ? pld / 2 : pld) / 4;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= a.M * ncol4) return;
  const int64_t m = idx / ncol4, c = (idx - m * ncol4) * 4;  // output column
  if (c >= a.out_n) return;
  const int64_t split = a.M * pld;
  if constexpr (EPI == kEpiSwiglu) {
    // Output column c of pair j = c / 16: gate column 32j + c % 16, up column 16 later.
    const int64_t gc = (c / kTileN) * 2 * kTileN + (c % kTileN);
    const float* pg = part + m * pld + gc;
    float4 gs = *reinterpret_cast<const float4*>(pg);
    float4 us = *reinterpret_cast<const float4*>(pg + kTileN);
    // Loads in groups of FIX_U, all in flight together (indices past the
    // last split re-read the last one and are not added); the adds stay in
    // split order.
    for (int y0 = 1; y0 < G; y0 += FIX_U) {
      float4 a4[FIX_U], b4[FIX_U];
#pragma unroll
      for (int u = 0; u < FIX_U; ++u) {
        const int64_t y = y0 + u < G ? y0 + u : G - 1;
        a4[u] = *reinterpret_cast<const float4*>(pg + y * split);
        b4[u] = *reinterpret_cast<const float4*>(pg + y * split + kTileN);
      }
#pragma unroll
      for (int u = 0; u < FIX_U; ++u)
        if (y0 + u < G) {
          add4(gs, a4[u]);
          add4(us, b4[u]);
        }
    }
    store_bf16x4(static_cast<uint16_t*>(a.out) + m * a.ldo + c, swiglu(gs.x, us.x),
                 swiglu(gs.y, us.y), swiglu(gs.z, us.z), swiglu(gs.w, us.w));
  } else {
    const float* pp = part + m * pld + c;
    float4 s = *reinterpret_cast<const float4*>(pp);
    for (int y0 = 1; y0 < G; y0 += FIX_U) {
      float4 b4[FIX_U];
#pragma unroll
      for (int u = 0; u < FIX_U; ++u) {
        const int64_t y = y0 + u < G ? y0 + u : G - 1;
        b4[u] = *reinterpret_cast<const float4*>(pp + y * split);
      }
#pragma unroll
      for (int u = 0; u < FIX_U; ++u)
        if (y0 + u < G) add4(s, b4[u]);
    }
    if constexpr (EPI == kEpiBf16) {
      store_bf16x4(static_cast<uint16_t*>(a.out) + m * a.ldo + c, s.x, s.y, s.z, s.w);
    } else {
      *reinterpret_cast<float4*>(static_cast<float*>(a.out) + m * a.ldo + c) = s;
    }
  }
}

// ---------------------------------------------------------------------------
// Launch plans
// ---------------------------------------------------------------------------

int pow2_at_least(int64_t v) {
  int p = 1;
  while (p < v && p < (1 << 20)) p <<= 1;
  return p;
}

template <int MB, int T, int EPI>
hipError_t launch_stream(const LinearArgs& a, hipStream_t s) {
  const int64_t groups = (a.ntiles + T - 1) / T;
  // Wavefronts per workgroup (each takes a contiguous k-range). Measured on
  // MI355X: a wave that streams a whole tile pair is fastest once the pairs
  // alone give ~900 waves; otherwise ~1500 (pairs) or ~2000 (single tiles)
  // waves in flight; at least 8 k-steps per wave.
  int S = (T == 2 && groups >= 768) ? 1 : pow2_at_least(((T == 2 ? 1536 : 2048) + groups - 1) / groups);
  if (S > 16) S = 16;
  while (S > 1 && a.ksteps / S < 8) S >>= 1;
  const int64_t chunk = (a.ksteps + S - 1) / S;
  const size_t lds = S > 1 ? (size_t)S * T * MB * 64 * sizeof(f32x4_t) : 0;
  const dim3 grid((unsigned)groups), block(64 * S);
  if (S <= 4) {
    hipLaunchKernelGGL((gemv_stream<MB, T, 8, EPI, 256>), grid, block, lds, s, a, chunk, rotate_starts(a.ksteps));
  } else if (S <= 8 && T == 2) {
    hipLaunchKernelGGL((gemv_stream<MB, T, 8, EPI, 512>), grid, block, lds, s, a, chunk, rotate_starts(a.ksteps));
  } else {
    hipLaunchKernelGGL((gemv_stream<MB, T, 4, EPI, 1024>), grid, block, lds, s, a, chunk, rotate_starts(a.ksteps));
  }
  return hipGetLastError();
}

// How gemv_shared splits the work: SN waves (one 32-column block each) per
// workgroup, G splits of the k-range of `per` k-steps each (a multiple of the
// chunk), G the smallest power of two that gives ~200 workgroups while each
// split keeps at least 2 chunks, and at most 16: beyond that the fix-up's
// reads cost more than the extra workgroups gain (the 70B TP = 8 QKV slice,
// 80 tiles, at M = 64: 32 splits 22 us, 16 splits 15.7 us, 8 splits 16.4 us).
struct SharedPlan {
  int G;
  int64_t per, groups;
};

constexpr int kSharedSN = 4;
constexpr int shared_chunk(int MB32) { return MB32 >= 2 ? 4 : 8; }

SharedPlan plan_shared(int64_t ntiles, int64_t ksteps, int MB32) {
  SharedPlan p;
  const int64_t nblk = (ntiles + 1) / 2;
  p.groups = (nblk + kSharedSN - 1) / kSharedSN;
  const int C = shared_chunk(MB32);
  int G = 1;
  while (p.groups * G < 200 && G < 16 && ksteps / (2 * G) >= 2 * C) G <<= 1;
  p.per = ((ksteps + G - 1) / G + C - 1) / C * C;
  p.G = (int)((ksteps + p.per - 1) / p.per);
  return p;
}

// F8: an 8-bit shard's weight steps are 64 k; the plan is made in bf16
// k-steps (the token chunks) and halved for the weight side.
template <int MB32, int EPI, bool F8 = false>
hipError_t launch_shared(const LinearArgs& a, float* ws, hipStream_t s) {
  constexpr int KX = F8 ? 2 : 1;
  const SharedPlan p = plan_shared(a.ntiles, a.ksteps * KX, MB32);
  constexpr int C = shared_chunk(MB32);
  constexpr int U = C / KX;
  const int64_t per = p.per / KX;  // p.per is a multiple of C
  if (p.G > 1 && ws == nullptr) return hipErrorInvalidValue;
  // A workgroup's weights are one buffer resource with 32-bit byte offsets.
  if ((int64_t)2 * kSharedSN * a.ksteps * 1024 >= (1LL << 31)) return hipErrorInvalidValue;
  float* part = p.G > 1 ? ws : nullptr;
  hipLaunchKernelGGL((gemv_shared<MB32, U, C, kSharedSN, EPI, F8>), dim3((unsigned)p.groups, (unsigned)p.G),
                     dim3(64 * kSharedSN), 0, s, a, per, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.G == 1) return e;
  const int64_t pld = a.ntiles * kTileN;
  const int64_t threads = a.M * (EPI == kEpiSwiglu ? pld / 2 : pld) / 4;
  hipLaunchKernelGGL((gemv_fixup<EPI>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, a,
                     static_cast<const float*>(ws), p.G);
  return hipGetLastError();
}

// 17 to 32 tokens over tile pairs that alone fill the GPU (256 or more),
// where the shared-token kernel would have to split K: two token blocks per
// wavefront in the streaming kernel, with no split and no fix-up launch. The
// tokens are re-read from L2 by every wavefront, which costs less than the
// fix-up only while K is short. Measured on the 70B TP = 8 shares at M = 24
// and 32: the O slice (K = 1024) went from 10.2 to 7.1 us; the down share
// (K = 3584) gained about 2 % alone and nothing inside the 8-rank step; every
// shape whose pairs do not fill the GPU was slower.
bool stream_two_blocks(int64_t M, int64_t ntiles, int64_t ksteps) {
  return M > 16 && M <= 32 && ntiles >= 512 && ksteps <= 64 && plan_shared(ntiles, ksteps, 1).G > 1;
}

template <int T, int EPI>
hipError_t launch_t(const LinearArgs& a, float* ws, hipStream_t s) {
  switch ((a.M + 15) / 16) {
    case 1: return launch_stream<1, T, EPI>(a, s);
    case 2:
      if (T == 2 && stream_two_blocks(a.M, a.ntiles, a.ksteps)) return launch_stream<2, T, EPI>(a, s);
      return launch_shared<1, EPI>(a, ws, s);
    case 3:
    case 4: return launch_shared<2, EPI>(a, ws, s);
    default: return hipErrorInvalidValue;
  }
}

// Launch plan of gemv8_stream (M <= 16): the same workgroup and wavefront counts as
// gemv_stream (pairs, S from the group count, at least 4 steps of 64 k per
// wavefront); the ring shrinks as the token blocks grow, keeping its
// registers bounded.
template <int MB, int T, int EPI>
hipError_t launch_stream8(const LinearArgs& a, hipStream_t s) {
  constexpr int U = MB == 1 ? 8 : (MB == 2 ? 4 : 2);
  const int64_t groups = a.ntiles / T;
  int S = (T == 2 && groups >= 768) ? 1 : pow2_at_least(((T == 2 ? 1536 : 2048) + groups - 1) / groups);
  if (S > 16) S = 16;
  while (S > 1 && a.ksteps / S < 4) S >>= 1;
  const int64_t chunk = (a.ksteps + S - 1) / S;
  const size_t lds = S > 1 ? (size_t)S * T * MB * 64 * sizeof(f32x4_t) : 0;
  const dim3 grid((unsigned)groups), block(64 * S);
  if (S <= 4) {
    hipLaunchKernelGGL((gemv8_stream<MB, T, U, EPI, 256>), grid, block, lds, s, a, chunk, rotate_starts(a.ksteps));
  } else if (S <= 8 && MB > 1) {
    // measured on the 70B TP = 8 shares: with several token blocks the deeper
    // ring of 8-wave workgroups wins; with one block, 16 waves of 4 steps
    hipLaunchKernelGGL((gemv8_stream<MB, T, U, EPI, 512>), grid, block, lds, s, a, chunk, rotate_starts(a.ksteps));
  } else {
    constexpr int U16 = MB == 1 ? 4 : (MB == 2 ? 2 : 1);  // 16 waves per workgroup: 128 VGPRs each
    hipLaunchKernelGGL((gemv8_stream<MB, T, U16, EPI, 1024>), grid, block, lds, s, a, chunk, rotate_starts(a.ksteps));
  }
  return hipGetLastError();
}

// Up to 16 tokens stream (one token block per wavefront); beyond, the
// shared-token kernel in its 8-bit form.
template <int T, int EPI>
hipError_t launch_t8(const LinearArgs& a, float* ws, hipStream_t s) {
  switch ((a.M + 15) / 16) {
    case 1: return launch_stream8<1, T, EPI>(a, s);
    case 2: return launch_shared<1, EPI, true>(a, ws, s);
    case 3:
    case 4: return launch_shared<2, EPI, true>(a, ws, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_gemv8(const LinearArgs& a, Epilogue epi, float* ws, hipStream_t s) {
  if (a.M <= 0 || a.ntiles == 0) return hipSuccess;
  if (a.wscale == nullptr || a.ntiles % 2) return hipErrorInvalidValue;
  switch (epi) {
    case kEpiSwiglu: return launch_t8<2, kEpiSwiglu>(a, ws, s);
    case kEpiBf16:
      return a.ntiles >= 512 ? launch_t8<2, kEpiBf16>(a, ws, s) : launch_t8<1, kEpiBf16>(a, ws, s);
    case kEpiF32:
      return a.ntiles >= 512 ? launch_t8<2, kEpiF32>(a, ws, s) : launch_t8<1, kEpiF32>(a, ws, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_split_fixup(const LinearArgs& a, Epilogue epi, const float* part, int G, hipStream_t s) {
  const int64_t pld = a.ntiles * kTileN;
  const int64_t threads = a.M * (epi == kEpiSwiglu ? pld / 2 : pld) / 4;
  const dim3 grid((unsigned)((threads + 255) / 256));
  switch (epi) {
    case kEpiSwiglu: hipLaunchKernelGGL(gemv_fixup<kEpiSwiglu>, grid, dim3(256), 0, s, a, part, G); break;
    case kEpiBf16: hipLaunchKernelGGL(gemv_fixup<kEpiBf16>, grid, dim3(256), 0, s, a, part, G); break;
    case kEpiF32: hipLaunchKernelGGL(gemv_fixup<kEpiF32>, grid, dim3(256), 0, s, a, part, G); break;
  }
  return hipGetLastError();
}

size_t gemv_workspace_bytes(int64_t M, int64_t ksteps, int64_t ntiles, Epilogue epi, bool f8) {
  if (M <= 16 || M > 64) return 0;
  if (!f8 && stream_two_blocks(M, ntiles, ksteps)) return 0;  // tile pairs (ntiles >= 512) stream, no split
  (void)epi;
  const SharedPlan p = plan_shared(ntiles, ksteps, (int)((M + 31) / 32));
  return p.G > 1 ? (size_t)p.G * M * ntiles * kTileN * sizeof(float) : 0;
}

hipError_t launch_gemv(const LinearArgs& a, Epilogue epi, float* ws, hipStream_t s) {
  if (a.M <= 0 || a.ntiles == 0) return hipSuccess;
  switch (epi) {
    case kEpiSwiglu: return launch_t<2, kEpiSwiglu>(a, ws, s);
    // Other kinds stream tile pairs only when the pairs still fill the GPU.
    case kEpiBf16:
      return a.ntiles >= 512 ? launch_t<2, kEpiBf16>(a, ws, s) : launch_t<1, kEpiBf16>(a, ws, s);
    case kEpiF32:
      return a.ntiles >= 512 ? launch_t<2, kEpiF32>(a, ws, s) : launch_t<1, kEpiF32>(a, ws, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace tpk
