// Internal declarations of the HIP library: packed-layout constants, device
// helpers and kernel launchers. Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "tp_shard.h"

namespace tpk {

// Packed weight layout (written by tp_shard_pack, read by every linear):
// the shard, zero-padded to [packed_k x packed_n] (packed_n a multiple of
// 32), is cut into tiles of kTileN output columns x kTileK k, 1 KiB each.
// Tiles come in pairs (2p, 2p + 1) whose k-steps alternate: tile (nt, ks)
// sits at 1 KiB index tile_index(nt, ks) = ((nt >> 1) * ksteps + ks) * 2 +
// (nt & 1). A pair's whole k range (32 output columns) is one contiguous
// run, read front to back as a single stream. Inside a tile, lane l = 16 g + i of a wavefront
// owns 16 bytes at offset 16 l: the 8 values W[ks*32 + 8g + e][nt*16 + i],
// e = 0..7 -- exactly the A operand of v_mfma_f32_16x16x32_bf16 with output
// columns as MFMA rows. A wavefront therefore loads a whole tile with one
// fully coalesced 1 KiB dwordx4 load. For TP_GATEUP_COL the gate and up tiles
// of the same 16 outputs are interleaved: packed tile 2j is gate tile j and
// 2j + 1 is up tile j, so SwiGLU pairs sit in the same lanes.
constexpr int kTileN = 16;
constexpr int kTileK = 32;
constexpr int kTileU4 = 64;  // uint4 per tile
// 8-bit shards (TP_W_FP8_E4M3): tiles of 16 columns x 64 k, also 1 KiB, in
// the same pair-interleaved order (tile_index with k-steps of 64). Lane l =
// 16 g + i owns 16 bytes: the codes of column i at k = 64 s + 8 g + e
// (bytes 0..7) and k = 64 s + 32 + 8 g + e (bytes 8..15), e = 0..7, i.e. the
// A operands of two consecutive bf16 k-steps. The packed_n fp32 column
// scales 2^e_n follow the codes.
constexpr int kTileK8 = 64;

// 1 KiB index of tile (nt, ks) in the packed layout.
__host__ __device__ __forceinline__ int64_t tile_index(int64_t nt, int64_t ks, int64_t ksteps) {
  return ((nt >> 1) * ksteps + ks) * 2 + (nt & 1);
}

enum Epilogue { kEpiBf16 = 0, kEpiSwiglu = 1, kEpiF32 = 2 };

// One linear: out = epilogue(X W_shard).
struct LinearArgs {
  const uint16_t* X;  // [M x K] bf16, leading dim ldx
  int64_t ldx;
  int64_t M;
  int64_t K;          // valid k (shard_k); packed tiles are zero past it
  const uint4* W;     // packed tiles
  int64_t ksteps;     // packed_k / kTileK
  int64_t ntiles;     // packed_n / kTileN
  void* out;          // bf16 or fp32 [M x out_n], leading dim ldo
  int64_t ldo;
  int64_t out_n;      // valid output columns
  const float* wscale;  // 8-bit shards: the ntiles kTileN column scales 2^e_n; else null
};

struct PackArgs {
  const uint16_t* W;
  int64_t ldw;
  uint4* out;
  int64_t row_begin, shard_k, shard_n, out_n;
  int64_t ksteps, ntiles;
  int64_t src[3], len[3], dst[3];
  int32_t n_ranges;
  int32_t gateup;
  float* scales;      // 8-bit shards: where the column scales go (ksteps counts 64-k steps); else null
};

hipError_t launch_pack(const PackArgs& a, hipStream_t s);
// 8-bit shards: column scales, then the E4M3 codes (a.scales must be set).
hipError_t launch_pack8(const PackArgs& a, hipStream_t s);
// 8-bit shard -> the bf16 packed layout of the dequantised weights (ksteps16
// = 2 ksteps8 k-steps of 32), for the prefill GEMM.
hipError_t launch_dequant8(const uint4* W8, const float* scales, int64_t ksteps8, int64_t ntiles,
                           uint4* W16, hipStream_t s);
// TP_DGRAD: the transposed shard of a forward plan, in the bf16 layout
// (a.shard_k = forward shard_n is the contraction, a.shard_n = forward
// shard_k the output columns; rows and column ranges are the forward's).
hipError_t launch_pack_dgrad(const PackArgs& a, hipStream_t s);
// dW [K x N] fp32 = A^T dC over M tokens (A [M x K], dC [M x N] bf16).
hipError_t launch_wgrad(const uint16_t* A, int64_t lda, const uint16_t* dC, int64_t lddc, int64_t M,
                        int64_t K, int64_t N, float* dW, int64_t lddw, hipStream_t s);
// [dG | dU] bf16 from [G | U] bf16 and dH fp32.
hipError_t launch_swiglu_bwd(const uint16_t* GU, int64_t ldgu, const float* dH, int64_t lddh,
                             int64_t M, int64_t w, uint16_t* dGU, int64_t lddgu, hipStream_t s);
// Decode path for 8-bit shards, 1 <= M <= 64. `ws` as for launch_gemv, with
// gemv_workspace_bytes(M, 2 ksteps, ntiles, epi, true) (the plan counts bf16
// k-steps).
hipError_t launch_gemv8(const LinearArgs& a, Epilogue epi, float* ws, hipStream_t s);
// Decode path. `ws` must hold gemv_workspace_bytes() bytes (fp32 split
// partials) when that is non-zero.
hipError_t launch_gemv(const LinearArgs& a, Epilogue epi, float* ws, hipStream_t s);
size_t gemv_workspace_bytes(int64_t M, int64_t ksteps, int64_t ntiles, Epilogue epi, bool f8 = false);
// Prefill path. `ws` must hold gemm_workspace_bytes() bytes (fp32 split-K
// partials, when the output tiles alone do not fill the GPU) when that is
// non-zero.
hipError_t launch_gemm(const LinearArgs& a, Epilogue epi, float* ws, hipStream_t s);
size_t gemm_workspace_bytes(int64_t M, int64_t ldx, int64_t ksteps, int64_t ntiles);
// Adds G fp32 split partials part[y] ([M x ntiles kTileN], split order) and
// applies the epilogue into a.out.
hipError_t launch_split_fixup(const LinearArgs& a, Epilogue epi, const float* part, int G, hipStream_t s);
hipError_t launch_reduce(const float* P, int64_t stride, int32_t t, int64_t M, int64_t N,
                         int64_t ldp, float* Y, int64_t ldy, hipStream_t s);
hipError_t launch_gather(const uint16_t* Xs, int64_t stride, int32_t t, int64_t Mt, int64_t N,
                         int64_t ldb, uint16_t* X, int64_t ldx, hipStream_t s);

// Attention core on a rank's heads (attention.hip). Rows s q_len .. s q_len +
// q_len - 1 of QKV (the rank's [Q_r | K_r | V_r]) and of A belong to sequence
// s; its cache is slot slot[s] and holds kv_len[s] positions once its new
// tokens are in. Caches are [n_slots x nkv x L_max x D] bf16, K and V apart.
struct AttnArgs {
  const uint16_t* QKV;
  int64_t ldqkv;
  const int32_t* kv_len;
  const int32_t* slot;
  const uint16_t* Kc;
  const uint16_t* Vc;
  uint16_t* Kw;  // append: the caches written
  uint16_t* Vw;
  int64_t n_slots, L_max;
  int32_t S, q_len, nq, nkv, G, D;  // G: query heads per key-value head of the rank
  int32_t max_kv;                   // kv_len entries above it (or below q_len) mark a sequence invalid
  uint16_t* A;
  int64_t lda;
  float* ws;       // decode: per-chunk partials
  int32_t nchunk;  // decode: chunks of positions per (sequence, key-value head)
  int32_t npw;     // decode: 512-position passes per chunk (1, 2, 4 or 8)
  float qscale;    // log2(e) / sqrt(D)
};

constexpr int kAttnDecodeRows = 16;    // query rows (heads x tokens) of one decode workgroup
constexpr int kAttnDecodePass = 512;   // positions per decode pass of a workgroup
size_t attn_decode_ws_bytes(int64_t S, int64_t nkv, int64_t nchunk, int D);
// Chunks per (sequence, key-value head) and passes per chunk for a decode call.
void attn_decode_split(int64_t S, int64_t nkv, int64_t max_kv, int32_t& nchunk, int32_t& npw);
hipError_t launch_kv_append(const AttnArgs& a, hipStream_t s);
hipError_t launch_attention(const AttnArgs& a, bool decode, hipStream_t s);

}  // namespace tpk

#ifdef __HIPCC__
namespace tpk {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// D = A B + C on one 16x16x32 bf16 MFMA. A: 16 output columns x 32 k (a
// packed weight tile), B: 32 k x 16 tokens. Lane l = 16 g + i supplies
// A[i][8g..8g+7] and B[8g..8g+7][i] and receives D[4g + r][i], r = 0..3.
__device__ __forceinline__ f32x4_t mfma_16x16x32(uint4 a, uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// fp32 -> bf16 bits, round to nearest, ties to even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// SiLU(g) * u with SiLU(g) = g / (1 + e^-g). For g -> -inf, e^-g = inf and
// the quotient is -0; for g -> +inf it is g.
__device__ __forceinline__ float swiglu(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// Four values rounded to bf16 and packed in order.
__device__ __forceinline__ uint2 bf16x4(float a, float b, float c, float d) {
  uint2 v;
  v.x = (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
  v.y = (uint32_t)f32_to_bf16(c) | ((uint32_t)f32_to_bf16(d) << 16);
  return v;
}

__device__ __forceinline__ void store_bf16x4(uint16_t* p, float a, float b, float c, float d) {
  *reinterpret_cast<uint2*>(p) = bf16x4(a, b, c, d);
}

}  // namespace tpk
#endif
