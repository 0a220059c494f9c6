// Load-time cut of one rank's shard out of the full weight into the packed
// tile layout described in tp_internal.h ("AI Infrastructure series, Part 5",
// "What does it look like in vLLM ...": the weights are split as they load).
// 8-bit shards are quantised on the way ("AI Infrastructure series, Part 5",
// "Reason 2": a 70B model in 8-bit reads half the bytes per token): OCP FP8
// E4M3 codes with one power-of-two scale per output column.
#include "tp_internal.h"

namespace tpk {
namespace {

// Column i of packed tile nt: the column of the full weight it holds, or
// false for padding.
__device__ __forceinline__ bool source_col(const PackArgs& a, int64_t nt, int i, int64_t* wcol) {
  int64_t n;
  bool valid;
  if (a.gateup) {
    const int64_t col = (nt >> 1) * kTileN + i;  // output column within the gate (or up) half
    valid = col < a.out_n;
    n = (nt & 1) * a.out_n + col;
  } else {
    n = nt * kTileN + i;
    valid = n < a.shard_n;
  }
  *wcol = 0;
  if (!valid) return false;
  for (int r = 0; r < a.n_ranges; ++r) {
    if (n >= a.dst[r] && n < a.dst[r] + a.len[r]) {
      *wcol = a.src[r] + (n - a.dst[r]);
      return true;
    }
  }
  return false;
}

__global__ __launch_bounds__(256) void pack_kernel(PackArgs a, int64_t total_u4) {
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= total_u4) return;
  const int lane = (int)(c & 63);
  // 1 KiB index -> (tile pair, k-step, tile of the pair); see tile_index().
  const int64_t idx = c >> 6;
  const int64_t pair = idx / (2 * a.ksteps), rem = idx - pair * 2 * a.ksteps;
  const int64_t ks = rem >> 1, nt = 2 * pair + (rem & 1);
  const int g = lane >> 4, i = lane & 15;
  int64_t wcol;
  const bool valid = source_col(a, nt, i, &wcol);
  uint16_t v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int64_t k = ks * kTileK + g * 8 + e;
    v[e] = (valid && k < a.shard_k) ? a.W[(a.row_begin + k) * a.ldw + wcol] : (uint16_t)0;
  }
  uint4 o;
  o.x = v[0] | ((uint32_t)v[1] << 16);
  o.y = v[2] | ((uint32_t)v[3] << 16);
  o.z = v[4] | ((uint32_t)v[5] << 16);
  o.w = v[6] | ((uint32_t)v[7] << 16);
  a.out[c] = o;
}

// ---------------------------------------------------------------------------
// 8-bit shards (TP_W_FP8_E4M3).
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Pass 1: the largest |w| of each packed column over the shard's rows, then
// its scale. A workgroup of kScaleWaves wavefronts takes 64 columns (lane =
// column); wavefront w reads rows w, w + kScaleWaves, ..., and the maxima
// meet in LDS (a maximum does not depend on the order). e = the smallest
// integer with amax <= 448 2^e: with amax = f 2^x, f in [0.5, 1) and
// 448 = 0.875 2^9, e = x - 9 if f <= 0.875, else x - 8. Padding and all-zero
// columns get 2^0.
constexpr int kScaleWaves = 16;

__global__ __launch_bounds__(64 * kScaleWaves) void pack8_scale_kernel(PackArgs a) {
  __shared__ float red[kScaleWaves][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t pc = (int64_t)blockIdx.x * 64 + lane;
  int64_t wcol;
  float amax = 0.0f;
  if (pc < a.ntiles * kTileN && source_col(a, pc / kTileN, (int)(pc % kTileN), &wcol)) {
#pragma unroll 4
    for (int64_t k = w; k < a.shard_k; k += kScaleWaves)
      amax = fmaxf(amax, fabsf(bf16_bits_to_f32(a.W[(a.row_begin + k) * a.ldw + wcol])));
  }
  red[w][lane] = amax;
  __syncthreads();
  if (w != 0 || pc >= a.ntiles * kTileN) return;
  for (int j = 1; j < kScaleWaves; ++j) amax = fmaxf(amax, red[j][lane]);
  int e = 0;
  if (amax > 0.0f) {
    int x;
    const float f = frexpf(amax, &x);
    e = f <= 0.875f ? x - 9 : x - 8;
  }
  a.scales[pc] = ldexpf(1.0f, e);
}

// E4M3 code of v, |v| <= 448, round to nearest, ties to even, sign kept.
// v = sig 2^(x - 23) (sig with its hidden bit); the code spacing at this
// magnitude is 2^q, q = max(x, -6) - 3, and n = v / 2^q is rounded to an
// integer: n in [8, 16] is a normal code (16 carries into the exponent),
// n in [0, 8] below 2^-6 is a subnormal code (8 is the smallest normal).
__device__ __forceinline__ uint32_t e4m3_rne(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t mag = u & 0x7FFFFFFFu;
  if (mag == 0) return sign;
  const int E = (int)(mag >> 23);
  const uint32_t sig = (mag & 0x7FFFFFu) | (E ? 0x800000u : 0u);
  const int x = E ? E - 127 : -126;
  const int q = (x < -6 ? -6 : x) - 3;
  const int sh = q - x + 23;  // >= 20
  if (sh >= 26) return sign;  // below a quarter of the smallest spacing: rounds to 0
  uint32_t n = sig >> sh;
  const uint32_t r = sig & ((1u << sh) - 1u), half = 1u << (sh - 1);
  if (r > half || (r == half && (n & 1u))) ++n;
  if (x < -6) return sign | n;  // subnormal codes 0..7, or 8 = 2^-6
  int ex = x + 7;
  if (n == 16) {
    n = 8;
    ++ex;
  }
  return sign | ((uint32_t)ex << 3) | (n - 8);
}

// Pass 2: one thread per 16-byte lane slot of a 1 KiB tile of 16 columns x
// 64 k: bytes 0..7 hold k = 64 s + 8 g + e, bytes 8..15 k = 64 s + 32 + 8 g + e.
__global__ __launch_bounds__(256) void pack8_kernel(PackArgs a, int64_t total_u4) {
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= total_u4) return;
  const int lane = (int)(c & 63);
  const int64_t idx = c >> 6;
  const int64_t pair = idx / (2 * a.ksteps), rem = idx - pair * 2 * a.ksteps;
  const int64_t s = rem >> 1, nt = 2 * pair + (rem & 1);
  const int g = lane >> 4, i = lane & 15;
  int64_t wcol;
  const bool valid = source_col(a, nt, i, &wcol);
  const float inv = 1.0f / a.scales[nt * kTileN + i];  // 2^-e: exact
  uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int b = 0; b < 16; ++b) {
    const int64_t k = s * kTileK8 + (b >> 3) * kTileK + g * 8 + (b & 7);
    const float v = (valid && k < a.shard_k) ? bf16_bits_to_f32(a.W[(a.row_begin + k) * a.ldw + wcol]) : 0.0f;
    w[b >> 2] |= e4m3_rne(v * inv) << (8 * (b & 3));
  }
  a.out[c] = make_uint4(w[0], w[1], w[2], w[3]);
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two E4M3 codes (word `hi` of d) -> two bf16 values decode * scale, packed:
// the scaled values are exact in fp32 with at most 4 significant bits, so
// their upper halves are the bf16 bits.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t d, float scale) {
  const f32x2_t f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(d, scale, HI);
  return __builtin_amdgcn_perm(__float_as_uint(f[1]), __float_as_uint(f[0]), 0x07060302u);
}

// Dequantise into the bf16 layout: output 1 KiB tile (nt, ks) lane l is half
// ks & 1 of the 8-bit tile (nt, ks >> 1), same lane.
__global__ __launch_bounds__(256) void dequant8_kernel(const uint4* W8, const float* scales,
                                                       int64_t ksteps8, uint4* W16, int64_t total_u4) {
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= total_u4) return;
  const int lane = (int)(c & 63);
  const int64_t ksteps16 = 2 * ksteps8;
  const int64_t idx = c >> 6;
  const int64_t pair = idx / (2 * ksteps16), rem = idx - pair * 2 * ksteps16;
  const int64_t ks = rem >> 1, nt = 2 * pair + (rem & 1);
  const uint4 q = W8[tile_index(nt, ks >> 1, ksteps8) * kTileU4 + lane];
  const float sc = scales[nt * kTileN + (lane & 15)];
  const uint32_t d0 = (ks & 1) ? q.z : q.x, d1 = (ks & 1) ? q.w : q.y;
  W16[c] = make_uint4(fp8x2_to_bf16x2<false>(d0, sc), fp8x2_to_bf16x2<true>(d0, sc),
                      fp8x2_to_bf16x2<false>(d1, sc), fp8x2_to_bf16x2<true>(d1, sc));
}

// TP_DGRAD: the transposed shard T = W_r^T in the bf16 layout. Output column
// n = 16 nt + i is forward row row_begin + n; contraction index k is forward
// shard column k, the column of W the forward's ranges map it to.
__global__ __launch_bounds__(256) void pack_dgrad_kernel(PackArgs a, int64_t total_u4) {
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= total_u4) return;
  const int lane = (int)(c & 63);
  const int64_t idx = c >> 6;
  const int64_t pair = idx / (2 * a.ksteps), rem = idx - pair * 2 * a.ksteps;
  const int64_t ks = rem >> 1, nt = 2 * pair + (rem & 1);
  const int g = lane >> 4, i = lane & 15;
  const int64_t n = nt * kTileN + i;
  const int64_t k0 = ks * kTileK + g * 8;  // the lane's 8 contraction indices k0 .. k0 + 7
  // When the octet lies inside one column range, its 8 values are 8
  // consecutive elements of forward row n: one 16-byte load if aligned.
  if (n < a.shard_n && k0 + 8 <= a.shard_k) {
    for (int r = 0; r < a.n_ranges; ++r) {
      if (k0 >= a.dst[r] && k0 + 8 <= a.dst[r] + a.len[r]) {
        const uint16_t* p = a.W + (a.row_begin + n) * a.ldw + a.src[r] + (k0 - a.dst[r]);
        if (((uintptr_t)p & 15) == 0) {
          a.out[c] = *reinterpret_cast<const uint4*>(p);
          return;
        }
      }
    }
  }
  uint16_t v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int64_t k = k0 + e;
    int64_t wcol = -1;
    if (n < a.shard_n && k < a.shard_k) {
      for (int r = 0; r < a.n_ranges; ++r)
        if (k >= a.dst[r] && k < a.dst[r] + a.len[r]) wcol = a.src[r] + (k - a.dst[r]);
    }
    v[e] = wcol >= 0 ? a.W[(a.row_begin + n) * a.ldw + wcol] : (uint16_t)0;
  }
  a.out[c] = make_uint4(v[0] | ((uint32_t)v[1] << 16), v[2] | ((uint32_t)v[3] << 16),
                        v[4] | ((uint32_t)v[5] << 16), v[6] | ((uint32_t)v[7] << 16));
}

}  // namespace

hipError_t launch_pack_dgrad(const PackArgs& a, hipStream_t s) {
  const int64_t total = a.ksteps * a.ntiles * kTileU4;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(pack_dgrad_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a, total);
  return hipGetLastError();
}

hipError_t launch_pack8(const PackArgs& a, hipStream_t s) {
  const int64_t cols = a.ntiles * kTileN;
  if (cols == 0) return hipSuccess;
  hipLaunchKernelGGL(pack8_scale_kernel, dim3((unsigned)((cols + 63) / 64)), dim3(64 * kScaleWaves), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t total = a.ksteps * a.ntiles * kTileU4;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(pack8_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a, total);
  return hipGetLastError();
}

hipError_t launch_dequant8(const uint4* W8, const float* scales, int64_t ksteps8, int64_t ntiles,
                           uint4* W16, hipStream_t s) {
  const int64_t total = 2 * ksteps8 * ntiles * kTileU4;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(dequant8_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, W8,
                     scales, ksteps8, W16, total);
  return hipGetLastError();
}

hipError_t launch_pack(const PackArgs& a, hipStream_t s) {
  const int64_t total = a.ksteps * a.ntiles * kTileU4;
  if (total == 0) return hipSuccess;
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a, total);
  return hipGetLastError();
}

}  // namespace tpk
