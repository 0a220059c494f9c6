// Decode path (M <= 64 tokens): Y = X W_shard streams every weight byte once
// and is bound by HBM bandwidth ("AI Infrastructure series, Part 5",
// "Reason 2": in decode every token needs a read of every weight; a rank of t
// reads 1/t of them).
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
//  * gemv_shared (16 < M <= 64): at larger M every wavefront would re-read
//    all the token fragments from L2 for its own tiles, which caps the rate.
//    Here SN wavefronts of a workgroup own different tiles over the same
//    k-range and share each chunk of C token k-steps through LDS (double
//    buffered, one barrier per chunk; the weight ring stays in flight across
//    it). When the column count is too small to fill the GPU, the k-range is
//    also split over G workgroups; each writes an fp32 partial and
//    gemv_fixup adds them in split order and applies the epilogue.
#include "tp_internal.h"

namespace tpk {
namespace {

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

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
__global__ __launch_bounds__(LB) void gemv_stream(LinearArgs a, int64_t chunk) {
  extern __shared__ f32x4_t red[];  // [S][T][MB][64]
  const int lane = threadIdx.x & 63, wave = wave_id(), S = blockDim.x >> 6;
  const int g = lane >> 4, i = lane & 15;
  const int64_t tile0 = (int64_t)blockIdx.x * T;
  const int64_t ksteps = a.ksteps;
  const int64_t k0 = (int64_t)wave * chunk;
  const int64_t k1 = k0 + chunk < ksteps ? k0 + chunk : ksteps;
  const int64_t n = k1 > k0 ? k1 - k0 : 0;
  const uint4* wp = a.W + (tile0 * ksteps + (n > 0 ? k0 : 0)) * kTileU4 + lane;
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
#define TP_FILL(SLOT, STEP)                                                                \
  {                                                                                        \
    _Pragma("unroll") for (int t = 0; t < T; ++t)                                          \
        wb[SLOT][t] = load_w(wp + ((int64_t)t * ksteps + (STEP)) * kTileU4);               \
    _Pragma("unroll") for (int mb = 0; mb < MB; ++mb)                                      \
        xb[SLOT][mb] = xr[mb].load(xk0 + (STEP) * kTileK);                                 \
  }
#define TP_MMA(SLOT, STEP)                                                                 \
  {                                                                                        \
    _Pragma("unroll") for (int mb = 0; mb < MB; ++mb) {                                    \
      const uint4 xv = xr[mb].use(xb[SLOT][mb], xk0 + (STEP) * kTileK);                    \
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
// gemv_shared
// ---------------------------------------------------------------------------

// Partial sums of split y go to part + y * M * pld (pld = ntiles * 16 columns).
template <int MB, int T, int U, int C, int SN, int EPI>
__global__ __launch_bounds__(64 * SN) void gemv_shared(LinearArgs a, int64_t per, float* part) {
  static_assert(C % U == 0, "the ring must divide the chunk");
  constexpr int F = C * MB;               // token fragments per chunk
  constexpr int FPW = (F + SN - 1) / SN;  // staged by each wave
  __shared__ uint4 xs[2 * F * 64];
  const int lane = threadIdx.x & 63, nw = wave_id();
  const int g = lane >> 4, i = lane & 15;
  const int64_t tile0 = (int64_t)blockIdx.x * (SN * T) + nw * T;
  const int64_t ksteps = a.ksteps;
  const int64_t kbeg = (int64_t)blockIdx.y * per;
  const int64_t kend = kbeg + per < ksteps ? kbeg + per : ksteps;
  const int64_t n = kend > kbeg ? kend - kbeg : 0;  // uniform over the workgroup
  const int64_t nch = (n + C - 1) / C;
  const uint4* wp = a.W + (tile0 * ksteps + (n > 0 ? kbeg : 0)) * kTileU4 + lane;

  // Staging sources: fragment f = c * MB + mb of a chunk is loaded by wave f % SN.
  TokenRow sr[FPW];
  int sc[FPW];
#pragma unroll
  for (int j = 0; j < FPW; ++j) {
    const int f = nw + j * SN;
    const int fc = f < F ? f : 0;
    sr[j] = token_row(a, (fc % MB) * 16 + i, g);
    sc[j] = fc / MB;
  }
  const int64_t xk0 = kbeg * kTileK;

  f32x4_t acc[T][MB];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[t][mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  uint4 wb[U][T], st[FPW];

#define TP_STAGE_LOAD(CH)                                  \
  _Pragma("unroll") for (int j = 0; j < FPW; ++j)          \
      st[j] = sr[j].get(xk0 + ((int64_t)(CH) * C + sc[j]) * kTileK);
#define TP_STAGE_STORE(BUF)                                \
  _Pragma("unroll") for (int j = 0; j < FPW; ++j) {        \
    const int f = nw + j * SN;                             \
    if (f < F) xs[((BUF) * F + f) * 64 + lane] = st[j];    \
  }

#pragma unroll
  for (int u = 0; u < U; ++u)
    if (u < n)
#pragma unroll
      for (int t = 0; t < T; ++t) wb[u][t] = load_w(wp + ((int64_t)t * ksteps + u) * kTileU4);
  if (nch > 0) {
    TP_STAGE_LOAD(0)
    TP_STAGE_STORE(0)
  }
  if (nch > 1) {
    TP_STAGE_LOAD(1)
  }
  __syncthreads();

  for (int64_t ch = 0; ch < nch; ++ch) {
    const int buf = (int)(ch & 1);
    const int64_t c0 = ch * C;
    if (c0 + C + U <= n) {
      // Every step of this chunk and every refill target exist: no branches.
#pragma unroll
      for (int c = 0; c < C; ++c) {
        uint4 xf[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) xf[mb] = xs[((buf * C + c) * MB + mb) * 64 + lane];
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) acc[t][mb] = mfma_16x16x32(wb[c % U][t], xf[mb], acc[t][mb]);
#pragma unroll
        for (int t = 0; t < T; ++t)
          wb[c % U][t] = load_w(wp + ((int64_t)t * ksteps + c0 + c + U) * kTileU4);
      }
    } else {
#pragma unroll
      for (int c = 0; c < C; ++c) {
        if (c0 + c < n) {
          uint4 xf[MB];
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) xf[mb] = xs[((buf * C + c) * MB + mb) * 64 + lane];
#pragma unroll
          for (int t = 0; t < T; ++t)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) acc[t][mb] = mfma_16x16x32(wb[c % U][t], xf[mb], acc[t][mb]);
          if (c0 + c + U < n)
#pragma unroll
            for (int t = 0; t < T; ++t)
              wb[c % U][t] = load_w(wp + ((int64_t)t * ksteps + c0 + c + U) * kTileU4);
        }
      }
    }
    if (ch + 1 < nch) {
      TP_STAGE_STORE(buf ^ 1)
      if (ch + 2 < nch) {
        TP_STAGE_LOAD(ch + 2)
      }
    }
    __syncthreads();
  }
#undef TP_STAGE_LOAD
#undef TP_STAGE_STORE

  if (part == nullptr) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      f32x4_t v[T];
#pragma unroll
      for (int t = 0; t < T; ++t) v[t] = acc[t][mb];
      epilogue<EPI, T>(a, v, mb * 16 + i, tile0, g);
    }
  } else {
    const int64_t pld = a.ntiles * kTileN;
    float* p = part + (int64_t)blockIdx.y * a.M * pld;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int64_t m = mb * 16 + i;
      if (m >= a.M) continue;
#pragma unroll
      for (int t = 0; t < T; ++t)
        *reinterpret_cast<float4*>(p + m * pld + (tile0 + t) * kTileN + g * 4) =
            make_float4(acc[t][mb][0], acc[t][mb][1], acc[t][mb][2], acc[t][mb][3]);
    }
  }
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
    for (int y = 1; y < G; ++y) {
      const float4 a4 = *reinterpret_cast<const float4*>(pg + y * split);
      const float4 b4 = *reinterpret_cast<const float4*>(pg + y * split + kTileN);
      gs.x += a4.x;
      gs.y += a4.y;
      gs.z += a4.z;
      gs.w += a4.w;
      us.x += b4.x;
      us.y += b4.y;
      us.z += b4.z;
      us.w += b4.w;
    }
    store_bf16x4(static_cast<uint16_t*>(a.out) + m * a.ldo + c, swiglu(gs.x, us.x),
                 swiglu(gs.y, us.y), swiglu(gs.z, us.z), swiglu(gs.w, us.w));
  } else {
    const float* pp = part + m * pld + c;
    float4 s = *reinterpret_cast<const float4*>(pp);
    for (int y = 1; y < G; ++y) {
      const float4 b4 = *reinterpret_cast<const float4*>(pp + y * split);
      s.x += b4.x;
      s.y += b4.y;
      s.z += b4.z;
      s.w += b4.w;
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
  const int64_t groups = a.ntiles / T;
  // Enough wavefronts for ~1500 rings in flight, at most 16 per workgroup,
  // and at least 8 k-steps each.
  int S = pow2_at_least((1536 + groups - 1) / groups);
  if (S > 16) S = 16;
  while (S > 1 && a.ksteps / S < 8) S >>= 1;
  const int64_t chunk = (a.ksteps + S - 1) / S;
  const size_t lds = S > 1 ? (size_t)S * T * MB * 64 * sizeof(f32x4_t) : 0;
  const dim3 grid((unsigned)groups), block(64 * S);
  if (S <= 4) {
    hipLaunchKernelGGL((gemv_stream<MB, T, 8, EPI, 256>), grid, block, lds, s, a, chunk);
  } else if (S <= 8) {
    hipLaunchKernelGGL((gemv_stream<MB, T, 8, EPI, 512>), grid, block, lds, s, a, chunk);
  } else {
    hipLaunchKernelGGL((gemv_stream<MB, T, 4, EPI, 1024>), grid, block, lds, s, a, chunk);
  }
  return hipGetLastError();
}

// How gemv_shared splits the work: SN waves per workgroup, G splits of the
// k-range of `per` k-steps each (a multiple of the chunk).
struct SharedPlan {
  int SN, G;
  int64_t per;
};

constexpr int shared_chunk(int MB) { return MB >= 4 ? 4 : 8; }

SharedPlan plan_shared(int64_t ntiles, int64_t ksteps, int MB, int T) {
  SharedPlan p;
  p.SN = 8;
  while (p.SN > 1 && (ntiles / T) % p.SN) p.SN >>= 1;
  const int64_t groups = ntiles / (T * p.SN);
  const int C = shared_chunk(MB);
  // Aim for ~224+ workgroups while keeping >= 4 chunks of k per split.
  int G = 1;
  while (groups * G < 224 && ksteps / (2 * G) >= 4 * C) G <<= 1;
  p.per = ((ksteps + G - 1) / G + C - 1) / C * C;
  p.G = (int)((ksteps + p.per - 1) / p.per);
  return p;
}

template <int MB, int T, int EPI>
hipError_t launch_shared(const LinearArgs& a, float* ws, hipStream_t s) {
  const SharedPlan p = plan_shared(a.ntiles, a.ksteps, MB, T);
  constexpr int C = shared_chunk(MB);
  constexpr int U = MB >= 4 ? 4 : 8;
  if (p.G > 1 && ws == nullptr) return hipErrorInvalidValue;
  float* part = p.G > 1 ? ws : nullptr;
  const dim3 grid((unsigned)(a.ntiles / (T * p.SN)), (unsigned)p.G);
  switch (p.SN) {
    case 8: hipLaunchKernelGGL((gemv_shared<MB, T, U, C, 8, EPI>), grid, dim3(512), 0, s, a, p.per, part); break;
    case 4: hipLaunchKernelGGL((gemv_shared<MB, T, U, C, 4, EPI>), grid, dim3(256), 0, s, a, p.per, part); break;
    case 2: hipLaunchKernelGGL((gemv_shared<MB, T, U, C, 2, EPI>), grid, dim3(128), 0, s, a, p.per, part); break;
    default: hipLaunchKernelGGL((gemv_shared<MB, T, U, C, 1, EPI>), grid, dim3(64), 0, s, a, p.per, part); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.G == 1) return e;
  const int64_t pld = a.ntiles * kTileN;
  const int64_t threads = a.M * (EPI == kEpiSwiglu ? pld / 2 : pld) / 4;
  hipLaunchKernelGGL((gemv_fixup<EPI>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, a,
                     static_cast<const float*>(ws), p.G);
  return hipGetLastError();
}

template <int T, int EPI>
hipError_t launch_t(const LinearArgs& a, float* ws, hipStream_t s) {
  switch ((a.M + 15) / 16) {
    case 1: return launch_stream<1, T, EPI>(a, s);
    case 2: return launch_shared<2, T, EPI>(a, ws, s);
    case 3: return launch_shared<3, T, EPI>(a, ws, s);
    case 4: return launch_shared<4, T, EPI>(a, ws, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

size_t gemv_workspace_bytes(int64_t M, int64_t ksteps, int64_t ntiles, Epilogue epi) {
  if (M <= 16 || M > 64) return 0;
  const int MB = (int)((M + 15) / 16);
  const SharedPlan p = plan_shared(ntiles, ksteps, MB, epi == kEpiSwiglu ? 2 : 1);
  return p.G > 1 ? (size_t)p.G * M * ntiles * kTileN * sizeof(float) : 0;
}

hipError_t launch_gemv(const LinearArgs& a, Epilogue epi, float* ws, hipStream_t s) {
  if (a.M <= 0 || a.ntiles == 0) return hipSuccess;
  switch (epi) {
    case kEpiSwiglu: return launch_t<2, kEpiSwiglu>(a, ws, s);
    case kEpiBf16: return launch_t<1, kEpiBf16>(a, ws, s);
    case kEpiF32: return launch_t<1, kEpiF32>(a, ws, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace tpk
