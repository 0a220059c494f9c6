// Attention core on one tensor-parallel rank's heads, with the rank's share of
// the KV cache ("Tensor vs Pipeline Parallelism", "Tensor parallelism: split
// inside each layer": the heads are shared out over the ranks and a rank
// keeps the KV cache of its own heads; "AI Infrastructure series, Part 5",
// "How does tensor parallelism split a layer?": ranks beyond the key-value
// head count hold copies of a key-value head). Per query head: softmax(q k^T / sqrt(D)) v over the positions of
// its sequence up to its own (causal), with the rank's key-value head of its
// group. No position encoding, no bias.
//
// Kernels:
//  * kv_append_kernel: the new tokens' K and V rows into their cache slots.
//  * attn_decode_kernel + attn_combine_kernel: few new tokens per sequence
//    (the rank's query heads of one key-value head times the new tokens fit
//    in 16 rows). The cache is split into chunks of 512, 1024, 2048 or 4096
//    positions, as few as still fill the GPU; each workgroup reads its chunk
//    of one key-value head once for all those rows, and with more than one
//    chunk the combine kernel merges the chunks' softmax partials.
//  * attn_prefill_kernel: many new tokens. 64 query tokens of one head per
//    workgroup of two or four wavefront groups that split the causal chain
//    of 32-position key-value blocks (shared through LDS) between them,
//    online softmax, merged at the end.
//
// Precision: q k^T accumulates in fp32 from bf16; the softmax runs in fp32
// (exp2 with log2(e) folded into the scale). The probabilities enter the
// p v product as two bf16 terms, hi = bf16(p) and lo = bf16(p - hi), so that
// their rounding (about 2^-9 relative for one bf16 term, which alone would
// put the output about 1e-3 from the exact value) drops to about 2^-17. The
// output is rounded once to bf16.
//
// Operand layouts (v_mfma 16x16x32 and 32x32x16, bf16): lane (g, i) supplies
// A[i][8g .. 8g + 7] and B[8g .. 8g + 7][i]; the 16x16 result lands as
// D[4g + r][i], the 32x32 one as D[8q + 4g + r][i] in element 4q + r.
// Scores are computed transposed, S^T = K Q^T, so that a lane holds one
// query's scores. The p v product then runs as O^T = V^T P^T with its
// contraction over positions taken in the order those registers hold them:
// element e of lane group g is position 4g + e for e < 4 and 4g + 8 + (e - 4)
// (32x32x16; 16 + 4g + (e - 4) for 16x16x32 over two 16-position blocks).
// V^T comes out of LDS with ds_read_b64_tr_b16: within each 16-lane group,
// output lane j, element q is element j % 4 of the 8 bytes addressed by lane
// 4q + j / 4, so a lane addressing row base + j / 4 at column c0 + 4 (j % 4)
// yields V[base + q][c0 + j].
#include "tp_internal.h"

namespace tpk {
namespace {

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4_t* lds_i16x4_p;

constexpr int kWaitVm0 = 0x0F70;    // s_waitcnt vmcnt(0)
constexpr int kWaitLgkm0 = 0xC07F;  // s_waitcnt lgkmcnt(0)

__device__ __forceinline__ f32x16_t mfma_32x32x16(uint4 a, uint4 b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint2 tr_read(const char* p) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_p)p));
}

__device__ __forceinline__ uint4 tr_pair(const char* p0, const char* p1) {
  const uint2 a = tr_read(p0), b = tr_read(p1);
  return make_uint4(a.x, a.y, b.x, b.y);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// a and b rounded to bf16 (to nearest, ties to even) in one v_cvt_pk_bf16_f32,
// a in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

// Two bf16 terms of 8 probabilities, packed as MFMA operands: hi = bf16(p),
// lo = bf16(p - hi) (the difference is exact in fp32). Per pair: two
// conversions, the two hi values back in fp32 by a shift and a mask, and two
// subtractions.
__device__ __forceinline__ void split8(const float (&p)[8], uint4& hi, uint4& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    h[e] = pack_bf16x2(p[2 * e], p[2 * e + 1]);
    l[e] = pack_bf16x2(p[2 * e] - __uint_as_float(h[e] << 16), p[2 * e + 1] - __uint_as_float(h[e] & 0xFFFF0000u));
  }
  hi = make_uint4(h[0], h[1], h[2], h[3]);
  lo = make_uint4(l[0], l[1], l[2], l[3]);
}

// Max / sum of x over lanes l and l ^ 16, and over l and l ^ 32: gfx950's
// v_permlane16_swap / v_permlane32_swap of x with itself leave {x[l],
// x[l ^ 16]} (resp. ^ 32) in the pair of results, in the same order on both
// lanes, so partners get bit-identical values.
__device__ __forceinline__ float max16(float x) {
  const auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(t[0]), __uint_as_float(t[1]));
}
__device__ __forceinline__ float max32(float x) {
  const auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(t[0]), __uint_as_float(t[1]));
}
__device__ __forceinline__ float sum16(float x) {
  const auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}
__device__ __forceinline__ float sum32(float x) {
  const auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}

// A sequence's cache length, or 0 when its kv_len or slot is out of range
// (max_kv <= L_max, checked on the host).
__device__ __forceinline__ int seq_len(const AttnArgs& a, int s, int& sl) {
  const int kl = a.kv_len[s];
  sl = a.slot[s];
  const bool ok = kl >= a.q_len && kl <= a.max_kv && sl >= 0 && sl < a.n_slots;
  return ok ? kl : 0;
}

// The key-value head's cache rows [0, kl) as a buffer resource: positions
// past kl read as zeros.
__device__ __forceinline__ uint64_t head_base(const uint16_t* C, const AttnArgs& a, int sl, int g, int kl, int D) {
  const uint64_t base = (uint64_t)(C + (kl > 0 ? ((int64_t)sl * a.nkv + g) * a.L_max * D : 0));
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)base);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(base >> 32));
  return lo | (hi << 32);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc(const uint16_t* C, const AttnArgs& a, int sl, int g,
                                                            int kl, int D) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)head_base(C, a, sl, g, kl, D), (short)0,
                                           __builtin_amdgcn_readfirstlane(kl * D * 2), 0x00020000);
}

// A head's cache from byte bo on (bo and the head's byte count nb uniform):
// the base moves in scalar registers, the range check still ends at the
// head's last position, and nothing at all is in range once bo >= nb.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tail_rsrc(uint64_t base, unsigned nb, unsigned bo) {
  const uint64_t p = base + bo;
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)p);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(p >> 32));
  return __builtin_amdgcn_make_buffer_rsrc((void*)(lo | (hi << 32)), (short)0,
                                           __builtin_amdgcn_readfirstlane((int)(nb > bo ? nb - bo : 0u)), 0x00020000);
}

// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void kv_append_kernel(AttnArgs a, int64_t total) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int cpr = a.D / 8;
  const int per_row = 2 * a.nkv * cpr;
  const int64_t m = idx / per_row;
  const int c = (int)(idx - m * per_row);
  const int s = (int)(m / a.q_len), i = (int)(m - (int64_t)s * a.q_len);
  int sl;
  const int kl = seq_len(a, s, sl);
  if (kl == 0) return;
  const bool isv = c >= a.nkv * cpr;
  const int cc = isv ? c - a.nkv * cpr : c;
  const int g = cc / cpr, col = (cc - g * cpr) * 8;
  const uint4 v = *reinterpret_cast<const uint4*>(a.QKV + m * a.ldqkv +
                                                  (int64_t)(a.nq + (isv ? a.nkv : 0) + g) * a.D + col);
  const int64_t pos = kl - a.q_len + i;
  uint16_t* dst = (isv ? a.Vw : a.Kw) + (((int64_t)sl * a.nkv + g) * a.L_max + pos) * a.D + col;
  *reinterpret_cast<uint4*>(dst) = v;
}

// ---------------------------------------------------------------------------
// Decode. Workgroup (chunk, g, s) of 4 wavefronts takes NPW passes of 512
// positions of one (sequence, key-value head); in each pass wavefront w takes
// two 64-position halves, half h of the chunk at [chunk 512 NPW + 64 (4 h + w),
// + 64). Row rho (< 16) of the 16x16x32 operands is query head g G + rho /
// q_len of token rho % q_len. K fragments come straight from the cache into
// registers (A operand rows = positions); V lands in the wavefront's own LDS
// region by DMA at a pitch of D/8 + 2 16-byte slots, which puts the four rows
// each 16-lane group reads on distinct banks. Halves alternate between two
// register sets and two LDS arrays: loads go out as Q, K0, V0, K1, V1, and
// half h + 2's K and V as soon as half h has left them, so each half is
// multiplied while the next two are arriving (online softmax across the
// halves). The four wavefronts' results merge through LDS: with one chunk per
// (sequence, key-value head) the workgroup normalises and writes the output
// rows itself; otherwise it writes one partial, m[rho] (log2 domain), l[rho]
// and the unnormalised output [rho][D], and attn_combine_kernel merges them.

template <int D, int NPW>
__global__ __launch_bounds__(256) void attn_decode_kernel(AttnArgs a) {
  constexpr int KS = D / 32;     // 32-deep k-steps of q k^T
  constexpr int DB = D / 16;     // 16-column output blocks
  constexpr int CPR = D / 8;     // 16-byte chunks per cache row
  constexpr int PITCH = CPR + 2;
  constexpr int HPOS = 64;       // positions per half
  constexpr int NH = 2 * NPW;    // halves per wavefront
  constexpr int HSL = HPOS * PITCH;  // LDS slots per half (a multiple of 64)
  constexpr int RED = kAttnDecodeRows * D + 2 * kAttnDecodeRows;
  constexpr int KN = 4 * KS;     // K load instructions per half
  static_assert(kAttnDecodePass == 2 * 4 * HPOS, "two halves per wavefront and pass");
  static_assert((D * (kAttnDecodeRows + 1) + 2 * kAttnDecodeRows) * 4 <= HSL * 16,
                "a wave's partial fits in its half-0 V region");
  static_assert(2 * KN + PITCH <= 63, "the in-flight loads fit the wait counter");
  // One array per parity of the half: the compiler then tracks their DMA
  // apart and lets the other parity fly while one is read.
  __shared__ uint4 Vs0[4][HSL], Vs1[4][HSL];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g4 = lane >> 4, i = lane & 15;
  const int chunk = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  int sl;
  const int kl = seq_len(a, s, sl);
  const int R = a.G * a.q_len;
  const int pc = chunk * kAttnDecodePass * NPW + wave * HPOS;  // half h starts at pc + 256 h
  const __amdgpu_buffer_rsrc_t rk = head_rsrc(a.Kc, a, sl, g, kl, D);
  const __amdgpu_buffer_rsrc_t rv = head_rsrc(a.Vc, a, sl, g, kl, D);

  const int rho = i;
  const int hh = rho / a.q_len, tok = rho - hh * a.q_len;
  const bool row_ok = kl > 0 && rho < R;
  const int pos_r = kl - a.q_len + tok;
  float m = -INFINITY, l = 0.f;
  f32x4_t o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  if (pc < kl) {  // wave-uniform: at least half 0 holds positions
    uint4 kf[2][4][KS];
#define AD_KLOAD(H)                                                                                \
  _Pragma("unroll") for (int b = 0; b < 4; ++b) _Pragma("unroll") for (int k = 0; k < KS; ++k)    \
      kf[(H) & 1][b][k] = __builtin_bit_cast(                                                      \
          uint4, __builtin_amdgcn_raw_buffer_load_b128(                                            \
                     rk, (unsigned)(((pc + 4 * HPOS * (H) + 16 * b + i) * D + 32 * k + 8 * g4) * 2), 0, 0));
#define AD_VLOAD(H)                                                                                \
  _Pragma("unroll") for (int u = 0; u < PITCH; ++u) {                                              \
    const int q = u * 64 + lane, row = q / PITCH, c = q - row * PITCH;                             \
    const unsigned off = c < CPR ? (unsigned)(((pc + 4 * HPOS * (H) + row) * D + 8 * c) * 2) : 0x80000000u; \
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void_t*)&(((H) & 1) ? Vs1 : Vs0)[wave][u * 64], 16, off, 0, 0, 0); \
  }
    // Q rows past R read row 0 (always in range) and are zeroed after the
    // load, so no load sits behind a branch. Halves past the cache are loaded
    // and multiplied all the same: their loads return zeros without touching
    // memory and their scores are masked, and straight-line code keeps the
    // compiler's own wait counts exact.
    uint4 qf[KS];
    const uint16_t* qp = a.QKV + ((int64_t)s * a.q_len + (row_ok ? tok : 0)) * a.ldqkv +
                         (int64_t)(g * a.G + (row_ok ? hh : 0)) * D + 8 * g4;
#pragma unroll
    for (int k = 0; k < KS; ++k) qf[k] = *reinterpret_cast<const uint4*>(qp + 32 * k);
    __builtin_amdgcn_sched_barrier(0);
    AD_KLOAD(0)
    __builtin_amdgcn_sched_barrier(0);
    AD_VLOAD(0)
    __builtin_amdgcn_sched_barrier(0);
    AD_KLOAD(1)
    __builtin_amdgcn_sched_barrier(0);
    AD_VLOAD(1)
    __builtin_amdgcn_sched_barrier(0);
    const uint32_t qm = row_ok ? 0xFFFFFFFFu : 0u;
#pragma unroll
    for (int k = 0; k < KS; ++k) qf[k] = make_uint4(qf[k].x & qm, qf[k].y & qm, qf[k].z & qm, qf[k].w & qm);
    const int vfo = ((4 * g4 + (i >> 2)) * PITCH + ((i & 3) >> 1)) * 16 + (i & 1) * 8;
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      const int p0 = pc + 4 * HPOS * h;
      f32x4_t sc[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        sc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < KS; ++k) sc[b] = mfma_16x16x32(kf[h & 1][b][k], qf[k], sc[b]);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (h + 2 < NH) AD_KLOAD(h + 2)  // this half's K registers are free again
      __builtin_amdgcn_sched_barrier(0);
      // Lane (g4, i) holds row i's raw scores at positions p0 + 16 b + 4 g4 + r.
      float bm = -INFINITY;
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int p = p0 + 16 * b + 4 * g4 + r;
          if (!(p < kl && p <= pos_r)) sc[b][r] = -INFINITY;
          bm = fmaxf(bm, sc[b][r]);
        }
      bm = max32(max16(bm));
      const float mn = fmaxf(m, bm * a.qscale);  // -inf while the row has seen no position
      const float ms = mn == -INFINITY ? 0.f : mn;
      float rs = 0.f;
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[b][r], a.qscale, -ms));
          sc[b][r] = e;
          rs += e;
        }
      rs = sum32(sum16(rs));
      if (h > 0) {
        const float alpha = __builtin_amdgcn_exp2f(m - ms);
        l *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] *= alpha;
      }
      l += rs;
      m = mn;
      // This half's V has landed; issued after it: K and V of half h + 1
      // and K of half h + 2 (those that exist).
      constexpr int kW2 = 2 * KN + PITCH, kW1 = KN + PITCH;
      if (h + 2 < NH)
        __builtin_amdgcn_s_waitcnt(0x0F70 | (kW2 & 15) | ((kW2 >> 4) << 14));
      else if (h + 1 < NH)
        __builtin_amdgcn_s_waitcnt(0x0F70 | (kW1 & 15) | ((kW1 >> 4) << 14));
      else
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
      const char* vh = (const char*)((h & 1) ? Vs1[wave] : Vs0[wave]) + vfo;
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        const float pe[8] = {sc[2 * t2][0],     sc[2 * t2][1],     sc[2 * t2][2],     sc[2 * t2][3],
                             sc[2 * t2 + 1][0], sc[2 * t2 + 1][1], sc[2 * t2 + 1][2], sc[2 * t2 + 1][3]};
        uint4 ph, pl;
        split8(pe, ph, pl);
        uint4 vf[DB];
#pragma unroll
        for (int db = 0; db < DB; ++db)
          vf[db] = tr_pair(vh + (32 * t2 * PITCH + 2 * db) * 16, vh + ((32 * t2 + 16) * PITCH + 2 * db) * 16);
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] = mfma_16x16x32(vf[db], ph, o[db]);
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] = mfma_16x16x32(vf[db], pl, o[db]);
      }
      if (h + 2 < NH) {  // this half's V region is free once its reads are done
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        __builtin_amdgcn_sched_barrier(0);
        AD_VLOAD(h + 2)
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#undef AD_KLOAD
#undef AD_VLOAD
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  }

  // This wave's result into its own half-0 region (its reads of V are
  // complete), [D columns][17] (row rho at rho: the pitch of 17 keeps a
  // column's 16 rows and the other lane groups' columns on distinct banks),
  // then m, l.
  constexpr int RP = kAttnDecodeRows + 1;
  float* red = reinterpret_cast<float*>(Vs0[wave]);
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[(16 * db + 4 * g4 + r) * RP + rho] = o[db][r];
  if (g4 == 0) {
    red[D * RP + i] = m;
    red[D * RP + kAttnDecodeRows + i] = l;
  }
  __syncthreads();

  // Merge the four waves: thread t owns row t % 16, columns (t / 16) D / 16 ...
  constexpr int CW = D / 16;
  const int t = threadIdx.x, row = t & 15, c0 = (t >> 4) * CW;
  float mw[4], M = -INFINITY;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    mw[w] = reinterpret_cast<const float*>(Vs0[w])[D * RP + row];
    M = fmaxf(M, mw[w]);
  }
  float L = 0.f, f[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    f[w] = mw[w] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw[w] - M);
    L += f[w] * reinterpret_cast<const float*>(Vs0[w])[D * RP + kAttnDecodeRows + row];
  }
  float acc[CW];
#pragma unroll
  for (int c = 0; c < CW; ++c) {
    acc[c] = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) acc[c] += f[w] * reinterpret_cast<const float*>(Vs0[w])[(c0 + c) * RP + row];
  }
  if (a.nchunk == 1) {  // the whole cache was this workgroup's: write the output rows
    if (row < R) {  // divided as the combine kernel divides, so both forms agree bit for bit
      const bool ok = kl > 0 && L > 0.f;
      const int hr = row / a.q_len, tr = row - hr * a.q_len;
      uint16_t* dst = a.A + ((int64_t)s * a.q_len + tr) * a.lda + (int64_t)(g * a.G + hr) * D + c0;
#pragma unroll
      for (int q = 0; q < CW / 4; ++q)
        store_bf16x4(dst + 4 * q, ok ? acc[4 * q] / L : 0.f, ok ? acc[4 * q + 1] / L : 0.f,
                     ok ? acc[4 * q + 2] / L : 0.f, ok ? acc[4 * q + 3] / L : 0.f);
    }
    return;
  }
  float* P = a.ws + (((int64_t)s * a.nkv + g) * a.nchunk + chunk) * RED;
  if (t < kAttnDecodeRows) {
    P[kAttnDecodeRows * D + row] = M;
    P[kAttnDecodeRows * D + kAttnDecodeRows + row] = L;
  }
#pragma unroll
  for (int c = 0; c < CW; ++c) P[row * D + c0 + c] = acc[c];
}

// Workgroup (rho, g, s), thread c: output column c of row rho, merged over
// the chunks in chunk order. Up to kCombineRegs chunks, every load goes out in
// one batch (each thread holds the chunks' maxima, sums and its column; the
// loads take a clamped chunk index, so none sits behind a branch and the
// entries past the last chunk are never used); beyond that the chunks' maxima
// and sums are fetched a tile of D chunks at a time, one per thread, and
// shared through LDS.
constexpr int kCombineRegs = 32;

template <int D, int NR>
__device__ __forceinline__ float combine_regs(const AttnArgs& a, const float* P0, int rho, int c) {
  constexpr int RED = kAttnDecodeRows * D + 2 * kAttnDecodeRows;
  float mc[NR], lc[NR], oc[NR];
#pragma unroll
  for (int j = 0; j < NR; ++j) {
    const float* Pj = P0 + (int64_t)(j < a.nchunk ? j : a.nchunk - 1) * RED;
    mc[j] = Pj[kAttnDecodeRows * D + rho];
    lc[j] = Pj[kAttnDecodeRows * D + kAttnDecodeRows + rho];
    oc[j] = Pj[rho * D + c];
  }
  float M = -INFINITY;
#pragma unroll
  for (int j = 0; j < NR; ++j)
    if (j < a.nchunk) M = fmaxf(M, mc[j]);
  float L = 0.f, acc = 0.f;
#pragma unroll
  for (int j = 0; j < NR; ++j)
    if (j < a.nchunk && mc[j] != -INFINITY) {
      const float f = __builtin_amdgcn_exp2f(mc[j] - M);
      L += f * lc[j];
      acc += f * oc[j];
    }
  return L > 0.f ? acc / L : 0.f;
}

template <int D>
__global__ __launch_bounds__(D) void attn_combine_kernel(AttnArgs a) {
  constexpr int RED = kAttnDecodeRows * D + 2 * kAttnDecodeRows;
  __shared__ float wgt[D];
  __shared__ float red[D];
  const int rho = blockIdx.x, g = blockIdx.y, s = blockIdx.z, c = threadIdx.x;
  int sl;
  const int kl = seq_len(a, s, sl);
  const float* P0 = a.ws + ((int64_t)s * a.nkv + g) * a.nchunk * RED;
  const int hh = rho / a.q_len, tok = rho - hh * a.q_len;
  uint16_t* dst = a.A + ((int64_t)s * a.q_len + tok) * a.lda + (int64_t)(g * a.G + hh) * D + c;
  if (a.nchunk <= kCombineRegs) {  // uniform
    const float v = a.nchunk <= 8    ? combine_regs<D, 8>(a, P0, rho, c)
                    : a.nchunk <= 16 ? combine_regs<D, 16>(a, P0, rho, c)
                                     : combine_regs<D, kCombineRegs>(a, P0, rho, c);
    *dst = f32_to_bf16(kl > 0 ? v : 0.f);
    return;
  }
  float M = -INFINITY;
  for (int ch = c; ch < a.nchunk; ch += D) M = fmaxf(M, P0[(int64_t)ch * RED + kAttnDecodeRows * D + rho]);
  red[c] = M;
  __syncthreads();
  for (int w = D / 2; w > 0; w >>= 1) {
    if (c < w) red[c] = fmaxf(red[c], red[c + w]);
    __syncthreads();
  }
  M = red[0];
  __syncthreads();
  float Lp = 0.f, acc = 0.f;
  for (int t0 = 0; t0 < a.nchunk; t0 += D) {
    const int ch = t0 + c;
    float f = 0.f;
    if (ch < a.nchunk) {
      const float* Pj = P0 + (int64_t)ch * RED;
      const float mc = Pj[kAttnDecodeRows * D + rho];
      f = mc == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mc - M);
      Lp += f * Pj[kAttnDecodeRows * D + kAttnDecodeRows + rho];
    }
    wgt[c] = f;
    __syncthreads();
    const int n = a.nchunk - t0 < D ? a.nchunk - t0 : D;
    const float* Pc = P0 + (int64_t)t0 * RED + rho * D + c;
    for (int j = 0; j < n; ++j) acc += wgt[j] * Pc[(int64_t)j * RED];
    __syncthreads();
  }
  red[c] = Lp;
  __syncthreads();
  for (int w = D / 2; w > 0; w >>= 1) {
    if (c < w) red[c] += red[c + w];
    __syncthreads();
  }
  const float L = red[0];
  *dst = f32_to_bf16(kl > 0 && L > 0.f ? acc / L : 0.f);
}

// ---------------------------------------------------------------------------
// Prefill. A workgroup of NG groups of 2 wavefronts (NG = 2 or 4) takes 64
// query tokens of one query head. Wavefront w belongs to group w / 2 and
// takes tokens 64 qb + 32 (w % 2) + j, j = lane % 32, the column of its
// 32x32x16 operands. Group gr multiplies key-value blocks gr, gr + NG, ... of
// 32 positions, so each group runs 1/NG of the causal chain; at the end
// every wavefront writes its (max, sum, output) to LDS, then merges and
// stores its own slice of columns over the NG groups. Workgroups take units
// (query block, head, sequence) longest first; with four groups and nearly
// two rounds of units, each workgroup takes a pair, the longest with the
// shortest.
//
// Each group stages its blocks in LDS by DMA, K and V apart, each double
// buffered in two arrays (even and odd blocks of its chain): 32 K rows at a
// pitch of D/8 + 1 16-byte slots (the A operand of S^T read whole, 32 rows
// per half-wavefront on distinct banks), 32 V rows at D/8 + 4 (transposed
// reads), each region padded to whole DMA instructions. With separate arrays
// read by name the compiler tells the DMA into one buffer apart from the
// reads of another and lets it fly.
//
// A step of the chain is two halves, each ended by a barrier: (1) the softmax
// of block t's scores and the probabilities' two bf16 terms, vector ALU only;
// (2) P V of block t and the scores S^T of block t + 1, matrix cores and LDS
// reads. K of block t + 1 is fetched two steps before it is used, V of block
// t two steps before. With four groups, groups 2 and 3 run one half behind
// groups 0 and 1: the two wavefronts that share a SIMD (w and w + 4) are then
// always in different halves, one on the vector ALU while the other keeps the
// matrix cores busy.

// One buffer's DMA: instruction n = 2 u + wq fills 16-byte slots 64 n + lane
// of dst from byte off[u] of the block at byte bo of the head's cache (base).
__device__ __forceinline__ void prefill_dma(int NU, uint64_t base, unsigned nb, unsigned bo, uint4* dst,
                                            const unsigned* off, int wq) {
#pragma unroll
  for (int u = 0; u < NU; ++u)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(tail_rsrc(base, nb, bo), (lds_void_t*)(dst + (2 * u + wq) * 64), 16,
                                             off[u], 0, 0, 0);
}

template <int D>
struct PrefillCfg {
  // V's pitch of D/8 + 4 slots puts the 8 row segments of a half-wavefront's
  // transposed read (4 rows x 2 column halves) on distinct banks.
  static constexpr int KP = D / 8 + 1, VP = D / 8 + 4;
  static constexpr int BK = 32;                       // positions per block
  static constexpr int NUK = (BK * KP + 127) / 128;   // K DMA instructions per wave
  static constexpr int NUV = (BK * VP + 127) / 128;   // V DMA instructions per wave
  static constexpr int KST = NUK * 128, VST = NUV * 128;  // slots of a K / V buffer, with the padding
  static_assert(NUK + 2 * NUV <= 15, "the prologue's wait fits the low vmcnt field");
};

template <int D, int NG>
__global__ __launch_bounds__(128 * NG, 4 / NG) void attn_prefill_kernel(AttnArgs a, int nqb, int units, int paired) {
  using C = PrefillCfg<D>;
  static_assert(NG == 2 || NG == 4, "two or four groups");
  constexpr int KS = D / 16;  // 16-deep k-steps of q k^T
  constexpr int DB = D / 32;  // 32-column output blocks
  constexpr int CPR = D / 8;
  // [group]: K of even and odd blocks of the group's chain, V of even and odd blocks
  __shared__ uint4 Ks0[NG][C::KST], Ks1[NG][C::KST], Vs0[NG][C::VST], Vs1[NG][C::VST];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int gr = wave >> 1, wq = wave & 1;
  const int h2 = lane >> 5, j = lane & 31;
  // Paired (four groups only): workgroup b also takes unit units - 1 - b
  // after unit b, the longest chains with the shortest, so each CU runs one
  // workgroup for two units instead of two workgroups in turn.
  const int bid = (int)blockIdx.x;
  const int npass = NG == 4 && paired && units - 1 - bid > bid ? 2 : 1;
  for (int pass = 0; pass < npass; ++pass) {
    const int unit = pass == 0 ? bid : units - 1 - bid;
    const int per = a.nq * a.S;
    const int qb = nqb - 1 - unit / per, h = (unit % per) % a.nq, s = (unit % per) / a.nq;
    const int g = h / a.G;
    int sl;
    const int kl = seq_len(a, s, sl);
    const int tok0 = qb * 64 + wq * 32;
    const int tok = tok0 + j;
    const bool row_ok = tok < a.q_len;
    uint16_t* out = a.A + ((int64_t)s * a.q_len + tok) * a.lda + (int64_t)h * D;
    if (kl == 0) {  // uniform over the workgroup: a sequence out of range gives zeros
      if (row_ok && gr == 0)
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int q = 0; q < 4; ++q) store_bf16x4(out + 32 * db + 8 * q + 4 * h2, 0.f, 0.f, 0.f, 0.f);
    } else {
      const int base_pos = kl - a.q_len;  // position of token 0
      const int last_tok = qb * 64 + 63 < a.q_len - 1 ? qb * 64 + 63 : a.q_len - 1;
      const int nblk = (base_pos + last_tok) / C::BK + 1;
      const int nstep = (nblk + NG - 1) / NG;
      const int wlast = tok0 + 31 < a.q_len - 1 ? tok0 + 31 : a.q_len - 1;
      const int wblk = tok0 < a.q_len ? (base_pos + wlast) / C::BK + 1 : 0;  // blocks this wave's tokens see
      const int wfirst_pos = base_pos + tok0;
      const int pos_j = base_pos + tok;

      const uint64_t kbase = head_base(a.Kc, a, sl, g, kl, D), vbase = head_base(a.Vc, a, sl, g, kl, D);
      const unsigned nb = (unsigned)__builtin_amdgcn_readfirstlane(kl * D * 2);
      // DMA offsets of this lane: slot 64 (2 u + wq) + lane of a buffer holds
      // byte offk[u] (offv[u]) of its block; 0x80000000 marks a padding slot
      // (out of range: zeros).
      unsigned offk[C::NUK], offv[C::NUV];
#pragma unroll
      for (int u = 0; u < C::NUK; ++u) {
        const int q = (2 * u + wq) * 64 + lane, row = q / C::KP, c = q - row * C::KP;
        offk[u] = row < C::BK && c < CPR ? (unsigned)((row * D + 8 * c) * 2) : 0x80000000u;
      }
#pragma unroll
      for (int u = 0; u < C::NUV; ++u) {
        const int q = (2 * u + wq) * 64 + lane, row = q / C::VP, c = q - row * C::VP;
        offv[u] = row < C::BK && c < CPR ? (unsigned)((row * D + 8 * c) * 2) : 0x80000000u;
      }
      // Block NG t + gr of this group's chain (t = its step) into a K or V
      // buffer; steps t >= nstep, which the loop issues as well, get an empty
      // range: all out of range, they write zeros without a memory access.
    #define AP_BO(T) ((T) < nstep ? (unsigned)((NG * (T) + gr) * C::BK * D * 2) : nb)
    #define AP_K(KB, T) prefill_dma(C::NUK, kbase, nb, AP_BO(T), KB[gr], offk, wq);
    #define AP_V(VB, T) prefill_dma(C::NUV, vbase, nb, AP_BO(T), VB[gr], offv, wq);

      // Q fragments. Tokens past q_len read token 0's row: their columns of S^T
      // are finite and independent of the others', and nothing stores them.
      uint4 qf[KS];
      {
        const uint16_t* qp = a.QKV + ((int64_t)s * a.q_len + (row_ok ? tok : 0)) * a.ldqkv + (int64_t)h * D + 8 * h2;
#pragma unroll
        for (int k = 0; k < KS; ++k) qf[k] = *reinterpret_cast<const uint4*>(qp + 16 * k);
      }
      // The explicit DMA wait counts below assume the Q loads went out first.
      __builtin_amdgcn_sched_barrier(0);
      f32x16_t o[DB];
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] = f32x16_t{};
      // Reference max m of the scaled scores (log2 domain; it trails the running
      // max by at most kSlack) and sum, per token column. Groups 1..NG-1 start at
      // blocks that early tokens do not see: while a token's m is still -inf the
      // exponents subtract 0 instead, so a masked (-inf) score gives exp2 = 0 and
      // no -inf - -inf arises.
      float m = -INFINITY, l = 0.f;
      const float c = a.qscale;
      constexpr float kSlack = 8.f;

      // Fragment bases: K row j, slot 2 k + h2; V (transposed reads) row
      // 16 k' + 4 h2 + jj / 4 (+ 8), slot 4 db + 2 uu + (jj % 4) / 2, half jj % 2,
      // where the lane is 32 h2 + 16 uu + jj.
      const int jj = j & 15, uu = j >> 4;
      const int kfb = (j * C::KP + h2) * 16;
      const int vfb = ((4 * h2 + (jj >> 2)) * C::VP + 2 * uu + ((jj & 3) >> 1)) * 16 + (jj & 1) * 8;

      // The scores S^T of block blk (this wave's 32 tokens x its 32 positions)
      // from the K buffer KB, all K fragments read before the chain of products.
      auto scores = [&](const uint4* KB, f32x16_t& sa) __attribute__((always_inline)) {
        const char* L = (const char*)KB;
        uint4 kf[KS];
#pragma unroll
        for (int k = 0; k < KS; ++k) kf[k] = *reinterpret_cast<const uint4*>(L + kfb + 2 * k * 16);
        sa = f32x16_t{};
#pragma unroll
        for (int k = 0; k < KS; ++k) sa = mfma_32x32x16(kf[k], qf[k], sa);
      };

      // Step t: V of block t is in VB, K of block t + 1 in KB (so VB is the
      // array of t's parity and KB the other); sa holds block t's scores.
      f32x16_t sa;
      auto step = [&](uint4 (&VB)[NG][C::VST], uint4 (&KB)[NG][C::KST], const int t) __attribute__((always_inline)) {
        const int blk = NG * t + gr;
        const bool live = blk < wblk, live1 = blk + NG < wblk;
        uint4 ph[2], pl[2];
        if (live) {
          // Lane (h2, j), element 4 q + r: position 32 blk + 8 q + 4 h2 + r.
          if (blk * C::BK + C::BK - 1 > wfirst_pos) {  // a diagonal block: mask what lies past the token
#pragma unroll
            for (int e = 0; e < 16; ++e)
              if (blk * C::BK + 8 * (e >> 2) + 4 * h2 + (e & 3) > pos_j) sa[e] = -INFINITY;
          }
          float bm = -INFINITY;
#pragma unroll
          for (int e = 0; e < 16; e += 4) bm = fmaxf(bm, fmaxf(fmaxf(sa[e], sa[e + 1]), fmaxf(sa[e + 2], sa[e + 3])));
          bm = max32(bm);
          // The subtracted reference mn moves only when the block's max passes
          // it by more than kSlack (log2 units), so the probabilities stay below
          // 2^kSlack and the output's rescale runs a few times per chain instead
          // of at nearly every step. Softmax does not depend on the constant
          // subtracted: only rounding changes.
          const float mb = bm * c;
          const float mn = mb > m + kSlack ? mb : m;
          const float ms = mn == -INFINITY ? 0.f : mn;
          float r4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[e], c, -ms));
            sa[e] = pe;
            r4[e & 3] += pe;
          }
          const float rs = sum32((r4[0] + r4[1]) + (r4[2] + r4[3]));
          if (__builtin_amdgcn_ballot_w64(mn != m) != 0) {  // some token's reference moved: rescale
            const float alpha = __builtin_amdgcn_exp2f(m - ms);
            l *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db) o[db] *= alpha;
          }
          l += rs;
          m = mn;
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
            const int q0 = 2 * kk;
            const float pe[8] = {sa[4 * q0],     sa[4 * q0 + 1], sa[4 * q0 + 2], sa[4 * q0 + 3],
                                 sa[4 * q0 + 4], sa[4 * q0 + 5], sa[4 * q0 + 6], sa[4 * q0 + 7]};
            split8(pe, ph[kk], pl[kk]);
          }
        }
        // V of block t and K of block t + 1 have landed; after them only V of
        // t + 1 and K of t + 2 may be in flight.
        __builtin_amdgcn_s_waitcnt(0x0F70 | (C::NUV + C::NUK));
        __builtin_amdgcn_s_barrier();  // end of the first half
        if (live) {
          const char* L = (const char*)VB[gr];
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
            uint4 vf[DB];
#pragma unroll
            for (int db = 0; db < DB; ++db) {
              const char* v0 = L + vfb + (16 * kk * C::VP + 4 * db) * 16;
              vf[db] = tr_pair(v0, v0 + 8 * C::VP * 16);
            }
#pragma unroll
            for (int db = 0; db < DB; ++db) o[db] = mfma_32x32x16(vf[db], ph[kk], o[db]);
#pragma unroll
            for (int db = 0; db < DB; ++db) o[db] = mfma_32x32x16(vf[db], pl[kk], o[db]);
          }
        }
        if (live1) scores(KB[gr], sa);
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        __builtin_amdgcn_s_barrier();  // end of the second half: V of t and K of t + 1 are read
        AP_V(VB, t + 2)
        AP_K(KB, t + 3)
      };

      // Prologue: K and V of steps 0 and 1 in flight, then step 0's scores; K of
      // step 2 follows once step 0's K buffer is free. Every DMA issue is
      // unconditional (the last ones have empty ranges): with conditional
      // issues the compiler could not tell which buffer's DMA is the newest and
      // would wait for all of them before a fragment read.
      AP_K(Ks0, 0)
      AP_V(Vs0, 0)
      AP_K(Ks1, 1)
      AP_V(Vs1, 1)
      __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * C::NUV + C::NUK));  // K of step 0 has landed
      __builtin_amdgcn_s_barrier();
      const bool late = NG == 4 && gr >= 2;  // wave-uniform
      if (late) __builtin_amdgcn_s_barrier();  // the half that groups 0 and 1 spend on step 0's scores
      if (gr < wblk) scores(Ks0[gr], sa);
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      __builtin_amdgcn_s_barrier();
      AP_K(Ks0, 2)
      // Whole pairs of steps (an odd count gets one step that multiplies
      // nothing), so that the loop's back edge always follows an odd step and the
      // compiler knows which buffers' DMAs are the newer ones at its top.
      const int npair = (nstep + 1) / 2;
      for (int tp = 0; tp < npair; ++tp) {
        step(Vs0, Ks1, 2 * tp);
        step(Vs1, Ks0, 2 * tp + 1);
      }
      if (!late) __builtin_amdgcn_s_barrier();  // the half that groups 2 and 3 spend on their last step
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      __builtin_amdgcn_s_barrier();  // no DMA is still landing when the buffers become the merge's regions
    #undef AP_BO
    #undef AP_K
    #undef AP_V

      // Every wave's partial into LDS, region w = the wave: [D columns][33]
      // (token j at j; a pitch of 33 keeps a column's 32 tokens and the other
      // half-wave's columns on distinct banks), then m and l. Lane (h2, j),
      // element 4 q + r of block db: column 32 db + 8 q + 4 h2 + r of token j.
      // Then wave (gr, wq) merges columns [gr D/NG, (gr + 1) D/NG) of its 32
      // tokens over the NG groups in group order, each half-wavefront half of
      // them, and stores them. Region r is region r % RK of Ks0, Ks1 (r < 2 RK),
      // else of Vs0, Vs1.
      constexpr int TP = 33;
      constexpr int WR = D * TP + 64;
      constexpr int RK = NG * C::KST * 16 / (WR * 4);  // regions per K buffer
      constexpr int RV = NG * C::VST * 16 / (WR * 4);  // regions per V buffer
      static_assert(RK >= 1 && RV >= 1 && 2 * RK + 2 * RV >= 2 * NG, "every wave's partial fits in LDS");
      auto region = [&](const int r) -> float* {
        if (r < RK) return reinterpret_cast<float*>(&Ks0[0][0]) + r * WR;
        if (r < 2 * RK) return reinterpret_cast<float*>(&Ks1[0][0]) + (r - RK) * WR;
        if (r < 2 * RK + RV) return reinterpret_cast<float*>(&Vs0[0][0]) + (r - 2 * RK) * WR;
        return reinterpret_cast<float*>(&Vs1[0][0]) + (r - 2 * RK - RV) * WR;
      };
      {
        float* rw = region(wave);
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int e = 0; e < 16; ++e) rw[(32 * db + 8 * (e >> 2) + 4 * h2 + (e & 3)) * TP + j] = o[db][e];
        if (h2 == 0) {
          rw[D * TP + j] = m;
          rw[D * TP + 32 + j] = l;
        }
      }
      __syncthreads();
      if (row_ok) {
        constexpr int CW = D / NG / 2;  // columns per lane
        static_assert(CW % 4 == 0, "whole 4-column stores");
        const float* rg[NG];
        float mg[NG], M = -INFINITY;
#pragma unroll
        for (int q = 0; q < NG; ++q) {
          rg[q] = region(2 * q + wq);
          mg[q] = rg[q][D * TP + j];
          M = fmaxf(M, mg[q]);
        }
        float f[NG], L = 0.f;
#pragma unroll
        for (int q = 0; q < NG; ++q) {
          f[q] = __builtin_amdgcn_exp2f(mg[q] - M);
          L += f[q] * rg[q][D * TP + 32 + j];
        }
        const float inv = L > 0.f ? 1.f / L : 0.f;
        const int c0 = gr * (D / NG) + h2 * CW;
#pragma unroll
        for (int i = 0; i < CW; i += 4) {
          float v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int col = c0 + i + r;
            float acc = f[0] * rg[0][col * TP + j];
#pragma unroll
            for (int q = 1; q < NG; ++q) acc += f[q] * rg[q][col * TP + j];
            v[r] = acc * inv;
          }
          store_bf16x4(out + c0 + i, v[0], v[1], v[2], v[3]);
        }
      }
    }  // kl > 0
    __syncthreads();  // the next unit's DMA reuses the merge's LDS
  }  // pass
}

template <int D>
hipError_t launch_attention_d(const AttnArgs& a, bool decode, hipStream_t s) {
  if (decode) {
    const dim3 grid(a.nchunk, a.nkv, a.S);
    switch (a.npw) {
      case 1: hipLaunchKernelGGL((attn_decode_kernel<D, 1>), grid, dim3(256), 0, s, a); break;
      case 2: hipLaunchKernelGGL((attn_decode_kernel<D, 2>), grid, dim3(256), 0, s, a); break;
      case 4: hipLaunchKernelGGL((attn_decode_kernel<D, 4>), grid, dim3(256), 0, s, a); break;
      default: hipLaunchKernelGGL((attn_decode_kernel<D, 8>), grid, dim3(256), 0, s, a); break;
    }
    if (a.nchunk > 1)
      hipLaunchKernelGGL(attn_combine_kernel<D>, dim3(a.G * a.q_len, a.nkv, a.S), dim3(D), 0, s, a);
  } else {
    const int nqb = (a.q_len + 63) / 64;
    // Two groups per workgroup (two workgroups per CU, which drift apart and
    // overlap one's softmax with the other's products) when the units fill
    // the CUs' two slots at least twice, or once with short chains; otherwise
    // four groups (one workgroup per CU), which halves the longest chain.
    const int64_t units = (int64_t)nqb * a.nq * a.S;
    if (units >= 1024 || (units >= 512 && nqb <= 16)) {
      hipLaunchKernelGGL((attn_prefill_kernel<D, 2>), dim3((unsigned)units), dim3(256), 0, s, a, nqb, (int)units, 0);
    } else {
      // Four groups run one workgroup per CU. When the units fill close to
      // two rounds of the 256 CUs, workgroups take them in pairs (longest
      // with shortest): one round, with no second wave of workgroup starts.
      // 70B rank 0 at 4096 tokens: 67.7-68.2 against 68.7-69.1 us.
      const int paired = units > 448 && units <= 512;
      const dim3 grid(paired ? (unsigned)((units + 1) / 2) : (unsigned)units);
      hipLaunchKernelGGL((attn_prefill_kernel<D, 4>), grid, dim3(512), 0, s, a, nqb, (int)units, paired);
    }
  }
  return hipGetLastError();
}

}  // namespace

size_t attn_decode_ws_bytes(int64_t S, int64_t nkv, int64_t nchunk, int D) {
  if (nchunk <= 1) return 0;  // one chunk writes the output itself
  return (size_t)(S * nkv * nchunk) * (size_t)(kAttnDecodeRows * D + 2 * kAttnDecodeRows) * sizeof(float);
}

void attn_decode_split(int64_t S, int64_t nkv, int64_t max_kv, int32_t& nchunk, int32_t& npw) {
  // The fewest chunks that still give about one workgroup per CU: passes of
  // 512 positions per chunk double while the workgroups stay at 256 or more.
  const int64_t full = (max_kv + kAttnDecodePass - 1) / kAttnDecodePass;
  const int64_t pairs = S * nkv;
  int64_t p = 1;
  while (p < 8 && p < full && pairs * ((full + 2 * p - 1) / (2 * p)) >= 256) p *= 2;
  npw = (int32_t)p;
  nchunk = (int32_t)((full + p - 1) / p);
}

hipError_t launch_kv_append(const AttnArgs& a, hipStream_t s) {
  const int64_t total = (int64_t)a.S * a.q_len * 2 * a.nkv * (a.D / 8);
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(kv_append_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a, total);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs& a, bool decode, hipStream_t s) {
  if (a.S == 0) return hipSuccess;
  return a.D == 128 ? launch_attention_d<128>(a, decode, s) : launch_attention_d<64>(a, decode, s);
}

}  // namespace tpk
