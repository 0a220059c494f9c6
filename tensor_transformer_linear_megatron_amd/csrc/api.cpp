// The C-ABI entry points: host-side validation and kernel dispatch. Nothing
// here allocates device memory or keeps state between calls.
#include <atomic>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "tp_internal.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool is_col(int32_t k) { return k == TP_COL || k == TP_QKV_COL || k == TP_GATEUP_COL; }
bool is_row(int32_t k) { return k == TP_ROW || k == TP_O_ROW || k == TP_DGRAD; }

// Self-consistency of a caller-held descriptor (it is plain data the caller
// may have edited).
tp_status check_desc(const tp_shard_desc* d) {
  if (d == nullptr) return TP_ERR_NULL;
  if (!is_col(d->kind) && !is_row(d->kind)) return TP_ERR_KIND;
  const bool gateup = d->kind == TP_GATEUP_COL;
  if (d->wformat != TP_W_BF16 && d->wformat != TP_W_FP8_E4M3) return TP_ERR_KIND;
  const bool fp8 = d->wformat == TP_W_FP8_E4M3;
  if (fp8 && d->kind == TP_DGRAD) return TP_ERR_KIND;
  if (d->shard_k <= 0 || d->shard_n <= 0 || d->out_n <= 0 || d->packed_k < d->shard_k ||
      d->packed_k % (fp8 ? tpk::kTileK8 : tpk::kTileK) || d->packed_n % (2 * tpk::kTileN) ||
      d->packed_bytes != (fp8 ? d->packed_k * d->packed_n + 4 * d->packed_n
                              : d->packed_k * d->packed_n * 2))
    return TP_ERR_SHAPE;
  if (gateup) {
    // gate and up tiles alternate: an even tile count, each half covering out_n
    if (d->shard_n != 2 * d->out_n || d->packed_n % (2 * tpk::kTileN) || d->packed_n / 2 < d->out_n)
      return TP_ERR_SHAPE;
  } else if (d->out_n != d->shard_n || d->packed_n < d->shard_n) {
    return TP_ERR_SHAPE;
  }
  if (d->shard_k % 8 || d->out_n % 8) return TP_ERR_ALIGN;
  if (d->path < TP_PATH_AUTO || d->path > TP_PATH_PREFILL) return TP_ERR_KIND;
  return TP_OK;
}

bool is_fp8(const tp_shard_desc* d) { return d->wformat == TP_W_FP8_E4M3; }

// k-steps of the packed layout: 32 k for bf16 tiles, 64 k for 8-bit tiles.
int64_t ksteps_of(const tp_shard_desc* d) {
  return d->packed_k / (is_fp8(d) ? tpk::kTileK8 : tpk::kTileK);
}

tpk::LinearArgs make_args(const tp_shard_desc* d, const uint16_t* X, int64_t M, int64_t ldx,
                          const void* Wp, void* out, int64_t ldo) {
  tpk::LinearArgs a;
  a.X = X;
  a.ldx = ldx;
  a.M = M;
  a.K = d->shard_k;
  a.W = static_cast<const uint4*>(Wp);
  a.ksteps = ksteps_of(d);
  a.ntiles = d->packed_n / tpk::kTileN;
  a.out = out;
  a.ldo = ldo;
  a.out_n = d->out_n;
  // An 8-bit shard's column scales follow its codes.
  a.wscale = is_fp8(d) ? reinterpret_cast<const float*>(static_cast<const uint8_t*>(Wp) +
                                                        d->packed_k * d->packed_n)
                       : nullptr;
  return a;
}

// An 8-bit shard at prefill is first dequantised into a bf16 packed copy
// (2 k-steps of 32 per step of 64) at the start of the workspace; the GEMM's
// own workspace follows it.
size_t dequant_bytes(const tp_shard_desc* d) {
  return ((size_t)d->packed_k * d->packed_n * 2 + 255) / 256 * 256;
}

tpk::Epilogue epilogue_of(const tp_shard_desc* d) {
  if (d->kind == TP_GATEUP_COL) return tpk::kEpiSwiglu;
  return is_col(d->kind) ? tpk::kEpiBf16 : tpk::kEpiF32;
}

int32_t path_of(const tp_shard_desc* d, int64_t M) {
  if (d->path != TP_PATH_AUTO) return d->path;
  return M <= 64 ? TP_PATH_DECODE : TP_PATH_PREFILL;
}

// Workspace of the kernels chosen for this shard at this M. The prefill plan
// is taken at the smallest leading dimension (shard_k); a wider X can only
// turn the split off, never need more.
size_t workspace_bytes(const tp_shard_desc* d, int64_t M, int64_t ldx) {
  if (M <= 0) return 0;
  const int64_t ntiles = d->packed_n / tpk::kTileN;
  if (is_fp8(d)) {
    if (path_of(d, M) == TP_PATH_DECODE)
      return tpk::gemv_workspace_bytes(M, 2 * ksteps_of(d), ntiles, epilogue_of(d), true);
    return dequant_bytes(d) + tpk::gemm_workspace_bytes(M, ldx, 2 * ksteps_of(d), ntiles);
  }
  if (path_of(d, M) == TP_PATH_DECODE)
    return tpk::gemv_workspace_bytes(M, ksteps_of(d), ntiles, epilogue_of(d));
  return tpk::gemm_workspace_bytes(M, ldx, ksteps_of(d), ntiles);
}
size_t workspace_bytes(const tp_shard_desc* d, int64_t M) { return workspace_bytes(d, M, d->shard_k); }

tp_status run_linear(const tp_shard_desc* d, const tpk::LinearArgs& a, void* ws, size_t ws_bytes,
                     hipStream_t s) {
  const int32_t path = path_of(d, a.M);
  if (path == TP_PATH_DECODE && a.M > 64) return TP_ERR_SHAPE;
  const size_t need = workspace_bytes(d, a.M, a.ldx);
  if (need > 0 && (ws == nullptr || ws_bytes < need)) return TP_ERR_WORKSPACE;
  if (need > 0 && !aligned16(ws)) return TP_ERR_ALIGN;
  float* w = need > 0 ? static_cast<float*>(ws) : nullptr;
  hipError_t e;
  if (is_fp8(d) && path == TP_PATH_DECODE) {
    e = tpk::launch_gemv8(a, epilogue_of(d), w, s);
  } else if (is_fp8(d)) {
    // prefill: dequantise into the workspace, then the bf16 GEMM on that copy
    uint4* w16 = static_cast<uint4*>(ws);
    e = tpk::launch_dequant8(a.W, a.wscale, a.ksteps, a.ntiles, w16, s);
    if (e == hipSuccess) {
      tpk::LinearArgs b = a;
      b.W = w16;
      b.ksteps = 2 * a.ksteps;
      b.wscale = nullptr;
      const size_t db = dequant_bytes(d);
      float* rest = need > db ? reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + db) : nullptr;
      e = tpk::launch_gemm(b, epilogue_of(d), rest, s);
    }
  } else {
    e = path == TP_PATH_DECODE ? tpk::launch_gemv(a, epilogue_of(d), w, s)
                               : tpk::launch_gemm(a, epilogue_of(d), w, s);
  }
  return e == hipSuccess ? TP_OK : TP_ERR_HIP;
}

tp_status check_linear_io(const tp_shard_desc* d, const uint16_t* X, int64_t M, int64_t ldx,
                          const void* Wp, const void* out, int64_t ldo, int64_t out_elem_align) {
  if (M < 0) return TP_ERR_SHAPE;
  if (M == 0) return TP_OK;  // nothing is read or written; empty tensors may have NULL data
  if (X == nullptr || Wp == nullptr || out == nullptr) return TP_ERR_NULL;
  if (ldx < d->shard_k || ldo < d->out_n) return TP_ERR_SHAPE;
  if (!aligned16(X) || !aligned16(Wp) || !aligned16(out) || ldx % 8 || ldo % out_elem_align)
    return TP_ERR_ALIGN;
  return TP_OK;
}

}  // namespace

extern "C" size_t tp_workspace_bytes(const tp_shard_desc* desc, int64_t M) {
  if (check_desc(desc) != TP_OK) return 0;
  return workspace_bytes(desc, M);
}

extern "C" tp_status tp_shard_pack(const tp_shard_desc* d, const uint16_t* W, int64_t ldw,
                                   void* W_packed, hipStream_t stream) {
  tp_status st = check_desc(d);
  if (st != TP_OK) return st;
  if (W == nullptr || W_packed == nullptr) return TP_ERR_NULL;
  if (ldw < d->N) return TP_ERR_SHAPE;
  if (!aligned16(W_packed)) return TP_ERR_ALIGN;
  // A TP_DGRAD plan keeps the forward shard's rows and column ranges: its
  // output columns are the forward rows, its contraction the forward columns.
  const bool dgrad = d->kind == TP_DGRAD;
  const int64_t nrows = dgrad ? d->shard_n : d->shard_k, ncols = dgrad ? d->shard_k : d->shard_n;
  if (d->row_begin < 0 || d->row_end > d->K || d->row_end - d->row_begin != nrows ||
      d->n_col_ranges < 1 || d->n_col_ranges > 3)
    return TP_ERR_SHAPE;
  tpk::PackArgs a;
  a.W = W;
  a.ldw = ldw;
  a.out = static_cast<uint4*>(W_packed);
  a.row_begin = d->row_begin;
  a.shard_k = d->shard_k;
  a.shard_n = d->shard_n;
  a.out_n = d->out_n;
  a.ksteps = ksteps_of(d);
  a.ntiles = d->packed_n / tpk::kTileN;
  a.n_ranges = d->n_col_ranges;
  a.gateup = d->kind == TP_GATEUP_COL;
  a.scales = is_fp8(d) ? reinterpret_cast<float*>(static_cast<uint8_t*>(W_packed) +
                                                  d->packed_k * d->packed_n)
                       : nullptr;
  for (int r = 0; r < 3; ++r) {
    const tp_col_range c = r < d->n_col_ranges ? d->col_ranges[r] : tp_col_range{0, 0, 0};
    if (r < d->n_col_ranges && (c.src_col < 0 || c.len < 0 || c.src_col + c.len > d->N ||
                                c.dst_col < 0 || c.dst_col + c.len > ncols))
      return TP_ERR_SHAPE;
    a.src[r] = c.src_col;
    a.len[r] = c.len;
    a.dst[r] = c.dst_col;
  }
  const hipError_t e = dgrad ? tpk::launch_pack_dgrad(a, stream)
                             : (is_fp8(d) ? tpk::launch_pack8(a, stream) : tpk::launch_pack(a, stream));
  return e == hipSuccess ? TP_OK : TP_ERR_HIP;
}

extern "C" tp_status tp_col_linear(const tp_shard_desc* d, const uint16_t* X, int64_t M,
                                   int64_t ldx, const void* W_packed, uint16_t* Y, int64_t ldy,
                                   void* ws, size_t ws_bytes, hipStream_t stream) {
  tp_status st = check_desc(d);
  if (st != TP_OK) return st;
  if (!is_col(d->kind)) return TP_ERR_KIND;
  st = check_linear_io(d, X, M, ldx, W_packed, Y, ldy, 8);
  if (st != TP_OK || M == 0) return st;
  const tpk::LinearArgs a = make_args(d, X, M, ldx, W_packed, Y, ldy);
  return run_linear(d, a, ws, ws_bytes, stream);
}

extern "C" tp_status tp_row_linear(const tp_shard_desc* d, const uint16_t* Z, int64_t M,
                                   int64_t ldz, const void* W_packed, float* P, int64_t ldp,
                                   void* ws, size_t ws_bytes, hipStream_t stream) {
  tp_status st = check_desc(d);
  if (st != TP_OK) return st;
  if (!is_row(d->kind)) return TP_ERR_KIND;
  st = check_linear_io(d, Z, M, ldz, W_packed, P, ldp, 4);
  if (st != TP_OK || M == 0) return st;
  const tpk::LinearArgs a = make_args(d, Z, M, ldz, W_packed, P, ldp);
  return run_linear(d, a, ws, ws_bytes, stream);
}

extern "C" tp_status tp_ffn_shard(const tp_shard_desc* gu, const tp_shard_desc* dn,
                                  const uint16_t* X, int64_t M, int64_t ldx,
                                  const void* Wgu_packed, const void* Wd_packed, uint16_t* H_ws,
                                  float* P, int64_t ldp, void* ws, size_t ws_bytes,
                                  hipStream_t stream) {
  tp_status st = check_desc(gu);
  if (st != TP_OK) return st;
  st = check_desc(dn);
  if (st != TP_OK) return st;
  if (gu->kind != TP_GATEUP_COL || dn->kind != TP_ROW) return TP_ERR_KIND;
  if (gu->t != dn->t || gu->rank != dn->rank || gu->out_n != dn->shard_k || gu->K != dn->N)
    return TP_ERR_SHAPE;
  // Validate both halves before queueing either.
  st = check_linear_io(gu, X, M, ldx, Wgu_packed, H_ws, gu->out_n, 8);
  if (st != TP_OK) return st;
  st = check_linear_io(dn, H_ws, M, gu->out_n, Wd_packed, P, ldp, 4);
  if (st != TP_OK || M == 0) return st;
  const size_t need_gu = workspace_bytes(gu, M), need_dn = workspace_bytes(dn, M);
  const size_t need = need_gu > need_dn ? need_gu : need_dn;
  if (need > 0 && (ws == nullptr || ws_bytes < need)) return TP_ERR_WORKSPACE;
  st = tp_col_linear(gu, X, M, ldx, Wgu_packed, H_ws, gu->out_n, ws, ws_bytes, stream);
  if (st != TP_OK) return st;
  return tp_row_linear(dn, H_ws, M, gu->out_n, Wd_packed, P, ldp, ws, ws_bytes, stream);
}

// ---------------------------------------------------------------------------
// The feed-forward share without a caller workspace: the split-K partials go
// to a static device array. In host code `scratch` is only a host-side
// stand-in for the symbol; its device address (one per GPU) comes from
// hipGetSymbolAddress and is the only form ever passed to a kernel.

static __device__ __align__(256) unsigned char scratch[TP_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// The device address of this GPU's scratch array, looked up once per device
// with that device current.
tp_status scratch_of(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return TP_ERR_HIP;
  if (stream != nullptr) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess || sdev != dev) return TP_ERR_HIP;
  }
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return TP_ERR_HIP;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return TP_OK;
}

}  // namespace

extern "C" tp_status tp_ffn_shard_noalloc(const tp_shard_desc* gu, const tp_shard_desc* dn,
                                          const uint16_t* X, int64_t M, int64_t ldx,
                                          const void* Wgu_packed, const void* Wd_packed,
                                          uint16_t* H_ws, float* P, int64_t ldp, hipStream_t stream) {
  tp_status st = check_desc(gu);
  if (st != TP_OK) return st;
  st = check_desc(dn);
  if (st != TP_OK) return st;
  if (M < 0) return TP_ERR_SHAPE;
  const size_t need_gu = workspace_bytes(gu, M), need_dn = workspace_bytes(dn, M);
  if ((need_gu > need_dn ? need_gu : need_dn) > TP_NOALLOC_SCRATCH_BYTES) return TP_ERR_WORKSPACE;
  void* ws = nullptr;
  if (M > 0) {
    st = scratch_of(stream, &ws);
    if (st != TP_OK) return st;
  }
  return tp_ffn_shard(gu, dn, X, M, ldx, Wgu_packed, Wd_packed, H_ws, P, ldp, ws,
                      TP_NOALLOC_SCRATCH_BYTES, stream);
}

extern "C" tp_status tp_reduce_partials(const float* P, int64_t stride_elems, int32_t t, int64_t M,
                                        int64_t N, int64_t ldp, float* Y, int64_t ldy,
                                        hipStream_t stream) {
  if (t <= 0 || M < 0 || N <= 0 || ldp < N || ldy < N) return TP_ERR_SHAPE;
  if (M == 0) return TP_OK;
  if (P == nullptr || Y == nullptr) return TP_ERR_NULL;
  if (t > 1 && stride_elems < M * ldp) return TP_ERR_SHAPE;
  if (!aligned16(P) || !aligned16(Y) || N % 4 || ldp % 4 || ldy % 4 || stride_elems % 4)
    return TP_ERR_ALIGN;
  // One partial summed into itself: the result is already in place.
  if (t == 1 && Y == P && ldy == ldp) return TP_OK;
  return tpk::launch_reduce(P, stride_elems, t, M, N, ldp, Y, ldy, stream) == hipSuccess
             ? TP_OK
             : TP_ERR_HIP;
}

extern "C" tp_status tp_reduce_scatter_partials(const float* P, int64_t stride_elems, int32_t t,
                                                int64_t M, int64_t N, int64_t ldp, int32_t rank,
                                                float* Y, int64_t ldy, hipStream_t stream) {
  if (t <= 0 || M < 0 || N <= 0 || ldp < N || ldy < N) return TP_ERR_SHAPE;
  if (rank < 0 || rank >= t) return TP_ERR_RANK;
  if (M % t) return TP_ERR_INDIVISIBLE;
  if (M == 0) return TP_OK;
  if (P == nullptr || Y == nullptr) return TP_ERR_NULL;
  if (t > 1 && stride_elems < M * ldp) return TP_ERR_SHAPE;
  if (!aligned16(P) || !aligned16(Y) || N % 4 || ldp % 4 || ldy % 4 || stride_elems % 4)
    return TP_ERR_ALIGN;
  const int64_t Mt = M / t;
  return tpk::launch_reduce(P + (int64_t)rank * Mt * ldp, stride_elems, t, Mt, N, ldp, Y, ldy,
                            stream) == hipSuccess
             ? TP_OK
             : TP_ERR_HIP;
}

extern "C" tp_status tp_gather_rows(const uint16_t* Xs, int64_t stride_elems, int32_t t, int64_t Mt,
                                    int64_t N, int64_t ldb, uint16_t* X, int64_t ldx,
                                    hipStream_t stream) {
  if (t <= 0 || Mt < 0 || N <= 0 || ldb < N || ldx < N) return TP_ERR_SHAPE;
  if (Mt == 0) return TP_OK;
  if (Xs == nullptr || X == nullptr) return TP_ERR_NULL;
  if (t > 1 && stride_elems < Mt * ldb) return TP_ERR_SHAPE;
  if (!aligned16(Xs) || !aligned16(X) || N % 8 || ldb % 8 || ldx % 8 || stride_elems % 8)
    return TP_ERR_ALIGN;
  return tpk::launch_gather(Xs, stride_elems, t, Mt, N, ldb, X, ldx, stream) == hipSuccess
             ? TP_OK
             : TP_ERR_HIP;
}

extern "C" tp_status tp_weight_grad(const tp_shard_desc* fwd, const uint16_t* A, int64_t lda,
                                    const uint16_t* dC, int64_t lddc, int64_t M, float* dW,
                                    int64_t lddw, hipStream_t stream) {
  tp_status st = check_desc(fwd);
  if (st != TP_OK) return st;
  if (fwd->kind == TP_DGRAD) return TP_ERR_KIND;
  const int64_t K = fwd->shard_k, N = fwd->shard_n;
  if (M < 0 || lda < K || lddc < N || lddw < N) return TP_ERR_SHAPE;
  if (dW == nullptr || (M > 0 && (A == nullptr || dC == nullptr))) return TP_ERR_NULL;
  if (!aligned16(dW) || (M > 0 && (!aligned16(A) || !aligned16(dC))) || lda % 8 || lddc % 8 ||
      lddw % 4)
    return TP_ERR_ALIGN;
  return tpk::launch_wgrad(A, lda, dC, lddc, M, K, N, dW, lddw, stream) == hipSuccess ? TP_OK
                                                                                      : TP_ERR_HIP;
}

extern "C" tp_status tp_swiglu_backward(const uint16_t* GU, int64_t ldgu, const float* dH,
                                        int64_t lddh, int64_t M, int64_t w, uint16_t* dGU,
                                        int64_t lddgu, hipStream_t stream) {
  if (M < 0 || w <= 0 || ldgu < 2 * w || lddh < w || lddgu < 2 * w) return TP_ERR_SHAPE;
  if (M == 0) return TP_OK;
  if (GU == nullptr || dH == nullptr || dGU == nullptr) return TP_ERR_NULL;
  if (!aligned16(GU) || !aligned16(dH) || !aligned16(dGU) || w % 8 || ldgu % 8 || lddgu % 8 ||
      lddh % 4)
    return TP_ERR_ALIGN;
  return tpk::launch_swiglu_bwd(GU, ldgu, dH, lddh, M, w, dGU, lddgu, stream) == hipSuccess
             ? TP_OK
             : TP_ERR_HIP;
}

// ---------------------------------------------------------------------------
// Attention core on the rank's heads and its KV-cache share.

namespace {

// Heads of a TP_QKV_COL shard: query heads, key-value heads, head dimension
// and query heads per key-value head (all of them when the key-value head is
// repeated).
tp_status attn_heads(const tp_shard_desc* d, int& nq, int& nkv, int& D, int& G) {
  tp_status st = check_desc(d);
  if (st != TP_OK) return st;
  if (d->kind != TP_QKV_COL) return TP_ERR_KIND;
  nq = d->q_head_end - d->q_head_begin;
  nkv = d->kv_head_end - d->kv_head_begin;
  if (nq <= 0 || nkv <= 0 || nq % nkv) return TP_ERR_SHAPE;
  const int64_t width = nq + 2 * nkv;
  if (d->shard_n % width) return TP_ERR_SHAPE;
  D = (int)(d->shard_n / width);
  if (D != 64 && D != 128) return TP_ERR_SHAPE;
  G = nq / nkv;
  return TP_OK;
}

// One key-value head's cache rows are addressed with 32-bit byte offsets.
bool cache_ok(int D, int64_t n_slots, int64_t L_max) {
  return n_slots >= 1 && L_max >= 1 && L_max <= INT32_MAX / (2 * D);
}

bool attn_decode(int G, int32_t q_len) { return (int64_t)G * q_len <= tpk::kAttnDecodeRows; }


// Checks shared by the append and the attention; fills the arguments.
tp_status attn_args(const tp_shard_desc* qkv, const uint16_t* QKV, int64_t ldqkv, int32_t S,
                    int32_t q_len, const int32_t* kv_len, const int32_t* slot, const void* Kc,
                    const void* Vc, int64_t n_slots, int64_t L_max, int32_t max_kv,
                    tpk::AttnArgs& a) {
  int nq, nkv, D, G;
  tp_status st = attn_heads(qkv, nq, nkv, D, G);
  if (st != TP_OK) return st;
  if (S < 0 || q_len < 1 || ldqkv < qkv->shard_n || !cache_ok(D, n_slots, L_max) ||
      max_kv < q_len || max_kv > L_max)
    return TP_ERR_SHAPE;
  if (S > 0 && (QKV == nullptr || kv_len == nullptr || slot == nullptr || Kc == nullptr ||
                Vc == nullptr))
    return TP_ERR_NULL;
  if (S > 0 && (!aligned16(QKV) || !aligned16(Kc) || !aligned16(Vc) || ldqkv % 8 ||
                (reinterpret_cast<uintptr_t>(kv_len) & 3u) || (reinterpret_cast<uintptr_t>(slot) & 3u)))
    return TP_ERR_ALIGN;
  a = tpk::AttnArgs{};
  a.QKV = QKV;
  a.ldqkv = ldqkv;
  a.kv_len = kv_len;
  a.slot = slot;
  a.Kc = static_cast<const uint16_t*>(Kc);
  a.Vc = static_cast<const uint16_t*>(Vc);
  a.n_slots = n_slots;
  a.L_max = L_max;
  a.S = S;
  a.q_len = q_len;
  a.nq = nq;
  a.nkv = nkv;
  a.G = G;
  a.D = D;
  a.max_kv = max_kv;
  a.qscale = (float)(1.4426950408889634 / std::sqrt((double)D));
  return TP_OK;
}

}  // namespace

extern "C" size_t tp_kv_cache_bytes(const tp_shard_desc* qkv, int64_t n_slots, int64_t L_max) {
  int nq, nkv, D, G;
  if (attn_heads(qkv, nq, nkv, D, G) != TP_OK || !cache_ok(D, n_slots, L_max)) return 0;
  return (size_t)n_slots * (size_t)nkv * (size_t)L_max * (size_t)D * 2;
}

extern "C" tp_status tp_kv_append(const tp_shard_desc* qkv, const uint16_t* QKV, int64_t ldqkv,
                                  int32_t S, int32_t q_len, const int32_t* kv_len,
                                  const int32_t* slot, uint16_t* Kc, uint16_t* Vc, int64_t n_slots,
                                  int64_t L_max, hipStream_t stream) {
  tpk::AttnArgs a;
  const int32_t max_kv = L_max < INT32_MAX ? (int32_t)L_max : INT32_MAX;
  tp_status st = attn_args(qkv, QKV, ldqkv, S, q_len, kv_len, slot, Kc, Vc, n_slots, L_max,
                           q_len > max_kv ? q_len : max_kv, a);
  if (st != TP_OK || S == 0) return st;
  a.Kw = Kc;
  a.Vw = Vc;
  return tpk::launch_kv_append(a, stream) == hipSuccess ? TP_OK : TP_ERR_HIP;
}

extern "C" size_t tp_attention_workspace_bytes(const tp_shard_desc* qkv, int32_t S, int32_t q_len,
                                               int32_t max_kv) {
  int nq, nkv, D, G;
  if (attn_heads(qkv, nq, nkv, D, G) != TP_OK || S < 0 || q_len < 1 || max_kv < q_len) return 0;
  if (!attn_decode(G, q_len)) return 0;
  int32_t nchunk, npw;
  tpk::attn_decode_split(S, nkv, max_kv, nchunk, npw);
  return tpk::attn_decode_ws_bytes(S, nkv, nchunk, D);
}

extern "C" tp_status tp_attention(const tp_shard_desc* qkv, const uint16_t* QKV, int64_t ldqkv,
                                  int32_t S, int32_t q_len, const int32_t* kv_len,
                                  const int32_t* slot, int32_t max_kv, const uint16_t* Kc,
                                  const uint16_t* Vc, int64_t n_slots, int64_t L_max, uint16_t* A,
                                  int64_t lda, void* ws, size_t ws_bytes, hipStream_t stream) {
  tpk::AttnArgs a;
  tp_status st = attn_args(qkv, QKV, ldqkv, S, q_len, kv_len, slot, Kc, Vc, n_slots, L_max, max_kv, a);
  if (st != TP_OK) return st;
  if (lda < (int64_t)a.nq * a.D) return TP_ERR_SHAPE;
  if (S == 0) return TP_OK;
  if (A == nullptr) return TP_ERR_NULL;
  if (!aligned16(A) || lda % 8) return TP_ERR_ALIGN;
  a.A = A;
  a.lda = lda;
  const bool decode = attn_decode(a.G, q_len);
  if (decode) {
    tpk::attn_decode_split(S, a.nkv, max_kv, a.nchunk, a.npw);
    const size_t need = tpk::attn_decode_ws_bytes(S, a.nkv, a.nchunk, a.D);
    if (need > 0 && (ws == nullptr || ws_bytes < need || !aligned16(ws))) return TP_ERR_WORKSPACE;
    a.ws = static_cast<float*>(ws);
  } else if ((int64_t)((q_len + 63) / 64) * a.nq * S > INT32_MAX) {
    return TP_ERR_SHAPE;
  }
  if (S > 65535) return TP_ERR_SHAPE;
  return tpk::launch_attention(a, decode, stream) == hipSuccess ? TP_OK : TP_ERR_HIP;
}
