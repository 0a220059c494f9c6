// Host-side shard planning: which rows and columns of the full weight a rank
// owns, and how big its packed copy is. Integer work only, no GPU calls.
//
// Rules: "Tensor vs Pipeline Parallelism" (xingyuzhitong.com), sections
// "Tensor parallelism: split inside each layer" (leading matrix cut by output
// columns, trailing one by input rows, heads shared out, head counts a
// multiple of the degree) and "Common
// mistakes" (a degree that does not divide the key-value heads is refused);
// "AI Infrastructure series, Part 5" (drpranayjha.com), "How does tensor
// parallelism split a layer?" (64 heads: 2, 4 or 8 ranks, not 3 or 6; past 8
// key-value heads, key-value heads are repeated).
#include <cstring>

#include "tp_internal.h"

namespace {

int64_t round_up(int64_t v, int64_t q) { return (v + q - 1) / q * q; }

// Key-value head block of one rank; returns TP_OK or TP_ERR_INDIVISIBLE.
tp_status assign_heads(const tp_heads& h, int32_t t, int32_t rank, tp_shard_desc* d) {
  if (h.n_q % t != 0) return TP_ERR_INDIVISIBLE;
  const int32_t q_per = h.n_q / t;
  d->q_head_begin = rank * q_per;
  d->q_head_end = d->q_head_begin + q_per;
  if (t <= h.n_kv) {
    if (h.n_kv % t != 0) return TP_ERR_INDIVISIBLE;
    const int32_t kv_per = h.n_kv / t;
    d->kv_head_begin = rank * kv_per;
    d->kv_head_end = d->kv_head_begin + kv_per;
    d->kv_replicated = 0;
  } else {
    if (t % h.n_kv != 0) return TP_ERR_INDIVISIBLE;
    // t / n_kv consecutive ranks share one key-value head.
    d->kv_head_begin = rank / (t / h.n_kv);
    d->kv_head_end = d->kv_head_begin + 1;
    d->kv_replicated = 1;
  }
  return TP_OK;
}

}  // namespace

extern "C" tp_status tp_shard_plan(tp_kind kind, int64_t K, int64_t N, int32_t t, int32_t rank,
                                   const tp_heads* heads, tp_shard_desc* out) {
  if (out == nullptr) return TP_ERR_NULL;
  if (kind < TP_COL || kind > TP_O_ROW) return TP_ERR_KIND;
  if (K <= 0 || N <= 0 || t <= 0) return TP_ERR_SHAPE;
  if (rank < 0 || rank >= t) return TP_ERR_RANK;
  const bool attention = kind == TP_QKV_COL || kind == TP_O_ROW;
  if (attention && heads == nullptr) return TP_ERR_NULL;

  tp_shard_desc d;
  std::memset(&d, 0, sizeof d);
  d.kind = kind;
  d.t = t;
  d.rank = rank;
  d.K = K;
  d.N = N;
  d.path = TP_PATH_AUTO;

  switch (kind) {
    case TP_COL: {
      if (N % t) return TP_ERR_INDIVISIBLE;
      const int64_t w = N / t;
      d.row_begin = 0;
      d.row_end = K;
      d.n_col_ranges = 1;
      d.col_ranges[0] = {rank * w, w, 0};
      d.shard_n = d.out_n = w;
      break;
    }
    case TP_ROW: {
      if (K % t) return TP_ERR_INDIVISIBLE;
      const int64_t h = K / t;
      d.row_begin = rank * h;
      d.row_end = d.row_begin + h;
      d.n_col_ranges = 1;
      d.col_ranges[0] = {0, N, 0};
      d.shard_n = d.out_n = N;
      break;
    }
    case TP_GATEUP_COL: {
      if (N % 2) return TP_ERR_SHAPE;
      const int64_t inter = N / 2;
      if (inter % t) return TP_ERR_INDIVISIBLE;
      const int64_t w = inter / t;
      d.row_begin = 0;
      d.row_end = K;
      d.n_col_ranges = 2;
      d.col_ranges[0] = {rank * w, w, 0};          // gate columns
      d.col_ranges[1] = {inter + rank * w, w, w};  // the matching up columns
      d.shard_n = 2 * w;
      d.out_n = w;
      break;
    }
    case TP_QKV_COL:
    case TP_O_ROW: {
      const tp_heads h = *heads;
      if (h.n_q <= 0 || h.n_kv <= 0 || h.head_dim <= 0 || h.n_q % h.n_kv) return TP_ERR_SHAPE;
      const int64_t hd = h.head_dim;
      if (kind == TP_QKV_COL && N != (int64_t)(h.n_q + 2 * h.n_kv) * hd) return TP_ERR_SHAPE;
      if (kind == TP_O_ROW && K != (int64_t)h.n_q * hd) return TP_ERR_SHAPE;
      tp_status s = assign_heads(h, t, rank, &d);
      if (s != TP_OK) return s;
      const int64_t q0 = d.q_head_begin * hd, nq = (int64_t)(d.q_head_end - d.q_head_begin) * hd;
      if (kind == TP_QKV_COL) {
        const int64_t kv0 = d.kv_head_begin * hd;
        const int64_t nkv = (int64_t)(d.kv_head_end - d.kv_head_begin) * hd;
        const int64_t k_base = (int64_t)h.n_q * hd, v_base = k_base + (int64_t)h.n_kv * hd;
        d.row_begin = 0;
        d.row_end = K;
        d.n_col_ranges = 3;
        d.col_ranges[0] = {q0, nq, 0};
        d.col_ranges[1] = {k_base + kv0, nkv, nq};
        d.col_ranges[2] = {v_base + kv0, nkv, nq + nkv};
        d.shard_n = d.out_n = nq + 2 * nkv;
      } else {
        d.row_begin = q0;
        d.row_end = q0 + nq;
        d.n_col_ranges = 1;
        d.col_ranges[0] = {0, N, 0};
        d.shard_n = d.out_n = N;
      }
      if (hd % 8) return TP_ERR_ALIGN;
      break;
    }
  }
  d.shard_k = d.row_end - d.row_begin;
  if (d.shard_k % 8 || d.out_n % 8 || d.shard_n % 8) return TP_ERR_ALIGN;

  d.packed_k = round_up(d.shard_k, tpk::kTileK);
  // Whole tile pairs (32 columns); gate/up pairs are a gate and an up tile.
  d.packed_n = kind == TP_GATEUP_COL ? 2 * round_up(d.out_n, tpk::kTileN)
                                     : round_up(d.shard_n, 2 * tpk::kTileN);
  d.packed_bytes = d.packed_k * d.packed_n * 2;
  d.wformat = TP_W_BF16;
  d.reserved = 0;
  *out = d;
  return TP_OK;
}

extern "C" tp_status tp_shard_plan_dgrad(const tp_shard_desc* fwd, tp_shard_desc* out) {
  if (fwd == nullptr || out == nullptr) return TP_ERR_NULL;
  if (fwd->kind < TP_COL || fwd->kind > TP_O_ROW) return TP_ERR_KIND;
  if (fwd->shard_k <= 0 || fwd->shard_n <= 0 || fwd->n_col_ranges < 1 || fwd->n_col_ranges > 3)
    return TP_ERR_SHAPE;
  if (fwd->shard_k % 8 || fwd->shard_n % 8) return TP_ERR_ALIGN;
  tp_shard_desc d = *fwd;  // keeps t, rank, K, N, rows, column ranges, heads
  d.kind = TP_DGRAD;
  d.shard_k = fwd->shard_n;  // contraction: the forward output columns
  d.shard_n = d.out_n = fwd->shard_k;
  d.path = TP_PATH_AUTO;
  d.packed_k = round_up(d.shard_k, tpk::kTileK);
  d.packed_n = round_up(d.shard_n, 2 * tpk::kTileN);
  d.packed_bytes = d.packed_k * d.packed_n * 2;
  d.wformat = TP_W_BF16;
  d.reserved = 0;
  *out = d;
  return TP_OK;
}

extern "C" tp_status tp_shard_set_wformat(tp_shard_desc* d, int32_t wformat) {
  if (d == nullptr) return TP_ERR_NULL;
  if (d->shard_k <= 0 || d->packed_n <= 0) return TP_ERR_SHAPE;
  if (d->kind == TP_DGRAD && wformat != TP_W_BF16) return TP_ERR_KIND;
  switch (wformat) {
    case TP_W_BF16:
      d->packed_k = round_up(d->shard_k, tpk::kTileK);
      d->packed_bytes = d->packed_k * d->packed_n * 2;
      break;
    case TP_W_FP8_E4M3:
      d->packed_k = round_up(d->shard_k, tpk::kTileK8);
      d->packed_bytes = d->packed_k * d->packed_n + 4 * d->packed_n;
      break;
    default:
      return TP_ERR_KIND;
  }
  d->wformat = wformat;
  return TP_OK;
}

extern "C" const char* tp_status_str(tp_status s) {
  switch (s) {
    case TP_OK: return "ok";
    case TP_ERR_NULL: return "null pointer";
    case TP_ERR_SHAPE: return "bad shape";
    case TP_ERR_INDIVISIBLE: return "tensor-parallel degree does not divide the split";
    case TP_ERR_RANK: return "rank out of range";
    case TP_ERR_ALIGN: return "misaligned pointer, leading dimension or width";
    case TP_ERR_WORKSPACE: return "workspace too small";
    case TP_ERR_HIP: return "HIP launch error";
    case TP_ERR_KIND: return "bad kind";
    default: return "unknown status";
  }
}
