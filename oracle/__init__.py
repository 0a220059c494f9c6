"""fp64 CPU oracle for one tensor-parallel rank's linear share.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package. It shares no code
with the HIP library (no kernels, headers, helpers or tables) and imports
nothing from it.

Sources (cited by page title and section):

* "How do tensor parallelism (TP) and pipeline parallelism (PP) split large
  model weights across multi-GPU nodes?" (iloveeagents.com), "Detail": a
  4096 x 4096 matrix W cut column-wise gives each of two GPUs a 4096 x 2048
  piece; "Example": a column-parallel linear keeps out_features / t output
  features and computes the local product x @ W_r.
* "Tensor vs Pipeline Parallelism" (xingyuzhitong.com), "Tensor parallelism:
  split inside each layer": the MLP's leading matrix is cut by output
  columns and its trailing one by input rows, the heads are shared out, and
  the ranks' partial products are added; head and key-value head counts
  have to be multiples of the degree. "Common mistakes": frameworks reject a
  degree that the key-value heads do not divide.
* "AI Infrastructure series, Part 5" (drpranayjha.com), "How does tensor
  parallelism split a layer?": a 64-query-head model takes 2, 4 or 8 ranks,
  never 3 or 6, and ranks beyond the 8 key-value heads hold copies of a
  key-value head. "Short answers": the split changes only the order of the
  additions, hence only the last digits.
* "Tensor Parallelism" glossary (aidolsgroup.com), "Full definition": every
  rank sees the same input; the partial products are added.

Readings where the pages are silent (the same list is in the design notes):

* W is logical [K_in x N_out], row-major, Y = X W; "column" = output feature.
* Column-shard outputs are concatenated; only row-shard partials are summed.
* The feed-forward nonlinearity is SwiGLU, H = SiLU(G) * U with
  SiLU(g) = g / (1 + e^-g) on the gate; the fused matrix is [Wg | Wu], gate
  first; rank r takes the same column range of Wg and of Wu. No bias.
* QKV is [Wq | Wk | Wv]; rank r takes Q heads [r n_q / t, (r+1) n_q / t);
  key-value heads [r n_kv / t, (r+1) n_kv / t) when t <= n_kv, else the one
  head floor(r n_kv / t), replicated. The O projection takes the rows of the
  rank's Q dims.
* A degree that does not divide is an error, never a ragged split.
* Rounding points: a column output consumed in bf16 (Y_r, H_r, QKV_r) is
  rounded to bf16 (nearest, ties to even) from the fp64 value; row partials
  and their sum stay unrounded.
* 8-bit weights (the pages fix no format): OCP FP8 E4M3 codes, one
  power-of-two scale per output column of the rank's shard, the smallest that
  keeps every scaled weight within 448; codes round to nearest, ties to even;
  activations stay bf16.
* Backward: the input gradient of a rank's linear is dC_r W_r^T (for the
  column kinds a partial, summed over the ranks like the forward partials),
  its weight gradient A_r^T dC_r; the gate/up gradient [dG | dU] is rounded
  to bf16 once, as the products that consume it read bf16.
* Attention core on the rank's heads (the pages give no formula): scaled
  dot-product attention softmax(q k^T / sqrt(d)) v per query head, causal (a
  new token at cache position p sees positions 0..p of its sequence), no
  position encoding, no bias; query head q uses key-value head
  floor(q / (n_q / n_kv)), which for a rank is its own local copy. The rank
  keeps K and V of its key-value heads for every token (its share of the KV
  cache). Output rows are the rank's query heads side by side, rounded to
  bf16 once (the O projection reads bf16).
* Sequence parallelism (the pages name only what it splits): after the
  row-parallel product rank r keeps rows [r M/t, (r+1) M/t) of the summed
  partials (a reduce-scatter along the tokens), and the full activations for
  the next column-parallel product are the ranks' row blocks stacked in rank
  order (an all-gather); M must divide by t.

Every product below, whatever its operands (bf16 shards, dequantised 8-bit
shards, gradients, attention scores), is the C core's in-order fp64 loop:
one accumulator per output, the contraction index ascending, no BLAS.

Every function below is parity-pinned by ``tests/test_oracle_pins.py`` and
``tests/test_oracle_attention_pins.py``.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.orc_bf16_to_f64.argtypes = [ctypes.c_uint16]
        lib.orc_bf16_to_f64.restype = ctypes.c_double
        lib.orc_f64_to_bf16.argtypes = [ctypes.c_double]
        lib.orc_f64_to_bf16.restype = ctypes.c_uint16
        lib.orc_round_bf16.argtypes = [P, I64, P]
        lib.orc_bf16_to_f64_array.argtypes = [P, I64, P]
        lib.orc_shard_matmul.argtypes = [P, I64, I64, I64, P, I64, P, P, I64, P]
        lib.orc_swiglu.argtypes = [P, P, I64, P]
        lib.orc_sum_partials.argtypes = [P, I64, ctypes.c_int32, I64, P]
        lib.orc_matmul_f64.argtypes = [P, I64, I64, I64, I64, P, I64, I64, I64, P]
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


# --------------------------------------------------------------------------
# Shard bookkeeping (independent of the HIP library's planner).
# --------------------------------------------------------------------------

KINDS = ("col", "row", "gateup_col", "qkv_col", "o_row")


class PlanError(ValueError):
    """Raised with ``code`` in {"shape", "indivisible", "rank", "kind"}."""

    def __init__(self, code: str, msg: str):
        super().__init__(f"{code}: {msg}")
        self.code = code


def _head_sets(t: int, rank: int, n_q: int, n_kv: int):
    """Q-head range, KV-head range and replication flag of rank ``rank``."""
    if n_q % t != 0:
        raise PlanError("indivisible", f"{n_q} query heads over {t} ranks")
    if t <= n_kv:
        if n_kv % t != 0:
            raise PlanError("indivisible", f"{n_kv} key-value heads over {t} ranks")
        per = n_kv // t
        kv = (rank * per, rank * per + per)
        replicated = False
    else:
        if t % n_kv != 0:
            raise PlanError("indivisible", f"{t} ranks do not repeat {n_kv} key-value heads evenly")
        h = (rank * n_kv) // t
        kv = (h, h + 1)
        replicated = True
    q_per = n_q // t
    return (rank * q_per, rank * q_per + q_per), kv, replicated


def plan(kind: str, K: int, N: int, t: int, rank: int, heads=None) -> dict:
    """Which rows and columns of the full logical weight W [K x N] rank
    ``rank`` of ``t`` uses, in shard order.

    Returns a dict with ``rows`` and ``cols`` (int64 index arrays into W),
    ``shard_k``/``shard_n``, and for the attention kinds the head sets.
    """
    if kind not in KINDS:
        raise PlanError("kind", kind)
    if K <= 0 or N <= 0 or t <= 0:
        raise PlanError("shape", f"K={K} N={N} t={t}")
    if not 0 <= rank < t:
        raise PlanError("rank", f"rank {rank} of {t}")
    out = dict(kind=kind, K=K, N=N, t=t, rank=rank, q_heads=None, kv_heads=None,
               kv_replicated=False)
    all_rows = np.arange(K, dtype=np.int64)
    all_cols = np.arange(N, dtype=np.int64)
    if kind == "col":
        if N % t:
            raise PlanError("indivisible", f"N={N} over {t}")
        w = N // t
        rows, cols = all_rows, np.arange(rank * w, rank * w + w, dtype=np.int64)
    elif kind == "row":
        if K % t:
            raise PlanError("indivisible", f"K={K} over {t}")
        h = K // t
        rows, cols = np.arange(rank * h, rank * h + h, dtype=np.int64), all_cols
    elif kind == "gateup_col":
        if N % 2:
            raise PlanError("shape", "fused gate/up width must be even")
        inter = N // 2
        if inter % t:
            raise PlanError("indivisible", f"I={inter} over {t}")
        w = inter // t
        gate = np.arange(rank * w, rank * w + w, dtype=np.int64)
        rows, cols = all_rows, np.concatenate([gate, gate + inter])
    else:
        if heads is None:
            raise PlanError("shape", "attention kinds need heads")
        n_q, n_kv, d = heads
        if n_q <= 0 or n_kv <= 0 or d <= 0 or n_q % n_kv:
            raise PlanError("shape", f"heads {heads}")
        (q0, q1), (k0, k1), rep = _head_sets(t, rank, n_q, n_kv)
        out.update(q_heads=(q0, q1), kv_heads=(k0, k1), kv_replicated=rep, heads=(n_q, n_kv, d))
        if kind == "qkv_col":
            if N != (n_q + 2 * n_kv) * d:
                raise PlanError("shape", f"N={N} != (n_q + 2 n_kv) d")
            q = np.arange(q0 * d, q1 * d, dtype=np.int64)
            k = np.arange(k0 * d, k1 * d, dtype=np.int64) + n_q * d
            v = k + n_kv * d
            rows, cols = all_rows, np.concatenate([q, k, v])
        else:  # o_row
            if K != n_q * d:
                raise PlanError("shape", f"K={K} != n_q d")
            rows, cols = np.arange(q0 * d, q1 * d, dtype=np.int64), all_cols
    out.update(rows=rows, cols=cols, shard_k=len(rows), shard_n=len(cols))
    return out


# --------------------------------------------------------------------------
# Arithmetic (C core, fp64).
# --------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(b.shape, dtype=np.float64)
    _load().orc_bf16_to_f64_array(_ptr(b), b.size, _ptr(out))
    return out


def round_bf16(x: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(a.shape, dtype=np.uint16)
    _load().orc_round_bf16(_ptr(a), a.size, _ptr(out))
    return out


def _rowmajor(a: np.ndarray) -> tuple[np.ndarray, int]:
    """uint16 2-D array with unit column stride; returns (array, leading dim)."""
    assert a.dtype == np.uint16 and a.ndim == 2
    if a.strides[1] != 2 or a.strides[0] % 2:
        a = np.ascontiguousarray(a)
    return a, max(a.strides[0] // 2, a.shape[1])


def shard_matmul(X: np.ndarray, W: np.ndarray, rows: np.ndarray, cols: np.ndarray) -> np.ndarray:
    """Y[m, j] = sum_kk X[m, kk] W[rows[kk], cols[j]] in fp64, kk ascending."""
    X, ldx = _rowmajor(X)
    W, ldw = _rowmajor(W)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    M, Kr = X.shape
    assert Kr == len(rows), (Kr, len(rows))
    assert len(rows) == 0 or (rows.min() >= 0 and rows.max() < W.shape[0])
    assert len(cols) == 0 or (cols.min() >= 0 and cols.max() < W.shape[1])
    Y = np.empty((M, len(cols)), dtype=np.float64)
    if M and len(cols):
        _load().orc_shard_matmul(_ptr(X), M, ldx, Kr, _ptr(W), ldw, _ptr(rows), _ptr(cols),
                                 len(cols), _ptr(Y))
    return Y


def _f64_strided(a: np.ndarray) -> tuple[np.ndarray, int, int]:
    """(array, row stride, column stride) in elements of a 2-D fp64 array;
    transposed views are passed as they are, anything else is copied."""
    a = np.asarray(a, dtype=np.float64)
    assert a.ndim == 2
    s0, s1 = a.strides
    if s0 < 0 or s1 < 0 or s0 % 8 or s1 % 8:
        a = np.ascontiguousarray(a)
        s0, s1 = a.strides
    return a, s0 // 8, s1 // 8


def matmul_f64(A: np.ndarray, B: np.ndarray) -> np.ndarray:
    """C[m, n] = sum_k A[m, k] B[k, n] in fp64, k ascending, one accumulator
    per output (the C core's in-order loop; no BLAS)."""
    A, sam, sak = _f64_strided(A)
    B, sbk, sbn = _f64_strided(B)
    M, K = A.shape
    assert B.shape[0] == K, (A.shape, B.shape)
    N = B.shape[1]
    C = np.empty((M, N), dtype=np.float64)
    if M and N:
        if K == 0:
            C[:] = 0.0
        else:
            _load().orc_matmul_f64(_ptr(A), M, K, sam, sak, _ptr(B), N, sbk, sbn, _ptr(C))
    return C


def swiglu(G: np.ndarray, U: np.ndarray) -> np.ndarray:
    """bf16 bits of SiLU(G) * U, rounded once from fp64."""
    G = np.ascontiguousarray(G, dtype=np.float64)
    U = np.ascontiguousarray(U, dtype=np.float64)
    assert G.shape == U.shape
    H = np.empty(G.shape, dtype=np.uint16)
    _load().orc_swiglu(_ptr(G), _ptr(U), G.size, _ptr(H))
    return H


def sum_partials(P: np.ndarray) -> np.ndarray:
    """Y = P[0] + P[1] + ... + P[t-1], added in rank order, fp64."""
    P = np.ascontiguousarray(P, dtype=np.float64)
    t = P.shape[0]
    Y = np.empty(P.shape[1:], dtype=np.float64)
    stride = int(np.prod(P.shape[1:]))
    _load().orc_sum_partials(_ptr(P), stride, t, stride, _ptr(Y))
    return Y


def reduce_scatter(P: np.ndarray, rank: int) -> np.ndarray:
    """Sequence-parallel partial sum of rank ``rank``: its own 1/t of the token
    rows of P[0] + ... + P[t-1], added in rank order, fp64 [M/t x N].

    "AI Infrastructure series, Part 5", "What about MoE models and very long
    prompts?": sequence parallelism splits the parts of a layer that tensor
    parallelism leaves whole along the sequence, inside the tensor-parallel
    group. After the row-parallel product each rank then keeps only its token
    rows of the summed output; rank r's rows are [r M/t, (r+1) M/t). M must
    divide by t."""
    P = np.asarray(P)
    t, M = P.shape[0], P.shape[1]
    if not 0 <= rank < t:
        raise PlanError("rank", f"rank {rank} of {t}")
    if M % t != 0:
        raise PlanError("indivisible", f"{M} token rows over {t} ranks")
    Mt = M // t
    return sum_partials(P[:, rank * Mt:(rank + 1) * Mt])


def gather_rows(blocks) -> np.ndarray:
    """The matching gather of the activations before the next column-parallel
    product: the t ranks' row blocks [M/t x N], stacked in rank order."""
    blocks = [np.asarray(b) for b in blocks]
    assert blocks and all(b.shape == blocks[0].shape for b in blocks)
    return np.concatenate(blocks, axis=0)


# --------------------------------------------------------------------------
# 8-bit weights for decode ("AI Infrastructure series, Part 5", "Reason 2":
# a decoded token streams all the weights, 70.6 GB for a 70B model stored in
# 8 bits, half of its 16-bit size). The pages fix no format. Reading
# taken: OCP FP8 E4M3 codes with one power-of-two scale per output column of
# the rank's shard; the activations stay bf16 (weight-only quantisation).
# --------------------------------------------------------------------------

E4M3_MAX = 448.0  # largest finite E4M3 value, 1.75 * 2^8


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """fp64 values of OCP E4M3 codes: sign bit, 4 exponent bits (bias 7), 3
    mantissa bits; exponent field 0 holds the subnormals m 2^-9; the two codes
    S.1111.111 are NaN; there are no infinities."""
    c = np.asarray(codes).astype(np.int64)
    s, e, m = c >> 7, (c >> 3) & 15, c & 7
    v = np.where(e == 0, m * 2.0 ** -9, (8 + m) * np.exp2(e - 10.0))
    v = np.where((e == 15) & (m == 7), np.nan, v)
    return np.where(s == 1, -v, v)


def column_exponents(W: np.ndarray) -> np.ndarray:
    """e_n = the smallest integer with max_k |W[k, n]| <= 448 * 2^e_n; 0 for an
    all-zero column. With amax = f 2^x, f in [0.5, 1), and 448 = 0.875 2^9:
    e = x - 9 when f <= 0.875, else x - 8 (exact, no rounding)."""
    amax = np.abs(np.asarray(W, dtype=np.float64)).max(axis=0)
    e = np.zeros(amax.shape, dtype=np.int64)
    nz = amax > 0
    f, x = np.frexp(amax[nz])
    e[nz] = np.where(f <= 0.875, x - 9, x - 8)
    return e


def e4m3_round(v: np.ndarray) -> np.ndarray:
    """E4M3 codes nearest to v (|v| <= 448), ties to the even code (mantissa bit
    0 clear); the sign is kept, so a negative value that rounds to zero gives
    the code of -0."""
    v = np.asarray(v, dtype=np.float64)
    assert np.all(np.abs(v) <= E4M3_MAX), "scaled weights must lie within the E4M3 range"
    table = e4m3_decode(np.arange(0x7F))  # non-negative finite codes 0 .. 0x7E, increasing
    a = np.abs(v).ravel()
    hi = np.minimum(np.searchsorted(table, a, side="left"), 0x7E)
    lo = np.maximum(hi - 1, 0)
    dlo, dhi = a - table[lo], table[hi] - a  # exact: both sides are short dyadic numbers
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    mag = np.where(a == table[hi], hi, np.where(pick_hi, hi, lo))
    sign = np.signbit(v.ravel()).astype(np.int64) << 7
    return (mag | sign).astype(np.uint8).reshape(v.shape)


def quantize_columns(W: np.ndarray):
    """(codes uint8 [K x N], exponents int64 [N]) of a weight matrix in fp64:
    codes = E4M3 round of W[k, n] 2^-e_n."""
    W = np.asarray(W, dtype=np.float64)
    e = column_exponents(W)
    return e4m3_round(W * np.exp2(-e.astype(np.float64))), e


def dequantize_columns(codes: np.ndarray, e: np.ndarray) -> np.ndarray:
    """The weights the 8-bit linear multiplies by: decode(q) 2^e_n, exact."""
    return e4m3_decode(codes) * np.exp2(np.asarray(e, dtype=np.float64))


def _shard_f64(W: np.ndarray, rows, cols) -> np.ndarray:
    return bf16_to_f64(np.ascontiguousarray(W[np.asarray(rows)][:, np.asarray(cols)]))


def shard_weight_fp8(W: np.ndarray, p: dict) -> np.ndarray:
    """The rank's shard as its 8-bit form multiplies it: each of the shard's
    output columns quantised on its own (for gate/up: gate and up columns
    separately), then dequantised, fp64 [shard_k x shard_n]."""
    q, e = quantize_columns(_shard_f64(W, p["rows"], p["cols"]))
    return dequantize_columns(q, e)


def col_linear_fp8(X: np.ndarray, W: np.ndarray, p: dict) -> np.ndarray:
    """X W'_r in fp64, unrounded (W'_r: the dequantised 8-bit shard)."""
    assert p["kind"] in ("col", "qkv_col")
    return matmul_f64(bf16_to_f64(X), shard_weight_fp8(W, p))


def gateup_swiglu_fp8(X: np.ndarray, Wgu: np.ndarray, p: dict) -> np.ndarray:
    """H_r = bf16(SiLU(X W'_g) * (X W'_u)) with 8-bit gate and up shards."""
    assert p["kind"] == "gateup_col"
    Wq = shard_weight_fp8(Wgu, p)
    half = p["shard_n"] // 2
    Xf = bf16_to_f64(X)
    return swiglu(matmul_f64(Xf, Wq[:, :half]), matmul_f64(Xf, Wq[:, half:]))


def row_linear_fp8(Z: np.ndarray, W: np.ndarray, p: dict) -> np.ndarray:
    """P_r = Z_r W'[rows_r, :] in fp64 with the 8-bit row shard."""
    assert p["kind"] in ("row", "o_row")
    return matmul_f64(bf16_to_f64(Z), shard_weight_fp8(W, p))


# --------------------------------------------------------------------------
# Backward of the rank share ("Tensor vs Pipeline Parallelism", "Tensor
# parallelism: split inside each layer": training adds two all-reduces per
# layer in the backward pass, one per block, which sum the ranks' input
# gradients; "AI Infrastructure series, Part 5", "Why are 8 GPUs not 8 times
# faster?": training costs 6 x parameters x tokens, the backward twice the
# forward -- one input-gradient and one weight-gradient product per linear).
# --------------------------------------------------------------------------

def _shard_weight_f64(W: np.ndarray, p: dict) -> np.ndarray:
    return bf16_to_f64(np.ascontiguousarray(W[np.asarray(p["rows"])][:, np.asarray(p["cols"])]))


def grad_input(dC: np.ndarray, W: np.ndarray, p: dict) -> np.ndarray:
    """dA_r = dC_r W_r^T, fp64 [M x shard_k]: the gradient of the rank's
    linear with respect to its input. dC_r (bf16 bits) is the gradient of the
    rank's output: [M x shard_n] in shard column order for the column kinds
    ([dG | dU] for gate/up), the full [M x N] output gradient for the row kinds."""
    return matmul_f64(bf16_to_f64(dC), _shard_weight_f64(W, p).T)


def grad_weight(A: np.ndarray, dC: np.ndarray, p: dict) -> np.ndarray:
    """dW_r = A_r^T dC_r, fp64 [shard_k x shard_n]: A_r (bf16 bits) is the
    rank's input (X for the column kinds, its own Z_r for the row kinds)."""
    return matmul_f64(bf16_to_f64(A).T, bf16_to_f64(dC))


def gateup_preact(X: np.ndarray, Wgu: np.ndarray, p: dict):
    """(G, U) in fp64: the gate/up products of rank p before SwiGLU."""
    assert p["kind"] == "gateup_col"
    half = p["shard_n"] // 2
    return (shard_matmul(X, Wgu, p["rows"], p["cols"][:half]),
            shard_matmul(X, Wgu, p["rows"], p["cols"][half:]))


def swiglu_backward_f64(G: np.ndarray, U: np.ndarray, dH: np.ndarray):
    """(dG, dU) of H = SiLU(G) U, SiLU(g) = g s, s = 1 / (1 + e^-g):
    dSiLU/dg = s (1 + g (1 - s)), so dG = dH U s (1 + g (1 - s)) and
    dU = dH g s, in fp64."""
    G, U, dH = (np.asarray(a, dtype=np.float64) for a in (G, U, dH))
    with np.errstate(over="ignore"):
        s = 1.0 / (1.0 + np.exp(-G))
    return dH * U * s * (1.0 + G * (1.0 - s)), dH * G * s


def swiglu_backward(G: np.ndarray, U: np.ndarray, dH: np.ndarray) -> np.ndarray:
    """bf16 bits of [dG | dU] [M x 2w], each rounded once from fp64: the
    gradient the gate/up weight and input gradients consume."""
    dG, dU = swiglu_backward_f64(G, U, dH)
    return round_bf16(np.concatenate([dG, dU], axis=1))


# --------------------------------------------------------------------------
# The rank share, step by step.
# --------------------------------------------------------------------------

def col_linear(X: np.ndarray, W: np.ndarray, p: dict) -> np.ndarray:
    """Column-parallel product of rank p["rank"], fp64 [M x shard_n], unrounded."""
    assert p["kind"] in ("col", "qkv_col")
    return shard_matmul(X, W, p["rows"], p["cols"])


def col_linear_bf16(X: np.ndarray, W: np.ndarray, p: dict) -> np.ndarray:
    """The column output as its bf16 consumer sees it."""
    return round_bf16(col_linear(X, W, p))


def gateup_swiglu(X: np.ndarray, Wgu: np.ndarray, p: dict) -> np.ndarray:
    """H_r = bf16(SiLU(X Wg[:, I_r]) * (X Wu[:, I_r])) for the fused [Wg | Wu]."""
    assert p["kind"] == "gateup_col"
    half = p["shard_n"] // 2
    G = shard_matmul(X, Wgu, p["rows"], p["cols"][:half])
    U = shard_matmul(X, Wgu, p["rows"], p["cols"][half:])
    return swiglu(G, U)


def row_linear(Z: np.ndarray, W: np.ndarray, p: dict) -> np.ndarray:
    """Row-parallel partial P_r = Z_r W[rows_r, :], fp64 [M x N]. ``Z`` is the
    rank's own input slice [M x shard_k]."""
    assert p["kind"] in ("row", "o_row")
    return shard_matmul(Z, W, p["rows"], p["cols"])


def ffn_shard(X: np.ndarray, Wgu: np.ndarray, Wd: np.ndarray, p_gu: dict, p_d: dict):
    """One rank's feed-forward share: (H_r bf16 bits, P_r fp64)."""
    H = gateup_swiglu(X, Wgu, p_gu)
    return H, row_linear(H, Wd, p_d)


def ffn_unsharded(X: np.ndarray, Wgu: np.ndarray, Wd: np.ndarray) -> np.ndarray:
    """The layer the shards must add up to: t = 1."""
    K, N2 = Wgu.shape
    p_gu = plan("gateup_col", K, N2, 1, 0)
    p_d = plan("row", Wd.shape[0], Wd.shape[1], 1, 0)
    return ffn_shard(X, Wgu, Wd, p_gu, p_d)[1]


def compare(got: np.ndarray, ref: np.ndarray) -> dict:
    """The parity bar's two measures of ``got`` against ``ref`` (same shape):
    rel_fro = ||got - ref||_F / ||ref||_F (||got - ref||_F when ref is all
    zero), max_err = max |got - ref|, max_ref = max |ref| and max_rel =
    max_err / max_ref. A shape mismatch is an error, not a broadcast."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if got.shape != ref.shape:  # never let broadcasting stand in for a missing row
        raise ValueError(f"compare: shapes differ, got {got.shape} and ref {ref.shape}")
    diff = got - ref
    nref = np.linalg.norm(ref)
    amax = float(np.abs(ref).max()) if ref.size else 0.0
    return dict(
        rel_fro=float(np.linalg.norm(diff) / nref) if nref > 0 else float(np.linalg.norm(diff)),
        max_err=float(np.abs(diff).max()) if diff.size else 0.0,
        max_ref=amax,
        max_rel=float(np.abs(diff).max() / amax) if amax > 0 else float(np.abs(diff).max() if diff.size else 0.0),
    )


# --------------------------------------------------------------------------
# Attention core on the rank's heads, with the rank's share of the KV cache
# ("Tensor vs Pipeline Parallelism", "Tensor parallelism: split inside each
# layer": the heads are shared out over the ranks and a rank keeps the KV
# cache of its own heads; "AI Infrastructure series, Part 5", "How does
# tensor parallelism split a layer?": a rank's KV cache is 1/N of the whole,
# and ranks beyond the 8 key-value heads hold copies of a key-value head,
# spending KV memory twice; "How do you choose a layout for serving?": Llama
# 3.1 70B in 16-bit needs 320 KB of KV cache per token).
#
# A batch is S sequences with q_len new tokens each: rows s q_len .. s q_len
# + q_len - 1 of QKV [M x shard_n] (the rank's [Q_r | K_r | V_r]) belong to
# sequence s, whose cache (slot slot[s]) holds kv_len[s] positions once the
# new tokens are in; new token i sits at position kv_len[s] - q_len + i.
# Cache arrays are [n_slots x n_kv_r x L_max x d] bf16 bits, K and V apart.
# --------------------------------------------------------------------------

def _attn_heads(p: dict):
    """(n_q_r, n_kv_r, d, local kv head of each local query head)."""
    assert p["kind"] == "qkv_col"
    n_q, n_kv, d = p["heads"]
    q0, q1 = p["q_heads"]
    k0, k1 = p["kv_heads"]
    group = n_q // n_kv
    kv_of = [(q0 + h) // group - k0 for h in range(q1 - q0)]
    return q1 - q0, k1 - k0, d, kv_of


def kv_cache_new(p: dict, n_slots: int, L_max: int):
    """Empty (zero) K and V cache arrays of a rank."""
    _, nkv, d, _ = _attn_heads(p)
    shape = (n_slots, nkv, L_max, d)
    return np.zeros(shape, dtype=np.uint16), np.zeros(shape, dtype=np.uint16)


def kv_append(QKV: np.ndarray, p: dict, q_len: int, kv_len, slot, Kc: np.ndarray, Vc: np.ndarray):
    """Write the new tokens' K and V (bf16 bits, copied) into their slots."""
    nq, nkv, d, _ = _attn_heads(p)
    for s in range(len(kv_len)):
        for i in range(q_len):
            row, pos = s * q_len + i, kv_len[s] - q_len + i
            for g in range(nkv):
                Kc[slot[s], g, pos] = QKV[row, (nq + g) * d:(nq + g + 1) * d]
                Vc[slot[s], g, pos] = QKV[row, (nq + nkv + g) * d:(nq + nkv + g + 1) * d]


def attention_f64(QKV: np.ndarray, p: dict, q_len: int, kv_len, slot, Kc: np.ndarray, Vc: np.ndarray,
                  rows=None) -> np.ndarray:
    """The rank's attention output in fp64, [M x n_q_r d] (or only ``rows``),
    from the queries in QKV and the keys and values in the cache."""
    nq, _, d, kv_of = _attn_heads(p)
    S = len(kv_len)
    want = range(S * q_len) if rows is None else rows
    out = np.zeros((len(want), nq * d))
    for o, row in enumerate(want):
        s, i = divmod(row, q_len)
        pos = kv_len[s] - q_len + i
        for h in range(nq):
            q = bf16_to_f64(QKV[row, h * d:(h + 1) * d])
            K = bf16_to_f64(Kc[slot[s], kv_of[h], :pos + 1])
            V = bf16_to_f64(Vc[slot[s], kv_of[h], :pos + 1])
            sc = matmul_f64(K, q[:, None])[:, 0] / np.sqrt(d)
            w = np.exp(sc - sc.max())
            total = matmul_f64(w[None, :], np.ones((len(w), 1)))[0, 0]
            out[o, h * d:(h + 1) * d] = matmul_f64(w[None, :], V)[0] / total
    return out


def attention(QKV: np.ndarray, p: dict, q_len: int, kv_len, slot, Kc: np.ndarray, Vc: np.ndarray,
              rows=None) -> np.ndarray:
    """bf16 bits of the rank's attention output, rounded once from fp64."""
    return round_bf16(attention_f64(QKV, p, q_len, kv_len, slot, Kc, Vc, rows))


def kv_bytes_per_token(p: dict, layers: int) -> int:
    """KV cache bytes a rank keeps per token over ``layers`` layers (bf16 K
    and V of its key-value heads)."""
    _, nkv, d, _ = _attn_heads(p)
    return 2 * nkv * d * 2 * layers
