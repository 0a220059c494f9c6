"""One tensor-parallel rank's linear share of a Megatron-style transformer
layer, on one MI355X (gfx950) GPU.

Thin Python binding over the C ABI of ``include/tp_shard.h``: the functions
below have the same names and only marshal arguments (torch tensors ->
device pointers, the current HIP stream). Every step runs in the library's
HIP kernels; torch supplies device memory and streams. Output tensors are
allocated with torch when the caller does not pass them.

The method ("Tensor vs Pipeline Parallelism" (xingyuzhitong.com), "Tensor
parallelism: split inside each layer"): a block's leading matrix is cut by
output columns, its trailing one by input rows, and the row shards' partial
products are added.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import (  # noqa: F401
    KIND_NAMES, TP_COL, TP_DGRAD, TP_GATEUP_COL, TP_O_ROW, TP_PATH_AUTO, TP_PATH_DECODE, TP_PATH_PREFILL,
    TP_W_BF16, TP_W_FP8_E4M3,
    TP_QKV_COL, TP_ROW, TpHeads, TpShardDesc,
)

__all__ = ["tp_shard_plan", "tp_shard_set_wformat", "tp_shard_pack", "tp_col_linear", "tp_row_linear", "tp_ffn_shard",
           "tp_reduce_partials", "tp_reduce_scatter_partials", "tp_gather_rows", "tp_shard_plan_dgrad",
           "tp_weight_grad", "tp_swiglu_backward", "tp_kv_cache_bytes", "tp_kv_cache_new", "tp_kv_append",
           "tp_attention", "tp_attention_workspace_bytes", "tp_workspace_bytes", "tp_status_str", "TpError",
           "TpShardDesc"]


class TpError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {tp_status_str(status)} ({status})")
        self.status = status


def tp_status_str(status: int) -> str:
    return _lib.load().tp_status_str(status).decode()


def _check(status: int, where: str):
    if status != _lib.TP_OK:
        raise TpError(status, where)


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _mat(x: torch.Tensor, dtype, name: str):
    """(pointer, leading dim) of a 2-D row-major device tensor."""
    if not isinstance(x, torch.Tensor) or not x.is_cuda:
        raise TypeError(f"{name} must be a CUDA/HIP tensor")
    if x.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {x.dtype}")
    if x.dim() != 2 or (x.numel() > 0 and x.size(1) > 1 and x.stride(1) != 1):
        raise ValueError(f"{name} must be 2-D with unit column stride")
    if x.size(0) > 1 and x.stride(0) < x.size(1):
        raise ValueError(f"{name}'s rows overlap (row stride {x.stride(0)} < {x.size(1)} columns)")
    return ctypes.c_void_p(x.data_ptr()), max(x.stride(0), x.size(1))


def _out_shape(x: torch.Tensor, rows: int, cols: int, name: str):
    """An output the kernels write: exactly [rows x cols], so that no write
    can land past the tensor (fewer rows) or in a neighbour's columns (a
    narrower column slice of a wider buffer)."""
    if not isinstance(x, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if tuple(x.shape) != (rows, cols):
        raise ValueError(f"{name} is {tuple(x.shape)}, the call writes [{rows} x {cols}]")


def tp_shard_plan(kind, K: int, N: int, t: int, rank: int, heads=None) -> TpShardDesc:
    """Plan rank ``rank`` of ``t`` for weight kind ``kind`` (name or TP_* value)."""
    k = KIND_NAMES[kind] if isinstance(kind, str) else int(kind)
    d = TpShardDesc()
    hp = None
    if heads is not None:
        hp = ctypes.pointer(TpHeads(*heads))
    _check(_lib.load().tp_shard_plan(k, K, N, t, rank, hp, ctypes.byref(d)), "tp_shard_plan")
    return d


def tp_shard_set_wformat(desc: TpShardDesc, wformat) -> TpShardDesc:
    """A copy of ``desc`` switched to ``wformat`` ("bf16", "fp8_e4m3" or a
    TP_W_* code): packed_k and packed_bytes follow the format."""
    codes = {"bf16": _lib.TP_W_BF16, "fp8_e4m3": _lib.TP_W_FP8_E4M3}
    f = codes[wformat] if isinstance(wformat, str) else int(wformat)
    d = desc.copy()
    _check(_lib.load().tp_shard_set_wformat(ctypes.byref(d), f), "tp_shard_set_wformat")
    return d


def tp_shard_pack(desc: TpShardDesc, W: torch.Tensor, out: torch.Tensor | None = None,
                  stream=None) -> torch.Tensor:
    """Pack the rank's shard of the full weight ``W`` [K x N] (bf16, device)."""
    wp, ldw = _mat(W, torch.bfloat16, "W")
    if tuple(W.shape) != (desc.K, desc.N):
        raise ValueError(f"W is {tuple(W.shape)}, plan expects {(desc.K, desc.N)}")
    if out is None:
        out = torch.empty(desc.packed_bytes, dtype=torch.uint8, device=W.device)
    if out.numel() * out.element_size() < desc.packed_bytes or not out.is_contiguous():
        raise ValueError("packed buffer too small or not contiguous")
    _check(_lib.load().tp_shard_pack(ctypes.byref(desc), wp, ldw, ctypes.c_void_p(out.data_ptr()),
                                     _stream(stream)), "tp_shard_pack")
    return out


def tp_workspace_bytes(desc: TpShardDesc, M: int) -> int:
    return int(_lib.load().tp_workspace_bytes(ctypes.byref(desc), M))


def _ws(descs, M, ws, device, stream=None):
    """Workspace pointer and size; allocated here (torch, on the device) when
    the caller passes none and the kernels need some. A workspace allocated
    here is marked as used by ``stream`` so that torch's caching allocator
    does not hand its memory out again before the queued kernels have run."""
    if ws is None:
        need = max(tp_workspace_bytes(d, M) for d in descs)
        if need == 0:
            return ctypes.c_void_p(0), 0, None
        ws = torch.empty(need, dtype=torch.uint8, device=device)
        if stream is not None:
            ws.record_stream(stream)
    return ctypes.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size(), ws


def _packed(W_packed: torch.Tensor, desc: TpShardDesc, name: str):
    """Pointer of a packed shard, after checking it holds the plan's bytes."""
    if not isinstance(W_packed, torch.Tensor) or not W_packed.is_cuda or not W_packed.is_contiguous():
        raise TypeError(f"{name} must be a contiguous CUDA/HIP tensor")
    if W_packed.numel() * W_packed.element_size() < desc.packed_bytes:
        raise ValueError(f"{name} holds {W_packed.numel() * W_packed.element_size()} bytes, "
                         f"the plan packs {desc.packed_bytes}")
    return ctypes.c_void_p(W_packed.data_ptr())


def tp_col_linear(desc: TpShardDesc, X: torch.Tensor, W_packed: torch.Tensor,
                  Y: torch.Tensor | None = None, ws: torch.Tensor | None = None,
                  stream=None) -> torch.Tensor:
    """Column-parallel linear: Y [M x out_n] bf16 (SwiGLU output for gate/up)."""
    xp, ldx = _mat(X, torch.bfloat16, "X")
    M = X.size(0)
    if X.size(1) != desc.shard_k:
        raise ValueError(f"X has {X.size(1)} columns, shard expects {desc.shard_k}")
    if Y is None:
        Y = torch.empty((M, desc.out_n), dtype=torch.bfloat16, device=X.device)
    _out_shape(Y, M, desc.out_n, "Y")
    yp, ldy = _mat(Y, torch.bfloat16, "Y")
    wsp, wsb, _keep = _ws((desc,), M, ws, X.device, stream)
    _check(_lib.load().tp_col_linear(ctypes.byref(desc), xp, M, ldx,
                                     _packed(W_packed, desc, "W_packed"), yp, ldy, wsp, wsb,
                                     _stream(stream)), "tp_col_linear")
    return Y


def tp_row_linear(desc: TpShardDesc, Z: torch.Tensor, W_packed: torch.Tensor,
                  P: torch.Tensor | None = None, ws: torch.Tensor | None = None,
                  stream=None) -> torch.Tensor:
    """Row-parallel linear: the fp32 partial P [M x out_n] of this rank (out_n
    = N for the row kinds, the forward shard's input width for TP_DGRAD)."""
    zp, ldz = _mat(Z, torch.bfloat16, "Z")
    M = Z.size(0)
    if Z.size(1) != desc.shard_k:
        raise ValueError(f"Z has {Z.size(1)} columns, shard expects {desc.shard_k}")
    if P is None:
        P = torch.empty((M, desc.out_n), dtype=torch.float32, device=Z.device)
    _out_shape(P, M, desc.out_n, "P")
    pp, ldp = _mat(P, torch.float32, "P")
    wsp, wsb, _keep = _ws((desc,), M, ws, Z.device, stream)
    _check(_lib.load().tp_row_linear(ctypes.byref(desc), zp, M, ldz,
                                     _packed(W_packed, desc, "W_packed"), pp, ldp, wsp, wsb,
                                     _stream(stream)), "tp_row_linear")
    return P


def tp_ffn_shard(gateup: TpShardDesc, down: TpShardDesc, X: torch.Tensor, Wgu_packed: torch.Tensor,
                 Wd_packed: torch.Tensor, H: torch.Tensor | None = None,
                 P: torch.Tensor | None = None, ws: torch.Tensor | None = None, stream=None):
    """One rank's feed-forward share; returns (H [M x I/t] bf16, P [M x hidden] fp32)."""
    xp, ldx = _mat(X, torch.bfloat16, "X")
    M = X.size(0)
    if H is None:
        H = torch.empty((M, gateup.out_n), dtype=torch.bfloat16, device=X.device)
    if not H.is_contiguous() or tuple(H.shape) != (M, gateup.out_n) or H.dtype != torch.bfloat16:
        raise ValueError("H must be a contiguous bf16 [M x I/t] tensor")
    if P is None:
        P = torch.empty((M, down.N), dtype=torch.float32, device=X.device)
    _out_shape(P, M, down.N, "P")
    pp, ldp = _mat(P, torch.float32, "P")
    wsp, wsb, _keep = _ws((gateup, down), M, ws, X.device, stream)
    _check(_lib.load().tp_ffn_shard(ctypes.byref(gateup), ctypes.byref(down), xp, M, ldx,
                                    _packed(Wgu_packed, gateup, "Wgu_packed"),
                                    _packed(Wd_packed, down, "Wd_packed"),
                                    ctypes.c_void_p(H.data_ptr()), pp, ldp, wsp, wsb,
                                    _stream(stream)), "tp_ffn_shard")
    return H, P


def tp_reduce_partials(P: torch.Tensor, Y: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Y = P[0] + P[1] + ... + P[t-1] (fp32, rank order). ``P`` is [t x M x N]
    with unit column stride; ``Y`` may be ``P[0]``."""
    if P.dim() != 3 or P.dtype != torch.float32 or not P.is_cuda or P.stride(2) != 1:
        raise ValueError("P must be a [t x M x N] fp32 device tensor with unit column stride")
    t, M, N = P.shape
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float32, device=P.device)
    _out_shape(Y, M, N, "Y")
    yp, ldy = _mat(Y, torch.float32, "Y")
    _check(_lib.load().tp_reduce_partials(ctypes.c_void_p(P.data_ptr()), P.stride(0), t, M, N,
                                          max(P.stride(1), N), yp, ldy, _stream(stream)),
           "tp_reduce_partials")
    return Y


def tp_reduce_scatter_partials(P: torch.Tensor, rank: int, Y: torch.Tensor | None = None,
                               stream=None) -> torch.Tensor:
    """Rank ``rank``'s token rows of P[0] + ... + P[t-1] (fp32, rank order):
    [M/t x N]. ``P`` is [t x M x N] with unit column stride."""
    if P.dim() != 3 or P.dtype != torch.float32 or not P.is_cuda or P.stride(2) != 1:
        raise ValueError("P must be a [t x M x N] fp32 device tensor with unit column stride")
    t, M, N = P.shape
    if Y is None:
        Y = torch.empty((M // t if t else 0, N), dtype=torch.float32, device=P.device)
    _out_shape(Y, M // t if t else 0, N, "Y")
    yp, ldy = _mat(Y, torch.float32, "Y")
    _check(_lib.load().tp_reduce_scatter_partials(ctypes.c_void_p(P.data_ptr()), P.stride(0), t, M, N,
                                                  max(P.stride(1), N), rank, yp, ldy, _stream(stream)),
           "tp_reduce_scatter_partials")
    return Y


def tp_gather_rows(Xs: torch.Tensor, X: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """The t ranks' bf16 row blocks ``Xs`` [t x Mt x N] stacked in rank order:
    [t Mt x N]."""
    if Xs.dim() != 3 or Xs.dtype != torch.bfloat16 or not Xs.is_cuda or Xs.stride(2) != 1:
        raise ValueError("Xs must be a [t x Mt x N] bf16 device tensor with unit column stride")
    t, Mt, N = Xs.shape
    if X is None:
        X = torch.empty((t * Mt, N), dtype=torch.bfloat16, device=Xs.device)
    _out_shape(X, t * Mt, N, "X")
    xp, ldx = _mat(X, torch.bfloat16, "X")
    _check(_lib.load().tp_gather_rows(ctypes.c_void_p(Xs.data_ptr()), Xs.stride(0), t, Mt, N,
                                      max(Xs.stride(1), N), xp, ldx, _stream(stream)),
           "tp_gather_rows")
    return X


def tp_shard_plan_dgrad(fwd: TpShardDesc) -> TpShardDesc:
    """The TP_DGRAD plan of ``fwd``'s transposed shard: packed with
    tp_shard_pack from the same full W, it turns tp_row_linear into the input
    gradient dA_r [M x fwd.shard_k] = dC_r W_r^T (fp32)."""
    d = TpShardDesc()
    _check(_lib.load().tp_shard_plan_dgrad(ctypes.byref(fwd), ctypes.byref(d)), "tp_shard_plan_dgrad")
    return d


def tp_weight_grad(fwd: TpShardDesc, A: torch.Tensor, dC: torch.Tensor, dW: torch.Tensor | None = None,
                   stream=None) -> torch.Tensor:
    """dW [fwd.shard_k x fwd.shard_n] fp32 = A^T dC, A [M x fwd.shard_k] and
    dC [M x fwd.shard_n] bf16."""
    ap, lda = _mat(A, torch.bfloat16, "A")
    cp, ldc = _mat(dC, torch.bfloat16, "dC")
    if A.size(0) != dC.size(0):
        raise ValueError(f"A has {A.size(0)} rows, dC {dC.size(0)}")
    if A.size(1) != fwd.shard_k or dC.size(1) != fwd.shard_n:
        raise ValueError(f"A, dC are {tuple(A.shape)}, {tuple(dC.shape)}; the shard is "
                         f"{fwd.shard_k} x {fwd.shard_n}")
    if dW is None:
        dW = torch.empty((fwd.shard_k, fwd.shard_n), dtype=torch.float32, device=A.device)
    wp, ldw = _mat(dW, torch.float32, "dW")
    if tuple(dW.shape) != (fwd.shard_k, fwd.shard_n):
        raise ValueError(f"dW is {tuple(dW.shape)}, expected {(fwd.shard_k, fwd.shard_n)}")
    _check(_lib.load().tp_weight_grad(ctypes.byref(fwd), ap, lda, cp, ldc, A.size(0), wp, ldw,
                                      _stream(stream)), "tp_weight_grad")
    return dW


def tp_swiglu_backward(GU: torch.Tensor, dH: torch.Tensor, dGU: torch.Tensor | None = None,
                       stream=None) -> torch.Tensor:
    """[dG | dU] bf16 [M x 2w] from the pre-activations GU = [G | U] bf16
    [M x 2w] and dH fp32 [M x w]."""
    gp, ldg = _mat(GU, torch.bfloat16, "GU")
    hp, ldh = _mat(dH, torch.float32, "dH")
    M, w = dH.shape
    if tuple(GU.shape) != (M, 2 * w):
        raise ValueError(f"GU is {tuple(GU.shape)}, dH {tuple(dH.shape)}")
    if dGU is None:
        dGU = torch.empty((M, 2 * w), dtype=torch.bfloat16, device=GU.device)
    op, ldo = _mat(dGU, torch.bfloat16, "dGU")
    if tuple(dGU.shape) != (M, 2 * w):
        raise ValueError(f"dGU is {tuple(dGU.shape)}, expected {(M, 2 * w)}")
    _check(_lib.load().tp_swiglu_backward(gp, ldg, hp, ldh, M, w, op, ldo, _stream(stream)),
           "tp_swiglu_backward")
    return dGU


def _heads(qkv: TpShardDesc):
    nq = qkv.q_head_end - qkv.q_head_begin
    nkv = qkv.kv_head_end - qkv.kv_head_begin
    return nq, nkv, qkv.shard_n // (nq + 2 * nkv) if nq + 2 * nkv else 0


def tp_kv_cache_bytes(qkv: TpShardDesc, n_slots: int, L_max: int) -> int:
    return int(_lib.load().tp_kv_cache_bytes(ctypes.byref(qkv), n_slots, L_max))


def tp_kv_cache_new(qkv: TpShardDesc, n_slots: int, L_max: int, device="cuda"):
    """Zeroed K and V caches of the rank: [n_slots x n_kv_r x L_max x d] bf16."""
    if tp_kv_cache_bytes(qkv, n_slots, L_max) == 0:
        raise ValueError("invalid descriptor or cache sizes")
    _, nkv, d = _heads(qkv)
    shape = (n_slots, nkv, L_max, d)
    return (torch.zeros(shape, dtype=torch.bfloat16, device=device),
            torch.zeros(shape, dtype=torch.bfloat16, device=device))


def _seq(kv_len: torch.Tensor, slot: torch.Tensor):
    for name, t in (("kv_len", kv_len), ("slot", slot)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != torch.int32 or not t.is_contiguous():
            raise TypeError(f"{name} must be a contiguous int32 device tensor")
    if kv_len.numel() != slot.numel():
        raise ValueError("kv_len and slot differ in length")
    return kv_len.numel(), ctypes.c_void_p(kv_len.data_ptr()), ctypes.c_void_p(slot.data_ptr())


def _cache(Kc: torch.Tensor, Vc: torch.Tensor):
    for name, t in (("Kc", Kc), ("Vc", Vc)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != torch.bfloat16 or not t.is_contiguous() \
                or t.dim() != 4:
            raise TypeError(f"{name} must be a contiguous 4-D bf16 device tensor")
    if Kc.shape != Vc.shape:
        raise ValueError("K and V caches differ in shape")
    return Kc.size(0), Kc.size(2)


def tp_kv_append(qkv: TpShardDesc, QKV: torch.Tensor, q_len: int, kv_len: torch.Tensor, slot: torch.Tensor,
                 Kc: torch.Tensor, Vc: torch.Tensor, stream=None):
    """Write the new tokens' K and V rows into their cache slots."""
    qp, ldq = _mat(QKV, torch.bfloat16, "QKV")
    S, kp, sp = _seq(kv_len, slot)
    n_slots, L_max = _cache(Kc, Vc)
    if QKV.size(0) != S * q_len:
        raise ValueError(f"QKV has {QKV.size(0)} rows, {S} sequences x {q_len} tokens expected")
    _check(_lib.load().tp_kv_append(ctypes.byref(qkv), qp, ldq, S, q_len, kp, sp, ctypes.c_void_p(Kc.data_ptr()),
                                    ctypes.c_void_p(Vc.data_ptr()), n_slots, L_max, _stream(stream)),
           "tp_kv_append")


def tp_attention_workspace_bytes(qkv: TpShardDesc, S: int, q_len: int, max_kv: int) -> int:
    return int(_lib.load().tp_attention_workspace_bytes(ctypes.byref(qkv), S, q_len, max_kv))


def tp_attention(qkv: TpShardDesc, QKV: torch.Tensor, q_len: int, kv_len: torch.Tensor, slot: torch.Tensor,
                 Kc: torch.Tensor, Vc: torch.Tensor, max_kv: int, A: torch.Tensor | None = None,
                 ws: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """The rank's attention output A [S q_len x n_q_r d] bf16 over the caches
    (the new tokens already appended)."""
    qp, ldq = _mat(QKV, torch.bfloat16, "QKV")
    S, kp, sp = _seq(kv_len, slot)
    n_slots, L_max = _cache(Kc, Vc)
    nq, _, d = _heads(qkv)
    if QKV.size(0) != S * q_len:
        raise ValueError(f"QKV has {QKV.size(0)} rows, {S} sequences x {q_len} tokens expected")
    if A is None:
        A = torch.empty((S * q_len, nq * d), dtype=torch.bfloat16, device=QKV.device)
    _out_shape(A, S * q_len, nq * d, "A")
    ap, lda = _mat(A, torch.bfloat16, "A")
    if ws is None:
        need = tp_attention_workspace_bytes(qkv, S, q_len, max_kv)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=QKV.device) if need else None
        if ws is not None and stream is not None:
            ws.record_stream(stream)
    wsp = ctypes.c_void_p(ws.data_ptr()) if ws is not None else ctypes.c_void_p(0)
    wsb = ws.numel() * ws.element_size() if ws is not None else 0
    _check(_lib.load().tp_attention(ctypes.byref(qkv), qp, ldq, S, q_len, kp, sp, max_kv,
                                    ctypes.c_void_p(Kc.data_ptr()), ctypes.c_void_p(Vc.data_ptr()), n_slots, L_max,
                                    ap, lda, wsp, wsb, _stream(stream)), "tp_attention")
    return A
