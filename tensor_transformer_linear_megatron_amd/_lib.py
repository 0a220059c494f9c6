"""ctypes view of ``libtpshard.so`` and of the structs in ``include/tp_shard.h``.

The library must already be built (``__graft_entry__.build()`` or
``python -m tensor_transformer_linear_megatron_amd.build``); there is no
fallback of any kind when it is missing.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  -- load torch's HIP runtime first; the library binds to it

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtpshard.so")

TP_OK = 0
TP_ERR_NULL = -1
TP_ERR_SHAPE = -2
TP_ERR_INDIVISIBLE = -3
TP_ERR_RANK = -4
TP_ERR_ALIGN = -5
TP_ERR_WORKSPACE = -6
TP_ERR_HIP = -7
TP_ERR_KIND = -8
TP_W_BF16, TP_W_FP8_E4M3 = 0, 1

TP_COL, TP_ROW, TP_GATEUP_COL, TP_QKV_COL, TP_O_ROW, TP_DGRAD = range(6)
TP_PATH_AUTO, TP_PATH_DECODE, TP_PATH_PREFILL = range(3)

KIND_NAMES = {"col": TP_COL, "row": TP_ROW, "gateup_col": TP_GATEUP_COL,
              "qkv_col": TP_QKV_COL, "o_row": TP_O_ROW}

EXPORTS = ("tp_shard_plan", "tp_shard_set_wformat", "tp_shard_pack", "tp_col_linear", "tp_row_linear", "tp_ffn_shard",
           "tp_reduce_partials", "tp_reduce_scatter_partials", "tp_gather_rows", "tp_shard_plan_dgrad",
           "tp_weight_grad", "tp_swiglu_backward", "tp_kv_cache_bytes", "tp_kv_append", "tp_attention",
           "tp_attention_workspace_bytes", "tp_workspace_bytes", "tp_status_str", "tp_ffn_shard_noalloc")
NOALLOC_SCRATCH_BYTES = 16 << 20  # TP_NOALLOC_SCRATCH_BYTES


class TpHeads(ctypes.Structure):
    _fields_ = [("n_q", ctypes.c_int32), ("n_kv", ctypes.c_int32), ("head_dim", ctypes.c_int32)]


class TpColRange(ctypes.Structure):
    _fields_ = [("src_col", ctypes.c_int64), ("len", ctypes.c_int64), ("dst_col", ctypes.c_int64)]


class TpShardDesc(ctypes.Structure):
    _fields_ = [
        ("kind", ctypes.c_int32), ("t", ctypes.c_int32), ("rank", ctypes.c_int32),
        ("n_col_ranges", ctypes.c_int32),
        ("K", ctypes.c_int64), ("N", ctypes.c_int64),
        ("shard_k", ctypes.c_int64), ("shard_n", ctypes.c_int64),
        ("row_begin", ctypes.c_int64), ("row_end", ctypes.c_int64),
        ("col_ranges", TpColRange * 3),
        ("q_head_begin", ctypes.c_int32), ("q_head_end", ctypes.c_int32),
        ("kv_head_begin", ctypes.c_int32), ("kv_head_end", ctypes.c_int32),
        ("kv_replicated", ctypes.c_int32), ("path", ctypes.c_int32),
        ("out_n", ctypes.c_int64),
        ("packed_k", ctypes.c_int64), ("packed_n", ctypes.c_int64),
        ("packed_bytes", ctypes.c_int64),
        ("wformat", ctypes.c_int32), ("reserved", ctypes.c_int32),
    ]

    def copy(self) -> "TpShardDesc":
        d = TpShardDesc()
        ctypes.pointer(d)[0] = self
        return d

    def __repr__(self):
        rng = [(self.col_ranges[i].src_col, self.col_ranges[i].len, self.col_ranges[i].dst_col)
               for i in range(self.n_col_ranges)]
        return (f"TpShardDesc(kind={self.kind}, t={self.t}, rank={self.rank}, K={self.K}, N={self.N}, "
                f"shard=[{self.shard_k}x{self.shard_n}], rows=[{self.row_begin},{self.row_end}), "
                f"cols={rng}, out_n={self.out_n}, packed=[{self.packed_k}x{self.packed_n}])")


_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built; run __graft_entry__.build() "
            "(python -m tensor_transformer_linear_megatron_amd.build)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    D = ctypes.POINTER(TpShardDesc)
    lib.tp_shard_plan.argtypes = [ctypes.c_int, I64, I64, I32, I32, ctypes.POINTER(TpHeads), D]
    lib.tp_shard_set_wformat.argtypes = [D, I32]
    lib.tp_shard_pack.argtypes = [D, P, I64, P, P]
    lib.tp_col_linear.argtypes = [D, P, I64, I64, P, P, I64, P, SZ, P]
    lib.tp_row_linear.argtypes = [D, P, I64, I64, P, P, I64, P, SZ, P]
    lib.tp_ffn_shard.argtypes = [D, D, P, I64, I64, P, P, P, P, I64, P, SZ, P]
    lib.tp_ffn_shard_noalloc.argtypes = [D, D, P, I64, I64, P, P, P, P, I64, P]
    lib.tp_reduce_partials.argtypes = [P, I64, I32, I64, I64, I64, P, I64, P]
    lib.tp_reduce_scatter_partials.argtypes = [P, I64, I32, I64, I64, I64, I32, P, I64, P]
    lib.tp_gather_rows.argtypes = [P, I64, I32, I64, I64, I64, P, I64, P]
    lib.tp_shard_plan_dgrad.argtypes = [D, D]
    lib.tp_weight_grad.argtypes = [D, P, I64, P, I64, I64, P, I64, P]
    lib.tp_swiglu_backward.argtypes = [P, I64, P, I64, I64, I64, P, I64, P]
    lib.tp_kv_cache_bytes.argtypes = [D, I64, I64]
    lib.tp_kv_cache_bytes.restype = SZ
    lib.tp_kv_append.argtypes = [D, P, I64, I32, I32, P, P, P, P, I64, I64, P]
    lib.tp_attention.argtypes = [D, P, I64, I32, I32, P, P, I32, P, P, I64, I64, P, I64, P, SZ, P]
    lib.tp_attention_workspace_bytes.argtypes = [D, I32, I32, I32]
    lib.tp_attention_workspace_bytes.restype = SZ
    lib.tp_workspace_bytes.argtypes = [D, I64]
    lib.tp_workspace_bytes.restype = SZ
    lib.tp_status_str.argtypes = [I32]
    lib.tp_status_str.restype = ctypes.c_char_p
    for name in ("tp_shard_plan", "tp_shard_set_wformat", "tp_shard_pack", "tp_col_linear", "tp_row_linear",
                 "tp_ffn_shard", "tp_reduce_partials", "tp_reduce_scatter_partials", "tp_gather_rows",
                 "tp_shard_plan_dgrad", "tp_weight_grad", "tp_swiglu_backward", "tp_kv_append", "tp_attention",
                 "tp_ffn_shard_noalloc"):
        getattr(lib, name).restype = I32
    _lib = lib
    return lib
