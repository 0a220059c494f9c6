"""The C-ABI library on the CPU: it loads, exports what the header declares,
plans shards exactly as the oracle's independent planner does, and rejects
bad arguments with the documented codes before any GPU work."""
from __future__ import annotations

import ctypes
import itertools
import os
import re

import numpy as np
import pytest

import oracle
import tensor_transformer_linear_megatron_amd as tp
from tensor_transformer_linear_megatron_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CODES = {"indivisible": _lib.TP_ERR_INDIVISIBLE, "rank": _lib.TP_ERR_RANK,
         "shape": _lib.TP_ERR_SHAPE, "kind": _lib.TP_ERR_KIND}


def declared_functions():
    src = open(os.path.join(ROOT, "include", "tp_shard.h")).read()
    return sorted(set(re.findall(r"TP_API\s+[\w\s\*]+?\b(tp_\w+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTS), names
    lib = _lib.load()
    for n in names:
        assert hasattr(lib, n), n
    nm = os.popen(f"nm -D --defined-only {_lib.LIB_PATH}").read()
    exported = set(re.findall(r" T (tp_\w+)", nm))
    assert exported == set(names), exported ^ set(names)


def test_binding_output_shape_rule():
    """The binding's check on every output the kernels write: exactly the
    [rows x cols] the call writes (host logic, no GPU)."""
    import torch
    from tensor_transformer_linear_megatron_amd import _out_shape
    buf = torch.empty((6, 16))
    _out_shape(buf[:4, :8], 4, 8, "Y")
    for view in (buf[:3, :8], buf[:4, :4], buf[:4], buf[:5, :8], buf[:4, :8].reshape(8, 4)):
        with pytest.raises(ValueError):
            _out_shape(view, 4, 8, "Y")
    with pytest.raises(TypeError):
        _out_shape(None, 4, 8, "Y")


def test_status_strings():
    for code in range(-8, 1):
        assert tp.tp_status_str(code) not in ("", "unknown status")
    assert tp.tp_status_str(-99) == "unknown status"


def _expand(d):
    rows = np.arange(d.row_begin, d.row_end)
    cols = np.concatenate([np.arange(d.col_ranges[i].src_col, d.col_ranges[i].src_col + d.col_ranges[i].len)
                           for i in range(d.n_col_ranges)])
    dst = [d.col_ranges[i].dst_col for i in range(d.n_col_ranges)]
    lens = [d.col_ranges[i].len for i in range(d.n_col_ranges)]
    assert dst == list(np.cumsum([0] + lens[:-1]))  # ranges tile the shard in order
    return rows, cols


def _cases():
    for kind in ("col", "row", "gateup_col"):
        for K, N in ((64, 96), (4096, 4096), (8192, 57344), (128, 256)):
            for t in (1, 2, 3, 4, 8):
                for r in sorted({0, t // 2, t - 1}):
                    yield kind, K, N, t, r, None
    for (nq, nkv, d) in ((64, 8, 128), (32, 8, 64), (16, 4, 8), (8, 8, 16)):
        for t in (1, 2, 3, 4, 6, 8, 16, 32):
            for r in sorted({0, t // 2, t - 1}):
                yield "qkv_col", 512, (nq + 2 * nkv) * d, t, r, (nq, nkv, d)
                yield "o_row", nq * d, 256, t, r, (nq, nkv, d)


@pytest.mark.parametrize("kind,K,N,t,r,heads", list(_cases()))
def test_plan_matches_oracle_planner(kind, K, N, t, r, heads):
    try:
        want = oracle.plan(kind, K, N, t, r, heads=heads)
    except oracle.PlanError as e:
        with pytest.raises(tp.TpError) as got:
            tp.tp_shard_plan(kind, K, N, t, r, heads=heads)
        assert got.value.status == CODES[e.code]
        return
    try:
        d = tp.tp_shard_plan(kind, K, N, t, r, heads=heads)
    except tp.TpError as e:  # the library may only add the 8-element alignment rule
        assert e.status == _lib.TP_ERR_ALIGN
        out_n = want["shard_n"] // 2 if kind == "gateup_col" else want["shard_n"]
        assert want["shard_k"] % 8 or out_n % 8 or (heads and heads[2] % 8)
        return
    rows, cols = _expand(d)
    np.testing.assert_array_equal(rows, want["rows"])
    np.testing.assert_array_equal(cols, want["cols"])
    assert (d.shard_k, d.shard_n, d.t, d.rank, d.K, d.N) == (want["shard_k"], want["shard_n"], t, r, K, N)
    if heads is not None:
        assert (d.q_head_begin, d.q_head_end) == want["q_heads"]
        assert (d.kv_head_begin, d.kv_head_end) == want["kv_heads"]
        assert bool(d.kv_replicated) == want["kv_replicated"]
    assert d.out_n == (d.shard_n // 2 if kind == "gateup_col" else d.shard_n)
    assert d.packed_k % 32 == 0 and d.packed_n % 32 == 0 and d.packed_k >= d.shard_k
    assert d.packed_bytes == d.packed_k * d.packed_n * 2
    assert d.path == tp.TP_PATH_AUTO


def test_plan_error_codes():
    lib = _lib.load()
    d = tp.TpShardDesc()
    assert lib.tp_shard_plan(0, 64, 64, 2, 0, None, None) == _lib.TP_ERR_NULL
    assert lib.tp_shard_plan(9, 64, 64, 2, 0, None, ctypes.byref(d)) == _lib.TP_ERR_KIND
    assert lib.tp_shard_plan(tp.TP_QKV_COL, 64, 64, 2, 0, None, ctypes.byref(d)) == _lib.TP_ERR_NULL
    assert lib.tp_shard_plan(0, 64, 64, 0, 0, None, ctypes.byref(d)) == _lib.TP_ERR_SHAPE
    assert lib.tp_shard_plan(0, 64, -8, 1, 0, None, ctypes.byref(d)) == _lib.TP_ERR_SHAPE
    assert lib.tp_shard_plan(0, 64, 64, 2, 2, None, ctypes.byref(d)) == _lib.TP_ERR_RANK
    assert lib.tp_shard_plan(0, 64, 96, 64, 0, None, ctypes.byref(d)) == _lib.TP_ERR_INDIVISIBLE
    assert lib.tp_shard_plan(0, 64, 48, 8, 0, None, ctypes.byref(d)) == _lib.TP_ERR_ALIGN  # 6 columns
    assert lib.tp_shard_plan(0, 60, 64, 1, 0, None, ctypes.byref(d)) == _lib.TP_ERR_ALIGN  # K % 8
    h = _lib.TpHeads(64, 8, 128)
    for t in (3, 5, 6, 7):
        assert lib.tp_shard_plan(tp.TP_QKV_COL, 8192, 10240, t, 0, ctypes.byref(h), ctypes.byref(d)) \
            == _lib.TP_ERR_INDIVISIBLE
    assert lib.tp_shard_plan(tp.TP_QKV_COL, 8192, 10000, 8, 0, ctypes.byref(h), ctypes.byref(d)) \
        == _lib.TP_ERR_SHAPE


def test_worked_tp2_split_through_the_abi(golden):
    g = golden("tp2_worked_split.json")
    for r in range(2):
        d = tp.tp_shard_plan("col", 4096, 4096, 2, r)
        assert [d.shard_k, d.shard_n] == g["column_shards"][r]
        assert d.packed_bytes == 4096 * 2048 * 2
        e = tp.tp_shard_plan("row", 4096, 4096, 2, r)
        assert [e.shard_k, e.shard_n] == g["row_shards"][r]


# Fake, 16-byte aligned host addresses: every call below is rejected on the
# host before anything is queued, so they are never dereferenced.
A = ctypes.c_void_p(0x100000)
B = ctypes.c_void_p(0x200000)
C = ctypes.c_void_p(0x300000)
MIS = ctypes.c_void_p(0x100008)
NUL = ctypes.c_void_p(0)


def test_linear_argument_errors():
    lib = _lib.load()
    col = tp.tp_shard_plan("col", 64, 64, 2, 0)
    row = tp.tp_shard_plan("row", 64, 64, 2, 0)
    gu = tp.tp_shard_plan("gateup_col", 64, 128, 2, 0)
    dn = tp.tp_shard_plan("row", 64, 64, 2, 0)
    cb, rb = ctypes.byref(col), ctypes.byref(row)
    S = ctypes.c_void_p(0)
    assert lib.tp_col_linear(None, A, 4, 64, B, C, 32, NUL, 0, S) == _lib.TP_ERR_NULL
    assert lib.tp_col_linear(cb, NUL, 4, 64, B, C, 32, NUL, 0, S) == _lib.TP_ERR_NULL
    assert lib.tp_col_linear(cb, A, 4, 64, NUL, C, 32, NUL, 0, S) == _lib.TP_ERR_NULL
    assert lib.tp_col_linear(cb, A, -1, 64, B, C, 32, NUL, 0, S) == _lib.TP_ERR_SHAPE
    assert lib.tp_col_linear(cb, A, 4, 56, B, C, 32, NUL, 0, S) == _lib.TP_ERR_SHAPE   # ldx < K
    assert lib.tp_col_linear(cb, A, 4, 64, B, C, 24, NUL, 0, S) == _lib.TP_ERR_SHAPE   # ldy < out_n
    assert lib.tp_col_linear(cb, MIS, 4, 64, B, C, 32, NUL, 0, S) == _lib.TP_ERR_ALIGN
    assert lib.tp_col_linear(cb, A, 4, 68, B, C, 32, NUL, 0, S) == _lib.TP_ERR_ALIGN   # ldx % 8
    assert lib.tp_col_linear(rb, A, 4, 64, B, C, 32, NUL, 0, S) == _lib.TP_ERR_KIND
    assert lib.tp_col_linear(cb, A, 0, 64, B, C, 32, NUL, 0, S) == _lib.TP_OK          # M == 0: no-op
    assert lib.tp_col_linear(cb, NUL, 0, 64, NUL, NUL, 32, NUL, 0, S) == _lib.TP_OK
    assert lib.tp_row_linear(cb, A, 4, 32, B, C, 64, NUL, 0, S) == _lib.TP_ERR_KIND
    assert lib.tp_row_linear(rb, A, 4, 32, B, C, 62, NUL, 0, S) == _lib.TP_ERR_SHAPE  # ldp < N
    assert lib.tp_row_linear(rb, A, 4, 32, B, C, 66, NUL, 0, S) == _lib.TP_ERR_ALIGN  # ldp % 4
    assert lib.tp_row_linear(rb, A, 0, 32, B, C, 64, NUL, 0, S) == _lib.TP_OK
    forced = col.copy()
    forced.path = tp.TP_PATH_DECODE
    assert lib.tp_col_linear(ctypes.byref(forced), A, 65, 64, B, C, 32, NUL, 0, S) == _lib.TP_ERR_SHAPE
    forced.path = 7
    assert lib.tp_col_linear(ctypes.byref(forced), A, 4, 64, B, C, 32, NUL, 0, S) == _lib.TP_ERR_KIND
    broken = col.copy()
    broken.packed_bytes += 2
    assert lib.tp_col_linear(ctypes.byref(broken), A, 4, 64, B, C, 32, NUL, 0, S) == _lib.TP_ERR_SHAPE
    # the feed-forward pairing: same t and rank, I/t of gate/up == k of down
    g, d = ctypes.byref(gu), ctypes.byref(dn)
    assert lib.tp_ffn_shard(g, d, A, 0, 64, B, B, C, A, 64, NUL, 0, S) == _lib.TP_OK
    assert lib.tp_ffn_shard(d, g, A, 4, 64, B, B, C, A, 64, NUL, 0, S) == _lib.TP_ERR_KIND
    other = tp.tp_shard_plan("row", 64, 64, 2, 1)
    assert lib.tp_ffn_shard(g, ctypes.byref(other), A, 4, 64, B, B, C, A, 64, NUL, 0, S) == _lib.TP_ERR_SHAPE
    wide = tp.tp_shard_plan("row", 128, 64, 2, 0)
    assert lib.tp_ffn_shard(g, ctypes.byref(wide), A, 4, 64, B, B, C, A, 64, NUL, 0, S) == _lib.TP_ERR_SHAPE
    assert lib.tp_ffn_shard(g, d, A, 4, 64, B, B, NUL, A, 64, NUL, 0, S) == _lib.TP_ERR_NULL
    assert lib.tp_ffn_shard(g, d, A, 4, 64, B, B, C, MIS, 64, NUL, 0, S) == _lib.TP_ERR_ALIGN


def test_set_wformat_sizes_and_errors():
    """tp_shard_plan gives bf16 storage; switching to 8-bit re-plans packed_k to
    a multiple of 64 and packed_bytes to codes + 4 bytes of scale per packed
    column; switching back restores the bf16 plan; a descriptor whose sizes do
    not match its format is refused before any launch."""
    lib = _lib.load()
    S = ctypes.c_void_p(0)
    for kind, K, N, t, r in (("col", 4104, 1040, 2, 1), ("gateup_col", 8192, 57344, 8, 3), ("row", 1000, 64, 1, 0)):
        d = tp.tp_shard_plan(kind, K, N, t, r)
        assert d.wformat == tp.TP_W_BF16 and d.reserved == 0
        e = tp.tp_shard_set_wformat(d, "fp8_e4m3")
        assert e.wformat == tp.TP_W_FP8_E4M3 and e.packed_k % 64 == 0
        assert e.packed_k == -(-d.shard_k // 64) * 64 and e.packed_n == d.packed_n
        assert e.packed_bytes == e.packed_k * e.packed_n + 4 * e.packed_n
        back = tp.tp_shard_set_wformat(e, "bf16")
        assert (back.packed_k, back.packed_bytes, back.wformat) == (d.packed_k, d.packed_bytes, 0)
        assert tp.tp_workspace_bytes(e, 1) == 0  # up to 16 tokens stream, no split
        ws64 = tp.tp_workspace_bytes(e, 64)  # shared-token kernel: split-K partials or none
        assert ws64 % (64 * e.packed_n * 4) == 0 and ws64 // (64 * e.packed_n * 4) <= 64
        assert tp.tp_workspace_bytes(e, 4096) >= e.packed_k * e.packed_n * 2
    d = tp.tp_shard_plan("col", 64, 64, 1, 0)
    assert lib.tp_shard_set_wformat(ctypes.byref(d), 7) == _lib.TP_ERR_KIND
    assert lib.tp_shard_set_wformat(None, 1) == _lib.TP_ERR_NULL
    bad = d.copy()
    bad.wformat = tp.TP_W_FP8_E4M3  # sizes still those of the bf16 plan
    assert lib.tp_col_linear(ctypes.byref(bad), A, 4, 64, B, C, 64, NUL, 0, S) == _lib.TP_ERR_SHAPE
    bad.wformat = 9
    assert lib.tp_col_linear(ctypes.byref(bad), A, 4, 64, B, C, 64, NUL, 0, S) == _lib.TP_ERR_KIND


def test_sequence_parallel_argument_errors():
    """Every refusal happens on the host, before any launch."""
    lib = _lib.load()
    S = ctypes.c_void_p(0)
    rs, g = lib.tp_reduce_scatter_partials, lib.tp_gather_rows
    assert rs(A, 256, 3, 4, 64, 64, 0, B, 64, S) == _lib.TP_ERR_INDIVISIBLE  # 4 rows over 3 ranks
    assert rs(A, 256, 2, 4, 64, 64, 2, B, 64, S) == _lib.TP_ERR_RANK
    assert rs(A, 256, 2, 4, 64, 64, -1, B, 64, S) == _lib.TP_ERR_RANK
    assert rs(NUL, 256, 2, 4, 64, 64, 0, B, 64, S) == _lib.TP_ERR_NULL
    assert rs(A, 256, 0, 4, 64, 64, 0, B, 64, S) == _lib.TP_ERR_SHAPE
    assert rs(A, 255, 2, 4, 64, 64, 0, B, 64, S) == _lib.TP_ERR_SHAPE  # stride < M ld
    assert rs(A, 256, 2, 4, 62, 64, 0, B, 64, S) == _lib.TP_ERR_ALIGN  # N % 4
    assert rs(MIS, 256, 2, 4, 64, 64, 0, B, 64, S) == _lib.TP_ERR_ALIGN
    assert rs(NUL, 256, 2, 0, 64, 64, 1, NUL, 64, S) == _lib.TP_OK  # M == 0
    assert g(NUL, 256, 2, 4, 64, 64, B, 64, S) == _lib.TP_ERR_NULL
    assert g(A, 256, 0, 4, 64, 64, B, 64, S) == _lib.TP_ERR_SHAPE
    assert g(A, 255, 2, 4, 64, 64, B, 64, S) == _lib.TP_ERR_SHAPE  # stride < Mt ldb
    assert g(A, 256, 2, 4, 60, 64, B, 64, S) == _lib.TP_ERR_ALIGN  # N % 8
    assert g(A, 256, 2, 4, 64, 64, MIS, 64, S) == _lib.TP_ERR_ALIGN
    assert g(A, 256, 2, 4, 64, 32, B, 64, S) == _lib.TP_ERR_SHAPE  # ldb < N
    assert g(NUL, 256, 2, 0, 64, 64, NUL, 64, S) == _lib.TP_OK  # Mt == 0


def test_reduce_and_pack_argument_errors():
    lib = _lib.load()
    S = ctypes.c_void_p(0)
    assert lib.tp_reduce_partials(NUL, 256, 2, 4, 64, 64, A, 64, S) == _lib.TP_ERR_NULL
    assert lib.tp_reduce_partials(A, 256, 0, 4, 64, 64, B, 64, S) == _lib.TP_ERR_SHAPE
    assert lib.tp_reduce_partials(A, 255, 2, 4, 64, 64, B, 64, S) == _lib.TP_ERR_SHAPE  # stride < M ld
    assert lib.tp_reduce_partials(A, 256, 2, 4, 62, 64, B, 64, S) == _lib.TP_ERR_ALIGN  # N % 4
    assert lib.tp_reduce_partials(MIS, 256, 2, 4, 64, 64, B, 64, S) == _lib.TP_ERR_ALIGN
    assert lib.tp_reduce_partials(A, 256, 2, 0, 64, 64, B, 64, S) == _lib.TP_OK
    assert lib.tp_reduce_partials(NUL, 256, 2, 0, 64, 64, NUL, 64, S) == _lib.TP_OK
    col = tp.tp_shard_plan("col", 64, 64, 2, 0)
    assert lib.tp_shard_pack(ctypes.byref(col), NUL, 64, B, S) == _lib.TP_ERR_NULL
    assert lib.tp_shard_pack(ctypes.byref(col), A, 32, B, S) == _lib.TP_ERR_SHAPE
    assert lib.tp_shard_pack(ctypes.byref(col), A, 64, MIS, S) == _lib.TP_ERR_ALIGN
    bad = col.copy()
    bad.col_ranges[0].src_col = 60
    assert lib.tp_shard_pack(ctypes.byref(bad), A, 64, B, S) == _lib.TP_ERR_SHAPE


def _big_tiles(d, M):
    """256 x 256 output tiles of a prefill linear (16 packed tiles x 256 tokens)."""
    return -(-d.packed_n // 256) * -(-M // 256)


def test_workspace_bytes():
    """Decode batches of 17..64 tokens may split K over workgroups; the fp32
    partials need G * M * packed_n * 4 bytes. Prefill splits K when its
    256 x 256 tiles cannot fill the 256 CUs: then G >= 2 splits of at least 16
    k-steps with G * tiles <= 256. With 256 or more tiles only a last round
    of at most 128 tiles may be split (see test_prefill_tail_workspace).
    M <= 16 and invalid descriptors need none."""
    lib = _lib.load()
    for kind, K, N, t in (("col", 4096, 4096, 2), ("gateup_col", 8192, 57344, 8), ("row", 28672, 8192, 8),
                          ("row", 14336, 4096, 1), ("gateup_col", 4096, 28672, 1), ("row", 1024, 8192, 1)):
        d = tp.tp_shard_plan(kind, K, N, t, 0)
        for M in (1, 16):
            assert tp.tp_workspace_bytes(d, M) == 0
        for M in (17, 32, 64):
            ws = tp.tp_workspace_bytes(d, M)
            assert ws % (M * d.packed_n * 4) == 0 and ws // (M * d.packed_n * 4) <= 64
        pre = d.copy()
        pre.path = tp.TP_PATH_PREFILL
        for M in (32, 65, 300, 4096, 8192):
            dd = pre if M <= 64 else d
            ws = tp.tp_workspace_bytes(dd, M)
            tiles, ksteps = _big_tiles(d, M), d.packed_k // 32
            if tiles >= 256:
                left = tiles % 256
                if left == 0 or left > 128:
                    assert ws == 0, (kind, K, N, M)
                else:  # the last round's tiles, split at most 256 // left ways
                    assert ws <= (256 // left) * M * d.packed_n * 4, (kind, K, N, M)
                continue
            assert ws % (M * d.packed_n * 4) == 0
            G = ws // (M * d.packed_n * 4)
            if min(256 // tiles, ksteps // 16) < 2:
                assert G == 0, (kind, K, N, M)
            else:
                assert G >= 2 and G * tiles <= 256 and -(-ksteps // G) >= 16, (kind, K, N, M, G)
    # The 70B attention QKV slice of one TP = 8 rank at 4096 tokens: 80 tiles, K split 3 ways.
    dq = tp.tp_shard_plan("qkv_col", 8192, 10240, 8, 0, heads=(64, 8, 128))
    assert tp.tp_workspace_bytes(dq, 4096) == 3 * 4096 * dq.packed_n * 4
    assert lib.tp_workspace_bytes(None, 32) == 0
    d = tp.tp_shard_plan("row", 14336, 4096, 1, 0)
    if tp.tp_workspace_bytes(d, 64):  # a too-small workspace is refused before any launch
        assert lib.tp_row_linear(ctypes.byref(d), A, 64, 14336, B, C, 4096, NUL, 0, ctypes.c_void_p(0)) \
            == _lib.TP_ERR_WORKSPACE
        assert lib.tp_row_linear(ctypes.byref(d), A, 64, 14336, B, C, 4096, A, 16, ctypes.c_void_p(0)) \
            == _lib.TP_ERR_WORKSPACE


def test_prefill_tail_workspace():
    """A last round of at most 128 big tiles whose tiles (in the kernel's
    grouped order: 8 token tiles deep, column-major inside a group) form a
    rectangle runs as a sub-GEMM with K split 256 // tiles ways (at least 16
    k-steps each), its fp32 partials in the workspace."""
    part = 16 * 4  # bytes per packed tile column per token
    # 405B gate/up, rank 0 of 8, 8192 tokens: 52 x 32 tiles, the last 128 are
    # token tiles 24..31 x column tiles 36..51: 2 splits of 2048 x 256 tiles
    d = tp.tp_shard_plan("gateup_col", 16384, 2 * 53248, 8, 0)
    assert tp.tp_workspace_bytes(d, 8192) == 2 * 2048 * 256 * part
    # 70B gate/up, rank 0 of 8: 28 x 32 tiles, the last 128 are 8 x 16
    d = tp.tp_shard_plan("gateup_col", 8192, 57344, 8, 0)
    assert tp.tp_workspace_bytes(d, 8192) == 2 * 2048 * 256 * part
    # 17 x 16 tiles, ragged everywhere: the last 16 are token tiles 8..15 x
    # column tiles 15, 16 (packed tiles 240 .. packed_n / 16), K = 1000 in 2 splits
    d = tp.tp_shard_plan("col", 1000, 4328, 1, 0)
    assert d.packed_n // 16 == 272
    assert tp.tp_workspace_bytes(d, 4000) == 2 * (4000 - 2048) * (272 - 240) * part
    # 21 x 13 tiles: the last 17 span column tiles 17..20 and token tiles
    # 8..12 without filling them, so they run as half tiles with no workspace
    d = tp.tp_shard_plan("col", 1024, 5376, 1, 0)
    assert tp.tp_workspace_bytes(d, 3300) == 0
    # 17 x 16 tiles with 1 k-step: too short to split
    d = tp.tp_shard_plan("col", 32, 4352, 1, 0)
    assert tp.tp_workspace_bytes(d, 4096) == 0


def test_prefill_tail_workspace_random_shapes():
    """Seeded random column shards with 256 or more big tiles (256 x 256):
    the workspace is non-zero only when the last round holds 1 .. 128 tiles,
    and then it holds G >= 2 fp32 partials of a sub-GEMM no larger than
    those tiles, G times the tiles fitting in one round. (That the kernels
    write only inside it, and read nothing of it they did not write, is
    checked on the GPU with a workspace of exactly this size.)"""
    rng = np.random.default_rng(5)
    seen = {"split": 0, "none": 0}
    for _ in range(300):
        M = int(rng.integers(2049, 12000))
        N = int(rng.integers(8, 600)) * 8 * 8
        K = int(rng.integers(1, 64)) * 8 * 8
        d = tp.tp_shard_plan("col", K, N, 1, 0)
        nb = -(-M // 256) * -(-(d.packed_n // 16) // 16)
        if nb < 256:
            continue
        left = nb % 256
        ws = tp.tp_workspace_bytes(d, M)
        if left == 0 or left > 128:
            assert ws == 0, (M, K, N)
            continue
        if ws == 0:
            seen["none"] += 1
            continue
        seen["split"] += 1
        per_split = left * 256 * 256 * 4  # the last round's tiles in fp32, whole
        assert ws % (16 * 4) == 0 and 2 * 16 * 4 <= ws <= (256 // left) * per_split, (M, K, N, ws, left)
        assert -(-K // 32) >= 2 * 16, (M, K, N)  # two splits of at least 16 k-steps
    assert seen["split"] >= 5 and seen["none"] >= 5, seen


@pytest.mark.parametrize("kind,K,N,t,r,heads", [("col", 4096, 1024, 4, 1, None), ("row", 1024, 4096, 4, 3, None),
                                                 ("gateup_col", 8192, 2 * 28672, 8, 5, None),
                                                 ("qkv_col", 512, (8 + 2 * 2) * 64, 2, 1, (8, 2, 64)),
                                                 ("o_row", 8 * 64, 512, 2, 0, (8, 2, 64))])
def test_plan_dgrad_is_the_transposed_shard(kind, K, N, t, r, heads):
    """The TP_DGRAD plan swaps the shard's two sizes, keeps the rows, the column
    ranges and the rank, and plans bf16 tiles over the swapped sizes."""
    f = tp.tp_shard_plan(kind, K, N, t, r, heads=heads)
    d = tp.tp_shard_plan_dgrad(f)
    assert d.kind == tp.TP_DGRAD and d.wformat == tp.TP_W_BF16
    assert (d.shard_k, d.shard_n, d.out_n) == (f.shard_n, f.shard_k, f.shard_k)
    assert (d.K, d.N, d.t, d.rank, d.row_begin, d.row_end) == (f.K, f.N, f.t, f.rank, f.row_begin, f.row_end)
    assert d.n_col_ranges == f.n_col_ranges
    for a, b in zip(d.col_ranges[:d.n_col_ranges], f.col_ranges[:f.n_col_ranges]):
        assert (a.src_col, a.len, a.dst_col) == (b.src_col, b.len, b.dst_col)
    assert d.packed_k == -(-f.shard_n // 32) * 32 and d.packed_n == -(-f.shard_k // 32) * 32
    assert d.packed_bytes == 2 * d.packed_k * d.packed_n
    p = oracle.plan(kind, K, N, t, r, heads=heads)
    assert (d.shard_k, d.shard_n) == (len(p["cols"]), len(p["rows"]))


def test_backward_argument_errors():
    """Every refusal happens on the host, before any launch."""
    lib = _lib.load()
    S = ctypes.c_void_p(0)
    f = tp.tp_shard_plan("col", 64, 128, 2, 1)  # shard 64 x 64
    d = tp.tp_shard_plan_dgrad(f)
    fb, db = ctypes.byref(f), ctypes.byref(d)
    out = tp.TpShardDesc()
    assert lib.tp_shard_plan_dgrad(None, ctypes.byref(out)) == _lib.TP_ERR_NULL
    assert lib.tp_shard_plan_dgrad(fb, None) == _lib.TP_ERR_NULL
    assert lib.tp_shard_plan_dgrad(db, ctypes.byref(out)) == _lib.TP_ERR_KIND  # no transpose of a transpose
    assert lib.tp_shard_set_wformat(ctypes.byref(d.copy()), tp.TP_W_FP8_E4M3) == _lib.TP_ERR_KIND
    edited = d.copy()
    edited.wformat = tp.TP_W_FP8_E4M3
    edited.packed_k, edited.packed_bytes = 64, 64 * edited.packed_n + 4 * edited.packed_n
    assert lib.tp_row_linear(ctypes.byref(edited), A, 4, 64, B, C, 64, NUL, 0, S) == _lib.TP_ERR_KIND
    # the transposed plan runs on the row entry point only
    assert lib.tp_col_linear(db, A, 4, 64, B, C, 64, NUL, 0, S) == _lib.TP_ERR_KIND
    assert lib.tp_row_linear(db, A, 4, 64, B, C, 60, NUL, 0, S) == _lib.TP_ERR_SHAPE  # ldp < out_n
    # pack: W is the forward's full [K x N]
    assert lib.tp_shard_pack(db, A, 120, B, S) == _lib.TP_ERR_SHAPE
    wg = lib.tp_weight_grad
    assert wg(None, A, 64, B, 64, 4, C, 64, S) == _lib.TP_ERR_NULL
    assert wg(db, A, 64, B, 64, 4, C, 64, S) == _lib.TP_ERR_KIND
    assert wg(fb, NUL, 64, B, 64, 4, C, 64, S) == _lib.TP_ERR_NULL
    assert wg(fb, A, 64, B, 64, 4, NUL, 64, S) == _lib.TP_ERR_NULL
    assert wg(fb, A, 56, B, 64, 4, C, 64, S) == _lib.TP_ERR_SHAPE  # lda < shard_k
    assert wg(fb, A, 64, B, 56, 4, C, 64, S) == _lib.TP_ERR_SHAPE  # lddc < shard_n
    assert wg(fb, A, 64, B, 64, 4, C, 60, S) == _lib.TP_ERR_SHAPE  # lddw < shard_n
    assert wg(fb, A, 64, B, 64, -1, C, 64, S) == _lib.TP_ERR_SHAPE
    assert wg(fb, A, 68, B, 64, 4, C, 64, S) == _lib.TP_ERR_ALIGN  # lda % 8
    assert wg(fb, A, 64, B, 64, 4, C, 66, S) == _lib.TP_ERR_ALIGN  # lddw % 4
    assert wg(fb, MIS, 64, B, 64, 4, C, 64, S) == _lib.TP_ERR_ALIGN
    sb = lib.tp_swiglu_backward
    assert sb(A, 120, B, 64, 4, 64, C, 128, S) == _lib.TP_ERR_SHAPE  # ldgu < 2w
    assert sb(A, 128, B, 60, 4, 64, C, 128, S) == _lib.TP_ERR_SHAPE  # lddh < w
    assert sb(A, 128, B, 64, 4, 64, C, 120, S) == _lib.TP_ERR_SHAPE  # lddgu < 2w
    assert sb(A, 128, B, 64, -1, 64, C, 128, S) == _lib.TP_ERR_SHAPE
    assert sb(A, 128, B, 64, 4, 0, C, 128, S) == _lib.TP_ERR_SHAPE
    assert sb(NUL, 128, B, 64, 4, 64, C, 128, S) == _lib.TP_ERR_NULL
    assert sb(A, 128, B, 64, 4, 64, NUL, 128, S) == _lib.TP_ERR_NULL
    assert sb(A, 120, B, 60, 4, 60, C, 120, S) == _lib.TP_ERR_ALIGN  # w % 8
    assert sb(MIS, 128, B, 64, 4, 64, C, 128, S) == _lib.TP_ERR_ALIGN
    assert sb(A, 128, B, 66, 4, 64, C, 128, S) == _lib.TP_ERR_ALIGN  # lddh % 4
    assert sb(NUL, 128, NUL, 64, 0, 64, NUL, 128, S) == _lib.TP_OK  # M == 0


H70 = (64, 8, 128)


def _qkv70(t, r):
    return tp.tp_shard_plan("qkv_col", 8192, (64 + 16) * 128, t, r, heads=H70)


def test_kv_cache_and_attention_workspace_sizes():
    """Cache bytes: n_slots x n_kv_r x L_max x d x 2 per array; the rank's
    share is 1/t of the layer's key-value heads up to t = n_kv, then one
    repeated head. The decode form needs one partial (16 rows x (d + 2) fp32)
    per sequence, key-value head and chunk, and none when each (sequence,
    key-value head) is one chunk: chunks take 512 x 2^j positions (j <= 3),
    as long as every chunk count still gives 256 or more workgroups."""
    for t, nkv in ((1, 8), (2, 4), (8, 1), (16, 1)):
        assert tp.tp_kv_cache_bytes(_qkv70(t, t - 1), 4, 4096) == 4 * nkv * 4096 * 128 * 2
    assert tp.tp_kv_cache_bytes(tp.tp_shard_plan("col", 64, 64, 1, 0), 1, 16) == 0
    assert tp.tp_kv_cache_bytes(tp.tp_shard_plan("qkv_col", 32, 12 * 16, 1, 0, heads=(8, 2, 16)), 1, 16) == 0  # d = 16
    assert tp.tp_kv_cache_bytes(_qkv70(8, 0), 1, 2 ** 23) == 0  # one head past 2^31 bytes
    q = _qkv70(8, 0)  # 8 query heads on one key-value head
    assert tp.tp_attention_workspace_bytes(q, 32, 1, 4096) == 32 * 8 * (16 * 128 + 32) * 4
    assert tp.tp_attention_workspace_bytes(q, 32, 2, 4097) == 32 * 9 * (16 * 128 + 32) * 4
    assert tp.tp_attention_workspace_bytes(q, 1, 3, 4096) == 0  # 24 rows: the prefill form
    q16 = _qkv70(16, 5)  # 4 query heads, repeated key-value head
    assert tp.tp_attention_workspace_bytes(q16, 2, 4, 300) == 0  # one chunk: no partials
    assert tp.tp_attention_workspace_bytes(q16, 2, 4, 513) == 2 * 2 * (16 * 128 + 32) * 4
    assert tp.tp_attention_workspace_bytes(q16, 2, 5, 300) == 0
    part = (16 * 128 + 32) * 4
    assert tp.tp_attention_workspace_bytes(q, 64, 1, 4096) == 64 * 4 * part  # 1024-position chunks
    assert tp.tp_attention_workspace_bytes(q, 128, 1, 4096) == 128 * 2 * part  # 2048-position chunks
    assert tp.tp_attention_workspace_bytes(q, 256, 1, 4096) == 0  # one 4096-position chunk each
    assert tp.tp_attention_workspace_bytes(q, 32, 1, 32768) == 32 * 8 * part  # 4096-position chunks
    assert tp.tp_attention_workspace_bytes(q, 1, 1, 32768) == 1 * 64 * part  # too few to lengthen
    assert tp.tp_attention_workspace_bytes(q, 300, 1, 1000) == 0  # 300 x 1: one 1024-position chunk


def test_attention_argument_errors():
    """Every refusal happens on the host, before any launch."""
    lib = _lib.load()
    S_ = ctypes.c_void_p(0)
    q = _qkv70(8, 0)
    qb = ctypes.byref(q)
    W = 10 * 128  # QKV row width of the rank
    KL, SL = ctypes.c_void_p(0x400000), ctypes.c_void_p(0x500000)
    ws_need = tp.tp_attention_workspace_bytes(q, 2, 1, 64)
    ws_long = tp.tp_attention_workspace_bytes(q, 2, 1, 1024)
    assert ws_need == 0 and ws_long > 0
    att = lib.tp_attention
    app = lib.tp_kv_append
    col = tp.tp_shard_plan("col", 64, 64, 1, 0)
    assert att(ctypes.byref(col), A, W, 2, 1, KL, SL, 64, B, C, 2, 64, A, 1024, A, ws_need, S_) == _lib.TP_ERR_KIND
    assert att(None, A, W, 2, 1, KL, SL, 64, B, C, 2, 64, A, 1024, A, ws_need, S_) == _lib.TP_ERR_NULL
    assert att(qb, NUL, W, 2, 1, KL, SL, 64, B, C, 2, 64, A, 1024, A, ws_need, S_) == _lib.TP_ERR_NULL
    assert att(qb, A, W, 2, 1, NUL, SL, 64, B, C, 2, 64, A, 1024, A, ws_need, S_) == _lib.TP_ERR_NULL
    assert att(qb, A, W, 2, 1, KL, SL, 64, B, NUL, 2, 64, A, 1024, A, ws_need, S_) == _lib.TP_ERR_NULL
    assert att(qb, A, W, 2, 1, KL, SL, 64, B, C, 2, 64, NUL, 1024, A, ws_need, S_) == _lib.TP_ERR_NULL
    assert att(qb, A, W - 8, 2, 1, KL, SL, 64, B, C, 2, 64, A, 1024, A, ws_need, S_) == _lib.TP_ERR_SHAPE  # ldqkv
    assert att(qb, A, W, 2, 0, KL, SL, 64, B, C, 2, 64, A, 1024, A, ws_need, S_) == _lib.TP_ERR_SHAPE  # q_len 0
    assert att(qb, A, W, -1, 1, KL, SL, 64, B, C, 2, 64, A, 1024, A, ws_need, S_) == _lib.TP_ERR_SHAPE
    assert att(qb, A, W, 2, 1, KL, SL, 65, B, C, 2, 64, A, 1024, A, ws_need, S_) == _lib.TP_ERR_SHAPE  # max_kv > L_max
    assert att(qb, A, W, 2, 4, KL, SL, 3, B, C, 2, 64, A, 1024, A, ws_need, S_) == _lib.TP_ERR_SHAPE  # max_kv < q_len
    assert att(qb, A, W, 2, 1, KL, SL, 64, B, C, 0, 64, A, 1024, A, ws_need, S_) == _lib.TP_ERR_SHAPE  # no slot
    assert att(qb, A, W, 2, 1, KL, SL, 64, B, C, 2, 2 ** 23, A, 1024, A, ws_need, S_) == _lib.TP_ERR_SHAPE
    assert att(qb, A, W, 2, 1, KL, SL, 64, B, C, 2, 64, A, 1016, A, ws_need, S_) == _lib.TP_ERR_SHAPE  # lda
    assert att(qb, MIS, W, 2, 1, KL, SL, 64, B, C, 2, 64, A, 1024, A, ws_need, S_) == _lib.TP_ERR_ALIGN
    assert att(qb, A, W + 4, 2, 1, KL, SL, 64, B, C, 2, 64, A, 1024, A, ws_need, S_) == _lib.TP_ERR_ALIGN
    assert att(qb, A, W, 2, 1, ctypes.c_void_p(0x400002), SL, 64, B, C, 2, 64, A, 1024, A, ws_need, S_) == \
        _lib.TP_ERR_ALIGN
    assert att(qb, A, W, 2, 1, KL, SL, 64, B, C, 2, 64, MIS, 1024, A, ws_need, S_) == _lib.TP_ERR_ALIGN
    assert att(qb, A, W, 2, 1, KL, SL, 1024, B, C, 2, 1024, A, 1024, A, ws_long - 4, S_) == _lib.TP_ERR_WORKSPACE
    assert att(qb, A, W, 2, 1, KL, SL, 1024, B, C, 2, 1024, A, 1024, NUL, ws_long, S_) == _lib.TP_ERR_WORKSPACE
    assert att(qb, A, W, 2, 1, KL, SL, 1024, B, C, 2, 1024, A, 1024, MIS, ws_long, S_) == _lib.TP_ERR_WORKSPACE
    assert att(qb, NUL, W, 0, 1, NUL, NUL, 64, NUL, NUL, 2, 64, NUL, 1024, NUL, 0, S_) == _lib.TP_OK  # S == 0
    assert app(qb, NUL, W, 2, 1, KL, SL, B, C, 2, 64, S_) == _lib.TP_ERR_NULL
    assert app(qb, A, W, 2, 1, KL, SL, B, NUL, 2, 64, S_) == _lib.TP_ERR_NULL
    assert app(qb, A, W, 2, 1, KL, SL, MIS, C, 2, 64, S_) == _lib.TP_ERR_ALIGN
    assert app(qb, A, W, 2, 65, KL, SL, B, C, 2, 64, S_) == _lib.TP_ERR_SHAPE  # q_len > L_max
    assert app(ctypes.byref(col), A, W, 2, 1, KL, SL, B, C, 2, 64, S_) == _lib.TP_ERR_KIND
    assert app(qb, NUL, W, 0, 1, NUL, NUL, NUL, NUL, 2, 64, S_) == _lib.TP_OK  # S == 0
