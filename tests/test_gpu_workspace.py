"""The workspace a call reports is what its kernels use, no more and no less.

Each case runs a call whose kernels keep data in the workspace (fp32
partials of the decode split-K, the prefill split-K, the prefill's split last
round and the attention decode's chunks; the 8-bit prefill's dequantised bf16
copy of the shard) with a workspace of exactly the reported size. That
workspace is filled with NaN bit patterns beforehand and sits at the start of
a larger buffer whose tail holds a canary. The whole output must be finite
and the sampled rows must match the oracle (so no kernel reads workspace
bytes that no kernel of the call wrote: a NaN would spread to the output),
and the canary must come back intact (so no kernel writes past the reported
size).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
import tensor_transformer_linear_megatron_amd as tp
from tputil import assert_parity, dev, host_bits, host_f64, say

pytestmark = pytest.mark.gpu

CANARY = 1 << 20  # bytes after the workspace
CANARY_BYTE = 0xA5


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def _buffer(need: int):
    """A workspace of exactly ``need`` bytes filled with 0xFF bytes (fp32 NaN)
    followed by the canary; returns (whole buffer, the workspace view)."""
    buf = torch.full((need + CANARY,), CANARY_BYTE, dtype=torch.uint8, device="cuda")
    buf[:need] = 0xFF
    return buf, buf[:need]


def _canary_intact(buf: torch.Tensor, need: int, what: str):
    torch.cuda.synchronize()
    tail = buf[need:].cpu().numpy()
    bad = np.flatnonzero(tail != CANARY_BYTE)
    assert bad.size == 0, f"{what}: {bad.size} canary bytes overwritten, first at workspace + {need + bad[0]}"


# (kind, K, N, t, r, M, path): decode split-K over few output tiles (ragged
# K), the prefill split-K over few big tiles, and prefill shapes whose last
# round of big tiles runs as a split-K rectangle.
LINEAR_CASES = [
    ("col", 8184, 80, 1, 0, 50, tp.TP_PATH_AUTO),
    ("gateup_col", 8184, 2 * 48, 1, 0, 64, tp.TP_PATH_AUTO),
    ("row", 2 * 8184, 72, 2, 1, 33, tp.TP_PATH_AUTO),
    ("gateup_col", 2056, 2 * 600, 1, 0, 520, tp.TP_PATH_PREFILL),
    ("row", 3088, 1000, 2, 1, 257, tp.TP_PATH_PREFILL),
    ("col", 1000, 4328, 1, 0, 4000, tp.TP_PATH_PREFILL),
    ("gateup_col", 1000, 2 * 2168, 1, 0, 4000, tp.TP_PATH_PREFILL),
    # drawn by a seeded search over random shapes for ones whose last round
    # of big tiles runs as a split-K sub-GEMM (ragged token counts)
    ("gateup_col", 2048, 5760, 1, 0, 2979, tp.TP_PATH_PREFILL),
    ("col", 2112, 15744, 1, 0, 8591, tp.TP_PATH_PREFILL),
    ("gateup_col", 1536, 9088, 1, 0, 8971, tp.TP_PATH_PREFILL),
    ("row", 2432, 5184, 1, 0, 6307, tp.TP_PATH_PREFILL),
]


@pytest.mark.parametrize("kind,K,N,t,r,M,path", LINEAR_CASES)
def test_linear_workspace_is_exactly_enough(kind, K, N, t, r, M, path):
    say("workspace", kind, K, N, t, r, M, path)
    d = tp.tp_shard_plan(kind, K, N, t, r)
    p = oracle.plan(kind, K, N, t, r)
    d.path = path
    need = tp.tp_workspace_bytes(d, M)
    assert need > 0, "the case does not use a workspace"
    X = si.normal_bf16(70, (M, K), 1.0)
    W = si.normal_bf16(71, (K, N), 0.05)
    Wp = tp.tp_shard_pack(d, dev(W))
    buf, ws = _buffer(need)
    # one row in every 256-token tile, plus the edges
    rows = sorted({0, 1, M // 3, M // 2, M - 2, M - 1} | {min(M - 1, t0 + 131) for t0 in range(0, M, 256)})
    if kind == "row":
        Zr = X[:, p["rows"]]
        out = tp.tp_row_linear(d, dev(Zr), Wp, ws=ws)
        ref = oracle.row_linear(Zr[rows], W, p)
    else:
        out = tp.tp_col_linear(d, dev(X), Wp, ws=ws)
        fn = oracle.gateup_swiglu if kind == "gateup_col" else oracle.col_linear_bf16
        ref = oracle.bf16_to_f64(fn(X[rows], W, p))
    # a workspace byte read before any kernel of the call wrote it is NaN, and
    # would leave a non-finite value somewhere in the output
    assert bool(torch.isfinite(out.float()).all()), f"{kind} K={K} N={N} M={M}: non-finite output"
    got = host_f64(out)[rows]
    _canary_intact(buf, need, f"{kind} K={K} N={N} M={M}")
    assert_parity(got, ref, f"{kind} K={K} N={N} M={M} with an exact workspace")


# 8-bit shards: the decode split-K (gemv_shared's 8-bit form), and the
# prefill path, whose workspace holds the dequantised bf16 copy of the shard
# (plus split-K partials when the big tiles do not fill the GPU).
FP8_CASES = [("col", 8192, 80, 1, 0, 40, tp.TP_PATH_AUTO), ("gateup_col", 4096, 2 * 64, 1, 0, 64, tp.TP_PATH_AUTO),
             ("col", 1024, 520, 1, 0, 300, tp.TP_PATH_PREFILL), ("row", 2048, 1000, 2, 1, 600, tp.TP_PATH_PREFILL)]


@pytest.mark.parametrize("kind,K,N,t,r,M,path", FP8_CASES)
def test_fp8_workspace_is_exactly_enough(kind, K, N, t, r, M, path):
    say("workspace fp8", kind, K, N, t, r, M, path)
    d = tp.tp_shard_set_wformat(tp.tp_shard_plan(kind, K, N, t, r), "fp8_e4m3")
    d.path = path
    p = oracle.plan(kind, K, N, t, r)
    need = tp.tp_workspace_bytes(d, M)
    assert need > 0, "the case does not use a workspace"
    X = si.normal_bf16(77, (M, K), 1.0)
    W = si.normal_bf16(78, (K, N), 0.05)
    Wp = tp.tp_shard_pack(d, dev(W))
    buf, ws = _buffer(need)
    rows = sorted({0, 1, M // 2, M - 1})
    if kind == "row":
        Zr = X[:, p["rows"]]
        out = tp.tp_row_linear(d, dev(Zr), Wp, ws=ws)
        ref = oracle.row_linear_fp8(Zr[rows], W, p)
    else:
        out = tp.tp_col_linear(d, dev(X), Wp, ws=ws)
        if kind == "gateup_col":
            ref = oracle.bf16_to_f64(oracle.gateup_swiglu_fp8(X[rows], W, p))
        else:
            ref = oracle.bf16_to_f64(oracle.round_bf16(oracle.col_linear_fp8(X[rows], W, p)))
    assert bool(torch.isfinite(out.float()).all()), f"fp8 {kind} K={K} N={N} M={M}: non-finite output"
    got = host_f64(out)[rows]
    _canary_intact(buf, need, f"fp8 {kind} K={K} N={N} M={M}")
    assert_parity(got, ref, f"fp8 {kind} K={K} N={N} M={M} with an exact workspace")


def test_workspace_one_byte_short_is_refused():
    """One byte less than the reported size is refused before any launch."""
    d = tp.tp_shard_plan("col", 8184, 80, 1, 0)
    M = 50
    need = tp.tp_workspace_bytes(d, M)
    X = dev(si.normal_bf16(72, (M, 8184), 1.0))
    Wp = tp.tp_shard_pack(d, dev(si.normal_bf16(73, (8184, 80), 0.05)))
    ws = torch.empty(need - 1, dtype=torch.uint8, device="cuda")
    with pytest.raises(tp.TpError):
        tp.tp_col_linear(d, X, Wp, ws=ws)


def test_attention_decode_workspace_is_exactly_enough():
    """The 70B TP = 8 rank-0 heads (8 query heads, 1 key-value head) over a
    few long caches: several 512-position chunks per sequence, their partials
    in the workspace, merged by the combine launch."""
    heads, t, r = (64, 8, 128), 8, 0
    n_q, n_kv, dh = heads
    K = 256
    N = (n_q + 2 * n_kv) * dh
    q = tp.tp_shard_plan("qkv_col", K, N, t, r, heads=heads)
    p = oracle.plan("qkv_col", K, N, t, r, heads=heads)
    S, L = 4, 4096
    kv = [L, 3000, 1025, 513]
    need = tp.tp_attention_workspace_bytes(q, S, 1, L)
    assert need > 0, "one chunk per sequence: no workspace"
    say("attention workspace", S, L, need)
    QKV = si.normal_bf16(74, (S, p["shard_n"]), 1.0)
    Kh, Vh = oracle.kv_cache_new(p, S, L)
    Kh[:] = si.normal_bf16(75, (int(np.prod(Kh.shape[:-1])), Kh.shape[-1]), 1.0).reshape(Kh.shape)
    Vh[:] = si.normal_bf16(76, (int(np.prod(Vh.shape[:-1])), Vh.shape[-1]), 1.0).reshape(Vh.shape)
    Kd, Vd = dev(Kh), dev(Vh)
    kl = torch.tensor(kv, dtype=torch.int32, device="cuda")
    sl = torch.arange(S, dtype=torch.int32, device="cuda")
    tp.tp_kv_append(q, dev(QKV), 1, kl, sl, Kd, Vd)
    oracle.kv_append(QKV, p, 1, kv, list(range(S)), Kh, Vh)
    buf, ws = _buffer(need)
    A = host_bits(tp.tp_attention(q, dev(QKV), 1, kl, sl, Kd, Vd, L, ws=ws))
    _canary_intact(buf, need, "attention decode")
    ref = oracle.attention(QKV, p, 1, kv, list(range(S)), Kh, Vh)
    assert_parity(oracle.bf16_to_f64(A), oracle.bf16_to_f64(ref), "attention decode with an exact workspace")
