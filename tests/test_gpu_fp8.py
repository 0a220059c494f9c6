"""GPU parity of the 8-bit weight path (TP_W_FP8_E4M3: OCP FP8 E4M3 codes, one
power-of-two scale per output column; "AI Infrastructure series, Part 5",
"Reason 2": a 70B model in 8-bit reads half the bytes per token) against the
fp64 oracle: the packed codes and scales bit-exact, the linears within the
tolerance, and bit-exact where the weights quantise exactly.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
import tensor_transformer_linear_megatron_amd as tp
from seeded_inputs import workloads as wl
from tputil import assert_parity, dev, host_f64, say, unpack8

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def plan8(kind, K, N, t, r, heads=None, path=tp.TP_PATH_AUTO):
    d = tp.tp_shard_set_wformat(tp.tp_shard_plan(kind, K, N, t, r, heads=heads), "fp8_e4m3")
    d.path = path
    return d, oracle.plan(kind, K, N, t, r, heads=heads)


PACK_CASES = [("col", 200, 96, 2, 1, None), ("gateup_col", 136, 2 * 80, 2, 0, None),
              ("row", 544, 64, 4, 3, None), ("qkv_col", 256, 1536, 4, 1, (16, 4, 64)),
              ("o_row", 1024, 136, 2, 0, (16, 4, 64)), ("col", 64, 32, 1, 0, None)]


@pytest.mark.parametrize("kind,K,N,t,r,heads", PACK_CASES)
def test_pack8_codes_and_scales_bit_exact(kind, K, N, t, r, heads):
    say("pack8", kind, K, N, t, r)
    W = si.normal_bf16(50, (K, N), 0.05)
    d, p = plan8(kind, K, N, t, r, heads)
    assert d.packed_bytes == d.packed_k * d.packed_n + 4 * d.packed_n and d.packed_k % 64 == 0
    codes, scales = unpack8(d, tp.tp_shard_pack(d, dev(W)))
    want_q, want_e = oracle.quantize_columns(oracle.bf16_to_f64(W[p["rows"]][:, p["cols"]]))
    np.testing.assert_array_equal(codes, want_q)
    np.testing.assert_array_equal(scales.astype(np.float64), np.exp2(want_e.astype(np.float64)))


def test_pack8_zero_and_wide_columns():
    """All-zero columns get 2^0 and zero codes; columns spanning many binades
    keep their largest value within 448 and subnormal codes for the smallest."""
    K, N = 128, 64
    rng = np.random.default_rng(3)
    Wf = rng.standard_normal((K, N)) * 10.0 ** rng.integers(-6, 3, size=(K, N))
    Wf[:, 5] = 0.0
    W = oracle.round_bf16(Wf)
    d, p = plan8("col", K, N, 1, 0)
    codes, scales = unpack8(d, tp.tp_shard_pack(d, dev(W)))
    want_q, want_e = oracle.quantize_columns(oracle.bf16_to_f64(W))
    np.testing.assert_array_equal(codes, want_q)
    np.testing.assert_array_equal(scales.astype(np.float64), np.exp2(want_e.astype(np.float64)))
    assert scales[5] == 1.0 and not codes[:, 5].any()


def _col8(kind, K, N, t, r, M, path, heads=None, seed=60):
    X = si.normal_bf16(seed, (M, K), 1.0)
    W = si.normal_bf16(seed + 1, (K, N), 0.05)
    d, p = plan8(kind, K, N, t, r, heads, path)
    Y = tp.tp_col_linear(d, dev(X), tp.tp_shard_pack(d, dev(W)))
    if kind == "gateup_col":
        ref = oracle.bf16_to_f64(oracle.gateup_swiglu_fp8(X, W, p))
    else:
        ref = oracle.bf16_to_f64(oracle.round_bf16(oracle.col_linear_fp8(X, W, p)))
    return host_f64(Y), ref


def _row8(kind, K, N, t, r, M, path, heads=None, seed=70):
    Z = si.normal_bf16(seed, (M, K), 1.0)
    W = si.normal_bf16(seed + 1, (K, N), 0.05)
    d, p = plan8(kind, K, N, t, r, heads, path)
    Zr = Z[:, p["rows"]]
    P = tp.tp_row_linear(d, dev(Zr), tp.tp_shard_pack(d, dev(W)))
    return host_f64(P), oracle.row_linear_fp8(Zr, W, p)


DECODE_M = [1, 5, 16, 17, 33, 64]
PREFILL_M = [65, 300]


@pytest.mark.parametrize("M", DECODE_M + PREFILL_M)
@pytest.mark.parametrize("kind,K,N,t,r,heads", [("col", 1000, 200, 1, 0, None), ("col", 4104, 1040, 2, 1, None),
                                                ("qkv_col", 1024, 1536, 4, 2, (16, 4, 64))])
def test_col8_parity(kind, K, N, t, r, heads, M):
    say("col8", kind, K, N, t, r, M)
    got, ref = _col8(kind, K, N, t, r, M, tp.TP_PATH_AUTO, heads)
    assert_parity(got, ref, f"{kind} K={K} N={N} M={M}")


@pytest.mark.parametrize("M", DECODE_M + PREFILL_M)
@pytest.mark.parametrize("K,N,t,r", [(264, 2 * 200, 1, 0), (4096, 2 * 1216, 4, 3)])
def test_gateup8_parity(K, N, t, r, M):
    say("gateup8", K, N, t, r, M)
    got, ref = _col8("gateup_col", K, N, t, r, M, tp.TP_PATH_AUTO)
    assert_parity(got, ref, f"gateup K={K} N={N} M={M}")


@pytest.mark.parametrize("M", DECODE_M + PREFILL_M)
@pytest.mark.parametrize("kind,K,N,t,r,heads", [("row", 2064, 520, 2, 1, None), ("row", 14336, 4096, 8, 5, None),
                                                ("o_row", 2048, 1000, 4, 3, (16, 4, 128))])
def test_row8_parity(kind, K, N, t, r, heads, M):
    say("row8", kind, K, N, t, r, M)
    got, ref = _row8(kind, K, N, t, r, M, tp.TP_PATH_AUTO, heads)
    assert_parity(got, ref, f"{kind} K={K} N={N} M={M}")


@pytest.mark.parametrize("path", [tp.TP_PATH_DECODE, tp.TP_PATH_PREFILL])
@pytest.mark.parametrize("M", [3, 64])
def test_fp8_exact_integer_weights_bit_exact(path, M):
    """Weights in [-15, 15] quantise exactly and activations in [-3, 3] keep
    every fp32 partial sum an exact integer: GPU == oracle bit for bit, on the
    decode and the prefill path, for the bf16, SwiGLU-free fp32 outputs."""
    say("fp8 exact", path, M)
    K, N = 2112, 272
    X = si.int_bf16(80, (M, K), -3, 3)
    W = si.int_bf16(81, (K, N), -15, 15)
    d, p = plan8("row", K, N, 1, 0, None, path)
    P = tp.tp_row_linear(d, dev(X), tp.tp_shard_pack(d, dev(W)))
    np.testing.assert_array_equal(host_f64(P), oracle.row_linear_fp8(X, W, p))
    dc, pc = plan8("col", K, N, 1, 0, None, path)
    Y = tp.tp_col_linear(dc, dev(X), tp.tp_shard_pack(dc, dev(W)))
    np.testing.assert_array_equal(host_f64(Y), oracle.bf16_to_f64(oracle.round_bf16(oracle.col_linear_fp8(X, W, pc))))


def test_fp8_decode_and_prefill_agree_with_oracle_at_boundary():
    """M = 64 on both paths: the GEMV decodes codes in registers, the prefill
    path dequantises into the workspace and runs the bf16 GEMM."""
    say("fp8 boundary")
    for path in (tp.TP_PATH_DECODE, tp.TP_PATH_PREFILL):
        got, ref = _col8("gateup_col", 1024, 2 * 320, 2, 1, 64, path)
        assert_parity(got, ref, f"gateup path={path}")


def test_fp8_workspace():
    """No workspace up to 16 tokens; split-K partials for the shared-token
    kernel when its column blocks do not fill the GPU; at prefill the
    dequantised bf16 copy (plus any split-K partials); a short workspace is
    refused."""
    d, _ = plan8("col", 4096, 1024, 1, 0)
    assert tp.tp_workspace_bytes(d, 1) == 0 and tp.tp_workspace_bytes(d, 16) == 0
    assert tp.tp_workspace_bytes(d, 64) % (64 * d.packed_n * 4) == 0
    ws = tp.tp_workspace_bytes(d, 300)
    assert ws >= d.packed_k * d.packed_n * 2
    X = dev(si.normal_bf16(90, (300, 4096), 1.0))
    Wp = tp.tp_shard_pack(d, dev(si.normal_bf16(91, (4096, 1024), 0.05)))
    short = torch.empty(ws - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(tp.TpError):
        tp.tp_col_linear(d, X, Wp, ws=short)


@pytest.mark.parametrize("M", [1, 8, 32])
def test_llama70b_ffn_tp8_rank_fp8(M):
    """One TP = 8 rank of the 70B feed-forward layer with 8-bit weights (the
    pages' decode example is this model in 8-bit): gate/up + SwiGLU then down,
    rank 3, against the oracle with the same quantisation."""
    say("70b ffn fp8 rank 3", M)
    c = wl.LLAMA70B
    H, I, t, r = c["hidden"], c["inter"], 8, 3
    w = I // t
    cols = range(r * w, (r + 1) * w)
    X = wl.activations(M, H)
    Wgu_r = wl.gateup(H, I, c["sigma"], cols=cols)
    Wd_r = wl.down(I, H, c["sigma"], rows=cols)
    gu = tp.tp_shard_set_wformat(tp.tp_shard_plan("gateup_col", H, 2 * w, 1, 0), "fp8_e4m3")
    dn = tp.tp_shard_set_wformat(tp.tp_shard_plan("row", w, H, 1, 0), "fp8_e4m3")
    Hh, P = tp.tp_ffn_shard(gu, dn, dev(X), tp.tp_shard_pack(gu, dev(Wgu_r)), tp.tp_shard_pack(dn, dev(Wd_r)))
    pg, pd = oracle.plan("gateup_col", H, 2 * w, 1, 0), oracle.plan("row", w, H, 1, 0)
    Href = oracle.gateup_swiglu_fp8(X, Wgu_r, pg)
    assert_parity(host_f64(Hh), oracle.bf16_to_f64(Href), "H")
    assert_parity(host_f64(P), oracle.row_linear_fp8(Href, Wd_r, pd), "P")


def _random_cases8(n=18, seed=2025):
    """Seeded random 8-bit shards (column, gate/up and row kinds, t in {1, 2,
    4, 8}, random rank), K and N up to 2048, token counts on either side of
    the decode / prefill boundary."""
    rng = np.random.default_rng(seed)
    cases = []
    for c in range(n):
        kind = ("col", "gateup_col", "row")[c % 3]
        t = int(rng.choice([1, 2, 4, 8]))
        r = int(rng.integers(0, t))
        wide = t * 8 * int(rng.integers(1, 1 + 2048 // (8 * t)))
        other = 8 * int(rng.integers(1, 257))
        if kind == "row":
            K, N = wide, other
        elif kind == "col":
            K, N = other, wide
        else:
            K, N = other, 2 * (wide // 2 // (8 * t) * 8 * t or 8 * t)
        M = int(rng.integers(1, 65)) if c % 2 else int(rng.integers(65, 600))
        cases.append((kind, K, N, t, r, M))
    return cases


@pytest.mark.parametrize("kind,K,N,t,r,M", _random_cases8())
def test_random_shards8_against_oracle(kind, K, N, t, r, M):
    """Random 8-bit shapes through the automatic path choice: every row at
    decode sizes, the edges and one row per 256-token tile at prefill sizes."""
    say("random shard8", kind, K, N, t, r, M)
    rows = list(range(M)) if M <= 64 else sorted({0, 1, M // 2, M - 2, M - 1} | set(range(100, M, 256)))
    X = si.normal_bf16(52, (M, K), 1.0)
    W = si.normal_bf16(53, (K, N), 0.05)
    d, p = plan8(kind, K, N, t, r)
    Wp = tp.tp_shard_pack(d, dev(W))
    if kind == "row":
        Zr = X[:, p["rows"]]
        got = host_f64(tp.tp_row_linear(d, dev(Zr), Wp))[rows]
        ref = oracle.row_linear_fp8(np.ascontiguousarray(Zr[rows]), W, p)
    else:
        got = host_f64(tp.tp_col_linear(d, dev(X), Wp))[rows]
        Xs = np.ascontiguousarray(X[rows])
        if kind == "gateup_col":
            ref = oracle.bf16_to_f64(oracle.gateup_swiglu_fp8(Xs, W, p))
        else:
            ref = oracle.bf16_to_f64(oracle.round_bf16(oracle.col_linear_fp8(Xs, W, p)))
    assert_parity(got, ref, f"fp8 {kind} K={K} N={N} t={t} r={r} M={M}")
