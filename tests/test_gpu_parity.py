"""GPU parity: the HIP path through the C ABI against the fp64 oracle on the
same seeded inputs, at small ragged sizes and at the full model-shaped sizes.

Bar: bit-exact for the shard bookkeeping and packing, for integer-valued and
identity inputs; relative Frobenius error <= 1e-3 and max element error
<= 1e-2 * max |oracle| otherwise.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
import tensor_transformer_linear_megatron_amd as tp
from seeded_inputs import workloads as wl
from tputil import assert_parity, dev, full_device, host_bits, host_f64, say, unpack

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def plan_both(kind, K, N, t, r, heads=None):
    return tp.tp_shard_plan(kind, K, N, t, r, heads=heads), oracle.plan(kind, K, N, t, r, heads=heads)


def with_path(d, path):
    e = d.copy()
    e.path = path
    return e


# ---------------------------------------------------------------------------
# Packing and bookkeeping: bit-exact.
# ---------------------------------------------------------------------------

PACK_CASES = [("col", 96, 64, 2, 1, None), ("col", 264, 40, 1, 0, None), ("row", 96, 72, 3, 2, None),
              ("gateup_col", 72, 2 * 24, 1, 0, None), ("gateup_col", 40, 2 * 96, 4, 3, None),
              ("qkv_col", 64, (8 + 2 * 2) * 16, 4, 1, (8, 2, 16)),
              ("qkv_col", 64, (8 + 2 * 2) * 16, 8, 5, (8, 2, 16)),
              ("o_row", 8 * 16, 48, 4, 3, (8, 2, 16)), ("col", 4096, 4096, 2, 1, None)]


@pytest.mark.parametrize("kind,K,N,t,r,heads", PACK_CASES)
def test_pack_is_the_planned_shard(kind, K, N, t, r, heads):
    say("pack", kind, K, N, t, r, heads)
    W = si.normal_bf16(21, (K, N), 1.0)
    d, p = plan_both(kind, K, N, t, r, heads)
    packed = tp.tp_shard_pack(d, dev(W))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(unpack(d, packed), W[np.ix_(p["rows"], p["cols"])])
    # the zero padding is really zero
    total = host_bits(packed.view(torch.bfloat16).view(1, -1))
    assert np.count_nonzero(total) <= d.shard_k * d.shard_n


# ---------------------------------------------------------------------------
# Small, ragged shapes spanning several tiles, both paths.
# ---------------------------------------------------------------------------

def _col_case(kind, K, N, t, r, M, path, heads=None, seed=30):
    X = si.normal_bf16(seed, (M, K), 1.0)
    W = si.normal_bf16(seed + 1, (K, N), 0.05)
    d, p = plan_both(kind, K, N, t, r, heads)
    d = with_path(d, path)
    Wp = tp.tp_shard_pack(d, dev(W))
    Y = tp.tp_col_linear(d, dev(X), Wp)
    if kind == "gateup_col":
        ref = oracle.bf16_to_f64(oracle.gateup_swiglu(X, W, p))
    else:
        ref = oracle.bf16_to_f64(oracle.col_linear_bf16(X, W, p))
    return host_f64(Y), ref


def _row_case(kind, K, N, t, r, M, path, heads=None, seed=40):
    Z = si.normal_bf16(seed, (M, K), 1.0)
    W = si.normal_bf16(seed + 1, (K, N), 0.05)
    d, p = plan_both(kind, K, N, t, r, heads)
    d = with_path(d, path)
    Zr = Z[:, p["rows"]]
    P = tp.tp_row_linear(d, dev(Zr), tp.tp_shard_pack(d, dev(W)))
    return host_f64(P), oracle.row_linear(Zr, W, p)


SMALL_M = [1, 3, 16, 17, 33, 64, 65, 130, 257]
SMALL_SHAPES = [(8, 32), (40, 24), (264, 136), (1000, 200)]
PATHS = [tp.TP_PATH_AUTO, tp.TP_PATH_PREFILL]


@pytest.mark.parametrize("M", SMALL_M)
@pytest.mark.parametrize("K,N", SMALL_SHAPES)
@pytest.mark.parametrize("path", PATHS)
def test_col_small(M, K, N, path):
    say("col small", M, K, N, path)
    got, ref = _col_case("col", K, N, 1, 0, M, path)
    assert_parity(got, ref, f"col M={M} K={K} N={N} path={path}")


@pytest.mark.parametrize("M", SMALL_M)
@pytest.mark.parametrize("path", PATHS)
def test_gateup_small(M, path):
    say("gateup small", M, path)
    for K, inter, t, r in ((40, 24, 1, 0), (264, 96, 4, 2), (1000, 48, 2, 1)):
        got, ref = _col_case("gateup_col", K, 2 * inter, t, r, M, path)
        assert_parity(got, ref, f"gateup M={M} K={K} I={inter} t={t} r={r}")


@pytest.mark.parametrize("M", SMALL_M)
@pytest.mark.parametrize("path", PATHS)
def test_row_small(M, path):
    say("row small", M, path)
    for K, N, t, r in ((64, 24, 2, 1), (528, 136, 2, 0), (2000, 40, 5, 4)):
        got, ref = _row_case("row", K, N, t, r, M, path)
        assert_parity(got, ref, f"row M={M} K={K} N={N} t={t} r={r}")


def _random_cases(n=36, seed=2024):
    """Seeded random shards: column, gate/up and row kinds at t in {1, 2, 4,
    8} on a random rank, K and N up to 2048 (multiples of 8 per shard), and
    token counts on either side of the decode / prefill boundary."""
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
        M = int(rng.integers(1, 65)) if c % 2 else int(rng.integers(65, 700))
        cases.append((kind, K, N, t, r, M))
    return cases


@pytest.mark.parametrize("kind,K,N,t,r,M", _random_cases())
def test_random_shards_against_oracle(kind, K, N, t, r, M):
    """Random shapes through the automatic path choice: every row at decode
    sizes, the edges and one row per 256-token tile at prefill sizes."""
    say("random shard", kind, K, N, t, r, M)
    rows = list(range(M)) if M <= 64 else sorted({0, 1, M // 2, M - 2, M - 1} | set(range(100, M, 256)))
    X = si.normal_bf16(50, (M, K), 1.0)
    W = si.normal_bf16(51, (K, N), 0.05)
    d, p = plan_both(kind, K, N, t, r)
    Wp = tp.tp_shard_pack(d, dev(W))
    if kind == "row":
        Zr = X[:, p["rows"]]
        got = host_f64(tp.tp_row_linear(d, dev(Zr), Wp))[rows]
        ref = oracle.row_linear(np.ascontiguousarray(Zr[rows]), W, p)
    else:
        got = host_f64(tp.tp_col_linear(d, dev(X), Wp))[rows]
        fn = oracle.gateup_swiglu if kind == "gateup_col" else oracle.col_linear_bf16
        ref = oracle.bf16_to_f64(fn(np.ascontiguousarray(X[rows]), W, p))
    assert_parity(got, ref, f"{kind} K={K} N={N} t={t} r={r} M={M}")


def _random_big_cases(n=10, seed=4096):
    """Seeded random prefill shapes large enough for the big-tile GEMM (whole
    rounds, a split last round, split K, half tiles), all three kinds."""
    rng = np.random.default_rng(seed)
    cases = []
    for c in range(n):
        kind = ("col", "gateup_col", "row")[c % 3]
        t = int(rng.choice([1, 2, 4]))
        r = int(rng.integers(0, t))
        M = int(rng.integers(2049, 8193))
        wide = t * 8 * int(rng.integers(16, 1 + 12288 // (8 * t)))
        other = 8 * int(rng.integers(4, 385))
        if kind == "row":
            K, N = wide // 4 // (8 * t) * 8 * t or 8 * t, other * 4
        elif kind == "col":
            K, N = other, wide
        else:
            K, N = other, 2 * (wide // 2 // (8 * t) * 8 * t or 8 * t)
        cases.append((kind, K, N, t, r, M))
    return cases


@pytest.mark.parametrize("kind,K,N,t,r,M", _random_big_cases())
def test_random_prefill_shapes_against_oracle(kind, K, N, t, r, M):
    """Random big prefill shapes: the first and last rows and two rows of
    every 256-token tile against the oracle."""
    say("random prefill", kind, K, N, t, r, M)
    rows = sorted({0, M - 1} | set(range(37, M, 256)) | set(range(200, M, 256)))
    X = si.normal_bf16(54, (M, K), 1.0)
    W = si.normal_bf16(55, (K, N), 0.05)
    d, p = plan_both(kind, K, N, t, r)
    Wp = tp.tp_shard_pack(d, dev(W))
    if kind == "row":
        Zr = X[:, p["rows"]]
        got = host_f64(tp.tp_row_linear(d, dev(Zr), Wp))[rows]
        ref = oracle.row_linear(np.ascontiguousarray(Zr[rows]), W, p)
    else:
        got = host_f64(tp.tp_col_linear(d, dev(X), Wp))[rows]
        fn = oracle.gateup_swiglu if kind == "gateup_col" else oracle.col_linear_bf16
        ref = oracle.bf16_to_f64(fn(np.ascontiguousarray(X[rows]), W, p))
    assert_parity(got, ref, f"{kind} K={K} N={N} t={t} r={r} M={M}")


# Grids of at least 256 workgroups of 256 x 256 run the big-tile prefill
# kernel: ragged token count, ragged last k-step, odd and partial column tiles.
# Grids of 256 + 16 tiles also run the half-height tail launch (including a
# half tile wholly past M and a partial second half).
BIG_CASES = [("col", 8, 3904, 1, 0, 4000), ("col", 200, 4040, 1, 0, 3965), ("col", 360, 3880, 1, 0, 4097),
             ("gateup_col", 200, 2 * 1944, 1, 0, 3965), ("gateup_col", 136, 2 * 7808, 4, 3, 4000),
             ("gateup_col", 136, 2 * 2000, 1, 0, 4100),
             ("row", 528, 3880, 2, 1, 4001), ("row", 64, 4096, 1, 0, 4096), ("row", 264, 3872, 1, 0, 4300)]


@pytest.mark.parametrize("kind,K,N,t,r,M", BIG_CASES)
def test_prefill_big_tile_ragged(kind, K, N, t, r, M):
    say("prefill big tile", kind, K, N, t, r, M)
    if kind == "row":
        got, ref = _row_case(kind, K, N, t, r, M, tp.TP_PATH_PREFILL)
    else:
        got, ref = _col_case(kind, K, N, t, r, M, tp.TP_PATH_PREFILL)
    assert_parity(got, ref, f"{kind} K={K} N={N} t={t} r={r} M={M}")


# 17 x 16 big tiles: 256 run whole, the last 16 (token tiles 8..15 x column
# tiles 15 and 16) form a rectangle and run as a sub-GEMM with K split 2 ways
# (fp32 partials, then the fix-up applies the epilogue). Ragged K, columns and
# tokens; rows sampled from both parts (rows are independent).
TAIL_CASES = [("col", 1000, 4328, 1, 0, 4000), ("gateup_col", 1000, 2 * 2168, 1, 0, 4000),
              ("row", 1000, 4328, 1, 0, 4000)]


@pytest.mark.parametrize("kind,K,N,t,r,M", TAIL_CASES)
def test_prefill_tail_split_k(kind, K, N, t, r, M):
    say("prefill tail split-K", kind, K, N, t, r, M)
    d, p = plan_both(kind, K, N, t, r)
    d = with_path(d, tp.TP_PATH_PREFILL)
    assert tp.tp_workspace_bytes(d, M) == 2 * (M - 2048) * (d.packed_n // 16 - 240) * 16 * 4
    X = si.normal_bf16(90, (M, K), 1.0)
    W = si.normal_bf16(91, (K, N), 0.05)
    Wp = tp.tp_shard_pack(d, dev(W))
    rows = [0, 1, 1000, 2047, 2048, 2049, 3000, 3998, 3999]
    if kind == "row":
        got = host_f64(tp.tp_row_linear(d, dev(X), Wp))[rows]
        ref = oracle.row_linear(X[rows], W, p)
    else:
        got = host_f64(tp.tp_col_linear(d, dev(X), Wp))[rows]
        if kind == "gateup_col":
            ref = oracle.bf16_to_f64(oracle.gateup_swiglu(X[rows], W, p))
        else:
            ref = oracle.bf16_to_f64(oracle.col_linear_bf16(X[rows], W, p))
    assert_parity(got, ref, f"{kind} K={K} N={N} M={M} (tail split)")
    # the tail rectangle on its own, against the same rows' reference
    assert_parity(got[4:], ref[4:], f"{kind} tail rows")


# Few 256 x 256 output tiles and a long ragged K: the prefill path splits K
# over workgroups (fp32 partials in the workspace, summed in split order by
# the fix-up, which applies the epilogue). The last split has an odd number of
# k-steps and ends inside a k-step; the last token tile is partial.
SPLIT_CASES = [("col", 4104, 520, 1, 0, 300, None), ("gateup_col", 2056, 2 * 600, 1, 0, 520, None),
               ("row", 3088, 1000, 2, 1, 257, None), ("qkv_col", 2048, 1536, 4, 1, 700, (16, 4, 64)),
               ("o_row", 4096, 1000, 2, 0, 300, (32, 8, 128)),
               # fewer tokens than one big tile: the tile's rows past M read as zeros
               ("col", 8192, 512, 1, 0, 100, None), ("gateup_col", 4096, 2 * 256, 1, 0, 65, None)]


@pytest.mark.parametrize("kind,K,N,t,r,M,heads", SPLIT_CASES)
def test_prefill_split_k_ragged(kind, K, N, t, r, M, heads):
    say("prefill split-K", kind, K, N, t, r, M, heads)
    d = with_path(tp.tp_shard_plan(kind, K, N, t, r, heads=heads), tp.TP_PATH_PREFILL)
    assert tp.tp_workspace_bytes(d, M) >= 2 * M * d.packed_n * 4, "the split path is not taken"
    if kind in ("row", "o_row"):
        got, ref = _row_case(kind, K, N, t, r, M, tp.TP_PATH_PREFILL, heads=heads)
    else:
        got, ref = _col_case(kind, K, N, t, r, M, tp.TP_PATH_PREFILL, heads=heads)
    assert_parity(got, ref, f"{kind} K={K} N={N} t={t} r={r} M={M}")


@pytest.mark.parametrize("M", [17, 24, 32])
def test_decode_two_token_blocks_wide_shards(M):
    """17 to 32 tokens over 256 or more tile pairs with a short K (the 70B
    TP = 8 O slice and the like): the streaming kernel with two token blocks
    per wavefront, with no split and no workspace; ragged K. Beyond 32 tokens
    the split returns."""
    say("decode two token blocks", M)
    for kind, K, N, t, r, heads in (("o_row", 8192, 8192, 8, 3, (64, 8, 128)), ("row", 8 * 1000, 8192, 8, 2, None),
                                    ("gateup_col", 2000, 2 * 4096, 1, 0, None), ("col", 1000, 8192, 1, 0, None)):
        d = tp.tp_shard_plan(kind, K, N, t, r, heads=heads)
        assert tp.tp_workspace_bytes(d, M) == 0
        assert tp.tp_workspace_bytes(d, 33) > 0
        if kind in ("row", "o_row"):
            got, ref = _row_case(kind, K, N, t, r, M, tp.TP_PATH_AUTO, heads=heads)
        else:
            got, ref = _col_case(kind, K, N, t, r, M, tp.TP_PATH_AUTO, heads=heads)
        assert_parity(got, ref, f"{kind} K={K} N={N} t={t} r={r} M={M}")


@pytest.mark.parametrize("M", [17, 33, 50, 64])
def test_decode_split_k_ragged(M):
    """Long ragged K with few output tiles: the decode path splits K over
    workgroups (fp32 partials in the workspace, summed in split order)."""
    say("decode split-K", M)
    for kind, K, N, t, r in (("col", 8184, 80, 1, 0), ("gateup_col", 8184, 2 * 48, 1, 0),
                             ("row", 2 * 8184, 72, 2, 1), ("col", 4096, 32, 1, 0)):
        d = tp.tp_shard_plan(kind, K, N, t, r)
        assert tp.tp_workspace_bytes(d, M) > 0, (kind, K, N)
        if kind == "row":
            got, ref = _row_case(kind, K, N, t, r, M, tp.TP_PATH_AUTO)
        else:
            got, ref = _col_case(kind, K, N, t, r, M, tp.TP_PATH_AUTO)
        assert_parity(got, ref, f"{kind} K={K} N={N} M={M}")


@pytest.mark.parametrize("M", [1, 64, 200])
def test_attention_kinds_small(M):
    say("qkv/o small", M)
    heads = (8, 2, 16)
    for t in (1, 2, 4, 8):
        for r in range(t):
            got, ref = _col_case("qkv_col", 64, (8 + 4) * 16, t, r, M, tp.TP_PATH_AUTO, heads)
            assert_parity(got, ref, f"qkv t={t} r={r}")
            got, ref = _row_case("o_row", 8 * 16, 40, t, r, M, tp.TP_PATH_AUTO, heads)
            assert_parity(got, ref, f"o t={t} r={r}")


def test_m_zero_is_a_noop():
    d = tp.tp_shard_plan("col", 64, 64, 1, 0)
    Wp = tp.tp_shard_pack(d, dev(si.normal_bf16(1, (64, 64), 1.0)))
    Y = torch.full((0, 64), 7.0, dtype=torch.bfloat16, device="cuda")
    tp.tp_col_linear(d, torch.empty((0, 64), dtype=torch.bfloat16, device="cuda"), Wp, Y)
    r = tp.tp_shard_plan("row", 64, 64, 1, 0)
    tp.tp_row_linear(r, torch.empty((0, 64), dtype=torch.bfloat16, device="cuda"), Wp)


# ---------------------------------------------------------------------------
# Exact inputs: bit-exact on the GPU.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M", [1, 8, 64, 130])
@pytest.mark.parametrize("path", PATHS)
def test_exact_integers_bit_exact(M, path):
    """X, W in {-3..3}: every fp32 partial sum is an integer below 2^24, so the
    GPU's sums are exact in any order and must match the oracle bit for bit
    (the bf16 rounding of an exact integer is the same on both sides)."""
    say("exact ints", M, path)
    K, N, t = 4096, 512, 4
    X = si.int_bf16(50, (M, K), -3, 3)
    W = si.int_bf16(51, (K, N), -3, 3)
    W2 = si.int_bf16(52, (N, K), -3, 3)
    Ps, Ps_ref = [], []
    for r in range(t):
        dc, pc = plan_both("col", K, N, t, r)
        dc = with_path(dc, path)
        Y = tp.tp_col_linear(dc, dev(X), tp.tp_shard_pack(dc, dev(W)))
        want_y = oracle.col_linear_bf16(X, W, pc)
        np.testing.assert_array_equal(host_bits(Y), want_y)
        dr, pr = plan_both("row", N, K, t, r)
        dr = with_path(dr, path)
        P = tp.tp_row_linear(dr, Y, tp.tp_shard_pack(dr, dev(W2)))
        Ps_ref.append(oracle.row_linear(want_y, W2, pr))
        np.testing.assert_array_equal(host_f64(P), Ps_ref[-1])
        Ps.append(P)
    Yr = tp.tp_reduce_partials(torch.stack(Ps))
    np.testing.assert_array_equal(host_f64(Yr), oracle.sum_partials(np.stack(Ps_ref)))


@pytest.mark.parametrize("M", [5, 64, 100])
def test_identity_weight_bit_exact(M):
    say("identity", M)
    n = 256
    X = si.normal_bf16(60, (M, n), 1.0)
    I = si.identity_bf16(n)
    parts = []
    for t in (1, 4):
        for r in range(t):
            dc, pc = plan_both("col", n, n, t, r)
            Y = tp.tp_col_linear(dc, dev(X), tp.tp_shard_pack(dc, dev(I)))
            np.testing.assert_array_equal(host_bits(Y), X[:, pc["cols"]])
            dr, pr = plan_both("row", n, n, t, r)
            parts.append(tp.tp_row_linear(dr, dev(X[:, pr["rows"]]), tp.tp_shard_pack(dr, dev(I))))
        Y = tp.tp_reduce_partials(torch.stack(parts[-t:]))
        np.testing.assert_array_equal(host_f64(Y), si.bf16_bits_to_f32(X).astype(np.float64))


def test_permutation_weight_bit_exact():
    X = si.normal_bf16(61, (70, 128), 1.0)
    W, perm = si.permutation_bf16(62, 128)
    d = tp.tp_shard_plan("col", 128, 128, 1, 0)
    for path in PATHS:
        Y = tp.tp_col_linear(with_path(d, path), dev(X), tp.tp_shard_pack(d, dev(W)))
        np.testing.assert_array_equal(host_bits(Y), X[:, perm])


# ---------------------------------------------------------------------------
# Reduction.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("t", [1, 2, 3, 8, 16])
@pytest.mark.parametrize("M,N", [(1, 8), (7, 4100), (64, 8192)])
def test_reduce_partials(t, M, N):
    say("reduce", t, M, N)
    P = si.normal_f32(t * 1000 + M, (t * M, N), 1.0).reshape(t, M, N)
    want = oracle.sum_partials(P.astype(np.float64))
    Pd = torch.from_numpy(P).cuda()
    got = host_f64(tp.tp_reduce_partials(Pd))
    assert_parity(got, want, "reduce")
    # fp32 rank-order sum is exactly what a sequential fp32 loop gives
    seq = P[0].copy()
    for r in range(1, t):
        seq = seq + P[r]
    np.testing.assert_array_equal(got, seq.astype(np.float64))
    tp.tp_reduce_partials(Pd, Y=Pd[0])  # in place into slot 0
    np.testing.assert_array_equal(host_f64(Pd[0]), got)


@pytest.mark.parametrize("t", [1, 2, 3, 8, 16])
@pytest.mark.parametrize("Mt,N", [(1, 8), (3, 4100), (8, 8192)])
def test_reduce_scatter_partials(t, Mt, N):
    """Sequence-parallel partial sum: each rank's token rows of the rank-order
    sum, bit for bit the rows of the full sum, within tolerance of the oracle,
    and exact against it on integer-valued partials."""
    say("reduce-scatter", t, Mt, N)
    M = t * Mt
    P = si.normal_f32(t * 2000 + Mt, (t * M, N), 1.0).reshape(t, M, N)
    Pd = torch.from_numpy(P).cuda()
    full = tp.tp_reduce_partials(Pd)
    Pi = si.int_bf16(t * 3000 + Mt, (t * M, N), -256, 256)
    Pi = oracle.bf16_to_f64(Pi).reshape(t, M, N)
    Pid = torch.from_numpy(Pi.astype(np.float32)).cuda()
    for r in range(t):
        Y = tp.tp_reduce_scatter_partials(Pd, r)
        assert Y.shape == (Mt, N)
        assert torch.equal(Y, full[r * Mt:(r + 1) * Mt]), r
        assert_parity(host_f64(Y), oracle.reduce_scatter(P.astype(np.float64), r), f"rank {r}")
        np.testing.assert_array_equal(host_f64(tp.tp_reduce_scatter_partials(Pid, r)),
                                      oracle.reduce_scatter(Pi, r))
    # into a column slice of a wider buffer
    wide = torch.zeros((Mt, N + 8), dtype=torch.float32, device="cuda")
    tp.tp_reduce_scatter_partials(Pd, t - 1, Y=wide[:, 4:4 + N])
    assert torch.equal(wide[:, 4:4 + N], full[(t - 1) * Mt:])
    assert not wide[:, :4].any() and not wide[:, 4 + N:].any()


@pytest.mark.parametrize("t", [1, 2, 3, 8, 16])
@pytest.mark.parametrize("Mt,N", [(1, 8), (5, 4104), (64, 8192)])
def test_gather_rows(t, Mt, N):
    """The row gather: the ranks' bf16 row blocks stacked in rank order, bit-exact."""
    say("gather", t, Mt, N)
    Xs = si.normal_bf16(t * 4000 + Mt, (t * Mt, N), 1.0).reshape(t, Mt, N)
    got = host_bits(tp.tp_gather_rows(dev(Xs)))
    np.testing.assert_array_equal(got, oracle.gather_rows(list(Xs)))


def test_sequence_parallel_round_trip():
    """All-reduce = reduce-scatter then gather: the 70B TP = 8 O-projection
    partials of 256 tokens, reduce-scattered per rank, rounded to bf16 and
    gathered, equal the rounded full sum bit for bit."""
    say("sequence-parallel round trip")
    t, M, N = 8, 256, 8192
    P = torch.from_numpy(si.normal_f32(77, (t * M, N), 1.0).reshape(t, M, N)).cuda()
    blocks = torch.stack([tp.tp_reduce_scatter_partials(P, r) for r in range(t)]).to(torch.bfloat16)
    X = tp.tp_gather_rows(blocks.contiguous())
    assert torch.equal(X, tp.tp_reduce_partials(P).to(torch.bfloat16))


# ---------------------------------------------------------------------------
# The two paths where both are legal, determinism, composition.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M", [16, 64])
def test_decode_and_prefill_agree_at_boundary(M):
    say("boundary", M)
    K, N = 4096, 1024
    X = si.normal_bf16(70, (M, K), 1.0)
    W = si.normal_bf16(71, (K, 2 * N), 0.02)
    d, p = plan_both("gateup_col", K, 2 * N, 2, 1)
    Wp = tp.tp_shard_pack(d, dev(W))
    ref = oracle.bf16_to_f64(oracle.gateup_swiglu(X, W, p))
    a = tp.tp_col_linear(with_path(d, tp.TP_PATH_DECODE), dev(X), Wp)
    b = tp.tp_col_linear(with_path(d, tp.TP_PATH_PREFILL), dev(X), Wp)
    assert_parity(host_f64(a), ref, "decode")
    assert_parity(host_f64(b), ref, "prefill")
    assert_parity(host_f64(a), host_f64(b), "decode vs prefill")


def _bits(t: torch.Tensor) -> torch.Tensor:
    return t.cpu().view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


def test_repeat_runs_are_bit_identical():
    K, N = 4096, 2048
    X = dev(si.normal_bf16(80, (48, K), 1.0))
    W = dev(si.normal_bf16(81, (K, N), 0.02))
    for kind, path in (("col", tp.TP_PATH_DECODE), ("col", tp.TP_PATH_PREFILL),
                       ("row", tp.TP_PATH_DECODE), ("row", tp.TP_PATH_PREFILL)):
        d = with_path(tp.tp_shard_plan(kind, K, N, 2, 1), path)
        Wp = tp.tp_shard_pack(d, W)
        f = tp.tp_col_linear if kind == "col" else tp.tp_row_linear
        x = X if kind == "col" else X[:, :d.shard_k].contiguous()
        assert torch.equal(_bits(f(d, x, Wp)), _bits(f(d, x, Wp))), (kind, path)


def test_ffn_shard_is_col_then_row_and_ldy_slices():
    K, inter, t = 512, 384, 3
    X = si.normal_bf16(90, (9, K), 1.0)
    Wgu = si.normal_bf16(91, (K, 2 * inter), 0.05)
    Wd = si.normal_bf16(92, (inter, K), 0.05)
    for r in range(t):
        gu = tp.tp_shard_plan("gateup_col", K, 2 * inter, t, r)
        dn = tp.tp_shard_plan("row", inter, K, t, r)
        gp, dp = tp.tp_shard_pack(gu, dev(Wgu)), tp.tp_shard_pack(dn, dev(Wd))
        H, P = tp.tp_ffn_shard(gu, dn, dev(X), gp, dp)
        H2 = tp.tp_col_linear(gu, dev(X), gp)
        P2 = tp.tp_row_linear(dn, H2, dp)
        assert torch.equal(H.view(torch.int16), H2.view(torch.int16))
        assert torch.equal(P.view(torch.int32), P2.view(torch.int32))
    # column outputs written through ldy into a wider buffer: concatenation
    W = si.normal_bf16(93, (K, 256), 0.05)
    full = torch.full((9, 256 + 8), 5.0, dtype=torch.bfloat16, device="cuda")
    for r in range(2):
        d = tp.tp_shard_plan("col", K, 256, 2, r)
        tp.tp_col_linear(d, dev(X), tp.tp_shard_pack(d, dev(W)), Y=full[:, r * 128:(r + 1) * 128])
    p1 = oracle.plan("col", K, 256, 1, 0)
    assert_parity(host_f64(full[:, :256]), oracle.bf16_to_f64(oracle.col_linear_bf16(X, W, p1)), "concat")
    assert torch.all(full[:, 256:] == 5.0)


# Prefill epilogues write 16-byte pieces of whole rows; an output width that
# is a multiple of 8 but not of 16, 32 or 128 leaves a half-filled last tile
# and a partly valid last piece of each wave's columns. Each case writes into
# the top-left [M x out_n] of a larger buffer (wider rows and extra rows hold
# a sentinel) through the big-tile kernel (whole rounds, the tail), the
# 128-token kernel and split K.
BOUNDS_CASES = [("col", 72, 1000, 16300), ("gateup_col", 72, 2 * 1000, 8200), ("row", 72, 1000, 16300),
                ("col", 200, 1000, 300), ("gateup_col", 200, 2 * 1000, 300), ("row", 200, 1000, 300),
                ("row", 4096, 1000, 1000), ("gateup_col", 4096, 2 * 1000, 1000)]


@pytest.mark.parametrize("kind,K,N,M", BOUNDS_CASES)
def test_prefill_outputs_stay_in_bounds(kind, K, N, M):
    say("prefill bounds", kind, K, N, M)
    X = si.normal_bf16(94, (M, K), 1.0)
    W = si.normal_bf16(95, (K, N), 0.05)
    d, p = plan_both(kind, K, N, 1, 0)
    d = with_path(d, tp.TP_PATH_PREFILL)
    Wp = tp.tp_shard_pack(d, dev(W))
    wide, extra = d.out_n + 24, 5
    rows = sorted({0, 1, 31, 32, M // 2, M - 33, M - 2, M - 1})
    if kind == "row":
        sentinel = 12345.0
        full = torch.full((M + extra, wide), sentinel, dtype=torch.float32, device="cuda")
        tp.tp_row_linear(d, dev(X), Wp, P=full[:M, :d.out_n])
        ref = oracle.row_linear(np.ascontiguousarray(X[rows]), W, p)
    else:
        sentinel = 5.0
        full = torch.full((M + extra, wide), sentinel, dtype=torch.bfloat16, device="cuda")
        tp.tp_col_linear(d, dev(X), Wp, Y=full[:M, :d.out_n])
        fn = oracle.gateup_swiglu if kind == "gateup_col" else oracle.col_linear_bf16
        ref = oracle.bf16_to_f64(fn(np.ascontiguousarray(X[rows]), W, p))
    torch.cuda.synchronize()
    assert torch.all(full[:M, d.out_n:] == sentinel), "a write landed right of the output columns"
    assert torch.all(full[M:] == sentinel), "a write landed below the last token row"
    assert_parity(host_f64(full[:M, :d.out_n][rows]), ref, f"{kind} K={K} N={N} M={M}")


# ---------------------------------------------------------------------------
# The model-shaped workloads at full size.
# ---------------------------------------------------------------------------

def test_worked_tp2_split_full():
    """X [8 x 4096]; W 4096 x 4096 cut into two 4096 x 2048 column shards; W2
    4096 x 4096 cut into two 2048 x 4096 row shards; both ranks in turn on one
    GPU; partials summed; against the unsharded bf16(X W) W2."""
    say("worked TP=2 full")
    X, W, W2 = wl.worked_tp2()
    Xd, Wd_, W2d = dev(X), dev(W), dev(W2)
    P = torch.empty((2, 8, 4096), dtype=torch.float32, device="cuda")
    Ys = []
    for r in range(2):
        dc, pc = plan_both("col", 4096, 4096, 2, r)
        dr, pr = plan_both("row", 4096, 4096, 2, r)
        assert (dc.shard_k, dc.shard_n, dr.shard_k, dr.shard_n) == (4096, 2048, 2048, 4096)
        Y = tp.tp_col_linear(dc, Xd, tp.tp_shard_pack(dc, Wd_))
        tp.tp_row_linear(dr, Y, tp.tp_shard_pack(dr, W2d), P=P[r])
        assert_parity(host_f64(Y), oracle.bf16_to_f64(oracle.col_linear_bf16(X, W, pc)), f"Y_{r}")
        Ys.append(host_f64(Y))
    out = host_f64(tp.tp_reduce_partials(P))
    Yref = oracle.col_linear_bf16(X, W, oracle.plan("col", 4096, 4096, 1, 0))
    ref = oracle.row_linear(Yref, W2, oracle.plan("row", 4096, 4096, 1, 0))
    assert_parity(np.concatenate(Ys, axis=1), oracle.bf16_to_f64(Yref), "concat Y")
    assert_parity(out, ref, "sum of partials vs unsharded")


@pytest.fixture(scope="module")
def llama8b():
    c = wl.LLAMA8B
    H, I = c["hidden"], c["inter"]
    X = wl.activations(64, H)
    Wgu = wl.gateup(H, I, c["sigma"])
    Wd = wl.down(I, H, c["sigma"])
    gu, pgu = plan_both("gateup_col", H, 2 * I, 1, 0)
    dn, pdn = plan_both("row", I, H, 1, 0)
    gp = tp.tp_shard_pack(gu, dev(Wgu))
    dp = tp.tp_shard_pack(dn, dev(Wd))
    torch.cuda.synchronize()
    yield dict(X=X, Wgu=Wgu, Wd=Wd, gu=gu, dn=dn, pgu=pgu, pdn=pdn, gp=gp, dp=dp)
    del gp, dp
    torch.cuda.empty_cache()


@pytest.mark.parametrize("M", [1, 8, 32, 64])
def test_llama8b_ffn_tp1_decode(llama8b, M):
    say("llama8b ffn", M)
    w = llama8b
    X = w["X"][:M]
    H, P = tp.tp_ffn_shard(w["gu"], w["dn"], dev(X), w["gp"], w["dp"])
    Y = tp.tp_reduce_partials(P.unsqueeze(0))
    Href, Pref = oracle.ffn_shard(X, w["Wgu"], w["Wd"], w["pgu"], w["pdn"])
    assert_parity(host_f64(H), oracle.bf16_to_f64(Href), "H")
    assert_parity(host_f64(P), Pref, "P")
    np.testing.assert_array_equal(host_f64(Y), host_f64(P))  # t = 1: the sum is the partial


@pytest.mark.parametrize("M", [96, 384, 513, 768, 1024])
def test_llama8b_ffn_tp1_batches(llama8b, M):
    """The 8B share at the batch sizes between decode and full prefill (the
    128-token kernel with split K up to 512 tokens; big tiles, a half-tile
    tail and split K beyond): the first and last rows and two rows of every
    128-token tile of H and P against the oracle."""
    say("llama8b ffn batch", M)
    w = llama8b
    X = wl.activations(M, wl.LLAMA8B["hidden"])
    H, P = tp.tp_ffn_shard(w["gu"], w["dn"], dev(X), w["gp"], w["dp"])
    rows = sorted({0, M - 1} | set(range(5, M, 128)) | set(range(100, M, 128)))
    Href, Pref = oracle.ffn_shard(np.ascontiguousarray(X[rows]), w["Wgu"], w["Wd"], w["pgu"], w["pdn"])
    assert_parity(host_f64(H[rows]), oracle.bf16_to_f64(Href), f"H M={M}")
    assert_parity(host_f64(P[rows]), Pref, f"P M={M}")


@pytest.fixture(scope="module")
def llama70b_ffn():
    c = wl.LLAMA70B
    H, I, t = c["hidden"], c["inter"], 8
    X = wl.activations(32, H)
    Wgu = wl.gateup(H, I, c["sigma"])
    Wd = wl.down(I, H, c["sigma"])
    Wgu_d, Wd_d = dev(Wgu), dev(Wd)
    ranks = []
    for r in range(t):
        gu, pgu = plan_both("gateup_col", H, 2 * I, t, r)
        dn, pdn = plan_both("row", I, H, t, r)
        assert (gu.shard_k, gu.shard_n, dn.shard_k, dn.shard_n) == (8192, 7168, 3584, 8192)
        ranks.append(dict(gu=gu, dn=dn, pgu=pgu, pdn=pdn, gp=tp.tp_shard_pack(gu, Wgu_d),
                          dp=tp.tp_shard_pack(dn, Wd_d)))
    del Wgu_d, Wd_d
    torch.cuda.synchronize()
    yield dict(X=X, Wgu=Wgu, Wd=Wd, ranks=ranks, t=t)
    ranks.clear()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("M", [1, 8, 32])
def test_llama70b_ffn_tp8_all_ranks(llama70b_ffn, M):
    say("llama70b ffn tp8", M)
    w = llama70b_ffn
    X = w["X"][:M]
    Xd = dev(X)
    P = torch.empty((w["t"], M, 8192), dtype=torch.float32, device="cuda")
    for r, rk in enumerate(w["ranks"]):
        tp.tp_ffn_shard(rk["gu"], rk["dn"], Xd, rk["gp"], rk["dp"], P=P[r])
    Y = host_f64(tp.tp_reduce_partials(P))
    rk = w["ranks"][0]
    H0, P0 = oracle.ffn_shard(X, w["Wgu"], w["Wd"], rk["pgu"], rk["pdn"])
    assert_parity(host_f64(P[0]), P0, "rank 0 partial")
    rows = list(range(M)) if M <= 8 else [0, 5, 17, 31]
    ref = oracle.ffn_unsharded(X[rows], w["Wgu"], w["Wd"])
    assert_parity(Y[rows], ref, "sum over 8 ranks vs unsharded FFN")


@pytest.mark.parametrize("M", [1536, 2048])
def test_llama70b_ffn_tp8_prefill_unfilled_grids(llama70b_ffn, M):
    """70B shares of TP = 8 at 1536 and 2048 tokens, whose gate/up grids of
    168 and 224 big tiles run on the 128-token kernel: rank 3's H and P and
    the sum over all 8 ranks against the oracle on sampled rows."""
    say("llama70b ffn tp8 prefill", M)
    w = llama70b_ffn
    X = wl.activations(M, wl.LLAMA70B["hidden"])
    Xd = dev(X)
    P = torch.empty((w["t"], M, 8192), dtype=torch.float32, device="cuda")
    Hs = []
    for r, rk in enumerate(w["ranks"]):
        H, _ = tp.tp_ffn_shard(rk["gu"], rk["dn"], Xd, rk["gp"], rk["dp"], P=P[r])
        if r == 3:
            Hs.append(H)
    Y = tp.tp_reduce_partials(P)
    rows = sorted({0, M - 1} | set(range(7, M, 256)) | set(range(200, M, 256)))
    rk = w["ranks"][3]
    H3, P3 = oracle.ffn_shard(np.ascontiguousarray(X[rows]), w["Wgu"], w["Wd"], rk["pgu"], rk["pdn"])
    assert_parity(host_f64(Hs[0][rows]), oracle.bf16_to_f64(H3), f"rank 3 H M={M}")
    assert_parity(host_f64(P[3][rows]), P3, f"rank 3 partial M={M}")
    ref = oracle.ffn_unsharded(np.ascontiguousarray(X[rows]), w["Wgu"], w["Wd"])
    assert_parity(host_f64(Y[rows]), ref, f"sum over 8 ranks vs unsharded FFN M={M}")


SAMPLE_ROWS_4096 = [0, 1, 15, 16, 127, 128, 129, 1000, 2047, 2048, 3071, 4094, 4095]


def test_llama70b_attention_tp8_prefill():
    """Every rank's QKV column slice (8 Q + 1 K + 1 V head: 8192 x 1280) and O
    row slice (1024 x 8192) at 4096 tokens, each against its share of the
    oracle, and the O partials of all 8 ranks summed against the unsharded
    projection, on sampled rows."""
    say("llama70b attention tp8 prefill")
    c = wl.LLAMA70B
    heads = (c["n_q"], c["n_kv"], c["head_dim"])
    Hd, t, M = c["hidden"], 8, 4096
    X = wl.activations(M, Hd)
    A = wl.attention_output(M, c["n_q"] * c["head_dim"])
    Wqkv = wl.qkv_weight(Hd, *heads, c["sigma"])
    Wo = wl.o_weight(c["n_q"], c["head_dim"], Hd, c["sigma"])
    Xd, Ad, Wqkv_d, Wo_d = dev(X), dev(A), dev(Wqkv), dev(Wo)
    rows = SAMPLE_ROWS_4096
    P = torch.empty((t, M, Hd), dtype=torch.float32, device="cuda")
    for r in range(t):
        dq, pq = plan_both("qkv_col", Hd, Wqkv.shape[1], t, r, heads)
        do, po = plan_both("o_row", c["n_q"] * c["head_dim"], Hd, t, r, heads)
        assert (dq.shard_n, do.shard_k) == (1280, 1024)
        QKV = tp.tp_col_linear(dq, Xd, tp.tp_shard_pack(dq, Wqkv_d))
        Ar = Ad[:, do.row_begin:do.row_end].contiguous()
        tp.tp_row_linear(do, Ar, tp.tp_shard_pack(do, Wo_d), P=P[r])
        got = host_f64(QKV)[rows]
        assert_parity(got, oracle.bf16_to_f64(oracle.col_linear_bf16(X[rows], Wqkv, pq)), f"QKV_{r}")
        assert_parity(host_f64(P[r])[rows], oracle.row_linear(A[rows][:, po["rows"]], Wo, po), f"O_{r}")
    Y = host_f64(tp.tp_reduce_partials(P))[rows]
    ref = oracle.row_linear(A[rows], Wo, oracle.plan("o_row", 8192, 8192, 1, 0, heads=heads))
    assert_parity(Y, ref, "O partials summed over 8 ranks vs unsharded")


def _rows_405b(M=8192, tile=256, per_tile=4, seed=405):
    """A seeded 128-row subset touching every one of the 32 token tiles of 256
    rows: each tile's first and last row and two drawn rows in between."""
    rng = np.random.default_rng(seed)
    rows = []
    for t0 in range(0, M, tile):
        mid = rng.choice(np.arange(t0 + 1, t0 + tile - 1), per_tile - 2, replace=False)
        rows += [t0, *sorted(int(x) for x in mid), t0 + tile - 1]
    return rows


@pytest.fixture(scope="module")
def llama405b_ffn():
    """The 405B feed-forward layer at 8192 tokens, TP = 8: all 8 rank shares
    in turn (each packed from the full weights, in the launch configuration
    the benchmark times), their partials kept, and their on-device sum."""
    say("llama405b ffn tp8, 8 ranks at 8192 tokens: generating the full layer")
    c = wl.LLAMA405B
    Hd, I, t, M = c["hidden"], c["inter"], 8, 8192
    X = wl.activations(M, Hd)
    Wgu = wl.gateup(Hd, I, c["sigma"])   # the full [Wg | Wu], 16384 x 106496
    Wd = wl.down(I, Hd, c["sigma"])      # 53248 x 16384
    Xd, Wgud, Wdd = dev(X), dev(Wgu), dev(Wd)
    P = torch.empty((t, M, Hd), dtype=torch.float32, device="cuda")
    H0 = None
    for r in range(t):
        say(f"llama405b ffn tp8 rank {r}")
        gu = tp.tp_shard_plan("gateup_col", Hd, 2 * I, t, r)
        dn = tp.tp_shard_plan("row", I, Hd, t, r)
        assert (gu.shard_k, gu.shard_n, dn.shard_k, dn.shard_n) == (16384, 13312, 6656, 16384)
        gp, dp = tp.tp_shard_pack(gu, Wgud), tp.tp_shard_pack(dn, Wdd)
        Hr, _ = tp.tp_ffn_shard(gu, dn, Xd, gp, dp, P=P[r])
        if r == 0:
            H0 = Hr
        del gp, dp
    del Wgud, Wdd
    say("llama405b ffn tp8: sum of 8 partials")
    Y = tp.tp_reduce_partials(P)
    rows = _rows_405b(M)
    torch.cuda.synchronize()
    out = dict(X=X, Wgu=Wgu, Wd=Wd, rows=rows, Hd=Hd, I=I, t=t,
               H0=host_f64(H0)[rows], P0=host_f64(P[0])[rows], Y=host_f64(Y)[rows])
    del P, Y, H0
    torch.cuda.empty_cache()
    return out


@pytest.mark.timeout(900)
def test_llama405b_ffn_tp8_rank0_prefill(llama405b_ffn):
    """Rank 0's share (gate/up 16384 x 13312 with SwiGLU, down 6656 x 16384,
    fp32 partial) on the 128 sampled rows, against its share of the oracle."""
    f = llama405b_ffn
    Hd, I, t, rows = f["Hd"], f["I"], f["t"], f["rows"]
    pgu, pdn = oracle.plan("gateup_col", Hd, 2 * I, t, 0), oracle.plan("row", I, Hd, t, 0)
    Xs = np.ascontiguousarray(f["X"][rows])
    Href = oracle.gateup_swiglu(Xs, f["Wgu"], pgu)
    assert_parity(f["H0"], oracle.bf16_to_f64(Href), "H_0")
    assert_parity(f["P0"], oracle.row_linear(Href, f["Wd"], pdn), "P_0")


@pytest.mark.timeout(900)
def test_llama405b_ffn_tp8_all_ranks_sum_to_unsharded(llama405b_ffn):
    """The invariant at prefill size ("Tensor Parallelism" glossary, "Full
    definition"; "Tensor vs Pipeline Parallelism", "Tensor parallelism: split
    inside each layer"): the 8 ranks' partials, summed on the GPU, equal the
    unsharded feed-forward layer (t = 1) on the 128 sampled rows."""
    f = llama405b_ffn
    say("llama405b ffn: unsharded oracle on 128 rows")
    ref = oracle.ffn_unsharded(np.ascontiguousarray(f["X"][f["rows"]]), f["Wgu"], f["Wd"])
    assert_parity(f["Y"], ref, "405B FFN: 8 partials summed vs unsharded")


def test_binding_rejects_short_packed_buffer():
    """The binding checks the packed buffer against the plan before any kernel
    reads it."""
    d = tp.tp_shard_plan("col", 256, 256, 1, 0)
    X = dev(si.normal_bf16(60, (4, 256), 1.0))
    short = torch.empty(d.packed_bytes - 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        tp.tp_col_linear(d, X, short)


def test_binding_rejects_wrong_output_shapes():
    """Every output the kernels write is checked against the shape the call
    writes before anything is queued: too few rows (writes past the tensor),
    a narrower column slice of a wider buffer (writes into the neighbour's
    columns), and rows that overlap (row stride below the width)."""
    M, K, N, t = 4, 256, 256, 2
    X = dev(si.normal_bf16(63, (M, K), 1.0))
    dc = tp.tp_shard_plan("col", K, N, t, 0)
    dr = tp.tp_shard_plan("row", K, N, t, 0)
    gu = tp.tp_shard_plan("gateup_col", K, 2 * N, t, 0)
    dn = tp.tp_shard_plan("row", N, K, t, 0)
    cp, rp = tp.tp_shard_pack(dc, dev(si.normal_bf16(64, (K, N), 0.05))), \
        tp.tp_shard_pack(dr, dev(si.normal_bf16(65, (K, N), 0.05)))
    gp, np_ = tp.tp_shard_pack(gu, dev(si.normal_bf16(66, (K, 2 * N), 0.05))), \
        tp.tp_shard_pack(dn, dev(si.normal_bf16(67, (N, K), 0.05)))
    bf, f32 = torch.bfloat16, torch.float32
    wide_bf = torch.zeros((M, 4 * N), dtype=bf, device="cuda")
    wide_f = torch.zeros((M, 4 * N), dtype=f32, device="cuda")
    Z = dev(si.normal_bf16(68, (M, dr.shard_k), 1.0))
    bad = [
        lambda: tp.tp_col_linear(dc, X, cp, Y=torch.empty((M - 1, dc.out_n), dtype=bf, device="cuda")),
        lambda: tp.tp_col_linear(dc, X, cp, Y=wide_bf[:, :dc.out_n // 2]),
        lambda: tp.tp_col_linear(dc, X, cp, Y=torch.empty((1, dc.out_n), dtype=bf, device="cuda").expand(M, -1)),
        lambda: tp.tp_row_linear(dr, Z, rp, P=torch.empty((M - 1, N), dtype=f32, device="cuda")),
        lambda: tp.tp_row_linear(dr, Z, rp, P=wide_f[:, :N - 8]),
        lambda: tp.tp_ffn_shard(gu, dn, X, gp, np_, P=torch.empty((M, K - 8), dtype=f32, device="cuda")),
        lambda: tp.tp_ffn_shard(gu, dn, X, gp, np_, P=torch.empty((M - 1, K), dtype=f32, device="cuda")),
        lambda: tp.tp_reduce_partials(torch.zeros((t, M, N), dtype=f32, device="cuda"), Y=wide_f[:M - 1, :N]),
        lambda: tp.tp_reduce_partials(torch.zeros((t, M, N), dtype=f32, device="cuda"), Y=wide_f[:, :N // 2]),
        lambda: tp.tp_reduce_scatter_partials(torch.zeros((t, M, N), dtype=f32, device="cuda"), 1,
                                              Y=wide_f[:M // t - 1, :N]),
        lambda: tp.tp_reduce_scatter_partials(torch.zeros((t, M, N), dtype=f32, device="cuda"), 1,
                                              Y=wide_f[:M // t, :N - 4]),
        lambda: tp.tp_gather_rows(torch.zeros((t, 2, N), dtype=bf, device="cuda"), X=wide_bf[:3, :N]),
        lambda: tp.tp_gather_rows(torch.zeros((t, 2, N), dtype=bf, device="cuda"), X=wide_bf[:, :N - 8]),
    ]
    torch.cuda.synchronize()
    for i, call in enumerate(bad):
        with pytest.raises(ValueError):
            call()
    torch.cuda.synchronize()
    assert not wide_bf.any() and not wide_f.any(), "a rejected call wrote into its output"


def test_binding_rejects_wrong_attention_output_shape():
    heads, t = (16, 4, 64), 2
    q = tp.tp_shard_plan("qkv_col", 256, (16 + 8) * 64, t, 0, heads=heads)
    QKV = dev(si.normal_bf16(69, (2, q.shard_n), 1.0))
    Kc, Vc = tp.tp_kv_cache_new(q, 2, 16)
    kl = torch.tensor([3, 5], dtype=torch.int32, device="cuda")
    sl = torch.tensor([0, 1], dtype=torch.int32, device="cuda")
    nqd = (q.q_head_end - q.q_head_begin) * 64
    wide = torch.zeros((2, 2 * nqd), dtype=torch.bfloat16, device="cuda")
    for A in (wide[:1, :nqd], wide[:, :nqd - 8]):
        with pytest.raises(ValueError):
            tp.tp_attention(q, QKV, 1, kl, sl, Kc, Vc, 16, A=A)
    torch.cuda.synchronize()
    assert not wide.any()


@pytest.mark.parametrize("M", [3, 40, 200])
def test_side_stream_with_library_workspace(M):
    """A call on a caller-given stream (not the current one), with the
    workspace allocated by the binding, matches the oracle."""
    say("side stream", M)
    K, N = 1040, 4096
    Z = si.normal_bf16(61, (M, K), 1.0)
    W = si.normal_bf16(62, (K, N), 0.05)
    d, p = plan_both("row", K, N, 1, 0)
    Wp = tp.tp_shard_pack(d, dev(W))
    Zd = dev(Z)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        P = torch.empty((M, N), dtype=torch.float32, device="cuda")
    tp.tp_row_linear(d, Zd, Wp, P=P, stream=side)
    side.synchronize()
    assert_parity(host_f64(P), oracle.row_linear(Z, W, p), f"side stream M={M}")
