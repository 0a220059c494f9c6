"""Pins for the fp64 oracle: each test checks it against something other than
itself -- values and rules the pages fix, closed forms, exact integer
arithmetic, an independent rational or high-precision computation, a library
routine for the t = 1 special case, or brute force on tiny shapes.

Page citations name the page title and the section.
"""
from __future__ import annotations

import decimal
import math
import struct
import types
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si

U53 = 2.0 ** -53


# ---------------------------------------------------------------------------
# Independent references (pure Python, no oracle code).
# ---------------------------------------------------------------------------

_BF16_MAX = Fraction(255) * Fraction(2) ** 120


def exact_round_bf16(x: float) -> int:
    """bf16 bits of x, round to nearest, ties to even, by exact rational
    arithmetic: 8 significant bits, binary32 exponent range."""
    if math.isnan(x):
        return 0x7FC0
    sign = 0x8000 if math.copysign(1.0, x) < 0 else 0
    if math.isinf(x):
        return sign | 0x7F80
    a = Fraction(abs(x))
    if a == 0:
        return sign
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    quantum = Fraction(2) ** max(e - 7, -133)
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    v = fl * quantum
    if v > _BF16_MAX:
        return sign | 0x7F80
    return sign | (struct.unpack(">I", struct.pack(">f", float(v)))[0] >> 16)


def bits_to_float(b: int) -> float:
    return struct.unpack(">f", struct.pack(">I", (b & 0xFFFF) << 16))[0]


def decode(bits: np.ndarray) -> np.ndarray:
    """bf16 bits -> float64 through torch's own bfloat16 type."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def reassoc_bound(Xf: np.ndarray, Wf: np.ndarray, terms: int) -> np.ndarray:
    """Two fp64 sums of the same products in different association differ by
    at most 2 * gamma_n * sum |x||w| (Higham, Accuracy and Stability, 3.1)."""
    g = terms * U53 / (1 - terms * U53)
    return 2 * g * (np.abs(Xf) @ np.abs(Wf))


def normal(seed, shape, sigma=1.0):
    return si.normal_bf16(seed, shape, sigma)


# ---------------------------------------------------------------------------
# bf16 conversions.
# ---------------------------------------------------------------------------

def test_bf16_decode_matches_torch():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = (bits & 0x7F80) != 0x7F80
    got = oracle.bf16_to_f64(bits[finite])
    np.testing.assert_array_equal(got, decode(bits[finite]))


def _rounding_cases():
    rng = np.random.default_rng(123)
    xs = list(rng.standard_normal(3000) * np.exp2(rng.integers(-140, 128, 3000)))
    # exact ties between adjacent bf16 values, and one fp64 ulp on either side
    for b in rng.integers(0, 0x7F7F, 400):
        lo, hi = bits_to_float(int(b)), bits_to_float(int(b) + 1)
        mid = (lo + hi) / 2  # exact: 9 significant bits
        xs += [mid, -mid, math.nextafter(mid, math.inf), math.nextafter(mid, -math.inf)]
    xs += [0.0, -0.0, 1e-45, 3e-40, -1.1e-38, 2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -135,
           3.3895313892515355e38, 3.3961e38, 3.4e38, -3.5e38, 1e300, math.inf, -math.inf]
    return xs


def test_bf16_round_matches_exact_rational():
    xs = _rounding_cases()
    got = oracle.round_bf16(np.array(xs, dtype=np.float64))
    want = np.array([exact_round_bf16(x) for x in xs], dtype=np.uint16)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(xs[i], hex(got[i]), hex(want[i])) for i in bad[:5]]


def test_bf16_round_matches_torch_from_binary32():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal(1 << 16) * np.exp2(rng.integers(-120, 120, 1 << 16))).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(oracle.round_bf16(x.astype(np.float64)), want)


# ---------------------------------------------------------------------------
# The matmul core.
# ---------------------------------------------------------------------------

def test_exact_integers_match_int64_matmul():
    # X, W in {-3..3}: every product and partial sum is an integer, exact in fp64
    X = si.int_bf16(11, (7, 200), -3, 3)
    W = si.int_bf16(12, (200, 48), -3, 3)
    Xi = decode(X).astype(np.int64)
    Wi = decode(W).astype(np.int64)
    got = oracle.shard_matmul(X, W, np.arange(200), np.arange(48))
    np.testing.assert_array_equal(got, (Xi @ Wi).astype(np.float64))
    # a gathered shard: columns in a scrambled order, rows a sub-range
    cols = np.array([5, 0, 47, 13, 13, 30])
    rows = np.arange(50, 150)
    got = oracle.shard_matmul(X[:, 50:150], W, rows, cols)
    np.testing.assert_array_equal(got, (Xi[:, 50:150] @ Wi[50:150][:, cols]).astype(np.float64))


def test_t1_matches_torch_fp64_matmul():
    X, W = normal(0, (16, 300)), normal(1, (300, 200), 0.02)
    got = oracle.shard_matmul(X, W, np.arange(300), np.arange(200))
    want = (torch.from_numpy(decode(X)) @ torch.from_numpy(decode(W))).numpy()
    assert np.linalg.norm(got - want) <= 1e-12 * np.linalg.norm(want)


def _brute(Xf, Wf):
    """Plain in-order dot products with Python floats (fp64)."""
    M, K = len(Xf), len(Xf[0])
    N = len(Wf[0])
    out = []
    for m in range(M):
        row = []
        for n in range(N):
            acc = 0.0
            for k in range(K):
                acc = acc + Xf[m][k] * Wf[k][n]
            row.append(acc)
        out.append(row)
    return np.array(out)


@pytest.mark.parametrize("K,N", [(k, n) for k in (1, 2, 3, 4, 6, 12) for n in (1, 2, 4, 6, 9, 12)])
def test_brute_force_tiny_shapes(K, N):
    X, W = normal(2, (3, K)), normal(3, (K, N), 0.5)
    Xf, Wf = decode(X).tolist(), decode(W).tolist()
    for t in range(1, 13):
        if N % t == 0:  # column shards: the rank's slice of output columns
            w = N // t
            for r in range(t):
                p = oracle.plan("col", K, N, t, r)
                got = oracle.col_linear(X, W, p)
                want = _brute(Xf, [row[r * w:(r + 1) * w] for row in Wf])
                np.testing.assert_array_equal(got, want)
        if K % t == 0:  # row shards: the rank's input slice times its rows of W
            h = K // t
            for r in range(t):
                p = oracle.plan("row", K, N, t, r)
                got = oracle.row_linear(X[:, r * h:(r + 1) * h], W, p)
                want = _brute([row[r * h:(r + 1) * h] for row in Xf], Wf[r * h:(r + 1) * h])
                np.testing.assert_array_equal(got, want)


def test_identity_weight():
    X = normal(4, (6, 64))
    Xf = decode(X)
    I = si.identity_bf16(64)
    for t in (1, 2, 4, 8):
        parts = []
        for r in range(t):
            pc = oracle.plan("col", 64, 64, t, r)
            np.testing.assert_array_equal(oracle.col_linear_bf16(X, I, pc), X[:, pc["cols"]])
            pr = oracle.plan("row", 64, 64, t, r)
            parts.append(oracle.row_linear(X[:, pr["rows"]], I, pr))
        np.testing.assert_array_equal(oracle.sum_partials(np.stack(parts)), Xf)


def test_permutation_weight_selects_columns():
    X = normal(5, (5, 96))
    W, perm = si.permutation_bf16(9, 96)
    p = oracle.plan("col", 96, 96, 1, 0)
    np.testing.assert_array_equal(oracle.col_linear_bf16(X, W, p), X[:, perm])


def test_sum_partials_in_rank_order():
    # 1e16 + 1 loses the 1 in fp64, so only the rank order 0, 1, 2 gives 0
    P = np.array([[1e16], [1.0], [-1e16]])
    assert oracle.sum_partials(P)[0] == 0.0
    assert oracle.sum_partials(P[[1, 0, 2]])[0] == 0.0
    assert oracle.sum_partials(P[[0, 2, 1]])[0] == 1.0


# ---------------------------------------------------------------------------
# Sequence-parallel partial sum and row gather ("AI Infrastructure series,
# Part 5", "What about MoE models and very long prompts?").
# ---------------------------------------------------------------------------

def test_reduce_scatter_brute_force():
    rng = np.random.default_rng(5)
    t, M, N = 4, 12, 5
    P = rng.standard_normal((t, M, N))
    for r in range(t):
        got = oracle.reduce_scatter(P, r)
        assert got.shape == (M // t, N)
        for i in range(M // t):
            for n in range(N):
                acc = 0.0
                for s_ in range(t):  # plain Python floats, rank order
                    acc += float(P[s_, r * (M // t) + i, n])
                assert got[i, n] == acc


def test_reduce_scatter_then_gather_is_the_full_sum():
    # all-reduce = reduce-scatter along the rows followed by the row gather,
    # bit for bit: each element is the same rank-order sum
    rng = np.random.default_rng(6)
    for t, M, N in ((1, 3, 4), (2, 8, 3), (8, 64, 16), (3, 9, 2)):
        P = rng.standard_normal((t, M, N)) * 10.0 ** rng.integers(-3, 4, size=(t, M, N))
        parts = [oracle.reduce_scatter(P, r) for r in range(t)]
        assert np.array_equal(oracle.gather_rows(parts), oracle.sum_partials(P))


def test_reduce_scatter_exact_integers():
    rng = np.random.default_rng(7)
    P = rng.integers(-1000, 1000, size=(8, 32, 24))
    for r in range(8):
        want = P[:, r * 4:(r + 1) * 4].sum(axis=0)  # int64, exact
        assert np.array_equal(oracle.reduce_scatter(P.astype(np.float64), r), want.astype(np.float64))


def test_reduce_scatter_keeps_rank_order():
    # row 1 of rank 1's block holds the 1e16 cancellation; only order 0, 1, 2 gives 0
    P = np.zeros((3, 6, 1))
    P[:, 3, 0] = [1e16, 1.0, -1e16]
    assert oracle.reduce_scatter(P, 1)[1, 0] == 0.0
    assert oracle.reduce_scatter(P[[0, 2, 1]], 1)[1, 0] == 1.0


def test_reduce_scatter_errors():
    P = np.zeros((4, 10, 2))
    with pytest.raises(oracle.PlanError) as e:
        oracle.reduce_scatter(P, 0)  # 10 rows over 4 ranks
    assert e.value.code == "indivisible"
    with pytest.raises(oracle.PlanError) as e:
        oracle.reduce_scatter(np.zeros((4, 8, 2)), 4)
    assert e.value.code == "rank"


def test_gather_rows_restores_the_activations():
    X = si.normal_bf16(21, (24, 40), 1.0)
    for t in (1, 2, 3, 4, 8):
        blocks = [X[r * (24 // t):(r + 1) * (24 // t)] for r in range(t)]
        assert np.array_equal(oracle.gather_rows(blocks), X)
    # a gather in the wrong rank order is caught
    blocks = [X[r * 6:(r + 1) * 6] for r in range(4)]
    assert not np.array_equal(np.concatenate(blocks[::-1], axis=0), X)


# ---------------------------------------------------------------------------
# 8-bit weights ("AI Infrastructure series, Part 5", "Reason 2": a 70B model
# in 8-bit reads 70.6 GB per token). Format reading: OCP FP8 E4M3 with one
# power-of-two scale per output column.
# ---------------------------------------------------------------------------

def _e4m3_exact(code: int) -> Fraction | None:
    """Exact value of an E4M3 code from the format's definition."""
    s, e, m = code >> 7, (code >> 3) & 15, code & 7
    if e == 15 and m == 7:
        return None
    v = Fraction(m, 8) * Fraction(1, 64) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
    return -v if s else v


def test_e4m3_decode_closed_forms():
    d = oracle.e4m3_decode(np.arange(256))
    for c in range(256):
        want = _e4m3_exact(c)
        if want is None:
            assert math.isnan(d[c]), hex(c)
        else:
            assert Fraction(d[c]) == want, hex(c)
    assert d[0x7E] == 448.0 and d[0x08] == 2.0 ** -6 and d[0x01] == 2.0 ** -9 and d[0x00] == 0.0
    assert math.copysign(1.0, d[0x80]) < 0 and d[0x80] == 0.0
    # a library routine: torch's float8_e4m3fn type
    t = torch.from_numpy(np.arange(256, dtype=np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(d), np.isnan(t)) and np.array_equal(d[~np.isnan(d)], t[~np.isnan(t)])


def test_e4m3_round_against_torch_on_every_bf16_value():
    # every bf16 value within +-448: one rounding from binary32 in torch's cast
    bits = np.arange(65536, dtype=np.uint32)
    f = ((bits << 16).astype(np.uint32)).view(np.float32)
    f = f[np.isfinite(f) & (np.abs(f) <= 448.0)]
    want = torch.from_numpy(f).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_round(f.astype(np.float64)), want)


def test_e4m3_round_midpoints_tie_to_even():
    d = oracle.e4m3_decode(np.arange(0x7F))
    for c in range(0x7E):
        mid = (d[c] + d[c + 1]) / 2  # exact in fp64
        even = c if c % 2 == 0 else c + 1
        assert oracle.e4m3_round(np.array([mid]))[0] == even, hex(c)
        assert oracle.e4m3_round(np.array([-mid]))[0] == even | 0x80, hex(c)
        # just off the midpoint, the nearest code wins, by exact rational comparison
        for x in (np.nextafter(mid, 0), np.nextafter(mid, 1000)):
            got = oracle.e4m3_round(np.array([x]))[0]
            lo, hi = Fraction(d[c]), Fraction(d[c + 1])
            want = c if abs(Fraction(x) - lo) < abs(Fraction(x) - hi) else c + 1
            assert got == want, (hex(c), x)
    # a negative value that rounds to zero keeps its sign
    assert oracle.e4m3_round(np.array([-2.0 ** -11]))[0] == 0x80


def test_column_exponent_rule():
    W = np.array([[448.0, 448.0 * (1 + 2 ** -20), 224.0, 0.0, -3.0e-5, 1.0, 449.0, 2.0 ** -30]])
    e = oracle.column_exponents(W)
    assert list(e) == [0, 1, -1, 0, math.ceil(math.log2(3.0e-5 / 448)), math.ceil(math.log2(1 / 448)), 1, -38]
    rng = np.random.default_rng(8)
    A = rng.standard_normal((64, 500)) * 10.0 ** rng.integers(-8, 8, size=500)
    e = oracle.column_exponents(A).astype(np.float64)
    amax = np.abs(A).max(axis=0)
    assert np.all(amax * np.exp2(-e) <= 448.0) and np.all(amax * np.exp2(-(e - 1)) > 448.0)


def test_dequantised_weight_error_bound():
    # 3 mantissa bits: within half a unit of the code spacing, i.e. 2^-4 relative
    # for normal codes and 2^-10 2^e absolute in the subnormal range
    W = si.normal_bf16(31, (256, 96), 0.02)
    Wf = decode(W)
    q, e = oracle.quantize_columns(Wf)
    Wq = oracle.dequantize_columns(q, e)
    scale = np.exp2(e.astype(np.float64))
    err = np.abs(Wq - Wf)
    assert np.all(err <= np.maximum(np.abs(Wf) * 2.0 ** -4, 2.0 ** -10 * scale))
    assert np.abs(Wq).max(axis=0).max() <= (np.abs(Wf).max(axis=0) * (1 + 2 ** -4)).max()


def test_small_integer_weights_quantise_exactly():
    # integers up to 15 in magnitude have at most 4 significant bits: the 8-bit
    # form is exact, so the 8-bit linear equals the exact integer product
    W = si.int_bf16(32, (64, 48), -15, 15)
    X = si.int_bf16(33, (5, 64), -3, 3)
    p = oracle.plan("col", 64, 48, 1, 0)
    assert np.array_equal(oracle.shard_weight_fp8(W, p), decode(W))
    Xi, Wi = decode(X).astype(np.int64), decode(W).astype(np.int64)
    assert np.array_equal(oracle.col_linear_fp8(X, W, p), (Xi @ Wi).astype(np.float64))


def test_fp8_shards_follow_the_plan():
    # columns are quantised one by one, so 8-bit column shards concatenate to the
    # unsharded 8-bit product; row shards quantise their own rows, so their
    # partials sum to the product with the ranks' dequantised rows stacked
    X, W = normal(34, (6, 128)), normal(35, (128, 96), 0.05)
    full = oracle.col_linear_fp8(X, W, oracle.plan("col", 128, 96, 1, 0))
    Xf = decode(X)
    for t in (2, 4):
        parts = [oracle.col_linear_fp8(X, W, oracle.plan("col", 128, 96, t, r)) for r in range(t)]
        np.testing.assert_allclose(np.concatenate(parts, axis=1), full, rtol=0, atol=1e-12)
        ps = [oracle.plan("row", 128, 96, t, r) for r in range(t)]
        P = sum(oracle.row_linear_fp8(X[:, p["rows"]], W, p) for p in ps)
        Wst = np.concatenate([oracle.shard_weight_fp8(W, p) for p in ps], axis=0)
        bound = reassoc_bound(Xf, np.abs(Wst), 128)
        assert np.all(np.abs(P - Xf @ Wst) <= bound + 1e-300)


def test_planted_round_toward_zero_is_caught():
    # truncating the scaled weights instead of rounding them moves many codes
    bits = np.arange(0, 65536, 7, dtype=np.uint32)
    f32 = ((bits << 16).astype(np.uint32)).view(np.float32)
    f = f32[np.isfinite(f32) & (np.abs(f32) <= 448.0)].astype(np.float64)
    table = oracle.e4m3_decode(np.arange(0x7F))
    trunc = np.searchsorted(table, np.abs(f), side="right") - 1
    assert np.count_nonzero(trunc != (oracle.e4m3_round(f) & 0x7F)) > 100


# ---------------------------------------------------------------------------
# Backward of the rank share ("Tensor vs Pipeline Parallelism", "Tensor
# parallelism: split inside each layer": two more all-reduces per layer in the
# backward pass).
# ---------------------------------------------------------------------------

def _ffn_backward_oracle(X, Wgu, Wd, dY, t):
    """Per rank: (dX_r, dWgu_r, dWd_r) from the oracle's backward pieces, in fp64
    (the gate/up gradient kept unrounded)."""
    H = Wd.shape[0]
    out = []
    for r in range(t):
        pg = oracle.plan("gateup_col", Wgu.shape[0], Wgu.shape[1], t, r)
        pd = oracle.plan("row", H, Wd.shape[1], t, r)
        G, U = oracle.gateup_preact(X, Wgu, pg)
        Hr = oracle.swiglu(G, U)
        dH = oracle.grad_input(dY, Wd, pd)
        dG, dU = oracle.swiglu_backward_f64(G, U, dH)
        dGU = np.concatenate([dG, dU], axis=1)
        Wgu_r = decode(np.ascontiguousarray(Wgu[:, pg["cols"]]))
        out.append((dGU @ Wgu_r.T, decode(X).T @ dGU, oracle.grad_weight(Hr, dY, pd)))
    return out


def test_ffn_backward_against_torch_autograd():
    """A library routine: torch autograd in fp64 on the same feed-forward share
    (loss = sum(P * dY)); the rank's H is used as the oracle rounds it (bf16),
    so the down projection's input matches exactly."""
    X, Wgu, Wd = normal(40, (5, 48)), normal(41, (48, 2 * 32), 0.2), normal(42, (32, 48), 0.2)
    dY = normal(43, (5, 48))
    for t in (1, 2, 4):
        for r, (dX_r, dWgu_r, dWd_r) in enumerate(_ffn_backward_oracle(X, Wgu, Wd, dY, t)):
            pg = oracle.plan("gateup_col", 48, 64, t, r)
            pd = oracle.plan("row", 32, 48, t, r)
            Xt = torch.tensor(decode(X), requires_grad=True)
            Wg = torch.tensor(decode(np.ascontiguousarray(Wgu[:, pg["cols"]])), requires_grad=True)
            Wdt = torch.tensor(decode(np.ascontiguousarray(Wd[pd["rows"]])), requires_grad=True)
            GU = Xt @ Wg
            w = pg["shard_n"] // 2
            Hh = torch.nn.functional.silu(GU[:, :w]) * GU[:, w:]
            Hq = Hh + (torch.tensor(oracle.bf16_to_f64(oracle.swiglu(GU[:, :w].detach().numpy(),
                                                                      GU[:, w:].detach().numpy()))) - Hh).detach()
            (Hq @ Wdt * torch.tensor(decode(dY))).sum().backward()
            np.testing.assert_allclose(dX_r, Xt.grad.numpy(), rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(dWgu_r, Wg.grad.numpy(), rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(dWd_r, Wdt.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_backward_exact_integers():
    """Integer inputs: every product is exact in fp64, so the input and
    weight gradients equal the int64 products exactly."""
    X, W, dC = si.int_bf16(44, (6, 40), -3, 3), si.int_bf16(45, (40, 24), -3, 3), si.int_bf16(46, (6, 24), -3, 3)
    Xi, Wi, dCi = (decode(a).astype(np.int64) for a in (X, W, dC))
    p = oracle.plan("col", 40, 24, 1, 0)
    assert np.array_equal(oracle.grad_input(dC, W, p), (dCi @ Wi.T).astype(np.float64))
    assert np.array_equal(oracle.grad_weight(X, dC, p), (Xi.T @ dCi).astype(np.float64))


def test_backward_shards_add_up():
    """The sum of the ranks' input gradients is the unsharded one (the
    backward all-reduce); the ranks' weight gradients tile the unsharded
    weight gradient (columns for the column kinds, rows for the row kinds)."""
    X, W, dY = normal(47, (7, 64), 1.0), normal(48, (64, 48), 0.1), normal(49, (7, 48), 1.0)
    full_dX = oracle.grad_input(dY, W, oracle.plan("col", 64, 48, 1, 0))
    full_dW = oracle.grad_weight(X, dY, oracle.plan("col", 64, 48, 1, 0))
    Xf, Wf, dYf = decode(X), decode(W), decode(dY)
    for t in (2, 4, 8):
        ps = [oracle.plan("col", 64, 48, t, r) for r in range(t)]
        dX = sum(oracle.grad_input(np.ascontiguousarray(dY[:, p["cols"]]), W, p) for p in ps)
        bound = reassoc_bound(np.abs(dYf), np.abs(Wf.T), 48)
        assert np.all(np.abs(dX - full_dX) <= bound + 1e-300)
        dW = np.concatenate([oracle.grad_weight(X, np.ascontiguousarray(dY[:, p["cols"]]), p) for p in ps], axis=1)
        np.testing.assert_allclose(dW, full_dW, rtol=0, atol=1e-12)
        prs = [oracle.plan("row", 64, 48, t, r) for r in range(t)]
        dWr = np.concatenate([oracle.grad_weight(np.ascontiguousarray(X[:, p["rows"]]), dY, p) for p in prs], axis=0)
        np.testing.assert_allclose(dWr, full_dW, rtol=0, atol=1e-12)
        dZ = np.concatenate([oracle.grad_input(dY, W, p) for p in prs], axis=1)
        np.testing.assert_allclose(dZ, full_dX, rtol=0, atol=1e-12)


def test_swiglu_backward_closed_forms_and_differences():
    # dSiLU/dg at 0 is 1/2; with dH = 1, U = 1: dG(0) = 1/2, dU(0) = 0
    dG, dU = oracle.swiglu_backward_f64(np.array([[0.0]]), np.array([[1.0]]), np.array([[1.0]]))
    assert dG[0, 0] == 0.5 and dU[0, 0] == 0.0
    # far from 0 the derivative tends to 1 (g > 0) and 0 (g < 0); no NaN at the extremes
    dG, dU = oracle.swiglu_backward_f64(np.array([[60.0, -800.0]]), np.ones((1, 2)), np.ones((1, 2)))
    assert abs(dG[0, 0] - 1.0) < 1e-20 and dG[0, 1] == 0.0 and np.isfinite(dU).all()
    # central differences of H = SiLU(g) u against the closed forms
    rng = np.random.default_rng(9)
    g, u, dh = rng.standard_normal(50) * 3, rng.standard_normal(50), rng.standard_normal(50)
    hfun = lambda gg, uu: gg / (1 + np.exp(-gg)) * uu
    eps = 1e-6
    dG, dU = oracle.swiglu_backward_f64(g[None], u[None], dh[None])
    np.testing.assert_allclose(dG[0], dh * (hfun(g + eps, u) - hfun(g - eps, u)) / (2 * eps), rtol=1e-7, atol=1e-9)
    np.testing.assert_allclose(dU[0], dh * (hfun(g, u + eps) - hfun(g, u - eps)) / (2 * eps), rtol=1e-7, atol=1e-9)


def _swiglu_backward_autograd_bits(G, U, dH):
    """[dG | dU] from torch's fp64 autograd of H = silu(G) * U (a library
    routine, no oracle code), each element rounded once by exact rational
    arithmetic."""
    Gt = torch.tensor(G, dtype=torch.float64, requires_grad=True)
    Ut = torch.tensor(U, dtype=torch.float64, requires_grad=True)
    (torch.nn.functional.silu(Gt) * Ut).backward(torch.tensor(dH, dtype=torch.float64))
    both = np.concatenate([Gt.grad.numpy(), Ut.grad.numpy()], axis=1)
    return np.array([[exact_round_bf16(float(v)) for v in row] for row in both], dtype=np.uint16)


def _swiglu_backward_cases():
    rng = np.random.default_rng(21)
    G = decode(si.normal_bf16(50, (7, 12), 3.0))
    G[0, :6] = [0.0, 40.0, -40.0, 89.0, -100.0, 1e-3]  # saturated and near-zero pre-activations
    U = decode(si.normal_bf16(51, (7, 12), 1.0))
    dH = rng.standard_normal((7, 12))
    return G, U, dH


def test_swiglu_backward_bits_match_torch_autograd():
    """oracle.swiglu_backward: the [dG | dU] order (gate half first, the
    order of [Wg | Wu]) and a single bf16 rounding of each fp64 gradient."""
    G, U, dH = _swiglu_backward_cases()
    np.testing.assert_array_equal(oracle.swiglu_backward(G, U, dH), _swiglu_backward_autograd_bits(G, U, dH))


def test_planted_swapped_swiglu_gradients_are_caught():
    """A planted [dU | dG] order in a copy of the oracle fails the pin above."""
    def swapped(G, U, dH):
        dG, dU = oracle.swiglu_backward_f64(G, U, dH)
        return oracle.round_bf16(np.concatenate([dU, dG], axis=1))

    G, U, dH = _swiglu_backward_cases()
    assert not np.array_equal(swapped(G, U, dH), _swiglu_backward_autograd_bits(G, U, dH))


# ---------------------------------------------------------------------------
# The oracle's in-order fp64 product (8-bit shards, gradients, attention).
# ---------------------------------------------------------------------------

def test_matmul_f64_is_the_in_order_sum():
    """Bit for bit a pure-Python loop that adds the products in ascending k
    from 0.0 (Python floats are IEEE fp64 without fused multiply-add), also
    for transposed operands read in place."""
    rng = np.random.default_rng(31)
    A, B = rng.standard_normal((5, 19)), rng.standard_normal((19, 7))
    want = np.empty((5, 7))
    for m in range(5):
        for n in range(7):
            acc = 0.0
            for k in range(19):
                acc += float(A[m, k]) * float(B[k, n])
            want[m, n] = acc
    np.testing.assert_array_equal(oracle.matmul_f64(A, B), want)
    np.testing.assert_array_equal(oracle.matmul_f64(np.ascontiguousarray(A.T).T, np.asfortranarray(B)), want)
    np.testing.assert_array_equal(oracle.matmul_f64(B.T, A.T), want.T)


def test_matmul_f64_exact_integers():
    Ai, Bi = si.int_bf16(52, (9, 300), -3, 3), si.int_bf16(53, (300, 11), -3, 3)
    Ai, Bi = decode(Ai).astype(np.int64), decode(Bi).astype(np.int64)
    assert np.array_equal(oracle.matmul_f64(Ai.astype(np.float64), Bi.astype(np.float64)),
                          (Ai @ Bi).astype(np.float64))
    assert np.array_equal(oracle.matmul_f64(np.zeros((3, 0)), np.zeros((0, 4))), np.zeros((3, 4)))


# ---------------------------------------------------------------------------
# 8-bit gate/up with SwiGLU (oracle.gateup_swiglu_fp8).
# ---------------------------------------------------------------------------

def _gateup_fp8_onehot(K=40, inter=12):
    """[Wg | Wu] whose columns each hold one nonzero weight of at most 3
    significant bits (exact in E4M3 after any power-of-two scale), gate and
    up columns on different rows with different values."""
    rng = np.random.default_rng(22)
    a, b = rng.integers(0, K, inter), rng.integers(0, K, inter)
    b = np.where(a == b, (b + 1) % K, b)
    vals = np.array([1.0, -1.5, 0.75, 1.25, -1.75, 0.5, 3.0, -0.625])
    va, vb = vals[rng.integers(0, len(vals), inter)], vals[rng.integers(0, len(vals), inter)] * 2.0
    W = np.zeros((K, 2 * inter))
    W[a, np.arange(inter)] = va
    W[b, inter + np.arange(inter)] = vb
    bits = np.array([[exact_round_bf16(float(v)) for v in row] for row in W], dtype=np.uint16)
    return bits, a, b, va, vb


def test_gateup_swiglu_fp8_onehot_against_high_precision():
    """With one-hot columns the 8-bit shard is exact, so H[m, j] must be
    bf16(SiLU(x[m, a_j] va_j) * x[m, b_j] vb_j), SiLU on the gate half, for
    every rank's share."""
    K, inter, M = 40, 12, 5
    X = normal(23, (M, K), 2.0)
    Wgu, a, b, va, vb = _gateup_fp8_onehot(K, inter)
    Xf = decode(X)
    for t in (1, 2, 3):
        w = inter // t
        for r in range(t):
            p = oracle.plan("gateup_col", K, 2 * inter, t, r)
            js = range(r * w, (r + 1) * w)
            want = np.array([[_silu_times_u_highprec(Xf[m, a[j]] * va[j], Xf[m, b[j]] * vb[j]) for j in js]
                             for m in range(M)], dtype=np.uint16)
            np.testing.assert_array_equal(oracle.gateup_swiglu_fp8(X, Wgu, p), want)


def _fp8_shard_torch(Wf: np.ndarray) -> np.ndarray:
    """Independent quantiser: scale 2^e per column from Python's frexp, codes
    from torch's float8_e4m3fn cast (round to nearest even), decoded by torch."""
    out = np.empty_like(Wf)
    for n in range(Wf.shape[1]):
        amax = float(np.abs(Wf[:, n]).max())
        e = 0
        if amax > 0:
            f, x = math.frexp(amax)
            e = x - 9 if f <= 0.875 else x - 8
        q = torch.tensor(Wf[:, n] * 2.0 ** -e, dtype=torch.float64).to(torch.float8_e4m3fn)
        out[:, n] = q.to(torch.float64).numpy() * 2.0 ** e
    return out


def _gateup_fp8_reference(X, Wgu, t, r):
    """H of rank r from the independent quantiser, per-half columns, exact
    integer sums (small integers times dyadic weights), decimal SwiGLU."""
    K, N2 = Wgu.shape
    inter = N2 // 2
    w = inter // t
    cols = list(range(r * w, (r + 1) * w))
    Wf = decode(Wgu)
    Wg = _fp8_shard_torch(Wf[:, cols])
    Wu = _fp8_shard_torch(Wf[:, [inter + c for c in cols]])
    Xf = decode(X)
    G = [[math.fsum(Xf[m, k] * Wg[k, j] for k in range(K)) for j in range(w)] for m in range(X.shape[0])]
    U = [[math.fsum(Xf[m, k] * Wu[k, j] for k in range(K)) for j in range(w)] for m in range(X.shape[0])]
    return np.array([[_silu_times_u_highprec(G[m][j], U[m][j]) for j in range(w)] for m in range(X.shape[0])],
                    dtype=np.uint16)


def _gateup_fp8_inputs():
    """Integer activations and weights whose columns need real rounding
    (values that are not E4M3 codes after their column's scale), with gate
    and up columns of very different ranges."""
    X = si.int_bf16(24, (4, 32), -3, 3)
    Wg = si.normal_bf16(25, (32, 8), 0.3)
    Wu = si.normal_bf16(26, (32, 8), 5.0)
    return X, np.concatenate([Wg, Wu], axis=1)


def test_gateup_swiglu_fp8_against_torch_float8():
    X, Wgu = _gateup_fp8_inputs()
    for t, r in ((1, 0), (2, 1), (4, 2)):
        p = oracle.plan("gateup_col", 32, 16, t, r)
        np.testing.assert_array_equal(oracle.gateup_swiglu_fp8(X, Wgu, p), _gateup_fp8_reference(X, Wgu, t, r))


def test_planted_gateup_fp8_half_swap_is_caught():
    """A copy of the oracle's 8-bit gate/up with the halves swapped (SiLU on
    the up products) fails both 8-bit gate/up pins."""
    def swapped(X, Wgu, p):
        Wq = oracle.shard_weight_fp8(Wgu, p)
        half = p["shard_n"] // 2
        Xf = oracle.bf16_to_f64(X)
        return oracle.swiglu(oracle.matmul_f64(Xf, Wq[:, half:]), oracle.matmul_f64(Xf, Wq[:, :half]))

    X, Wgu = _gateup_fp8_inputs()
    p = oracle.plan("gateup_col", 32, 16, 2, 1)
    assert not np.array_equal(swapped(X, Wgu, p), _gateup_fp8_reference(X, Wgu, 2, 1))
    Xo = normal(23, (5, 40), 2.0)
    Wo, a, b, va, vb = _gateup_fp8_onehot()
    po = oracle.plan("gateup_col", 40, 24, 1, 0)
    Xf = decode(Xo)
    want = np.array([[_silu_times_u_highprec(Xf[m, a[j]] * va[j], Xf[m, b[j]] * vb[j]) for j in range(12)]
                     for m in range(5)], dtype=np.uint16)
    assert not np.array_equal(swapped(Xo, Wo, po), want)


# ---------------------------------------------------------------------------
# The parity measure (oracle.compare).
# ---------------------------------------------------------------------------

def test_compare_closed_forms():
    s = oracle.compare(np.array([[3.0, 4.5]]), np.array([[3.0, 4.0]]))
    # diff (0, 0.5): ||diff|| / ||(3, 4)|| = 0.5 / 5
    assert s == dict(rel_fro=0.1, max_err=0.5, max_ref=4.0, max_rel=0.125)
    s = oracle.compare(np.array([1.0, -2.0, 2.0]), np.array([0.0, 0.0, 0.0]))
    assert s["rel_fro"] == 3.0 and s["max_err"] == 2.0 and s["max_ref"] == 0.0
    s = oracle.compare(np.arange(12.0).reshape(3, 4), np.arange(12.0).reshape(3, 4))
    assert s["rel_fro"] == 0.0 and s["max_err"] == 0.0 and s["max_ref"] == 11.0


def test_compare_refuses_shape_mismatch():
    """One row must not stand in for M rows by broadcasting."""
    ref = np.ones((4, 8))
    for got in (np.ones((1, 8)), np.ones(8), np.ones((4, 8, 1)), np.ones((8, 4))):
        with pytest.raises(ValueError):
            oracle.compare(got, ref)


# ---------------------------------------------------------------------------
# SwiGLU.
# ---------------------------------------------------------------------------

def _silu_times_u_highprec(g: float, u: float) -> int:
    with decimal.localcontext() as ctx:
        ctx.prec = 60
        G = decimal.Decimal(g)
        s = G / (1 + (-G).exp()) * decimal.Decimal(u)
    return exact_round_bf16(float(s)) if abs(s) < decimal.Decimal("1e300") else 0


def test_swiglu_closed_forms():
    G = np.array([0.0, 0.0, 1.5, -2.0, 3.0])
    U = np.array([2.0, -7.0, 0.0, 0.0, 1.0])
    H = decode(oracle.swiglu(G, U))
    assert np.all(H[:4] == 0.0)
    # large |g|: SiLU(g) -> g for g -> +inf and -> 0 for g -> -inf, no NaN
    H = decode(oracle.swiglu(np.array([800.0, -800.0, -1e308]), np.array([0.5, 3.0, 1.0])))
    assert H[0] == 400.0 and H[1] == 0.0 and H[2] == 0.0


def test_swiglu_onehot_gate_against_high_precision():
    """With one-hot gate and up columns, G and U equal chosen columns of X
    exactly, so H[m, j] must be bf16(SiLU(x[m, a_j]) * x[m, b_j]) with SiLU
    applied to the gate half (the first half of [Wg | Wu])."""
    K, inter, M = 40, 24, 6
    X = normal(6, (M, K), 2.0)
    rng = np.random.default_rng(1)
    a, b = rng.integers(0, K, inter), rng.integers(0, K, inter)
    Wgu = np.zeros((K, 2 * inter), dtype=np.uint16)
    Wgu[a, np.arange(inter)] = 0x3F80
    Wgu[b, inter + np.arange(inter)] = 0x3F80
    Xf = decode(X)
    for t in (1, 2, 3, 4):
        w = inter // t
        for r in range(t):
            p = oracle.plan("gateup_col", K, 2 * inter, t, r)
            H = oracle.gateup_swiglu(X, Wgu, p)
            js = range(r * w, (r + 1) * w)
            want = np.array([[_silu_times_u_highprec(Xf[m, a[j]], Xf[m, b[j]]) for j in js]
                             for m in range(M)], dtype=np.uint16)
            np.testing.assert_array_equal(H, want)


def test_swiglu_matches_torch_silu_fp64():
    rng = np.random.default_rng(2)
    G = rng.standard_normal(20000) * 4
    U = rng.standard_normal(20000)
    want = torch.nn.functional.silu(torch.from_numpy(G)) * torch.from_numpy(U)
    want_bits = np.array([exact_round_bf16(v) for v in want.numpy()], dtype=np.uint16)
    got = oracle.swiglu(G, U)
    # both round once from an fp64 value; the two exp() may differ by an fp64
    # ulp, which can flip a bf16 decision only next to an exact tie
    assert np.count_nonzero(got != want_bits) <= 2


# ---------------------------------------------------------------------------
# Shard bookkeeping and the sharding invariants.
# ---------------------------------------------------------------------------

def test_worked_tp2_split_shapes(golden):
    g = golden("tp2_worked_split.json")
    K, N = g["W"]
    for r in range(g["t"]):
        p = oracle.plan("col", K, N, g["t"], r)
        assert [p["shard_k"], p["shard_n"]] == g["column_shards"][r]
        assert [int(p["cols"][0]), int(p["cols"][-1]) + 1] == g["column_ranges"][r]
        q = oracle.plan("row", K, N, g["t"], r)
        assert [q["shard_k"], q["shard_n"]] == g["row_shards"][r]
        assert [int(q["rows"][0]), int(q["rows"][-1]) + 1] == g["row_ranges"][r]


def test_head_tables(golden):
    g = golden("heads_64q_8kv.json")
    nq, nkv, d = g["n_q"], g["n_kv"], g["head_dim"]
    assert g["layers"] * nkv * d * 2 * 2 == g["kv_bytes_per_token"]  # K and V, 2 bytes
    N, K = (nq + 2 * nkv) * d, nq * d
    for t in g["accepted_t"]:
        rows = []
        for r in range(t):
            p = oracle.plan("qkv_col", 8192, N, t, r, heads=(nq, nkv, d))
            rows.append([*p["q_heads"], *p["kv_heads"], p["kv_replicated"]])
            o = oracle.plan("o_row", K, 8192, t, r, heads=(nq, nkv, d))
            assert o["shard_k"] == (nq // t) * d and o["rows"][0] == p["q_heads"][0] * d
            # every local query head finds its key-value head locally
            group = nq // nkv
            for q in range(*p["q_heads"]):
                assert p["kv_heads"][0] <= q // group < p["kv_heads"][1]
        assert rows == g["per_rank"][str(t)]
    for t in g["refused_t"]:
        for kind, KK, NN in (("qkv_col", 8192, N), ("o_row", K, 8192)):
            with pytest.raises(oracle.PlanError) as e:
                oracle.plan(kind, KK, NN, t, 0, heads=(nq, nkv, d))
            assert e.value.code == "indivisible"


def test_llama70b_rank_share_qkv_and_o():
    p = oracle.plan("qkv_col", 8192, 10240, 8, 0, heads=(64, 8, 128))
    assert p["shard_n"] == 1280  # 8 Q heads + 1 K + 1 V head of 128
    assert list(p["cols"][[0, 1023, 1024, 1151, 1152, 1279]]) == [0, 1023, 8192, 8319, 9216, 9343]
    o = oracle.plan("o_row", 8192, 8192, 8, 0, heads=(64, 8, 128))
    assert (o["shard_k"], o["shard_n"]) == (1024, 8192)


def test_plan_errors():
    for args, code in [(("col", 64, 60, 8, 0), "indivisible"), (("row", 60, 64, 8, 0), "indivisible"),
                       (("col", 64, 64, 4, 4), "rank"), (("col", 64, 64, 4, -1), "rank"),
                       (("col", 0, 64, 1, 0), "shape"), (("gateup_col", 64, 63, 1, 0), "shape"),
                       (("gateup_col", 64, 96, 32, 0), "indivisible"), (("foo", 8, 8, 1, 0), "kind")]:
        with pytest.raises(oracle.PlanError) as e:
            oracle.plan(*args)
        assert e.value.code == code, args


def test_size_closed_forms(golden):
    g = golden("sizes.json")
    for hidden, nbytes in g["reduce_message"]["cases"]:
        assert oracle.plan("row", 28672, hidden, 8, 0)["shard_n"] * 2 == nbytes
    pm = g["prefill_message"]
    assert pm["tokens"] * oracle.plan("row", 1024, pm["hidden"], 8, 0)["shard_n"] * 2 == pm["bytes"]
    s = g["per_rank_share"]["llama70b_ffn"]
    H, I, t = s["hidden"], s["intermediate"], s["t"]
    total = 0
    for r in range(t):
        gu = oracle.plan("gateup_col", H, 2 * I, t, r)
        dn = oracle.plan("row", I, H, t, r)
        share = (gu["shard_k"] * gu["shard_n"] + dn["shard_k"] * dn["shard_n"]) * 2
        assert share == s["per_rank_bytes"]
        total += share
    assert total == s["total_bytes"] == 3 * H * I * 2


def test_gateup_pairs_same_columns():
    p = oracle.plan("gateup_col", 16, 16, 2, 1)
    assert list(p["cols"]) == [4, 5, 6, 7, 12, 13, 14, 15]


def _concat_invariant(orc, X, W, t):
    K, N = W.shape
    full = orc.col_linear(X, W, orc.plan("col", K, N, 1, 0))
    parts = [orc.col_linear(X, W, orc.plan("col", K, N, t, r)) for r in range(t)]
    np.testing.assert_array_equal(np.concatenate(parts, axis=1), full)


def _row_sum_invariant(orc, Z, W, t):
    K, N = W.shape
    full = orc.row_linear(Z, W, orc.plan("row", K, N, 1, 0))
    parts = []
    for r in range(t):
        p = orc.plan("row", K, N, t, r)
        parts.append(orc.row_linear(Z[:, p["rows"]], W, p))
    got = orc.sum_partials(np.stack(parts))
    assert np.all(np.abs(got - full) <= reassoc_bound(decode(Z), decode(W), K + t))


def _ffn_invariant(orc, X, Wgu, Wd, t):
    K, N2 = Wgu.shape
    I, H = Wd.shape
    want = orc.ffn_unsharded(X, Wgu, Wd)
    H_full = orc.gateup_swiglu(X, Wgu, orc.plan("gateup_col", K, N2, 1, 0))
    parts = []
    for r in range(t):
        Hr, Pr = orc.ffn_shard(X, Wgu, Wd, orc.plan("gateup_col", K, N2, t, r),
                               orc.plan("row", I, H, t, r))
        # each element of H is the same in-order sum, so the shard is bit-exact
        np.testing.assert_array_equal(Hr, H_full[:, r * (I // t):(r + 1) * (I // t)])
        parts.append(Pr)
    got = orc.sum_partials(np.stack(parts))
    assert np.all(np.abs(got - want) <= reassoc_bound(decode(H_full), decode(Wd), I + t))


def test_concat_invariant_small():
    X, W = normal(7, (5, 72)), normal(8, (72, 96), 0.1)
    for t in (1, 2, 3, 4, 6, 8, 12):
        _concat_invariant(oracle, X, W, t)


def test_row_sum_invariant_small():
    Z, W = normal(9, (5, 96), 1.0), normal(10, (96, 40), 0.1)
    for t in (2, 3, 4, 8, 12):
        _row_sum_invariant(oracle, Z, W, t)


def test_ffn_invariant_small():
    X, Wgu, Wd = normal(0, (4, 64)), normal(1, (64, 2 * 48), 0.1), normal(3, (48, 64), 0.1)
    for t in (1, 2, 3, 4, 8):
        _ffn_invariant(oracle, X, Wgu, Wd, t)


@pytest.mark.slow
def test_worked_split_full_size_invariants():
    """The worked TP=2 split at its own size: X [8 x 4096], W and W2 4096 x 4096."""
    X = si.normal_bf16(0, (8, 4096), 1.0)
    W = si.normal_bf16(1, (4096, 4096), 0.02)
    W2 = si.normal_bf16(2, (4096, 4096), 0.02)
    _concat_invariant(oracle, X, W, 2)
    Y = oracle.col_linear_bf16(X, W, oracle.plan("col", 4096, 4096, 1, 0))
    _row_sum_invariant(oracle, Y, W2, 2)


# ---------------------------------------------------------------------------
# The pins bite: a planted mistake in a copy of the oracle fails them.
# ---------------------------------------------------------------------------

def _mutant(**over):
    ns = types.SimpleNamespace(**{k: getattr(oracle, k) for k in dir(oracle) if not k.startswith("__")})
    for k, v in over.items():
        setattr(ns, k, v)
    return ns


def test_planted_contiguous_gateup_cut_is_caught():
    def bad_plan(kind, K, N, t, rank, heads=None):
        p = oracle.plan(kind, K, N, t, rank, heads)
        if kind == "gateup_col":  # a plain 1/t cut of [Wg | Wu]
            w = N // t
            p["cols"] = np.arange(rank * w, rank * w + w, dtype=np.int64)
        return p

    def ffn_shard(X, Wgu, Wd, pg, pd):
        Hh = oracle.gateup_swiglu(X, Wgu, pg)
        return Hh, oracle.row_linear(Hh, Wd, pd)

    X, Wgu, Wd = normal(0, (4, 64)), normal(1, (64, 96), 0.1), normal(3, (48, 64), 0.1)
    with pytest.raises(AssertionError):
        _ffn_invariant(_mutant(plan=bad_plan, ffn_shard=ffn_shard), X, Wgu, Wd, 2)


def test_planted_truncating_round_is_caught():
    xs = _rounding_cases()
    trunc = np.array([struct.unpack(">I", struct.pack(">f", x))[0] >> 16 if abs(x) < 3e38 else 0
                      for x in xs], dtype=np.uint16)
    want = np.array([exact_round_bf16(x) for x in xs], dtype=np.uint16)
    assert np.count_nonzero(trunc != want) > 100
