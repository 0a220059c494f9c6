"""GPU parity of the attention core on a rank's heads and its KV-cache share:
tp_kv_append against the oracle's append (bit-exact), tp_attention against
the fp64 oracle (both rounded once to bf16) on the decode form (split into
chunks of 512 to 4096 positions, merged when there are several) and the
prefill form, on several head layouts: grouped
query heads at t = 2 and 8, a repeated key-value head at t = 16, d = 64 and
128; ragged lengths, a prefill on top of an earlier cache, out-of-range
sequences, and the 70B TP = 8 rank-0 shapes the benchmark times.

Bar: bit-exact for the cache and for outputs the softmax fixes exactly (one
position; equal keys over equal values); relative Frobenius error <= 1e-3 and
max element error <= 1e-2 * max |oracle| otherwise.
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


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def draw(fn, seed, shape, *args):
    return fn(seed, (int(np.prod(shape[:-1])), shape[-1]), *args).reshape(shape)


def i32(x):
    return torch.tensor(list(x), dtype=torch.int32, device="cuda")


def plans(heads, t, r, K=256):
    n_q, n_kv, d = heads
    N = (n_q + 2 * n_kv) * d
    return tp.tp_shard_plan("qkv_col", K, N, t, r, heads=heads), oracle.plan("qkv_col", K, N, t, r, heads=heads)


class Case:
    """Seeded QKV rows and caches with random earlier contents, on both sides."""

    def __init__(self, heads, t, r, q_len, kv_len, slot, n_slots, L_max, seed, sigma_q=1.0):
        self.q, self.p = plans(heads, t, r)
        self.q_len, self.kv_len, self.slot = q_len, list(kv_len), list(slot)
        S = len(kv_len)
        self.QKV = si.normal_bf16(seed, (S * q_len, self.p["shard_n"]), 1.0)
        nq = self.p["q_heads"][1] - self.p["q_heads"][0]
        d = heads[2]
        if sigma_q != 1.0:  # sharper or flatter attention
            self.QKV[:, :nq * d] = si.normal_bf16(seed + 3, (S * q_len, nq * d), sigma_q)
        self.Kh, self.Vh = oracle.kv_cache_new(self.p, n_slots, L_max)
        self.Kh[:] = draw(si.normal_bf16, seed + 1, self.Kh.shape, 1.0)
        self.Vh[:] = draw(si.normal_bf16, seed + 2, self.Vh.shape, 1.0)
        self.Kd, self.Vd = dev(self.Kh), dev(self.Vh)
        self.QKVd = dev(self.QKV)

    def append(self):
        tp.tp_kv_append(self.q, self.QKVd, self.q_len, i32(self.kv_len), i32(self.slot), self.Kd, self.Vd)
        valid = [(k, s) for k, s in zip(self.kv_len, self.slot)]
        # the oracle appends only what is in range, as the library does
        L_max, n_slots = self.Kh.shape[2], self.Kh.shape[0]
        for s, (k, sl) in enumerate(valid):
            if self.q_len <= k <= L_max and 0 <= sl < n_slots:
                rows = self.QKV[s * self.q_len:(s + 1) * self.q_len]
                oracle.kv_append(rows, self.p, self.q_len, [k], [sl], self.Kh, self.Vh)

    def run(self, max_kv=None):
        max_kv = max_kv or max(self.kv_len)
        return tp.tp_attention(self.q, self.QKVd, self.q_len, i32(self.kv_len), i32(self.slot), self.Kd, self.Vd,
                               max_kv)

    def ref(self, rows=None):
        return oracle.attention(self.QKV, self.p, self.q_len, self.kv_len, self.slot, self.Kh, self.Vh, rows)


LAYOUTS = [((64, 8, 128), 8, 0), ((64, 8, 128), 2, 1), ((64, 8, 128), 16, 11), ((16, 4, 64), 2, 1),
           ((16, 2, 64), 8, 7)]


@pytest.mark.parametrize("heads,t,r", LAYOUTS)
def test_append_writes_the_oracles_cache(heads, t, r):
    say("kv append", heads, t, r)
    c = Case(heads, t, r, 5, [5, 300, 77], [2, 0, 3], 4, 320, 400)
    c.append()
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host_bits(c.Kd), c.Kh)
    np.testing.assert_array_equal(host_bits(c.Vd), c.Vh)


def test_append_skips_out_of_range_sequences():
    say("kv append invalid")
    c = Case((64, 8, 128), 8, 0, 3, [3, 2, 400, 50], [0, 1, 2, 7], 4, 320, 410)
    before_k, before_v = c.Kh.copy(), c.Vh.copy()
    c.append()  # only sequence 0 is in range: 2 < q_len, 400 > L_max, slot 7 >= n_slots
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host_bits(c.Kd), c.Kh)
    np.testing.assert_array_equal(host_bits(c.Kd)[1:], before_k[1:])
    np.testing.assert_array_equal(host_bits(c.Vd)[1:], before_v[1:])


@pytest.mark.parametrize("heads,t,r", LAYOUTS)
@pytest.mark.parametrize("q_len", [1, 2])
def test_decode_matches_oracle(heads, t, r, q_len):
    """Ragged cache lengths: one position, less than a chunk, several chunks
    with a ragged last one."""
    say("decode", heads, t, r, q_len)
    c = Case(heads, t, r, q_len, [q_len, 200, 1000, 513], [3, 1, 0, 2], 4, 1024, 420 + q_len)
    c.append()
    A = c.run()
    n_q, n_kv, d = heads
    G = (c.p["q_heads"][1] - c.p["q_heads"][0]) // (c.p["kv_heads"][1] - c.p["kv_heads"][0])
    assert G * q_len <= 16  # the decode form
    assert_parity(host_f64(A), oracle.bf16_to_f64(c.ref()), f"decode {heads} t={t}")


@pytest.mark.parametrize("heads,t,r", LAYOUTS)
@pytest.mark.parametrize("q_len,prior", [(200, 0), (130, 77), (64, 0), (17, 300)])
def test_prefill_matches_oracle(heads, t, r, q_len, prior):
    """Many new tokens: a fresh sequence, a ragged last query block, and new
    tokens on top of an earlier cache (chunked prefill)."""
    say("prefill", heads, t, r, q_len, prior)
    c = Case(heads, t, r, q_len, [q_len + prior, q_len + prior + 33], [1, 0], 2, 512, 440 + q_len)
    G = (c.p["q_heads"][1] - c.p["q_heads"][0]) // (c.p["kv_heads"][1] - c.p["kv_heads"][0])
    if G * q_len <= 16:
        pytest.skip("decode form")
    c.append()
    A = c.run()
    assert_parity(host_f64(A), oracle.bf16_to_f64(c.ref()), f"prefill {heads} t={t} q={q_len}")


@pytest.mark.parametrize("heads,t,r,S,q_len", [((64, 8, 128), 8, 0, 8, 1024), ((16, 4, 64), 2, 1, 4, 1000)])
def test_prefill_two_group_form(heads, t, r, S, q_len):
    """Enough query blocks for the two-group workgroups (1024 units of 64
    tokens, or 512 with chains of at most 16 blocks), on top of ragged earlier
    caches; sampled rows around the 64-token block edges and the ragged end."""
    say("prefill two groups", heads, t, r, S, q_len)
    prior = [0, 77, 300, 5, 64, 1, 200, 31][:S]
    kv = [q_len + p for p in prior]
    c = Case(heads, t, r, q_len, kv, list(range(S))[::-1], S, max(kv), 540 + S)
    c.append()
    A = host_bits(c.run())
    rows = sorted({0, 63, 64, q_len - 1, q_len, q_len + 500, 2 * q_len + 127, S * q_len - 1, (S - 1) * q_len + 960})
    assert_parity(oracle.bf16_to_f64(A[rows]), oracle.bf16_to_f64(c.ref(rows)), f"prefill two groups {heads}")


@pytest.mark.parametrize("q_len", [1, 3, 40])
def test_sharp_and_flat_attention(q_len):
    """Large query scale (nearly one-hot weights) and tiny scale (nearly
    uniform weights)."""
    for sig in (8.0, 0.01):
        say("sharp/flat", q_len, sig)
        c = Case((64, 8, 128), 8, 3, q_len, [q_len + 700, q_len + 5], [0, 1], 2, 800, 460, sigma_q=sig)
        c.append()
        assert_parity(host_f64(c.run()), oracle.bf16_to_f64(c.ref()), f"sigma_q={sig}")


@pytest.mark.parametrize("q_len", [1, 2, 33])
def test_single_position_is_exact(q_len):
    """A sequence whose only visible position is its first token's own: the
    weight is exactly 1 and the output is that value row, bit for bit."""
    say("single position", q_len)
    c = Case((64, 8, 128), 8, 0, q_len, [q_len, q_len], [0, 1], 2, 64, 470)
    c.append()
    got = host_bits(c.run())
    ref = c.ref()
    d = 128
    for s in range(2):
        np.testing.assert_array_equal(got[s * q_len], ref[s * q_len])  # token 0: position 0 only
        for h in range(8):
            np.testing.assert_array_equal(got[s * q_len, h * d:(h + 1) * d], c.Vh[c.slot[s], 0, 0])


@pytest.mark.parametrize("q_len", [1, 40])
def test_equal_keys_over_equal_values_is_exact(q_len):
    """Zero keys give equal weights; a value row repeated at every position is
    then returned exactly, whatever the number of positions."""
    say("equal keys", q_len)
    c = Case((16, 4, 64), 2, 0, q_len, [q_len + 600], [0], 1, 700, 480)
    nq, nkv, d = 8, 2, 64
    c.QKV[:, nq * d:(nq + nkv) * d] = 0  # new keys
    c.Kh[:] = 0
    row = si.normal_bf16(481, (nkv, d), 1.0)
    c.Vh[:] = row[None, :, None, :]
    for i in range(q_len):
        c.QKV[i, (nq + nkv) * d:] = row.reshape(-1)
    c.Kd, c.Vd, c.QKVd = dev(c.Kh), dev(c.Vh), dev(c.QKV)
    c.append()
    got = host_bits(c.run())
    np.testing.assert_array_equal(got, c.ref())
    for h in range(nq):
        np.testing.assert_array_equal(got[:, h * d:(h + 1) * d], np.broadcast_to(row[h // 4], (q_len, d)))


@pytest.mark.parametrize("q_len", [1, 40])
def test_out_of_range_sequence_gives_zero_rows(q_len):
    say("invalid sequence", q_len)
    c = Case((64, 8, 128), 8, 0, q_len, [q_len + 10, q_len + 900, q_len + 5], [0, 1, 5], 2, 128, 490)
    c.append()
    A = host_bits(c.run(max_kv=128))  # sequence 1 exceeds max_kv, sequence 2's slot is out of range
    assert not A[q_len:].any()
    np.testing.assert_allclose(oracle.bf16_to_f64(A[:q_len]), oracle.bf16_to_f64(c.ref(range(q_len))),
                               rtol=1e-2, atol=1e-2)


def test_decode_long_cache_merges_many_chunks():
    """More chunks than the merge keeps in registers (17000 positions = 34
    chunks of 512): the tiled merge path."""
    say("decode long cache")
    c = Case((64, 8, 128), 8, 0, 1, [17000, 300], [1, 0], 2, 17024, 497)
    c.append()
    rows = [0, 1]
    assert_parity(host_f64(c.run())[rows], oracle.bf16_to_f64(c.ref(rows)), "long cache")


def test_max_kv_above_every_length():
    """A larger max_kv only adds empty chunks; one chunk (the output written
    by the chunk's own workgroup) and several (merged by the combine kernel)
    give the same bits."""
    say("max_kv slack")
    c = Case((64, 8, 128), 8, 0, 1, [300, 17], [0, 1], 2, 2048, 495)
    c.append()
    a1 = host_bits(c.run(max_kv=300))
    a2 = host_bits(c.run(max_kv=2048))
    np.testing.assert_array_equal(a1, a2)


@pytest.mark.parametrize("heads,t,r,S,L,chunk", [
    ((64, 8, 128), 8, 0, 128, 2048, 1024), ((64, 8, 128), 8, 0, 64, 4096, 1024),
    ((64, 8, 128), 8, 0, 128, 4096, 2048), ((64, 8, 128), 8, 0, 256, 4096, 4096),
    ((64, 8, 128), 8, 0, 32, 32768, 4096), ((64, 8, 128), 8, 0, 300, 700, 1024),
    ((16, 4, 64), 2, 1, 128, 4096, 4096), ((16, 4, 64), 2, 1, 32, 4096, 1024)])
def test_decode_longer_chunks_for_large_batches(heads, t, r, S, L, chunk):
    """Many (sequence, key-value head) pairs: each workgroup takes 2, 4 or 8
    passes of 512 positions, or the whole cache (no combine); ragged lengths
    around the chunk edges; d = 128 and 64. Sampled rows."""
    say("decode large batch", heads, S, L)
    q, p = plans(heads, t, r)
    nkv = p["kv_heads"][1] - p["kv_heads"][0]
    part = (16 * heads[2] + 32) * 4
    n_chunks = -(-L // chunk)
    assert tp.tp_attention_workspace_bytes(q, S, 1, L) == (S * nkv * n_chunks * part if n_chunks > 1 else 0)
    rng = np.random.default_rng(S + L)
    kv = [int(x) for x in rng.integers(1, L + 1, S)]
    kv[0], kv[-1] = L, min(L, chunk + 1)
    kv[1] = min(L, chunk)
    c = Case(heads, t, r, 1, kv, list(range(S)), S, L, 530)
    c.append()
    A = host_bits(c.run(max_kv=L))
    rows = sorted({0, 1, S // 2, S - 1})
    assert_parity(oracle.bf16_to_f64(A[rows]), oracle.bf16_to_f64(c.ref(rows)), f"decode {heads} {S} x {L}")


# ---------------------------------------------------------------------------
# Llama-3.1-70B attention, rank 0 of TP = 8 (8 query heads, 1 key-value head,
# d = 128), in the benchmark's launch shapes; sampled rows.
# ---------------------------------------------------------------------------

def _random_attention_cases(n=16, seed=77):
    """Seeded random calls: a head layout, 1 to 3 sequences in shuffled cache
    slots, each with its own cache length, and new-token counts on both sides
    of the decode / prefill choice."""
    rng = np.random.default_rng(seed)
    cases = []
    for c in range(n):
        heads, t, r = LAYOUTS[int(rng.integers(0, len(LAYOUTS)))]
        q_len = int(rng.choice([1, 2, 3, 5, 16, 17, 64, 100, 250]))
        S = int(rng.integers(1, 4))
        L_max = q_len + int(rng.integers(0, 1500))
        kv_len = [int(rng.integers(q_len, L_max + 1)) for _ in range(S)]
        n_slots = S + int(rng.integers(0, 3))
        slot = [int(x) for x in rng.permutation(n_slots)[:S]]
        cases.append((heads, t, r, q_len, kv_len, slot, n_slots, L_max))
    return cases


@pytest.mark.parametrize("heads,t,r,q_len,kv_len,slot,n_slots,L_max", _random_attention_cases())
def test_random_calls_match_oracle(heads, t, r, q_len, kv_len, slot, n_slots, L_max):
    """Append then attend, against the oracle: the caches bit-exact, the
    output on every row (or 48 seeded rows of larger calls)."""
    say("random attention", heads, t, r, q_len, kv_len, slot, n_slots, L_max)
    c = Case(heads, t, r, q_len, kv_len, slot, n_slots, L_max, 900 + q_len + L_max % 97)
    c.append()
    A = host_bits(c.run())
    np.testing.assert_array_equal(host_bits(c.Kd), c.Kh)
    np.testing.assert_array_equal(host_bits(c.Vd), c.Vh)
    M = len(kv_len) * q_len
    rows = list(range(M)) if M <= 64 else sorted(int(x) for x in np.random.default_rng(M).choice(M, 48, replace=False))
    assert_parity(oracle.bf16_to_f64(A[rows]), oracle.bf16_to_f64(c.ref(rows)),
                  f"heads={heads} t={t} r={r} q_len={q_len} kv={kv_len}")


def test_llama70b_tp8_decode_batch():
    """32 sequences, one new token each, 4096 cached positions."""
    say("70b decode 32 x 4096")
    S, L = 32, 4096
    c = Case((64, 8, 128), 8, 0, 1, [L] * S, list(range(S)), S, L, 500)
    c.append()
    A = host_bits(c.run())
    rows = [0, 7, 31]
    np.testing.assert_array_equal(A.shape, (32, 1024))
    assert_parity(oracle.bf16_to_f64(A[rows]), oracle.bf16_to_f64(c.ref(rows)), "70b decode")


def test_llama70b_tp8_prefill_4096():
    say("70b prefill 4096")
    T = 4096
    c = Case((64, 8, 128), 8, 0, T, [T], [0], 1, T, 510)
    c.append()
    A = host_bits(c.run())
    rows = [0, 1, 127, 128, 2047, 4000, 4095]
    assert_parity(oracle.bf16_to_f64(A[rows]), oracle.bf16_to_f64(c.ref(rows)), "70b prefill")


# ---------------------------------------------------------------------------
# The whole attention block of a layer, each rank's share through the
# library, on a prefill chunk and then two decode steps.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("t", [2, 4])
def test_attention_block_all_ranks(t):
    """X -> QKV slice -> append -> attention -> O slice (fp32 partial), for
    every rank, then the sum over the ranks; on a 40-token prefill of two
    sequences and two decode steps after it. Compared with the oracle taking
    the same steps, and with the unsharded block (t = 1) computed the same way
    by the oracle."""
    heads, hidden = (8, 2, 64), 192
    n_q, n_kv, d = heads
    S, T0, L = 2, 40, 64
    Wq = si.normal_bf16(600, (hidden, (n_q + 2 * n_kv) * d), 0.08)
    Wo = si.normal_bf16(601, (n_q * d, hidden), 0.08)
    steps = [(T0, si.normal_bf16(602, (S * T0, hidden), 1.0)),
             (1, si.normal_bf16(603, (S, hidden), 1.0)),
             (1, si.normal_bf16(604, (S, hidden), 1.0))]
    Wqd, Wod = dev(Wq), dev(Wo)
    ranks = []
    for r in range(t):
        q = tp.tp_shard_plan("qkv_col", hidden, Wq.shape[1], t, r, heads=heads)
        o = tp.tp_shard_plan("o_row", n_q * d, hidden, t, r, heads=heads)
        pq = oracle.plan("qkv_col", hidden, Wq.shape[1], t, r, heads=heads)
        po = oracle.plan("o_row", n_q * d, hidden, t, r, heads=heads)
        Kd, Vd = tp.tp_kv_cache_new(q, S, L)
        Kh, Vh = oracle.kv_cache_new(pq, S, L)
        ranks.append(dict(q=q, o=o, pq=pq, po=po, qp=tp.tp_shard_pack(q, Wqd), op=tp.tp_shard_pack(o, Wod),
                          Kd=Kd, Vd=Vd, Kh=Kh, Vh=Vh))
    p1 = oracle.plan("qkv_col", hidden, Wq.shape[1], 1, 0, heads=heads)
    o1 = oracle.plan("o_row", n_q * d, hidden, 1, 0, heads=heads)
    K1, V1 = oracle.kv_cache_new(p1, S, L)
    slot = [1, 0]
    pos = 0
    for q_len, X in steps:
        say("attention block", t, q_len)
        pos += q_len
        kv_len = [pos] * S
        P = torch.empty((t, S * q_len, hidden), dtype=torch.float32, device="cuda")
        ref = np.zeros((S * q_len, hidden))
        Xd = dev(X)
        for r, R in enumerate(ranks):
            QKV = tp.tp_col_linear(R["q"], Xd, R["qp"])
            tp.tp_kv_append(R["q"], QKV, q_len, i32(kv_len), i32(slot), R["Kd"], R["Vd"])
            A = tp.tp_attention(R["q"], QKV, q_len, i32(kv_len), i32(slot), R["Kd"], R["Vd"], L)
            tp.tp_row_linear(R["o"], A, R["op"], P=P[r])
            # the oracle, step by step
            QKVh = oracle.col_linear_bf16(X, Wq, R["pq"])
            oracle.kv_append(QKVh, R["pq"], q_len, kv_len, slot, R["Kh"], R["Vh"])
            Ah = oracle.attention(QKVh, R["pq"], q_len, kv_len, slot, R["Kh"], R["Vh"])
            ref += oracle.row_linear(Ah, Wo, R["po"])
            assert_parity(host_f64(QKV), oracle.bf16_to_f64(QKVh), f"QKV_{r}")
            assert_parity(host_f64(A), oracle.bf16_to_f64(Ah), f"A_{r}")
        Y = host_f64(tp.tp_reduce_partials(P))
        assert_parity(Y, ref, f"block t={t} q_len={q_len}")
        # the unsharded layer: the heads concatenate, so the block is the same
        QKV1 = oracle.col_linear_bf16(X, Wq, p1)
        oracle.kv_append(QKV1, p1, q_len, kv_len, slot, K1, V1)
        Y1 = oracle.row_linear(oracle.attention(QKV1, p1, q_len, kv_len, slot, K1, V1), Wo, o1)
        assert_parity(Y, Y1, f"block t={t} vs unsharded")
