"""The library's calls under HIP graph capture.

Each case runs a decode step eagerly, then captures the same calls once with
torch.cuda.graph and replays the graph several times. Between the replays the
outputs are overwritten by eager work, with synchronisations around it.

- A decode step of both ranks' feed-forward shares at t = 2: column GEMM with
  SwiGLU, then row GEMM, then the sum of the two partials. At M = 8 the
  streaming kernels run; at M = 40 the split form runs, with its workspace
  and fix-up.
- A decode step of the attention core: KV append, then chunked attention
  with the merge.
- A prefill call of the attention core.
- A prefill of one rank's feed-forward share: the 128-token kernel, and the
  big-tile kernel with its tail and a split-K down projection with its fix-up.
- The same share on 8-bit shards: streaming decode, split decode, and prefill
  through the bf16 copy of the shard in the workspace.

Every replay must reproduce the eager result bit for bit. That holds only if
the calls make no host synchronisation, allocation or memset of their own.

A last case queues split-K calls on two streams at once, each with its own
workspace, and checks them against the same calls made one after another:
the calls keep no state of their own between launches.
"""
from __future__ import annotations

import pytest
import torch

import seeded_inputs as si
import tensor_transformer_linear_megatron_amd as tp
from tputil import dev, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def _bits(x: torch.Tensor) -> torch.Tensor:
    return x.view(torch.int16) if x.element_size() == 2 else x.view(torch.int32)


def _check_replays(step, outs, n=3, keep=()):
    """Eager run, capture, then n replays, each against the eager bits.
    ``outs`` are overwritten before each replay; ``keep`` (state the step
    updates in place, such as a cache) is left as it is and compared after
    each replay."""
    step()
    torch.cuda.synchronize()
    want = [_bits(o).clone() for o in outs]
    want_keep = [_bits(o).clone() for o in keep]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(n):
        for o in outs:  # eager work between the replays
            _bits(o).fill_(0x5A5A)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, w) in enumerate(zip(outs, want)):
            assert torch.equal(_bits(o), w), f"replay {rep}, output {i} differs from the eager run"
        for i, (o, w) in enumerate(zip(keep, want_keep)):
            assert torch.equal(_bits(o), w), f"replay {rep}, state {i} differs from the eager run"


@pytest.mark.parametrize("M", [8, 40])
def test_ffn_decode_step_replays(M):
    say("graph ffn step", M)
    K, inter, t = 1024, 1536, 2
    X = dev(si.normal_bf16(700, (M, K), 1.0))
    Wgu = dev(si.normal_bf16(701, (K, 2 * inter), 0.02))
    Wd = dev(si.normal_bf16(702, (inter, K), 0.02))
    gu = [tp.tp_shard_plan("gateup_col", K, 2 * inter, t, r) for r in range(t)]
    dn = [tp.tp_shard_plan("row", inter, K, t, r) for r in range(t)]
    Pgu = [tp.tp_shard_pack(d, Wgu) for d in gu]
    Pd = [tp.tp_shard_pack(d, Wd) for d in dn]
    need = max(tp.tp_workspace_bytes(d, M) for d in gu + dn)
    if M == 40:
        assert need > 0  # the split form, with its workspace and fix-up
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    H = torch.empty((t, M, inter // t), dtype=torch.bfloat16, device="cuda")
    P = torch.empty((t, M, K), dtype=torch.float32, device="cuda")
    Y = torch.empty((M, K), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()

    def step():
        for r in range(t):
            tp.tp_ffn_shard(gu[r], dn[r], X, Pgu[r], Pd[r], H=H[r], P=P[r], ws=ws)
        tp.tp_reduce_partials(P, Y=Y)

    _check_replays(step, [H, P, Y])
    assert torch.isfinite(Y).all()


def _attention_inputs(S, q_len, kv_len, L_max, seed):
    heads = (64, 8, 128)
    q = tp.tp_shard_plan("qkv_col", 256, (64 + 16) * 128, 8, 0, heads=heads)
    nq, d = q.q_head_end - q.q_head_begin, heads[2]
    QKV = dev(si.normal_bf16(seed, (S * q_len, q.shard_n), 1.0))
    Kc, Vc = tp.tp_kv_cache_new(q, S, L_max)
    Kc.copy_(dev(si.normal_bf16(seed + 1, (S * L_max, d), 1.0)).view(Kc.shape))
    Vc.copy_(dev(si.normal_bf16(seed + 2, (S * L_max, d), 1.0)).view(Vc.shape))
    kl = torch.tensor(kv_len, dtype=torch.int32, device="cuda")
    sl = torch.arange(S, dtype=torch.int32, device="cuda")
    A = torch.empty((S * q_len, nq * d), dtype=torch.bfloat16, device="cuda")
    return q, QKV, Kc, Vc, kl, sl, A


def test_attention_decode_step_replays():
    say("graph attention decode")
    S, L = 4, 2048
    q, QKV, Kc, Vc, kl, sl, A = _attention_inputs(S, 1, [L, 1500, 700, 1], L, 710)
    need = tp.tp_attention_workspace_bytes(q, S, 1, L)
    assert need > 0  # several chunks per sequence: the merge runs
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()

    def step():
        tp.tp_kv_append(q, QKV, 1, kl, sl, Kc, Vc)
        tp.tp_attention(q, QKV, 1, kl, sl, Kc, Vc, L, A=A, ws=ws)

    _check_replays(step, [A], keep=[Kc, Vc])


def test_attention_prefill_replays():
    say("graph attention prefill")
    S, T = 2, 100
    q, QKV, Kc, Vc, kl, sl, A = _attention_inputs(S, T, [T, T + 37], T + 64, 720)
    assert tp.tp_attention_workspace_bytes(q, S, T, T + 37) == 0
    torch.cuda.synchronize()

    def step():
        tp.tp_kv_append(q, QKV, T, kl, sl, Kc, Vc)
        tp.tp_attention(q, QKV, T, kl, sl, Kc, Vc, T + 37, A=A)

    _check_replays(step, [A], keep=[Kc, Vc])


@pytest.mark.parametrize("M", [300, 4100])
def test_ffn_prefill_step_replays(M):
    """A prefill of one rank's feed-forward share: at 300 tokens the 128-token
    kernel; at 4100 the big-tile gate/up GEMM (a whole round and its tail)
    and the down GEMM with K split, its workspace and fix-up."""
    say("graph ffn prefill", M)
    K, inter = 512, 2048
    X = dev(si.normal_bf16(730, (M, K), 1.0))
    Wgu = dev(si.normal_bf16(731, (K, 2 * inter), 0.02))
    Wd = dev(si.normal_bf16(732, (inter, K), 0.02))
    gu = tp.tp_shard_plan("gateup_col", K, 2 * inter, 1, 0)
    dn = tp.tp_shard_plan("row", inter, K, 1, 0)
    Pgu, Pd = tp.tp_shard_pack(gu, Wgu), tp.tp_shard_pack(dn, Wd)
    need = max(tp.tp_workspace_bytes(gu, M), tp.tp_workspace_bytes(dn, M))
    if M == 4100:
        assert need > 0  # the down projection splits K
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    H = torch.empty((M, inter), dtype=torch.bfloat16, device="cuda")
    P = torch.empty((M, K), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()

    def step():
        tp.tp_ffn_shard(gu, dn, X, Pgu, Pd, H=H, P=P, ws=ws)

    _check_replays(step, [H, P])
    assert torch.isfinite(P).all()


def test_two_streams_do_not_interfere():
    """Split-K calls (decode at 40 tokens, prefill at 1000) queued on two
    streams at once, each with its own workspace, give the bits of the same
    calls made one after another."""
    say("two streams")
    K, N = 4096, 1024
    d = tp.tp_shard_plan("row", K, N, 1, 0)
    Wp = tp.tp_shard_pack(d, dev(si.normal_bf16(740, (K, N), 0.02)))
    cases = [(40, 741), (1000, 742), (40, 743), (1000, 744)]
    Xs = [dev(si.normal_bf16(seed, (M, K), 1.0)) for M, seed in cases]
    want = [_bits(tp.tp_row_linear(d, X, Wp)).clone() for X in Xs]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    wss = [torch.empty(max(tp.tp_workspace_bytes(d, M), 16), dtype=torch.uint8, device="cuda") for M, _ in cases]
    outs = [torch.empty((M, N), dtype=torch.float32, device="cuda") for M, _ in cases]
    torch.cuda.synchronize()
    for rep in range(3):
        for i, X in enumerate(Xs):
            with torch.cuda.stream(streams[i % 2]):
                tp.tp_row_linear(d, X, Wp, P=outs[i], ws=wss[i], stream=streams[i % 2])
        torch.cuda.synchronize()
        for i, (o, w) in enumerate(zip(outs, want)):
            assert torch.equal(_bits(o), w), f"round {rep}, call {i} differs from the sequential run"


@pytest.mark.parametrize("M", [8, 40, 300])
def test_ffn_8bit_steps_replay(M):
    """One rank's feed-forward share on 8-bit shards: the streaming decode
    kernel (8 tokens), the split shared-token kernel with its fix-up (40),
    and prefill through the bf16 copy in the workspace (300)."""
    say("graph ffn 8-bit", M)
    K, inter = 1024, 1536
    X = dev(si.normal_bf16(750, (M, K), 1.0))
    gu = tp.tp_shard_set_wformat(tp.tp_shard_plan("gateup_col", K, 2 * inter, 2, 1), "fp8_e4m3")
    dn = tp.tp_shard_set_wformat(tp.tp_shard_plan("row", inter, K, 2, 1), "fp8_e4m3")
    Pgu = tp.tp_shard_pack(gu, dev(si.normal_bf16(751, (K, 2 * inter), 0.02)))
    Pd = tp.tp_shard_pack(dn, dev(si.normal_bf16(752, (inter, K), 0.02)))
    need = max(tp.tp_workspace_bytes(gu, M), tp.tp_workspace_bytes(dn, M))
    if M > 16:
        assert need > 0  # split partials, or the prefill's bf16 copy of the shard
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    H = torch.empty((M, inter // 2), dtype=torch.bfloat16, device="cuda")
    P = torch.empty((M, K), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()

    def step():
        tp.tp_ffn_shard(gu, dn, X, Pgu, Pd, H=H, P=P, ws=ws)

    _check_replays(step, [H, P])
    assert torch.isfinite(P).all()
