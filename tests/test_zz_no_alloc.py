"""tp_ffn_shard_noalloc: the feed-forward share with its split-K scratch in the
library's static device array instead of a caller workspace. Called through
the C ABI and checked against tp_ffn_shard (same kernels, caller workspace)
bit for bit, and against the oracle, on two calls in a row with the second
smaller; a shape whose scratch exceeds the array is refused on the host; and
captured into a HIP graph, whose replays give the eager call's bits."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
import tensor_transformer_linear_megatron_amd as tp
from tensor_transformer_linear_megatron_amd import _lib
from tputil import assert_parity, dev, host_bits, host_f64, say

VP = ctypes.c_void_p


def _noalloc(gu, dn, X, Wgp, Wdp, H, P):
    lib = _lib.load()
    return lib.tp_ffn_shard_noalloc(ctypes.byref(gu), ctypes.byref(dn), VP(X.data_ptr()), X.size(0), X.stride(0),
                                    VP(Wgp.data_ptr()), VP(Wdp.data_ptr()), VP(H.data_ptr()), VP(P.data_ptr()),
                                    P.stride(0), VP(torch.cuda.current_stream().cuda_stream))


def test_noalloc_refuses_scratch_beyond_its_array():
    """Host-side: a split-K prefill shape needing 47 MiB is refused before
    any GPU work (null pointers are never touched)."""
    gu = tp.tp_shard_plan("gateup_col", 8192, 2 * 1024, 1, 0)
    dn = tp.tp_shard_plan("row", 1024, 8192, 1, 0)
    assert tp.tp_workspace_bytes(gu, 600) > _lib.NOALLOC_SCRATCH_BYTES
    lib = _lib.load()
    st = lib.tp_ffn_shard_noalloc(ctypes.byref(gu), ctypes.byref(dn), VP(0), 600, 8192, VP(0), VP(0), VP(0), VP(0),
                                  8192, VP(0))
    assert st == _lib.TP_ERR_WORKSPACE


@pytest.mark.gpu
def test_noalloc_matches_ffn_shard_twice_second_smaller():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    K, I, t, r = 4096, 2048, 1, 0
    X = si.normal_bf16(90, (64, K), 1.0)
    Wgu = np.concatenate([si.normal_bf16(91, (K, I), 0.02), si.normal_bf16(92, (K, I), 0.02)], axis=1)
    Wd = si.normal_bf16(93, (I, K), 0.02)
    gu, dn = tp.tp_shard_plan("gateup_col", K, 2 * I, t, r), tp.tp_shard_plan("row", I, K, t, r)
    pgu, pdn = oracle.plan("gateup_col", K, 2 * I, t, r), oracle.plan("row", I, K, t, r)
    Wgp, Wdp = tp.tp_shard_pack(gu, dev(Wgu)), tp.tp_shard_pack(dn, dev(Wd))
    Xd = dev(X)
    for M in (64, 40):
        need = max(tp.tp_workspace_bytes(gu, M), tp.tp_workspace_bytes(dn, M))
        assert 0 < need <= _lib.NOALLOC_SCRATCH_BYTES  # the split-K path runs and uses the scratch
        say(f"noalloc ffn M={M} K={K} I={I} scratch {need} bytes")
        Xm = Xd[:M]
        H = torch.empty((M, I), dtype=torch.bfloat16, device="cuda")
        P = torch.empty((M, K), dtype=torch.float32, device="cuda")
        st = _noalloc(gu, dn, Xm, Wgp, Wdp, H, P)
        assert st == _lib.TP_OK, tp.tp_status_str(st)
        Hw, Pw = tp.tp_ffn_shard(gu, dn, Xm, Wgp, Wdp)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host_bits(H), host_bits(Hw))
        np.testing.assert_array_equal(P.cpu().numpy(), Pw.cpu().numpy())
        Href = oracle.gateup_swiglu(X[:M], Wgu, pgu)
        assert_parity(host_f64(H), oracle.bf16_to_f64(Href), f"H M={M}")
        assert_parity(host_f64(P), oracle.row_linear(Href, Wd, pdn), f"P M={M}")


@pytest.mark.gpu
def test_noalloc_under_graph_capture():
    """The callers it is for: captured once into a HIP graph (after one eager
    call, which looks up the scratch array's address) and replayed three
    times, with the outputs overwritten in between; every replay gives the
    eager bits."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    K, I, M = 2048, 1024, 48
    gu, dn = tp.tp_shard_plan("gateup_col", K, 2 * I, 1, 0), tp.tp_shard_plan("row", I, K, 1, 0)
    assert 0 < max(tp.tp_workspace_bytes(gu, M), tp.tp_workspace_bytes(dn, M)) <= _lib.NOALLOC_SCRATCH_BYTES
    Wgp = tp.tp_shard_pack(gu, dev(si.normal_bf16(95, (K, 2 * I), 0.02)))
    Wdp = tp.tp_shard_pack(dn, dev(si.normal_bf16(96, (I, K), 0.02)))
    X = dev(si.normal_bf16(97, (M, K), 1.0))
    H = torch.empty((M, I), dtype=torch.bfloat16, device="cuda")
    P = torch.empty((M, K), dtype=torch.float32, device="cuda")
    say(f"noalloc graph M={M} K={K} I={I}")
    assert _noalloc(gu, dn, X, Wgp, Wdp, H, P) == _lib.TP_OK
    torch.cuda.synchronize()
    want_h, want_p = H.view(torch.int16).clone(), P.view(torch.int32).clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st = _noalloc(gu, dn, X, Wgp, Wdp, H, P)
    assert st == _lib.TP_OK, tp.tp_status_str(st)
    torch.cuda.synchronize()
    for rep in range(3):
        H.view(torch.int16).fill_(0x5A5A)
        P.view(torch.int32).fill_(0x5A5A5A5A)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(H.view(torch.int16), want_h), f"replay {rep}: H differs from the eager call"
        assert torch.equal(P.view(torch.int32), want_p), f"replay {rep}: P differs from the eager call"
