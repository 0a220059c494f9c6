"""Helpers shared by the GPU tests: host <-> device bit transfers, the parity
bar, and a host-side reader of the packed weight layout."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle

# The parity bar for floating-point outputs: relative Frobenius error <= 1e-3
# and max element error <= 1e-2 * max |oracle|.
REL_FRO = 1e-3
MAX_REL = 1e-2


def say(*a):
    """Name the case before GPU work, flushed, so a failure can be traced."""
    print(*a, file=sys.stderr, flush=True)


def dev(bits: np.ndarray) -> torch.Tensor:
    """numpy bf16 bits -> device bf16 tensor (same bits)."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_f64(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.to(torch.float32).cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def assert_parity(got: np.ndarray, ref: np.ndarray, what: str = ""):
    s = oracle.compare(got, ref)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert s["rel_fro"] <= REL_FRO and s["max_err"] <= MAX_REL * s["max_ref"], f"{what}: {s}"
    return s


def full_device(shape, blocks, dtype=torch.bfloat16) -> torch.Tensor:
    """A device tensor of the full logical shape holding only the given
    (row range, col range, bits) blocks; the rest is never read."""
    W = torch.empty(shape, dtype=dtype, device="cuda")
    for rows, cols, bits in blocks:
        W[rows.start:rows.stop, cols.start:cols.stop].copy_(dev(bits))
    return W


def unpack(desc, packed: torch.Tensor) -> np.ndarray:
    """Read the packed tiles back into the logical shard [shard_k x shard_n]:
    tiles come in pairs (2p, 2p + 1) whose k-steps alternate, so tile
    (nt, ks) is 1 KiB at index ((nt // 2) * ksteps + ks) * 2 + nt % 2; lane
    l = 16 g + i holds W[32 ks + 8 g + e][16 nt + i], e = 0..7; for gate/up,
    packed tile 2j is gate tile j and 2j + 1 is up tile j."""
    ks_n = desc.packed_k // 32
    nt_n = desc.packed_n // 16
    assert nt_n % 2 == 0
    q = packed.view(torch.int16).cpu().numpy().view(np.uint16).reshape(nt_n // 2, ks_n, 2, 4, 16, 8)
    p = q.transpose(0, 2, 1, 3, 4, 5).reshape(nt_n, ks_n, 4, 16, 8)
    # -> [nt, i, ks, g, e] -> columns (nt, i), rows (ks, g, e)
    t = p.transpose(0, 3, 1, 2, 4).reshape(nt_n * 16, ks_n * 32)
    if desc.kind == 2:  # gate/up interleaved by tile
        cols = t.reshape(nt_n // 2, 2, 16, -1)
        gate = cols[:, 0].reshape(-1, ks_n * 32)[:desc.out_n]
        up = cols[:, 1].reshape(-1, ks_n * 32)[:desc.out_n]
        t = np.concatenate([gate, up], axis=0)
    return np.ascontiguousarray(t[:desc.shard_n, :desc.shard_k].T)


def unpack8(desc, packed: torch.Tensor):
    """Read an 8-bit packed shard back: (codes uint8 [shard_k x shard_n],
    column scales float32 [shard_n]). Tiles of 16 columns x 64 k, 1 KiB, in
    the same pair-interleaved order as the bf16 layout (k-steps of 64); lane
    l = 16 g + i holds the codes of column 16 nt + i at k = 64 s + 32 h + 8 g + e
    in byte 8 h + e; the packed_n fp32 scales follow the codes."""
    ks_n = desc.packed_k // 64
    nt_n = desc.packed_n // 16
    assert nt_n % 2 == 0 and desc.wformat == 1
    buf = packed.view(torch.uint8).cpu().numpy()
    nc = desc.packed_k * desc.packed_n
    q = buf[:nc].reshape(nt_n // 2, ks_n, 2, 4, 16, 2, 8)          # pair, s, t, g, i, h, e
    t = q.transpose(0, 2, 4, 1, 5, 3, 6).reshape(nt_n * 16, ks_n * 64)  # (nt, i) x (s, h, g, e)
    sc = buf[nc:nc + 4 * desc.packed_n].view(np.float32)
    if desc.kind == 2:  # gate/up interleaved by tile
        cols = t.reshape(nt_n // 2, 2, 16, -1)
        t = np.concatenate([cols[:, 0].reshape(-1, ks_n * 64)[:desc.out_n],
                            cols[:, 1].reshape(-1, ks_n * 64)[:desc.out_n]], axis=0)
        s2 = sc.reshape(nt_n // 2, 2, 16)
        sc = np.concatenate([s2[:, 0].reshape(-1)[:desc.out_n], s2[:, 1].reshape(-1)[:desc.out_n]])
    return np.ascontiguousarray(t[:desc.shard_n, :desc.shard_k].T), np.ascontiguousarray(sc[:desc.shard_n])
