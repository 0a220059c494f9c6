"""Synthetic workloads shaped like the pages' models (input recipes only).

Shapes: hidden 8192 and 80 layers for the 70B model ("Tensor vs Pipeline
Parallelism", "A worked communication estimate"); 64 query heads and 8
key-value heads ("AI Infrastructure series, Part 5", "How does tensor
parallelism split a layer?"); head_dim 128 from the 320 KB of KV cache per
token (same page, "How do you choose a layout for serving?"); hidden 16384
for 405B from the 32 KB per-token hand-off (same page, pipeline section).
The feed-forward widths 14336 / 28672 / 53248 (SwiGLU) and the 8B hidden size
4096 are the published Llama 3.1 shapes the pages' models refer to.

Values: activations N(0, 1), weights N(0, 0.02) (0.01 for 405B), bf16.
Seeds: X 0, W or Wg or Wqkv 1, W2 or Wu 2, Wd or Wo 3, attention output A 4.
The fused gate/up weight is the logical [Wg | Wu] (gate first).
"""
from __future__ import annotations

import numpy as np

from . import normal_bf16

SEED_X, SEED_W1, SEED_W2, SEED_W3, SEED_A = 0, 1, 2, 3, 4

LLAMA8B = dict(hidden=4096, inter=14336, sigma=0.02)
LLAMA70B = dict(hidden=8192, inter=28672, sigma=0.02, n_q=64, n_kv=8, head_dim=128)
LLAMA405B = dict(hidden=16384, inter=53248, sigma=0.01)


def activations(M: int, hidden: int, rows: range | None = None) -> np.ndarray:
    return normal_bf16(SEED_X, (M, hidden), 1.0, rows=rows)


def attention_output(M: int, width: int, rows: range | None = None, cols: range | None = None):
    return normal_bf16(SEED_A, (M, width), 1.0, rows=rows, cols=cols)


def gateup(hidden: int, inter: int, sigma: float, cols: range | None = None) -> np.ndarray:
    """[Wg[:, cols] | Wu[:, cols]]; with cols = None the full logical [Wg | Wu]."""
    cols = range(0, inter) if cols is None else cols
    g = normal_bf16(SEED_W1, (hidden, inter), sigma, cols=cols)
    u = normal_bf16(SEED_W2, (hidden, inter), sigma, cols=cols)
    return np.concatenate([g, u], axis=1)


def down(inter: int, hidden: int, sigma: float, rows: range | None = None) -> np.ndarray:
    return normal_bf16(SEED_W3, (inter, hidden), sigma, rows=rows)


def worked_tp2():
    """X [8 x 4096] ~ N(0,1); W, W2 4096 x 4096 ~ N(0, 0.02); seed 0 stream order."""
    X = normal_bf16(SEED_X, (8, 4096), 1.0)
    W = normal_bf16(SEED_W1, (4096, 4096), 0.02)
    W2 = normal_bf16(SEED_W2, (4096, 4096), 0.02)
    return X, W, W2


def qkv_weight(hidden: int, n_q: int, n_kv: int, head_dim: int, sigma: float) -> np.ndarray:
    """Logical [Wq | Wk | Wv], [hidden x (n_q + 2 n_kv) head_dim]."""
    return normal_bf16(SEED_W1, (hidden, (n_q + 2 * n_kv) * head_dim), sigma)


def o_weight(n_q: int, head_dim: int, hidden: int, sigma: float) -> np.ndarray:
    return normal_bf16(SEED_W3, (n_q * head_dim, hidden), sigma)
