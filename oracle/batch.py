"""Batched decode products: B tokens through the same weights (float64).

TEST INFRASTRUCTURE (see the package docstring): only tests, the smoke check
and the benchmark's CPU-baseline leg may import this module.

Decoding B sequences together applies every weight matrix to B activation
vectors at once; the MoE block gives each token its own routed experts (the
SemiAnalysis TileRT page names batch sizes 2, 4 and 8 as the next step of its
benchmark). What a batched product computes is fixed per token by the batch-1
definitions in `model`: a batch is B independent rows. Nothing here merges
experts across tokens; that is an implementation choice of the engine, and the
oracle stays the per-token definition.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from .model import swiglu


def batch_gemm(W: np.ndarray, X: np.ndarray) -> np.ndarray:
    """Y[b, r] = sum_k W[r, k] X[b, k]: W [N, K] (dequantised), X [B, K]."""
    return np.asarray(X, dtype=np.float64) @ np.asarray(W, dtype=np.float64).T


def batch_ffn(W, cfg, layer: int, H: np.ndarray, idx: Optional[np.ndarray] = None,
              w: Optional[np.ndarray] = None) -> np.ndarray:
    """The feed-forward block of `layer` for each row of H (the RMS-normalised
    FFN inputs, [B, D]), residual not added.

    Dense layer: its SwiGLU. MoE layer ("What is TileRT" section 5.2, the
    DeepSeek-V3 layer: shared experts plus the routed top-k): the shared
    experts with weight 1 plus, for token b, w[b, j] times expert idx[b, j]'s
    SwiGLU, the same combination `model.ffn_decode` takes for one token with
    its own routing.
    """
    H = np.asarray(H, dtype=np.float64)
    out = np.zeros_like(H)
    for b in range(H.shape[0]):
        h = H[b]
        if cfg.layers[layer] == "dense":
            out[b] = swiglu(W, layer, -1, h)
            continue
        y = np.zeros_like(h)
        for j in range(cfg.n_shared):
            y = y + swiglu(W, layer, cfg.n_experts + j, h)
        for e, we in zip(idx[b], w[b]):
            y = y + float(we) * swiglu(W, layer, int(e), h)
        out[b] = y
    return out
