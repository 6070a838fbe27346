"""Plain float64 CPU definition of one batch-1 decode step of a DeepSeek-V3
style MLA + MoE transformer, plus the full causal forward it must agree with.

TEST INFRASTRUCTURE (see the package docstring).

What the TileRT pages fix and what is read into them:
  * The step is one autoregressive decode token at batch 1 through MLA
    attention and dense / MoE feed-forward layers ("What is TileRT",
    section 5.2: MLA, 256 routed experts with 8 active, hidden 7168,
    vocabulary 129,280; SemiAnalysis TileRT page, "how it works" section:
    RMSNorm, GEMM, attention and Top-K routing are the operators named).
  * The pages give no formula for any operator. The readings used here are
    the plainest ones: pre-norm RMSNorm (eps 1e-6) before attention and FFN,
    RMSNorm on the query and key/value latents; rotary embedding on
    consecutive pairs (2i, 2i+1) with base 10000 and no scaling; softmax
    scale 1/sqrt(qk_nope + rope); SwiGLU experts; sigmoid router scores, top-k
    by score with ties to the lower index, weights normalised over the chosen
    experts, no bias or group limit; shared experts with weight 1.
  * Declared rounding points ("parity" mode): R1 every latent cache row is
    stored in bf16 and attention reads the stored values; R2 the residual
    stream handed from one layer to the next is rounded to bf16. Everything
    else is exact float64 arithmetic of the dequantised weights.

A dequantised FP8 or MXFP4 weight is exactly code_value * block_scale; bf16
tensors widen exactly. Weights come from a store with a `numpy(name, layer, expert)`
method returning the storage-form arrays (see synth.gen.LogicalWeights).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

from .numerics import bf16_bits_to_f64, bf16_round, dequant_fp8, dequant_mxfp4


# ---------------------------------------------------------------------------
# weights
# ---------------------------------------------------------------------------

class OracleWeights:
    """Dequantised float64 view of a logical weight store, with a small cache."""

    def __init__(self, store, cache_limit_bytes: int = 2 << 30):
        self.store = store
        self.cfg = store.cfg
        self._cache: Dict[tuple, np.ndarray] = {}
        self._bytes = 0
        self.limit = cache_limit_bytes

    def __call__(self, name: str, layer: int = -1, expert: int = -1) -> np.ndarray:
        key = (name, layer, expert)
        if key in self._cache:
            return self._cache[key]
        t = self.store.numpy(name, layer, expert)
        if "codes" in t:
            w = dequant_fp8(t["codes"], t["scales"])
        elif "mx_codes" in t:
            w = dequant_mxfp4(t["mx_codes"], t["mx_scales"])
        elif t["data"].dtype == np.uint16:
            w = bf16_bits_to_f64(t["data"])
        else:
            w = t["data"].astype(np.float64)
        if self._bytes + w.nbytes <= self.limit:
            self._cache[key] = w
            self._bytes += w.nbytes
        return w

    def bf16_row(self, name: str, row: int) -> np.ndarray:
        """One row of a global bf16 matrix (the embedding), without the full dequant."""
        t = self.store.numpy(name)
        return bf16_bits_to_f64(t["data"][row])


# ---------------------------------------------------------------------------
# operators
# ---------------------------------------------------------------------------

def rmsnorm(v: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """v / sqrt(mean(v^2) + eps) * g over the last axis."""
    ms = np.mean(v * v, axis=-1, keepdims=True)
    return v / np.sqrt(ms + eps) * g


def rope(v: np.ndarray, pos, base: float) -> np.ndarray:
    """Rotate consecutive pairs (2i, 2i+1) of the last axis by pos * base^(-2i/d).

    `pos` is a scalar or an array broadcasting against v's leading axes.
    """
    d = v.shape[-1]
    i = np.arange(d // 2, dtype=np.float64)
    inv_freq = base ** (-2.0 * i / d)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv_freq
    cos, sin = np.cos(ang), np.sin(ang)
    a, b = v[..., 0::2], v[..., 1::2]
    out = np.empty_like(v)
    out[..., 0::2] = a * cos - b * sin
    out[..., 1::2] = a * sin + b * cos
    return out


def softmax(s: np.ndarray, axis: int = -1) -> np.ndarray:
    m = np.max(s, axis=axis, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=axis, keepdims=True)


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def sigmoid(z: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-z))


def topk_indices(scores: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest scores, larger first; equal scores: lower index first."""
    order = np.argsort(-scores, kind="stable")
    return order[:k]


def route(z: np.ndarray, k: int):
    """Sigmoid-scored top-k routing with weights normalised over the chosen experts."""
    sig = sigmoid(z)
    idx = topk_indices(sig, k)
    w = sig[idx] / np.sum(sig[idx])
    return idx, w


def swiglu(W, layer: int, expert: int, h: np.ndarray) -> np.ndarray:
    """down(silu(gate h) * (up h)); h may be [D] or [T, D]."""
    g = h @ W("w_gate", layer, expert).T
    u = h @ W("w_up", layer, expert).T
    return (silu(g) * u) @ W("w_down", layer, expert).T


# ---------------------------------------------------------------------------
# MLA attention, both forms
# ---------------------------------------------------------------------------

def split_wkv_b(W, cfg, layer: int):
    """Per-head key and value up-projections from the stacked W_UKV.

    W_UKV rows are grouped per head as [qk_nope key rows ; v_head value rows],
    columns are the kv_lora latent.
    """
    wkv = W("wkv_b", layer).reshape(cfg.n_heads, cfg.qk_nope + cfg.v_head, cfg.kv_lora)
    return wkv[:, :cfg.qk_nope, :], wkv[:, cfg.qk_nope:, :]


def mla_absorbed(qn, qp, C, R, W_UK, W_UV, tau):
    """Attention of one query over cached latents with W_UK folded into the query.

    qn [H, d_n], qp [H, d_r] (rotated), C [T, d_c], R [T, d_r] -> o [H, d_v].
    Returns o and the attention probabilities [H, T].
    """
    ql = np.einsum("hnc,hn->hc", W_UK, qn)
    s = (ql @ C.T + qp @ R.T) * tau
    p = softmax(s, axis=1)
    ol = p @ C
    o = np.einsum("hvc,hc->hv", W_UV, ol)
    return o, p


def mla_naive(qn, qp, C, R, W_UK, W_UV, tau):
    """Same attention with keys and values expanded per head from the latents."""
    K = np.einsum("hnc,tc->htn", W_UK, C)
    V = np.einsum("hvc,tc->htv", W_UV, C)
    s = (np.einsum("hn,htn->ht", qn, K) + qp @ R.T) * tau
    p = softmax(s, axis=1)
    o = np.einsum("ht,htv->hv", p, V)
    return o, p


# ---------------------------------------------------------------------------
# decode step
# ---------------------------------------------------------------------------

@dataclass
class DecodeState:
    """Latent cache per layer ([max_len, kv_lora + rope] float64) and its length."""
    cache: List[np.ndarray]
    length: int = 0

    @classmethod
    def empty(cls, cfg, max_len: int):
        return cls([np.zeros((max_len, cfg.kv_row)) for _ in range(cfg.n_layers)], 0)

    def copy(self):
        return DecodeState([c.copy() for c in self.cache], self.length)


def _r1(v, parity):
    return bf16_round(v) if parity else v


def attention_decode(W, cfg, l: int, x: np.ndarray, pos: int, state: DecodeState,
                     parity: bool, absorbed: bool = True, taps: Optional[dict] = None):
    """x + W_O * MLA(x) for one token at position pos; appends the cache row."""
    h = rmsnorm(x, W("attn_norm", l), cfg.rms_eps)
    cq = rmsnorm(W("wq_a", l) @ h, W("q_norm", l), cfg.rms_eps)
    kv = W("wkv_a", l) @ h
    c = rmsnorm(kv[:cfg.kv_lora], W("kv_norm", l), cfg.rms_eps)
    kp = rope(kv[cfg.kv_lora:], pos, cfg.rope_base)
    state.cache[l][pos] = _r1(np.concatenate([c, kp]), parity)
    q = (W("wq_b", l) @ cq).reshape(cfg.n_heads, cfg.qk_head)
    qn = q[:, :cfg.qk_nope]
    qp = rope(q[:, cfg.qk_nope:], pos, cfg.rope_base)
    W_UK, W_UV = split_wkv_b(W, cfg, l)
    C = state.cache[l][:pos + 1, :cfg.kv_lora]
    R = state.cache[l][:pos + 1, cfg.kv_lora:]
    tau = 1.0 / np.sqrt(cfg.qk_head)
    o, p = (mla_absorbed if absorbed else mla_naive)(qn, qp, C, R, W_UK, W_UV, tau)
    if taps is not None:
        taps.setdefault("attn_probs", []).append(p)
    return x + W("wo", l) @ o.reshape(-1)


def ffn_decode(W, cfg, l: int, x: np.ndarray, taps: Optional[dict] = None):
    h2 = rmsnorm(x, W("ffn_norm", l), cfg.rms_eps)
    if cfg.layers[l] == "dense":
        return x + swiglu(W, l, -1, h2)
    z = W("router", l) @ h2
    idx, w = route(z, cfg.top_k)
    y = np.zeros_like(x)
    for j in range(cfg.n_shared):
        y = y + swiglu(W, l, cfg.n_experts + j, h2)
    for e, we in zip(idx, w):
        y = y + we * swiglu(W, l, int(e), h2)
    if taps is not None:
        taps.setdefault("router_logits", []).append(z)
        taps.setdefault("router_idx", []).append(idx)
        taps.setdefault("router_w", []).append(w)
    return x + y


def lm_logits(W: OracleWeights, cfg, x: np.ndarray, rows_per_block: int = 8192) -> np.ndarray:
    """Final RMSNorm and LM head product, taken a block of vocabulary rows at a
    time so that a 129,280-row bf16 head never sits in memory as one float64
    matrix. Row i of the result is the same dot product as in decode_step."""
    hf = rmsnorm(x, W("final_norm"), cfg.rms_eps)
    data = W.store.numpy("lm_head")["data"]
    return np.concatenate([bf16_bits_to_f64(data[i:i + rows_per_block]) @ hf
                           for i in range(0, data.shape[0], rows_per_block)])


def decode_step(W: OracleWeights, state: DecodeState, pos: int, token: Optional[int] = None,
                x_in: Optional[np.ndarray] = None, parity: bool = True, absorbed: bool = True):
    """One decode step at position pos == state.length.

    Input is the embedding row of `token`, or the hidden vector `x_in` for a
    bare layer stack. Returns a dict with the per-layer outputs ("hidden",
    R2-rounded in parity mode), router taps, and for configs with a vocabulary
    the logits of the final RMSNorm + LM head and their argmax (lowest index
    on ties).
    """
    cfg = W.cfg
    assert pos == state.length, "decode appends at the end of the cache"
    x = W.bf16_row("embed", token) if x_in is None else np.asarray(x_in, dtype=np.float64)
    taps: dict = {"hidden": []}
    for l in range(cfg.n_layers):
        x = attention_decode(W, cfg, l, x, pos, state, parity, absorbed, taps)
        taps.setdefault("hidden_attn", []).append(x)
        x = ffn_decode(W, cfg, l, x, taps)
        if parity:
            x = bf16_round(x)
        taps["hidden"].append(x)
    state.length = pos + 1
    if cfg.has_vocab:
        hf = rmsnorm(x, W("final_norm"), cfg.rms_eps)
        logits = W("lm_head") @ hf
        taps["logits"] = logits
        taps["argmax"] = int(np.argmax(logits))
    return taps


# ---------------------------------------------------------------------------
# full causal forward over a sequence (prefill, and the decode invariant)
# ---------------------------------------------------------------------------

def forward_full(W: OracleWeights, tokens=None, xs: Optional[np.ndarray] = None,
                 parity: bool = True, absorbed: bool = False, pos0: int = 0,
                 state: Optional[DecodeState] = None):
    """Causal forward of T tokens at positions pos0..pos0+T-1, all rows at once.

    Row t attends to every cached row up to its own position. With a `state`
    holding pos0 earlier rows, those rows are attended too and the new rows
    are appended. Returns the per-layer outputs [T, D], the logits [T, V] if
    the config has a vocabulary, and the state.
    """
    cfg = W.cfg
    if xs is None:
        X = np.stack([W.bf16_row("embed", int(t)) for t in tokens])
    else:
        X = np.asarray(xs, dtype=np.float64)
    T = X.shape[0]
    if state is None:
        state = DecodeState.empty(cfg, pos0 + T)
    assert state.length == pos0
    pos = np.arange(pos0, pos0 + T)
    tau = 1.0 / np.sqrt(cfg.qk_head)
    hidden = []
    for l in range(cfg.n_layers):
        h = rmsnorm(X, W("attn_norm", l), cfg.rms_eps)
        cq = rmsnorm(h @ W("wq_a", l).T, W("q_norm", l), cfg.rms_eps)
        kv = h @ W("wkv_a", l).T
        c = rmsnorm(kv[:, :cfg.kv_lora], W("kv_norm", l), cfg.rms_eps)
        kp = rope(kv[:, cfg.kv_lora:], pos, cfg.rope_base)
        state.cache[l][pos0:pos0 + T] = _r1(np.concatenate([c, kp], axis=1), parity)
        q = (cq @ W("wq_b", l).T).reshape(T, cfg.n_heads, cfg.qk_head)
        qn = q[:, :, :cfg.qk_nope]
        qp = rope(q[:, :, cfg.qk_nope:], pos[:, None], cfg.rope_base)
        W_UK, W_UV = split_wkv_b(W, cfg, l)
        C = state.cache[l][:pos0 + T, :cfg.kv_lora]
        R = state.cache[l][:pos0 + T, cfg.kv_lora:]
        if absorbed:
            ql = np.einsum("hnc,thn->thc", W_UK, qn)
            s = np.einsum("thc,sc->ths", ql, C)
        else:
            K = np.einsum("hnc,sc->hsn", W_UK, C)
            s = np.einsum("thn,hsn->ths", qn, K)
        s = (s + np.einsum("thr,sr->ths", qp, R)) * tau
        causal = np.arange(pos0 + T)[None, None, :] > pos[:, None, None]
        s = np.where(causal, -np.inf, s)
        p = softmax(s, axis=2)
        if absorbed:
            ol = np.einsum("ths,sc->thc", p, C)
            o = np.einsum("hvc,thc->thv", W_UV, ol)
        else:
            V = np.einsum("hvc,sc->hsv", W_UV, C)
            o = np.einsum("ths,hsv->thv", p, V)
        X = X + o.reshape(T, -1) @ W("wo", l).T
        h2 = rmsnorm(X, W("ffn_norm", l), cfg.rms_eps)
        if cfg.layers[l] == "dense":
            X = X + swiglu(W, l, -1, h2)
        else:
            Z = h2 @ W("router", l).T
            Y = np.zeros_like(X)
            for j in range(cfg.n_shared):
                Y = Y + swiglu(W, l, cfg.n_experts + j, h2)
            for t in range(T):
                idx, w = route(Z[t], cfg.top_k)
                for e, we in zip(idx, w):
                    Y[t] = Y[t] + we * swiglu(W, l, int(e), h2[t])
            X = X + Y
        if parity:
            X = bf16_round(X)
        hidden.append(X)
    state.length = pos0 + T
    out = {"hidden": hidden, "state": state}
    if cfg.has_vocab:
        out["logits"] = rmsnorm(X, W("final_norm"), cfg.rms_eps) @ W("lm_head").T
    return out


def prefill(W: OracleWeights, tokens, max_len: int, parity: bool = True) -> DecodeState:
    """Latent cache after the causal forward of the prompt, sized for max_len positions."""
    st = DecodeState.empty(W.cfg, max_len)
    forward_full(W, tokens=tokens, parity=parity, absorbed=True, state=st)
    return st
