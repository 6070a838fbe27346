"""Per-token byte counts and the HBM roofline of batch-1 decode.

At batch 1 every weight is read once per token and the latent cache once per
layer, so the ideal interactivity is bandwidth divided by the bytes a token
reads (SemiAnalysis TileRT page, introduction and how-it-works sections: the
per-user token rate bound is the aggregate HBM bandwidth over the active bytes
per token). Interactivity is the inverse of the time per output token (same
page, trade-off section).

Algorithmic bytes of one decode step (what the method must read):
  * FP8 e4m3 codes of every active matrix: attention projections of every
    layer, the dense FFNs, and the top-k routed plus shared experts of every
    MoE layer (never all experts);
  * one bf16 scale per 128x128 block of those matrices;
  * for MXFP4 experts (expert_format "mxfp4") half a byte per element and
    one e8m0 scale byte per 32 elements instead;
  * bf16 router and LM head;
  * the latent cache: every layer reads ctx = pos + 1 rows of kv_lora + rope
    bf16 values.
The embedding row and norm gains (well under 0.01%) are not counted.
"""
from __future__ import annotations

HBM_PEAK_BYTES_PER_S = 8.0e12   # MI355X HBM3E peak


def _blocks(n, k):
    return ((n + 127) // 128) * ((k + 127) // 128)


def weight_bytes(cfg) -> dict:
    D, H = cfg.hidden, cfg.n_heads
    fp8 = []  # (rows, cols) of every active FP8 matrix of one token
    mx = []   # the same for MXFP4 matrices
    bf16 = 0
    experts = mx if getattr(cfg, "expert_format", "fp8") == "mxfp4" else fp8
    for kind in cfg.layers:
        fp8 += [(cfg.q_lora, D), (cfg.kv_row, D), (H * cfg.qk_head, cfg.q_lora),
                (H * (cfg.qk_nope + cfg.v_head), cfg.kv_lora), (D, H * cfg.v_head)]
        if kind == "dense":
            fp8 += [(cfg.ffn, D), (cfg.ffn, D), (D, cfg.ffn)]
        else:
            experts += [(cfg.moe_ffn, D), (cfg.moe_ffn, D), (D, cfg.moe_ffn)] * (cfg.top_k + cfg.n_shared)
            bf16 += cfg.n_experts * D * 2
    if cfg.vocab:
        bf16 += cfg.vocab * D * 2
    codes = sum(n * k for n, k in fp8)
    scales = sum(_blocks(n, k) * 2 for n, k in fp8)
    mx_codes = sum(n * k // 2 for n, k in mx)
    mx_scales = sum(n * k // 32 for n, k in mx)
    return {"fp8_codes": codes, "block_scales": scales, "mxfp4_codes": mx_codes, "mxfp4_scales": mx_scales,
            "bf16": bf16, "total": codes + scales + mx_codes + mx_scales + bf16}


def kv_bytes(cfg, ctx: int) -> int:
    """Latent cache bytes one step reads at context length ctx (rows 0..pos)."""
    return cfg.n_layers * ctx * cfg.kv_row * 2


def bytes_per_token(cfg, ctx: int) -> int:
    return weight_bytes(cfg)["total"] + kv_bytes(cfg, ctx)


def mean_bytes_per_token(cfg, pos0: int, steps: int) -> float:
    """Average over decode steps at positions pos0 .. pos0 + steps - 1."""
    w = weight_bytes(cfg)["total"]
    kv = sum(kv_bytes(cfg, p + 1) for p in range(pos0, pos0 + steps))
    return w + kv / steps


def roofline_tokens_per_s(bandwidth_bytes_per_s: float, bytes_per_token: float) -> float:
    return bandwidth_bytes_per_s / bytes_per_token


def interactivity(tpot_s: float) -> float:
    """Tokens per second per user from the time per output token."""
    return 1.0 / tpot_s
