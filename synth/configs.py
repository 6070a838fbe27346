"""Model shapes and workloads of the batch-1 MLA+MoE decode configurations.

Pure data: dimensions, layer order and workload sizes. No arithmetic of the
decode step lives here, so both the CPU oracle and the HIP engine may use it.

Shapes follow the DeepSeek-V3 layout that the TileRT pages describe
("What is TileRT", section 5.2: 61 layers of which 3 dense and 58 MoE, hidden
7168, 256 routed experts with 8 active, vocabulary 129,280). The small
configuration is a scaled-down copy of the same structure.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Tuple


@dataclass(frozen=True)
class ModelConfig:
    name: str
    hidden: int            # D
    n_heads: int           # H
    q_lora: int            # d_q, rank of the query latent
    kv_lora: int           # d_c, rank of the shared key/value latent
    qk_nope: int           # d_n, per-head query/key width without rotary part
    rope: int              # d_r, rotary width (shared key part is one head)
    v_head: int            # d_v, per-head value width
    ffn: int               # F, dense SwiGLU intermediate
    n_experts: int         # E, routed experts per MoE layer
    moe_ffn: int           # F_e, per-expert SwiGLU intermediate
    top_k: int             # k, routed experts per token
    n_shared: int          # shared experts per MoE layer (weight 1)
    vocab: int             # V; 0 means a bare layer stack fed by a hidden vector
    layers: Tuple[str, ...]  # "dense" or "moe", in execution order
    prompt_len: int        # P, positions already in the latent cache before decode
    decode_steps: int      # teacher-forced decode steps of the workload
    rms_eps: float = 1e-6
    rope_base: float = 10000.0
    weight_std: float = 0.02
    # how the prompt cache is filled: "prefill" (full causal forward of the
    # prompt tokens) or "latent" (i.i.d. N(0,1) latents, rounded to bf16)
    prompt_fill: str = "prefill"
    # storage of the routed and shared expert matrices: "fp8" (e4m3 with
    # 128x128 bf16 block scales, like every other matrix) or "mxfp4"
    expert_format: str = "fp8"

    @property
    def n_layers(self) -> int:
        return len(self.layers)

    @property
    def qk_head(self) -> int:
        return self.qk_nope + self.rope

    @property
    def kv_row(self) -> int:
        """Width of one latent cache row: compressed latent then rotary key."""
        return self.kv_lora + self.rope

    @property
    def has_vocab(self) -> bool:
        return self.vocab > 0

    def with_(self, **kw) -> "ModelConfig":
        return replace(self, **kw)


_DSV3_ATTN = dict(hidden=7168, n_heads=128, q_lora=1536, kv_lora=512,
                  qk_nope=128, rope=64, v_head=128)
_DSV3_FFN = dict(ffn=18432, n_experts=256, moe_ffn=2048, top_k=8, n_shared=1)

CONFIGS = {
    # two-layer stack small enough for the oracle to run every step in seconds
    "tiny": ModelConfig(
        name="tiny", hidden=512, n_heads=8, q_lora=128, kv_lora=128, qk_nope=32,
        rope=32, v_head=32, ffn=1024, n_experts=16, moe_ffn=256, top_k=2,
        n_shared=1, vocab=2048, layers=("dense", "moe"), prompt_len=256,
        decode_steps=64),
    # three layers with ragged shapes: rows that are not whole KB (partial
    # units), 24 heads (head groups of 8), two shared experts, top-3 of 12,
    # a vocabulary and a prompt that fill no tile exactly
    "ragged": ModelConfig(
        name="ragged", hidden=1040, n_heads=24, q_lora=176, kv_lora=128, qk_nope=32,
        rope=32, v_head=32, ffn=1072, n_experts=12, moe_ffn=64, top_k=3,
        n_shared=2, vocab=1000, layers=("dense", "moe", "moe"), prompt_len=100,
        decode_steps=16),
    # one dense layer at DeepSeek-V3 shape, fed by an N(0,1) hidden vector
    "dsv3_dense_layer": ModelConfig(
        name="dsv3_dense_layer", **_DSV3_ATTN, **_DSV3_FFN, vocab=0,
        layers=("dense",), prompt_len=1024, decode_steps=1, prompt_fill="latent"),
    # one MoE layer at DeepSeek-V3 shape
    "dsv3_moe_layer": ModelConfig(
        name="dsv3_moe_layer", **_DSV3_ATTN, **_DSV3_FFN, vocab=0,
        layers=("moe",), prompt_len=1024, decode_steps=1, prompt_fill="latent"),
    # 3 dense + 8 MoE + LM head, 1k prompt / 1k decode
    "dsv3_stack_1k": ModelConfig(
        name="dsv3_stack_1k", **_DSV3_ATTN, **_DSV3_FFN, vocab=129280,
        layers=("dense",) * 3 + ("moe",) * 8, prompt_len=1024, decode_steps=1024,
        prompt_fill="latent"),
    # same stack, 8k prompt / 1k decode
    "dsv3_stack_8k": ModelConfig(
        name="dsv3_stack_8k", **_DSV3_ATTN, **_DSV3_FFN, vocab=129280,
        layers=("dense",) * 3 + ("moe",) * 8, prompt_len=8192, decode_steps=1024,
        prompt_fill="latent"),
}

# The same models with MXFP4 expert matrices (OCP Microscaling: e2m1
# elements, one power-of-two e8m0 scale per 32 consecutive elements of a row):
# the 4-bit weights the pages' roofline figures assume, which halve the bytes
# of every expert a token reads.
# (MXFP4 needs whole 32-element blocks: the ragged model's hidden size moves
# from 1040 to 1056, still no multiple of 64)
for _n in ("tiny", "ragged", "dsv3_moe_layer", "dsv3_stack_1k", "dsv3_stack_8k"):
    CONFIGS[_n + "_fp4"] = CONFIGS[_n].with_(name=_n + "_fp4", expert_format="mxfp4")
CONFIGS["ragged_fp4"] = CONFIGS["ragged_fp4"].with_(hidden=1056)

# the workloads in the order the project's configuration list gives them
CONFIG_ORDER = ("tiny", "dsv3_dense_layer", "dsv3_moe_layer", "dsv3_stack_1k", "dsv3_stack_8k")


def get(name: str) -> ModelConfig:
    return CONFIGS[name]


# ---------------------------------------------------------------------------
# Logical weight inventory. Names and shapes of every tensor of a config; the
# FP8 matrices carry one bf16 scale per 128x128 block (edge blocks partial).
# ---------------------------------------------------------------------------
FP8 = "fp8"      # uint8 e4m3 codes [N, K] + uint16 bf16 bit patterns [ceil(N/128), ceil(K/128)]
MXFP4 = "mxfp4"  # uint8 codes [N, K/2] (element 2j in the low nibble of byte j, e2m1) + uint8 e8m0 scales [N, K/32]
BF16 = "bf16"    # uint16 bf16 bit patterns
F32 = "f32"      # float32 (norm gains)

BLOCK = 128
MX_BLOCK = 32


@dataclass(frozen=True)
class TensorSpec:
    name: str
    kind: str
    shape: Tuple[int, ...]
    layer: int = -1      # -1 for global tensors
    expert: int = -1     # routed expert index; n_experts + j for shared expert j

    @property
    def key(self):
        return (self.name, self.layer, self.expert)


def layer_tensors(cfg: ModelConfig, l: int):
    D, H = cfg.hidden, cfg.n_heads
    out = [
        TensorSpec("attn_norm", F32, (D,), l),
        TensorSpec("wq_a", FP8, (cfg.q_lora, D), l),
        TensorSpec("q_norm", F32, (cfg.q_lora,), l),
        TensorSpec("wq_b", FP8, (H * cfg.qk_head, cfg.q_lora), l),
        TensorSpec("wkv_a", FP8, (cfg.kv_row, D), l),
        TensorSpec("kv_norm", F32, (cfg.kv_lora,), l),
        TensorSpec("wkv_b", FP8, (H * (cfg.qk_nope + cfg.v_head), cfg.kv_lora), l),
        TensorSpec("wo", FP8, (D, H * cfg.v_head), l),
        TensorSpec("ffn_norm", F32, (D,), l),
    ]
    if cfg.layers[l] == "dense":
        out += [TensorSpec("w_gate", FP8, (cfg.ffn, D), l),
                TensorSpec("w_up", FP8, (cfg.ffn, D), l),
                TensorSpec("w_down", FP8, (D, cfg.ffn), l)]
    else:
        out.append(TensorSpec("router", BF16, (cfg.n_experts, D), l))
        ek = MXFP4 if cfg.expert_format == "mxfp4" else FP8
        for e in range(cfg.n_experts + cfg.n_shared):
            out += [TensorSpec("w_gate", ek, (cfg.moe_ffn, D), l, e),
                    TensorSpec("w_up", ek, (cfg.moe_ffn, D), l, e),
                    TensorSpec("w_down", ek, (D, cfg.moe_ffn), l, e)]
    return out


def global_tensors(cfg: ModelConfig):
    if not cfg.has_vocab:
        return []
    return [TensorSpec("embed", BF16, (cfg.vocab, cfg.hidden)),
            TensorSpec("final_norm", F32, (cfg.hidden,)),
            TensorSpec("lm_head", BF16, (cfg.vocab, cfg.hidden))]


def all_tensors(cfg: ModelConfig):
    out = list(global_tensors(cfg))
    for l in range(cfg.n_layers):
        out += layer_tensors(cfg, l)
    return out


def scale_shape(shape):
    n, k = shape
    return ((n + BLOCK - 1) // BLOCK, (k + BLOCK - 1) // BLOCK)
