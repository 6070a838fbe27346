"""Seeded synthetic inputs: weights in their logical FP8/bf16 storage form,
prompt and teacher-forced token ids, prompt latents and layer inputs.

Every tensor is drawn from its own seed, derived from (master seed, tensor
name, layer, expert), so any tensor can be regenerated alone, on the CPU or on
a GPU, without generating the others. The same seed on two different devices
gives two different (but each reproducible) draws: a test always hands the
*same* generated tensors to both sides it compares.

Storage forms (the interface the decode step consumes):
  * FP8 matrix [N, K]: OCP e4m3 codes (uint8, row-major) plus one bf16 scale
    per 128x128 block, stored as uint16 bit patterns [ceil(N/128), ceil(K/128)].
    Pre-quantisation values are N(0, std^2); the scale is bf16(amax / 448)
    (1 for an all-zero block) and the code is the e4m3 encoding of
    clamp(w / scale, -448, 448), using torch's float8_e4m3fn conversion.
  * MXFP4 matrix [N, K] (expert matrices of the *_fp4 configs): OCP
    Microscaling FP4, e2m1 codes packed two per byte (element 2j in the low
    nibble of byte j) [N, K/2] plus one e8m0 scale byte per 32 consecutive
    elements of a row [N, K/32]. Pre-quantisation values are N(0, std^2); a
    block's scale is 2^(floor(log2(amax)) - 2) (2 = exponent of the largest
    e2m1 value, 6 = 1.5 * 2^2) and each element is w / scale rounded to the
    nearest e2m1 value, ties to the even code, saturating at +-6.
  * bf16 tensors (router, embedding, LM head): N(0, std^2) rounded to bf16,
    stored as uint16 bit patterns.
  * norm gains: float32, all ones unless random gains are requested.

Nothing in this module computes any part of the decode step itself.
"""
from __future__ import annotations

import zlib
from typing import Dict, Optional

import numpy as np
import torch

from . import configs as C

FP8_MAX = 448.0


def tensor_seed(master: int, name: str, layer: int = -1, expert: int = -1, extra: int = 0) -> int:
    ss = np.random.SeedSequence([int(master) & 0xFFFFFFFF, zlib.crc32(name.encode()),
                                 layer + 1, expert + 1, extra])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1))


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def quantize_blocks(w: torch.Tensor):
    """FP8 block quantisation of an fp32 matrix (input preparation only)."""
    n, k = w.shape
    nb, kb = (n + C.BLOCK - 1) // C.BLOCK, (k + C.BLOCK - 1) // C.BLOCK
    pad = torch.zeros(nb * C.BLOCK, kb * C.BLOCK, dtype=torch.float32, device=w.device)
    pad[:n, :k] = w
    blocks = pad.view(nb, C.BLOCK, kb, C.BLOCK)
    amax = blocks.abs().amax(dim=(1, 3))
    s = (amax / FP8_MAX).to(torch.bfloat16)
    s = torch.where(amax == 0, torch.ones_like(s), s)
    sf = s.float()[:, None, :, None]
    q = (blocks / sf).clamp(-FP8_MAX, FP8_MAX).view(nb * C.BLOCK, kb * C.BLOCK)[:n, :k]
    codes = q.contiguous().to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, s.view(torch.int16)


def quantize_mxfp4(w: torch.Tensor):
    """MXFP4 quantisation of an fp32 matrix [N, K], K a multiple of 32 (input
    preparation only; the scale and rounding rules are in the module doc)."""
    n, k = w.shape
    blocks = w.reshape(n, k // C.MX_BLOCK, C.MX_BLOCK)
    amax = blocks.abs().amax(dim=2)
    e = torch.where(amax > 0, torch.floor(torch.log2(torch.where(amax > 0, amax, torch.ones_like(amax)))) - 2,
                    torch.zeros_like(amax)).clamp(-127, 127)
    a = (blocks / torch.exp2(e)[:, :, None]).abs()
    # nearest e2m1 magnitude code (0, .5, 1, 1.5, 2, 3, 4, 6 -> 0..7); a tie
    # goes to the even code: down at .25, 1.25, 2.5, 5 and up at .75, 1.75, 3.5
    code = ((a > 0.25).int() + (a >= 0.75).int() + (a > 1.25).int() + (a >= 1.75).int() + (a > 2.5).int()
            + (a >= 3.5).int() + (a > 5.0).int())
    code = code | ((blocks < 0).int() << 3)
    code = code.reshape(n, k).to(torch.uint8)
    packed = code[:, 0::2] | (code[:, 1::2] << 4)
    scales = (e + 127).to(torch.uint8)
    return packed.contiguous(), scales.contiguous()


def gen_tensor(spec: C.TensorSpec, master: int, device="cpu", std: float = 0.02,
               gains: str = "one") -> Dict[str, torch.Tensor]:
    seed = tensor_seed(master, spec.name, spec.layer, spec.expert)
    g = _gen(seed, device)
    if spec.kind == C.F32:
        if gains == "one":
            return {"data": torch.ones(spec.shape, dtype=torch.float32, device=device)}
        x = torch.randn(spec.shape, generator=g, device=device, dtype=torch.float32)
        return {"data": 1.0 + 0.25 * x}
    w = torch.randn(spec.shape, generator=g, device=device, dtype=torch.float32) * std
    if spec.kind == C.BF16:
        return {"data": w.to(torch.bfloat16).view(torch.int16)}
    if spec.kind == C.MXFP4:
        codes, scales = quantize_mxfp4(w)
        return {"mx_codes": codes, "mx_scales": scales}
    codes, scales = quantize_blocks(w)
    return {"codes": codes, "scales": scales}


class LogicalWeights:
    """All weights of a config in storage form, generated lazily per tensor.

    Small tensors are cached; FP8 expert matrices of large configs can be
    regenerated on demand instead (cache=False) so that the full expert set
    never has to sit in memory twice.
    """

    def __init__(self, cfg: C.ModelConfig, master_seed: int = 0, device="cpu",
                 gains: str = "one", cache: bool = True, cache_limit_bytes: int = 1 << 30):
        self.cfg = cfg
        self.seed = master_seed
        self.device = device
        self.gains = gains
        self.cache = cache
        self.cache_limit = cache_limit_bytes
        self._cache: Dict[tuple, Dict[str, torch.Tensor]] = {}
        self._specs = {s.key: s for s in C.all_tensors(cfg)}

    def spec(self, name, layer=-1, expert=-1) -> C.TensorSpec:
        return self._specs[(name, layer, expert)]

    def specs(self):
        return list(self._specs.values())

    def get(self, name, layer=-1, expert=-1) -> Dict[str, torch.Tensor]:
        key = (name, layer, expert)
        if key in self._cache:
            return self._cache[key]
        t = gen_tensor(self._specs[key], self.seed, self.device, self.cfg.weight_std, self.gains)
        nbytes = sum(v.numel() * v.element_size() for v in t.values())
        if self.cache and nbytes <= self.cache_limit:
            self._cache[key] = t
        return t

    def numpy(self, name, layer=-1, expert=-1) -> Dict[str, np.ndarray]:
        """Host copies: codes uint8, scales/bf16 data uint16, gains float32."""
        out = {}
        for k, v in self.get(name, layer, expert).items():
            a = v.detach().cpu().numpy()
            if a.dtype == np.int16:
                a = a.view(np.uint16)
            out[k] = a
        return out


# ---------------------------------------------------------------------------
# Workload inputs
# ---------------------------------------------------------------------------

def prompt_tokens(cfg: C.ModelConfig, seed: int = 0) -> np.ndarray:
    rng = np.random.default_rng(np.random.SeedSequence([seed, 1, 0]))
    return rng.integers(0, cfg.vocab, size=cfg.prompt_len, dtype=np.int64)


def decode_token(cfg: C.ModelConfig, step: int, attempt: int = 0, seed: int = 0) -> int:
    """Teacher-forced token of decode step `step`; `attempt` > 0 redraws it."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 1, 1, step, attempt]))
    return int(rng.integers(0, cfg.vocab))


def latent_rows(cfg: C.ModelConfig, layer: int, n: int, seed: int = 0, device="cpu") -> torch.Tensor:
    """n latent cache rows [n, kv_lora + rope] drawn N(0,1), as bf16 bit patterns."""
    g = _gen(tensor_seed(seed, "latent", layer, extra=2), device)
    x = torch.randn(n, cfg.kv_row, generator=g, device=device, dtype=torch.float32)
    return x.to(torch.bfloat16).view(torch.int16)


def layer_input(cfg: C.ModelConfig, step: int, attempt: int = 0, seed: int = 0, device="cpu") -> torch.Tensor:
    """Hidden input [D] of a bare layer stack, N(0,1) rounded to bf16 (bit patterns)."""
    g = _gen(tensor_seed(seed, "layer_input", step, attempt, extra=3), device)
    x = torch.randn(cfg.hidden, generator=g, device=device, dtype=torch.float32)
    return x.to(torch.bfloat16).view(torch.int16)


def batch_rows(B: int, K: int, seed: int = 0, tag: int = 0) -> np.ndarray:
    """B activation rows [B, K] drawn N(0,1) (float32): the normalised inputs
    of a batch of B decode tokens."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 4, tag, B, K]))
    return rng.standard_normal((B, K)).astype(np.float32)


def batch_routing(cfg: C.ModelConfig, B: int, seed: int = 0, tag: int = 0):
    """Routing of B tokens: top_k distinct experts per token drawn uniformly
    (idx int32 [B, top_k]) with positive weights that sum to 1 per token
    (float32 [B, top_k]), the shape of sigmoid-scored, normalised top-k
    routing on inputs that favour no expert."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 5, tag, B]))
    idx = np.stack([rng.choice(cfg.n_experts, cfg.top_k, replace=False) for _ in range(B)]).astype(np.int32)
    w = rng.uniform(0.5, 1.5, size=(B, cfg.top_k))
    return idx, (w / w.sum(axis=1, keepdims=True)).astype(np.float32)


def dsa_inputs(n: int, HI: int, dI: int, H: int, dc: int, dr: int, seed: int = 0, tag: int = 0):
    """Inputs of one sparse-attention decode token over a cache of n rows:
    indexer queries q [HI, dI] and head weights w [HI] (N(0,1) and
    N(0, 1/HI), float32), indexer keys [n, dI] and latent cache rows
    [n, dc + dr] (N(0,1), bf16 bit patterns as int16), absorbed latent
    queries [H, dc] and rotary queries [H, dr] (N(0,1), float32)."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 6, tag, n, HI, dI, H, dc, dr]))
    f32 = np.float32
    q = rng.standard_normal((HI, dI)).astype(f32)
    w = (rng.standard_normal(HI) / np.sqrt(HI)).astype(f32)
    keys = torch.from_numpy(rng.standard_normal((n, dI)).astype(f32)).to(torch.bfloat16).view(torch.int16)
    rows = torch.from_numpy(rng.standard_normal((n, dc + dr)).astype(f32)).to(torch.bfloat16).view(torch.int16)
    q_lat = rng.standard_normal((H, dc)).astype(f32)
    q_pe = rng.standard_normal((H, dr)).astype(f32)
    return q, w, keys, rows, q_lat, q_pe


def dsa_scores_sample(n: int, kind: str, seed: int = 0) -> np.ndarray:
    """Index scores [n] float32 for the selection: 'normal' N(0,1); 'ties'
    values on a grid of 8 levels (many equal scores); 'zeros' +0.0 and -0.0
    mixed with negatives; 'equal' one value everywhere."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 7, n, len(kind)]))
    if kind == "normal":
        return rng.standard_normal(n).astype(np.float32)
    if kind == "ties":
        return (rng.integers(-4, 4, n) * 0.5).astype(np.float32)
    if kind == "zeros":
        v = rng.choice(np.array([0.0, -0.0, -1.0, -2.5], np.float32), n)
        return v.astype(np.float32)
    return np.full(n, 0.75, np.float32)
