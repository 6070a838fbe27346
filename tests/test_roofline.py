"""Pins of the roofline arithmetic against the pages' printed figures and
against the byte counts of the model shapes."""
import json
import os

import pytest

from persistent_decode_megakernel_amd import roofline as R
from synth import configs

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_roofline.json")))


def test_pages_nvfp4_roofline():
    g = GOLD["nvfp4_b200_roofline"]
    v = R.roofline_tokens_per_s(g["bandwidth_bytes_per_s"], g["bytes_per_token"])
    assert int(v) == g["printed_tokens_per_s"]


def test_pages_mxfp8_roofline_rounds_to_printed():
    g = GOLD["mxfp8_h200_roofline"]
    v = R.roofline_tokens_per_s(g["bandwidth_bytes_per_s"], g["bytes_per_token"])
    assert 900 < v < 1000 and round(v, -3) == g["printed_tokens_per_s_rounded"]


def test_pages_interactivity_is_inverse_tpot():
    g = GOLD["decode_tail_8k1k"]
    v = R.interactivity(g["seconds"] / g["tokens"])
    assert round(v) == g["printed_tokens_per_s"]
    # 494.2 tok/s/user means a 2.02 ms time per output token
    assert abs(1e3 / GOLD["interactivity_1k1k"]["printed_tokens_per_s"] - 2.0235) < 1e-3


def test_stack_bytes_per_token():
    cfg = configs.get("dsv3_stack_1k")
    w = R.weight_bytes(cfg)
    # attention per layer, dense FFN, 9 active experts + router, LM head
    attn = 2112 * 7168 + 24576 * 1536 + 32768 * 512 + 7168 * 16384
    assert attn == 187_105_280
    assert w["fp8_codes"] + w["bf16"] == 11 * attn + 3 * 3 * 18432 * 7168 + 8 * (9 * 3 * 2048 * 7168 + 256 * 7168 * 2) + 129280 * 7168 * 2
    assert w["fp8_codes"] + w["bf16"] == 8_300_855_296
    assert w["block_scales"] == 784_080
    # KV: 11 layers x ctx rows x 576 bf16
    assert R.kv_bytes(cfg, 1025) == 11 * 1025 * 1152
    mean = R.mean_bytes_per_token(cfg, 1024, 1024)
    assert abs(mean / 1e9 - 8.3211) < 5e-4
    mean8k = R.mean_bytes_per_token(configs.get("dsv3_stack_8k"), 8192, 1024)
    assert abs(mean8k / 1e9 - 8.4119) < 5e-4


def test_single_layer_bytes():
    d = configs.get("dsv3_dense_layer")
    m = configs.get("dsv3_moe_layer")
    assert abs(R.bytes_per_token(d, 1025) / 1e6 - 584.7) < 0.1
    assert abs(R.bytes_per_token(m, 1025) / 1e6 - 588.4) < 0.1


def test_mxfp4_expert_bytes():
    """MXFP4 experts: half a byte per element plus one scale byte per 32."""
    f8, f4 = configs.get("dsv3_stack_1k"), configs.get("dsv3_stack_1k_fp4")
    w8, w4 = R.weight_bytes(f8), R.weight_bytes(f4)
    expert_elems = 8 * 9 * 3 * 2048 * 7168
    assert w4["mxfp4_codes"] == expert_elems // 2
    assert w4["mxfp4_scales"] == expert_elems // 32
    assert w8["fp8_codes"] - w4["fp8_codes"] == expert_elems
    assert w4["bf16"] == w8["bf16"]


def test_plan_weight_bytes_agree_with_roofline():
    """The planner's per-stage weight bytes (scales included) add up to the
    roofline's per-token weight bytes, for FP8 and MXFP4 experts."""
    from persistent_decode_megakernel_amd import describe_plan
    for name in ("dsv3_stack_1k", "dsv3_stack_1k_fp4", "tiny", "tiny_fp4"):
        cfg = configs.get(name)
        plan = describe_plan(cfg, cfg.prompt_len + 8)
        gains = {"qkv": cfg.hidden * 4, "qb": cfg.q_lora * 4, "attn": cfg.kv_lora * 4, "router": cfg.hidden * 4,
                 "lm": cfg.hidden * 4}
        total = sum(s["weight_bytes"] - gains.get(s["type"], 0) for s in plan)
        w = R.weight_bytes(cfg)
        # the plan counts the scales it streams (an FP8 block scale is repeated
        # for every 8 packed rows: 2 bytes per 1024 code bytes), the roofline
        # one per 128x128 block (the algorithmic bytes); MXFP4 scales agree
        fp8_scales_streamed = w["fp8_codes"] // 512
        assert total - w["total"] >= 0, name
        assert abs(total - w["total"] - fp8_scales_streamed + w["block_scales"]) / w["total"] < 1e-4, (
            name, total, w["total"])
