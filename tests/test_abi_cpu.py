"""The C-ABI library loads on a machine without a GPU, exports every symbol
include/pdm.h declares, and its pure entry points (sizes, stage plan) are
consistent. No compute call is made here."""
import ctypes as C
import os
import re

import pytest

from synth import configs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    from persistent_decode_megakernel_amd import _lib as L
    if not os.path.exists(L.LIB_PATH):
        pytest.skip("library not built")
    return L.load()


def header_functions():
    text = open(os.path.join(ROOT, "include", "pdm.h")).read()
    return sorted(set(re.findall(r"^\s*(?:int|uint64_t|const char\*)\s+(pdm_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol(lib):
    from persistent_decode_megakernel_amd import _lib as L
    names = header_functions()
    assert len(names) >= 18
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(L.EXPORTED)


def test_strerror(lib):
    from persistent_decode_megakernel_amd import _lib as L
    assert L.strerror(0) == "ok"
    assert L.strerror(L.ERR_WATCHDOG) == "device dependency wait timed out"
    assert L.strerror(L.ERR_POS).startswith("position")
    assert L.strerror(-999) == "unknown error"


def test_create_without_gpu_reports_device_error(lib):
    import torch
    from persistent_decode_megakernel_amd import _lib as L
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    h = C.c_void_p()
    d = L.dims_of(configs.get("tiny"))
    assert lib.pdm_create(C.byref(d), 64, 0, C.byref(h)) == L.ERR_DEVICE


@pytest.mark.parametrize("name", configs.CONFIG_ORDER + ("ragged",))
def test_sizes(lib, name):
    from persistent_decode_megakernel_amd import query_sizes
    cfg = configs.get(name)
    ctx = cfg.prompt_len + cfg.decode_steps
    s = query_sizes(cfg, ctx)
    fp8 = 0
    for spec in configs.all_tensors(cfg):
        if spec.kind == configs.FP8:
            fp8 += spec.shape[0] * spec.shape[1]
    assert s.weight_bytes >= fp8
    assert s.weight_bytes < fp8 * 1.01 + 2 * cfg.vocab * cfg.hidden * 2 + (1 << 24)
    assert s.kv_bytes >= cfg.n_layers * ctx * cfg.kv_row * 2
    assert s.alignment == 256 and s.n_workgroups == 256


def test_invalid_shapes_rejected(lib):
    from persistent_decode_megakernel_amd import _lib as L
    base = configs.get("tiny")
    for bad in (dict(n_heads=3), dict(kv_lora=96), dict(hidden=520), dict(moe_ffn=200),
                dict(top_k=20), dict(rope=8)):
        d = L.dims_of(base.with_(**bad))
        s = L.Sizes()
        assert lib.pdm_query_sizes(C.byref(d), 64, 256, C.byref(s)) == L.ERR_CONFIG, bad
    d = L.dims_of(base)
    s = L.Sizes()
    assert lib.pdm_query_sizes(C.byref(d), 0, 256, C.byref(s)) == L.ERR_ARG
    assert lib.pdm_query_sizes(None, 64, 256, C.byref(s)) == L.ERR_ARG


def test_dsa_argument_checks(lib):
    """The sparse-attention calls reject bad arguments before any HIP call."""
    from persistent_decode_megakernel_amd import _lib as L
    fake = C.c_void_p(1 << 20)      # never dereferenced: every call below fails its checks first
    odd = C.c_void_p((1 << 20) + 4)
    assert lib.pdm_dsa_index_scores(None, fake, fake, 10, 64, 128, fake, None) == L.ERR_ARG
    assert lib.pdm_dsa_index_scores(fake, fake, fake, -1, 64, 128, fake, None) == L.ERR_ARG
    for HI, dI in ((8, 128), (80, 128), (24, 128), (64, 16), (64, 100), (64, 288)):
        assert lib.pdm_dsa_index_scores(fake, fake, fake, 10, HI, dI, fake, None) == L.ERR_CONFIG, (HI, dI)
    assert lib.pdm_dsa_index_scores(fake, fake, odd, 10, 64, 128, fake, None) == L.ERR_ALIGN
    assert lib.pdm_dsa_topk(None, 10, 5, fake, fake, 1 << 20, None) == L.ERR_ARG
    assert lib.pdm_dsa_topk(fake, 10, -1, fake, fake, 1 << 20, None) == L.ERR_ARG
    assert lib.pdm_dsa_topk(fake, 10, 5, fake, None, 1 << 20, None) == L.ERR_ARG
    need = lib.pdm_dsa_topk_work_bytes(131072)
    assert need == (1024 + 2 * 64) * 4
    assert lib.pdm_dsa_topk(fake, 131072, 5, fake, fake, need - 1, None) == L.ERR_SIZE
    assert lib.pdm_dsa_attention_work_bytes(128, 512) == 128 * 32 * 514 * 4
    assert lib.pdm_dsa_attention_work_bytes(0, 512) == 0

    def att(cache=fake, n_sel=4, H=16, dc=512, dr=64, wb=1 << 30, sel=fake, rows=10):
        return lib.pdm_dsa_attention(fake, fake, cache, rows, sel, n_sel, H, dc, dr, 0.1, fake, wb, fake, None)
    assert att(sel=None) == L.ERR_ARG
    assert att(n_sel=0) == L.ERR_ARG
    assert att(H=0) == L.ERR_ARG
    assert att(rows=0) == L.ERR_ARG
    for dc, dr in ((384, 64), (512, 65), (512, 160), (64, 32)):
        assert att(dc=dc, dr=dr) == L.ERR_CONFIG, (dc, dr)
    assert att(cache=odd) == L.ERR_ALIGN
    assert att(wb=lib.pdm_dsa_attention_work_bytes(16, 512) - 1) == L.ERR_SIZE


def _validate_dag(plan, cfg):
    """Every buffer a stage reads is produced by a stage that the stage's wait
    covers (stage index <= wait), so it is complete before the read. The
    attention stage builds the new cache row itself (its older rows come from
    earlier steps)."""
    from persistent_decode_megakernel_amd import _lib as L
    producers = {}
    for i, st in enumerate(plan):
        for b in st["writes"]:
            producers.setdefault(b, []).append(i)
    for i, st in enumerate(plan):
        assert st["wait"] < i
        for b in st["reads"]:
            if b % 16 == L.BUF_INPUT and b // 16 == 0:   # the step input
                continue
            if b % 16 == L.BUF_KV and st["type"] == "attn":
                assert producers[b] == [i], (i, producers[b])
                continue
            assert b in producers, (i, st["type"], b)
            for p in producers[b]:
                assert p < i and p <= st["wait"], (i, st["type"], b, p, st["wait"])
    # the layer order is dense first, and every layer has its stages
    kinds = [st["type"] for st in plan]
    assert kinds.count("qkv") == cfg.n_layers and kinds.count("down") == cfg.n_layers
    assert kinds.count("lm") == (1 if cfg.vocab else 0)


@pytest.mark.parametrize("name", configs.CONFIG_ORDER + ("ragged",))
def test_stage_plan_is_a_valid_dag(lib, name):
    from persistent_decode_megakernel_amd import describe_plan
    cfg = configs.get(name)
    plan = describe_plan(cfg, cfg.prompt_len + cfg.decode_steps)
    _validate_dag(plan, cfg)
    per_layer = {"dense": 7, "moe": 8}
    assert len(plan) == sum(per_layer[k] for k in cfg.layers) + (1 if cfg.vocab else 0)


def test_dag_validator_catches_a_dropped_dependency(lib):
    from persistent_decode_megakernel_amd import describe_plan
    cfg = configs.get("tiny")
    plan = describe_plan(cfg, 320)
    i = next(i for i, st in enumerate(plan) if st["type"] == "uv")
    plan[i]["wait"] = plan[i]["wait"] - 1     # no longer waits for attention
    with pytest.raises(AssertionError):
        _validate_dag(plan, cfg)


def test_plan_weight_bytes_match_active_parameters(lib):
    """Per-step weight bytes of the plan: FP8 codes of the active experts plus
    packed scales, bf16 router and LM head, f32 norm gains."""
    from persistent_decode_megakernel_amd import describe_plan
    cfg = configs.get("dsv3_stack_1k")
    plan = describe_plan(cfg, 2048)
    tot = sum(st["weight_bytes"] for st in plan)
    D, H = cfg.hidden, cfg.n_heads
    attn = D * (cfg.q_lora + cfg.kv_row) + H * cfg.qk_head * cfg.q_lora + H * (cfg.qk_nope + cfg.v_head) * cfg.kv_lora + D * H * cfg.v_head
    dense = 3 * D * cfg.ffn
    moe = 3 * D * cfg.moe_ffn * (cfg.top_k + cfg.n_shared) + cfg.n_experts * D * 2
    codes = 11 * attn + 3 * dense + 8 * moe + cfg.vocab * D * 2
    assert codes <= tot <= codes * 1.003 + 11 * 4 * (2 * D + cfg.q_lora + cfg.kv_lora) + 4 * D


def test_engine_kernel_resource_usage():
    """The persistent kernel keeps one 512-thread workgroup per CU and does not
    spill vector registers: a spill turns into scratch traffic that every
    stage's completion wait then has to drain."""
    import json
    from persistent_decode_megakernel_amd import build
    if not os.path.exists(build.USAGE):
        pytest.skip("library not built")
    usage = json.load(open(build.USAGE))
    ks = [v for n, v in usage.items() if "engine_kernel" in n]
    assert len(ks) == 2  # one instance per expert weight format (FP8, MXFP4)
    for k in ks:
        assert k["Occupancy [waves/SIMD]"] >= 2
        assert k["LDS Size [bytes/block]"] <= 160 * 1024
        # no vector registers spilled to scratch; SGPR spills go to VGPR
        # lanes (no memory traffic) and are bounded against a large jump
        assert k["ScratchSize [bytes/lane]"] == 0, k
        assert k["VGPRs Spill"] == 0, k
        assert k["SGPRs Spill"] <= 1024, k
