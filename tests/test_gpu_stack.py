"""GPU parity of the whole decode stack at full DeepSeek-V3 size: 3 dense + 8
MoE MLA layers, final norm and the bf16 LM head over 129,280 tokens, in the
benchmark's launch configuration (engine sized for prompt + 1024 decode steps,
one persistent launch of one workgroup per CU per step).

The oracle runs one step at that size per case (about a minute of float64 CPU
work) and is checked two ways:
  * chained: the oracle's own step from the same token and cache, compared
    with every per-layer output, the logits and the argmax of the engine;
  * isolated: each oracle layer fed the engine's own input to that layer (and
    each FFN the engine's post-attention residual), so a per-layer error
    cannot hide behind the tolerance of the chain.
The prompt cache holds N(0, 1) bf16 latents (the oracle prefill of 1024 or
8192 tokens through 94 GB of experts is far beyond a CPU test); the bytes the
step reads are the same.
"""
import numpy as np
import pytest
import torch

import oracle as O
from synth import configs, gen

from parity_util import MARGIN, REL_TOL, rel_l2

pytestmark = pytest.mark.gpu

SEED = 0


def _gap(z, k):
    s = np.sort(np.asarray(z))[::-1]
    return float(s[k - 1] - s[k])


def _engine_step(eng, cfg, lat, pos, tok):
    eng.reset()
    for l in range(cfg.n_layers):
        eng.import_kv(l, 0, lat[l])
    eng.decode(pos, token=tok)
    rc, st = eng.status()
    assert rc == 0, f"engine status {rc} at stage {st.stage}"
    t = eng.taps()
    out = {k: t[k].cpu().numpy().astype(np.float64 if t[k].dtype == torch.float32 else np.int64)
           for k in ("hidden", "hidden_attn", "router_idx", "router_w")}
    out["logits"] = eng.logits.cpu().numpy().astype(np.float64)
    out["argmax"] = int(eng.argmax.item())
    out["kv"] = [eng.export_kv(l, pos, 1).view(torch.bfloat16).float().cpu().numpy()[0]
                 for l in range(cfg.n_layers)]
    return out


def _check_step(store, cfg, base_state, pos, tok, g):
    """Oracle chained and isolated passes against the engine's step `g`.
    Returns the smallest decision margin of the chained oracle step."""
    st_c, st_i = base_state.copy(), base_state.copy()
    W0 = O.OracleWeights(store, cache_limit_bytes=0)
    x_emb = W0.bf16_row("embed", tok)
    x_c = x_emb
    margin = np.inf
    report = []
    for l in range(cfg.n_layers):
        W = O.OracleWeights(store, cache_limit_bytes=12 << 30)
        x_i = x_emb if l == 0 else g["hidden"][l - 1]
        # chained
        tc = {}
        xa_c = O.attention_decode(W, cfg, l, x_c, pos, st_c, True)
        x_c = O.bf16_round(O.ffn_decode(W, cfg, l, xa_c, tc))
        # isolated
        ti = {}
        xa_i = O.attention_decode(W, cfg, l, x_i, pos, st_i, True)
        xo_i = O.bf16_round(O.ffn_decode(W, cfg, l, g["hidden_attn"][l], ti))
        e = {
            "attn": rel_l2(g["hidden_attn"][l], xa_i),
            "attn_delta": rel_l2(g["hidden_attn"][l] - x_i, xa_i - x_i),
            "ffn": rel_l2(g["hidden"][l], xo_i),
            "chain": rel_l2(g["hidden"][l], x_c),
            "kv_row": rel_l2(g["kv"][l], st_i.cache[l][pos]),
        }
        report.append((l, e))
        print(f"layer {l}: " + " ".join(f"{k} {v:.2e}" for k, v in e.items()), flush=True)
        assert e["attn"] < REL_TOL and e["attn_delta"] < REL_TOL, (l, e)
        assert e["ffn"] < REL_TOL and e["kv_row"] < REL_TOL, (l, e)
        assert e["chain"] < REL_TOL, (l, e)
        if cfg.layers[l] == "moe":
            k = cfg.top_k
            margin = min(margin, _gap(tc["router_logits"][0], k))
            z = ti["router_logits"][0]
            got = [int(i) for i in g["router_idx"][l]]
            if _gap(z, k) > MARGIN:
                assert got == [int(i) for i in ti["router_idx"][0]], (l, got)
                np.testing.assert_allclose(g["router_w"][l], ti["router_w"][0], rtol=1e-4)
            else:  # an ambiguous choice: the engine's set must still be a top-k
                assert min(z[got]) >= np.sort(z)[::-1][k - 1] - MARGIN, (l, got)
        del W
    lg_c = O.lm_logits(W0, cfg, x_c)
    lg_i = O.lm_logits(W0, cfg, g["hidden"][-1])
    margin = min(margin, _gap(lg_c, 1))
    e_c, e_i = rel_l2(g["logits"], lg_c), rel_l2(g["logits"], lg_i)
    print(f"pos {pos} token {tok}: logits chained {e_c:.2e} isolated {e_i:.2e}", flush=True)
    assert e_c < REL_TOL and e_i < REL_TOL, (e_c, e_i)
    assert g["argmax"] == int(np.argmax(g["logits"]))
    if _gap(lg_i, 1) > MARGIN:
        assert g["argmax"] == int(np.argmax(lg_i))
    if margin > MARGIN:
        assert g["argmax"] == int(np.argmax(lg_c))
    return margin


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,where", [("dsv3_stack_1k", "first"), ("dsv3_stack_8k", "last")])
def test_stack_fullsize(name, where):
    from persistent_decode_megakernel_amd import Engine
    cfg = configs.get(name)
    P = cfg.prompt_len
    max_ctx = P + cfg.decode_steps
    pos = P if where == "first" else max_ctx - 1
    eng = Engine(cfg, max_ctx=max_ctx, device=0)
    try:
        assert eng.sizes.n_workgroups == torch.cuda.get_device_properties(0).multi_processor_count
        store = gen.LogicalWeights(cfg, SEED, "cuda", cache=False)
        eng.load_weights(store)
        base = O.DecodeState.empty(cfg, pos + 1)
        lat = []
        for l in range(cfg.n_layers):
            rows = gen.latent_rows(cfg, l, pos, SEED, device="cuda")
            base.cache[l][:pos] = O.bf16_bits_to_f64(rows.cpu().numpy().view(np.uint16))
            lat.append(rows)
        base.length = pos
        for attempt in range(4):
            tok = gen.decode_token(cfg, pos - P, attempt, SEED)
            g = _engine_step(eng, cfg, lat, pos, tok)
            if _check_step(store, cfg, base, pos, tok, g) > MARGIN:
                break
        else:
            pytest.fail(f"no token with router and logit margins above {MARGIN}")
    finally:
        eng.close()
        del eng
        torch.cuda.empty_cache()
