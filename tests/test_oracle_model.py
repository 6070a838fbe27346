"""Whole-step invariants of the oracle: decode step t equals the last row of the
causal forward over t+1 tokens; absorbed and expanded MLA agree; parity-mode
rounding points behave as declared."""
import numpy as np
import pytest

import oracle as O
from synth import configs, gen


def _rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


def _decode_all(W, cfg, toks, parity, absorbed=True, max_len=None):
    st = O.DecodeState.empty(cfg, max_len or len(toks))
    outs = []
    for t, tok in enumerate(toks):
        outs.append(O.decode_step(W, st, t, token=int(tok), parity=parity, absorbed=absorbed))
    return outs, st


@pytest.mark.parametrize("parity", [False, True])
def test_decode_equals_causal_forward_tiny(tiny_cfg, tiny_store, parity):
    """Every decode step over the tiny workload's 320 positions equals the
    corresponding row of one causal forward (expanded MLA form)."""
    cfg = tiny_cfg
    W = O.OracleWeights(tiny_store)
    n = cfg.prompt_len + cfg.decode_steps
    toks = np.concatenate([gen.prompt_tokens(cfg), [gen.decode_token(cfg, j) for j in range(cfg.decode_steps)]])
    assert len(toks) == n == 320
    full = O.forward_full(W, tokens=toks, parity=parity, absorbed=False)
    outs, st = _decode_all(W, cfg, toks, parity)
    tol = 1e-12 if not parity else 1e-12
    for t in range(n):
        for l in range(cfg.n_layers):
            assert _rel(outs[t]["hidden"][l], full["hidden"][l][t]) < tol, (t, l)
        assert _rel(outs[t]["logits"], full["logits"][t]) < tol
        assert outs[t]["argmax"] == int(np.argmax(full["logits"][t]))
    for l in range(cfg.n_layers):
        np.testing.assert_allclose(st.cache[l][:n], full["state"].cache[l][:n], rtol=1e-12, atol=1e-14)


def test_causal_forward_prefix_property(tiny_cfg, tiny_store):
    """Row t of a longer causal forward equals the last row of the forward over t+1 tokens."""
    W = O.OracleWeights(tiny_store)
    toks = gen.prompt_tokens(tiny_cfg)[:48]
    full = O.forward_full(W, tokens=toks, parity=False)
    for t in (0, 1, 17, 47):
        part = O.forward_full(W, tokens=toks[:t + 1], parity=False)
        assert _rel(part["hidden"][-1][-1], full["hidden"][-1][t]) < 1e-12


def test_absorbed_equals_expanded_decode(tiny_cfg, tiny_store):
    W = O.OracleWeights(tiny_store)
    toks = gen.prompt_tokens(tiny_cfg)[:24]
    a, _ = _decode_all(W, tiny_cfg, toks, parity=False, absorbed=True)
    b, _ = _decode_all(W, tiny_cfg, toks, parity=False, absorbed=False)
    for t in range(len(toks)):
        assert _rel(a[t]["hidden"][-1], b[t]["hidden"][-1]) < 1e-10


def test_invariant_on_other_shape():
    """Same invariant on a differently shaped stack (odd head count, MoE first, top-3)."""
    cfg = configs.get("tiny").with_(name="odd", hidden=256, n_heads=3, q_lora=64, kv_lora=96,
                                    qk_nope=24, rope=16, v_head=40, ffn=384, n_experts=7,
                                    moe_ffn=128, top_k=3, n_shared=2, vocab=300,
                                    layers=("moe", "dense", "moe"))
    store = gen.LogicalWeights(cfg, 7, "cpu", gains="random")
    W = O.OracleWeights(store)
    toks = np.random.default_rng(0).integers(0, cfg.vocab, size=30)
    full = O.forward_full(W, tokens=toks, parity=False, absorbed=False)
    outs, _ = _decode_all(W, cfg, toks, parity=False)
    for t in range(len(toks)):
        assert _rel(outs[t]["logits"], full["logits"][t]) < 1e-11


def test_prefill_then_decode_continues(tiny_cfg, tiny_store):
    """A decode step after the oracle prefill of the prompt equals the causal forward."""
    W = O.OracleWeights(tiny_store)
    toks = gen.prompt_tokens(tiny_cfg)[:40]
    st = O.prefill(W, toks[:32], max_len=40)
    assert st.length == 32
    full = O.forward_full(W, tokens=toks, parity=True, absorbed=False)
    for t in range(32, 40):
        out = O.decode_step(W, st, t, token=int(toks[t]), parity=True)
        assert _rel(out["logits"], full["logits"][t]) < 1e-12


def test_parity_rounding_points(tiny_cfg, tiny_store):
    """R1: cache rows are bf16 values. R2: each layer output is a bf16 value.
    Pure mode keeps neither, and the two modes stay within bf16 resolution."""
    W = O.OracleWeights(tiny_store)
    toks = gen.prompt_tokens(tiny_cfg)[:12]
    par, stp = _decode_all(W, tiny_cfg, toks, parity=True)
    pure, st0 = _decode_all(W, tiny_cfg, toks, parity=False)
    for l in range(tiny_cfg.n_layers):
        np.testing.assert_array_equal(O.bf16_round(stp.cache[l][:12]), stp.cache[l][:12])
        assert not np.array_equal(O.bf16_round(st0.cache[l][:12]), st0.cache[l][:12])
    for t in range(12):
        for h in par[t]["hidden"]:
            np.testing.assert_array_equal(O.bf16_round(h), h)
        assert _rel(par[t]["logits"], pure[t]["logits"]) < 2e-2


def test_bare_layer_stack_input(tiny_cfg, tiny_store):
    """A config without vocabulary runs from a hidden vector and returns only hidden taps."""
    cfg = tiny_cfg.with_(vocab=0)
    store = gen.LogicalWeights(cfg, 0, "cpu")
    W = O.OracleWeights(store)
    x = O.bf16_bits_to_f64(gen.layer_input(cfg, 0).numpy().view(np.uint16))
    st = O.DecodeState.empty(cfg, 4)
    out = O.decode_step(W, st, 0, x_in=x)
    assert "logits" not in out and len(out["hidden"]) == cfg.n_layers
    full = O.forward_full(W, xs=x[None, :], parity=True)
    assert _rel(out["hidden"][-1], full["hidden"][-1][0]) < 1e-12


def test_blocked_lm_head_matches_step_logits(tiny_cfg, tiny_store):
    """The row-blocked LM head equals the step's LM head for any block size,
    including blocks that do not divide the vocabulary."""
    W = O.OracleWeights(tiny_store)
    st = O.DecodeState.empty(tiny_cfg, 4)
    out = O.decode_step(W, st, 0, token=5)
    x = out["hidden"][-1]
    for rows in (7, 300, 2048, 5000):
        got = O.lm_logits(W, tiny_cfg, x, rows_per_block=rows)
        assert got.shape == out["logits"].shape
        assert _rel(got, out["logits"]) < 1e-13


def test_decode_equals_causal_forward_mxfp4_experts():
    """The same invariant with MXFP4 expert matrices (tiny_fp4): 40 positions."""
    cfg = configs.get("tiny_fp4")
    store = gen.LogicalWeights(cfg, 0, "cpu")
    W = O.OracleWeights(store)
    moe = cfg.layers.index("moe")
    assert "mx_codes" in store.numpy("w_gate", moe, 0)
    toks = gen.prompt_tokens(cfg)[:40]
    full = O.forward_full(W, tokens=toks, parity=True, absorbed=False)
    outs, _ = _decode_all(W, cfg, toks, True)
    for t in range(len(toks)):
        for l in range(cfg.n_layers):
            assert _rel(outs[t]["hidden"][l], full["hidden"][l][t]) < 1e-12, (t, l)
        assert outs[t]["argmax"] == int(np.argmax(full["logits"][t]))
