"""GPU parity of the batched decode step (pdm_batch_decode_step): B sequences
with their own prompts, positions and caches step together; every sequence's
logits, argmax, layer outputs and appended cache rows must match the oracle's
batch-1 step of that sequence alone (oracle/model.py decode_step), on
margin-filtered teacher-forced inputs. Tolerances as the batch-1 engine's:
1e-2 relative L2 on hidden states and logits against the oracle's chain, exact
argmax, and every appended cache row equal, up to one bf16 step, to the row
the oracle computes from this path's own input of that layer."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle as O
from persistent_decode_megakernel_amd import _lib as L
from synth import configs, gen

from parity_util import REL_TOL, assert_bf16_rows_match, rel_l2, teacher_forced

pytestmark = pytest.mark.gpu


def _bits(v):
    return torch.from_numpy(O.bf16_round(v).astype(np.float32)).to(torch.bfloat16).view(torch.int16)


def _case(name, prompt_lens, steps, x_inputs=False):
    from persistent_decode_megakernel_amd import Engine
    cfg = configs.get(name)
    big = cfg.hidden >= 2048
    store = gen.LogicalWeights(cfg, 0, "cuda" if big else "cpu", cache=not big)
    W = O.OracleWeights(store, cache_limit_bytes=(8 << 30) if big else (2 << 30))
    B = len(prompt_lens)
    eng = Engine(cfg, max_ctx=max(prompt_lens) + steps + 1, device=0)
    eng.load_weights(store)
    caches = eng.batch_caches(B)
    states, streams = [], []
    for b, P in enumerate(prompt_lens):
        if big:   # N(0,1) latent prompt rows, as the single-layer parity tests
            st = O.DecodeState.empty(cfg, P + steps + 1)
            for l in range(cfg.n_layers):
                rows = gen.latent_rows(cfg, l, P, seed=b, device="cuda")
                st.cache[l][:P] = O.bf16_bits_to_f64(rows.cpu().numpy().view(np.uint16))
                caches[b, l, :P] = rows
            st.length = P
        else:     # an oracle prefill of the sequence's own prompt
            toks = gen.prompt_tokens(dataclasses.replace(cfg, prompt_len=max(P, cfg.prompt_len)), seed=b)[:P]
            st = O.prefill(W, toks, max_len=P + steps + 1)
            for l in range(cfg.n_layers):
                caches[b, l, :P] = _bits(st.cache[l][:P]).cuda()
        streams.append(teacher_forced(W, st, cfg, P, steps, seed=100 + b, x_inputs=x_inputs))
        states.append(st)
    return cfg, eng, caches, states, streams, W


def _check(name, prompt_lens, steps, x_inputs=False):
    cfg, eng, caches, states, streams, W = _case(name, prompt_lens, steps, x_inputs)
    B = len(prompt_lens)
    for j in range(steps):
        pos = [prompt_lens[b] + j for b in range(B)]
        hidden = torch.empty(cfg.n_layers, B, cfg.hidden, device="cuda")
        if x_inputs:
            x = torch.stack([torch.from_numpy(streams[b][j][0].view(np.int16).copy()) for b in range(B)]).cuda()
            am, lg = eng.batch_decode_step(pos, caches, x_in=x, hidden=hidden)
        else:
            am, lg = eng.batch_decode_step(pos, caches, tokens=[streams[b][j][0] for b in range(B)], hidden=hidden)
        torch.cuda.synchronize()
        hid = hidden.cpu().numpy().astype(np.float64)
        worst = 0.0
        for b in range(B):
            inp, out = streams[b][j]
            for l in range(cfg.n_layers):
                e = rel_l2(hid[l, b], out["hidden"][l])
                worst = max(worst, e)
                assert e < REL_TOL, (name, j, b, l, e)
                # the appended cache row, against the oracle's row from this
                # path's own layer input (the previous layer's bf16 output can
                # sit one rounding step from the oracle's chain)
                if l == 0:
                    x_l = O.bf16_bits_to_f64(inp) if x_inputs else W.bf16_row("embed", inp)
                else:
                    x_l = hid[l - 1, b]
                tmp = O.DecodeState.empty(cfg, pos[b] + 1)
                O.attention_decode(W, cfg, l, x_l, pos[b], tmp, parity=True)
                row = O.bf16_bits_to_f64(caches[b, l, pos[b]].cpu().numpy().view(np.uint16))
                assert_bf16_rows_match(row[None], tmp.cache[l][pos[b]][None], f"{name} seq {b} layer {l}")
            if cfg.vocab > 0:
                e = rel_l2(lg[b].cpu().numpy(), out["logits"])
                worst = max(worst, e)
                assert e < REL_TOL, (name, j, b, "logits", e)
                assert int(am[b].item()) == out["argmax"], (name, j, b)
        print(f"{name} step {j} (positions {pos}): worst rel L2 {worst:.2e}")
    return eng


def test_batch_step_tiny():
    """Three sequences at different positions (prompts of 16, 40 and 7 tokens)."""
    _check("tiny", [16, 40, 7], 3)


def test_batch_step_tiny_single():
    """One sequence: the router and LM head rows take the vector-ALU path."""
    _check("tiny", [33], 2)


def test_batch_step_tiny_sixteen():
    """The largest batch: 16 sequences with prompts of 1 to 60 tokens."""
    _check("tiny", [1, 7, 16, 40, 60, 3, 22, 35, 9, 48, 13, 2, 57, 30, 5, 44], 2)


def test_batch_step_tiny_long_context():
    """Five sequences (a token bound of 8 with three unused slots), one of them
    2100 positions long: attention chunks of two 64-position blocks."""
    _check("tiny", [2100, 12, 300, 64, 65], 2)


def test_batch_step_tiny_mxfp4():
    """The small model with MXFP4 routed and shared experts."""
    _check("tiny_fp4", [16, 40, 7], 2)


def test_batch_step_ragged():
    """24 heads (a padded second head group), two shared experts, top-3 of 12."""
    _check("ragged", [20, 33], 2)


def test_batch_step_dsv3_moe_layer():
    """DeepSeek-V3 MoE layer shapes, two sequences with 1024- and 700-position
    caches, bare-layer inputs."""
    _check("dsv3_moe_layer", [1024, 700], 1, x_inputs=True)


def test_batch_step_errors():
    from persistent_decode_megakernel_amd import Engine
    cfg = configs.get("tiny")
    eng = Engine(cfg, max_ctx=32, device=0)
    caches = eng.batch_caches(2)
    lg = torch.empty(2, cfg.vocab, device="cuda")
    am = torch.empty(2, dtype=torch.int32, device="cuda")
    assert eng.batch_decode_step_raw([1, 2], [0, 0], caches, logits=lg, argmax=am) == L.OK
    assert eng.batch_decode_step_raw([], [], caches, logits=lg) == L.ERR_ARG
    assert eng.batch_decode_step_raw([1] * 17, [0] * 17, caches, logits=lg) == L.ERR_ARG
    assert eng.batch_decode_step_raw([1, 2], [0, 32], caches, logits=lg) == L.ERR_CTX
    assert eng.batch_decode_step_raw([1, 2], [-1, 0], caches, logits=lg) == L.ERR_POS
    assert eng.batch_decode_step_raw([1, cfg.vocab], [0, 0], caches, logits=lg) == L.ERR_TOKEN
    assert eng.batch_decode_step_raw(None, [0, 0], caches, logits=lg) == L.ERR_TOKEN
    assert eng.batch_decode_step_raw([1, 2], [0, 0], caches, logits=None) == L.ERR_ARG
    assert eng.batch_decode_step_raw([1, 2], [0, 0], caches.view(-1)[1:], logits=lg) == L.ERR_ALIGN
    torch.cuda.synchronize()
    e4 = Engine(configs.get("tiny_fp4"), max_ctx=32, device=0)  # MXFP4 experts are served too
    assert e4.batch_decode_step_raw([1, 2], [0, 0], e4.batch_caches(2), logits=lg) == L.OK
    torch.cuda.synchronize()
