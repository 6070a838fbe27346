"""Helpers shared by the parity tests: margin-filtered teacher-forced streams
from the oracle, and comparison of engine outputs with oracle outputs."""
from __future__ import annotations

import numpy as np

import oracle as O
from synth import gen

MARGIN = 1e-3       # router logit gap at the k-th choice and LM top-1 gap
REL_TOL = 1e-2      # relative L2 error of hidden states and logits


def rel_l2(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def margins(cfg, out) -> float:
    """Smallest decision margin of one oracle step (router k-th gap, LM top-1 gap)."""
    m = np.inf
    for z in out.get("router_logits", []):
        s = np.sort(z)[::-1]
        m = min(m, s[cfg.top_k - 1] - s[cfg.top_k])
    if "logits" in out:
        s = np.sort(out["logits"])[::-1]
        m = min(m, s[0] - s[1])
    return m


def teacher_forced(W, state, cfg, pos0, n_steps, seed=0, max_attempts=40, x_inputs=False):
    """Run n_steps oracle decode steps from pos0 with tokens (or hidden inputs)
    redrawn until every step's router and LM margins exceed MARGIN.
    Returns a list of (input, oracle step output). Mutates `state`."""
    steps = []
    for j in range(n_steps):
        for attempt in range(max_attempts):
            trial = state.copy()
            if x_inputs:
                bits = gen.layer_input(cfg, j, attempt, seed).numpy().view(np.uint16)
                inp = O.bf16_bits_to_f64(bits)
                out = O.decode_step(W, trial, pos0 + j, x_in=inp)
                inp = bits
            else:
                inp = gen.decode_token(cfg, j, attempt, seed)
                out = O.decode_step(W, trial, pos0 + j, token=inp)
            if margins(cfg, out) > MARGIN:
                break
        else:
            raise AssertionError(f"no input with margin > {MARGIN} at step {j}")
        state.cache, state.length = trial.cache, trial.length
        steps.append((inp, out))
    return steps


def cache_rows_bf16(state, layer, n):
    """The oracle's first n cache rows of a layer as bf16 bit patterns (int16 tensor)."""
    import torch
    vals = state.cache[layer][:n]
    assert np.array_equal(O.bf16_round(vals), vals), "cache rows must be bf16 values"
    return torch.from_numpy(vals.astype(np.float32)).to(torch.bfloat16).view(torch.int16)
