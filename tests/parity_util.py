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


def bf16_ulps(got, want) -> np.ndarray:
    """Distance in bf16 steps between two arrays of bf16 values (given as
    floats): both are mapped to their 16-bit patterns, ordered so that
    consecutive bf16 numbers are consecutive integers (+0 and -0 coincide)."""
    def key(v):
        v = np.asarray(v, dtype=np.float64)
        assert np.array_equal(O.bf16_round(v), v), "values must be bf16 values"
        b = (v.astype(np.float32).view(np.uint32) >> 16).astype(np.int64)
        return np.where(b & 0x8000, -(b & 0x7FFF), b)
    return np.abs(key(got) - key(want))


ROW_ATOL = 1e-4     # absolute slack of a bf16 cache value, in units of its row's rms


def assert_bf16_rows_match(got, want, what=""):
    """Cache rows are bf16 on both sides (rounding point R1). An element may
    differ by one bf16 step where the fp32 value before rounding lies within
    summation-order noise of a rounding boundary. Near zero one bf16 step is
    smaller than that noise itself (an fp32 dot product of ~10^3 terms against
    the float64 one: ~10^-6 of the row's scale), so there the elements must
    instead agree to ROW_ATOL times the row's rms. Returns the number of
    elements one step apart."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    d = bf16_ulps(got, want)
    rms = np.sqrt(np.mean(want * want, axis=-1, keepdims=True))
    bad = (d > 1) & (np.abs(got - want) > ROW_ATOL * rms)
    if bad.any():
        i = np.argwhere(bad)[:4]
        raise AssertionError((what, int(bad.sum()), [(tuple(int(x) for x in ix), float(got[tuple(ix)]),
                                                      float(want[tuple(ix)]), int(d[tuple(ix)])) for ix in i]))
    return int((d == 1).sum())


def cache_rows_bf16(state, layer, n):
    """The oracle's first n cache rows of a layer as bf16 bit patterns (int16 tensor)."""
    import torch
    vals = state.cache[layer][:n]
    assert np.array_equal(O.bf16_round(vals), vals), "cache rows must be bf16 values"
    return torch.from_numpy(vals.astype(np.float32)).to(torch.bfloat16).view(torch.int16)


def poison_scratch(eng):
    """Fill the part of an engine's scratch buffer that every step must write
    before reading (logits, step-input tap, layer taps and all working
    activations: everything from the internal logits buffer on) with 0xFF
    bytes, a NaN pattern, so that a read of a value no stage wrote this step
    shows up in the results instead of reading zeros."""
    import ctypes as C
    from persistent_decode_megakernel_amd import _lib as L
    t = L.Taps()
    L.check("pdm_get_taps", eng.lib.pdm_get_taps(eng.h, C.byref(t)))
    off = t.logits_dev - eng.scratch.data_ptr()
    assert 0 < off < eng.scratch.numel()
    eng.scratch[off:].fill_(0xFF)


def isolated_cache_rows(W, cfg, pos, x0, hidden, caches):
    """The oracle's new cache row of every layer at position pos, each layer
    fed the engine's own input to it (x0 for layer 0, the engine's output of
    the layer before otherwise) and the engine's own cache rows [0, pos), so
    that only summation order separates the two sides."""
    out = []
    for l in range(cfg.n_layers):
        st = O.DecodeState.empty(cfg, pos + 1)
        st.cache[l][:pos] = caches[l][:pos]
        st.length = pos
        x_in = x0 if l == 0 else np.asarray(hidden[l - 1], dtype=np.float64)
        O.attention_decode(W, cfg, l, x_in, pos, st, True)
        out.append(st.cache[l][pos].copy())
    return out
