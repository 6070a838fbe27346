"""Pins of the batched oracle (oracle/batch.py): a batch is B independent
tokens, so its rows must equal the batch-1 definitions they restate."""
import numpy as np

import oracle as O
from synth import gen


def test_batch_gemm_brute_force():
    """Y[b, r] against a pure-Python triple loop on a tiny ragged shape."""
    rng = np.random.default_rng(7)
    W, X = rng.standard_normal((7, 5)), rng.standard_normal((3, 5))
    Y = O.batch_gemm(W, X)
    assert Y.shape == (3, 7)
    for b in range(3):
        for r in range(7):
            s = 0.0
            for k in range(5):
                s += W[r, k] * X[b, k]
            assert abs(Y[b, r] - s) <= 1e-14 * max(1.0, abs(s))


def _ffn_input(W, cfg, l, seed):
    x = gen.batch_rows(1, cfg.hidden, seed=seed, tag=9)[0].astype(np.float64)
    return x, O.rmsnorm(x, W("ffn_norm", l), cfg.rms_eps)


def test_batch_ffn_one_token_is_ffn_decode(tiny_cfg, tiny_store):
    """A batch of one token with its own routing is the batch-1 FFN block
    minus the residual (dense layer 0 and MoE layer 1 of the tiny model)."""
    cfg, W = tiny_cfg, O.OracleWeights(tiny_store)
    for l in range(cfg.n_layers):
        x, h = _ffn_input(W, cfg, l, 3 + l)
        if cfg.layers[l] == "moe":
            idx, w = O.route(W("router", l) @ h, cfg.top_k)
            got = O.batch_ffn(W, cfg, l, h[None], idx[None], w[None])[0]
        else:
            got = O.batch_ffn(W, cfg, l, h[None])[0]
        ref = O.ffn_decode(W, cfg, l, x) - x
        assert np.linalg.norm(got - ref) <= 1e-12 * np.linalg.norm(ref), l


def test_batch_ffn_rows_are_independent(tiny_cfg, tiny_store):
    """Each row is its token alone; permuting the tokens permutes the rows;
    a zero routing weight drops an expert (only the shared ones remain)."""
    cfg, W = tiny_cfg, O.OracleWeights(tiny_store)
    l = 1
    H = gen.batch_rows(5, cfg.hidden, seed=1).astype(np.float64)
    idx, w = gen.batch_routing(cfg, 5, seed=1)
    Y = O.batch_ffn(W, cfg, l, H, idx, w)
    for b in range(5):
        np.testing.assert_array_equal(Y[b], O.batch_ffn(W, cfg, l, H[b:b + 1], idx[b:b + 1], w[b:b + 1])[0])
    p = np.array([3, 0, 4, 1, 2])
    np.testing.assert_array_equal(O.batch_ffn(W, cfg, l, H[p], idx[p], w[p]), Y[p])
    shared = sum(O.model.swiglu(W, l, cfg.n_experts + j, H[0]) for j in range(cfg.n_shared))
    np.testing.assert_allclose(O.batch_ffn(W, cfg, l, H[:1], idx[:1], np.zeros_like(w[:1]))[0], shared,
                               rtol=1e-13, atol=0)


def test_batch_routing_shape(tiny_cfg):
    """The synthetic routing draws distinct experts with weights summing to 1."""
    idx, w = gen.batch_routing(tiny_cfg, 16, seed=2)
    assert idx.shape == w.shape == (16, tiny_cfg.top_k)
    assert all(len(set(r.tolist())) == tiny_cfg.top_k for r in idx)
    assert idx.min() >= 0 and idx.max() < tiny_cfg.n_experts
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-6)
    assert (w > 0).all()
