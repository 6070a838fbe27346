"""Pins of the oracle's operators: closed forms, library routines, brute force,
and planted mistakes that the pins must catch."""
import itertools

import numpy as np
import pytest
import scipy.special as sp
import torch
import torch.nn.functional as F

import oracle as O
from oracle import model as M

RNG = np.random.default_rng(11)


# --------------------------------------------------------------------------- rmsnorm

def pin_rmsnorm():
    x = RNG.standard_normal((7, 96))
    g = 1.0 + 0.3 * RNG.standard_normal(96)
    for eps in (1e-6, 0.5):
        ref = F.rms_norm(torch.from_numpy(x), (96,), torch.from_numpy(g), eps=eps).numpy()
        np.testing.assert_allclose(O.rmsnorm(x, g, eps), ref, rtol=1e-12, atol=1e-14)
    # closed form on a constant vector: g * c / sqrt(c^2 + eps)
    c, eps = 0.37, 1e-6
    v = np.full(64, c)
    g = np.linspace(0.5, 1.5, 64)
    np.testing.assert_allclose(O.rmsnorm(v, g, eps), g * c / np.sqrt(c * c + eps), rtol=1e-14)


def test_rmsnorm():
    pin_rmsnorm()


# --------------------------------------------------------------------------- rope

def pin_rope():
    base = 10000.0
    d = 8
    v = RNG.standard_normal((5, d))
    pos = 13
    # consecutive pairs as complex numbers, rotated by pos * base^(-2i/d)
    z = v[:, 0::2] + 1j * v[:, 1::2]
    theta = pos * base ** (-2.0 * np.arange(d // 2) / d)
    zr = z * np.exp(1j * theta)
    ref = np.empty_like(v)
    ref[:, 0::2], ref[:, 1::2] = zr.real, zr.imag
    np.testing.assert_allclose(O.rope(v, pos, base), ref, rtol=1e-12, atol=1e-14)
    # position 0 is the identity, rotation preserves the norm
    np.testing.assert_array_equal(O.rope(v, 0, base), v)
    np.testing.assert_allclose(np.linalg.norm(O.rope(v, 977, base), axis=1), np.linalg.norm(v, axis=1), rtol=1e-12)
    # relative property: <R(m) q, R(n) k> == <R(m - n) q, k>
    q, k = RNG.standard_normal(64), RNG.standard_normal(64)
    for m, n in ((5, 3), (1000, 17), (9215, 9000)):
        lhs = O.rope(q, m, base) @ O.rope(k, n, base)
        rhs = O.rope(q, m - n, base) @ k
        assert abs(lhs - rhs) < 1e-9 * (1 + abs(rhs))
    # per-row positions broadcast like a loop over rows
    P = np.array([3, 70, 500])
    rows = RNG.standard_normal((3, 2, d))
    out = O.rope(rows, P[:, None], base)
    for i in range(3):
        np.testing.assert_allclose(out[i], O.rope(rows[i], P[i], base), rtol=1e-13)


def test_rope():
    pin_rope()


# --------------------------------------------------------------------------- softmax / silu / sigmoid

def pin_softmax():
    s = RNG.standard_normal((6, 300)) * 5
    p = O.softmax(s, axis=1)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-12)
    np.testing.assert_allclose(p, sp.softmax(s, axis=1), rtol=1e-12)
    np.testing.assert_allclose(O.softmax(s + 1000.0, axis=1), p, rtol=1e-12)


def test_softmax():
    pin_softmax()


def test_silu_sigmoid_library():
    z = RNG.standard_normal(1000) * 6
    np.testing.assert_allclose(M.silu(z), F.silu(torch.from_numpy(z)).numpy(), rtol=1e-13, atol=1e-300)
    np.testing.assert_allclose(M.sigmoid(z), sp.expit(z), rtol=1e-13)


# --------------------------------------------------------------------------- routing

def pin_topk():
    # exhaustive over all C(16, 2) subsets: the chosen set maximises the summed score
    for trial in range(20):
        z = RNG.standard_normal(16)
        idx, w = O.route(z, 2)
        sig = sp.expit(z)
        best = max(itertools.combinations(range(16), 2), key=lambda c: sum(sig[list(c)]))
        assert sorted(idx.tolist()) == sorted(best)
        assert abs(w.sum() - 1.0) < 1e-14
        np.testing.assert_allclose(w, sig[idx] / sig[idx].sum(), rtol=1e-14)
    for n in range(2, 13):
        for k in range(1, min(4, n) + 1):
            z = np.round(RNG.standard_normal(n), 1)  # coarse values make ties common
            idx = O.topk_indices(sp.expit(z), k)
            sig = sp.expit(z)
            # brute force: lexicographically (score desc, index asc) best k-subset
            cand = sorted(range(n), key=lambda i: (-sig[i], i))[:k]
            assert idx.tolist() == cand
            # every chosen score >= every unchosen score
            rest = [i for i in range(n) if i not in idx]
            if rest:
                assert sig[idx].min() >= sig[rest].max()


def test_topk():
    pin_topk()


def test_topk_ties_lower_index():
    z = np.array([0.5, 1.0, 1.0, 0.2, 1.0])
    assert O.topk_indices(z, 2).tolist() == [1, 2]
    assert O.topk_indices(z, 3).tolist() == [1, 2, 4]


# --------------------------------------------------------------------------- MLA

def _mla_inputs(H=4, dn=16, dr=8, dv=12, dc=32, T=9):
    qn = RNG.standard_normal((H, dn))
    qp = RNG.standard_normal((H, dr))
    C = RNG.standard_normal((T, dc))
    R = RNG.standard_normal((T, dr))
    W_UK = RNG.standard_normal((H, dn, dc)) * 0.2
    W_UV = RNG.standard_normal((H, dv, dc)) * 0.2
    return qn, qp, C, R, W_UK, W_UV, 1.0 / np.sqrt(dn + dr)


def pin_mla():
    qn, qp, C, R, W_UK, W_UV, tau = _mla_inputs()
    oa, pa = O.mla_absorbed(qn, qp, C, R, W_UK, W_UV, tau)
    on, pn = O.mla_naive(qn, qp, C, R, W_UK, W_UV, tau)
    np.testing.assert_allclose(oa, on, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(pa.sum(axis=1), 1.0, atol=1e-12)
    # the naive form is ordinary multi-head attention over per-head keys [K | R]
    # and values V with the default 1/sqrt(query width) scale
    H, T = qn.shape[0], C.shape[0]
    K = np.einsum("hnc,tc->htn", W_UK, C)
    V = np.einsum("hvc,tc->htv", W_UV, C)
    q = torch.from_numpy(np.concatenate([qn, qp], axis=1))[:, None, :]          # [H, 1, dn+dr]
    k = torch.from_numpy(np.concatenate([K, np.broadcast_to(R, (H,) + R.shape)], axis=2))
    ref = F.scaled_dot_product_attention(q, k, torch.from_numpy(V))[:, 0, :].numpy()
    np.testing.assert_allclose(oa, ref, rtol=1e-10, atol=1e-12)
    # one cached position: the probability is 1, so o[h] = W_UV[h] c
    o1, _ = O.mla_absorbed(qn, qp, C[:1], R[:1], W_UK, W_UV, tau)
    np.testing.assert_allclose(o1, np.einsum("hvc,c->hv", W_UV, C[0]), rtol=1e-12)
    # equal scores everywhere: the latent output is the mean of the cached latents
    Ceq = np.tile(C[:1], (T, 1))
    Req = np.tile(R[:1], (T, 1))
    oe, pe = O.mla_absorbed(qn, qp, Ceq + 0.0, Req, W_UK, W_UV, tau)
    np.testing.assert_allclose(pe, 1.0 / T, rtol=1e-12)


def test_mla():
    pin_mla()


# --------------------------------------------------------------------------- MoE special case

class _DictW:
    def __init__(self, d, cfg):
        self.d, self.cfg = d, cfg

    def __call__(self, name, layer=-1, expert=-1):
        return self.d[(name, layer, expert)]


def test_moe_one_expert_equals_dense():
    from synth import configs
    cfg = configs.get("tiny").with_(n_experts=1, top_k=1, n_shared=0, layers=("moe",))
    D, Fe = 24, 10
    cfg = cfg.with_(hidden=D, moe_ffn=Fe, ffn=Fe)
    g = RNG.standard_normal((Fe, D)) * 0.3
    u = RNG.standard_normal((Fe, D)) * 0.3
    dn = RNG.standard_normal((D, Fe)) * 0.3
    ws = {("ffn_norm", 0, -1): np.ones(D), ("router", 0, -1): RNG.standard_normal((1, D)),
          ("w_gate", 0, 0): g, ("w_up", 0, 0): u, ("w_down", 0, 0): dn,
          ("w_gate", 0, -1): g, ("w_up", 0, -1): u, ("w_down", 0, -1): dn}
    W = _DictW(ws, cfg)
    x = RNG.standard_normal(D)
    moe = M.ffn_decode(W, cfg, 0, x)
    dense = M.ffn_decode(W, cfg.with_(layers=("dense",)), 0, x)
    np.testing.assert_allclose(moe, dense, rtol=1e-14)
    # and the dense SwiGLU is down(silu(gate h) * up h) as torch composes it
    h = O.rmsnorm(x, np.ones(D), cfg.rms_eps)
    ref = (F.silu(torch.from_numpy(g @ h)) * torch.from_numpy(u @ h)).numpy() @ dn.T
    np.testing.assert_allclose(dense - x, ref, rtol=1e-12)


# --------------------------------------------------------------------------- MoE combination, closed forms
#
# The routed experts enter with their sigmoid scores normalised over the
# chosen set, every shared expert with weight 1 ("What is TileRT" section 5.2:
# routed experts with a few active per token; the combination rule itself is
# a reading). Router rows are built so that the logits take chosen values:
# with x = c * 1 and unit gains, h = RMSNorm(x) is the constant vector
# c / sqrt(c^2 + eps), and a router row t_e * u with u . h = 1 gives z_e = t_e.

def _swiglu_torch(g, u, dn, h):
    """down(silu(gate h) * (up h)), composed from torch's SiLU."""
    return (F.silu(torch.from_numpy(g @ h)) * torch.from_numpy(u @ h)).numpy() @ dn.T


def _moe_case(n_exp, top_k, n_shared, logits, D=32, Fe=12, seed=5):
    from synth import configs
    rng = np.random.default_rng(seed)
    cfg = configs.get("tiny").with_(hidden=D, moe_ffn=Fe, n_experts=n_exp, top_k=top_k,
                                    n_shared=n_shared, layers=("moe",))
    c = 0.7
    x = np.full(D, c)
    h = np.full(D, c / np.sqrt(c * c + cfg.rms_eps))
    u = h / (h @ h)
    ws = {("ffn_norm", 0, -1): np.ones(D),
          ("router", 0, -1): np.asarray(logits, dtype=np.float64)[:, None] * u[None, :]}
    mats = {}
    for e in range(n_exp + n_shared):
        mats[e] = (rng.standard_normal((Fe, D)) * 0.3, rng.standard_normal((Fe, D)) * 0.3,
                   rng.standard_normal((D, Fe)) * 0.3)
    return cfg, ws, mats, x, h


def _put(ws, mats):
    for e, (g, u, dn) in mats.items():
        ws[("w_gate", 0, e)], ws[("w_up", 0, e)], ws[("w_down", 0, e)] = g, u, dn
    return ws


def pin_moe_combination():
    sig = lambda t: 1.0 / (1.0 + np.exp(-np.asarray(t, dtype=np.float64)))
    # (1) top-1 with one shared expert whose weights equal the chosen routed
    #     expert's: the routed weight normalises to 1, the shared one is 1, so
    #     the FFN adds exactly twice that expert's SwiGLU
    cfg, ws, mats, x, h = _moe_case(4, 1, 1, [0.1, 2.0, -1.0, 0.5])
    mats[4] = mats[1]
    W = _DictW(_put(ws, mats), cfg)
    taps = {}
    y = M.ffn_decode(W, cfg, 0, x, taps) - x
    assert [int(i) for i in taps["router_idx"][0]] == [1]
    np.testing.assert_allclose(y, 2.0 * _swiglu_torch(*mats[1], h), rtol=1e-12, atol=1e-14)
    # (2) two routed experts with equal logits and no shared expert: 1/2 each
    cfg, ws, mats, x, h = _moe_case(5, 2, 0, [0.3, 1.25, -2.0, 1.25, 0.9])
    W = _DictW(_put(ws, mats), cfg)
    y = M.ffn_decode(W, cfg, 0, x) - x
    np.testing.assert_allclose(y, 0.5 * _swiglu_torch(*mats[1], h) + 0.5 * _swiglu_torch(*mats[3], h),
                               rtol=1e-12, atol=1e-14)
    # (3) general case: top-3 of 6 with two shared experts, unequal logits;
    #     weights sigma(t_i) / sum over the chosen three, shared with weight 1
    t = [0.2, -0.4, 1.7, 0.9, -1.1, 1.3]
    cfg, ws, mats, x, h = _moe_case(6, 3, 2, t)
    W = _DictW(_put(ws, mats), cfg)
    taps = {}
    y = M.ffn_decode(W, cfg, 0, x, taps) - x
    chosen = [2, 5, 3]
    assert [int(i) for i in taps["router_idx"][0]] == chosen
    w = sig([t[i] for i in chosen])
    w = w / w.sum()
    want = _swiglu_torch(*mats[6], h) + _swiglu_torch(*mats[7], h)
    for wi, e in zip(w, chosen):
        want = want + wi * _swiglu_torch(*mats[e], h)
    np.testing.assert_allclose(y, want, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(taps["router_w"][0], w, rtol=1e-14)


def test_moe_combination_closed_forms():
    pin_moe_combination()


# --------------------------------------------------------------------------- planted mistakes

def _expect_pin_failure(monkeypatch, target, attr, bad, pin):
    monkeypatch.setattr(target, attr, bad)
    with pytest.raises(AssertionError):
        pin()


def test_planted_mistakes_are_caught(monkeypatch):
    good_rope = M.rope

    def rope_half_split(v, pos, base):  # rotates (i, i + d/2) instead of (2i, 2i + 1)
        d = v.shape[-1]
        perm = np.concatenate([np.arange(0, d, 2), np.arange(1, d, 2)])
        inv = np.argsort(perm)
        return good_rope(v[..., inv], pos, base)[..., perm]
    with monkeypatch.context() as mp:
        _expect_pin_failure(mp, O, "rope", rope_half_split, pin_rope)

    with monkeypatch.context() as mp:
        _expect_pin_failure(mp, O, "rope", lambda v, pos, base: good_rope(v, -pos, base), pin_rope)

    with monkeypatch.context() as mp:
        _expect_pin_failure(mp, O, "rmsnorm",
                            lambda v, g, eps: v / (np.sqrt(np.mean(v * v, -1, keepdims=True)) + eps) * g,
                            pin_rmsnorm)

    good_abs = M.mla_absorbed
    with monkeypatch.context() as mp:   # softmax scale dropped
        _expect_pin_failure(mp, O, "mla_absorbed",
                            lambda qn, qp, C, R, UK, UV, tau: good_abs(qn, qp, C, R, UK, UV, 1.0), pin_mla)
    with monkeypatch.context() as mp:   # rotary term of the score dropped
        _expect_pin_failure(mp, O, "mla_absorbed",
                            lambda qn, qp, C, R, UK, UV, tau: good_abs(qn, 0 * qp, C, R, UK, UV, tau), pin_mla)
    with monkeypatch.context() as mp:   # key and value projections swapped
        _expect_pin_failure(mp, O, "mla_absorbed",
                            lambda qn, qp, C, R, UK, UV, tau: good_abs(qn, qp, C, R, UK, UK[:, :UV.shape[1]], tau),
                            pin_mla)

    with monkeypatch.context() as mp:   # picks the smallest scores
        _expect_pin_failure(mp, O, "route",
                            lambda z, k: (np.argsort(z, kind="stable")[:k], np.full(k, 1.0 / k)), pin_topk)
    with monkeypatch.context() as mp:   # weights not normalised
        _expect_pin_failure(mp, O, "route",
                            lambda z, k: (O.topk_indices(sp.expit(z), k), sp.expit(z)[O.topk_indices(sp.expit(z), k)]),
                            pin_topk)
    with monkeypatch.context() as mp:
        _expect_pin_failure(mp, O, "softmax", lambda s, axis=-1: np.exp(s) / np.exp(s).sum(axis=axis, keepdims=True) * 1.01,
                            pin_softmax)

    # MoE combination mistakes: shared expert dropped, shared expert scaled by
    # the first routed weight, routed weights left unnormalised
    good_ffn = M.ffn_decode

    def ffn_variant(shared_w, normalise):
        def ffn(W, cfg, l, x, taps=None):
            h2 = M.rmsnorm(x, W("ffn_norm", l), cfg.rms_eps)
            z = W("router", l) @ h2
            s = M.sigmoid(z)
            idx = M.topk_indices(s, cfg.top_k)
            w = s[idx] / np.sum(s[idx]) if normalise else s[idx]
            y = np.zeros_like(x)
            for j in range(cfg.n_shared):
                y = y + shared_w(w) * M.swiglu(W, l, cfg.n_experts + j, h2)
            for e, we in zip(idx, w):
                y = y + we * M.swiglu(W, l, int(e), h2)
            if taps is not None:
                taps.setdefault("router_logits", []).append(z)
                taps.setdefault("router_idx", []).append(idx)
                taps.setdefault("router_w", []).append(w)
            return x + y
        return ffn
    # the variant with the reading's own choices passes (the harness is sound)
    with monkeypatch.context() as mp:
        mp.setattr(M, "ffn_decode", ffn_variant(lambda w: 1.0, True))
        pin_moe_combination()
    for bad in (ffn_variant(lambda w: 0.0, True), ffn_variant(lambda w: w[0], True),
                ffn_variant(lambda w: 1.0, False)):
        with monkeypatch.context() as mp:
            _expect_pin_failure(mp, M, "ffn_decode", bad, pin_moe_combination)
    assert M.ffn_decode is good_ffn
