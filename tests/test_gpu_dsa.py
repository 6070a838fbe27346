"""GPU parity of sparse (DSA) decode attention (pdm_dsa_index_scores,
pdm_dsa_topk, pdm_dsa_attention) against the oracle (oracle/dsa.py).

Bars:
  * selection: bit-exact positions against the oracle's top-k of the same
    float32 scores (ties, -0.0 / +0.0, every position, one position, lists
    longer than the kernel's register-resident size);
  * indexer scores: |gpu - oracle| <= 1e-4 * sum_j |w_j| sum_i |q_ji k_si| +
    1e-6 per position (the query enters as bf16 high + residual parts, about
    2^-17 relative per product, accumulated in fp32);
  * attention: |gpu - oracle| <= 1e-4 on the latent outputs (cache values are
    N(0,1) bf16, an output is a convex combination of them; queries and
    probabilities enter as bf16 high + residual parts, ~2^-17 relative);
  * the whole path at the DeepSeek-V3 attention shape over a 9216-row cache:
    the GPU's selection is exact for its own scores and valid for the
    oracle's scores within the score bound."""
import numpy as np
import pytest
import torch

from oracle import dsa as D
from persistent_decode_megakernel_amd import _lib as L
from persistent_decode_megakernel_amd import dsa as G
from synth import gen

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _f64(bits: torch.Tensor) -> np.ndarray:
    return bits.view(torch.bfloat16).float().numpy().astype(np.float64)


def _score_bound(q, w, K):
    return 1e-4 * (np.abs(K) @ np.abs(q).T.astype(np.float64)) @ np.abs(w).astype(np.float64) + 1e-6


@pytest.mark.parametrize("n,HI,dI", [(1, 64, 128), (63, 64, 128), (64, 16, 32), (65, 32, 64), (1000, 48, 96),
                                     (9216, 64, 128), (5000, 64, 256), (70001, 64, 128), (33000, 16, 256)])
def test_index_scores(n, HI, dI):
    print(f"index scores n={n} HI={HI} dI={dI}", flush=True)
    q, w, keys, _, _, _ = gen.dsa_inputs(n, HI, dI, 16, 128, 32, tag=1)
    got = G.index_scores(torch.from_numpy(q).to(DEV), torch.from_numpy(w).to(DEV), keys.to(DEV)).cpu().numpy()
    K = _f64(keys)
    ref = D.index_scores(q, w, K)
    err = np.abs(got.astype(np.float64) - ref)
    bound = _score_bound(q, w, K)
    assert np.all(err <= bound), f"worst {np.max(err / bound):.2f} x bound at {int(np.argmax(err / bound))}"


TOPK_CASES = [(1, 1, "normal"), (5, 2, "normal"), (5, 9, "normal"), (100, 100, "ties"), (2047, 2048, "normal"),
              (2048, 2048, "normal"), (2049, 2048, "normal"), (9216, 2048, "normal"), (9216, 2048, "ties"),
              (9216, 64, "zeros"), (9216, 2048, "zeros"), (9216, 7, "equal"), (16384, 2048, "ties"),
              (16385, 2048, "normal"), (131072, 2048, "normal"), (131072, 2048, "ties"), (40000, 1, "normal"),
              (40000, 39999, "ties"), (20000, 20000, "normal"), (100000, 2048, "zeros"), (65537, 4096, "equal"),
              (300000, 2048, "normal")]


@pytest.mark.parametrize("n,k,kind", TOPK_CASES)
def test_topk_exact(n, k, kind):
    print(f"topk n={n} k={k} {kind}", flush=True)
    s = gen.dsa_scores_sample(n, kind, seed=n + k)
    got = G.topk(torch.from_numpy(s).to(DEV), k).cpu().numpy().astype(np.int64)
    np.testing.assert_array_equal(got, D.select_topk(s.astype(np.float64), k))


def test_topk_empty_and_arguments():
    s = torch.zeros(4, device=DEV)
    out = torch.full((4,), -7, dtype=torch.int32, device=DEV)
    work = torch.zeros(G.topk_work_bytes(4) // 4, dtype=torch.int32, device=DEV)
    call = lambda n, k: L.load().pdm_dsa_topk(G._p(s), n, k, G._p(out), G._p(work), work.numel() * 4,  # noqa: E731
                                              G._stream())
    assert call(0, 5) == L.OK
    assert call(4, 0) == L.OK
    torch.cuda.synchronize()
    assert out.cpu().tolist() == [-7] * 4       # nothing written
    assert call(-1, 5) == L.ERR_ARG


def test_topk_reuses_its_work_buffer():
    """Two long selections in a row through one work buffer (the histograms
    are cleared by each call), the second shorter."""
    work = torch.zeros(G.topk_work_bytes(131072) // 4, dtype=torch.int32, device=DEV)
    for n, k, kind in ((131072, 2048, "normal"), (50000, 300, "ties")):
        s = gen.dsa_scores_sample(n, kind, seed=7)
        got = G.topk(torch.from_numpy(s).to(DEV), k, work=work).cpu().numpy().astype(np.int64)
        np.testing.assert_array_equal(got, D.select_topk(s.astype(np.float64), k))


ATT_CASES = [  # H, dc, dr, rows, n_sel
    (128, 512, 64, 9216, 1), (128, 512, 64, 9216, 63), (128, 512, 64, 9216, 64), (128, 512, 64, 9216, 65),
    (128, 512, 64, 9216, 2048), (128, 512, 64, 9216, 2049), (128, 512, 64, 4096, 4096),
    (16, 256, 32, 700, 300), (20, 128, 32, 500, 129), (8, 128, 64, 80, 80)]


@pytest.mark.parametrize("H,dc,dr,rows,n_sel", ATT_CASES)
def test_sparse_attention(H, dc, dr, rows, n_sel):
    print(f"sparse attention H={H} dc={dc} dr={dr} rows={rows} n_sel={n_sel}", flush=True)
    _, _, _, cache, q_lat, q_pe = gen.dsa_inputs(rows, 16, 32, H, dc, dr, tag=2)
    rng = np.random.default_rng(rows + n_sel)
    sel = rng.choice(rows, n_sel, replace=False).astype(np.int32)
    tau = 1.0 / np.sqrt(192.0)
    got = G.attention(torch.from_numpy(q_lat).to(DEV), torch.from_numpy(q_pe).to(DEV), cache.to(DEV),
                      torch.from_numpy(sel).to(DEV), tau).cpu().numpy()
    C = _f64(cache)
    ref = D.sparse_mla(q_lat, q_pe, C[:, :dc], C[:, dc:], sel, tau)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-4)


def test_sparse_attention_order_and_clamp():
    """The list's order does not change the result beyond rounding; an entry
    past the cache reads the last row, never outside it."""
    H, dc, dr, rows = 32, 512, 64, 1000
    _, _, _, cache, q_lat, q_pe = gen.dsa_inputs(rows, 16, 32, H, dc, dr, tag=3)
    tau = 0.1
    args = (torch.from_numpy(q_lat).to(DEV), torch.from_numpy(q_pe).to(DEV), cache.to(DEV))
    sel = np.arange(0, 600, 3, dtype=np.int32)
    a = G.attention(*args, torch.from_numpy(sel).to(DEV), tau).cpu().numpy()
    b = G.attention(*args, torch.from_numpy(sel[::-1].copy()).to(DEV), tau).cpu().numpy()
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-5)
    over = sel.copy()
    over[5] = rows + 40
    last = sel.copy()
    last[5] = rows - 1
    c = G.attention(*args, torch.from_numpy(over).to(DEV), tau).cpu().numpy()
    d = G.attention(*args, torch.from_numpy(last).to(DEV), tau).cpu().numpy()
    np.testing.assert_array_equal(c, d)


def test_attention_argument_errors():
    lib = L.load()
    q = torch.zeros(16, 512, device=DEV)
    pe = torch.zeros(16, 64, device=DEV)
    cache = torch.zeros(10, 576, dtype=torch.int16, device=DEV)
    sel = torch.zeros(4, dtype=torch.int32, device=DEV)
    out = torch.zeros(16, 512, device=DEV)
    need = G.work_bytes(16, 512)
    work = torch.zeros(need // 4, device=DEV)
    p = G._p
    call = lambda dc, dr, n_sel, wb: lib.pdm_dsa_attention(  # noqa: E731
        p(q), p(pe), p(cache), 10, p(sel), n_sel, 16, dc, dr, 0.1, p(work), wb, p(out), G._stream())
    assert call(512, 64, 0, need) == L.ERR_ARG
    assert call(384, 64, 4, need) == L.ERR_CONFIG
    assert call(512, 65, 4, need) == L.ERR_CONFIG
    assert call(512, 64, 4, need - 4) == L.ERR_SIZE
    assert call(512, 64, 4, need) == L.OK
    torch.cuda.synchronize()


def test_dsa_path_deepseek_v3_shape():
    """Indexer (64 heads x 128), top-2048 of a 9216-row cache, attention of
    128 heads over the chosen rows, each step through the library."""
    n, HI, dI, H, dc, dr, k = 9216, 64, 128, 128, 512, 64, 2048
    q, w, keys, cache, q_lat, q_pe = gen.dsa_inputs(n, HI, dI, H, dc, dr, tag=4)
    tau = 1.0 / np.sqrt(192.0)
    sc = G.index_scores(torch.from_numpy(q).to(DEV), torch.from_numpy(w).to(DEV), keys.to(DEV))
    sel = G.topk(sc, k)
    o = G.attention(torch.from_numpy(q_lat).to(DEV), torch.from_numpy(q_pe).to(DEV), cache.to(DEV), sel, tau)
    sc, sel, o = sc.cpu().numpy(), sel.cpu().numpy().astype(np.int64), o.cpu().numpy()
    K = _f64(keys)
    ref_sc = D.index_scores(q, w, K)
    bound = _score_bound(q, w, K)
    assert np.all(np.abs(sc - ref_sc) <= bound)
    np.testing.assert_array_equal(sel, D.select_topk(sc.astype(np.float64), k))
    # valid for the oracle's scores: nothing left out scores clearly above anything chosen
    rest = np.setdiff1d(np.arange(n), sel)
    assert ref_sc[rest].max() <= ref_sc[sel].min() + 2 * bound.max()
    C = _f64(cache)
    np.testing.assert_allclose(o, D.sparse_mla(q_lat, q_pe, C[:, :dc], C[:, dc:], sel, tau), rtol=0, atol=1e-4)


def test_dsa_path_long_context():
    """The whole path over a 131072-row cache: the indexer's workgroups stride
    over several position groups and the selection runs over many
    workgroups; the attention is checked on the chosen rows."""
    n, HI, dI, H, dc, dr, k = 131072, 64, 128, 128, 512, 64, 2048
    print(f"dsa path n={n}", flush=True)
    q, w, keys, cache, q_lat, q_pe = gen.dsa_inputs(n, HI, dI, H, dc, dr, tag=5)
    tau = 1.0 / np.sqrt(192.0)
    sc = G.index_scores(torch.from_numpy(q).to(DEV), torch.from_numpy(w).to(DEV), keys.to(DEV))
    sel = G.topk(sc, k)
    o = G.attention(torch.from_numpy(q_lat).to(DEV), torch.from_numpy(q_pe).to(DEV), cache.to(DEV), sel, tau)
    sc, sel, o = sc.cpu().numpy(), sel.cpu().numpy().astype(np.int64), o.cpu().numpy()
    K = _f64(keys)
    ref_sc = D.index_scores(q, w, K)
    bound = _score_bound(q, w, K)
    assert np.all(np.abs(sc - ref_sc) <= bound)
    np.testing.assert_array_equal(sel, D.select_topk(sc.astype(np.float64), k))
    rest = np.setdiff1d(np.arange(n), sel)
    assert ref_sc[rest].max() <= ref_sc[sel].min() + 2 * bound.max()
    rows = _f64(cache[torch.from_numpy(sel)])
    np.testing.assert_allclose(o, D.sparse_mla(q_lat, q_pe, rows[:, :dc], rows[:, dc:], np.arange(k), tau),
                               rtol=0, atol=1e-4)
