"""GPU parity of the batched products (pdm_batch_gemm, pdm_batch_ffn) against
the oracle's per-token definitions (oracle/batch.py), on the engine's own
packed weights.

Tolerance: activations enter the matrix cores as a bf16 high part plus a bf16
residual (representation error <= 2^-18 relative), FP8 weights are exact in
bf16, and products are summed in fp32 with per-slab partials added in no
fixed order. Every output element must lie within 4e-5 * sum_k |W_rk x_k| of
the float64 value (a dropped or misplaced term of a K <= 18432 sum moves it
by more), and each row within 1e-5 relative L2.
"""
import numpy as np
import pytest
import torch

import oracle as O
from persistent_decode_megakernel_amd import _lib as L
from synth import configs, gen

pytestmark = pytest.mark.gpu

ELEM_TOL, ROW_TOL = 4e-5, 1e-5


def packed_matrix(W, cfg, name, layer, expert, part):
    """Dequantised matrix in packed row order (the row map pdm_packed_layout
    documents), float64."""
    if name in ("wq_a", "wkv_a"):
        return np.concatenate([W("wq_a", layer), W("wkv_a", layer)])
    if name == "wkv_b":
        wkv = W("wkv_b", layer).reshape(cfg.n_heads, cfg.qk_nope + cfg.v_head, cfg.kv_lora)
        m = wkv[:, :cfg.qk_nope] if part == 0 else wkv[:, cfg.qk_nope:]
        return m.reshape(-1, cfg.kv_lora)
    if name in ("w_gate", "w_up"):
        g, u = W("w_gate", layer, expert), W("w_up", layer, expert)
        F = g.shape[0]
        out = np.empty((2 * F, g.shape[1]))
        v = out.reshape(F // 8, 16, g.shape[1])
        v[:, :8] = g.reshape(F // 8, 8, -1)
        v[:, 8:] = u.reshape(F // 8, 8, -1)
        return out
    return W(name, layer, expert)


def check_rows(got, ref, bound, what):
    err = np.abs(got - ref)
    worst = float((err / np.maximum(bound, 1e-300)).max())
    print(f"{what}: worst element error {worst:.2e} of sum |w x|")
    assert worst <= ELEM_TOL, f"{what}: element error {worst:.2e} of sum |w x|"
    for b in range(ref.shape[0]):
        rel = np.linalg.norm(got[b] - ref[b]) / np.linalg.norm(ref[b])
        assert rel <= ROW_TOL, f"{what}: row {b} rel L2 {rel:.2e}"


_ENGINES = {}


def engine(name):
    from persistent_decode_megakernel_amd import Engine
    if name not in _ENGINES:
        cfg = configs.get(name)
        store = gen.LogicalWeights(cfg, 0, "cpu" if cfg.hidden < 2048 else "cuda", cache=cfg.hidden < 2048)
        eng = Engine(cfg, max_ctx=64, device=0)
        eng.load_weights(store)
        _ENGINES[name] = (cfg, store, eng, O.OracleWeights(store))
    return _ENGINES[name]


def run_gemm(name, mats, batches):
    cfg, _, eng, W = engine(name)
    for tname, layer, expert, part in mats:
        Wp = packed_matrix(W, cfg, tname, layer, expert, part)
        for B in batches:
            X = gen.batch_rows(B, Wp.shape[1], seed=layer * 31 + B, tag=L.TENSOR_IDS[tname])
            y = eng.batch_gemm(L.TENSOR_IDS[tname], layer, torch.from_numpy(X).cuda(), expert=expert, part=part)
            torch.cuda.synchronize()
            Xd = X.astype(np.float64)
            check_rows(y.cpu().numpy().astype(np.float64), O.batch_gemm(Wp, Xd), np.abs(Xd) @ np.abs(Wp).T,
                       f"{name} {tname} l{layer} e{expert} p{part} B{B}")


def test_batch_gemm_tiny():
    run_gemm("tiny", [("wq_a", 0, -1, 0), ("wq_b", 1, -1, 0), ("wkv_b", 0, -1, 0), ("wkv_b", 1, -1, 1),
                      ("wo", 1, -1, 0), ("w_gate", 0, -1, 0), ("w_down", 0, -1, 0), ("w_gate", 1, 3, 0),
                      ("w_down", 1, 16, 0)], (1, 3, 8, 16))


def test_batch_gemm_ragged():
    """Columns that fill no 64-column window or 128-column scale block
    (hidden 1040, ffn 1072, moe_ffn 64) and row counts off a 128 multiple."""
    run_gemm("ragged", [("wq_a", 0, -1, 0), ("wo", 2, -1, 0), ("w_gate", 0, -1, 0), ("w_down", 0, -1, 0),
                        ("w_gate", 1, 11, 0), ("w_down", 2, 12, 0)], (2, 7))


def run_ffn(name, layer, B, seed, idx=None, w=None):
    cfg, _, eng, W = engine(name)
    H = gen.batch_rows(B, cfg.hidden, seed=seed, tag=100 + layer)
    moe = cfg.layers[layer] == "moe"
    if moe and idx is None:
        idx, w = gen.batch_routing(cfg, B, seed=seed)
    y = eng.batch_ffn(layer, torch.from_numpy(H).cuda(),
                      torch.from_numpy(idx).cuda() if moe else None, torch.from_numpy(w).cuda() if moe else None)
    torch.cuda.synchronize()
    got = y.cpu().numpy().astype(np.float64)
    keep = [(i[(i >= 0) & (i < cfg.n_experts)], ww[(i >= 0) & (i < cfg.n_experts)]) for i, ww in zip(idx, w)] \
        if moe else None
    ref = np.stack([O.batch_ffn(W, cfg, layer, H[b:b + 1].astype(np.float64),
                                [keep[b][0]] if moe else None, [keep[b][1]] if moe else None)[0]
                    for b in range(B)])
    rels = [np.linalg.norm(got[b] - ref[b]) / np.linalg.norm(ref[b]) for b in range(B)]
    n_u = len(set(np.concatenate([k[0] for k in keep]).tolist())) + cfg.n_shared if moe else 1
    print(f"{name} layer {layer} B{B}: {n_u} experts, worst token rel L2 {max(rels):.2e}")
    for b, rel in enumerate(rels):
        assert rel <= 2 * ROW_TOL, f"{name} layer {layer} B{B} token {b}: rel L2 {rel:.2e}"
    return got, ref


@pytest.mark.parametrize("B", [1, 2, 5, 8, 16])
def test_batch_ffn_tiny(B):
    run_ffn("tiny", 0, B, seed=B)   # dense SwiGLU
    run_ffn("tiny", 1, B, seed=B)   # MoE: union of the tokens' experts + shared


def test_batch_ffn_shared_choices_and_skips():
    """All tokens on the same experts (a union of top_k), and entries outside
    [0, n_experts) that the call skips."""
    cfg = configs.get("tiny")
    idx = np.tile(np.array([[5, 9]], dtype=np.int32), (6, 1))
    w = np.tile(np.array([[0.75, 0.25]], dtype=np.float32), (6, 1))
    run_ffn("tiny", 1, 6, seed=11, idx=idx, w=w)
    idx2 = idx.copy()
    idx2[1, 0], idx2[4, 1] = -1, cfg.n_experts
    run_ffn("tiny", 1, 6, seed=11, idx=idx2, w=w)


def test_batch_ffn_ragged():
    """Two shared experts, top-3 of 12, moe_ffn 64 (one K slab per expert)."""
    run_ffn("ragged", 1, 4, seed=3)
    run_ffn("ragged", 0, 3, seed=3)


def test_batch_errors():
    cfg, _, eng, _ = engine("tiny")
    x = torch.zeros(4, cfg.hidden + 4, device="cuda")
    y = torch.zeros(4, 4096, device="cuda")
    ok = eng.batch_gemm_raw(L.T_WO, 1, -1, 0, x, 4, y)
    assert ok == L.OK
    assert eng.batch_gemm_raw(L.T_WO, 1, -1, 0, x, 0, y) == L.ERR_ARG
    assert eng.batch_gemm_raw(L.T_WO, 1, -1, 0, x, 17, y) == L.ERR_ARG
    assert eng.batch_gemm_raw(L.T_WO, 1, -1, 0, None, 4, y) == L.ERR_ARG
    assert eng.batch_gemm_raw(L.T_WO, 1, -1, 0, x[:, 1:], 4, y) == L.ERR_ALIGN
    assert eng.batch_gemm_raw(L.T_WO, 9, -1, 0, x, 4, y) == L.ERR_ARG        # no such layer
    assert eng.batch_gemm_raw(L.T_ROUTER, 1, -1, 0, x, 4, y) == L.ERR_ARG    # not an FP8 matrix
    assert eng.batch_gemm_raw(L.T_WKV_B, 1, -1, 2, x, 4, y) == L.ERR_ARG     # no third part
    assert eng.batch_ffn_raw(1, x, 4, None, None, y) == L.ERR_ARG           # MoE layer needs routing
    assert eng.batch_ffn_raw(0, x, 4, None, None, y) == L.OK                # dense layer does not
    torch.cuda.synchronize()


def test_batch_gemm_mxfp4_experts():
    """MXFP4 expert matrices (e2m1 codes, an e8m0 scale per row and 32
    columns) on the matrix cores: routed and shared gate/up and down of the
    small model at B = 1, 3, 8, 16, and of the ragged one (hidden 1056: 33
    scale bytes per row, a last 64-column window only half inside the row) at
    B = 2, 7; the FP8 attention matrices of the same engines alongside."""
    run_gemm("tiny_fp4", [("w_gate", 1, 3, 0), ("w_down", 1, 3, 0), ("w_gate", 1, 16, 0), ("w_down", 1, 16, 0),
                          ("wo", 1, -1, 0)], (1, 3, 8, 16))
    run_gemm("ragged_fp4", [("w_gate", 1, 11, 0), ("w_down", 2, 12, 0), ("w_gate", 2, 13, 0), ("wq_a", 1, -1, 0)],
             (2, 7))


@pytest.mark.parametrize("B", [1, 5, 16])
def test_batch_ffn_mxfp4_experts(B):
    """The union-of-experts block over MXFP4 experts (the dense layer of the
    same model stays FP8)."""
    run_ffn("tiny_fp4", 1, B, seed=20 + B)
    run_ffn("tiny_fp4", 0, B, seed=20 + B)
    run_ffn("ragged_fp4", 1, min(B, 8), seed=30 + B)


def test_batch_dsv3_moe_layer():
    """DeepSeek-V3 shapes: B = 8 through W_O (K = 16384) and [W_DQ ; W_DKV] on
    sampled 128-row blocks, and the MoE block for B = 4 tokens (a union of
    about 30 of 256 experts plus the shared one) on every output."""
    cfg, store, eng, W = engine("dsv3_moe_layer")
    B = 8
    for tname, blocks in (("wo", (0, 27, 55)), ("wq_a", (0, 11, 16))):
        X = gen.batch_rows(B, cfg.hidden if tname == "wq_a" else cfg.n_heads * cfg.v_head, seed=5,
                           tag=L.TENSOR_IDS[tname])
        y = eng.batch_gemm(L.TENSOR_IDS[tname], 0, torch.from_numpy(X).cuda()).cpu().numpy().astype(np.float64)
        Xd = X.astype(np.float64)
        if tname == "wq_a":
            parts = [store.numpy("wq_a", 0), store.numpy("wkv_a", 0)]
            codes = np.concatenate([p["codes"] for p in parts])
            scales = [p["scales"] for p in parts]
        else:
            p = store.numpy("wo", 0)
            codes, scales = p["codes"], [p["scales"]]
        for blk in blocks:
            r0 = blk * 128
            r1 = min(r0 + 128, codes.shape[0])
            if tname == "wq_a" and r0 >= cfg.q_lora:   # second tensor: its own scale rows
                s = scales[1][(r0 - cfg.q_lora) // 128][None]
            else:
                s = scales[0][r0 // 128][None]
            Wb = O.dequant_fp8(codes[r0:r1], s)
            check_rows(y[:, r0:r1], O.batch_gemm(Wb, Xd), np.abs(Xd) @ np.abs(Wb).T, f"dsv3 {tname} rows {r0}")
    got, ref = run_ffn("dsv3_moe_layer", 0, 4, seed=2)
    assert got.shape == (4, cfg.hidden)
