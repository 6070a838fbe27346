"""GPU parity at DeepSeek-V3 shapes: one dense layer and one MoE layer
(hidden 7168, 128 MLA heads, 256 experts top-8 + 1 shared) over a
1024-position synthetic latent cache, in the engine's benchmark launch
configuration (one 256-workgroup persistent launch per step)."""
import numpy as np
import pytest
import torch

import oracle as O
from synth import configs, gen

from parity_util import REL_TOL, assert_bf16_rows_match, rel_l2, teacher_forced

pytestmark = pytest.mark.gpu


def _layer_case(name, steps):
    from persistent_decode_megakernel_amd import Engine
    cfg = configs.get(name)
    P = cfg.prompt_len
    store = gen.LogicalWeights(cfg, 0, "cuda", cache=False)
    eng = Engine(cfg, max_ctx=P + steps + 1, device=0)
    eng.load_weights(store)
    st = O.DecodeState.empty(cfg, P + steps + 1)
    lat = []
    for l in range(cfg.n_layers):
        rows = gen.latent_rows(cfg, l, P, 0, device="cuda")
        lat.append(rows)
        st.cache[l][:P] = O.bf16_bits_to_f64(rows.cpu().numpy().view(np.uint16))
        eng.import_kv(l, 0, rows)
    st.length = P
    W = O.OracleWeights(store, cache_limit_bytes=8 << 30)
    ref = teacher_forced(W, st, cfg, P, steps, x_inputs=True)
    return cfg, eng, ref, st


@pytest.mark.parametrize("name,steps", [("dsv3_dense_layer", 3), ("dsv3_moe_layer", 3), ("dsv3_moe_layer_fp4", 3)])
def test_dsv3_layer_parity(name, steps):
    cfg, eng, ref, st_ref = _layer_case(name, steps)
    P = cfg.prompt_len
    for j, (bits, out) in enumerate(ref):
        x = torch.from_numpy(bits.view(np.int16).copy()).cuda()
        eng.decode(P + j, x_in=x)
        rc, st = eng.status()
        assert rc == 0, (j, st.stage)
        taps = eng.taps()
        x0 = O.bf16_bits_to_f64(bits)
        xa = taps["hidden_attn"][0].cpu().numpy().astype(np.float64)
        xo = taps["hidden"][0].cpu().numpy().astype(np.float64)
        e_attn = rel_l2(xa, out["hidden_attn"][0])
        e = rel_l2(xo, out["hidden"][0])
        # the residual input dominates the sums: also compare what each sublayer adds
        d_attn = rel_l2(xa - x0, out["hidden_attn"][0] - x0)
        d_ffn = rel_l2(xo - xa, out["hidden"][0] - out["hidden_attn"][0])
        print(f"{name} step {j}: rel err attn {e_attn:.2e} layer {e:.2e}; "
              f"attention delta {d_attn:.2e} ffn delta {d_ffn:.2e}")
        assert e_attn < REL_TOL and e < REL_TOL, (j, e_attn, e)
        assert d_attn < REL_TOL and d_ffn < REL_TOL, (j, d_attn, d_ffn)
        if cfg.layers[0] == "moe":
            assert taps["router_idx"][0].cpu().numpy().tolist() == [int(i) for i in out["router_idx"][0]]
            np.testing.assert_allclose(taps["router_w"][0].cpu().numpy(), out["router_w"][0], rtol=1e-4)
    # the appended cache rows equal the oracle's bf16 rows (up to an ulp where fp32 rounding differs)
    got = eng.export_kv(0, P, len(ref)).view(torch.bfloat16).float().cpu().numpy().astype(np.float64)
    assert_bf16_rows_match(got, st_ref.cache[0][P:P + len(ref)], name)
