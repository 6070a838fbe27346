"""GPU parity of the MXFP4 expert path (expert_format "mxfp4"): the tiny and
ragged models with MXFP4 routed and shared experts, teacher-forced against the
oracle from a prefilled cache, and the host packer's blob against the device
packer's arena. The DeepSeek-V3-shaped MoE layer with MXFP4 experts is in
test_gpu_dsv3.py."""
import numpy as np
import pytest
import torch

import oracle as O
from synth import configs, gen

from parity_util import REL_TOL, assert_bf16_rows_match, cache_rows_bf16, rel_l2, teacher_forced

pytestmark = pytest.mark.gpu


def _case(name, steps):
    from persistent_decode_megakernel_amd import Engine
    cfg = configs.get(name)
    store = gen.LogicalWeights(cfg, 0, "cpu")
    W = O.OracleWeights(store)
    P = cfg.prompt_len
    state = O.prefill(W, gen.prompt_tokens(cfg), max_len=P + steps)
    st0 = state.copy()
    ref = teacher_forced(W, state, cfg, P, steps)
    eng = Engine(cfg, max_ctx=P + steps, device=0)
    eng.load_weights(store)
    eng.reset()
    for l in range(cfg.n_layers):
        eng.import_kv(l, 0, cache_rows_bf16(st0, l, P).cuda())
    return cfg, store, eng, ref, state


@pytest.mark.parametrize("name,steps", [("tiny_fp4", 16), ("ragged_fp4", 8)])
def test_mxfp4_experts_teacher_forced(name, steps):
    cfg, store, eng, ref, st_ref = _case(name, steps)
    assert cfg.expert_format == "mxfp4"
    P = cfg.prompt_len
    moe_layers = [l for l, k in enumerate(cfg.layers) if k == "moe"]
    worst = 0.0
    for j, (tok, out) in enumerate(ref):
        print(f"{name} step {j}", flush=True)
        am, lg = eng.decode(P + j, token=tok)
        rc, st = eng.status()
        assert rc == 0, (j, st.code, st.stage)
        taps = eng.taps()
        hid = taps["hidden"].cpu().numpy()
        for l in range(cfg.n_layers):
            e = rel_l2(hid[l], out["hidden"][l])
            worst = max(worst, e)
            assert e < REL_TOL, (j, l, e)
        assert rel_l2(lg.cpu().numpy(), out["logits"]) < REL_TOL, j
        assert int(am.item()) == out["argmax"], (j, int(am.item()), out["argmax"])
        ridx = taps["router_idx"].cpu().numpy()
        for i, l in enumerate(moe_layers):
            assert ridx[l].tolist() == [int(x) for x in out["router_idx"][i]], (j, l)
    got = eng.export_kv(0, P, len(ref)).view(torch.bfloat16).float().cpu().numpy().astype(np.float64)
    assert_bf16_rows_match(got, st_ref.cache[0][P:P + len(ref)], name)
    print(f"{name}: worst hidden rel err {worst:.2e}")


def test_mxfp4_host_packer_equals_device_packer():
    from persistent_decode_megakernel_amd import Engine, pack
    cfg = configs.get("tiny_fp4")
    store = gen.LogicalWeights(cfg, 0, "cpu")
    eng = Engine(cfg, max_ctx=cfg.prompt_len + 4, device=0)
    eng.load_weights(store)
    blob = pack.pack_store(cfg, store)
    dev = eng.weights.cpu().numpy()
    diff = np.nonzero(dev != blob)[0]
    assert diff.size == 0, f"{diff.size} bytes differ, first at {diff[:8].tolist()}"
