"""GPU parity of the persistent engine against the oracle on the small
two-layer MLA + MoE stack (dense + MoE, 256-token prefill, 64 decode steps),
plus edge cases of the C ABI. Run on an MI355X through the HIP library."""
import numpy as np
import pytest
import torch

import oracle as O
from synth import configs, gen

from parity_util import (REL_TOL, assert_bf16_rows_match, cache_rows_bf16, isolated_cache_rows, poison_scratch,
                         rel_l2, teacher_forced)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tiny_case():
    from persistent_decode_megakernel_amd import Engine
    cfg = configs.get("tiny")
    store = gen.LogicalWeights(cfg, 0, "cpu")
    W = O.OracleWeights(store)
    P = cfg.prompt_len
    state = O.prefill(W, gen.prompt_tokens(cfg), max_len=P + cfg.decode_steps)
    prefill_state = state.copy()
    steps = teacher_forced(W, state, cfg, P, cfg.decode_steps)
    eng = Engine(cfg, max_ctx=P + cfg.decode_steps, device=0, trace=True)
    eng.load_weights(store)
    return cfg, store, W, prefill_state, steps, eng


def _import_prefill(eng, cfg, st, n):
    eng.reset()
    for l in range(cfg.n_layers):
        eng.import_kv(l, 0, cache_rows_bf16(st, l, n).cuda())


def test_tiny_teacher_forced_parity(tiny_case):
    cfg, store, W, st0, steps, eng = tiny_case
    P = cfg.prompt_len
    _import_prefill(eng, cfg, st0, P)
    worst = {"logits": 0.0, "hidden": 0.0}
    for j, (tok, ref) in enumerate(steps):
        am, lg = eng.decode(P + j, token=tok)
        rc, st = eng.status()
        assert rc == 0, (j, st.code, st.stage)
        taps = eng.taps()
        hid = taps["hidden"].cpu().numpy()
        for l in range(cfg.n_layers):
            e = rel_l2(hid[l], ref["hidden"][l])
            worst["hidden"] = max(worst["hidden"], e)
            assert e < REL_TOL, (j, l, e)
        e = rel_l2(lg.cpu().numpy(), ref["logits"])
        worst["logits"] = max(worst["logits"], e)
        assert e < REL_TOL, (j, e)
        assert int(am.item()) == ref["argmax"], (j, int(am.item()), ref["argmax"])
        ridx = taps["router_idx"].cpu().numpy()
        moe_layers = [l for l, k in enumerate(cfg.layers) if k == "moe"]
        for i, l in enumerate(moe_layers):
            assert ridx[l].tolist() == [int(x) for x in ref["router_idx"][i]], (j, l)
            np.testing.assert_allclose(taps["router_w"].cpu().numpy()[l], ref["router_w"][i], rtol=1e-4)
    print(f"worst rel err over {len(steps)} steps: {worst}")


def test_tiny_poisoned_scratch(tiny_case):
    """Working buffers start as NaN bytes: every value a step reads is written
    earlier in the same step, so the results still match the oracle."""
    cfg, store, W, st0, steps, eng = tiny_case
    P = cfg.prompt_len
    _import_prefill(eng, cfg, st0, P)
    for j, (tok, ref) in enumerate(steps[:6]):
        poison_scratch(eng)
        am, lg = eng.decode(P + j, token=tok)
        assert eng.status()[0] == 0
        got = lg.cpu().numpy()
        assert np.isfinite(got).all(), j
        assert rel_l2(got, ref["logits"]) < REL_TOL, j
        assert int(am.item()) == ref["argmax"], j
        hid = eng.taps()["hidden"].cpu().numpy()
        for l in range(cfg.n_layers):
            assert rel_l2(hid[l], ref["hidden"][l]) < REL_TOL, (j, l)


def test_tiny_cache_rows_match_oracle(tiny_case):
    """Every appended cache row against the oracle's row for the same layer
    input (isolated per layer), element by element."""
    cfg, store, W, st0, steps, eng = tiny_case
    P = cfg.prompt_len
    _import_prefill(eng, cfg, st0, P)
    n1 = 0
    for j, (tok, _) in enumerate(steps[:8]):
        pos = P + j
        eng.decode(pos, token=tok)
        assert eng.status()[0] == 0
        hid = eng.taps()["hidden"].cpu().numpy()
        caches = [eng.export_kv(l, 0, pos + 1).view(torch.bfloat16).float().cpu().numpy().astype(np.float64)
                  for l in range(cfg.n_layers)]
        want = isolated_cache_rows(W, cfg, pos, W.bf16_row("embed", tok), hid, caches)
        for l in range(cfg.n_layers):
            n1 += assert_bf16_rows_match(caches[l][pos], want[l], f"step {j} layer {l}")
    print(f"{n1} cache values one bf16 step apart over 8 steps")


def test_tiny_from_empty_cache(tiny_case):
    """Decode from position 0 (context 1, no prefill) for a few steps."""
    cfg, store, W, st0, steps, eng = tiny_case
    eng.reset()
    st = O.DecodeState.empty(cfg, 16)
    toks = gen.prompt_tokens(cfg)[:6]
    for t, tok in enumerate(toks):
        ref = O.decode_step(W, st, t, token=int(tok))
        am, lg = eng.decode(t, token=int(tok))
        rc, _ = eng.status()
        assert rc == 0
        assert rel_l2(lg.cpu().numpy(), ref["logits"]) < REL_TOL, t


def test_abi_argument_errors(tiny_case):
    from persistent_decode_megakernel_amd import _lib as L
    cfg, store, W, st0, steps, eng = tiny_case
    eng.reset()
    assert eng.decode_raw(1, token=5) == L.ERR_POS                 # cache is empty: pos must be 0
    assert eng.decode_raw(0, token=cfg.vocab) == L.ERR_TOKEN       # token out of range
    assert eng.decode_raw(0, token=-3) == L.ERR_TOKEN
    assert eng.decode_raw(eng.max_ctx, token=1) == L.ERR_CTX
    rows = torch.zeros(4, cfg.kv_row, dtype=torch.int16, device="cuda")
    for l in range(cfg.n_layers):
        eng.import_kv(l, 0, rows)
    assert eng.cache_length() == 4
    with pytest.raises(L.PdmError):
        eng.import_kv(0, 9, rows)                                   # gap in the cache
    with pytest.raises(L.PdmError):
        eng.import_kv(0, eng.max_ctx - 2, rows)                     # past max_ctx


def test_last_position_fits(tiny_case):
    """The step at pos = max_ctx - 1 (cache full after it) runs and matches the oracle."""
    cfg, store, W, st0, steps, eng = tiny_case
    n = eng.max_ctx - 1
    st = st0.copy()
    # extend the oracle cache to n rows with the teacher-forced steps
    P = cfg.prompt_len
    for j, (tok, _) in enumerate(steps[:n - P]):
        O.decode_step(W, st, P + j, token=tok)
    _import_prefill(eng, cfg, st, n)
    tok = steps[-1][0]
    ref = O.decode_step(W, st, n, token=tok)
    am, lg = eng.decode(n, token=tok)
    assert eng.status()[0] == 0
    assert rel_l2(lg.cpu().numpy(), ref["logits"]) < REL_TOL


def test_watchdog_trips_and_recovers(tiny_case):
    """A stage that never signals trips the bounded wait; reset recovers."""
    from persistent_decode_megakernel_amd import _lib as L
    cfg, store, W, st0, steps, eng = tiny_case
    _import_prefill(eng, cfg, st0, cfg.prompt_len)
    eng.set_debug(spin_limit=2000, skip_signal_stage=3)
    eng.decode(cfg.prompt_len, token=steps[0][0])
    rc, st = eng.status()
    assert rc == L.ERR_WATCHDOG and st.stage > 3, (rc, st.stage)
    eng.set_debug(0, -1)
    _import_prefill(eng, cfg, st0, cfg.prompt_len)
    am, lg = eng.decode(cfg.prompt_len, token=steps[0][0])
    assert eng.status()[0] == 0
    assert int(am.item()) == steps[0][1]["argmax"]


def test_packed_blob_roundtrip(tiny_case):
    """The weight arena is the packed blob: a second engine loads it and matches."""
    from persistent_decode_megakernel_amd import Engine, _lib as L
    cfg, store, W, st0, steps, eng = tiny_case
    blob = eng.weights.clone()
    eng2 = Engine(cfg, max_ctx=eng.max_ctx, device=0)
    eng2.load_packed(blob)
    bad = blob.clone()
    bad[0] ^= 1
    with pytest.raises(L.PdmError):
        eng2.load_packed(bad)
    for e in (eng, eng2):
        _import_prefill(e, cfg, st0, cfg.prompt_len)
    a1, l1 = eng.decode(cfg.prompt_len, token=steps[0][0])
    a2, l2 = eng2.decode(cfg.prompt_len, token=steps[0][0])
    torch.cuda.synchronize()
    assert int(a1.item()) == int(a2.item())
    assert torch.equal(l1, l2)


def test_host_packer_equals_device_packer(tiny_case):
    """The host packer's blob (pdm_pack_*) is byte for byte the weight arena the
    device packer (pdm_load_fp8 / pdm_load_raw) and pdm_bind produced, and an
    engine loaded from it decodes like the original."""
    from persistent_decode_megakernel_amd import Engine, pack
    cfg, store, W, st0, steps, eng = tiny_case
    blob = pack.pack_store(cfg, store)
    dev = eng.weights.cpu().numpy()
    assert dev.nbytes == blob.nbytes
    diff = np.nonzero(dev != blob)[0]
    assert diff.size == 0, f"{diff.size} bytes differ, first at {diff[:8].tolist()}"
    eng2 = Engine(cfg, max_ctx=eng.max_ctx, device=0)
    eng2.load_packed(torch.from_numpy(blob))
    torch.cuda.synchronize()
    for e in (eng, eng2):
        _import_prefill(e, cfg, st0, cfg.prompt_len)
    a1, l1 = eng.decode(cfg.prompt_len, token=steps[0][0])
    a2, l2 = eng2.decode(cfg.prompt_len, token=steps[0][0])
    torch.cuda.synchronize()
    assert int(a1.item()) == int(a2.item()) and torch.equal(l1, l2)


def test_trace_records(tiny_case):
    cfg, store, W, st0, steps, eng = tiny_case
    _import_prefill(eng, cfg, st0, cfg.prompt_len)
    eng.decode(cfg.prompt_len, token=steps[0][0])
    assert eng.status()[0] == 0
    taps = eng.taps()
    tr = taps["trace"].cpu().numpy()
    assert (tr[:, :, 3] == taps["epoch"]).all()
    assert (tr[:, :, 2] >= tr[:, :, 1]).all() and (tr[:, :, 1] >= tr[:, :, 0]).all()
    # intra-stage marks: 0 where a stage has none, else ordered inside [ready, done]
    for i in (4, 5, 6):
        m = tr[:, :, i]
        has = m != 0
        assert (m[has] >= tr[:, :, 1][has]).all() and (m[has] <= tr[:, :, 2][has]).all()
    # stage entry precedes the dependency wait
    assert (tr[:, :, 7] > 0).all() and (tr[:, :, 7] <= tr[:, :, 0]).all()
