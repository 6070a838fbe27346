"""The allocation-free binding (pdm_bind_static: scratch in the library's
static per-device array) against the ordinary binding (caller-owned scratch)
through the C ABI: two bindings in a row on one device, the second with a
smaller engine (fewer positions), every decode step's logits and argmax and
the appended cache rows identical."""
import numpy as np
import pytest
import torch

import oracle as O
from synth import configs, gen

from parity_util import cache_rows_bf16, teacher_forced

pytestmark = pytest.mark.gpu


def _run(eng, cfg, st0, P, steps):
    eng.reset()
    for l in range(cfg.n_layers):
        eng.import_kv(l, 0, cache_rows_bf16(st0, l, P).cuda())
    out = []
    for j, (tok, _) in enumerate(steps):
        lg = torch.empty(cfg.vocab, dtype=torch.float32, device="cuda")
        am = torch.zeros(1, dtype=torch.int32, device="cuda")
        eng.decode(P + j, token=tok, logits=lg, argmax=am)
        out.append((lg, am))
    rc, st = eng.status()
    assert rc == 0, (rc, st.stage)
    kv = [eng.export_kv(l, P, len(steps)).cpu() for l in range(cfg.n_layers)]
    return [(lg.cpu(), int(am.item())) for lg, am in out], kv


@pytest.mark.parametrize("P,n_steps", [(256, 8), (96, 4)])
def test_static_scratch_matches_caller_scratch(P, n_steps):
    from persistent_decode_megakernel_amd import Engine
    from persistent_decode_megakernel_amd import _lib as L
    cfg = configs.get("tiny")
    store = gen.LogicalWeights(cfg, 0, "cpu")
    W = O.OracleWeights(store)
    st = O.prefill(W, gen.prompt_tokens(cfg)[:P], max_len=P + n_steps)
    st0 = st.copy()
    steps = teacher_forced(W, st, cfg, P, n_steps)
    max_ctx = P + n_steps
    ref = Engine(cfg, max_ctx=max_ctx, device=0)
    ref.load_weights(store)
    eng = Engine(cfg, max_ctx=max_ctx, device=0, static_scratch=True)
    assert eng.sizes.scratch_bytes <= L.STATIC_SCRATCH_BYTES
    eng.load_packed(ref.weights)
    a, kva = _run(ref, cfg, st0, P, steps)
    b, kvb = _run(eng, cfg, st0, P, steps)
    for j, ((la, ia), (lb, ib)) in enumerate(zip(a, b)):
        assert ia == ib == steps[j][1]["argmax"], (j, ia, ib)
        assert torch.equal(la, lb), j
    for l in range(cfg.n_layers):
        assert torch.equal(kva[l], kvb[l]), l
    ref.close()
    eng.close()


def test_static_scratch_rejects_an_engine_too_large():
    """An engine whose scratch exceeds the static array is refused with
    PDM_ERR_SIZE (the 8k-context DeepSeek-shaped stack needs more)."""
    import ctypes as C
    from persistent_decode_megakernel_amd import _lib as L
    lib = L.load()
    cfg = configs.get("dsv3_stack_8k")
    d = L.dims_of(cfg)
    h = C.c_void_p()
    # a context long enough that the rotary table alone exceeds the array
    max_ctx = (L.STATIC_SCRATCH_BYTES // (cfg.rope * 4)) + 1024
    assert lib.pdm_create(C.byref(d), max_ctx, 0, C.byref(h)) == 0
    s = L.Sizes()
    assert lib.pdm_get_sizes(h, C.byref(s)) == 0 and s.scratch_bytes > L.STATIC_SCRATCH_BYTES
    dummy = torch.empty(256, dtype=torch.uint8, device="cuda")
    rc = lib.pdm_bind_static(h, C.c_void_p(dummy.data_ptr()), s.weight_bytes, C.c_void_p(dummy.data_ptr()),
                             s.kv_bytes)
    assert rc == L.ERR_SIZE
    assert lib.pdm_destroy(h) == 0
