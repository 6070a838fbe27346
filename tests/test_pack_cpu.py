"""Offline packer on the host (pdm_pack_* in include/pdm.h), byte for byte.

The packed layout is re-derived here in numpy from its documented rules (the
comment of pdm_packed_matrix in include/pdm.h): which logical row each packed
row holds, and that a scale tile of 8 packed rows x 128 columns carries the
scale of the logical 128x128 block holding its first element. Every packed
matrix of the tiny and ragged models is checked against that, and the logical
codes are recovered from the blob (a round trip). No GPU needed.
"""
import numpy as np
import pytest

from persistent_decode_megakernel_amd import _lib as L
from persistent_decode_megakernel_amd import pack
from synth import configs, gen


def _logical_rows(cfg, name, part, rows):
    """Logical row of each packed row of one part (-1: from another tensor)."""
    r = np.arange(rows)
    dn, dv, dr = cfg.qk_nope, cfg.v_head, cfg.rope
    if name == "wq_a":
        return np.where(r < cfg.q_lora, r, -1)
    if name == "wkv_a":
        return np.where(r >= cfg.q_lora, r - cfg.q_lora, -1)
    if name == "wkv_b":
        if part == 0:
            return r // dn * (dn + dv) + r % dn
        return r // dv * (dn + dv) + dn + r % dv
    if name in ("w_gate", "w_up"):
        i, j = r // 16, r % 16
        mine = (j >= 8) == (name == "w_up")
        return np.where(mine, 8 * i + j % 8, -1)
    return r


def _check_mx_tensor(cfg, arena, spec, t):
    """An MXFP4 expert matrix: the same row map, codes and e8m0 scales per row."""
    codes, scales = t["mx_codes"], t["mx_scales"]
    m = pack.packed_layout(cfg, spec.name, spec.layer, spec.expert, 0)
    assert m.format == L.FMT_MXFP4 and m.parts == 1
    assert m.K == codes.shape[1] and m.n_kblocks == scales.shape[1] == m.K // 16
    pc = arena[m.codes_offset:m.codes_offset + m.rows * m.K].reshape(m.rows, m.K)
    ps = arena[m.scales_offset:m.scales_offset + m.rows * m.n_kblocks].reshape(m.rows, m.n_kblocks)
    src = _logical_rows(cfg, spec.name, 0, m.rows)
    mine = src >= 0
    np.testing.assert_array_equal(pc[mine], codes[src[mine]], err_msg=f"{spec} codes")
    np.testing.assert_array_equal(ps[mine], scales[src[mine]], err_msg=f"{spec} scales")
    assert sorted(src[mine].tolist()) == list(range(codes.shape[0]))  # every row lands once


def _check_tensor(cfg, arena, spec, t):
    codes, scales = t["codes"], t["scales"]
    first = pack.packed_layout(cfg, spec.name, spec.layer, spec.expert, 0)
    recovered = np.full(codes.shape, -1, dtype=np.int32)
    for part in range(first.parts):
        m = pack.packed_layout(cfg, spec.name, spec.layer, spec.expert, part)
        assert m.K == codes.shape[1] and m.n_kblocks == -(-m.K // 128) and m.rows % 8 == 0
        pc = arena[m.codes_offset:m.codes_offset + m.rows * m.K].reshape(m.rows, m.K)
        ps = arena[m.scales_offset:m.scales_offset + (m.rows // 8) * m.n_kblocks * 2].view(np.uint16)
        ps = ps.reshape(m.rows // 8, m.n_kblocks)
        src = _logical_rows(cfg, spec.name, part, m.rows)
        mine = src >= 0
        assert src[mine].max() < codes.shape[0]
        np.testing.assert_array_equal(pc[mine], codes[src[mine]], err_msg=f"{spec} part {part} codes")
        recovered[src[mine]] = pc[mine]
        g_src = src[0::8]  # logical row of each tile's first packed row
        for g in np.nonzero(g_src >= 0)[0]:
            np.testing.assert_array_equal(ps[g], scales[g_src[g] // 128, :m.n_kblocks],
                                          err_msg=f"{spec} part {part} scale tile row {g}")
    # every logical row landed somewhere, unchanged
    np.testing.assert_array_equal(recovered, codes.astype(np.int32), err_msg=f"{spec} round trip")


@pytest.mark.parametrize("name", ["tiny", "ragged", "tiny_fp4", "ragged_fp4"])
def test_host_packer_layout_byte_exact(name):
    cfg = configs.get(name)
    store = gen.LogicalWeights(cfg, 0, "cpu")
    arena = pack.pack_store(cfg, store)
    n_fp8 = n_mx = 0
    for spec in store.specs():
        t = store.numpy(spec.name, spec.layer, spec.expert)
        if "codes" in t:
            _check_tensor(cfg, arena, spec, t)
            n_fp8 += 1
        elif "mx_codes" in t:
            _check_mx_tensor(cfg, arena, spec, t)
            n_mx += 1
    assert n_fp8 > 0 and (n_mx > 0) == (cfg.expert_format == "mxfp4")


def test_host_packer_header_and_errors():
    cfg = configs.get("tiny")
    arena = pack.new_arena(cfg)
    pack.pack_header(cfg, arena)
    assert int.from_bytes(arena[:4].tobytes(), "little") == 0x57444D50  # "PDMW"
    assert int.from_bytes(arena[4:8].tobytes(), "little") == L.ABI_VERSION
    assert int.from_bytes(arena[16:24].tobytes(), "little") == arena.nbytes
    codes = np.zeros((cfg.hidden, cfg.ffn), np.uint8)
    scales = np.zeros((-(-cfg.hidden // 128), -(-cfg.ffn // 128)), np.uint16)
    moe_layer = cfg.layers.index("moe")
    with pytest.raises(L.PdmError) as e:  # a dense-FFN tensor on a MoE layer
        pack.pack_fp8(cfg, "w_down", moe_layer, -1, codes, scales, arena)
    assert e.value.code == L.ERR_ARG
    with pytest.raises(L.PdmError) as e:  # arena too small
        pack.pack_fp8(cfg, "w_down", cfg.layers.index("dense"), -1, codes, scales, arena[:1024])
    assert e.value.code == L.ERR_SIZE
    with pytest.raises(L.PdmError) as e:  # wrong byte count for a raw tensor
        pack.pack_raw(cfg, "attn_norm", 0, -1, np.ones(cfg.hidden + 1, np.float32), arena)
    assert e.value.code == L.ERR_SIZE
