"""Host side of the offline packer (pdm_pack_header / pdm_pack_fp8 /
pdm_pack_raw / pdm_packed_layout in include/pdm.h): argument marshalling
only. The packing itself runs in the library, no GPU needed; the result is a
host weight blob for Engine.load_packed."""
from __future__ import annotations

import ctypes as C

import numpy as np

from . import _lib as L


def _np_ptr(a: np.ndarray):
    if not a.flags["C_CONTIGUOUS"]:
        raise ValueError("array must be C-contiguous")
    return C.c_void_p(a.ctypes.data)


def weight_bytes(cfg) -> int:
    s = L.Sizes()
    d = L.dims_of(cfg)
    L.check("pdm_query_sizes", L.load().pdm_query_sizes(C.byref(d), 1, 0, C.byref(s)))
    return int(s.weight_bytes)


def new_arena(cfg) -> np.ndarray:
    """A zeroed host image of the weight arena of cfg."""
    return np.zeros(weight_bytes(cfg), dtype=np.uint8)


def pack_header(cfg, arena: np.ndarray):
    d = L.dims_of(cfg)
    L.check("pdm_pack_header", L.load().pdm_pack_header(C.byref(d), _np_ptr(arena), arena.nbytes))


def pack_fp8(cfg, name: str, layer: int, expert: int, codes: np.ndarray, scales: np.ndarray, arena: np.ndarray):
    d = L.dims_of(cfg)
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    L.check("pdm_pack_fp8", L.load().pdm_pack_fp8(C.byref(d), L.TENSOR_IDS[name], layer, expert, _np_ptr(codes),
                                                  _np_ptr(scales), _np_ptr(arena), arena.nbytes))


def pack_mxfp4(cfg, name: str, layer: int, expert: int, codes: np.ndarray, scales: np.ndarray, arena: np.ndarray):
    d = L.dims_of(cfg)
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    L.check("pdm_pack_mxfp4", L.load().pdm_pack_mxfp4(C.byref(d), L.TENSOR_IDS[name], layer, expert,
                                                      _np_ptr(codes), _np_ptr(scales), _np_ptr(arena), arena.nbytes))


def pack_raw(cfg, name: str, layer: int, expert: int, data: np.ndarray, arena: np.ndarray):
    d = L.dims_of(cfg)
    data = np.ascontiguousarray(data)
    L.check("pdm_pack_raw", L.load().pdm_pack_raw(C.byref(d), L.TENSOR_IDS[name], layer, expert, _np_ptr(data),
                                                  data.nbytes, _np_ptr(arena), arena.nbytes))


def packed_layout(cfg, name: str, layer: int, expert: int = -1, part: int = 0) -> L.PackedMatrix:
    d = L.dims_of(cfg)
    out = L.PackedMatrix()
    L.check("pdm_packed_layout", L.load().pdm_packed_layout(C.byref(d), L.TENSOR_IDS[name], layer, expert, part,
                                                            C.byref(out)))
    return out


def pack_store(cfg, store) -> np.ndarray:
    """Pack every tensor of a logical weight store (synth.gen.LogicalWeights,
    numpy view) into a new host blob."""
    arena = new_arena(cfg)
    pack_header(cfg, arena)
    for spec in store.specs():
        t = store.numpy(spec.name, spec.layer, spec.expert)
        if "codes" in t:
            pack_fp8(cfg, spec.name, spec.layer, spec.expert, t["codes"], t["scales"], arena)
        elif "mx_codes" in t:
            pack_mxfp4(cfg, spec.name, spec.layer, spec.expert, t["mx_codes"], t["mx_scales"], arena)
        else:
            pack_raw(cfg, spec.name, spec.layer, spec.expert, t["data"], arena)
    return arena
