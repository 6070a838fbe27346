"""Thin binding of the sparse (DSA) decode attention calls of include/pdm.h:
indexer scores, top-k position selection and MLA attention over the selected
cache rows. Tensors are marshalled into pointers on torch's current stream;
every step runs in the HIP library, which must be built (no fallback)."""
from __future__ import annotations

import ctypes as C

import torch

from . import _lib as L


def _p(t: torch.Tensor):
    return C.c_void_p(t.data_ptr())


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(*ts):
    for t in ts:
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("DSA calls take contiguous device tensors")


def index_scores(q: torch.Tensor, w: torch.Tensor, k: torch.Tensor, out: torch.Tensor = None) -> torch.Tensor:
    """q f32 [HI, dI], w f32 [HI], k bf16 [n, dI] -> f32 [n]."""
    _dev(q, w, k)
    n, dI = k.shape
    out = torch.empty(n, dtype=torch.float32, device=k.device) if out is None else out
    L.check("pdm_dsa_index_scores", L.load().pdm_dsa_index_scores(_p(q), _p(w), _p(k), n, q.shape[0], dI, _p(out),
                                                                  _stream()))
    return out


def topk_work_bytes(n: int) -> int:
    return int(L.load().pdm_dsa_topk_work_bytes(n))


def topk(scores: torch.Tensor, k: int, out: torch.Tensor = None, work: torch.Tensor = None) -> torch.Tensor:
    """The min(k, n) positions of largest score, ascending, int32."""
    _dev(scores)
    n = scores.shape[0]
    out = torch.empty(min(k, n), dtype=torch.int32, device=scores.device) if out is None else out
    if work is None:
        work = torch.empty(topk_work_bytes(n) // 4, dtype=torch.int32, device=scores.device)
    L.check("pdm_dsa_topk", L.load().pdm_dsa_topk(_p(scores), n, int(k), _p(out), _p(work), work.numel() * 4,
                                                  _stream()))
    return out


def work_bytes(H: int, kv_lora: int) -> int:
    return int(L.load().pdm_dsa_attention_work_bytes(H, kv_lora))


def attention(q_lat: torch.Tensor, q_pe: torch.Tensor, cache: torch.Tensor, sel: torch.Tensor, tau: float,
              work: torch.Tensor = None, out: torch.Tensor = None) -> torch.Tensor:
    """q_lat f32 [H, dc], q_pe f32 [H, dr], cache bf16 [rows, dc + dr], sel int32 [n_sel] -> o_lat f32 [H, dc]."""
    _dev(q_lat, q_pe, cache, sel)
    H, dc = q_lat.shape
    dr = q_pe.shape[1]
    if work is None:
        work = torch.empty(work_bytes(H, dc) // 4, dtype=torch.float32, device=q_lat.device)
    out = torch.empty(H, dc, dtype=torch.float32, device=q_lat.device) if out is None else out
    L.check("pdm_dsa_attention", L.load().pdm_dsa_attention(
        _p(q_lat), _p(q_pe), _p(cache), cache.shape[0], _p(sel), sel.shape[0], H, dc, dr, float(tau), _p(work),
        work.numel() * 4, _p(out), _stream()))
    return out
