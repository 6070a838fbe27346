"""Thin Python binding of the persistent decode engine.

PyTorch only provides device memory and the stream; every step of the decode
path runs in the HIP library (include/pdm.h). Methods marshal tensors into
pointers and check return codes; they compute nothing of the step.
"""
from __future__ import annotations

import ctypes as C
from typing import Optional

import torch

from . import _lib as L


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else C.c_void_p(t.data_ptr())


class Engine:
    """One decode engine bound to torch-allocated device buffers."""

    def __init__(self, cfg, max_ctx: int, device: int = 0, trace: bool = False, static_scratch: bool = False):
        """static_scratch: bind with pdm_bind_static (the library's own scratch
        array; no trace buffer, no taps views)."""
        self.lib = L.load()
        if not torch.cuda.is_available():
            raise RuntimeError("the decode engine needs a HIP GPU")
        self.cfg = cfg
        self.max_ctx = int(max_ctx)
        self.device = torch.device("cuda", device)
        self.dims = L.dims_of(cfg)
        h = C.c_void_p()
        L.check("pdm_create", self.lib.pdm_create(C.byref(self.dims), self.max_ctx, device, C.byref(h)))
        self.h = h
        s = L.Sizes()
        L.check("pdm_get_sizes", self.lib.pdm_get_sizes(h, C.byref(s)))
        self.sizes = s
        u8 = torch.uint8
        self.static_scratch = bool(static_scratch)
        # zeroed, so that the gaps between packed tensors are reproducible bytes
        self.weights = torch.zeros(s.weight_bytes, dtype=u8, device=self.device)
        self.kv = torch.zeros(s.kv_bytes, dtype=u8, device=self.device)
        if self.static_scratch:
            if trace:
                raise ValueError("an engine on the static scratch array has no trace buffer")
            self.scratch = self.trace = None
            torch.cuda.synchronize(self.device)
            L.check("pdm_bind_static", self.lib.pdm_bind_static(
                h, _ptr(self.weights), s.weight_bytes, _ptr(self.kv), s.kv_bytes))
        else:
            self.scratch = torch.zeros(s.scratch_bytes, dtype=u8, device=self.device)
            self.trace = torch.zeros(s.trace_bytes, dtype=u8, device=self.device) if trace else None
            torch.cuda.synchronize(self.device)
            L.check("pdm_bind", self.lib.pdm_bind(
                h, _ptr(self.weights), s.weight_bytes, _ptr(self.kv), s.kv_bytes, _ptr(self.scratch),
                s.scratch_bytes, _ptr(self.trace), s.trace_bytes if trace else 0))
        self.logits = torch.empty(max(cfg.vocab, 1), dtype=torch.float32, device=self.device)
        self.argmax = torch.zeros(1, dtype=torch.int32, device=self.device)

    # ------------------------------------------------------------------ setup
    @property
    def stream(self):
        return C.c_void_p(torch.cuda.current_stream(self.device).cuda_stream)

    def load_tensor(self, spec, t: dict):
        tid = L.TENSOR_IDS[spec.name]
        if "codes" in t:
            codes = t["codes"].to(self.device).contiguous()
            scales = t["scales"].to(self.device).contiguous()
            L.check("pdm_load_fp8", self.lib.pdm_load_fp8(self.h, tid, spec.layer, spec.expert, _ptr(codes),
                                                          _ptr(scales), self.stream))
            return codes, scales
        if "mx_codes" in t:
            codes = t["mx_codes"].to(self.device).contiguous()
            scales = t["mx_scales"].to(self.device).contiguous()
            L.check("pdm_load_mxfp4", self.lib.pdm_load_mxfp4(self.h, tid, spec.layer, spec.expert, _ptr(codes),
                                                              _ptr(scales), self.stream))
            return codes, scales
        data = t["data"].to(self.device).contiguous()
        nbytes = data.numel() * data.element_size()
        L.check("pdm_load_raw", self.lib.pdm_load_raw(self.h, tid, spec.layer, spec.expert, _ptr(data), nbytes,
                                                      self.stream))
        return (data,)

    def load_weights(self, store, sync_every: int = 64):
        """Pack every tensor of a logical weight store (synth.gen.LogicalWeights)."""
        keep = []
        for i, spec in enumerate(store.specs()):
            keep.append(self.load_tensor(spec, store.get(spec.name, spec.layer, spec.expert)))
            if (i + 1) % sync_every == 0:
                torch.cuda.current_stream(self.device).synchronize()
                keep.clear()
        torch.cuda.current_stream(self.device).synchronize()

    def load_packed(self, blob: torch.Tensor):
        on_dev = 1 if blob.is_cuda else 0
        L.check("pdm_load_packed_weights", self.lib.pdm_load_packed_weights(
            self.h, _ptr(blob), blob.numel() * blob.element_size(), on_dev, self.stream))

    def reset(self):
        L.check("pdm_reset_cache", self.lib.pdm_reset_cache(self.h, self.stream))

    def import_kv(self, layer: int, pos0: int, rows: torch.Tensor):
        """rows: bf16 bit patterns (int16) [n, kv_lora + rope] on the device."""
        rows = rows.to(self.device).contiguous()
        assert rows.dtype == torch.int16 and rows.shape[1] == self.cfg.kv_row
        L.check("pdm_import_kv", self.lib.pdm_import_kv(self.h, layer, pos0, rows.shape[0], _ptr(rows), self.stream))
        return rows

    def export_kv(self, layer: int, pos0: int, n: int) -> torch.Tensor:
        out = torch.empty(n, self.cfg.kv_row, dtype=torch.int16, device=self.device)
        L.check("pdm_export_kv", self.lib.pdm_export_kv(self.h, layer, pos0, n, _ptr(out), self.stream))
        return out

    def cache_length(self) -> int:
        v = C.c_int32()
        L.check("pdm_cache_length", self.lib.pdm_cache_length(self.h, C.byref(v)))
        return v.value

    # ------------------------------------------------------------------ step
    def decode(self, pos: int, token: Optional[int] = None, x_in: Optional[torch.Tensor] = None,
               logits: Optional[torch.Tensor] = None, argmax: Optional[torch.Tensor] = None):
        """Enqueue one decode step (asynchronous); returns (argmax, logits) device tensors."""
        lg = self.logits if logits is None else logits
        am = self.argmax if argmax is None else argmax
        if self.cfg.vocab == 0:
            lg = am = None
        rc = self.lib.pdm_decode_step(self.h, -1 if token is None else int(token), int(pos), _ptr(x_in),
                                      _ptr(lg), _ptr(am), self.stream)
        L.check("pdm_decode_step", rc)
        return am, lg

    def decode_steps(self, pos0: int, tokens: torch.Tensor, n_steps: Optional[int] = None, greedy: bool = False,
                     logits: Optional[torch.Tensor] = None, argmax: Optional[torch.Tensor] = None):
        """Enqueue n_steps decode steps as one resident launch (asynchronous).
        tokens: int32 device tensor (n_steps teacher-forced tokens, or the first
        token when greedy). Returns the per-step argmax tensor and the last
        step's logits (or None)."""
        assert tokens.dtype == torch.int32 and tokens.is_cuda
        n = int(n_steps if n_steps is not None else tokens.numel())
        if not greedy:
            assert tokens.numel() >= n
        am = argmax if argmax is not None else torch.zeros(n, dtype=torch.int32, device=self.device)
        L.check("pdm_decode_steps", self.lib.pdm_decode_steps(self.h, int(pos0), n, _ptr(tokens), 1 if greedy else 0,
                                                              _ptr(logits), _ptr(am), self.stream))
        return am, logits

    def decode_steps_raw(self, pos0, tokens, n_steps, greedy=False, logits=None, argmax=None) -> int:
        """Like decode_steps but returns the ABI code instead of raising."""
        return self.lib.pdm_decode_steps(self.h, int(pos0), int(n_steps), _ptr(tokens), 1 if greedy else 0,
                                         _ptr(logits), _ptr(argmax), self.stream)

    def decode_raw(self, pos, token=None, x_in=None, logits=None, argmax=None) -> int:
        """Like decode but returns the ABI code instead of raising."""
        return self.lib.pdm_decode_step(self.h, -1 if token is None else int(token), int(pos), _ptr(x_in),
                                        _ptr(logits), _ptr(argmax), self.stream)

    # ------------------------------------------------------------------ batched products
    def batch_gemm_raw(self, tensor: int, layer: int, expert: int, part: int, x: Optional[torch.Tensor],
                       B: int, y: Optional[torch.Tensor]) -> int:
        """pdm_batch_gemm on the bound weights; returns the ABI code."""
        return self.lib.pdm_batch_gemm(self.h, int(tensor), int(layer), int(expert), int(part), _ptr(x), int(B),
                                       _ptr(y), self.stream)

    def batch_gemm(self, tensor: int, layer: int, x: torch.Tensor, expert: int = -1, part: int = 0,
                   out: Optional[torch.Tensor] = None) -> torch.Tensor:
        """y[b] = W x[b] for the packed FP8 matrix holding (tensor, layer,
        expert) (rows in packed order); x: f32 [B, K] on the device."""
        assert x.dtype == torch.float32 and x.is_cuda and x.is_contiguous() and x.dim() == 2
        lay = L.PackedMatrix()
        L.check("pdm_packed_layout", self.lib.pdm_packed_layout(C.byref(self.dims), int(tensor), int(layer),
                                                                int(expert), int(part), C.byref(lay)))
        y = out if out is not None else torch.empty(x.shape[0], lay.rows, dtype=torch.float32, device=x.device)
        L.check("pdm_batch_gemm", self.batch_gemm_raw(tensor, layer, expert, part, x, x.shape[0], y))
        return y

    def batch_ffn_raw(self, layer: int, h: Optional[torch.Tensor], B: int, idx: Optional[torch.Tensor],
                      w: Optional[torch.Tensor], y: Optional[torch.Tensor]) -> int:
        """pdm_batch_ffn; returns the ABI code."""
        return self.lib.pdm_batch_ffn(self.h, int(layer), _ptr(h), int(B), _ptr(idx), _ptr(w), _ptr(y), self.stream)

    def batch_ffn(self, layer: int, h: torch.Tensor, idx: Optional[torch.Tensor] = None,
                  w: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
        """The SwiGLU / MoE block of `layer` for B tokens (no residual): h f32
        [B, hidden] normalised inputs, idx int32 [B, top_k] and w f32 [B,
        top_k] the routing of a MoE layer."""
        assert h.dtype == torch.float32 and h.is_cuda and h.is_contiguous() and h.dim() == 2
        if idx is not None:
            assert idx.dtype == torch.int32 and idx.is_contiguous() and w.dtype == torch.float32 and w.is_contiguous()
        y = out if out is not None else torch.empty_like(h)
        L.check("pdm_batch_ffn", self.batch_ffn_raw(layer, h, h.shape[0], idx, w, y))
        return y

    def batch_caches(self, B: int) -> torch.Tensor:
        """Zeroed latent caches for B sequences: bf16 bits [B, n_layers, max_ctx, kv_lora + rope]."""
        return torch.zeros(B, self.cfg.n_layers, self.max_ctx, self.cfg.kv_lora + self.cfg.rope, dtype=torch.int16,
                           device=self.device)

    def batch_decode_step_raw(self, tokens, positions, caches, x_in=None, logits=None, argmax=None,
                              hidden=None) -> int:
        """pdm_batch_decode_step; returns the ABI code."""
        B = len(positions)
        pos = (C.c_int32 * B)(*[int(p) for p in positions])
        tok = None if tokens is None else (C.c_int32 * B)(*[int(t) for t in tokens])
        return self.lib.pdm_batch_decode_step(self.h, B, tok, pos, _ptr(x_in), _ptr(caches), _ptr(logits),
                                              _ptr(argmax), _ptr(hidden), self.stream)

    def batch_decode_step(self, positions, caches: torch.Tensor, tokens=None, x_in: Optional[torch.Tensor] = None,
                          hidden: Optional[torch.Tensor] = None):
        """One decode step of B = len(positions) sequences (asynchronous).
        Returns (argmax int32 [B], logits f32 [B, vocab]) device tensors, or
        (None, None) for a bare layer stack."""
        B = len(positions)
        lg = am = None
        if self.cfg.vocab > 0:
            lg = torch.empty(B, self.cfg.vocab, dtype=torch.float32, device=self.device)
            am = torch.empty(B, dtype=torch.int32, device=self.device)
        L.check("pdm_batch_decode_step", self.batch_decode_step_raw(tokens, positions, caches, x_in, lg, am, hidden))
        return am, lg

    def status(self):
        st = L.Status()
        rc = self.lib.pdm_sync_status(self.h, self.stream, C.byref(st))
        return rc, st

    def set_debug(self, spin_limit: int = 0, skip_signal_stage: int = -1):
        L.check("pdm_set_debug", self.lib.pdm_set_debug(self.h, spin_limit, skip_signal_stage))

    def set_trace(self, on: bool):
        L.check("pdm_set_trace", self.lib.pdm_set_trace(self.h, 1 if on else 0))

    def taps(self) -> dict:
        """Views of the last step's taps inside the scratch buffer."""
        if self.static_scratch:
            raise RuntimeError("taps of an engine on the static scratch array are not viewable from torch")
        t = L.Taps()
        L.check("pdm_get_taps", self.lib.pdm_get_taps(self.h, C.byref(t)))
        base = self.scratch.data_ptr()
        cfg = self.cfg

        def view(ptr, n, dtype, shape):
            off = ptr - base
            nb = n * torch.empty((), dtype=dtype).element_size()
            return self.scratch[off:off + nb].view(dtype).view(shape)
        k = max(cfg.top_k, 1)
        out = {
            "hidden": view(t.hidden_dev, cfg.n_layers * cfg.hidden, torch.float32, (cfg.n_layers, cfg.hidden)),
            "hidden_attn": view(t.hidden_attn_dev, cfg.n_layers * cfg.hidden, torch.float32,
                                (cfg.n_layers, cfg.hidden)),
            "router_idx": view(t.router_idx_dev, cfg.n_layers * k, torch.int32, (cfg.n_layers, k)),
            "router_w": view(t.router_w_dev, cfg.n_layers * k, torch.float32, (cfg.n_layers, k)),
            "n_stages": t.n_stages, "n_workgroups": t.n_workgroups, "epoch": t.epoch,
        }
        if self.trace is not None:
            out["trace"] = self.trace.view(torch.int64).view(t.n_stages, t.n_workgroups, 8)
        return out

    def close(self):
        if getattr(self, "h", None) is not None:
            self.lib.pdm_destroy(self.h)
            self.h = None
        # the buffers are useless without the handle: let torch reuse the memory
        self.weights = self.kv = self.scratch = self.trace = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def describe_plan(cfg, max_ctx: int, n_workgroups: int = 256):
    """Stage list of one decode step (pure; no GPU needed)."""
    lib = L.load()
    d = L.dims_of(cfg)
    n = C.c_int32()
    L.check("pdm_describe_plan", lib.pdm_describe_plan(C.byref(d), max_ctx, n_workgroups, None, 0, C.byref(n)))
    arr = (L.StageInfo * n.value)()
    L.check("pdm_describe_plan", lib.pdm_describe_plan(C.byref(d), max_ctx, n_workgroups, arr, n.value, C.byref(n)))
    return [{"type": L.ST_NAMES[s.type], "layer": s.layer, "wait": s.wait_stage, "rows": s.rows, "k": s.k,
             "reads": [r for r in s.reads if r >= 0], "writes": [w for w in s.writes if w >= 0],
             "weight_bytes": s.weight_bytes} for s in arr]


def query_sizes(cfg, max_ctx: int, n_workgroups: int = 256) -> L.Sizes:
    lib = L.load()
    d = L.dims_of(cfg)
    s = L.Sizes()
    L.check("pdm_query_sizes", lib.pdm_query_sizes(C.byref(d), max_ctx, n_workgroups, C.byref(s)))
    return s
