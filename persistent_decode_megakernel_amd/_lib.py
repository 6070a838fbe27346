"""ctypes declarations of the C ABI in include/pdm.h (argument marshalling only)."""
from __future__ import annotations

import ctypes as C
import os

MAX_LAYERS = 128
STATIC_SCRATCH_BYTES = 32 << 20
ABI_VERSION = 3
FMT_FP8, FMT_MXFP4 = 0, 1

LIB_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_lib")
LIB_PATH = os.path.join(LIB_DIR, "libpdm.so")

# error codes
OK, ERR_ARG, ERR_CONFIG, ERR_DEVICE, ERR_OOM, ERR_ALIGN, ERR_SIZE, ERR_FORMAT = 0, -1, -2, -3, -4, -5, -6, -7
ERR_POS, ERR_TOKEN, ERR_CTX, ERR_LAUNCH, ERR_WATCHDOG, ERR_UNBOUND = -8, -9, -10, -11, -12, -13

# tensor ids
T_EMBED, T_FINAL_NORM, T_LM_HEAD, T_ATTN_NORM, T_WQ_A, T_Q_NORM, T_WQ_B, T_WKV_A = range(8)
T_KV_NORM, T_WKV_B, T_WO, T_FFN_NORM, T_W_GATE, T_W_UP, T_W_DOWN, T_ROUTER = range(8, 16)
TENSOR_IDS = {
    "embed": T_EMBED, "final_norm": T_FINAL_NORM, "lm_head": T_LM_HEAD, "attn_norm": T_ATTN_NORM,
    "wq_a": T_WQ_A, "q_norm": T_Q_NORM, "wq_b": T_WQ_B, "wkv_a": T_WKV_A, "kv_norm": T_KV_NORM,
    "wkv_b": T_WKV_B, "wo": T_WO, "ffn_norm": T_FFN_NORM, "w_gate": T_W_GATE, "w_up": T_W_UP,
    "w_down": T_W_DOWN, "router": T_ROUTER,
}

# stage types and buffer ids
ST_NAMES = ["qkv", "qb", "attn", "uv", "wo", "router", "gu", "gu_routed", "down", "lm"]
BUF_INPUT, BUF_QKV, BUF_QLAT, BUF_ATTN, BUF_O, BUF_XATTN, BUF_ROUTER = range(7)
BUF_ACT, BUF_XOUT, BUF_LOGITS, BUF_KV = range(7, 11)


class Dims(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("n_heads", C.c_int32), ("q_lora", C.c_int32),
                ("kv_lora", C.c_int32), ("qk_nope", C.c_int32), ("rope", C.c_int32),
                ("v_head", C.c_int32), ("ffn", C.c_int32), ("n_experts", C.c_int32),
                ("moe_ffn", C.c_int32), ("top_k", C.c_int32), ("n_shared", C.c_int32),
                ("vocab", C.c_int32), ("n_layers", C.c_int32),
                ("layer_moe", C.c_uint8 * MAX_LAYERS), ("rms_eps", C.c_float), ("rope_base", C.c_float),
                ("expert_format", C.c_int32)]


class Sizes(C.Structure):
    _fields_ = [("weight_bytes", C.c_uint64), ("kv_bytes", C.c_uint64), ("scratch_bytes", C.c_uint64),
                ("trace_bytes", C.c_uint64), ("alignment", C.c_uint64), ("n_stages", C.c_int32),
                ("n_workgroups", C.c_int32)]


class Status(C.Structure):
    _fields_ = [("code", C.c_int32), ("stage", C.c_int32), ("workgroup", C.c_int32),
                ("observed", C.c_int32), ("epoch", C.c_uint32), ("pad", C.c_int32 * 3)]


class Taps(C.Structure):
    _fields_ = [("hidden_dev", C.c_void_p), ("hidden_attn_dev", C.c_void_p), ("router_idx_dev", C.c_void_p),
                ("router_w_dev", C.c_void_p), ("logits_dev", C.c_void_p), ("trace_dev", C.c_void_p),
                ("n_stages", C.c_int32), ("n_workgroups", C.c_int32), ("epoch", C.c_uint32)]


class StageInfo(C.Structure):
    _fields_ = [("type", C.c_int32), ("layer", C.c_int32), ("wait_stage", C.c_int32), ("rows", C.c_int32),
                ("k", C.c_int32), ("reads", C.c_int32 * 4), ("writes", C.c_int32 * 2),
                ("weight_bytes", C.c_uint64)]


class PackedMatrix(C.Structure):
    _fields_ = [("codes_offset", C.c_uint64), ("scales_offset", C.c_uint64), ("rows", C.c_int32),
                ("K", C.c_int32), ("n_kblocks", C.c_int32), ("parts", C.c_int32), ("format", C.c_int32),
                ("pad", C.c_int32)]


_P = C.c_void_p
_SIGS = {
    "pdm_query_sizes": (C.c_int, [C.POINTER(Dims), C.c_int32, C.c_int32, C.POINTER(Sizes)]),
    "pdm_describe_plan": (C.c_int, [C.POINTER(Dims), C.c_int32, C.c_int32, C.POINTER(StageInfo), C.c_int32,
                                    C.POINTER(C.c_int32)]),
    "pdm_create": (C.c_int, [C.POINTER(Dims), C.c_int32, C.c_int, C.POINTER(_P)]),
    "pdm_get_sizes": (C.c_int, [_P, C.POINTER(Sizes)]),
    "pdm_bind": (C.c_int, [_P, _P, C.c_uint64, _P, C.c_uint64, _P, C.c_uint64, _P, C.c_uint64]),
    "pdm_bind_static": (C.c_int, [_P, _P, C.c_uint64, _P, C.c_uint64]),
    "pdm_load_fp8": (C.c_int, [_P, C.c_int32, C.c_int32, C.c_int32, _P, _P, _P]),
    "pdm_load_mxfp4": (C.c_int, [_P, C.c_int32, C.c_int32, C.c_int32, _P, _P, _P]),
    "pdm_load_raw": (C.c_int, [_P, C.c_int32, C.c_int32, C.c_int32, _P, C.c_uint64, _P]),
    "pdm_load_packed_weights": (C.c_int, [_P, _P, C.c_uint64, C.c_int, _P]),
    "pdm_pack_header": (C.c_int, [C.POINTER(Dims), _P, C.c_uint64]),
    "pdm_pack_fp8": (C.c_int, [C.POINTER(Dims), C.c_int32, C.c_int32, C.c_int32, _P, _P, _P, C.c_uint64]),
    "pdm_pack_mxfp4": (C.c_int, [C.POINTER(Dims), C.c_int32, C.c_int32, C.c_int32, _P, _P, _P, C.c_uint64]),
    "pdm_pack_raw": (C.c_int, [C.POINTER(Dims), C.c_int32, C.c_int32, C.c_int32, _P, C.c_uint64, _P, C.c_uint64]),
    "pdm_packed_layout": (C.c_int, [C.POINTER(Dims), C.c_int32, C.c_int32, C.c_int32, C.c_int32,
                                    C.POINTER(PackedMatrix)]),
    "pdm_reset_cache": (C.c_int, [_P, _P]),
    "pdm_import_kv": (C.c_int, [_P, C.c_int32, C.c_int32, C.c_int32, _P, _P]),
    "pdm_export_kv": (C.c_int, [_P, C.c_int32, C.c_int32, C.c_int32, _P, _P]),
    "pdm_decode_step": (C.c_int, [_P, C.c_int32, C.c_int32, _P, _P, _P, _P]),
    "pdm_decode_steps": (C.c_int, [_P, C.c_int32, C.c_int32, _P, C.c_int, _P, _P, _P]),
    "pdm_sync_status": (C.c_int, [_P, _P, C.POINTER(Status)]),
    "pdm_get_taps": (C.c_int, [_P, C.POINTER(Taps)]),
    "pdm_cache_length": (C.c_int, [_P, C.POINTER(C.c_int32)]),
    "pdm_set_debug": (C.c_int, [_P, C.c_int32, C.c_int32]),
    "pdm_set_trace": (C.c_int, [_P, C.c_int32]),
    "pdm_batch_gemm": (C.c_int, [_P, C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_void_p, C.c_int32,
                                 C.c_void_p, C.c_void_p]),
    "pdm_batch_ffn": (C.c_int, [_P, C.c_int32, C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p,
                                C.c_void_p]),
    "pdm_batch_decode_step": (C.c_int, [_P, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                        C.c_void_p, C.c_void_p, C.c_void_p]),
    "pdm_dsa_index_scores": (C.c_int, [_P, _P, _P, C.c_int32, C.c_int32, C.c_int32, _P, _P]),
    "pdm_dsa_topk_work_bytes": (C.c_uint64, [C.c_int32]),
    "pdm_dsa_topk": (C.c_int, [_P, C.c_int32, C.c_int32, _P, _P, C.c_uint64, _P]),
    "pdm_dsa_attention_work_bytes": (C.c_uint64, [C.c_int32, C.c_int32]),
    "pdm_dsa_attention": (C.c_int, [_P, _P, _P, C.c_int32, _P, C.c_int32, C.c_int32, C.c_int32, C.c_int32,
                                    C.c_float, _P, C.c_uint64, _P, _P]),
    "pdm_destroy": (C.c_int, [_P]),
    "pdm_strerror": (C.c_char_p, [C.c_int]),
}
EXPORTED = tuple(_SIGS)

_lib = None


class PdmError(RuntimeError):
    def __init__(self, fn, code):
        self.code = code
        super().__init__(f"{fn} failed: {code} ({strerror(code)})")


def load(path: str = LIB_PATH):
    """Load the built library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"HIP engine library not built: {path} missing (run __graft_entry__.build())")
    lib = C.CDLL(path)
    for name, (res, args) in _SIGS.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def strerror(code: int) -> str:
    return load().pdm_strerror(code).decode()


def check(fn: str, code: int):
    if code != OK:
        raise PdmError(fn, code)
    return code


def dims_of(cfg) -> Dims:
    """pdm_dims of a synth.configs.ModelConfig."""
    d = Dims()
    d.hidden, d.n_heads, d.q_lora, d.kv_lora = cfg.hidden, cfg.n_heads, cfg.q_lora, cfg.kv_lora
    d.qk_nope, d.rope, d.v_head, d.ffn = cfg.qk_nope, cfg.rope, cfg.v_head, cfg.ffn
    d.n_experts, d.moe_ffn, d.top_k, d.n_shared = cfg.n_experts, cfg.moe_ffn, cfg.top_k, cfg.n_shared
    d.vocab, d.n_layers = cfg.vocab, cfg.n_layers
    for i, kind in enumerate(cfg.layers):
        d.layer_moe[i] = 1 if kind == "moe" else 0
    d.rms_eps, d.rope_base = cfg.rms_eps, cfg.rope_base
    d.expert_format = FMT_MXFP4 if getattr(cfg, "expert_format", "fp8") == "mxfp4" else FMT_FP8
    return d
