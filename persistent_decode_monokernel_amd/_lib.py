"""ctypes view of libkie.so (include/kie.h).  Argument marshalling only."""
from __future__ import annotations

import ctypes
import os
import re

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkie.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "kie.h")

KIE_OK = 0
STATUS = {
    0: "KIE_OK", -1: "KIE_ERR_INVALID_ARG", -2: "KIE_ERR_BAD_STATE",
    -3: "KIE_ERR_CONTEXT_OVERFLOW", -4: "KIE_ERR_TOKEN_RANGE", -5: "KIE_ERR_OCCUPANCY",
    -6: "KIE_ERR_HIP", -7: "KIE_ERR_TIMEOUT", -8: "KIE_ERR_UNSUPPORTED",
}
KIE_MODE_GRAPH = 0x1
KIE_TRACE = 0x2
KIE_PLAIN_LAUNCH = 0x4
KIE_MOE_RENORM = 0x10


class KieError(RuntimeError):
    def __init__(self, code: int, func: str, msg: str):
        super().__init__(f"{func}: {STATUS.get(code, code)}: {msg}")
        self.code = code
        self.status = STATUS.get(code, str(code))


class Config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("n_layers", "d_model", "n_heads", "n_kv_heads", "head_dim", "ffn_hidden",
                 "vocab_in", "vocab_out", "max_seq", "n_experts", "top_k",
                 "n_shared_experts", "expert_hidden")] + [
        ("rms_eps", ctypes.c_float), ("rope_base", ctypes.c_float),
        ("flags", ctypes.c_uint32), ("n_workgroups", ctypes.c_int32),
        ("timeout_ms", ctypes.c_int32)]


class LayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up", "w_down",
                 "router", "e_gate", "e_up", "e_down")]


class Weights(ctypes.Structure):
    _fields_ = [("tok_emb", ctypes.c_void_p), ("final_norm", ctypes.c_void_p),
                ("lm_head", ctypes.c_void_p), ("layers", ctypes.POINTER(LayerWeights))]


_lib = None


def declared_functions(header: str = HEADER_PATH) -> list:
    """Names of the functions include/kie.h declares."""
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kie_\w+)\s*\(", text)))


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Loads libkie.so; fails loudly when it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(path)
    P, I32, VP = ctypes.POINTER, ctypes.c_int32, ctypes.c_void_p
    sig = {
        "kie_config_check": (ctypes.c_int, [P(Config)]),
        "kie_create": (ctypes.c_int, [P(Config), P(Weights), VP, P(VP)]),
        "kie_prefill": (ctypes.c_int, [VP, P(I32), I32]),
        "kie_prefill_batched": (ctypes.c_int, [VP, P(I32), I32]),
        "kie_prefill_batched_noalloc": (ctypes.c_int, [VP, P(I32), I32]),
        "kie_decode": (ctypes.c_int, [VP, I32, VP, VP]),
        "kie_decode_sampled": (ctypes.c_int, [VP, I32, ctypes.c_uint64, ctypes.c_float, VP, VP]),
        "kie_debug_stage": (ctypes.c_int, [VP, I32, I32]),
        "kie_debug_read_act": (ctypes.c_int, [VP, I32, I32, VP, I32]),
        "kie_decode_sampled_topkp": (ctypes.c_int, [VP, I32, ctypes.c_uint64, ctypes.c_float, I32,
                                                    ctypes.c_float, VP, VP]),
        "kie_reset": (ctypes.c_int, [VP]),
        "kie_get_position": (ctypes.c_int, [VP, P(I32)]),
        "kie_destroy": (None, [VP]),
        "kie_last_error": (ctypes.c_char_p, []),
        "kie_last_elapsed_ms": (ctypes.c_int, [VP, P(ctypes.c_float)]),
        "kie_debug_read_kv": (ctypes.c_int, [VP, I32, I32, I32, VP, VP]),
        "kie_debug_expert_ids": (ctypes.c_int, [VP, I32, I32, P(I32)]),
        "kie_debug_gemv": (ctypes.c_int, [VP, VP, VP, I32, I32, I32, VP]),
        "kie_debug_gemm": (ctypes.c_int, [VP, VP, VP, I32, I32, I32, I32, VP]),
        "kie_debug_barrier": (ctypes.c_int, [I32, I32, I32, P(I32), P(ctypes.c_float), VP]),
        "kie_debug_read_trace": (ctypes.c_int, [VP, P(ctypes.c_uint64), I32, P(I32), P(I32)]),
        "kie_debug_stream": (ctypes.c_int, [VP, VP, ctypes.c_size_t, I32, I32, P(ctypes.c_float), VP]),
        "kie_debug_stream_ex": (ctypes.c_int, [VP, VP, ctypes.c_size_t, I32, I32, I32, I32,
                                               P(ctypes.c_float), VP]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def check(rc: int, func: str):
    if rc != KIE_OK:
        msg = _lib.kie_last_error().decode(errors="replace") if _lib else ""
        raise KieError(rc, func, msg)
