"""Python face of libkie.so: the same calls as include/kie.h, with torch used
only to hold device memory and to name the stream.  Every step of decode
runs in the library's HIP kernels; nothing here computes."""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence

import numpy as np
import torch

from . import _lib
from ._lib import Config, KieError, LayerWeights, Weights, check

_CFG_FIELDS = ("n_layers", "d_model", "n_heads", "n_kv_heads", "head_dim", "ffn_hidden",
               "vocab_in", "vocab_out", "n_experts", "top_k", "n_shared_experts",
               "expert_hidden", "rms_eps", "rope_base")


def make_config(model, max_seq: Optional[int] = None, graph: bool = False,
                n_workgroups: int = 0, timeout_ms: int = 0, trace: bool = False,
                plain_launch: bool = False) -> Config:
    """kie_config from any object with the model-shape attributes."""
    c = Config()
    for f in _CFG_FIELDS:
        setattr(c, f, getattr(model, f))
    if max_seq is None:
        max_seq = getattr(model, "kv_capacity")
    c.max_seq = int(max_seq)
    c.flags = ((_lib.KIE_MODE_GRAPH if graph else 0) | (_lib.KIE_TRACE if trace else 0)
               | (_lib.KIE_PLAIN_LAUNCH if plain_launch else 0)
               | (_lib.KIE_MOE_RENORM if getattr(model, "moe_renorm", False) else 0))
    c.n_workgroups = int(n_workgroups)
    c.timeout_ms = int(timeout_ms)
    return c


def config_check(model, **kw) -> None:
    lib = _lib.load()
    c = make_config(model, **kw)
    check(lib.kie_config_check(ctypes.byref(c)), "kie_config_check")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda or t.dtype != torch.float16 or not t.is_contiguous():
        raise ValueError("weights must be contiguous fp16 CUDA tensors")
    return t.data_ptr()


class Engine:
    """One decoder handle (kie_create .. kie_destroy)."""

    def __init__(self, model, weights: dict, max_seq: Optional[int] = None, graph: bool = False,
                 n_workgroups: int = 0, timeout_ms: int = 0, stream: Optional[torch.cuda.Stream] = None,
                 trace: bool = False, plain_launch: bool = False):
        self.lib = _lib.load()
        self.model = model
        self.cfg = make_config(model, max_seq, graph, n_workgroups, timeout_ms, trace, plain_launch)
        self._weights = weights                       # keep the device memory alive
        L = model.n_layers
        self._layers = (LayerWeights * L)()
        for l, lw in enumerate(weights["layers"]):
            for name in LayerWeights._fields_:
                key = name[0]
                if key in lw:
                    setattr(self._layers[l], key, _ptr(lw[key]))
        self._w = Weights(_ptr(weights["tok_emb"]), _ptr(weights["final_norm"]),
                          _ptr(weights["lm_head"]), self._layers)
        self.stream = stream if stream is not None else torch.cuda.current_stream()
        h = ctypes.c_void_p()
        check(self.lib.kie_create(ctypes.byref(self.cfg), ctypes.byref(self._w),
                                  ctypes.c_void_p(self.stream.cuda_stream), ctypes.byref(h)),
              "kie_create")
        self.h = h

    # ---- calls -------------------------------------------------------------
    def prefill(self, tokens: Sequence[int]) -> None:
        t = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
        check(self.lib.kie_prefill(self.h, t.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                   int(t.size)), "kie_prefill")

    def prefill_batched(self, tokens: Sequence[int]) -> None:
        """kie_prefill_batched: the prompt's positions through each layer together."""
        t = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
        check(self.lib.kie_prefill_batched(self.h, t.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                           int(t.size)), "kie_prefill_batched")

    def prefill_batched_noalloc(self, tokens: Sequence[int]) -> None:
        """kie_prefill_batched_noalloc: as prefill_batched, with the workspace in
        the library's static device array (no device allocation)."""
        t = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
        check(self.lib.kie_prefill_batched_noalloc(self.h, t.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                                   int(t.size)), "kie_prefill_batched_noalloc")

    def decode_into(self, n: int, out_tokens: Optional[torch.Tensor],
                    out_logits: Optional[torch.Tensor] = None) -> None:
        tp = out_tokens.data_ptr() if out_tokens is not None else None
        lp = out_logits.data_ptr() if out_logits is not None else None
        check(self.lib.kie_decode(self.h, int(n), tp, lp), "kie_decode")

    def decode_sampled_into(self, n: int, seed: int, temperature: float, out_tokens: Optional[torch.Tensor],
                            out_logits: Optional[torch.Tensor] = None) -> None:
        """kie_decode_sampled: tokens drawn from softmax(z / temperature)."""
        tp = out_tokens.data_ptr() if out_tokens is not None else None
        lp = out_logits.data_ptr() if out_logits is not None else None
        check(self.lib.kie_decode_sampled(self.h, int(n), ctypes.c_uint64(int(seed) & (2**64 - 1)),
                                          ctypes.c_float(float(temperature)), tp, lp), "kie_decode_sampled")

    def decode_topkp_into(self, n: int, seed: int, temperature: float, top_k: int, top_p: float,
                          out_tokens: Optional[torch.Tensor], out_logits: Optional[torch.Tensor] = None) -> None:
        """kie_decode_sampled_topkp: the temperature draw restricted by top-k / top-p."""
        tp = out_tokens.data_ptr() if out_tokens is not None else None
        lp = out_logits.data_ptr() if out_logits is not None else None
        check(self.lib.kie_decode_sampled_topkp(self.h, int(n), ctypes.c_uint64(int(seed) & (2**64 - 1)),
                                                ctypes.c_float(float(temperature)), int(top_k),
                                                ctypes.c_float(float(top_p)), tp, lp), "kie_decode_sampled_topkp")

    def decode(self, n: int, logits: bool = True, seed: Optional[int] = None, temperature: float = 0.0,
               top_k: Optional[int] = None, top_p: Optional[float] = None):
        """n decode steps; greedy unless a seed and a temperature > 0 are given
        (then restricted by top_k / top_p when either is given)."""
        dev = self._weights["tok_emb"].device
        toks = torch.empty(max(n, 1), dtype=torch.int32, device=dev)
        lg = torch.empty((max(n, 1), self.model.vocab_out), dtype=torch.float32, device=dev) if logits else None
        if seed is None:
            self.decode_into(n, toks, lg)
        elif top_k is not None or top_p is not None:
            self.decode_topkp_into(n, seed, temperature, top_k or 0, 1.0 if top_p is None else top_p, toks, lg)
        else:
            self.decode_sampled_into(n, seed, temperature, toks, lg)
        return toks[:n], (lg[:n] if lg is not None else None)

    def reset(self) -> None:
        check(self.lib.kie_reset(self.h), "kie_reset")

    @property
    def position(self) -> int:
        p = ctypes.c_int32()
        check(self.lib.kie_get_position(self.h, ctypes.byref(p)), "kie_get_position")
        return p.value

    def last_elapsed_ms(self) -> float:
        ms = ctypes.c_float()
        check(self.lib.kie_last_elapsed_ms(self.h, ctypes.byref(ms)), "kie_last_elapsed_ms")
        return ms.value

    STAGES = {"qkv": 0, "attention": 1, "o": 2, "gateup": 3, "down": 4, "router": 5, "moe_gateup": 6,
              "moe_down": 7, "lm_head": 8}
    ACTS = {"x_attn": 0, "x": 1, "qkv": 2, "o": 3, "u": 4, "router": 5, "logits": 6, "token": 7}

    def debug_stage(self, stage: str, layer: int = 0) -> None:
        """kie_debug_stage: one stage of the next decode step."""
        check(self.lib.kie_debug_stage(self.h, self.STAGES[stage], int(layer)), "kie_debug_stage")

    def debug_read_act(self, what: str, layer: int = 0):
        """kie_debug_read_act: what that stage wrote (float32 array, or the token as int)."""
        m = self.model
        sizes = {"x_attn": m.d_model, "x": m.d_model, "qkv": (m.n_heads + 2 * m.n_kv_heads) * m.head_dim,
                 "o": m.n_heads * m.head_dim,
                 "u": ((m.top_k + m.n_shared_experts) * m.expert_hidden) if m.n_experts else m.ffn_hidden,
                 "router": max(1, m.n_experts), "logits": m.vocab_out, "token": 1}
        if what == "token":
            out = np.zeros(1, np.int32)
        else:
            out = np.zeros(sizes[what], np.float32)
        check(self.lib.kie_debug_read_act(self.h, self.ACTS[what], int(layer), out.ctypes.data, int(out.size)),
              "kie_debug_read_act")
        return int(out[0]) if what == "token" else out

    def read_kv(self, layer: int, pos0: int, pos1: int):
        m = self.model
        shape = (m.n_kv_heads, pos1 - pos0, m.head_dim)
        k = np.empty(shape, np.float16)
        v = np.empty(shape, np.float16)
        check(self.lib.kie_debug_read_kv(self.h, layer, pos0, pos1, k.ctypes.data, v.ctypes.data),
              "kie_debug_read_kv")
        return k, v

    def expert_ids(self, pos0: int, pos1: int) -> np.ndarray:
        """MoE routing at positions [pos0, pos1): int32 [pos1-pos0][n_layers][top_k]."""
        m = self.model
        ids = np.empty((max(0, pos1 - pos0), m.n_layers, m.top_k), np.int32)
        check(self.lib.kie_debug_expert_ids(self.h, pos0, pos1,
                                            ids.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))),
              "kie_debug_expert_ids")
        return ids

    def read_trace(self) -> np.ndarray:
        """Clock stamps (100 MHz) of the traced step: uint64 [n_workgroups, n_events];
        event 0 is the step start, then three per stage in execution order
        (inputs complete, main loop start, end)."""
        n_wg = 4096
        buf = np.zeros((n_wg, 1024), np.uint64)
        ne = ctypes.c_int32()
        nw = ctypes.c_int32()
        check(self.lib.kie_debug_read_trace(self.h, buf.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)),
                                            1024, ctypes.byref(ne), ctypes.byref(nw)),
              "kie_debug_read_trace")
        return buf[:nw.value, :ne.value].copy()

    def close(self) -> None:
        if getattr(self, "h", None) is not None and self.h.value:
            self.lib.kie_destroy(self.h)
            self.h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


def debug_gemv(w: torch.Tensor, x: torch.Tensor, n_workgroups: int = 0) -> torch.Tensor:
    """y = w x through the decode kernel's GEMV stage code (w fp16 [rows][cols], x fp32)."""
    lib = _lib.load()
    rows, cols = w.shape
    y = torch.empty(rows, dtype=torch.float32, device=w.device)
    s = torch.cuda.current_stream()
    check(lib.kie_debug_gemv(w.data_ptr(), x.data_ptr(), y.data_ptr(), rows, cols, n_workgroups,
                             ctypes.c_void_p(s.cuda_stream)), "kie_debug_gemv")
    return y


def debug_gemm(w: torch.Tensor, a: torch.Tensor, c: Optional[torch.Tensor] = None) -> torch.Tensor:
    """c = a w^T (c += a w^T when c is given) through the batched prefill's
    matrix-core product (w fp16 [n][k], a fp32 [m][k])."""
    lib = _lib.load()
    n, k = w.shape
    m = a.shape[0]
    acc = c is not None
    if c is None:
        c = torch.empty(m, n, dtype=torch.float32, device=w.device)
    s = torch.cuda.current_stream()
    check(lib.kie_debug_gemm(w.data_ptr(), a.data_ptr(), c.data_ptr(), m, n, k, int(acc),
                             ctypes.c_void_p(s.cuda_stream)), "kie_debug_gemm")
    return c


def debug_barrier(n_workgroups: int = 0, rounds: int = 1000, spin_limit: int = 0):
    """Grid-barrier stress: returns (violations, ms per barrier)."""
    lib = _lib.load()
    v = ctypes.c_int32()
    ms = ctypes.c_float()
    s = torch.cuda.current_stream()
    check(lib.kie_debug_barrier(n_workgroups, rounds, spin_limit, ctypes.byref(v), ctypes.byref(ms),
                                ctypes.c_void_p(s.cuda_stream)), "kie_debug_barrier")
    return v.value, ms.value


def debug_stream(src: torch.Tensor, dst: Optional[torch.Tensor] = None, n_workgroups: int = 0,
                 reps: int = 10, depth: int = 8, kind: int = 0) -> float:
    """HBM streaming probe: ms per launch to read ``src`` (and copy it to
    ``dst``) with ``depth`` 128-bit loads in flight per lane; ``kind`` 0 is a
    non-temporal global load, 1 a plain global load, 2 the decode kernel's
    non-temporal buffer load."""
    lib = _lib.load()
    ms = ctypes.c_float()
    s = torch.cuda.current_stream()
    nbytes = src.numel() * src.element_size()
    if dst is not None and dst.numel() * dst.element_size() != nbytes:
        raise ValueError("dst must have the size of src")
    check(lib.kie_debug_stream_ex(src.data_ptr(), dst.data_ptr() if dst is not None else None,
                                  nbytes, n_workgroups, depth, kind, reps, ctypes.byref(ms),
                                  ctypes.c_void_p(s.cuda_stream)), "kie_debug_stream_ex")
    return ms.value


__all__ = ["Engine", "KieError", "make_config", "config_check", "debug_gemv", "debug_barrier",
           "debug_stream"]
