"""Seeded synthetic inputs for batch-1 decode: model shapes, fp16 weights, prompts.

This module is the only code shared by the HIP decode path's callers and by the
CPU oracle.  It draws random numbers and lays them out; it holds none of the
decoder's arithmetic (no normalisation, attention, projection or sampling).

The pages study single-request decode of a ~2B-parameter FP16 model
(page "Breaking the memory wall: 3,000 tokens/s inference on standard GPUs",
agentlenshq.com, intro and section "The bottleneck: memory bandwidth, not
compute").  They publish neither that model's architecture nor its weights,
so every workload here is a synthetic stand-in with the stated shapes:
weights ~ N(0, 0.02) rounded to fp16, RMSNorm gains exactly 1, prompts
uniform over the input vocabulary.
"""
from __future__ import annotations

from dataclasses import dataclass, asdict, replace
from typing import Dict, List, Optional

import torch

__all__ = ["ModelConfig", "PRESETS", "get_config", "make_weights", "make_prompt",
           "weights_to_numpy", "tensor_specs"]


@dataclass(frozen=True)
class ModelConfig:
    """Shape of one decoder workload (batch 1).

    A dense model has ``n_experts == 0``.  A mixture-of-experts model has
    ``n_experts`` routed experts (``top_k`` chosen per token) plus
    ``n_shared_experts`` always-on experts, all of hidden size
    ``expert_hidden``; its ``ffn_hidden`` is unused (0).
    """
    name: str
    n_layers: int
    d_model: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn_hidden: int
    vocab_in: int            # embedding rows
    vocab_out: int           # lm_head rows (a vocabulary slice may be smaller)
    prompt_len: int
    n_decode: int
    n_experts: int = 0
    top_k: int = 0
    n_shared_experts: int = 0
    expert_hidden: int = 0
    rms_eps: float = 1e-5
    rope_base: float = 10000.0
    max_seq: int = 0         # KV capacity; 0 -> prompt_len + n_decode
    moe_renorm: bool = False # MoE: rescale the selected experts' probabilities to sum to 1

    @property
    def kv_capacity(self) -> int:
        return self.max_seq if self.max_seq > 0 else self.prompt_len + self.n_decode

    @property
    def is_moe(self) -> bool:
        return self.n_experts > 0

    @property
    def q_dim(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    def with_(self, **kw) -> "ModelConfig":
        return replace(self, **kw)

    def as_dict(self) -> dict:
        return asdict(self)


# The five workloads: a tiny parity model, the ~2.2B dense model the pages'
# 2B-class figures refer to, one tensor-parallel-8 share of it run standalone,
# a long-context GQA variant and a single-GPU mixture-of-experts model.
PRESETS: Dict[str, ModelConfig] = {
    "tiny": ModelConfig("tiny", n_layers=2, d_model=256, n_heads=4, n_kv_heads=4,
                        head_dim=64, ffn_hidden=1024, vocab_in=4096, vocab_out=4096,
                        prompt_len=128, n_decode=64),
    "2b": ModelConfig("2b", n_layers=25, d_model=2560, n_heads=20, n_kv_heads=20,
                      head_dim=128, ffn_hidden=6912, vocab_in=32768, vocab_out=32768,
                      prompt_len=512, n_decode=512),
    "tp8share": ModelConfig("tp8share", n_layers=25, d_model=2560, n_heads=3,
                            n_kv_heads=3, head_dim=128, ffn_hidden=864,
                            vocab_in=32768, vocab_out=4096,
                            prompt_len=256, n_decode=1024),
    "longctx": ModelConfig("longctx", n_layers=25, d_model=2560, n_heads=32,
                           n_kv_heads=8, head_dim=80, ffn_hidden=6912,
                           vocab_in=32768, vocab_out=32768,
                           prompt_len=8192, n_decode=256),
    "moe": ModelConfig("moe", n_layers=24, d_model=2048, n_heads=16, n_kv_heads=16,
                       head_dim=128, ffn_hidden=0, vocab_in=32768, vocab_out=32768,
                       prompt_len=512, n_decode=512, n_experts=64, top_k=6,
                       n_shared_experts=2, expert_hidden=1408),
}


def get_config(name: str, **overrides) -> ModelConfig:
    cfg = PRESETS[name]
    return cfg.with_(**overrides) if overrides else cfg


def tensor_specs(cfg: ModelConfig) -> List[tuple]:
    """Canonical tensor order: (path, shape, kind) with kind 'normal' or 'ones'.

    Linear weights are row-major ``[out][in]``.  Stacked expert tensors hold
    the routed experts first, then the shared experts.
    """
    d, F = cfg.d_model, cfg.ffn_hidden
    specs = [("tok_emb", (cfg.vocab_in, d), "normal")]
    for l in range(cfg.n_layers):
        p = f"layers.{l}."
        specs += [(p + "attn_norm", (d,), "ones"),
                  (p + "wq", (cfg.q_dim, d), "normal"),
                  (p + "wk", (cfg.kv_dim, d), "normal"),
                  (p + "wv", (cfg.kv_dim, d), "normal"),
                  (p + "wo", (d, cfg.q_dim), "normal"),
                  (p + "ffn_norm", (d,), "ones")]
        if cfg.is_moe:
            ne = cfg.n_experts + cfg.n_shared_experts
            fe = cfg.expert_hidden
            specs += [(p + "router", (cfg.n_experts, d), "normal"),
                      (p + "e_gate", (ne, fe, d), "normal"),
                      (p + "e_up", (ne, fe, d), "normal"),
                      (p + "e_down", (ne, d, fe), "normal")]
        else:
            specs += [(p + "w_gate", (F, d), "normal"),
                      (p + "w_up", (F, d), "normal"),
                      (p + "w_down", (d, F), "normal")]
    specs += [("final_norm", (d,), "ones"),
              ("lm_head", (cfg.vocab_out, d), "normal")]
    return specs


def _tensor_seed(seed: int, index: int) -> int:
    # One independent torch generator stream per (seed, tensor index).
    return (seed * 0x9E3779B1 + index * 0x85EBCA77 + 0x27D4EB2F) % (1 << 62)


def make_weights(cfg: ModelConfig, seed: int = 0, device="cpu", std: float = 0.02) -> dict:
    """fp16 weights ~ N(0, std) (fp32 draw, scaled, rounded to nearest fp16).

    Returns ``{"tok_emb", "final_norm", "lm_head", "layers": [dict, ...]}`` of
    contiguous torch tensors on ``device``.  The draw depends on the device's
    generator (CPU and GPU streams differ); every comparison hands the same
    bytes to both sides, so only reproducibility on one device matters.
    """
    device = torch.device(device)
    out: dict = {"layers": [dict() for _ in range(cfg.n_layers)]}
    for i, (path, shape, kind) in enumerate(tensor_specs(cfg)):
        if kind == "ones":
            t = torch.ones(shape, dtype=torch.float16, device=device)
        else:
            g = torch.Generator(device=device)
            g.manual_seed(_tensor_seed(seed, i))
            t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
            t.mul_(std)
            t = t.to(torch.float16)
        if path.startswith("layers."):
            _, l, name = path.split(".")
            out["layers"][int(l)][name] = t
        else:
            out[path] = t
    return out


def make_prompt(cfg: ModelConfig, seed: int = 0, length: Optional[int] = None):
    """Prompt token ids, uniform over ``[0, vocab_in)``, as an int32 numpy array.

    Drawn on the CPU so that a prompt is the same on every machine."""
    n = cfg.prompt_len if length is None else length
    g = torch.Generator(device="cpu")
    g.manual_seed(_tensor_seed(seed, 1 << 20))
    return torch.randint(0, cfg.vocab_in, (n,), generator=g, dtype=torch.int64).to(torch.int32).numpy()


def weights_to_numpy(w: dict) -> dict:
    """Host copies of the fp16 weights as numpy arrays (same bytes)."""
    def cv(t):
        return t.detach().to("cpu").contiguous().numpy()
    out = {k: cv(v) for k, v in w.items() if k != "layers"}
    out["layers"] = [{k: cv(v) for k, v in lw.items()} for lw in w["layers"]]
    return out
