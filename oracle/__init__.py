"""CPU oracle for batch-1 decode — TEST INFRASTRUCTURE, not part of the product.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline
leg may import or call anything in this package.  It shares no code with the
HIP decode path (``persistent_decode_monokernel_amd``); both read the same
fp16 weight bytes from ``kie_synth``.

What it computes, and where that comes from
-------------------------------------------
The pages describe the persistent monokernel as one GPU-resident program that
runs the whole decode path — matrix multiplies, attention, normalisation and
sampling — without handing control back to the CPU (page "Breaking the memory
wall: 3,000 tokens/s inference on standard GPUs", agentlenshq.com, section
"1. The Monokernel Runtime").  The monokernel is a schedule, not an
approximation: it must produce what a plain layer-by-layer decoder produces.
This package is that plain decoder, written in numpy in the precision the
workload fixes (fp32, weights widened exactly from fp16), with an fp64 switch
used by the pins.

The pages give no layer equations.  The workloads name RMSNorm (eps 1e-5),
RoPE (base 10000), SwiGLU, multi-head / grouped-query attention, untied
embeddings, greedy decoding and softmax top-k routing with shared experts;
every point they leave open is read the plain (Llama-style) way, stated at
the function that makes the choice.

``sampling`` defines temperature sampling (a draw from softmax(z / T) by the
Gumbel-max method, with Philox4x64-10 counter-based random numbers) exactly
as the decode kernel computes it.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against closed forms, invariants, special cases, brute force and library
routines; none is "parity unpinned".
"""
from .decoder import (Oracle, rmsnorm, rope_cos_sin, rope, softmax, attend,
                      silu, swiglu, moe_route, moe_ffn, argmax_first)
from .sampling import philox4x64, uniforms, gumbel, sample_keys, sample_token

__all__ = ["Oracle", "rmsnorm", "rope_cos_sin", "rope", "softmax", "attend",
           "silu", "swiglu", "moe_route", "moe_ffn", "argmax_first",
           "philox4x64", "uniforms", "gumbel", "sample_keys", "sample_token"]
