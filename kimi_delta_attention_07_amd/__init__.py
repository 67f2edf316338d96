"""Kimi Delta Attention (KDA) on AMD Instinct MI355X (gfx950).

The work runs in libkda.so (hand-written HIP kernels behind the C ABI of
include/kda.h); this package is its thin Python binding:

    prologue(...)       short conv + activation + L2(q, k) + sigmoid gates
    chunk_forward(...)  chunked prefill over packed varlen sequences
    prefill(...)        the same from raw inputs, prologue fused into the chunk path
    prefill_noalloc(...) prefill() on the library's fixed per-GPU scratch (no workspace)
    chunk_backward(...) gradients of chunk_forward
    prologue_backward(...) gradients of prologue, back to the raw inputs and conv taps
    decode_step(...)    one token for a batch of resident fp32 states
    in_projection(...), out_projection(...), mixer_prefill(...)
                        the mixer's linear maps around the operator, and the whole mixer
    mla_decode_step(...) the MLA mixer's decode token: K/V append, attention, output gate

Build the library with ``python -m kimi_delta_attention_07_amd.build``.
"""
from ._lib import (  # noqa: F401
    CHUNK,
    EXPORTS,
    KdaError,
    chunk_backward,
    chunk_backward_workspace_bytes,
    chunk_forward,
    chunk_prepare,
    chunk_scan,
    chunk_workspace,
    chunk_workspace_bytes,
    decode_step,
    load,
    prefill,
    prefill_noalloc,
    in_projection,
    out_projection,
    mixer_prefill,
    mixer_workspace_bytes,
    mla_decode_step,
    mla_decode_workspace_bytes,
    prefill_prepare,
    prefill_scan,
    prologue,
    prologue_backward,
)
