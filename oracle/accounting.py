"""Oracle: closed-form work and KV-cache byte counts.

TEST INFRASTRUCTURE ONLY -- never imported by the GPU library.

The ISPA pages (technical summary, section 2 stage 3 "Memory-Efficient
Inference") say the converted L-layers drop their historical K/V and keep only
local context, while the remaining F-layers keep full attention; section 4
reports up to 50% of the KV cache removed with half the layers converted.  The
byte counts below are that statement written out for a cache of bf16 K and V.
"""
from __future__ import annotations


def attn_flops(n_q: int, n_k: int, head_dim: int, n_heads: int) -> int:
    """QK^T plus PV multiply-adds of one attention over n_k keys, as FLOPs (2 per multiply-add)."""
    return 4 * n_q * n_k * head_dim * n_heads


def kv_cache_bytes(chunk: int, n_layers: int, n_local: int, frame: int, chunk_frames: int, d: int,
                   elem_bytes: int = 2) -> int:
    """K+V bytes held while chunk ``chunk`` is generated (current chunk included).

    F-layer rows: sink frame + history frames 1..chunk_frames*chunk + current chunk.
    L-layer rows: sink frame + current chunk.
    """
    f_rows = frame * (1 + chunk_frames * chunk + chunk_frames)
    l_rows = frame * (1 + chunk_frames)
    n_full = n_layers - n_local
    return 2 * d * elem_bytes * (n_full * f_rows + n_local * l_rows)


def kv_removed_fraction(chunk: int, n_layers: int, n_local: int, frame: int, chunk_frames: int,
                        d: int) -> float:
    full = kv_cache_bytes(chunk, n_layers, 0, frame, chunk_frames, d)
    mixed = kv_cache_bytes(chunk, n_layers, n_local, frame, chunk_frames, d)
    return 1.0 - mixed / full
