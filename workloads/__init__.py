"""Seeded synthetic workloads for the ISPA hot path.

This module only *draws* inputs: shapes, seeds, random tensors and their
rounding to the storage type a kernel reads.  It contains none of the
method's arithmetic (no attention, no statistics, no solve), so both the
CPU oracle's tests and the GPU path's tests and bench may use it without
sharing any computation.

Source of the shapes: the pages give no tensor shapes.  The workloads are
the layer shapes of the autoregressive video models the ISPA pages evaluate
(1.3B and 14B parameters; "Towards Memory-Efficient Autoregressive Video
Generation via Instance-Specific Parametric Absorption", gist.science
technical summary, section 4 "Experimental results"): hidden 1536 = 12 heads
x 128 and hidden 5120 = 40 heads x 128, 1560 tokens per latent frame,
chunks of 3 frames, frame 0 as the sink ("current frame and sink tokens",
section 2, stage 1 "Dual-Stream Warmup").  Q, K, V ~ N(0, 1) and
W ~ N(0, 1/d).  The pages evaluate on VBench-Long / MovieGen prompts with
trained models; these synthetic tensors at the models' layer shapes stand in
for those (no dataset items are reproduced).

Seeds: every tensor is drawn from
``np.random.SeedSequence([20260701, cfg, layer, unit, tensor])`` with
tensor ids Q=0, K=1, V=2, W=3.  Values are sampled in float64, rounded to
float32 and then (for bf16 workloads) rounded to nearest-even bfloat16.
The exact values the kernel sees are returned as float64 for the oracle.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Iterator, Optional

import numpy as np

ROOT_SEED = 20260701
T_Q, T_K, T_V, T_W = 0, 1, 2, 3
SINK_UNIT = 1_000_000      # the shared sink K/V of the tiny snapshot workload
PERM_UNIT = 1_000_001      # the per-layer temporal-correlation permutation


# ----------------------------------------------------------------------------
# storage rounding (data preparation only)
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to nearest-even bfloat16; return the 16-bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    out = ((u + bias) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round to the storage type ("f32", "bf16", "f16"); return float64 of the stored values."""
    x32 = np.asarray(x, dtype=np.float32)
    if dtype == "f32":
        return x32.astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f32(f32_to_bf16_bits(x32)).astype(np.float64)
    if dtype == "f16":
        return x32.astype(np.float16).astype(np.float64)
    raise ValueError(dtype)


def normal(shape, cfg: int, layer: int, unit: int, tensor: int, std: float = 1.0) -> np.ndarray:
    """Seeded N(0, std^2) draw in float64 (before any storage rounding)."""
    rng = np.random.default_rng(np.random.SeedSequence([ROOT_SEED, cfg, layer, unit, tensor]))
    x = rng.standard_normal(shape)
    if std != 1.0:
        x *= std
    return x


# ----------------------------------------------------------------------------
# workload shapes
# ----------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class AttnShape:
    """Rows of one layer's KV cache: [0,n_sink) sink | history | current chunk."""
    n_q: int
    n_sink: int
    n_hist: int
    n_cur: int
    n_heads: int
    head_dim: int

    @property
    def d(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def n_loc(self) -> int:
        return self.n_sink + self.n_cur

    @property
    def n_k(self) -> int:
        return self.n_sink + self.n_hist + self.n_cur

    def attn_flops(self) -> float:
        """Algorithmic FLOPs of one dual-stream call: one full attention (QK^T and PV)."""
        return 4.0 * self.n_q * self.n_k * self.head_dim * self.n_heads

    def local_flops(self) -> float:
        return 4.0 * self.n_q * self.n_loc * self.head_dim * self.n_heads


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    cfg: int                 # seed id
    shape: AttnShape
    dtype: str               # storage type of Q, K, V, W, A_full ("f32" | "bf16")
    stat_dtype: str          # storage type of A_loc, dA fed to the Gram ("f32" | "f16")
    lam: float
    lam_relative: bool       # lambda * tr(G)/d when True
    frame: int = 1560
    n_layers: int = 1
    chunk_frames: int = 3


TINY = Workload("tiny_f32_d128", 1, AttnShape(64, 64, 256, 64, 2, 64), "f32", "f32", 1e-2, False,
                frame=64)
LAYER_1P3B = Workload("layer_1p3b_bf16", 2, AttnShape(4680, 1560, 14040, 4680, 12, 128), "bf16", "f16",
                      1e-3, True)
WARMUP_1P3B = Workload("warmup_1p3b_30x4", 3, AttnShape(4680, 1560, 0, 4680, 12, 128), "bf16", "f16",
                       1e-3, True, n_layers=30)
LAYER_14B = Workload("layer_14b_bf16", 4, AttnShape(4680, 1560, 31200, 4680, 40, 128), "bf16", "f16",
                     1e-3, True)
ROLLOUT_1P3B = Workload("rollout_1p3b_30x40", 3, AttnShape(4680, 1560, 0, 4680, 12, 128), "bf16", "f16",
                        1e-3, True, n_layers=30)

WORKLOADS = {w.name: w for w in (TINY, LAYER_1P3B, WARMUP_1P3B, LAYER_14B, ROLLOUT_1P3B)}


# ----------------------------------------------------------------------------
# single-layer workloads (tiny, 1.3B layer, 14B layer)
# ----------------------------------------------------------------------------
def layer_inputs(w: Workload, chunk: int = 0, layer: int = 0, with_w: bool = True) -> Dict[str, np.ndarray]:
    """Q [n_q,d], K/V [n_k,d], W [d,d] as float64 holding exactly the stored values.

    For the tiny workload every chunk is a snapshot: the sink K/V are shared by all
    chunks (unit SINK_UNIT), history/current K/V and Q are drawn per chunk (unit=chunk).
    """
    s = w.shape
    d = s.d
    out: Dict[str, np.ndarray] = {}
    out["q"] = round_to(normal((s.n_q, d), w.cfg, layer, chunk, T_Q), w.dtype)
    if w is TINY or w.name == TINY.name:
        rest = s.n_hist + s.n_cur
        for name, t in (("k", T_K), ("v", T_V)):
            sink = normal((s.n_sink, d), w.cfg, layer, SINK_UNIT, t)
            tail = normal((rest, d), w.cfg, layer, chunk, t)
            out[name] = round_to(np.concatenate([sink, tail]), w.dtype)
    else:
        out["k"] = round_to(normal((s.n_k, d), w.cfg, layer, chunk, T_K), w.dtype)
        out["v"] = round_to(normal((s.n_k, d), w.cfg, layer, chunk, T_V), w.dtype)
    if with_w:
        out["w"] = round_to(normal((d, d), w.cfg, layer, 0, T_W, std=1.0 / math.sqrt(d)), w.dtype)
    return out


# ----------------------------------------------------------------------------
# temporally correlated multi-layer rollout (30 layers x frames)
# ----------------------------------------------------------------------------
def layer_rho(layer: int, n_layers: int = 30, cfg: int = 3) -> float:
    """Per-layer AR(1) frame correlation rho_l = 0.9 * pi(l) / (n_layers - 1), pi a seeded permutation.

    With i.i.d. frames every layer's reconstruction error would be statistically the same;
    distinct temporal correlations make the per-layer ranking meaningful.  Marginals stay N(0,1).
    """
    rng = np.random.default_rng(np.random.SeedSequence([ROOT_SEED, cfg, 0, PERM_UNIT, 0]))
    perm = rng.permutation(n_layers)
    return 0.9 * float(perm[layer]) / float(n_layers - 1)


def frames(w: Workload, layer: int, tensor: int, n_frames: int, rows: Optional[int] = None) -> Iterator[np.ndarray]:
    """AR(1) frame sequence X_f = rho X_{f-1} + sqrt(1-rho^2) Z_f, X_0 = Z_0 (float64, unrounded)."""
    rho = layer_rho(layer, w.n_layers, w.cfg)
    c = math.sqrt(1.0 - rho * rho)
    rows = w.frame if rows is None else rows
    x = None
    for f in range(n_frames):
        z = normal((rows, w.shape.d), w.cfg, layer, f, tensor)
        x = z if x is None else rho * x + c * z
        yield x


def rollout_frames(w: Workload, layer: int, n_frames: int, tensors=("q", "k", "v"),
                   as_f32: bool = False) -> Dict[str, np.ndarray]:
    """Stored (rounded) Q, K, V for frames 0..n_frames-1 of one layer, each [n_frames*frame, d].

    as_f32 returns float32 arrays (exact for bf16 storage) to halve host memory on long rollouts.
    """
    out = {}
    ids = {"q": T_Q, "k": T_K, "v": T_V}
    for name in tensors:
        x = np.concatenate([round_to(f, w.dtype).astype(np.float32) for f in frames(w, layer, ids[name], n_frames)])
        out[name] = x if as_f32 else x.astype(np.float64)
    return out


def rollout_weight(w: Workload, layer: int) -> np.ndarray:
    d = w.shape.d
    return round_to(normal((d, d), w.cfg, layer, 0, T_W, std=1.0 / math.sqrt(d)), w.dtype)


def chunk_shape(w: Workload, chunk: int) -> AttnShape:
    """Chunk c covers frames 3c+1..3c+3; history = frames 1..3c; sink = frame 0."""
    f = w.frame
    return AttnShape(w.chunk_frames * f, f, w.chunk_frames * f * chunk, w.chunk_frames * f,
                     w.shape.n_heads, w.shape.head_dim)


def chunk_rows(w: Workload, chunk: int):
    """(query row slice, cache row count) of chunk c into a rollout_frames() tensor."""
    f = w.frame
    q0 = (w.chunk_frames * chunk + 1) * f
    q1 = q0 + w.chunk_frames * f
    return slice(q0, q1), q1

