"""The method's three stages for one generation instance, driven through the C ABI.

Technical summary (gist.science, nl/pt), section 2 "Methodology":

* stage 1 "Dual-Stream Warmup": for the first T_warm chunks every layer attends to its whole KV cache
  with the dual stream, which yields A_full (what the model consumes) and A_loc (sink + current
  chunk only); the absorption statistics G, C, D accumulate chunk by chunk;
* stage 2 "Layer Absorb": at the transition each layer gets dW in closed form and its
  reconstruction error epsilon;
* "Dynamic layer selection": the k layers with the lowest epsilon are converted;
* stage 3 "Memory-Efficient Inference": converted layers drop their cached history and run local
  attention projected by W_new = W + dW; the other layers keep full attention over the growing cache.

Every step runs in libispa's kernels (attention, statistics, solve, ranking, cache copies).  This
class orders the calls, owns the buffers (PyTorch device memory, plus the library's KV cache) and
reads the role map back to the host once, at the transition, to decide which caches to release.
"""
from __future__ import annotations

from typing import List, Optional, Sequence, Tuple

from . import (AttnShape, CALL_ABSORB_SOLVE, CALL_DUAL_ATTN, CALL_DUAL_ATTN_VT, CALL_LOCAL_ATTN_FP8_PROJ_W8A8,
               CALL_LOCAL_ATTN_PROJ, IspaError, KVCache, absorb_solve_batched, dual_attn, dual_attn_vt, gram_accum,
               local_attn_fp8_proj_w8a8, local_attn_fused_proj_wt, quantize_weight_fp8, select_layers, transpose16,
               transpose_rows, workspace_bytes)

WARMUP, STEADY = "warmup", "steady"
L_LAYER_KINDS = ("bf16", "w8a8_fp8")


class IspaRuntime:
    """One instance of an n_layers attention stack under the method.

    forward(layer, q, k, v) appends the chunk's K/V rows to the layer's cache and returns
    (out, projected):
      * during the warmup and for layers that keep full attention: out = A_full [n_q, d], the
        attention output over the whole cache, projected = False (the caller applies its W);
      * for converted layers after the transition: out = LocalAttn(q; sink + current) @ W_new,
        projected = True.
    transition(weights) runs the absorption for every layer, ranks the layers by epsilon, converts
    the k_local lowest and releases their history rows.
    l_layer selects the converted layers' step: "bf16" (16-bit attention, projection by W_new^T
    transposed once at the fold) or "w8a8_fp8" (the method combined with W8A8: W_new coded once to
    FP8 E4M3 per output channel at the fold; FP8 attention, per-token activation codes and the FP8
    product per step).
    During the warmup each layer also keeps V^T in fp16 (the dual stream's PV type) for the rows the
    warmup can hold, so a chunk's V rows are transposed once, when appended, instead of the whole
    cache on every call (when sink_rows and chunk_rows are multiples of 8, which the V^T columns'
    16-byte alignment needs; otherwise each call copies).  These buffers are freed at the
    transition; the layers that keep full attention then grow their cache for the rest of the
    rollout, and each of their calls transposes it (a V^T of the whole rollout would be committed
    up front, while the cache's memory follows the rows it holds).
    """

    def __init__(self, n_layers: int, n_heads: int, head_dim: int, sink_rows: int, chunk_rows: int,
                 warmup_chunks: int, max_chunks: int, k_local: int, dtype=None, stat_dtype=None,
                 lam: float = 1e-3, lam_relative: bool = True, refine: int = 0, keep_delta_w: bool = False,
                 l_layer: str = "bf16", stream=None):
        import torch
        if not 0 <= k_local <= n_layers:
            raise ValueError("k_local must be in [0, n_layers]")
        if l_layer not in L_LAYER_KINDS:
            raise ValueError(f"l_layer must be one of {L_LAYER_KINDS}")
        self.l_layer = l_layer
        if warmup_chunks < 1 or warmup_chunks > max_chunks:
            raise ValueError("need 1 <= warmup_chunks <= max_chunks")
        self.torch = torch
        self.n_layers, self.n_heads, self.head_dim = n_layers, n_heads, head_dim
        self.d = n_heads * head_dim
        self.sink_rows, self.chunk_rows = sink_rows, chunk_rows
        self.warmup_chunks, self.k_local = warmup_chunks, k_local
        self.dtype = dtype or torch.bfloat16
        self.stat_dtype = stat_dtype or torch.float16
        self.lam, self.lam_relative, self.refine = lam, lam_relative, refine
        self.keep_delta_w = keep_delta_w
        # every call goes to one torch stream; buffers made per call are recorded on it so the caching
        # allocator never hands them out while that stream may still use them
        self.stream = stream if stream is not None else torch.cuda.current_stream()
        dev = "cuda"
        self.kv = KVCache(n_layers, self.d, self.dtype, sink_rows, chunk_rows, max_chunks)
        self.chunks = [0] * n_layers
        self.stage = WARMUP
        d = self.d
        self.ld = (chunk_rows + 7) // 8 * 8
        self.a_t = torch.empty((d, self.ld), dtype=self.stat_dtype, device=dev)
        self.da_t = torch.empty((d, self.ld), dtype=self.stat_dtype, device=dev)
        # G, C, D of every layer, fp32 [n_layers, d, d]; started[l] once layer l's first chunk is in
        self.G, self.C, self.D = (torch.empty((n_layers, d, d), device=dev) for _ in range(3))
        self.started = [False] * n_layers
        self.eps = torch.full((n_layers,), float("nan"), device=dev)
        self.lambdas = torch.zeros((n_layers,), device=dev)
        self.info = torch.zeros((n_layers,), dtype=torch.int32, device=dev)
        self.role = torch.zeros((n_layers,), dtype=torch.int32, device=dev)
        self.order = torch.zeros((n_layers,), dtype=torch.int32, device=dev)
        self.roles: Optional[List[int]] = None
        self.w_new = [None] * n_layers
        self.w_new_t = [None] * n_layers   # W_new^T of the converted layers, transposed once at the fold
        self.w_codes = [None] * n_layers   # ("w8a8_fp8") their FP8 codes W_new^T and per-channel scales
        self.delta_w = None
        self.vt_resident = (sink_rows % 8 == 0 and chunk_rows % 8 == 0
                            and self.dtype in (torch.bfloat16, torch.float16))
        self.ldv_warm = (sink_rows + warmup_chunks * chunk_rows + 7) // 8 * 8 + 64
        self.vt: List[Optional[object]] = [None] * n_layers

    # ------------------------------------------------------------------ helpers
    def _vt(self, layer: int):
        """The layer's warmup V^T [d, ldv_warm] (fp16), made on first use."""
        if self.vt[layer] is None:
            self.vt[layer] = self._buf(self.d, self.ldv_warm, dtype=self.torch.float16)
            with self.torch.cuda.stream(self.stream):
                self.vt[layer].zero_()
        return self.vt[layer]

    def _shape(self, layer: int, n_q: int) -> Tuple[AttnShape, object, object]:
        k, v, (n_s, n_h, n_c) = self.kv.layer(layer)
        return AttnShape(n_q, n_s, n_h, n_c, self.n_heads, self.head_dim, 0.0), k, v

    def _buf(self, *shape, dtype=None):
        t = self.torch.empty(shape, dtype=dtype or self.torch.float32, device="cuda")
        if self.stream != self.torch.cuda.current_stream():
            t.record_stream(self.stream)
        return t

    def _ws(self, call: int, shape: Optional[AttnShape], d: int = 0, count: int = 1):
        return self._buf(count * workspace_bytes(call, shape, d), dtype=self.torch.uint8)

    # ------------------------------------------------------------------ stages
    def write_sink(self, layer: int, k, v) -> None:
        self.kv.write_sink(layer, k, v, stream=self.stream)
        if self.vt_resident and self.stage == WARMUP:
            transpose_rows(v, self._vt(layer), 0, stream=self.stream)

    def forward(self, layer: int, q, k, v):
        """Append this chunk's K/V to the layer's cache and run the layer's attention for the stage."""
        torch = self.torch
        if self.stage == WARMUP and self.chunks[layer] >= self.warmup_chunks:
            raise RuntimeError(f"layer {layer}: warmup chunks done; call transition() first")
        self.kv.append_chunk(layer, k, v, stream=self.stream)
        if self.stage == WARMUP and self.vt_resident:
            transpose_rows(v, self._vt(layer), self.sink_rows + self.chunks[layer] * self.chunk_rows,
                           stream=self.stream)
        self.chunks[layer] += 1
        shape, kc, vc = self._shape(layer, q.shape[0])
        out = self._buf(shape.n_q, self.d, dtype=self.dtype)
        if self.stage == WARMUP:
            if shape.n_q > self.chunk_rows:
                raise ValueError("a warmup chunk has at most chunk_rows queries")
            if self.vt_resident:
                dual_attn_vt(shape, q, kc, self._vt(layer), a_full=out, a_loc_t=self.a_t, delta_a_t=self.da_t,
                             ld_stat=self.ld, workspace=self._ws(CALL_DUAL_ATTN_VT, shape), stream=self.stream)
            else:
                dual_attn(shape, q, kc, vc, a_full=out, a_loc_t=self.a_t, delta_a_t=self.da_t, ld_stat=self.ld,
                          workspace=self._ws(CALL_DUAL_ATTN, shape), stream=self.stream)
            gram_accum(self.a_t, self.da_t, shape.n_q, self.G[layer], self.C[layer], self.D[layer],
                       accumulate=self.started[layer], stream=self.stream)
            self.started[layer] = True
            return out, False
        if self.roles[layer] == 1:
            if self.l_layer == "w8a8_fp8":
                wq, sw = self.w_codes[layer]
                local_attn_fp8_proj_w8a8(shape, q, kc, vc, wq, sw, out, self._ws(CALL_LOCAL_ATTN_FP8_PROJ_W8A8, shape),
                                         stream=self.stream)
            else:
                local_attn_fused_proj_wt(shape, q, kc, vc, self.w_new_t[layer], out,
                                         self._ws(CALL_LOCAL_ATTN_PROJ, shape), stream=self.stream)
            return out, True
        dual_attn(shape, q, kc, vc, a_full=out, workspace=self._ws(CALL_DUAL_ATTN, shape), stream=self.stream)
        return out, False

    def transition(self, weights: Sequence) -> List[int]:
        """Absorb every layer (dW, epsilon, W_new), convert the k_local lowest-epsilon layers and release
        their history.  weights[l] is layer l's output projection W [d, d] (y = A W), in the io dtype.
        Returns the role map: 1 = converted (local attention with W_new), 0 = full attention."""
        torch = self.torch
        if self.stage != WARMUP:
            raise RuntimeError("transition() runs once, after the warmup")
        if not all(self.started):
            raise RuntimeError("every layer needs at least one warmup chunk before the transition")
        if len(weights) != self.n_layers:
            raise ValueError("one weight matrix per layer")
        d, n = self.d, self.n_layers
        with torch.cuda.stream(self.stream):
            W = torch.stack(list(weights))
        w_new = self._buf(n, d, d, dtype=W.dtype)
        self.delta_w = self._buf(n, d, d)
        ws = self._ws(CALL_ABSORB_SOLVE, None, d, count=n)
        # all layers' absorptions in one batched solve: each layer's Cholesky chain is sequential, side
        # by side they fill the GPU
        absorb_solve_batched(self.G, self.C, W, self.lam, self.lam_relative, self.delta_w, self.info, ws, D=self.D,
                             w_new=w_new, eps=self.eps, lambda_out=self.lambdas, refine=self.refine,
                             stream=self.stream)
        self.w_new = [w_new[l] for l in range(n)]
        # a layer whose factorisation failed (info != 0) has no valid epsilon and ranks last
        select_layers(self.eps, self.k_local, self.role, self.order, info=self.info, stream=self.stream)
        self.stream.synchronize()                                     # the one wait: read the role map back
        self.roles = [int(r) for r in self.role.cpu().tolist()]
        for layer, r in enumerate(self.roles):
            if r == 1:
                self.kv.release_history(layer, stream=self.stream)
                # W_new is fixed from here on: the steady-state step takes it transposed (or coded)
                if self.l_layer == "w8a8_fp8":
                    wq = self._buf(d, d, dtype=torch.uint8)
                    sw = self._buf(d)
                    quantize_weight_fp8(self.w_new[layer], wq, sw, stream=self.stream)
                    self.w_codes[layer] = (wq, sw)
                else:
                    self.w_new_t[layer] = self._buf(d, d, dtype=W.dtype)
                    transpose16(self.w_new[layer], self.w_new_t[layer], stream=self.stream)
            else:
                self.w_new[layer] = None
        self.G = self.C = self.D = None
        self.vt = [None] * n
        if not self.keep_delta_w:
            self.delta_w = None
        self.stage = STEADY
        return list(self.roles)

    def close(self) -> None:
        self.kv.close()

    def converted(self) -> List[int]:
        if self.roles is None:
            raise IspaError(1, "converted(): no transition yet")
        return [i for i, r in enumerate(self.roles) if r == 1]
