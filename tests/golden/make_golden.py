"""Write the full-size expected values the GPU parity tests compare against.

Calls only oracle/ and workloads/ (the CPU oracle in float64 on the seeded
synthetic workloads); nothing here touches the GPU library.  Output: one JSON
file per workload in this directory.

* layer_1p3b_bf16 / layer_14b_bf16: lambda, ||dW||_F, the reconstruction error
  epsilon, and a Gaussian sketch S^T dW X (S, X seeded [d, 16]) from which the
  tests estimate ||dW_gpu - dW||_F / ||dW||_F without storing dW; for the 14B
  layer also four seeded whole rows and four whole columns of dW (float32), which
  the test compares element by element.
* warmup_1p3b_30x4: for each of the 30 layers (4 warmup chunks of 3 frames,
  per-layer temporal correlation), lambda, epsilon, ||dW||_F, the sketch of
  dW, and G, C, D (accumulated over the 4 x 4680 warmup tokens) at seeded
  sampled entries; the 15 layers selected for conversion (lowest epsilon); and,
  for the first selected layer, its output rows in the first steady-state chunk
  (chunk 4) as a converted layer, with W_new = W + dW stored in bf16: the 16-bit
  step and the W8A8 step with FP8 attention.

Usage: OMP_NUM_THREADS=1 python tests/golden/make_golden.py [layer_1p3b_bf16 layer_14b_bf16 warmup_1p3b_30x4]
       python tests/golden/make_golden.py warmup_1p3b_30x4:steady   (adds only the steady-state rows to
       the existing file, recomputing the one layer's dW)
"""
from __future__ import annotations

import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads as wl  # noqa: E402

SKETCH_CFG = 99          # seeds of the sketch matrices (unit 0: S, unit 1: X)
SKETCH_K = 16
THREADS = int(os.environ.get("GOLDEN_THREADS", "8"))


def sketch_mats(d: int):
    return wl.normal((d, SKETCH_K), SKETCH_CFG, 0, 0, 0), wl.normal((d, SKETCH_K), SKETCH_CFG, 0, 1, 0)


def sample_entries(d: int, n: int = 64, n_diag: int = 16):
    """Seeded (row, column) pairs of a d x d statistic: n random pairs, then n_diag diagonal entries."""
    rng = np.random.default_rng(np.random.SeedSequence([wl.ROOT_SEED, SKETCH_CFG, d, 2]))
    ii, jj = rng.integers(0, d, n), rng.integers(0, d, n)
    dg = rng.integers(0, d, n_diag)
    return np.concatenate([ii, dg]), np.concatenate([jj, dg])


def sample_lines(d: int, n: int = 4):
    """Seeded row and column indices of dW stored whole."""
    rng = np.random.default_rng(np.random.SeedSequence([wl.ROOT_SEED, SKETCH_CFG, d, 3]))
    return np.sort(rng.choice(d, n, replace=False)), np.sort(rng.choice(d, n, replace=False))


def layer_golden(w: wl.Workload) -> dict:
    s = w.shape
    t0 = time.time()
    x = wl.layer_inputs(w)
    r = oracle.dual_stream(x["q"], x["k"], x["v"], s.n_sink, s.n_hist, s.n_cur, s.n_heads, threads=THREADS)
    G, C, D = oracle.gram_stats([(r["a_loc"], r["delta_a"])])
    lam = oracle.ridge_lambda(G, w.lam, w.lam_relative)
    dW = oracle.solve_delta_w(G, C, x["w"], lam)
    S, X = sketch_mats(s.d)
    lines = {}
    if w.name == wl.LAYER_14B.name:
        rows, cols = sample_lines(s.d)
        lines = {"dw_rows": {"index": rows.tolist(), "values": dW[rows].astype(np.float32).tolist()},
                 "dw_cols": {"index": cols.tolist(), "values": dW[:, cols].T.astype(np.float32).tolist()}}
    return {
        **lines,
        "workload": w.name,
        "lambda": lam,
        "dw_fro": float(np.linalg.norm(dW)),
        "dw_sketch": (S.T @ dW @ X).tolist(),
        "eps": oracle.recon_error_direct(r["a_loc"], r["a_full"], x["w"], dW),
        "eps_traces": oracle.recon_error_traces(G, C, D, x["w"], dW, lam),
        "normal_equation_residual": oracle.normal_equation_residual(G, C, x["w"], dW, lam),
        "seconds": round(time.time() - t0, 1),
    }


def warmup_layer_dw(w: wl.Workload, layer: int, n_chunks: int):
    """The oracle's statistics and dW of one layer over its warmup chunks (plus the local and full
    outputs and dA per chunk)."""
    n_frames = 1 + w.chunk_frames * n_chunks
    fr = wl.rollout_frames(w, layer, n_frames)
    W = wl.rollout_weight(w, layer)
    loc, full, da = [], [], []
    for c in range(n_chunks):
        sh = wl.chunk_shape(w, c)
        qs, n_rows = wl.chunk_rows(w, c)
        r = oracle.dual_stream(fr["q"][qs], fr["k"][:n_rows], fr["v"][:n_rows], sh.n_sink, sh.n_hist, sh.n_cur,
                               sh.n_heads, threads=THREADS)
        loc.append(r["a_loc"])
        full.append(r["a_full"])
        da.append(r["delta_a"])
    G, C, D = oracle.gram_stats(zip(loc, da))
    lam = oracle.ridge_lambda(G, w.lam, w.lam_relative)
    dW = oracle.solve_delta_w(G, C, W, lam)
    return W, G, C, D, lam, dW, loc, full


def steady_rows(w: wl.Workload, layer: int, W, dW, n_chunks: int) -> dict:
    """Output rows of `layer` as a converted layer in the first steady-state chunk (chunk n_chunks):
    local attention over sink + current chunk, projected by W_new = W + dW stored in bf16 (the layer's
    weight dtype); the 16-bit step and the W8A8 step with FP8 attention.  Six rows spread over the
    chunk's queries (the test reads the same ones)."""
    c = n_chunks
    sh = wl.chunk_shape(w, c)
    qs, n_rows = wl.chunk_rows(w, c)
    fr = wl.rollout_frames(w, layer, n_rows // w.frame, as_f32=True)
    q = np.asarray(fr["q"][qs], dtype=np.float64)
    k = np.asarray(fr["k"][:n_rows], dtype=np.float64)
    v = np.asarray(fr["v"][:n_rows], dtype=np.float64)
    rows = np.linspace(0, sh.n_q - 1, 6).astype(int)
    loc = oracle.branch_rows(sh.n_sink, sh.n_hist, sh.n_cur)["local"]
    w_new = wl.round_to(oracle.fold_weights(W, dW), "bf16")
    out16 = oracle.local_layer_output(q[rows], k[loc], v[loc], sh.n_sink, sh.n_cur, sh.n_heads, w_new, threads=THREADS)
    out8 = oracle.fp8.local_layer_output_w8a8_fp8attn(q[rows], k[loc], v[loc], sh.n_sink, sh.n_cur, sh.n_heads,
                                                      w_new)
    return {"chunk": c, "layer": layer, "rows": rows.tolist(), "out_bf16": out16.tolist(), "out_w8a8_fp8": out8.tolist()}


def warmup_golden(w: wl.Workload, n_chunks: int = 4, k_local: int = 15) -> dict:
    layers = []
    dws = []
    for layer in range(w.n_layers):
        t0 = time.time()
        W, G, C, D, lam, dW, loc, full = warmup_layer_dw(w, layer, n_chunks)
        dws.append((W, dW))
        eps = oracle.recon_error_direct(np.concatenate(loc), np.concatenate(full), W, dW)
        S, X = sketch_mats(G.shape[0])
        ii, jj = sample_entries(G.shape[0])
        layers.append({"layer": layer, "rho": wl.layer_rho(layer, w.n_layers, w.cfg), "lambda": lam,
                       "eps": eps, "dw_fro": float(np.linalg.norm(dW)), "dw_sketch": (S.T @ dW @ X).tolist(),
                       "g_samples": G[ii, jj].tolist(), "c_samples": C[ii, jj].tolist(),
                       "d_samples": D[ii, jj].tolist(), "seconds": round(time.time() - t0, 1)})
        print(f"layer {layer}: eps {eps:.6f} ({layers[-1]['seconds']} s)", flush=True)
    eps = [l["eps"] for l in layers]
    ii, jj = sample_entries(w.shape.d)
    selected = [int(i) for i in oracle.select_local_layers(eps, k_local)]
    return {"workload": w.name, "n_chunks": n_chunks, "k_local": k_local, "layers": layers,
            "sample_rows": ii.tolist(), "sample_cols": jj.tolist(), "selected": selected,
            "steady": steady_rows(w, selected[0], *dws[selected[0]], n_chunks)}


def add_steady(w: wl.Workload) -> None:
    path = os.path.join(HERE, f"{w.name}.json")
    with open(path) as f:
        g = json.load(f)
    layer = g["selected"][0]
    W, _, _, _, _, dW, _, _ = warmup_layer_dw(w, layer, g["n_chunks"])
    g["steady"] = steady_rows(w, layer, W, dW, g["n_chunks"])
    with open(path, "w") as f:
        json.dump(g, f, indent=1)
    print("added the steady-state rows to", w.name, flush=True)


def main(names):
    for name in names:
        if name.endswith(":steady"):
            add_steady(wl.WORKLOADS[name.split(":")[0]])
            continue
        w = wl.WORKLOADS[name]
        out = warmup_golden(w) if name == wl.WARMUP_1P3B.name else layer_golden(w)
        out["citation"] = ("ISPA technical summary (gist.science, nl/pt), section 2: stage 1 dual-stream "
                           "warmup, stage 2 closed-form absorption, dynamic layer selection by epsilon; "
                           "values computed by the float64 CPU oracle on the seeded synthetic workload")
        with open(os.path.join(HERE, f"{name}.json"), "w") as f:
            json.dump(out, f, indent=1)
        print("wrote", name, flush=True)


if __name__ == "__main__":
    main(sys.argv[1:] or [wl.LAYER_1P3B.name, wl.LAYER_14B.name, wl.WARMUP_1P3B.name])
