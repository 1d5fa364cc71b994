"""Write the full-size expected values the GPU parity tests compare against.

Calls only oracle/ and workloads/ (the CPU oracle in float64 on the seeded
synthetic workloads); nothing here touches the GPU library.  Output: one JSON
file per workload in this directory.

* layer_1p3b_bf16 / layer_14b_bf16: lambda, ||dW||_F, the reconstruction error
  epsilon, and a Gaussian sketch S^T dW X (S, X seeded [d, 16]) from which the
  tests estimate ||dW_gpu - dW||_F / ||dW||_F without storing dW.
* warmup_1p3b_30x4: for each of the 30 layers (4 warmup chunks of 3 frames,
  per-layer temporal correlation), lambda, epsilon and ||dW||_F, and the 15
  layers selected for conversion (lowest epsilon).

Usage: OMP_NUM_THREADS=1 python tests/golden/make_golden.py [layer_1p3b_bf16 layer_14b_bf16 warmup_1p3b_30x4]
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


def layer_golden(w: wl.Workload) -> dict:
    s = w.shape
    t0 = time.time()
    x = wl.layer_inputs(w)
    r = oracle.dual_stream(x["q"], x["k"], x["v"], s.n_sink, s.n_hist, s.n_cur, s.n_heads, threads=THREADS)
    G, C, D = oracle.gram_stats([(r["a_loc"], r["delta_a"])])
    lam = oracle.ridge_lambda(G, w.lam, w.lam_relative)
    dW = oracle.solve_delta_w(G, C, x["w"], lam)
    S, X = sketch_mats(s.d)
    return {
        "workload": w.name,
        "lambda": lam,
        "dw_fro": float(np.linalg.norm(dW)),
        "dw_sketch": (S.T @ dW @ X).tolist(),
        "eps": oracle.recon_error_direct(r["a_loc"], r["a_full"], x["w"], dW),
        "eps_traces": oracle.recon_error_traces(G, C, D, x["w"], dW, lam),
        "normal_equation_residual": oracle.normal_equation_residual(G, C, x["w"], dW, lam),
        "seconds": round(time.time() - t0, 1),
    }


def warmup_golden(w: wl.Workload, n_chunks: int = 4, k_local: int = 15) -> dict:
    layers = []
    for layer in range(w.n_layers):
        t0 = time.time()
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
        eps = oracle.recon_error_direct(np.concatenate(loc), np.concatenate(full), W, dW)
        layers.append({"layer": layer, "rho": wl.layer_rho(layer, w.n_layers, w.cfg), "lambda": lam,
                       "eps": eps, "dw_fro": float(np.linalg.norm(dW)), "seconds": round(time.time() - t0, 1)})
        print(f"layer {layer}: eps {eps:.6f} ({layers[-1]['seconds']} s)", flush=True)
    eps = [l["eps"] for l in layers]
    return {"workload": w.name, "n_chunks": n_chunks, "k_local": k_local, "layers": layers,
            "selected": [int(i) for i in oracle.select_local_layers(eps, k_local)]}


def main(names):
    for name in names:
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
