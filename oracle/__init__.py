"""CPU oracle for the ISPA hot path -- TEST INFRASTRUCTURE ONLY.

Plain, slow, float64 NumPy/SciPy implementation of what the hot path computes,
written from the ISPA pages ("Towards Memory-Efficient Autoregressive Video
Generation via Instance-Specific Parametric Absorption"; the gist.science
technical summaries in Dutch and Portuguese, section 2 "Methodology").

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or run anything in this package.  The GPU library never
does, and this package imports nothing from it: the two share no code.

Where the method reaches a result that has a plain definition, the oracle is
that definition written out:

* dual-stream attention -> two *separate* plain two-pass softmax passes (the
  local set and the full set) plus a history-only pass; it never uses the
  log-sum-exp merge to produce A_full (``attention``);
* the absorption -> the ridge normal equations solved by a float64 Cholesky
  factorisation (``absorb``);
* layer selection -> a stable sort of the reconstruction errors (``absorb``);
* KV-cache accounting -> closed-form byte counts (``accounting``);
* the W8A8 variant of the L-layer projection -> per-channel absmax E4M3 codes
  taken from the format definition, then a float64 product of the decoded
  values (``fp8``).

Every function is pinned by ``tests/test_oracle_*.py`` against things other
than itself: brute force on tiny inputs, hand-computed fixtures under
``tests/golden/``, closed forms, limits and invariants.  The only results with
no such pin are the pages' video-quality claims, which are out of scope.
"""
from .attention import (branch_rows, softmax_attention, dual_stream, lse_merge,  # noqa: F401
                        default_scale)
from .absorb import (gram_stats, ridge_lambda, solve_delta_w, recon_error_direct,  # noqa: F401
                     recon_error_traces, select_local_layers, fold_weights, local_layer_output,
                     normal_equation_residual)
from .accounting import attn_flops, kv_cache_bytes, kv_removed_fraction  # noqa: F401
from .fp8 import (local_layer_output_w8a8, local_attention_fp8, local_layer_output_w8a8_fp8attn,  # noqa: F401
                  quantize_weight)
