"""Float64 CPU oracle for the sparse decode step.

TEST INFRASTRUCTURE ONLY. Nothing in the product path (the HIP library under
``kv_cache_activation_amd/`` and its Python binding) may import, call or link
anything in this package.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.

The oracle is plain numpy in float64.  It shares no code with the HIP path:
both sides receive the same seeded inputs from ``synth`` (which holds no
arithmetic of the method) and are compared element by element.

Sources, cited by title and section (the text of the pages, not any code):

* [Cross]  "Where Activation Sparsity and KV-Cache Sparsity Cross in LLM
  Decoding" -- the subject: byte account (§3), SnapKV-style one-time KV
  selection gathered into a contiguous buffer (§4.1), split-K decode attention
  shared by dense and sparse modes (§1, §4.1, §4.4), composition (§4.2, §5.3).
* [SATS]   "Sensitivity-Aware Thresholding and Token Routing for Activation
  Sparsification in Large Language Models" -- the CATS runtime mask on the
  post-gate (SiLU) activation magnitude with a per-layer threshold, and the
  percentile calibration of that threshold (text around Eq. 6).
* [CateKV] "CateKV: On Sequential Consistency for Long-Context LLM Inference
  Acceleration" (summary page) -- observation-window sizes used by SnapKV
  (Appendix B.1).

Modules
-------
byte_account  bytes per step, savings, speedup bounds, crossover lengths.
selection     observation-window scoring, per-KV-head top-k, gather.
attention     exact softmax attention over a row set; split-K combine.
cats          SiLU gate, |a| > t mask, masked-dense SwiGLU MLP, calibration.
step          RMSNorm, RoPE, bf16 rounding, one decoder layer, a full step.

Parity status of each function is stated in its module header.
"""

from . import byte_account, selection, attention, cats, step  # noqa: F401
