"""CPU oracle for the SPTS prefill hot path -- TEST INFRASTRUCTURE ONLY.

Source: "Probe and Skip: Self-Predictive Token Skipping for Efficient
Long-Context LLM Inference" (Wu, Wang, Jin, Chen, Wang), cited below as
[SPTS] with the abstract, figure or table each step follows.

This package is a plain, slow, obviously-correct restatement of what the hot
path computes, in numpy float64 with bfloat16 rounding only at the storage
points the GPU path also has.  It exists to check the HIP library.  Only the
test suite, the smoke entry point and the CPU-baseline leg of the benchmark
may import it; the product path (the C-ABI library and its Python binding)
never does, and shares no code, tables or helpers with it.

Modules
  numerics   bf16 round-to-nearest-even via integer ops on the fp32 pattern
  pap        Partial Attention Probing score          [SPTS] Fig. 2(a), abstract
  select     top-k token selection, MaxNorm-Add fusion [SPTS] Fig. 2(a)(b), Table D
  attention  reduced causal attention over selected queries [SPTS] Fig. 2(a)
  ltp        Low-rank Transformation Probing score    [SPTS] Fig. 2(b), abstract
  ffn        reduced SwiGLU feed-forward               [SPTS] Fig. 2(b)
  normrope   RMSNorm and rotary embedding (LLaMA-shaped stack only; the pages
             name neither, the workload does)
  layer      one SPTS layer, and the Multi-Stage Delayed Pruning stack
             [SPTS] Fig. 2(c), Fig. A(c), Table B
  costs      KV-cache bookkeeping of Table 5 and proxy cost of Table A

Parity status: every function here is pinned by tests under tests/ against
closed forms, brute force, library routines or the tables the pages print,
except the whole-method composition, whose accuracy against the paper's
model is "parity unpinned" (the pages print no example values for it).
"""

from . import numerics, pap, select, attention, ltp, ffn, normrope, layer, costs  # noqa: F401
