"""Plain CPU oracle for the ISD verify-and-propose step.  TEST INFRASTRUCTURE.

This package is the checker, not the product.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  The GPU library never calls it and shares no code with it: the
two sides meet only through the seeded input generators, which hold none of
the method's arithmetic.

Everything here is numpy in float64 (bfloat16 and float32 inputs widen to
float64 exactly), written for reading rather than speed.  Sources, cited by
page title and section:

* "Introspective Diffusion Language Models" (news.routley.io mirror of the
  project README), sections "Inference & ISD", "Serving (SGLang)",
  "Training" and "How do DLMs perform as they approach compute-bound?", plus
  the speedup-explorer panel with the tokens-per-forward formula.
* "I-DLM - Icgozlemsel Difuzyon Dil Modelleri" (GeekNews summary of the same
  README), sections "I-DLM Yontemi", "Throughput", "Speedup Factor Explorer"
  and "Inference & ISD".
* "Introspective Diffusion Language Models" abstract (chatpaper.ai).

Modules
-------
philox     Philox4x64-10 from its published definition (Salmon et al., SC'11).
attention  Strictly causal GQA attention of the 2N-1 step rows over the paged
           KV cache.
accept     The p/q acceptance loop, residual resampling and truncation.
tpf        The tokens-per-forward closed form and the two-state decode chain
           it is the stationary mean of.
kv_cache   KV-cache append (before attention) and rollback to the accepted
           prefix (after acceptance), with a free-list page stack.
propose    The next step's drafts from this forward's MASK rows, and the
           fresh / verify alternation.
lora       R-ISD's gated LoRA on MASK rows after the base projection.
dtypes     Exact widening of bfloat16 bit patterns.

Every function listed has at least one pin in ``tests/`` that ties it to
something other than itself (see the module docstrings).  None is "parity
unpinned".
"""

from . import accept, attention, dtypes, philox, tpf  # noqa: F401
