"""CPU oracle for the Memory Sparse Attention (MSA) hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call,
link or execute this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code,
header, table or helper with the HIP library in ``sparse_latent_memory_amd``
and imports nothing from it.

The oracle is the plain definition of what the method computes, in NumPy
float64, over the exact stored input values.  Sources (web pages about the
method; cited by page title and section):

* [HL] "EverMind-AI/MSA: Memory Sparse Attention for 100M-Token Contexts"
  (hysenlabs.com), section "How MSA compresses and routes documents".
* [TM] "EverMind Releases Memory-Sparse Attention Code for Long-Context AI
  Models" (toolmesh.ai), section "Architectural Design and Inference".
* [GF] "MSA (Memory Sparse Attention) - An Open-Source Answer to AI's Memory
  Bottleneck" (gfox.flashj.cn), section "Key Technical Details".

Every function is pinned by tests under ``tests/`` (closed forms, invariants,
library special cases, hand-derived worked examples).  What stays unpinned is
the link to the original MSA code itself: the pages print no code and no
worked numbers, so the readings listed in each docstring are this project's.
"""

from .msa_oracle import (  # noqa: F401
    EPS,
    round_to_storage,
    round_to_bf16,
    rope_inv_freq,
    rope,
    pool_doc,
    pool,
    pool_offsets,
    row_scores,
    doc_scores,
    topk,
    assemble,
    decode,
    attend,
)
