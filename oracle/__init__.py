"""CPU oracle for the one-GPU MoE layer hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and ``bench.py``'s CPU-baseline leg use it.  It shares no code with the HIP
path (``mixture_experts_layer_device_amd``) and imports nothing from it; the
only thing both sides take from a common module is the seeded input draw
(``workloads``), which holds none of the layer's arithmetic.

The oracle is plain numpy, slow and obviously correct: float work in fp64
unless a step's precision decides an integer (router top-k, MXFP8 codes), in
which case that step is done in the precision the step itself defines.

Sources.  The pages describe Mixture-of-Kittens (MoK), a deterministic MoE
training megakernel:

* [MTP] MarkTechPost, "Cursor Open-Sources Mixture-of-Kittens (MoK): A
  Deterministic MoE Training Megakernel for GB300 NVL72 Racks" (English
  original on news.ainew.jp) -- sections "Three design decisions that
  matter", "Results", "Key Takeaways" and the paragraph after the design
  decisions.
* [CARD] agentlenshq project card "Mixture‑of‑Kittens (MoK)" (English) --
  "Use the functional API", "Core concepts", "Limitations".
* [WIKI] notes.yuuk.io wiki page "Mixture-of-Kittens: our open-source MoE
  megakernel for NVL72s" -- "technical focus" items 1-3.

Readings where the pages are silent or garbled are listed per function and
collected in the repository's design notes.

Pin status: every function here is pinned by ``tests/test_oracle_*.py``
(brute force, closed forms, invariants, finite differences, exhaustive
quantiser checks, independent library casts).  None is "parity unpinned".
"""
from . import bf16, route, schedule, mxfp8, layer, sizing  # noqa: F401

__all__ = ["bf16", "route", "schedule", "mxfp8", "layer", "sizing"]
