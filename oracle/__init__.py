"""CPU oracle for the decode-layer megakernel path.  TEST INFRASTRUCTURE ONLY.

Plain, slow, float64 NumPy implementations of what the decode-layer chain
computes, written from the pages' definitions.  Only ``tests/``,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
this package; the product path (the HIP library and its Python binding) never
does, and shares no code, tables or helpers with it.

Modules
  numerics  bf16 / fp32 rounding and the OCP e4m3 codec, from the format definitions
  ops       one function per step of the chain (add+RMSNorm, quantisation, projections,
            QK-norm, RoPE, cache write, attention, split-KV combine, SiLU-mul, argmax,
            indexer score)
  model     the workloads: one Qwen3-shaped layer, the full decode step, the indexer front
  queue     the host tile-instruction queue builder (tiles -> events -> round-robin queues)
  taskgraph the generic op-graph lowering (tile regions -> pairing rules -> events -> queues),
            pinned by the MegaRTP page's worked attention-pre plan
  bytes     the decode byte / gap estimate model of the handbook

Pages cited: "Kernel-Mega-PDL" (MegaRTP; qingkeai.online), the handbook chapter on
PDL and megakernels (anrans.github.io), the Hazy/MPK/MegaMoE survey
(icarus.shaojiemike.top) and "kernel prologue/epilogue" (xuesongtap.github.io).

Parity status: every numeric step is pinned by closed forms, invariants, brute force
or library special cases in tests/test_oracle_*.py; the composed layer / step /
indexer front have no printed values on the pages and are pinned by their steps plus
an independent torch-CPU formulation on small shapes.
"""
