"""Plain, slow fp64 CPU reference for jagged attention — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import anything from this package. The GPU library never calls it and shares no code with it:
not a kernel, a helper, a table or a constant generator. It reads operands from ``jfa_inputs``
(seeded generators that hold no attention arithmetic) and computes, with numpy float64, the plain
definition of what the jagged attention kernels reach by tiling:

* ``attention.forward`` / ``attention.backward`` — softmax attention (the FlashAttention result
  that "Jagged Sequence Flash Attention" computes on values+offsets tensors, aihot.vn GEM page,
  section "Jagged Sequence Flash Attention"; kerneldigest.dev page, section "Fundamentos
  Teóricos", for the FlashAttention lineage) and the generalised dot-product attention where a
  pointwise SiLU or GELU replaces softmax between the two matrix products (aihot.vn GEM page,
  section "Generalized Dot-Product Attention (GDPA)"); per-sequence lengths come from offsets
  (vibekk.com GEM page, FAQ entry on jagged tensors);
* ``bucket.bucket`` — the 64-way log-bucketed relative distance that indexes the learned bias
  table (a reading: the pages give no bucket law);
* ``schedule.*`` — the work lists the planner must emit, written from the scheduling rules.

Every function here is pinned by ``tests/test_oracle_*.py`` against something other than itself
(brute-force padded attention through a library routine, closed forms, invariants, finite
differences, a boundary-enumeration bucket construction). No function is "parity unpinned".
"""
