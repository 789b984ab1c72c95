"""Plain fp64 CPU oracle for the rotated grouped-affine low-bit linear layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls, links
or runs anything in this package.  Its only users are the tests under
``tests/``, ``__graft_entry__.smoke()`` (which checks one small GPU result
against it) and the ``cpu_baseline`` leg of ``bench.py`` (which times it as
a reported CPU baseline).  It shares no code, header, table or constant
generator with the HIP library; the two meet only in the seeded inputs of
the ``workloads`` module.

Every function is written to be checked by eye against the model cards it
follows.  The sources are five model cards; the ones used here are

* "24B0978 - Week 01 - Track 2, 20% target - Submission 01"
  (section "How these techniques accelerate inference on CUDA", paragraphs
  on group-wise affine integer quantisation, on the random Hadamard
  transform, on the absence of unstructured sparsity, and on trained scales
  and zero points), cited below as [W01];
* "24B0978 - Week 02 - Track 2, 40% target - Submission 01"
  (sections "Recipe" and "Recipe (exact)"), cited as [W02];
* "24B0908 ... Mixed-precision GPTQ" (section "CUDA speedup potential"),
  cited as [GPTQ3];
* "25M2111-Week02-Track2-40-Submission01" (section "Method, selection, and
  reproduction"), cited as [MIX].

Modules:
  hadamard  - Sylvester Hadamard matrix, block random Hadamard rotation
  rtn       - weight-side rotation and round-to-nearest quantisation
  pack      - bit placement of codes into 32-bit words (uniform and mixed)
  linear    - dequantisation and the plain triple-loop contraction (C)
  embed     - rows of a quantised table, dequantised (tied-embedding gather)

Every function carries a pin in ``tests/test_oracle_*.py``.
"""

from . import hadamard, rtn, pack, linear, embed  # noqa: F401
