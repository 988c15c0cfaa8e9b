"""CPU oracle for pyramid top-K block selection and block-sparse causal attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  The
product path (``hierarchical_block_sparse_amd``) never imports it, and this
package imports nothing from the product path: the two share no code.

Everything here is plain NumPy in float64, one unit at a time, written from the
method as the pages describe it:

* PISA (peercurrent.com record of the PISA preprint), abstract: keys are pooled
  into a coarse-to-fine hierarchy of O(log N) levels; selection starts at the
  coarsest level, scores a bounded candidate set at each level with LogSumExp,
  keeps the top K and continues at the next finer level down to the finest one;
  no query-key score matrix is needed.
* PHBA: Prefix-State Hybrid Block Attention (paperlayer.ai summary),
  §A.1.2 "Routing metadata kernels": block summaries are means over the valid
  rows of a block, accumulated in fp32 registers there; routes go only to
  strictly preceding blocks; unavailable route slots hold -1.
* PHBA §3.1 "Top-k block routing": the current block always supplies local
  causal attention.
* PHBA §A.1.3 / §A.2.2 (the fused forward): exact online-softmax attention over
  the routed tokens, writing the output and its log-sum-exp.

Modules:
  reference  -- level-synchronous oracle: pyramid, selection (with per-level
                trace), attention; the readings of the pages it rests on are
                listed in its header.
  tree_walk  -- an independent second formulation of the selection that builds
                the tree explicitly from token ranges (used only to pin
                ``reference`` in the CPU tests).
  check      -- tie-tolerant comparison of a device selection against the
                oracle, level by level along the device's own trace.
"""

from . import reference, tree_walk, check  # noqa: F401
