"""CPU oracle for the tree-masked verify/expand attention path.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, float64 statement
of what the GPU library computes.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import it; the library itself never does, and
it shares no code, tables or helpers with the HIP kernels.

Sources (the pages are cited by title and section/figure):

* "SwiftSpec summary -- Disaggregated Speculative Decoding": draft tree
  (Section 3.1), non-square expansion mask (Section 3.1.3, Figure 3),
  maximum-likelihood expansion (Section 3.1.3), evolving tree cache invariant
  and re-root (Section 3.2, Figure 4), iteration example (Section 3.1.2,
  Figure 2).
* "MineDraft notes": the residual distribution a rejected draft token is
  resampled from (the PEARL walkthrough), sampling at temperature 1.0.
* "Draft-length co-design" article: acceptance up to the first mismatch plus
  the target's own token, AL in [1, 1+D], G x (1+D) query rows per KV head
  (its "key mechanism" and "how speculative decoding works" parts).

Modules:

* ``tree``      -- ancestors, depth, descendants, validity (brute force).
* ``attention`` -- explicit-mask softmax attention in float64.
* ``accept``    -- greedy longest accepted path by enumerating every node.
* ``reroot``    -- evolving-tree-cache re-root and KV compaction.
* ``topw``      -- top-w maximum-likelihood candidate selection (the draft
  expansion rounds).
* ``draft``     -- the draft side's walk along the verified tokens and the
  choice of the subtree to send (Algorithm 1, Re-root and Select).
* ``rope``      -- rotary position embedding at tree positions and the KV
  append of the new nodes.
* ``sampling``  -- tree verification by speculative sampling (temperature
  > 0, residual resampling on rejection).
* ``bf16``      -- exact bfloat16 -> float64 decoding.

Pins: every function here is checked in ``tests/test_oracle_*.py`` against
facts fixed by the pages or by mathematics (causal attention from a library
routine, closed forms, the Figure 2/3/4 examples, exhaustive small trees,
exact losslessness of the sampling rule).  What no pin fixes is a matter of
precision or of the pages' silence, not a function: bfloat16 output rounding
is covered by tolerances only, Figure 3 fixes the visible set of one row
(t7), and ties among top-w candidates beyond the stated tie order have
several valid answers.
"""
from .bf16 import bf16_to_f64, to_f64  # noqa: F401
from .tree import ancestors, depth, descendants, is_valid_parent, root_path  # noqa: F401
from .attention import tree_attention, verify, expand, gather_sequence_kv  # noqa: F401
from .accept import accept_greedy_path, argmax_first  # noqa: F401
from .reroot import reroot_node_arrays, tree_cache_reroot  # noqa: F401
from .topw import cumulative_scores, select_top_w  # noqa: F401
from .draft import token_walk, select_subtree  # noqa: F401
from .rope import rope, tree_positions, rope_append  # noqa: F401
from .sampling import accept_sampling_path, residual, sample_inverse_cdf, softmax_t  # noqa: F401
