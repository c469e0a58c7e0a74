"""CPU oracle for the tree-verify hot path -- TEST INFRASTRUCTURE ONLY.

A plain, slow, float64 NumPy implementation of what the three library calls compute,
written from the pages' statement of the method and kept independent of the HIP path
(no shared kernels, headers, helpers, tables or pre/post-processing).  Only the test
suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it; the product path never does.

Sources (page title, section):

* "Luce DFlash" server README -- "How it works" (DDTree tree verify: one forward scores
  every draft-tree node under a mask derived from parent pointers; per-step rollback to
  the committed prefix; the tree-mode gated-delta-net kernels) and "Architecture note"
  (every 4th layer is softmax attention with 24 query / 4 KV heads of length 256, the
  rest Gated DeltaNet with a recurrent state cache); "Asymmetric K/V quantization" and
  the results table on long context (Q8_0 / Q4_0 KV cache, the FA window, 0 = full);
  "Scope and limits" (the verify skeleton stays argmax: greedy acceptance); the
  tree-aware convolution window gathered along the parent chain ("How it works").
* PR #606 "perf(qwen36): add SpecLA factor-capture speculative decoding" -- "Paper
  mapping" (the method needs scored candidates plus parent topology; a chain is a
  degenerate tree) and the review comment naming the commit / flush routines.

The pages name the gated delta rule, the tree mask, the window and the block formats
but never write them out.  The readings taken are stated in each function's docstring.

Parity status: every public function here is pinned by tests in ``tests/`` against
closed forms, hand-worked fixtures or brute force (see ``tests/test_oracle_*.py``).
The byte layouts of Q8_0 / Q4_0 are pinned to hand-written fixtures of the GGUF block
convention, not to the pages (which only name the formats).
"""
from .tree import depths, root_path, ancestor_matrix, validate_tree, validate_path  # noqa: F401
from .delta import (bf16_bits_to_f64, lin_tree_verify, lin_commit_replay,  # noqa: F401
                    lin_chain_recurrence, lin_tree_verify_commit, lin_tree_verify_bank)
from .attention import (dequant_q8_0, dequant_q4_0, dequant_rows, attn_tree_verify,  # noqa: F401
                        attn_tree_verify_rows, attn_tree_verify_dense, visible_slots)
from .accept import (logits_f64, argmax_rows, greedy_walk, tree_accept_greedy,  # noqa: F401
                     kv_compact)
from .conv import conv_tree_verify, conv_tree_commit  # noqa: F401
