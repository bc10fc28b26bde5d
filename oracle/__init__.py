"""fp64 CPU oracle for the gated delta rule forward pass.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports, calls or links
this package: only the tests, the smoke check and the benchmark's CPU-baseline
leg do. It shares no code with the HIP library.

Three independent statements of the method:
  * ``recurrent``  - the tokenwise recurrence (the definition);
  * ``chunkwise``  - the exact chunk regrouping with a hand-written forward
                     substitution (pins the regrouping the kernels rely on);
  * ``bruteforce`` - closed parallel forms on tiny inputs (masked linear
                     attention, decayed scores, the full-sequence delta solve).
``product`` states Gated DeltaProduct (n_h transitions per token) the same
tokenwise way; ``backward`` the gradients of causal linear attention;
``ring`` the speculative-decode verify ring and its state fold;
``recurrent_bwd`` the gradients of the gated delta and gated linear rules.
Every function names the passage of the pages it follows. Where the pages are
silent the reading taken is stated in the function's docstring.

Parity status: every function here is pinned by a CPU test against a property
the pages or the mathematics fix (tests/test_oracle_*.py). None is "parity
unpinned".
"""
from .recurrent import (recurrent_fp64, round_to_storage, round_f64_to_bf16,
                        l2_normalise_fp64, L2_EPS)
from .chunkwise import chunkwise_fp64, forward_substitution_unit_lower
from .bruteforce import (linear_parallel_fp64, delta_parallel_fp64,
                         four_token_chunk_fractions)
from .product import delta_product_fp64
from .backward import linear_attention_grads_fp64
from .ring import ring_record_elements, verify_ring_fp64, state_fold_fp64
from .recurrent_bwd import recurrent_grads_fp64

__all__ = ["recurrent_fp64", "round_to_storage", "round_f64_to_bf16",
           "l2_normalise_fp64", "L2_EPS",
           "chunkwise_fp64", "forward_substitution_unit_lower",
           "linear_parallel_fp64", "delta_parallel_fp64",
           "four_token_chunk_fractions", "delta_product_fp64",
           "linear_attention_grads_fp64", "ring_record_elements", "verify_ring_fp64",
           "state_fold_fp64", "recurrent_grads_fp64"]
