"""Plain fp64 CPU oracle for exact attention: forward pass and gradients.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check
in ``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import
or call anything in this package.  The product path (the HIP library and its
Python binding) never calls it and shares no code with it.

Every function here follows the definition of exact attention given on the
page "FlashAttention: Fast and Memory-Efficient Exact Attention with
IO-Awareness" (reading notes at notes.yuuk.io), section "problem setting":
inputs Q, K, V hold N rows of d features per head, and the output is
softmax(Q K^T) V, here with the caller's scale and optional causal mask.

Pins (see ``tests/test_oracle_pins.py``): materialised brute force, an
exactly rounded ``math.fsum`` variant, torch's float64 SDPA, closed forms
(uniform, identity, single peak, causal prefix means), invariants (rows of P
sum to one, constant V, one key, causal row 0, key/value permutation, score
shift), the one-hot limit, and the worked mask example printed on the page
"flash-attnの代役がVRAMを18GB溶かしていたので87%削った話" (Qiita), section 6;
key-padding and block-sparse masks against shard merges and sub-problems.
Gradients (``oracle.backward``): central finite differences of the forward
oracle and torch's float64 autograd.
"""

from .backward import attention_backward, attention_backward_sampled  # noqa: F401
from .fp64 import (  # noqa: F401
    attention,
    attention_fsum,
    attention_materialised,
)
