"""CPU float64 oracle for exact scaled dot-product attention.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports, calls or links this
package: only the tests, the smoke entry point and the bench's CPU baseline leg may.
It shares no code, constant or helper with the HIP path.

Contents
--------
attention         The plain definition: S = scale*Q K^T with the causal and key-padding
                  masks, safe softmax, O = P V, LSE = m + ln(l), and the chain-rule
                  backward. Materialises S and P (per head, in row blocks).
page_algorithms   The softmax / attention recurrences the pages derive (3-pass safe
                  softmax, 2-pass online softmax, 2-pass and 1-pass FlashAttention rows,
                  the tiled recurrence, the Br x Bc block update, the statistics merge,
                  and the issue thread's deferred P V variant), written as scalar
                  float64 loops. They cross-check the definition.
split             Split-KV: attention over contiguous key ranges (normalised partial
                  outputs with their LSE, empty rows O = 0, LSE = -inf) and the merge
                  of partials by the incremental softmax tracking rule.
sparse            Block-sparse attention: the definition with a block mask over
                  query/key blocks (empty rows O = 0, LSE = -inf) and its gradient.
dropout           Dropout on the probabilities with the counter-based Philox4x32-10
                  generator (the mask replayed from (seed, offset)), and its gradient.

Every function is pinned by tests in tests/test_oracle_*.py against closed forms,
invariants, brute force, finite differences, independent library routines and
hand-derived fixtures in tests/golden/. No function here is "parity unpinned".
"""
from .attention import (  # noqa: F401
    allowed_mask,
    head_forward,
    head_backward,
    head_row_block,
    attention_forward,
    attention_backward,
    attention_forward_heads,
    attention_backward_heads,
)
from .dropout import (  # noqa: F401
    philox4x32,
    dropout_threshold,
    keep_scale,
    random_bytes,
    keep_mask,
    head_forward_dropout,
    head_backward_dropout,
    attention_forward_dropout,
    attention_backward_dropout,
)
from .sparse import (  # noqa: F401
    block_allowed,
    head_forward_sparse,
    head_backward_sparse,
    head_row_block_sparse,
    attention_forward_sparse,
    attention_backward_sparse,
)
from .split import (  # noqa: F401
    split_ranges,
    head_forward_range,
    attention_forward_split,
    merge_pair,
    merge_partials,
)
