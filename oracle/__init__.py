"""Float64 CPU oracle for the attention forward and backward (test infrastructure).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package. The HIP library never calls it and shares no code
with it; the two meet only in the seeded inputs of ``workloads``.
"""
from .attention_f64 import (  # noqa: F401
    softmax,
    streamed_softmax,
    block_states,
    merge_states,
    reduce_states,
    attention_naive,
    attention_naive_rows,
    attention_dense,
    attention_dense_rows,
    attention_varlen,
    attention_varlen_rows,
    blocked_attention,
    scores_to_weights,
)
from .attention_bwd_f64 import (  # noqa: F401
    attention_backward,
    attention_backward_lse,
    attention_backward_dense,
    attention_backward_lse_dense,
    row_dot,
)
from .attention_band_f64 import (  # noqa: F401
    attention_banded,
    attention_banded_rows,
    attention_banded_dense,
    attention_banded_dense_rows,
)
from .dropout_add_norm_f64 import (  # noqa: F401
    philox4x32_10,
    keep_threshold,
    dropout_keep,
    dropout_add_norm,
)
