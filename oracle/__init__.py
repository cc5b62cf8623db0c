"""CPU oracle for exact multi-head self-attention — TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import or call this package. The GPU library never does, and nothing here is
shared with it.

See ``oracle.attention`` (the definition), ``oracle.masked`` (key-padding and
causal masks) and ``oracle.projection`` (the query/key/value projection that
feeds attention) for the definitions and their citations.
"""
from .attention import (  # noqa: F401
    attention_probs,
    attention_fwd,
    attention_bwd,
    attention_ds,
    brute_attention_fwd,
    brute_attention_grads_fd,
)
from .masked import (masked_attention_bwd, masked_attention_dq_rows, masked_attention_ds,  # noqa: F401
                     masked_attention_fwd, visible_keys)
from .projection import brute_qkv_projection, qkv_projection, qkv_projection_bwd, split_qkv  # noqa: F401
