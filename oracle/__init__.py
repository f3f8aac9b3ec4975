"""CPU oracle for the fused block O = f(A.B).C (test infrastructure only).

This package is the independent checker of the HIP path.  Only the test
suite, the smoke check and the CPU-baseline leg of the benchmark may import
it; the product path never calls it and shares no code with it.
"""
from .fab_oracle import (  # noqa: F401
    attention_forward,
    attention_backward,
    attention_forward_rows,
    attention_backward_rows,
    attention_backward_keys,
    attention_probs,
    attention_merge,
    mlp_forward,
    mlp_backward,
    mlp_forward_rows,
    gelu,
    gelu_grad,
    brute_attention_forward,
    brute_attention_backward,
    brute_mlp_forward,
    ulysses_heads_per_rank,
    ulysses_pack,
    ulysses_unpack,
    ulysses_sequence_view,
    all_to_all,
)
