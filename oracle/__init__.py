"""fp64 CPU oracle for the chunkwise TTT layer and the In-Place W_down update.

Test infrastructure: imported only by tests, the smoke check and the CPU
baseline of the benchmark.  It shares no code with the HIP library.
"""
from .ttt_oracle import (chunk_forward, chunk_backward, token_loop_forward, lr_gate,
                         act_f, act_df, act_d2f, sigmoid)
from .mlp_oracle import mlp_chunk_backward, mlp_chunk_forward, mlp_token_loop_forward
from .norm_oracle import norm_chunk_backward, norm_chunk_forward, norm_token_loop_forward
from .inplace_oracle import (inplace_forward, inplace_rows, inplace_forward_guarded, inplace_rows_guarded,
                             update_norms, inplace_backward, inplace_backward_sampled, inplace_backward_guarded)

__all__ = ["chunk_forward", "chunk_backward", "token_loop_forward", "lr_gate", "act_f",
           "act_df", "act_d2f", "sigmoid", "inplace_forward", "inplace_rows", "inplace_forward_guarded",
           "inplace_rows_guarded", "update_norms", "inplace_backward", "inplace_backward_guarded",
           "inplace_backward_sampled", "mlp_chunk_forward", "mlp_chunk_backward", "mlp_token_loop_forward", "norm_chunk_forward",
           "norm_chunk_backward", "norm_token_loop_forward"]
