"""CPU float64 oracle of the tensor-parallel shard — TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
anything here. The oracle shares no code with the HIP path (only the seeded
input generator tp_inputs serves both) and imports nothing from it.
"""
from .oracle import (  # noqa: F401
    column_linear_fwd,
    gelu_tanh,
    gelu_tanh_grad,
    linear_bwd_dgrad,
    linear_bwd_wgrad,
    mlp_unsharded,
    reduce_partials,
    rel_fro,
    row_linear_fwd_partial,
    run_config,
    sampled_dot,
    shard_columns,
    shard_rows,
    tp_attn_proj,
    tp_mlp,
)
