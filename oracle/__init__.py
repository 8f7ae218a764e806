"""fp64 CPU oracle for the retention hot path -- test infrastructure only.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may use
this package.  It shares no code with the HIP library.
"""
from .retention import (XPOS, SCALE_QK, NORM_DROW, NORM_SCORE, NORM_ALL,  # noqa: F401
                        gammas, thetas, xpos_rotate, retention_recurrent,
                        retention_parallel, retention_chunkwise, retention_parallel_bwd, recurrent_step,
                        swish, group_norm_heads, gate_norm, split_heads, msr_forward,
                        layer_norm, gelu, ffn, retnet_layer, retnet_stack, msr_step,
                        retnet_decode_step, zero_states)
