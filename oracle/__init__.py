"""CPU oracle of the tensor-parallel block shard (fp64 NumPy).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the package entry point's smoke check and by
the benchmark's CPU-baseline leg, never by the product path. It shares no code with the HIP
library or its binding.

Parity unpinned: the absolute values of a whole block's output. The pages print no numeric
example of a block; the output is pinned only through the pins of its parts (sharded equals
unsharded, library cross-checks of every sublayer, brute force on tiny shapes, closed forms).
"""
from .block import (  # noqa: F401
    ACTIVATIONS, attend, attention_sharded, bf16_bits_to_f64, block_sharded, block_unsharded, caches_f64,
    dequant_q8_0, embed_lookup, f16_bits_to_f64, gelu_tanh, head_table_f64, lm_head, params_f64,
    moe_ffn_sharded, moe_ffn_unsharded, moe_params_f64, moe_route, moe_select, rank_caches,
    rms_norm, rope, rope_cos_sin, round_to_bf16, run_block, run_model, run_moe_block, run_stack,
    shard_slices, shard_weights, silu, to_f64,
)
