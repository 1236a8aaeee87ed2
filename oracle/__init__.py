"""Oracle: a plain, slow, unsharded CPU reference of the tensor-parallel
linear path, in float64.

TEST INFRASTRUCTURE ONLY. It is imported by the tests, by the smoke check of
``__graft_entry__`` and by the CPU-baseline leg of ``bench.py``, and by nothing
else. It shares no code with the HIP library and imports nothing from it.

Parity status of each function (what pins it, in tests/test_oracle_pins.py):
  round_bf16            pinned: torch's float32->bfloat16 cast on every float32
                        class (normal, subnormal, ties, overflow) and hand cases.
  linear                pinned: exact rational brute force on tiny inputs; the
                        row-split sum and column-split concat identities on
                        integer inputs.
  silu / swiglu         pinned: closed forms (silu(0)=0, sigmoid(1)), the
                        identity silu(x) = x (1 + tanh(x/2)) / 2, asymptotes.
  all_reduce_sum        pinned: integer partials and closed-form sums.
  all_gather_concat     pinned: hand-built shards with known positions.
  embedding_lookup      pinned: the masked-shard sum identity, planted -0.0,
                        subnormal and NaN-padding rows.
  head / vocab maps     pinned: per-card KV sizes printed on the pages, the
                        GQA grouping invariant, hand-worked tiny cases in
                        tests/golden, the workload shard sizes.
  rms_norm              pinned: closed forms (constant rows, unit-RMS rows, a
                        hand-worked 3-4 row), invariance under positive
                        scaling, per-row independence, eps monotonicity.
  add_rms_norm          pinned: the add rounded once to bf16 (hand cases,
                        torch's bf16 add), then rms_norm.
  gqa_decode_attention  pinned: uniform scores give the mean of V, one
                        dominant score selects its V row, invariance under a
                        joint permutation of positions, GQA head grouping,
                        torch's float64 scaled_dot_product_attention.
  append_kv             pinned: hand-placed rows.
  layer_linear_path     composed of the pinned functions above.
"""

from .bf16 import round_bf16, bf16_bits
from .tp_ref import (
    linear, silu, swiglu, all_reduce_sum, all_gather_concat, embedding_lookup,
    q_heads_of_rank, kv_heads_of_rank, gqa_group, vocab_shard_rows,
    vocab_range_of_rank, qkv_shard_rows, gate_up_shard_rows, o_shard_cols,
    down_shard_cols, vocab_shard, shard_weight, vocab_embed_shard,
    vocab_embed_from_shard, column_linear_rank, row_linear_rank_partial, layer_linear_path,
    rms_norm, add_rms_norm, gqa_decode_attention, append_kv,
)

__all__ = [
    "round_bf16", "bf16_bits", "linear", "silu", "swiglu", "all_reduce_sum",
    "all_gather_concat", "embedding_lookup", "q_heads_of_rank",
    "kv_heads_of_rank", "gqa_group", "vocab_shard_rows", "vocab_range_of_rank",
    "qkv_shard_rows", "gate_up_shard_rows", "o_shard_cols", "down_shard_cols",
    "vocab_shard", "shard_weight", "vocab_embed_shard", "vocab_embed_from_shard", "column_linear_rank",
    "row_linear_rank_partial", "layer_linear_path", "rms_norm", "add_rms_norm",
    "gqa_decode_attention", "append_kv",
]
