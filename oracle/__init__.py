"""Oracle for one decode step of attention over a KV cache.

TEST INFRASTRUCTURE ONLY: the tests, the package smoke check and the
benchmark's CPU-baseline leg use it; the library never imports it.

Independent CPU implementations of the same definition,
softmax(Q K^T / sqrt(d)) V with explicit masks, in float64:
  * `decode` / `decode_rows` - the C oracle (kvattn_oracle.c), OpenMP;
  * `decode_np` - a NumPy twin with its own slot mapping and mask;
  * `decode_matmul_np` - the same definition in matrix form (library float64
    matmuls per sequence and KV head), for the hundreds of rows of a prefill chunk.
Plus the pieces the pins need: a full T x T causal attention, the tiled
online-softmax form and a split + log-sum-exp merge; and `append_np`, the KV
append (the new rows written to their cache slots) that precedes a decode.
"""
from .oracle import (  # noqa: F401
    DTYPE_CODES, CACHE_CODES, MASK_CODES, load, decode, decode_rows, attended,
    decode_np, decode_matmul_np, attended_positions_np, slot_np, full_causal_np,
    tiled_softmax_dot_np, split_merge_np, to_f64, threads, append_np, tree_words,
)
