"""Byte and flop accounting for one decode step (measurement code, no GPU work).

KV bytes per token follow the closed form both the nextadmin.net lesson
("KV cache math") and the dothoosh.com StreamingLLM article ("KV-cache memory
bottleneck") give: 2 (one K and one V vector) x layers x KV heads x head width x
bytes per element.

Algorithmic bytes of one step are what a perfect kernel must move: the K and V
rows of every attended position read once, Q read once, the output written
once, seq_lens, and the page-table entries of the pages touched.  Algorithmic
flops are 2 per multiply-add of Q K^T and of P V (4 x Hq x q_len x d per
attended position); the few masked entries of the causal corner are ignored.
"""
from __future__ import annotations

from typing import Sequence

ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "fp8": 1}


def kv_dtype(case) -> str:
    """Element type of the caches (the case's kv_dtype, else its dtype)."""
    return getattr(case, "kv_dtype", None) or case.dtype


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, bytes_per_element: int) -> int:
    return 2 * layers * kv_heads * head_dim * bytes_per_element


def attended_span(mask_mode: str, T: int, q_len: int, n_sink: int, window: int):
    """Logical positions any of the q_len new rows attends, as (sink_count, tail_start, T):
    the union is [0, sink_count) + [tail_start, T)."""
    if T <= 0:
        return 0, 0, 0
    if mask_mode in ("causal", "tree"):  # a tree's rows jointly see every position
        return 0, 0, T
    s = min(n_sink, T)
    w0 = max(T - q_len - window + 1, 0)
    if w0 <= s:
        return 0, 0, T
    return s, w0, T


def attended_count(mask_mode: str, T: int, q_len: int, n_sink: int, window: int) -> int:
    s, w0, T = attended_span(mask_mode, T, q_len, n_sink, window)
    return s + (T - w0)


def pages_touched(mask_mode: str, T: int, q_len: int, n_sink: int, window: int,
                  block_size: int) -> int:
    s, w0, T = attended_span(mask_mode, T, q_len, n_sink, window)
    if T == 0:
        return 0
    tail = set(range(w0 // block_size, (T - 1) // block_size + 1))
    head = set(range(0, (s - 1) // block_size + 1)) if s > 0 else set()
    return len(tail | head)


def step_bytes(case, seq_lens: Sequence[int]) -> int:
    e = ELEM_BYTES[case.dtype]
    ekv = ELEM_BYTES[kv_dtype(case)]
    total = 0
    for T in seq_lens:
        n = attended_count(case.mask_mode, int(T), case.q_len, case.n_sink, case.window)
        total += 2 * n * case.num_kv_heads * case.head_dim * ekv
        if case.cache_mode == "paged":
            total += 4 * pages_touched(case.mask_mode, int(T), case.q_len, case.n_sink,
                                       case.window, case.block_size)
    qo = case.batch * case.q_len * case.num_q_heads * case.head_dim * e
    scales = 2 * 4 * case.num_kv_heads if kv_dtype(case) == "fp8" else 0  # k_scale, v_scale
    return total + 2 * qo + 4 * case.batch + scales


def attended_pairs(case, seq_lens: Sequence[int]) -> int:
    """(query row, attended position) pairs of a step with the causal or sink/window mask,
    counted row by row (row i of a sequence of T positions sits at T - q_len + i)."""
    n = 0
    for T in seq_lens:
        T = int(T)
        for i in range(case.q_len):
            P = T - case.q_len + i
            if P < 0:
                continue
            if case.mask_mode == "sink_window":
                n += min(case.n_sink, P + 1) + max(0, P + 1 - max(case.n_sink, P - case.window + 1))
            else:
                n += P + 1
    return n * case.num_q_heads


def step_flops(case, seq_lens: Sequence[int]) -> int:
    n = sum(attended_count(case.mask_mode, int(T), case.q_len, case.n_sink, case.window)
            for T in seq_lens)
    return 4 * case.num_q_heads * case.q_len * case.head_dim * n
