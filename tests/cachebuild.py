"""Test helpers: store a logical K/V sequence into each cache form by simulating the
write process itself (copy, page-table block copy, ring with a rolling cursor).
Independent of both the oracle's and the library's slot arithmetic."""
import torch


def store_contiguous(logical, capacity):
    """logical: list over b of [T_b, Hkv, D] -> [B, capacity, Hkv, D] (unused slots NaN)."""
    B = len(logical)
    Hkv, D = logical[0].shape[1:]
    cache = torch.full((B, capacity, Hkv, D), float("nan"), dtype=logical[0].dtype)
    for b, x in enumerate(logical):
        cache[b, : x.shape[0]] = x
    return cache


def store_paged(logical, block_table, num_blocks, block_size):
    """Copy page j of sequence b (tokens [j*bs, (j+1)*bs)) into physical block block_table[b, j]."""
    Hkv, D = logical[0].shape[1:]
    pool = torch.full((num_blocks, block_size, Hkv, D), float("nan"), dtype=logical[0].dtype)
    for b, x in enumerate(logical):
        T = x.shape[0]
        for j in range((T + block_size - 1) // block_size):
            piece = x[j * block_size:(j + 1) * block_size]
            pool[int(block_table[b, j]), : piece.shape[0]] = piece
    return pool


def ring_cursor_contents(T, capacity, n_sink):
    """Write positions 0..T-1 into a ring of `capacity` slots whose first n_sink slots are
    never overwritten; the cursor starts after the sinks and wraps back to n_sink.
    Returns a list: slot -> position held (-1 = never written)."""
    held = [-1] * capacity
    cursor = 0
    for p in range(T):
        held[cursor] = p
        cursor += 1
        if cursor == capacity:
            cursor = n_sink
    return held


def store_ring(logical, capacity, n_sink):
    """logical: list over b of [T_b, Hkv, D]; returns ([B, capacity, Hkv, D], held lists)."""
    B = len(logical)
    Hkv, D = logical[0].shape[1:]
    cache = torch.full((B, capacity, Hkv, D), float("nan"), dtype=logical[0].dtype)
    helds = []
    for b, x in enumerate(logical):
        held = ring_cursor_contents(x.shape[0], capacity, n_sink)
        for s, p in enumerate(held):
            if p >= 0:
                cache[b, s] = x[p]
        helds.append(held)
    return cache, helds
