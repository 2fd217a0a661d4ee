"""Pins of the oracle's KV append (oracle.append_np) against what the pages fix
independently of its slot formula: a StreamingLLM ring driven by a write cursor
that skips the sinks, pages read back in logical order through the page table,
several rows at once equal to one row at a time, and rows without a slot left
untouched."""
import types

import numpy as np
import pytest
import torch

import oracle


def _pr(cache_mode, capacity, q_len, Hkv=2, D=8, block_size=4):
    return types.SimpleNamespace(cache_mode=cache_mode, capacity=capacity, q_len=q_len,
                                 num_kv_heads=Hkv, head_dim=D, block_size=block_size)


def _rows(batch, q_len, Hkv=2, D=8, seed=0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(batch, q_len, Hkv, D, generator=g),
            torch.randn(batch, q_len, Hkv, D, generator=g))


def test_ring_append_follows_a_cursor_that_skips_the_sinks():
    # StreamingLLM article, "The StreamingLLM solution": the first n_sink tokens stay,
    # the rest of the cache holds the most recent tokens.  A write cursor over the
    # non-sink slots that wraps back to the first non-sink slot gives the same slots.
    C, S, N = 11, 3, 40
    pr = _pr("ring", C, 1)
    kc = torch.zeros(1, C, 2, 8)
    vc = torch.zeros(1, C, 2, 8)
    expect_k = torch.zeros(1, C, 2, 8)
    cursor = S
    kn, vn = _rows(1, N)
    for p in range(N):
        kc, vc = oracle.append_np(pr, kc, vc, kn[:, p:p + 1], vn[:, p:p + 1], None, [p + 1], S)
        if p < S:
            slot = p
        else:
            slot = cursor
            cursor = S if cursor + 1 == C else cursor + 1
        expect_k[0, slot] = kn[0, p]
        assert torch.equal(kc, expect_k), p
    # the ring holds the sinks and the C - S most recent positions
    live = list(range(S)) + list(range(N - (C - S), N))
    assert sorted(torch.unique(kc[0, :, 0, 0]).tolist()) == sorted(kn[0, live, 0, 0].tolist())


@pytest.mark.parametrize("q_len", [1, 3, 5])
def test_paged_append_reads_back_in_logical_order(q_len):
    # nextadmin.net lesson, "PagedAttention": logical page p / 16 of a sequence lives in
    # the physical block its page-table entry names.  Reading the pages back in
    # logical order must show the appended rows at their logical positions.
    bs, pages, batch = 4, 6, 3
    cap = bs * pages
    pr = _pr("paged", cap, q_len, block_size=bs)
    rng = np.random.default_rng(0)
    table = torch.as_tensor(rng.permutation(batch * pages).reshape(batch, pages), dtype=torch.int32)
    kc = torch.zeros(batch * pages, bs, 2, 8)
    vc = torch.zeros_like(kc)
    T = [q_len, 13, cap]
    kn, vn = _rows(batch, q_len)
    kc2, vc2 = oracle.append_np(pr, kc, vc, kn, vn, table, T)
    for b in range(batch):
        logical = kc2[table[b].long()].reshape(cap, 2, 8)  # pages in logical order
        for i in range(q_len):
            assert torch.equal(logical[T[b] - q_len + i], kn[b, i])
        assert int((logical.abs().sum(dim=(1, 2)) > 0).sum()) == q_len
    assert torch.equal(vc2.abs().sum() > 0, torch.tensor(True))


@pytest.mark.parametrize("mode", ["contiguous", "ring"])
def test_several_rows_equal_one_row_at_a_time(mode):
    C, q_len, S = 16, 4, 2
    pr = _pr(mode, C, q_len)
    pr1 = _pr(mode, C, 1)
    T = [4, 9, 16] if mode == "contiguous" else [4, 9, 30]
    kn, vn = _rows(3, q_len, seed=3)
    kc = torch.zeros(3, C, 2, 8)
    vc = torch.zeros_like(kc)
    a_k, a_v = oracle.append_np(pr, kc, vc, kn, vn, None, T, S)
    b_k, b_v = kc, vc
    for i in range(q_len):
        b_k, b_v = oracle.append_np(pr1, b_k, b_v, kn[:, i:i + 1], vn[:, i:i + 1], None,
                                    [t - q_len + i + 1 for t in T], S)
    assert torch.equal(a_k, b_k) and torch.equal(a_v, b_v)


def test_rows_without_a_slot_are_not_written():
    # P < 0 (T < q_len), P >= capacity, and a page entry outside the pool
    pr = _pr("contiguous", 8, 3)
    kn, vn = _rows(2, 3)
    kc = torch.full((2, 8, 2, 8), 7.0)
    k2, _ = oracle.append_np(pr, kc, kc.clone(), kn, vn, None, [1, 10])
    assert torch.equal(k2[0, 0], kn[0, 2]) and torch.equal(k2[0, 1:], kc[0, 1:])
    assert torch.equal(k2[1, :7], kc[1, :7]) and torch.equal(k2[1, 7], kn[1, 0])
    prp = _pr("paged", 8, 2, block_size=4)
    table = torch.tensor([[0, 99]], dtype=torch.int32)
    kc = torch.full((2, 4, 2, 8), 7.0)
    k3, _ = oracle.append_np(prp, kc, kc.clone(), kn[:1, :2], vn[:1, :2], table, [5], 0,
                             num_blocks=2)
    assert torch.equal(k3[0, 3], kn[0, 0])                       # position 3, block 0
    assert torch.equal(k3[:, :3], kc[:, :3]) and torch.equal(k3[1], kc[1])  # position 4 dropped
