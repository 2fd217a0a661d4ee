"""Pins of the oracle against what the pages and the mathematics fix (CPU only).

Each test names the passage it follows.  The oracle is pinned to things other
than itself: values the pages print, closed forms, a library routine
(torch's scaled_dot_product_attention in float64), brute-force recomputation of
full causal attention, exhaustive format decoding, and caches built by
simulating the write process.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from kv_cache_attention_amd import accounting, workloads
from tests import cachebuild

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _case(**kw):
    base = dict(name="t", seed=0, batch=1, num_q_heads=4, num_kv_heads=4, head_dim=16,
                dtype="f32", cache_mode="contiguous", capacity=64, q_len=1,
                mask_mode="causal", n_sink=0, window=0, block_size=16, num_blocks=0,
                seq_lens=(64,))
    base.update(kw)
    return workloads.Case(**base)


# --------------------------------------------------------------------------- formats

def test_f16_decode_exhaustive(oracle_lib):
    """The C oracle's binary16 decoder agrees with torch's conversion on all 65,536 codes."""
    codes = torch.arange(65536, dtype=torch.int32).to(torch.int16).contiguous()
    ref = codes.view(torch.float16).to(torch.float64).numpy()
    got = np.array([oracle_lib.oracle_decode_elem(codes.data_ptr(), 1, i) for i in range(65536)])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])


def test_bf16_decode_exhaustive(oracle_lib):
    codes = torch.arange(65536, dtype=torch.int32).to(torch.int16).contiguous()
    ref = codes.view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle_lib.oracle_decode_elem(codes.data_ptr(), 2, i) for i in range(65536)])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])


def test_e4m3_decode_exhaustive(oracle_lib):
    """8-bit caches: the C oracle's E4M3 decoder (written from the format's bit
    definition) agrees with torch's float8_e4m3fn conversion on all 256 codes, and with
    the values that define the OCP E4M3 format: largest finite magnitude 448 (0x7E),
    smallest normal 2^-6 (0x08), smallest subnormal 2^-9 (0x01), 1.0 = 0x38, NaN for
    S.1111.111 and no infinities."""
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).contiguous()
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle_lib.oracle_decode_elem(codes.data_ptr(), 3, i) for i in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
    spot = {0x7E: 448.0, 0xFE: -448.0, 0x08: 2.0 ** -6, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9,
            0x38: 1.0, 0x00: 0.0, 0x3F: 1.875, 0x40: 2.0}
    for c, v in spot.items():
        assert got[c] == v, hex(c)
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF])
    assert np.isfinite(got[[c for c in range(256) if c & 0x7F != 0x7F]]).all()


# --------------------------------------------------------------------------- closed forms

def test_kv_bytes_golden():
    """KV bytes per token = 2 x layers x KV heads x head width x bytes (lesson 'KV cache
    math'; StreamingLLM article 'KV-cache memory bottleneck')."""
    with open(os.path.join(GOLDEN, "kv_bytes.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        got = accounting.kv_bytes_per_token(c["layers"], c["kv_heads"], c["head_dim"],
                                            c["bytes_per_element"]) * c["tokens"]
        if c["rel_tol"] == 0:
            assert got == c["value"], c["what"]
        else:
            assert abs(got - c["value"]) <= c["rel_tol"] * c["value"], c["what"]


def test_four_equal_scores_give_quarter_weights():
    """StreamingLLM article, 'The softmax problem': equal scores -> uniform weights,
    four zeros -> 0.25 each.  q = 0 makes every score 0; V = the 4 unit vectors reads
    the weights out directly."""
    with open(os.path.join(GOLDEN, "page_facts.json")) as f:
        fact = json.load(f)["equal_scores"]
    case = _case(num_q_heads=1, num_kv_heads=1, head_dim=4, capacity=4, seq_lens=(4,))
    q = torch.zeros(1, 1, 1, 4)
    k = torch.randn(1, 4, 1, 4, generator=torch.Generator().manual_seed(3))
    v = torch.eye(4).view(1, 4, 1, 4).contiguous()
    out = oracle.decode(case, q, k, v, None, torch.tensor([4], dtype=torch.int32))
    assert np.allclose(out.reshape(4), fact["weights"], rtol=0, atol=1e-15)
    assert np.allclose(oracle.decode_np(case, q, k, v, None, torch.tensor([4])).reshape(4),
                       fact["weights"], rtol=0, atol=1e-15)


def test_naive_vs_cached_decoder():
    """Lesson, implementation step 3 and exercise 1: the O(N^2) decoder that recomputes
    attention over the whole prefix and the KV-cached O(N) decoder give the same outputs;
    for 100 tokens they make 5050 and 100 row-attention computations."""
    with open(os.path.join(GOLDEN, "page_facts.json")) as f:
        fact = json.load(f)["naive_vs_cached"]
    N, H, D = fact["tokens"], 2, 8
    g = torch.Generator().manual_seed(7)
    Q, K, V = (torch.randn(N, H, D, generator=g, dtype=torch.float64) for _ in range(3))
    scale = 1 / math.sqrt(D)
    naive_rows = 0
    naive_last = []
    for t in range(1, N + 1):        # recompute every row of the prefix, keep the last
        full = oracle.full_causal_np(Q[:t].numpy(), K[:t].numpy(), V[:t].numpy(), scale)
        naive_rows += t
        naive_last.append(full[-1])
    cached_rows = 0
    cache_k = torch.zeros(1, N, H, D, dtype=torch.float32)
    cache_v = torch.zeros(1, N, H, D, dtype=torch.float32)
    case = _case(num_q_heads=H, num_kv_heads=H, head_dim=D, capacity=N, seq_lens=(N,))
    # the oracle reads float32 storage; use float32-representable values
    Q32, K32, V32 = Q.float(), K.float(), V.float()
    cached_last = []
    for t in range(1, N + 1):         # append one K/V row, attend one query row
        cache_k[0, t - 1] = K32[t - 1]
        cache_v[0, t - 1] = V32[t - 1]
        out = oracle.decode(case, Q32[t - 1].view(1, 1, H, D), cache_k, cache_v, None,
                            torch.tensor([t], dtype=torch.int32))
        cached_rows += 1
        cached_last.append(out[0, 0])
    assert naive_rows == fact["naive_attention_rows"]
    assert cached_rows == fact["cached_attention_rows"]
    naive32 = [oracle.full_causal_np(Q32[:t].double().numpy(), K32[:t].double().numpy(),
                                     V32[:t].double().numpy(), scale)[-1] for t in (1, 37, N)]
    for t, ref in zip((1, 37, N), naive32):
        assert np.allclose(cached_last[t - 1], ref, rtol=1e-12, atol=1e-13)
    assert len(naive_last) == N


# --------------------------------------------------------------------------- library routine

def _sdpa_ref(q, k_logical, v_logical, mask, scale):
    """torch SDPA on CPU in float64 with an explicit boolean mask.
    q: [ql, Hq, D]; k/v_logical: [T, Hkv, D]; mask: [ql, T]."""
    Hq, Hkv = q.shape[1], k_logical.shape[1]
    g = Hq // Hkv
    K = k_logical.double().repeat_interleave(g, dim=1).permute(1, 0, 2).contiguous()
    V = v_logical.double().repeat_interleave(g, dim=1).permute(1, 0, 2).contiguous()
    Qh = q.double().permute(1, 0, 2).contiguous()
    out = torch.nn.functional.scaled_dot_product_attention(
        Qh, K, V, attn_mask=torch.as_tensor(mask)[None], scale=scale)
    return out.permute(1, 0, 2).numpy()


def _explicit_mask(mode, T, ql, n_sink, window):
    m = np.zeros((ql, T), bool)
    for i in range(ql):
        P = T - ql + i
        for p in range(T):
            ok = p <= P
            if mode == "sink_window":
                ok = ok and (p < n_sink or p >= P - window + 1)
            m[i, p] = ok
    return m


@pytest.mark.parametrize("mode,ql,hq,hkv,T,n_sink,window", [
    ("causal", 1, 4, 4, 37, 0, 0),
    ("causal", 5, 8, 2, 50, 0, 0),
    ("causal", 3, 6, 3, 3, 0, 0),
    ("sink_window", 1, 4, 4, 60, 4, 10),
    ("sink_window", 4, 4, 2, 60, 2, 7),
    ("sink_window", 2, 2, 1, 9, 4, 20),
])
def test_oracle_matches_sdpa(mode, ql, hq, hkv, T, n_sink, window):
    """Contiguous cache, explicit masks: the oracle equals torch's attention routine."""
    D = 16
    g = torch.Generator().manual_seed(T * 31 + ql)
    case = _case(num_q_heads=hq, num_kv_heads=hkv, head_dim=D, capacity=T, q_len=ql,
                 mask_mode=mode, n_sink=n_sink, window=window, seq_lens=(T,))
    q = torch.randn(1, ql, hq, D, generator=g)
    k = torch.randn(1, T, hkv, D, generator=g)
    v = torch.randn(1, T, hkv, D, generator=g)
    sl = torch.tensor([T], dtype=torch.int32)
    ref = _sdpa_ref(q[0], k[0], v[0], _explicit_mask(mode, T, ql, n_sink, window), 1 / math.sqrt(D))
    got = oracle.decode(case, q, k, v, None, sl)[0]
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)
    got_np = oracle.decode_np(case, q, k, v, None, sl)[0]
    assert np.allclose(got_np, ref, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------- brute force

@pytest.mark.parametrize("T,ql,hq,hkv", [(1, 1, 2, 2), (64, 1, 4, 4), (300, 5, 8, 2), (511, 3, 4, 1)])
def test_new_rows_are_last_rows_of_full_causal(T, ql, hq, hkv):
    """Lesson, problem statement + KV cache: the q_len new rows against the cache equal the
    last q_len rows of full causal attention recomputed from scratch; the verify rows
    see every earlier position (speculative-decoding article, verify phase)."""
    D = 32
    g = torch.Generator().manual_seed(T + 100 * ql)
    Qall = torch.randn(T, hq, D, generator=g)
    K = torch.randn(T, hkv, D, generator=g)
    V = torch.randn(T, hkv, D, generator=g)
    rep = hq // hkv
    full = oracle.full_causal_np(Qall.double().numpy(),
                                 K.double().repeat_interleave(rep, 1).numpy(),
                                 V.double().repeat_interleave(rep, 1).numpy(), 1 / math.sqrt(D))
    case = _case(num_q_heads=hq, num_kv_heads=hkv, head_dim=D, capacity=T, q_len=ql,
                 seq_lens=(T,))
    q = Qall[T - ql:].unsqueeze(0).contiguous()
    got = oracle.decode(case, q, K.unsqueeze(0).contiguous(), V.unsqueeze(0).contiguous(), None,
                        torch.tensor([T], dtype=torch.int32))[0]
    assert np.allclose(got, full[T - ql:], rtol=1e-11, atol=1e-12)


# --------------------------------------------------------------------------- invariants

@pytest.mark.parametrize("T", [1, 5, 129, 1000])
def test_tiled_and_split_forms_equal_oracle(T):
    """Lesson, 'Flash Attention - the tiling trick' and implementation step 2: the running
    (max, sum) form over tiles is exact; a split into pieces merged with log-sum-exp weights
    is the same identity across splits."""
    D = 64
    g = torch.Generator().manual_seed(T)
    case = _case(num_q_heads=1, num_kv_heads=1, head_dim=D, capacity=T, seq_lens=(T,))
    q = torch.randn(1, 1, 1, D, generator=g) * 2
    k = torch.randn(1, T, 1, D, generator=g)
    v = torch.randn(1, T, 1, D, generator=g)
    ref = oracle.decode(case, q, k, v, None, torch.tensor([T], dtype=torch.int32))[0, 0, 0]
    qv, K, V = q.double().view(D).numpy(), k.double().view(T, D).numpy(), v.double().view(T, D).numpy()
    sc = 1 / math.sqrt(D)
    scale_ref = np.abs(ref).max()
    for tile in (1, 3, 4, 16, 128, T):
        got = oracle.tiled_softmax_dot_np(qv, K, V, tile, sc)
        assert np.abs(got - ref).max() <= 1e-13 * max(scale_ref, 1.0)
    for n_split in (1, 2, 7, 64):
        got = oracle.split_merge_np(qv, K, V, n_split, sc)
        assert np.abs(got - ref).max() <= 1e-13 * max(scale_ref, 1.0)


def test_page_permutation_is_bit_identical():
    """Lesson, 'PagedAttention': the page table is pure address indirection.  Two different
    physical placements of the same logical sequence give bit-identical oracle output."""
    T, bs, D, H = 150, 16, 32, 2
    nb = 40
    g = torch.Generator().manual_seed(11)
    logical_k = [torch.randn(T, H, D, generator=g)]
    logical_v = [torch.randn(T, H, D, generator=g)]
    q = torch.randn(1, 1, H, D, generator=g)
    case = _case(num_q_heads=H, num_kv_heads=H, head_dim=D, cache_mode="paged", capacity=160,
                 block_size=bs, num_blocks=nb, seq_lens=(T,))
    outs = []
    for seed in (1, 2, 3):
        bt = torch.randperm(nb, generator=torch.Generator().manual_seed(seed))[:10].view(1, 10).int()
        kc = cachebuild.store_paged(logical_k, bt, nb, bs)
        vc = cachebuild.store_paged(logical_v, bt, nb, bs)
        outs.append(oracle.decode(case, q, kc, vc, bt, torch.tensor([T], dtype=torch.int32)))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
    # and equal to the same sequence stored contiguously
    cont = _case(num_q_heads=H, num_kv_heads=H, head_dim=D, capacity=T, seq_lens=(T,))
    ref = oracle.decode(cont, q, logical_k[0].unsqueeze(0), logical_v[0].unsqueeze(0), None,
                        torch.tensor([T], dtype=torch.int32))
    assert np.array_equal(outs[0], ref)


def test_gqa_equals_mha_with_repeated_heads():
    """Lesson, 'KV cache math': under GQA several query heads share one K/V head.  The GQA
    result equals MHA with each K/V head repeated for its group."""
    T, D, hq, hkv, ql = 77, 16, 12, 3, 2
    g = torch.Generator().manual_seed(5)
    q = torch.randn(1, ql, hq, D, generator=g)
    k = torch.randn(1, T, hkv, D, generator=g)
    v = torch.randn(1, T, hkv, D, generator=g)
    sl = torch.tensor([T], dtype=torch.int32)
    gqa = oracle.decode(_case(num_q_heads=hq, num_kv_heads=hkv, head_dim=D, capacity=T, q_len=ql,
                              seq_lens=(T,)), q, k, v, None, sl)
    rep = hq // hkv
    mha = oracle.decode(_case(num_q_heads=hq, num_kv_heads=hq, head_dim=D, capacity=T, q_len=ql,
                              seq_lens=(T,)), q, k.repeat_interleave(rep, 2).contiguous(),
                        v.repeat_interleave(rep, 2).contiguous(), None, sl)
    assert np.array_equal(gqa, mha)


def test_sink_window_special_cases():
    """StreamingLLM article, 'Why sliding windows fail' / 'The StreamingLLM solution':
    n_sink = 0 with a window covering everything is plain causal attention; T within
    n_sink + window attends everything; n_sink = 0 is the plain sliding window (last
    `window` positions)."""
    D, H, T = 16, 2, 90
    g = torch.Generator().manual_seed(9)
    q = torch.randn(1, 1, H, D, generator=g)
    k = torch.randn(1, T, H, D, generator=g)
    v = torch.randn(1, T, H, D, generator=g)
    sl = torch.tensor([T], dtype=torch.int32)
    causal = oracle.decode(_case(num_q_heads=H, num_kv_heads=H, head_dim=D, capacity=T,
                                 seq_lens=(T,)), q, k, v, None, sl)
    wide = oracle.decode(_case(num_q_heads=H, num_kv_heads=H, head_dim=D, capacity=T,
                               mask_mode="sink_window", n_sink=0, window=T, seq_lens=(T,)),
                         q, k, v, None, sl)
    assert np.array_equal(causal, wide)
    both = oracle.decode(_case(num_q_heads=H, num_kv_heads=H, head_dim=D, capacity=T,
                               mask_mode="sink_window", n_sink=10, window=80, seq_lens=(T,)),
                         q, k, v, None, sl)
    assert np.array_equal(causal, both)
    W = 25
    slide = oracle.decode(_case(num_q_heads=H, num_kv_heads=H, head_dim=D, capacity=T,
                                mask_mode="sink_window", n_sink=0, window=W, seq_lens=(T,)),
                          q, k, v, None, sl)
    last = oracle.decode(_case(num_q_heads=H, num_kv_heads=H, head_dim=D, capacity=W,
                               seq_lens=(W,)), q, k[:, T - W:].contiguous(),
                         v[:, T - W:].contiguous(), None, torch.tensor([W], dtype=torch.int32))
    assert np.allclose(slide, last, rtol=0, atol=1e-15)


def test_single_dominant_key():
    """StreamingLLM article, 'Rethinking attention': one position can take most of the
    weight.  With k_p* = c q and c large, the output tends to v_p* - pinning one gather
    index through the whole numeric path, in every cache form."""
    D, H, T, bs, cap = 16, 1, 100, 16, 112
    g = torch.Generator().manual_seed(21)
    q = torch.randn(1, 1, H, D, generator=g)
    q = q / q.norm()
    k = torch.randn(T, H, D, generator=g) * 0.01
    v = torch.randn(T, H, D, generator=g)
    pstar = 42
    k[pstar, 0] = 200.0 * q[0, 0, 0]
    bt = torch.randperm(7, generator=g)[:7].view(1, 7).int()
    sl = torch.tensor([T], dtype=torch.int32)
    forms = [
        (_case(num_q_heads=H, num_kv_heads=H, head_dim=D, capacity=cap, seq_lens=(T,)),
         cachebuild.store_contiguous([k], cap), cachebuild.store_contiguous([v], cap), None),
        (_case(num_q_heads=H, num_kv_heads=H, head_dim=D, cache_mode="paged", capacity=cap,
               block_size=bs, num_blocks=7, seq_lens=(T,)),
         cachebuild.store_paged([k], bt, 7, bs), cachebuild.store_paged([v], bt, 7, bs), bt),
    ]
    for case, kc, vc, table in forms:
        out = oracle.decode(case, q, kc, vc, table, sl)[0, 0, 0]
        assert np.allclose(out, v[pstar, 0].double().numpy(), atol=1e-12)


# --------------------------------------------------------------------------- gather pins

@pytest.mark.parametrize("T", [1, 3, 4, 5, 40, 44, 45, 63, 64, 65, 200, 1013])
def test_ring_slots_match_cursor_simulation(T):
    """StreamingLLM article, 'The StreamingLLM solution': first tokens kept, a rolling window
    of recent ones.  Every position the oracle attends sits, in a ring written by a rolling
    cursor that skips the sink slots, exactly where the oracle reads it."""
    cap, n_sink, window = 64, 4, 40
    held = cachebuild.ring_cursor_contents(T, cap, n_sink)
    case = _case(cache_mode="ring", capacity=cap, mask_mode="sink_window", n_sink=n_sink,
                 window=window, seq_lens=(T,))
    pos, slots = oracle.attended(case, None, torch.tensor([T], dtype=torch.int32), 0, 0)
    expect = [p for p in range(T) if p < n_sink or p >= T - window]
    assert list(pos) == expect
    for p, s in zip(pos, slots):
        assert held[s] == p
    assert len(set(slots.tolist())) == len(slots)


def test_streaming_budget_at_full_size():
    """StreamingLLM article: 4 sinks + 4,092 recent = 4,096 kept.  For the ring workload's
    lengths (no wrap, wrap straddling, deep wrap) every row attends exactly 4,096 positions,
    each in its own live slot, with the sinks in the first slots."""
    with open(os.path.join(GOLDEN, "page_facts.json")) as f:
        fact = json.load(f)["streaming_budget"]
    case = workloads.SINK_WINDOW
    assert (case.n_sink, case.window) == (fact["n_sink"], fact["window"])
    for b, T in enumerate(case.seq_lens):
        sl = torch.tensor(case.seq_lens, dtype=torch.int32)
        pos, slots = oracle.attended(case, None, sl, b, 0)
        assert len(pos) == fact["kept"]
        assert list(pos[:4]) == [0, 1, 2, 3]
        assert list(slots[:4] - b * case.capacity) == [0, 1, 2, 3]
        assert np.array_equal(pos[4:], np.arange(T - fact["window"], T))
        assert len(np.unique(slots)) == len(slots)
        assert ((slots - b * case.capacity) < case.capacity).all()
        # ring written by the cursor: the last write of each attended slot is its position
        local = slots - b * case.capacity
        R = case.capacity - case.n_sink
        # the cursor writes position p >= n_sink at n_sink + (p - n_sink) mod R; the last
        # position written at a slot s is the largest p < T with that slot
        for p, s in zip(pos[4:][::511], local[4:][::511]):
            last_p = p + ((T - 1 - p) // R) * R
            assert last_p == p


def test_paged_gather_matches_block_copy():
    """Lesson, 'PagedAttention': page j of a sequence lives in physical block
    block_table[b][j].  The oracle reads the logical sequence back from a pool filled by
    copying whole pages."""
    case = workloads.small_variants()["paged_small"]
    inp = workloads.make_inputs(case)
    bt, sl = inp["block_table"], inp["seq_lens"]
    for b in range(case.batch):
        T = int(sl[b])
        logical = torch.randn(T, 1, 1, generator=torch.Generator().manual_seed(b))
        pool = cachebuild.store_paged([logical], bt[b:b + 1], case.num_blocks, case.block_size)
        # a pool indexed through row b of the table: use a one-row problem
        one = case.replace(batch=1, seq_lens=(T,))
        pos, slots = oracle.attended(one, bt[b:b + 1], torch.tensor([T], dtype=torch.int32), 0, 0)
        assert np.array_equal(pos, np.arange(T))
        assert torch.equal(pool.view(-1)[torch.as_tensor(slots)], logical.view(-1))


def test_q_zero_gives_mean_of_attended_values():
    """StreamingLLM article, 'The softmax problem': equal scores give uniform weights, so with
    q = 0 each row returns the mean of V over exactly the positions it attends.  The caches
    are filled by simulated writes and the attended sets come from the mask definition, so
    this pins the oracle's gather and mask."""
    D, H = 8, 2
    g = torch.Generator().manual_seed(4)
    for mode, cache_mode, ql, n_sink, window, T, cap in [
        ("causal", "contiguous", 1, 0, 0, 70, 80),
        ("causal", "contiguous", 4, 0, 0, 70, 80),
        ("causal", "paged", 3, 0, 0, 70, 80),
        ("sink_window", "ring", 1, 4, 30, 500, 64),
        ("sink_window", "ring", 3, 2, 20, 333, 40),
        ("sink_window", "contiguous", 2, 3, 9, 70, 80),
    ]:
        logical_v = torch.randn(T, H, D, generator=g)
        logical_k = torch.randn(T, H, D, generator=g)
        bt = None
        if cache_mode == "contiguous":
            kc = cachebuild.store_contiguous([logical_k], cap)
            vc = cachebuild.store_contiguous([logical_v], cap)
        elif cache_mode == "paged":
            bt = torch.randperm(cap // 16 + 3, generator=g)[:cap // 16].view(1, -1).int()
            kc = cachebuild.store_paged([logical_k], bt, cap // 16 + 3, 16)
            vc = cachebuild.store_paged([logical_v], bt, cap // 16 + 3, 16)
        else:
            kc, _ = cachebuild.store_ring([logical_k], cap, n_sink)
            vc, _ = cachebuild.store_ring([logical_v], cap, n_sink)
        case = _case(num_q_heads=H, num_kv_heads=H, head_dim=D, cache_mode=cache_mode,
                     capacity=cap, q_len=ql, mask_mode=mode, n_sink=n_sink, window=window,
                     num_blocks=cap // 16 + 3, seq_lens=(T,))
        q = torch.zeros(1, ql, H, D)
        out = oracle.decode(case, q, kc, vc, bt, torch.tensor([T], dtype=torch.int32))[0]
        mask = _explicit_mask(mode, T, ql, n_sink, window)
        for i in range(ql):
            expect = logical_v[torch.as_tensor(mask[i])].double().mean(0).numpy()
            assert np.allclose(out[i], expect, rtol=0, atol=1e-14), (mode, cache_mode, i)


# --------------------------------------------------------------------------- twins, accounting

@pytest.mark.parametrize("name", list(workloads.small_variants()))
def test_c_oracle_equals_numpy_twin(name):
    """The two independent implementations agree on every small workload (incl. NaN-free
    results where never-attended slots are poisoned)."""
    case = workloads.small_variants()[name]
    inp = workloads.make_inputs(case)
    args = (case, inp["q"], inp["k_cache"], inp["v_cache"], inp["block_table"], inp["seq_lens"])
    a = oracle.decode(*args)
    b = oracle.decode_np(*args)
    assert np.isfinite(a).all()
    assert np.allclose(a, b, rtol=1e-12, atol=1e-13)


def _all_small_cases():
    cases = dict(workloads.small_variants())
    for more in (workloads.small_prefill_variants(), workloads.small_tree_variants(),
                 workloads.small_fp8_variants()):
        cases.update(more)
    return cases


@pytest.mark.parametrize("name", list(_all_small_cases()))
def test_matrix_form_equals_c_oracle(name):
    """The matrix form of the definition (whole blocks of query rows against a
    sequence's attended positions with library float64 products, explicit mask) and the
    C oracle (row by row, position by position) agree on every reduced case: causal,
    sink/window, token-tree masks, all three cache forms, 8-bit caches, prefill chunks."""
    case = _all_small_cases()[name]
    inp = workloads.make_inputs(case)
    args = (case, inp["q"], inp["k_cache"], inp["v_cache"], inp["block_table"], inp["seq_lens"])
    kw = dict(k_scale=inp["k_scale"], v_scale=inp["v_scale"], tree_mask=inp["tree_mask"])
    a = oracle.decode(*args, **kw)
    b = oracle.decode_matmul_np(*args, **kw)
    assert np.isfinite(b).all()
    assert np.allclose(a, b, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("name", list(workloads.small_fp8_variants()))
def test_fp8_cache_c_oracle_equals_dequantized_twin(name):
    """8-bit caches: the C oracle (bit-definition decoder, dequantise, attend) and the
    NumPy twin (torch's E4M3 conversion times the per-head scales) agree."""
    case = workloads.small_fp8_variants()[name]
    inp = workloads.make_inputs(case)
    args = (case, inp["q"], inp["k_cache"], inp["v_cache"], inp["block_table"], inp["seq_lens"])
    kw = dict(k_scale=inp["k_scale"], v_scale=inp["v_scale"])
    a = oracle.decode(*args, **kw)
    b = oracle.decode_np(*args, **kw)
    assert np.isfinite(a).all()
    assert np.allclose(a, b, rtol=1e-12, atol=1e-13)


def test_fp8_scales_enter_k_and_v_where_the_definition_puts_them():
    """k = code * k_scale and v = code * v_scale, per KV head: doubling one head's
    k_scale while halving its query rows leaves the output unchanged; multiplying its
    v_scale by 4 multiplies exactly that head's output rows by 4; the other heads do
    not move."""
    case = workloads.small_fp8_variants()["paged_small_fp8"]
    inp = workloads.make_inputs(case)
    ks, vs = inp["k_scale"].clone(), inp["v_scale"].clone()
    base = oracle.decode(case, inp["q"], inp["k_cache"], inp["v_cache"], inp["block_table"],
                         inp["seq_lens"], k_scale=ks, v_scale=vs)
    g = case.group
    q2 = inp["q"].clone()
    q2[:, :, 0:g] *= 0.5                          # query heads of KV head 0
    ks2 = ks.clone()
    ks2[0] *= 2.0
    a = oracle.decode(case, q2, inp["k_cache"], inp["v_cache"], inp["block_table"],
                      inp["seq_lens"], k_scale=ks2, v_scale=vs)
    assert np.allclose(a, base, rtol=1e-12, atol=1e-14)
    vs3 = vs.clone()
    vs3[1] *= 4.0  # a power of two: exact in float32
    b = oracle.decode(case, inp["q"], inp["k_cache"], inp["v_cache"], inp["block_table"],
                      inp["seq_lens"], k_scale=ks, v_scale=vs3)
    assert np.allclose(b[:, :, g:2 * g], 4.0 * base[:, :, g:2 * g], rtol=1e-12, atol=1e-14)
    assert np.array_equal(b[:, :, 0:g], base[:, :, 0:g])


@pytest.mark.parametrize("name", list(workloads.CONFIGS))
def test_step_bytes_count_oracle_attended_union(name):
    """Bench accounting: the attended positions per sequence equal the union over rows of
    what the oracle attends."""
    case = workloads.CONFIGS[name]
    if case.seq_lens is None:
        sl = workloads.make_inputs(case.replace(batch=1, seq_len_range=(1024, 1024), num_q_heads=1,
                                                num_kv_heads=1, head_dim=1, capacity=1024))["seq_lens"]
        lens = [int(sl[0]), 1024, 4096, 1]
    else:
        lens = list(case.seq_lens)
    for T in lens[:2]:
        one = case.replace(batch=1, seq_lens=(T,), seq_len_range=None)
        bt = None
        if case.cache_mode == "paged":
            bt = torch.arange(case.blocks_per_seq, dtype=torch.int32).view(1, -1)
        words = [0] * case.q_len
        if case.mask_mode == "tree":  # any tree: every node sees itself
            words = workloads.tree_words_from_parents(
                workloads.draw_tree(case.q_len, torch.Generator().manual_seed(T)))
        union = set()
        for i in range(case.q_len):
            pos, _ = oracle.attended(one, bt, torch.tensor([T], dtype=torch.int32), 0, i,
                                     words[i])
            union.update(pos.tolist())
        assert accounting.attended_count(case.mask_mode, T, case.q_len, case.n_sink,
                                         case.window) == len(union)
        if case.cache_mode == "paged":
            pages = {p // case.block_size for p in union}
            assert accounting.pages_touched(case.mask_mode, T, case.q_len, case.n_sink,
                                            case.window, case.block_size) == len(pages)


def test_oracle_rejects_invalid_problems():
    g = torch.Generator().manual_seed(0)
    q = torch.randn(1, 1, 2, 8, generator=g)
    k = torch.randn(1, 16, 2, 8, generator=g)
    # ring with a causal mask cannot reach evicted positions
    with pytest.raises(ValueError):
        oracle.decode(_case(num_q_heads=2, num_kv_heads=2, head_dim=8, cache_mode="ring",
                            capacity=16, seq_lens=(40,)), q, k, k, None,
                      torch.tensor([40], dtype=torch.int32))
    # contiguous length beyond capacity
    with pytest.raises(ValueError):
        oracle.decode(_case(num_q_heads=2, num_kv_heads=2, head_dim=8, capacity=16,
                            seq_lens=(17,)), q, k, k, None, torch.tensor([17], dtype=torch.int32))


def test_oracle_sharp_scores_match_sdpa():
    """Scores far beyond exp's range (hundreds to thousands) still give the library
    routine's result: the softmax is taken relative to the row maximum."""
    D, H, T = 16, 2, 37
    g = torch.Generator().manual_seed(77)
    q = torch.randn(1, 1, H, D, generator=g) * 1000.0
    k = torch.randn(1, T, H, D, generator=g)
    v = torch.randn(1, T, H, D, generator=g)
    case = _case(num_q_heads=H, num_kv_heads=H, head_dim=D, capacity=T, seq_lens=(T,))
    ref = _sdpa_ref(q[0], k[0], v[0], _explicit_mask("causal", T, 1, 0, 0), 1 / math.sqrt(D))
    got = oracle.decode(case, q, k, v, None, torch.tensor([T], dtype=torch.int32))[0]
    assert np.isfinite(got).all()
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("name", ["spec_verify_small", "sink_window_small", "paged_small"])
def test_attended_pairs_count_the_oracles_rows(name):
    """Bench accounting for matrix-core-bound steps: (row, position) pairs row by row."""
    case = workloads.small_variants()[name].replace(q_len=7)
    inp = workloads.make_inputs(case.replace(num_q_heads=case.num_kv_heads, head_dim=8))
    n = 0
    for b in range(case.batch):
        for i in range(case.q_len):
            pos, _ = oracle.attended(case, inp["block_table"], inp["seq_lens"], b, i)
            n += len(pos)
    assert accounting.attended_pairs(case, inp["seq_lens"].tolist()) == n * case.num_q_heads
