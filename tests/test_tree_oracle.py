"""Pins of the oracle's token-tree mask (decode with mask "tree") against facts that do
not come from its own mask code: a chain of draft tokens is plain causal
verification; a token whose only ancestor is the cached prefix attends exactly what a
single-token decode over prefix + that token does; the C oracle agrees with the NumPy
twin and with an explicit softmax over hand-listed positions; a row that sees nothing
gives zeros.  Also the tree words' ancestor property."""
import math

import numpy as np
import pytest
import torch

import oracle
from kv_cache_attention_amd import workloads

TREES = workloads.small_tree_variants()


def _inputs(case):
    return workloads.make_inputs(case)


def test_tree_words_are_ancestor_sets():
    g = torch.Generator().manual_seed(0)
    for q_len in (1, 2, 7, 33, 64):
        parents = workloads.draw_tree(q_len, g)
        words = workloads.tree_words_from_parents(parents)
        for i in range(q_len):
            path, j = set(), i
            while j >= 0:
                path.add(j)
                j = parents[j]
            assert {b for b in range(q_len) if (words[i] >> b) & 1} == path


@pytest.mark.parametrize("name", ["tree_small", "tree_valu", "tree_paged"])
def test_chain_tree_is_causal_verification(name):
    case = TREES[name]
    inp = _inputs(case)
    chain = [(1 << (i + 1)) - 1 for i in range(case.q_len)]  # node i: nodes 0..i
    words = torch.tensor([chain] * case.batch, dtype=torch.int64)
    got = oracle.decode(case, inp["q"], inp["k_cache"], inp["v_cache"], inp["block_table"],
                        inp["seq_lens"], tree_mask=words)
    want = oracle.decode(case.replace(mask_mode="causal"), inp["q"], inp["k_cache"],
                         inp["v_cache"], inp["block_table"], inp["seq_lens"])
    assert np.array_equal(got, want)


def test_star_tree_rows_equal_single_token_decodes():
    # every draft token hangs off the prefix: row i sees the prefix and itself, i.e.
    # a one-token decode over a cache whose last position holds token i
    case = TREES["tree_small"]
    inp = _inputs(case)
    words = torch.tensor([[1 << i for i in range(case.q_len)]] * case.batch, dtype=torch.int64)
    got = oracle.decode(case, inp["q"], inp["k_cache"], inp["v_cache"], None, inp["seq_lens"],
                        tree_mask=words)
    one = case.replace(q_len=1, mask_mode="causal")
    for b in range(case.batch):
        T = int(inp["seq_lens"][b])
        P0 = T - case.q_len
        for i in range(case.q_len):
            if P0 + i < 0:
                continue
            kc, vc = inp["k_cache"].clone(), inp["v_cache"].clone()
            kc[b, P0], vc[b, P0] = kc[b, P0 + i], vc[b, P0 + i]
            sl = inp["seq_lens"].clone()
            sl[b] = P0 + 1
            q1 = inp["q"][:, i:i + 1].contiguous()
            ref = oracle.decode(one, q1, kc, vc, None, sl)
            assert np.array_equal(got[b, i], ref[b, 0]), (b, i)


@pytest.mark.parametrize("name", list(TREES))
def test_c_oracle_equals_numpy_twin(name):
    case = TREES[name]
    inp = _inputs(case)
    c = oracle.decode(case, inp["q"], inp["k_cache"], inp["v_cache"], inp["block_table"],
                      inp["seq_lens"], tree_mask=inp["tree_mask"])
    n = oracle.decode_np(case, inp["q"], inp["k_cache"], inp["v_cache"], inp["block_table"],
                         inp["seq_lens"], tree_mask=inp["tree_mask"])
    assert np.abs(c - n).max() <= 1e-12


def test_explicit_softmax_over_listed_positions():
    case = TREES["tree_small_q8"]
    inp = _inputs(case)
    out = oracle.decode(case, inp["q"], inp["k_cache"], inp["v_cache"], None, inp["seq_lens"],
                        tree_mask=inp["tree_mask"])
    words = oracle.tree_words(inp["tree_mask"])
    b, g = 0, case.num_q_heads // case.num_kv_heads
    T = int(inp["seq_lens"][b])
    P0 = T - case.q_len
    for i in (0, 3, 7):
        for h in (0, 9):
            pos = list(range(P0)) + [P0 + j for j in range(case.q_len) if (int(words[b, i]) >> j) & 1]
            K = inp["k_cache"][b, pos, h // g].double().numpy()
            V = inp["v_cache"][b, pos, h // g].double().numpy()
            s = K @ inp["q"][b, i, h].double().numpy() / math.sqrt(case.head_dim)
            w = np.exp(s - s.max())
            ref = (w / w.sum()) @ V
            assert np.abs(out[b, i, h] - ref).max() <= 1e-12


def test_rows_that_see_nothing_are_zero():
    case = TREES["tree_short"]  # sequence 1 holds 3 positions, its tree 8 tokens
    inp = _inputs(case)
    words = torch.tensor([[1 << i for i in range(case.q_len)]] * case.batch, dtype=torch.int64)
    out = oracle.decode(case, inp["q"], inp["k_cache"], inp["v_cache"], None, inp["seq_lens"],
                        tree_mask=words)
    P0 = 3 - case.q_len
    for i in range(case.q_len):
        if P0 + i < 0:
            assert not out[1, i].any()
        else:
            assert out[1, i].any()
