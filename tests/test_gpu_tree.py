"""GPU parity of token-tree verification (kvattn_decode_tree) through the C ABI: the
reduced tree cases (split-KV matrix-core, vector-ALU and prefill kernels, contiguous and
paged caches, sequences shorter than their tree) against the oracle in both layouts
with never-attended slots poisoned, sharp softmax, a chain tree bit-equal to the causal
decode, the tree gather bit-exact against the oracle's enumerator, the kernel each case
takes, and the argument checks."""
import numpy as np
import pytest
import torch

import oracle
from kv_cache_attention_amd import binding as kb
from kv_cache_attention_amd import workloads
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu

TREES = workloads.small_tree_variants()


def _prep(case, scale_q=1.0):
    inp = workloads.make_inputs(case)
    if scale_q != 1.0:
        inp["q"] = (inp["q"].float() * scale_q).to(inp["q"].dtype)
    gh.poison_unattended(case, inp)
    ref = oracle.decode(case, inp["q"], inp["k_cache"], inp["v_cache"], inp["block_table"],
                        inp["seq_lens"], tree_mask=inp["tree_mask"])
    return inp, ref


@pytest.mark.parametrize("name", list(TREES))
@pytest.mark.parametrize("layout", ["token_major", "head_major"])
def test_tree_small_workloads_match_oracle(name, layout):
    case = TREES[name]
    print(f"tree case={name} layout={layout}", flush=True)
    inp, ref = _prep(case)
    out = gh.run(case, gh.to_device(inp), layout=layout)
    gh.check(out, ref, case.dtype, f"{name}/{layout}")


@pytest.mark.parametrize("name", list(TREES))
def test_tree_sharp_softmax_matches_oracle(name):
    case = TREES[name]
    print(f"tree case={name} sharp", flush=True)
    inp, ref = _prep(case, scale_q=8.0)
    out = gh.run(case, gh.to_device(inp), layout="head_major")
    gh.check(out, ref, case.dtype, f"{name}/sharp")


# kernel codes of kvattn_plan: 0 vector ALU, 1 split-KV matrix core, 2 prefill
KERNELS = {"tree_small": 1, "tree_small_q8": 1, "tree_short": 1, "tree_valu": 0,
           "tree_paged": 1, "tree_wide": 2, "tree_q64": 2, "tree_wide_paged": 2}


@pytest.mark.parametrize("name", list(TREES))
def test_tree_cases_take_the_expected_kernel(name):
    case = TREES[name]
    h = kb.KVAttn.for_case(case)
    assert h.plan(case.q_len, "tree")[2] == KERNELS[name]


@pytest.mark.parametrize("name", ["tree_small", "tree_valu", "tree_paged", "tree_wide",
                                  "tree_wide_paged"])
def test_chain_tree_equals_causal_decode_bit_for_bit(name):
    case = TREES[name]
    print(f"tree case={name} chain", flush=True)
    d = gh.to_device(workloads.make_inputs(case))
    chain = [(1 << (i + 1)) - 1 for i in range(case.q_len)]
    d["tree_mask"] = torch.tensor([chain] * case.batch, dtype=torch.int64, device="cuda")
    h = kb.KVAttn.for_case(case, layout="head_major", deterministic=True)
    tree = gh.run(case, d, layout="head_major", handle=h)
    causal = gh.run(case.replace(mask_mode="causal"), d, layout="head_major", handle=h)
    assert torch.equal(tree.cpu(), causal.cpu())


@pytest.mark.parametrize("name", ["tree_small", "tree_short", "tree_paged"])
def test_tree_gather_is_bit_exact(name):
    case = TREES[name]
    inp = workloads.make_inputs(case)
    d = gh.to_device(inp)
    max_slots = case.capacity + 1
    h = kb.KVAttn.for_case(case)
    slots, counts = h.debug_gather_tree(d["block_table"], d["seq_lens"], case.q_len,
                                        d["tree_mask"], max_slots)
    torch.cuda.synchronize()
    slots, counts = slots.cpu().numpy(), counts.cpu().numpy()
    words = oracle.tree_words(inp["tree_mask"])
    for b in range(case.batch):
        for i in range(case.q_len):
            _, want = oracle.attended(case, inp["block_table"], inp["seq_lens"], b, i,
                                      int(words[b, i]))
            assert counts[b, i] == len(want), (b, i)
            assert np.array_equal(slots[b, i, :len(want)], want), (b, i)


def test_tree_argument_errors():
    case = TREES["tree_small"]
    d = gh.to_device(workloads.make_inputs(case))
    h = kb.KVAttn.for_case(case)
    with pytest.raises(kb.KVAttnError):   # a tree mask only through kvattn_decode_tree
        h.decode(d["q"], d["k_cache"], d["v_cache"], None, d["seq_lens"], case.q_len, "tree")
    ring = workloads.small_variants()["sink_window_small"].replace(q_len=2)
    rd = gh.to_device(workloads.make_inputs(ring))
    hr = kb.KVAttn.for_case(ring)
    words = torch.tensor([[1, 3]] * ring.batch, dtype=torch.int64, device="cuda")
    with pytest.raises(kb.KVAttnError):   # ring caches take the sink/window mask only
        hr.decode_tree(rd["q"], rd["k_cache"], rd["v_cache"], None, rd["seq_lens"], 2, words)
    big = case.replace(q_len=65, num_q_heads=2, num_kv_heads=2)
    hb = kb.KVAttn.for_case(big)
    with pytest.raises(kb.KVAttnError):   # 64 draft tokens at most (one mask word per row)
        hb.plan(65, "tree")
