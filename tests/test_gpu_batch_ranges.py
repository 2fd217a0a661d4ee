"""GPU: a decode cut into launches over batch ranges (the per-launch flat range lowered
with KVATTN_MAX_FLAT so that one or two sequences fit a launch) matches the oracle, on
every kernel and cache form, both layouts, the 8-bit caches, the tree mask and the
fused append.  Each range starts the batch-indexed arguments (queries, outputs,
lengths, page-table rows, per-sequence cache regions, tree words, new rows) at its
first sequence and reuses the handle's workspace."""
import pytest
import torch

import oracle
from kv_cache_attention_amd import binding as kb
from kv_cache_attention_amd import workloads
from tests import gpu_helpers as gh
from tests.test_gpu_append import _bytes, _new_rows

pytestmark = pytest.mark.gpu

CASES = {**workloads.small_variants(), **workloads.small_tree_variants(),
         **workloads.small_prefill_variants(), **workloads.small_fp8_variants()}
# row blocks per (sequence, KV head): 256-row blocks of the prefill kernel where a KV
# head has more than 64 rows, one block otherwise
ROW_BLOCKS = {"tree_wide": 2, "tree_q64": 2, "prefill_small": 2, "prefill_paged": 2}
NAMES = ["decode_7b_small", "spec_verify_small", "sink_window_small", "paged_small",
         "tree_small", "tree_paged", "tree_wide", "prefill_small", "prefill_paged",
         "prefill_ring", "spec_verify_small_fp8", "paged_small_q5_fp8", "sink_window_small_fp8"]


def per_seq(case):
    att = case.capacity
    if case.mask_mode == "sink_window":
        att = min(case.n_sink + case.window + case.q_len - 1, case.capacity)
    return case.num_kv_heads * ROW_BLOCKS.get(case.name, 1) * att


def _inputs(case):
    inp = workloads.make_inputs(case)
    gh.poison_unattended(case, inp)
    return inp


def _ref(case, inp, k=None, v=None):
    kw = {}
    if case.mask_mode == "tree":
        kw["tree_mask"] = inp["tree_mask"]
    return oracle.decode(case, inp["q"], inp["k_cache"] if k is None else k,
                         inp["v_cache"] if v is None else v, inp["block_table"],
                         inp["seq_lens"], k_scale=inp.get("k_scale"), v_scale=inp.get("v_scale"),
                         **kw)


@pytest.mark.parametrize("seqs", [1, 2])
@pytest.mark.parametrize("name", NAMES)
@pytest.mark.parametrize("layout", ["token_major", "head_major"])
def test_batch_ranges_match_oracle(name, layout, seqs, monkeypatch):
    case = CASES[name]
    seqs = min(seqs, case.batch - 1)  # at least two launches
    assert seqs >= 1
    monkeypatch.setenv("KVATTN_MAX_FLAT", str(per_seq(case) * seqs))
    print(f"batch ranges case={name} layout={layout} seqs_per_launch={seqs}", flush=True)
    inp = _inputs(case)
    out = gh.run(case, gh.to_device(inp), layout=layout)
    gh.check(out, _ref(case, inp), case.dtype, f"{name}/{layout}/{seqs}")


def test_one_sequence_over_the_limit_is_refused(monkeypatch):
    case = CASES["decode_7b_small"]
    monkeypatch.setenv("KVATTN_MAX_FLAT", str(per_seq(case) - 1))
    d = gh.to_device(_inputs(case))
    with pytest.raises(kb.KVAttnError, match="exceeds 2"):
        gh.run(case, d)


@pytest.mark.parametrize("name", ["decode_7b_small", "paged_small", "prefill_small",
                                  "spec_verify_small_fp8"])
def test_fused_append_over_batch_ranges(name, monkeypatch):
    case = CASES[name]
    monkeypatch.setenv("KVATTN_MAX_FLAT", str(per_seq(case)))
    print(f"batch ranges append_decode case={name}", flush=True)
    inp = workloads.make_inputs(case)
    kn, vn = _new_rows(case, seed=7)
    ek, ev = oracle.append_np(case, inp["k_cache"], inp["v_cache"], kn, vn, inp["block_table"],
                              inp["seq_lens"], 0)
    d = gh.to_device(inp)
    h = kb.KVAttn.for_case(case, layout="token_major")
    if case.kv_dtype == "fp8":
        h.set_kv_scales(d["k_scale"], d["v_scale"])
    kc, vc = d["k_cache"], d["v_cache"]
    out = h.append_decode(d["q"], kn.cuda(), vn.cuda(), kc, vc, d["block_table"], d["seq_lens"],
                          case.q_len, case.mask_mode, case.n_sink, case.window)
    torch.cuda.synchronize()
    assert torch.equal(_bytes(kc.cpu()), _bytes(ek)), "k_cache"
    assert torch.equal(_bytes(vc.cpu()), _bytes(ev)), "v_cache"
    gh.check(out, _ref(case, inp, ek, ev), case.dtype, name)
