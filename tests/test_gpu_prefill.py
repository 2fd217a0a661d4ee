"""GPU parity of chunked prefill (q_len in the hundreds: the prefill kernel's 256-row
blocks for 16-bit caches of every form, 64-row blocks of the split-KV matrix-core kernel
for 8-bit ones) through the C ABI against the oracle: reduced cases in both layouts with
never-attended slots poisoned (contiguous, ring with the sink/window mask, paged, a
sequence shorter than its chunk, head_dim 64), sharp softmax, forced unit lengths
(blocks cut into many pieces), the first rows of a chunk equal to a decode of the
shorter prefix, and chunks of the largest q_len (1024) on each kernel, with sequences
shorter than their chunk."""
import pytest
import torch

import oracle
from kv_cache_attention_amd import binding as kb
from kv_cache_attention_amd import workloads
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu

PREFILL = workloads.small_prefill_variants()

# q_len 1024 (the most a handle accepts): 4,096 rows per KV head on the prefill kernel
# (16 blocks; contiguous and paged) and on the split-KV kernel (8-bit paged cache, 64
# blocks), 1,024 on the vector-ALU kernel (f32); one sequence in each is shorter than
# its chunk.
_SV = workloads.small_variants()
MAX_Q = {
    "prefill_max": (workloads.CHUNKED_PREFILL.replace(
        name="prefill_max", batch=2, num_q_heads=8, num_kv_heads=2, capacity=1536,
        q_len=1024, seq_lens=(1536, 1000), seed=45), 2),
    "prefill_max_paged": (_SV["paged_small"].replace(
        name="prefill_max_paged", q_len=1024, seq_lens=(1600, 1377, 33), seed=46), 2),
    "prefill_max_paged_fp8": (_SV["paged_small"].replace(
        name="prefill_max_paged_fp8", kv_dtype="fp8", q_len=1024, seq_lens=(1600, 1377, 33),
        seed=48), 1),
    "prefill_max_f32": (_SV["decode_7b_small"].replace(
        name="prefill_max_f32", dtype="f32", batch=2, capacity=1200, seq_len_range=None,
        seq_lens=(1200, 1100), q_len=1024, seed=47), 0),
}


def _prep(case, scale_q=1.0):
    inp = workloads.make_inputs(case)
    if scale_q != 1.0:
        inp["q"] = (inp["q"].float() * scale_q).to(inp["q"].dtype)
    gh.poison_unattended(case, inp)
    ref = oracle.decode(case, inp["q"], inp["k_cache"], inp["v_cache"], inp["block_table"],
                        inp["seq_lens"], k_scale=inp["k_scale"], v_scale=inp["v_scale"])
    return inp, ref


@pytest.mark.parametrize("name", list(PREFILL))
@pytest.mark.parametrize("layout", ["token_major", "head_major"])
def test_prefill_small_workloads_match_oracle(name, layout):
    case = PREFILL[name]
    print(f"prefill case={name} layout={layout}", flush=True)
    h = kb.KVAttn.for_case(case, layout=layout)
    kernel = h.plan(case.q_len, case.mask_mode, case.n_sink, case.window)[2]
    assert kernel == 2, "prefill kernel"
    inp, ref = _prep(case)
    out = gh.run(case, gh.to_device(inp), layout=layout, handle=h)
    gh.check(out, ref, case.dtype, f"{name}/{layout}")


@pytest.mark.parametrize("name", list(PREFILL))
def test_prefill_sharp_softmax_matches_oracle(name):
    case = PREFILL[name]
    print(f"prefill case={name} sharp", flush=True)
    inp, ref = _prep(case, scale_q=8.0)
    out = gh.run(case, gh.to_device(inp), layout="head_major")
    gh.check(out, ref, case.dtype, f"{name}/sharp")


@pytest.mark.parametrize("split_len", [64, 320])
def test_prefill_unit_length_does_not_change_the_result(split_len):
    case = PREFILL["prefill_small"]
    print(f"prefill split_len={split_len}", flush=True)
    inp, ref = _prep(case, scale_q=4.0)
    out = gh.run(case, gh.to_device(inp), layout="head_major", split_len=split_len)
    gh.check(out, ref, case.dtype, f"split{split_len}")


def test_first_chunk_rows_equal_a_decode_of_the_prefix():
    # the first 20 rows of a 100-row chunk see the same positions as a 20-row verify
    # of a cache holding 80 fewer positions (bit-equal in deterministic mode)
    case = PREFILL["prefill_small"].replace(seq_lens=(700, 300))
    d = gh.to_device(workloads.make_inputs(case))
    h = kb.KVAttn.for_case(case, layout="head_major", deterministic=True)
    full = gh.run(case, d, layout="head_major", handle=h)
    short = case.replace(q_len=20)
    ds = dict(d)
    ds["q"] = d["q"][:, :20].contiguous()
    ds["seq_lens"] = d["seq_lens"] - 80
    hs = kb.KVAttn.for_case(short, layout="head_major", deterministic=True)
    part = gh.run(short, ds, layout="head_major", handle=hs)
    ref = oracle.decode(short, ds["q"].cpu(), d["k_cache"].cpu(), d["v_cache"].cpu(), None,
                        ds["seq_lens"].cpu())
    gh.check(part, ref, case.dtype, "prefix verify")
    gh.check(full[:, :20], ref, case.dtype, "chunk head")


@pytest.mark.parametrize("name", list(MAX_Q))
@pytest.mark.parametrize("layout", ["token_major", "head_major"])
def test_largest_chunk_matches_oracle(name, layout):
    case, kernel = MAX_Q[name]
    print(f"prefill case={name} layout={layout}", flush=True)
    h = kb.KVAttn.for_case(case, layout=layout)
    assert h.plan(case.q_len)[2] == kernel
    inp, ref = _prep(case)
    out = gh.run(case, gh.to_device(inp), layout=layout, handle=h)
    gh.check(out, ref, case.dtype, f"{name}/{layout}")
