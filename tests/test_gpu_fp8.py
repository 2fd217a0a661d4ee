"""GPU parity for 8-bit (OCP E4M3) K/V caches with per-KV-head scales: the HIP path
through the C ABI against the oracle, which decodes the codes from their bit
definition and dequantises in float64.  Reduced workloads in both layouts (never-
attended slots poisoned with the E4M3 NaN code), sharp softmax, forced unit lengths
(many pieces per sequence), and the argument checks of the 8-bit path."""
import pytest
import torch

import oracle
from kv_cache_attention_amd import binding as kb
from kv_cache_attention_amd import workloads
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu

FP8 = workloads.small_fp8_variants()


def _prep(case, scale_q=1.0):
    inp = workloads.make_inputs(case)
    if scale_q != 1.0:
        inp["q"] = (inp["q"].float() * scale_q).to(inp["q"].dtype)
    gh.poison_unattended(case, inp)
    ref = oracle.decode(case, inp["q"], inp["k_cache"], inp["v_cache"], inp["block_table"],
                        inp["seq_lens"], k_scale=inp["k_scale"], v_scale=inp["v_scale"])
    return inp, ref


@pytest.mark.parametrize("name", list(FP8))
@pytest.mark.parametrize("layout", ["token_major", "head_major"])
def test_fp8_small_workloads_match_oracle(name, layout):
    case = FP8[name]
    print(f"case={name} layout={layout}", flush=True)
    inp, ref = _prep(case)
    out = gh.run(case, gh.to_device(inp), layout=layout)
    gh.check(out, ref, case.dtype, f"{name}/{layout}")


@pytest.mark.parametrize("name", list(FP8))
def test_fp8_sharp_softmax_matches_oracle(name):
    case = FP8[name]
    print(f"case={name} sharp", flush=True)
    inp, ref = _prep(case, scale_q=8.0)
    out = gh.run(case, gh.to_device(inp), layout="head_major")
    gh.check(out, ref, case.dtype, f"{name}/sharp")


@pytest.mark.parametrize("name", ["decode_7b_small_fp8", "paged_small_q5_fp8", "spec_verify_small_fp8"])
@pytest.mark.parametrize("split_len", [64, 192])
def test_fp8_unit_length_does_not_change_the_result(name, split_len):
    case = FP8[name]
    print(f"case={name} split_len={split_len}", flush=True)
    inp, ref = _prep(case, scale_q=4.0)
    out = gh.run(case, gh.to_device(inp), split_len=split_len)
    gh.check(out, ref, case.dtype, f"{name}/split{split_len}")


def test_fp8_scales_are_applied_per_kv_head():
    """Doubling one KV head's V scale doubles exactly that head's output rows (the
    deterministic mode keeps the summation order, so the bits scale exactly), and a
    different K scale on another head moves only that head's rows."""
    case = FP8["paged_small_fp8"]
    print(f"case={case.name} per-head scales", flush=True)
    inp = workloads.make_inputs(case)
    d = gh.to_device(inp)
    base = gh.run(case, d, handle=kb.KVAttn.for_case(case, deterministic=True)).float()
    d2 = dict(d, v_scale=d["v_scale"].clone(), k_scale=d["k_scale"].clone())
    d2["v_scale"][1] *= 2.0
    d2["k_scale"][0] *= 1.5
    out = gh.run(case, d2, handle=kb.KVAttn.for_case(case, deterministic=True)).float()
    g = case.group
    assert torch.equal(out[:, :, g:2 * g], 2.0 * base[:, :, g:2 * g])
    ref = oracle.decode(case, inp["q"], inp["k_cache"], inp["v_cache"], inp["block_table"],
                        inp["seq_lens"], k_scale=d2["k_scale"].cpu(), v_scale=d2["v_scale"].cpu())
    gh.check(out, ref, case.dtype, "per-head scales")


def test_fp8_decode_needs_scales_and_16bit_queries():
    case = FP8["decode_7b_small_fp8"]
    d = gh.to_device(workloads.make_inputs(case))
    h = kb.KVAttn.for_case(case)
    with pytest.raises(kb.KVAttnError) as e:   # no scales set
        h.decode(d["q"], d["k_cache"], d["v_cache"], None, d["seq_lens"], case.q_len)
    assert e.value.code == -1
    with pytest.raises(kb.KVAttnError) as e:   # 8-bit caches with float32 queries
        kb.KVAttn.for_case(case.replace(dtype="f32"))
    assert e.value.code == -2
