"""GPU parity when the scores keep rising along the positions, so that a row's running
maximum moves again and again in the middle of a piece (the kernels move their softmax
reference only when a score exceeds it by more than 2^8, and take a tile's weights
again when it moves).  Keys are a common direction times a weight that grows with the
position, plus noise; every query row points along that direction, so the score grows
by about 0.1 in log2 units per position.  Three kernels (vector ALU, split-KV matrix
core, prefill) on contiguous caches, against the oracle at the dtype bars."""
import math

import pytest
import torch

import oracle
from kv_cache_attention_amd import binding as kb
from kv_cache_attention_amd import workloads
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu

_SV = workloads.small_variants()
CASES = {
    "growth_valu": (_SV["decode_7b_small"], 0),
    "growth_split_kv": (_SV["spec_verify_small"], 1),
    "growth_prefill": (workloads.small_prefill_variants()["prefill_small"], 2),
}


def _growth_inputs(case, slope_log2=0.1, seed=0):
    inp = workloads.make_inputs(case)
    g = torch.Generator().manual_seed(seed)
    d = case.head_dim
    u = torch.ones(d, dtype=torch.float64) / math.sqrt(d)
    # score(pos) = c(pos) * (q . u) / sqrt(d) with q = u: c = slope * pos * sqrt(d) / log2(e)
    pos = torch.arange(case.capacity, dtype=torch.float64)
    c = slope_log2 * pos * math.sqrt(d) / math.log2(math.e)
    k = c[None, :, None, None] * u + 0.3 * torch.randn(
        case.batch, case.capacity, case.num_kv_heads, d, generator=g, dtype=torch.float64)
    q = u + 0.02 * torch.randn(case.batch, case.q_len, case.num_q_heads, d, generator=g,
                               dtype=torch.float64)
    dt = workloads.DTYPES[case.dtype]
    inp["k_cache"] = k.to(dt)
    inp["q"] = q.to(dt)
    return inp


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("layout", ["token_major", "head_major"])
def test_rising_scores_match_oracle(name, layout):
    case, kernel = CASES[name]
    print(f"growth case={name} layout={layout}", flush=True)
    h = kb.KVAttn.for_case(case, layout=layout)
    assert h.plan(case.q_len, case.mask_mode, case.n_sink, case.window)[2] == kernel
    inp = _growth_inputs(case)
    ref = oracle.decode(case, inp["q"], inp["k_cache"], inp["v_cache"], inp["block_table"],
                        inp["seq_lens"])
    out = gh.run(case, gh.to_device(inp), layout=layout, handle=h)
    gh.check(out, ref, case.dtype, f"{name}/{layout}")


@pytest.mark.parametrize("name", list(CASES))
def test_rising_scores_with_short_units(name):
    # many pieces per segment: every piece starts without a reference and the merge
    # combines partials whose references differ by far more than the slack
    case, _ = CASES[name]
    print(f"growth case={name} split_len=64", flush=True)
    inp = _growth_inputs(case, seed=1)
    ref = oracle.decode(case, inp["q"], inp["k_cache"], inp["v_cache"], inp["block_table"],
                        inp["seq_lens"])
    out = gh.run(case, gh.to_device(inp), layout="head_major", split_len=64)
    gh.check(out, ref, case.dtype, f"{name}/split64")
