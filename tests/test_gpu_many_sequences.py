"""GPU: batches of more sequences than the plan keeps lengths of in LDS (1,024): the
work plan, the piece search and the fused lengths reads then go to seq_lens in
global memory.  Short sequences (empty ones included for the vector-ALU case), the
vector-ALU and matrix-core kernels and a paged cache, both layouts, against the
oracle."""
import pytest

import oracle
from kv_cache_attention_amd import workloads
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu

CASES = {
    "many_valu": workloads.DECODE_7B.replace(name="many_valu", batch=1100, num_q_heads=4,
                                             num_kv_heads=2, capacity=96,
                                             seq_len_range=(0, 96), seed=41),
    "many_mfma": workloads.SPEC_VERIFY.replace(name="many_mfma", batch=1100, num_q_heads=16,
                                               num_kv_heads=2, capacity=96, q_len=2,
                                               seq_lens=None, seq_len_range=(2, 96), seed=42),
    "many_paged": workloads.PAGED_100K.replace(name="many_paged", batch=1100, num_q_heads=8,
                                               num_kv_heads=2, capacity=96,
                                               num_blocks=1100 * 6 + 10, seq_lens=None,
                                               seq_len_range=(1, 96), seed=43),
}


@pytest.mark.parametrize("layout", ["token_major", "head_major"])
@pytest.mark.parametrize("name", list(CASES))
def test_more_sequences_than_the_lds_length_copy(name, layout):
    case = CASES[name]
    assert case.batch > 1024
    print(f"case={name} layout={layout}", flush=True)
    inp = workloads.make_inputs(case)
    gh.poison_unattended(case, inp)
    ref = oracle.decode(case, inp["q"], inp["k_cache"], inp["v_cache"], inp["block_table"],
                        inp["seq_lens"])
    out = gh.run(case, gh.to_device(inp), layout=layout)
    gh.check(out, ref, case.dtype, f"{name}/{layout}")
