"""kvattn_decode_noalloc - the decode for callers that cannot allocate device memory,
its scratch in a static device array - against kvattn_decode through the C ABI: two
calls in a row on each kernel family, the second with a smaller input (fewer
sequences, shorter lengths), each bit-identical to kvattn_decode in deterministic
mode and within the acceptance bars against the oracle; steps beyond the array's
size are rejected before anything is enqueued."""
import pytest
import torch

import oracle
from kv_cache_attention_amd import binding as kb
from kv_cache_attention_amd import workloads
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu

SMALL = workloads.small_variants()
CASES = {
    "paged_small": SMALL["paged_small"],              # vector-ALU kernel, paged cache
    "sink_window_small": SMALL["sink_window_small"],  # vector-ALU kernel, ring cache
    "spec_verify_small": SMALL["spec_verify_small"],  # split-KV matrix-core kernel
    "prefill_small": workloads.small_prefill_variants()["prefill_small"],  # prefill kernel
}


def _smaller(case):
    """The same shape with one sequence fewer and shorter lengths (a new draw)."""
    n = case.batch - 1
    lens = case.seq_lens[:n] if case.seq_lens else None
    if lens is not None:
        lens = tuple(max(case.q_len, (t * 2) // 3) if case.cache_mode != "ring" else t // 2 + 1
                     for t in lens)
    return case.replace(batch=n, seq_lens=lens, seed=case.seed + 500)


def _run_both(case, cfg, h, inp):
    """(kvattn_decode output, kvattn_decode_noalloc output) for inputs of `case`,
    whose batch may be below the configuration's max_batch."""
    d = gh.to_device(inp)
    s = torch.cuda.current_stream()
    ref_out = torch.empty_like(d["q"])
    h.set_batch(case.batch)
    h.decode(d["q"], d["k_cache"], d["v_cache"], d["block_table"], d["seq_lens"], case.q_len,
             case.mask_mode, case.n_sink, case.window, out=ref_out)
    out = torch.full_like(d["q"], float("nan"))
    kb.kvattn_decode_noalloc(cfg, case.batch, d["q"], d["k_cache"], d["v_cache"],
                             d["block_table"], d["seq_lens"], case.q_len, kb.MASK[case.mask_mode],
                             case.n_sink, case.window, out, s.cuda_stream)
    torch.cuda.synchronize()
    return ref_out, out


@pytest.mark.parametrize("name", list(CASES))
def test_noalloc_matches_decode_on_two_calls(name):
    big = CASES[name]
    print(f"noalloc case={name}", flush=True)
    h = kb.KVAttn.for_case(big, deterministic=True)
    cfg = h.cfg
    for case in (big, _smaller(big)):
        inp = workloads.make_inputs(case)
        if case.cache_mode == "paged":   # the smaller draw uses the big pool's page table rows
            inp["block_table"] = inp["block_table"][:case.batch].contiguous()
        gh.poison_unattended(case, inp)
        ref = oracle.decode(case, inp["q"], inp["k_cache"], inp["v_cache"], inp["block_table"],
                            inp["seq_lens"])
        if case.batch < big.batch:       # caches sized for the configuration, fewer sequences
            inp = _pad_to_config(big, case, inp)
        want, got = _run_both(case, cfg, h, inp)
        assert torch.equal(got, want), f"{name} batch {case.batch}: differs from kvattn_decode"
        gh.check(got[:case.batch], ref, case.dtype, f"{name} batch {case.batch}")
    h.close()


def _pad_to_config(big, case, inp):
    """Inputs of the smaller case laid into tensors of the configuration's shape (a
    contiguous or ring cache holds max_batch sequences; a paged pool is shared)."""
    out = dict(inp)
    if big.cache_mode != "paged":
        for k in ("k_cache", "v_cache"):
            full = torch.zeros((big.batch,) + tuple(inp[k].shape[1:]), dtype=inp[k].dtype)
            full[:case.batch] = inp[k]
            out[k] = full
    return out


def test_noalloc_rejects_steps_beyond_its_scratch():
    """A 512-row prefill chunk per sequence over 4 sequences needs more partials than
    the 32 MiB array holds: rejected with KVATTN_ERR_CAPACITY before any launch."""
    case = workloads.CONFIGS["chunked_prefill"]
    cfg = kb.make_config(dtype=case.dtype, num_q_heads=case.num_q_heads,
                         num_kv_heads=case.num_kv_heads, head_dim=case.head_dim,
                         max_batch=case.batch, max_q_len=case.q_len, cache_mode=case.cache_mode,
                         capacity=case.capacity)
    t = torch.zeros(64, dtype=torch.bfloat16, device="cuda")
    sl = torch.full((case.batch,), case.capacity, dtype=torch.int32, device="cuda")
    with pytest.raises(kb.KVAttnError, match="32 MiB") as e:
        kb.kvattn_decode_noalloc(cfg, case.batch, t, t, t, None, sl, case.q_len, 0, 0, 0, t,
                                 torch.cuda.current_stream().cuda_stream)
    assert e.value.code == -3
    fp8 = kb.make_config(dtype="bf16", num_q_heads=8, num_kv_heads=2, head_dim=128, max_batch=2,
                         max_q_len=1, cache_mode="contiguous", capacity=256, kv_dtype="fp8")
    with pytest.raises(kb.KVAttnError) as e:
        kb.kvattn_decode_noalloc(fp8, 2, t, t, t, None, sl, 1, 0, 0, 0, t, 0)
    assert e.value.code == -2
