"""The boundary's contract on the GPU, through the C ABI.

* A decode captured into a HIP graph and replayed gives the bits of a direct call
  (deterministic mode), replay after replay, with eager calls on the same handle in
  between: the step allocates nothing, synchronises nothing and keeps its buffers at
  fixed addresses (the fixed-buffer, graph-replayed decode step of the dothoosh.com
  Moondream article, "Mechanism one: the ping-pong slot system").
* Two handles with steps in flight at once on two streams (the article's two
  alternating slots) each match the oracle.
* A handle refuses a second stream until it is moved there.
* Debug handles report out-of-range device-resident arguments through kvattn_check.
"""
import pytest
import torch

import oracle
from kv_cache_attention_amd import binding as kb
from kv_cache_attention_amd import workloads
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu

SMALL = workloads.small_variants()
CASES = {"paged_small": SMALL["paged_small"],                 # vector-ALU split-KV
         "spec_verify_small": SMALL["spec_verify_small"],     # matrix-core split-KV
         "prefill_small": workloads.small_prefill_variants()["prefill_small"]}  # prefill


def _prep(case, seed_shift=0):
    inp = workloads.make_inputs(case.replace(seed=case.seed + seed_shift))
    gh.poison_unattended(case, inp)
    ref = oracle.decode(case, inp["q"], inp["k_cache"], inp["v_cache"], inp["block_table"],
                        inp["seq_lens"])
    d = gh.to_device(inp)
    d["k_cache"] = gh.to_head_major(case, d["k_cache"])
    d["v_cache"] = gh.to_head_major(case, d["v_cache"])
    return d, ref


def _decode(h, case, d, out, q=None):
    h.decode(d["q"] if q is None else q, d["k_cache"], d["v_cache"], d["block_table"],
             d["seq_lens"], case.q_len, case.mask_mode, case.n_sink, case.window, out=out)


@pytest.mark.parametrize("name", list(CASES))
def test_decode_replays_from_a_hip_graph(name):
    case = CASES[name]
    print(f"graph case={name}", flush=True)
    d, ref = _prep(case)
    d2, ref2 = _prep(case, seed_shift=100)
    h = kb.KVAttn.for_case(case, layout="head_major", deterministic=True)
    s = torch.cuda.Stream()
    h.set_stream(s)
    out = torch.empty_like(d["q"])
    other = torch.empty_like(d2["q"])
    with torch.cuda.stream(s):
        _decode(h, case, d, out)            # warm-up, eager
    s.synchronize()
    eager = out.clone()
    gh.check(eager, ref, case.dtype, f"{name}/eager")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        _decode(h, case, d, out)
    for r in range(4):
        with torch.cuda.stream(s):
            out.fill_(float("nan"))
            g.replay()
        s.synchronize()
        assert torch.equal(out, eager), f"replay {r} differs from the direct call"
        # an eager step of other inputs on the same handle between replays
        with torch.cuda.stream(s):
            _decode(h, case, d2, other)
        s.synchronize()
        gh.check(other, ref2, case.dtype, f"{name}/eager between replays")
    del g
    h.close()


def test_two_handles_in_flight_on_two_streams():
    case = SMALL["decode_7b_small"]
    print("two handles, two streams", flush=True)
    runs = [_prep(case, seed_shift=k) for k in (0, 1)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    handles = [kb.KVAttn.for_case(case, layout="head_major") for _ in streams]
    outs = [torch.empty_like(r[0]["q"]) for r in runs]
    for h, s in zip(handles, streams):
        h.set_stream(s)
    torch.cuda.synchronize()
    for it in range(3):
        for h, s, (d, _), o in zip(handles, streams, runs, outs):
            with torch.cuda.stream(s):
                o.fill_(float("nan"))
                _decode(h, case, d, o)   # both steps in flight, no wait between them
        torch.cuda.synchronize()
        for k, ((_, ref), o) in enumerate(zip(runs, outs)):
            gh.check(o, ref, case.dtype, f"slot {k}, step {it}")
    for h in handles:
        h.close()


def test_a_handle_serves_one_stream_at_a_time():
    case = SMALL["decode_7b_small"]
    d, ref = _prep(case)
    h = kb.KVAttn.for_case(case, layout="head_major")
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    out = torch.empty_like(d["q"])
    with torch.cuda.stream(s1):
        _decode(h, case, d, out)
    with pytest.raises(ValueError, match="stream"):
        with torch.cuda.stream(s2):
            _decode(h, case, d, out)
    h.set_stream(s2)   # waits for s1's work, then moves the handle
    with torch.cuda.stream(s2):
        _decode(h, case, d, out)
    s2.synchronize()
    gh.check(out, ref, case.dtype, "after set_stream")
    h.close()


def test_debug_check_reports_bad_device_arguments():
    case = SMALL["paged_small"]
    d, ref = _prep(case)
    h = kb.KVAttn.for_case(case, layout="head_major", debug=True)
    out = _run_debug(h, case, d)
    h.check()                                   # every value in range
    gh.check(out, ref, case.dtype, "debug handle, valid inputs")
    bt = d["block_table"].clone()
    bt[1, 3] = case.num_blocks + 7              # a block id outside the pool
    _run_debug(h, case, dict(d, block_table=bt))
    with pytest.raises(kb.KVAttnError, match="block_table") as e:
        h.check()
    assert e.value.code == -5
    h.check()                                   # cleared by the check that reported it
    sl = d["seq_lens"].clone()
    sl[0] = case.capacity + 1                   # longer than the cache holds
    _run_debug(h, case, dict(d, seq_lens=sl))
    with pytest.raises(kb.KVAttnError, match="seq_lens"):
        h.check()
    sl[0] = -4
    kn = torch.zeros(case.batch, 1, case.num_kv_heads, case.head_dim, dtype=d["q"].dtype,
                     device="cuda")
    h.append(kn, kn, d["k_cache"], d["v_cache"], d["block_table"], sl, 1)
    with pytest.raises(kb.KVAttnError, match="seq_lens"):
        h.check()
    h.close()
    plain = kb.KVAttn.for_case(case, layout="head_major")
    with pytest.raises(kb.KVAttnError) as e:    # no validation without the flag
        plain.check()
    assert e.value.code == -1
    plain.close()


def test_debug_check_reports_tree_words_beyond_the_block():
    case = workloads.small_tree_variants()["tree_small"]
    inp = workloads.make_inputs(case)
    d = gh.to_device(inp)
    h = kb.KVAttn.for_case(case, debug=True)
    h.decode_tree(d["q"], d["k_cache"], d["v_cache"], None, d["seq_lens"], case.q_len,
                  d["tree_mask"])
    h.check()
    bad = d["tree_mask"].clone()
    bad[0, 1] |= 1 << case.q_len                # names a position past the new block
    h.decode_tree(d["q"], d["k_cache"], d["v_cache"], None, d["seq_lens"], case.q_len, bad)
    with pytest.raises(kb.KVAttnError, match="tree_mask"):
        h.check()
    h.close()


def _run_debug(h, case, d):
    out = torch.empty_like(d["q"])
    _decode(h, case, d, out)
    torch.cuda.synchronize()
    return out
