"""GPU parity of the KV append (kvattn_append, kvattn_append_decode) through the C ABI:
the caches after the append equal the oracle's append byte for byte (every element
type, both layouts, the three cache forms, q_len 1..100, sequences shorter than the
new block, ring wrap-around).  The fused call (one launch whose workgroups write the
new rows they read) leaves the same cache bytes, its output matches the oracle's
decode of the oracle-appended caches, and in deterministic mode equals the two calls
made separately bit for bit, on all three kernel families (vector-ALU, split-KV
matrix-core with one and with several row blocks per KV head, prefill)."""
import pytest
import torch

import oracle
from kv_cache_attention_amd import binding as kb
from kv_cache_attention_amd import workloads
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu

_S = workloads.small_variants()
CASES = {**_S, **workloads.small_fp8_variants(), **workloads.small_prefill_variants()}
# a sequence shorter than its block of new rows (no slot for its first rows)
CASES["spec_verify_short"] = _S["spec_verify_small"].replace(name="spec_verify_short",
                                                             seq_lens=(1000, 3, 5))
# a ring taking several rows per step, around the wrap
CASES["sink_window_q3"] = _S["sink_window_small"].replace(name="sink_window_q3", q_len=3)


def _kv_torch(case):
    return kb.TORCH_DTYPE[case.kv_dtype or case.dtype]


def _new_rows(case, seed=11):
    g = torch.Generator().manual_seed(seed)
    shape = (case.batch, case.q_len, case.num_kv_heads, case.head_dim)
    k = torch.randn(shape, generator=g) * 0.5
    v = torch.randn(shape, generator=g) * 0.5
    if (case.kv_dtype or case.dtype) == "fp8":
        k, v = k * 100, v * 100  # spread over the E4M3 range
    return k.to(_kv_torch(case)), v.to(_kv_torch(case))


def _bytes(t):
    return t.contiguous().view(torch.uint8)


def _from_head_major(case, t):
    return t.permute(0, 2, 1, 3).contiguous()


def _handle(case, layout, deterministic=False):
    h = kb.KVAttn.for_case(case, layout=layout, deterministic=deterministic)
    return h


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("layout", ["token_major", "head_major"])
def test_append_writes_the_oracles_slots(name, layout):
    case = CASES[name]
    print(f"append case={name} layout={layout}", flush=True)
    inp = workloads.make_inputs(case)
    kn, vn = _new_rows(case)
    n_sink = case.n_sink if case.cache_mode == "ring" else 0
    ek, ev = oracle.append_np(case, inp["k_cache"], inp["v_cache"], kn, vn, inp["block_table"],
                              inp["seq_lens"], n_sink, num_blocks=case.num_blocks or None)
    d = gh.to_device(inp)
    kc, vc = d["k_cache"], d["v_cache"]
    if layout == "head_major":
        kc, vc = gh.to_head_major(case, kc), gh.to_head_major(case, vc)
    h = _handle(case, layout)
    h.append(kn.cuda(), vn.cuda(), kc, vc, d["block_table"], d["seq_lens"], case.q_len, n_sink)
    torch.cuda.synchronize()
    if layout == "head_major":
        kc, vc = _from_head_major(case, kc), _from_head_major(case, vc)
    assert torch.equal(_bytes(kc.cpu()), _bytes(ek)), "k_cache"
    assert torch.equal(_bytes(vc.cpu()), _bytes(ev)), "v_cache"


FUSED = ["decode_7b_small", "spec_verify_short", "sink_window_q3", "paged_small",
         "paged_small_q5_fp8", "tiny", "spec_verify_small", "spec_verify_small_fp8",
         "prefill_small", "prefill_paged", "prefill_ring", "prefill_d64"]


@pytest.mark.parametrize("name", FUSED)
def test_append_decode_matches_oracle_and_the_two_calls(name):
    case = CASES[name]
    print(f"append_decode case={name}", flush=True)
    inp = workloads.make_inputs(case)
    kn, vn = _new_rows(case, seed=5)
    n_sink = case.n_sink if case.mask_mode == "sink_window" else 0
    ek, ev = oracle.append_np(case, inp["k_cache"], inp["v_cache"], kn, vn, inp["block_table"],
                              inp["seq_lens"], n_sink)
    ref = oracle.decode(case, inp["q"], ek, ev, inp["block_table"], inp["seq_lens"],
                        k_scale=inp["k_scale"], v_scale=inp["v_scale"])
    outs = []
    for fused in (True, False):
        d = gh.to_device(inp)
        h = _handle(case, "head_major", deterministic=True)
        if (case.kv_dtype or case.dtype) == "fp8":
            h.set_kv_scales(d["k_scale"], d["v_scale"])
        kc, vc = gh.to_head_major(case, d["k_cache"]), gh.to_head_major(case, d["v_cache"])
        if fused:
            out = h.append_decode(d["q"], kn.cuda(), vn.cuda(), kc, vc, d["block_table"],
                                  d["seq_lens"], case.q_len, case.mask_mode, case.n_sink,
                                  case.window)
        else:
            h.append(kn.cuda(), vn.cuda(), kc, vc, d["block_table"], d["seq_lens"], case.q_len,
                     n_sink)
            out = h.decode(d["q"], kc, vc, d["block_table"], d["seq_lens"], case.q_len,
                           case.mask_mode, case.n_sink, case.window)
        torch.cuda.synchronize()
        outs.append(out.cpu())
        kc, vc = _from_head_major(case, kc), _from_head_major(case, vc)
        assert torch.equal(_bytes(kc.cpu()), _bytes(ek)), f"k_cache (fused={fused})"
        assert torch.equal(_bytes(vc.cpu()), _bytes(ev)), f"v_cache (fused={fused})"
    gh.check(outs[0], ref, case.dtype, name)
    assert torch.equal(outs[0], outs[1]), "fused call differs from append then decode"


@pytest.mark.parametrize("name", ["decode_7b_small", "sink_window_q3", "paged_small",
                                  "spec_verify_small", "prefill_small", "prefill_paged"])
def test_fused_append_decode_token_major_shared_queue(name):
    """The default (shared work queue) mode, token-major caches, two steps in a row:
    the second step appends the next rows of the sequences the first one grew."""
    case = CASES[name]
    print(f"append_decode token-major case={name}", flush=True)
    inp = workloads.make_inputs(case)
    n_sink = case.n_sink if case.mask_mode == "sink_window" else 0
    d = gh.to_device(inp)
    kc, vc = d["k_cache"], d["v_cache"]
    ek, ev = inp["k_cache"], inp["v_cache"]
    h = _handle(case, "token_major")
    lens = inp["seq_lens"].clone()
    for step in range(2):
        kn, vn = _new_rows(case, seed=21 + step)
        ek, ev = oracle.append_np(case, ek, ev, kn, vn, inp["block_table"], lens, n_sink)
        ref = oracle.decode(case, inp["q"], ek, ev, inp["block_table"], lens,
                            k_scale=inp["k_scale"], v_scale=inp["v_scale"])
        out = h.append_decode(d["q"], kn.cuda(), vn.cuda(), kc, vc, d["block_table"],
                              lens.cuda(), case.q_len, case.mask_mode, case.n_sink, case.window)
        torch.cuda.synchronize()
        gh.check(out.cpu(), ref, case.dtype, f"{name}/step{step}")
        assert torch.equal(_bytes(kc.cpu()), _bytes(ek)), f"k_cache step {step}"
        assert torch.equal(_bytes(vc.cpu()), _bytes(ev)), f"v_cache step {step}"
        # the next step's lengths (contiguous and paged caches hold at most capacity)
        lens = lens + case.q_len
        if case.cache_mode != "ring":
            lens = torch.clamp(lens, max=case.capacity)


def test_append_skips_page_entries_outside_the_pool():
    case = CASES["paged_small"].replace(name="paged_small_q3", q_len=3)
    inp = workloads.make_inputs(case)
    bt = inp["block_table"].clone()
    # sequence 2 (T = 33): positions 30..32 on pages 1 and 2; page 2 points outside,
    # and so does the page of position 1376 of sequence 1 (T = 1377)
    bt[2, 2] = case.num_blocks + 5
    bt[1, 1376 // 16] = -3
    kn, vn = _new_rows(case, seed=9)
    ek, ev = oracle.append_np(case, inp["k_cache"], inp["v_cache"], kn, vn, bt, inp["seq_lens"],
                              num_blocks=case.num_blocks)
    d = gh.to_device(inp)
    h = _handle(case, "token_major")
    kc, vc = d["k_cache"], d["v_cache"]
    h.append(kn.cuda(), vn.cuda(), kc, vc, bt.cuda(), d["seq_lens"], case.q_len, 0)
    torch.cuda.synchronize()
    assert torch.equal(_bytes(kc.cpu()), _bytes(ek)) and torch.equal(_bytes(vc.cpu()), _bytes(ev))
    # only the rows with a slot changed: 3 + 3 + 2 minus the dropped ones
    changed = (_bytes(kc.cpu()).view(-1, case.num_kv_heads * case.head_dim * 2) !=
               _bytes(inp["k_cache"]).view(-1, case.num_kv_heads * case.head_dim * 2)).any(1)
    assert int(changed.sum()) <= 3 + 2 + 2


def test_append_argument_errors():
    case = CASES["sink_window_small"]
    inp = gh.to_device(workloads.make_inputs(case))
    kn, vn = (t.cuda() for t in _new_rows(case))
    h = _handle(case, "token_major")
    with pytest.raises(kb.KVAttnError):   # ring: n_sink + q_len > capacity
        h.append(kn, vn, inp["k_cache"], inp["v_cache"], None, inp["seq_lens"], 1,
                 case.capacity)
    with pytest.raises(kb.KVAttnError):   # q_len above max_q_len (the C ABI's own check)
        kb.kvattn_append(h.h, kn, vn, inp["k_cache"], inp["v_cache"], None, inp["seq_lens"], 99, 4)
    with pytest.raises(ValueError):       # element type of the new rows
        h.append(kn.float(), vn.float(), inp["k_cache"], inp["v_cache"], None, inp["seq_lens"],
                 1, 4)
    with pytest.raises(kb.KVAttnError):   # the fused call checks the decode's arguments first
        h.append_decode(inp["q"], kn, vn, inp["k_cache"], inp["v_cache"], None, inp["seq_lens"],
                        1, "causal", 0, 0)
