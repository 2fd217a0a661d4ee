"""GPU parity: the HIP path through the C ABI against the oracle, element by element.

Reduced-size versions of every workload (several tiles per split, ragged tails),
never-attended slots poisoned with NaN, both cache layouts, forced split counts,
sharp (far from uniform) softmax variants, the q = 0 closed form, page-table
permutations, and the degenerate lengths.
"""
import numpy as np
import pytest
import torch

import oracle
from kv_cache_attention_amd import binding as kb
from kv_cache_attention_amd import workloads
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu

SMALL = workloads.small_variants()


def _prep(case, scale_q=1.0):
    inp = workloads.make_inputs(case)
    if scale_q != 1.0:
        inp["q"] = (inp["q"].float() * scale_q).to(inp["q"].dtype)
    gh.poison_unattended(case, inp)
    ref = oracle.decode(case, inp["q"], inp["k_cache"], inp["v_cache"], inp["block_table"],
                        inp["seq_lens"])
    return inp, ref


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("layout", ["token_major", "head_major"])
def test_small_workloads_match_oracle(name, layout):
    case = SMALL[name]
    print(f"case={name} layout={layout}", flush=True)
    inp, ref = _prep(case)
    out = gh.run(case, gh.to_device(inp), layout=layout)
    gh.check(out, ref, case.dtype, f"{name}/{layout}")


@pytest.mark.parametrize("name", list(SMALL))
def test_sharp_softmax_matches_oracle(name):
    """q x 8: weights far from uniform, so a dropped split or a wrong rescale shows."""
    case = SMALL[name]
    print(f"case={name} sharp", flush=True)
    inp, ref = _prep(case, scale_q=8.0)
    out = gh.run(case, gh.to_device(inp))
    gh.check(out, ref, case.dtype, f"{name}/sharp")


@pytest.mark.parametrize("name", ["decode_7b_small", "spec_verify_small", "sink_window_small",
                                  "paged_small"])
@pytest.mark.parametrize("split_len", [64, 128, 192, 512])
def test_split_count_does_not_change_the_result(name, split_len):
    case = SMALL[name]
    print(f"case={name} split_len={split_len}", flush=True)
    inp, ref = _prep(case, scale_q=4.0)
    out = gh.run(case, gh.to_device(inp), split_len=split_len)
    gh.check(out, ref, case.dtype, f"{name}/split{split_len}")


@pytest.mark.parametrize("name", list(SMALL))
def test_q_zero_gives_mean_of_attended_values(name):
    """Equal scores -> uniform weights: each row is the mean of V over its attended set."""
    case = SMALL[name]
    print(f"case={name} q=0", flush=True)
    inp = workloads.make_inputs(case)
    gh.poison_unattended(case, inp)
    inp["q"].zero_()
    vflat = inp["v_cache"].reshape(-1, case.num_kv_heads, case.head_dim).double()
    ref = np.zeros((case.batch, case.q_len, case.num_q_heads, case.head_dim))
    for b in range(case.batch):
        for i in range(case.q_len):
            _, slots = oracle.attended(case, inp["block_table"], inp["seq_lens"], b, i)
            if len(slots) == 0:
                continue
            mean = vflat[torch.as_tensor(slots)].mean(0).numpy()  # [Hkv, D]
            ref[b, i] = np.repeat(mean, case.group, axis=0)
    out = gh.run(case, gh.to_device(inp))
    gh.check(out, ref, case.dtype, f"{name}/q0")


@pytest.mark.parametrize("q_len", [1, 5, 80])
def test_out_of_pool_page_entries_are_skipped(q_len):
    """Page-table entries outside [0, num_blocks) are skipped (their positions are
    dropped, nothing outside the pool is read).  With q = 0 every row is the mean of V
    over the attended positions whose pages are valid.  q_len 1 runs the vector-ALU
    kernel, q_len 5 (20 rows per KV head) the split-KV matrix-core one, q_len 80 (320
    rows) the prefill kernel; the bad pages sit mid-sequence, at a sequence start and
    in a short sequence."""
    case = SMALL["paged_small"].replace(q_len=q_len)
    print(f"case=paged_small q_len={q_len} out-of-pool entries", flush=True)
    inp = workloads.make_inputs(case)
    gh.poison_unattended(case, inp)
    inp["q"].zero_()
    bad = {(0, 3): -1, (0, 40): case.num_blocks + 3, (1, 0): -7, (1, 50): case.num_blocks,
           (2, 1): 1 << 30}
    bt_bad = inp["block_table"].clone()
    for (b, page), v in bad.items():
        bt_bad[b, page] = v
    vflat = inp["v_cache"].reshape(-1, case.num_kv_heads, case.head_dim).double()
    ref = np.zeros((case.batch, case.q_len, case.num_q_heads, case.head_dim))
    for b in range(case.batch):
        for i in range(case.q_len):
            pos, slots = oracle.attended(case, inp["block_table"], inp["seq_lens"], b, i)
            keep = [s for p_, s in zip(pos, slots) if (b, int(p_) // case.block_size) not in bad]
            if keep:
                mean = vflat[torch.as_tensor(keep)].mean(0).numpy()
                ref[b, i] = np.repeat(mean, case.group, axis=0)
    d = dict(gh.to_device(inp), block_table=bt_bad.cuda())
    out = gh.run(case, d)
    gh.check(out, ref, case.dtype, f"paged_small/q_len{q_len}/out-of-pool")


def test_page_permutation_is_bit_identical():
    """The same logical sequences under two different page tables give the same bits."""
    case = SMALL["paged_small"]
    inp = workloads.make_inputs(case)
    bt1 = inp["block_table"]
    perm = torch.randperm(case.num_blocks, generator=torch.Generator().manual_seed(99))
    # move every physical block p to perm[p]; the table follows it
    bt2 = perm[bt1.long()].int()
    k2 = torch.empty_like(inp["k_cache"])
    v2 = torch.empty_like(inp["v_cache"])
    k2[perm] = inp["k_cache"]
    v2[perm] = inp["v_cache"]
    d1 = gh.to_device(inp)
    d2 = dict(d1, block_table=bt2.cuda(), k_cache=k2.cuda(), v_cache=v2.cuda())
    o1 = gh.run(case, d1, handle=kb.KVAttn.for_case(case, deterministic=True))
    o2 = gh.run(case, d2, handle=kb.KVAttn.for_case(case, deterministic=True))
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    # the default (shared tile queue) mode agrees to rounding
    o3 = gh.run(case, d2)
    gh.check(o3, o1.double().cpu().numpy(), case.dtype, "paged_small/queue-vs-fixed")


@pytest.mark.parametrize("name", ["decode_7b_small", "sink_window_small", "paged_small"])
def test_deterministic_mode_repeats_bit_for_bit(name):
    """With KVATTN_FLAG_DETERMINISTIC, repeated decodes of the same inputs (several tiles
    per wave, several pieces per sequence) give identical bits."""
    case = SMALL[name]
    print(f"case={name} deterministic", flush=True)
    d = gh.to_device(workloads.make_inputs(case))
    h = kb.KVAttn.for_case(case, deterministic=True)
    h.set_split_len(64)
    outs = [gh.run(case, d, handle=h) for _ in range(4)]
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))


@pytest.mark.parametrize("name", ["sink_window_small", "paged_small", "decode_7b_small",
                                  "spec_verify_small"])
def test_gather_indices_are_bit_exact(name):
    """kvattn_debug_gather (the kernels' own gather code) lists exactly the oracle's slots."""
    case = SMALL[name]
    inp = workloads.make_inputs(case)
    d = gh.to_device(inp)
    h = kb.KVAttn.for_case(case)
    max_slots = case.capacity
    slots, counts = h.debug_gather(d["block_table"], d["seq_lens"], case.q_len, case.mask_mode,
                                   case.n_sink, case.window, max_slots)
    slots, counts = slots.cpu().numpy(), counts.cpu().numpy()
    for b in range(case.batch):
        for i in range(case.q_len):
            _, ref = oracle.attended(case, inp["block_table"], inp["seq_lens"], b, i)
            assert counts[b, i] == len(ref), (b, i)
            assert np.array_equal(slots[b, i, :len(ref)], ref), (b, i)


@pytest.mark.parametrize("T", [1, 3, 4, 5, 300, 303, 304, 305, 700, 701, 1003, 5000])
@pytest.mark.parametrize("q_len", [1, 5])
def test_ring_gather_edges(T, q_len):
    """Ring edge lengths: T in {1, n_sink, n_sink+1, n_sink+window(+ql-1), S, S+1, wraps}."""
    case = SINK = SMALL["sink_window_small"].replace(batch=1, seq_lens=(T,), q_len=q_len,
                                                     num_q_heads=4, num_kv_heads=4)
    sl = torch.tensor([T], dtype=torch.int32)
    h = kb.KVAttn.for_case(SINK)
    slots, counts = h.debug_gather(None, sl.cuda(), q_len, case.mask_mode, case.n_sink,
                                   case.window, case.capacity)
    slots, counts = slots.cpu().numpy(), counts.cpu().numpy()
    for i in range(q_len):
        _, ref = oracle.attended(case, None, sl, 0, i)
        assert counts[0, i] == len(ref)
        assert np.array_equal(slots[0, i, :len(ref)], ref)


def test_degenerate_lengths():
    """T = 0 gives zero rows; T < q_len gives zero rows for the rows with no position;
    T = 1 returns V of the one position."""
    case = workloads.Case("deg", seed=31, batch=4, num_q_heads=8, num_kv_heads=2, head_dim=128,
                          dtype="f16", cache_mode="contiguous", capacity=256, q_len=3,
                          seq_lens=(0, 1, 2, 256), value_scale=0.5)
    inp, ref = _prep(case)
    out = gh.run(case, gh.to_device(inp))
    gh.check(out, ref, case.dtype, "degenerate")
    o = out.float().cpu()
    assert torch.all(o[0] == 0)
    assert torch.all(o[1, :2] == 0) and torch.all(o[2, :1] == 0)


def test_batch_zero_and_subset_batches():
    case = SMALL["decode_7b_small"]
    inp, ref = _prep(case)
    d = gh.to_device(inp)
    h = kb.KVAttn.for_case(case)
    out = torch.full_like(d["q"], 7.0)
    h.set_batch(0)
    h.decode(d["q"], d["k_cache"], d["v_cache"], None, d["seq_lens"], 1, out=out)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
    h.set_batch(2)
    h.decode(d["q"], d["k_cache"], d["v_cache"], None, d["seq_lens"], 1, out=out)
    torch.cuda.synchronize()
    gh.check(out[:2], ref[:2], case.dtype, "batch2")
    assert torch.all(out[2:] == 7.0)


def test_lengths_beyond_capacity_are_clamped():
    """A device-side length past the cache's end is clamped, never read past the buffer."""
    case = SMALL["decode_7b_small"].replace(seq_len_range=None, seq_lens=(1200,) * 5)
    inp, ref = _prep(case)
    d = gh.to_device(inp)
    d["seq_lens"] = torch.full((5,), 1_000_000, dtype=torch.int32, device="cuda")
    out = gh.run(case, d)
    gh.check(out, ref, case.dtype, "clamped")


def test_host_side_errors_with_a_device():
    case = SMALL["sink_window_small"]
    inp = gh.to_device(workloads.make_inputs(case))
    h = kb.KVAttn.for_case(case)
    with pytest.raises(kb.KVAttnError) as e:   # window too large for the ring
        h.decode(inp["q"], inp["k_cache"], inp["v_cache"], None, inp["seq_lens"], 1,
                 "sink_window", 4, case.capacity)
    assert e.value.code == -1
    with pytest.raises(kb.KVAttnError) as e:   # ring needs the sink/window mask
        h.decode(inp["q"], inp["k_cache"], inp["v_cache"], None, inp["seq_lens"], 1, "causal")
    assert e.value.code == -1
    with pytest.raises(kb.KVAttnError) as e:   # q_len beyond the handle (the C ABI's own check)
        kb.kvattn_decode(h.h, inp["q"], inp["k_cache"], inp["v_cache"], None, inp["seq_lens"], 2,
                         kb.MASK["sink_window"], 4, 300, torch.empty_like(inp["q"]))
    assert e.value.code == -3
    with pytest.raises(kb.KVAttnError) as e:
        h.set_batch(case.batch + 1)
    assert e.value.code == -3


@pytest.mark.parametrize("name", ["decode_7b_small", "spec_verify_small", "paged_small",
                                  "sink_window_small"])
def test_repeated_calls_reuse_the_workspace(name):
    """Back-to-back calls on one handle with different inputs and split plans: the
    fused merge's arrival counters return to zero after every call and no call sees
    another's partials."""
    case = SMALL[name]
    h = kb.KVAttn.for_case(case)
    for it, split_len in enumerate([64, 0, 128, 64, 192]):
        inp = workloads.make_inputs(case.replace(seed=case.seed + 100 * it))
        gh.poison_unattended(case, inp)
        ref = oracle.decode(case, inp["q"], inp["k_cache"], inp["v_cache"], inp["block_table"],
                            inp["seq_lens"])
        h.set_split_len(split_len)
        out = gh.run(case, gh.to_device(inp), handle=h)
        gh.check(out, ref, case.dtype, f"{name}/call{it}/split{split_len}")
