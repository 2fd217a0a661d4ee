"""GPU parity at the workloads' full sizes (the five, the 8-bit-cache versions of three
of them, token-tree verification and chunked prefill).

Every output row of every workload is compared with the oracle (plain and sharp, q x 8,
queries), in both cache layouts, with NaN in every never-attended slot; the launch
configuration is the benchmark's (automatic plan).  At the same shapes: q = 0 gives
each row the mean of V over exactly its attended positions (closed form, from the
oracle's enumerator), and the kernels' own gather code lists, bit for bit, the slots
the oracle's enumerator lists for every row (the 12,500-block page permutation of the
100K paged workload, the four ring lengths of the StreamingLLM workload).

Inputs are drawn on the host (the same values on every machine) and kept for one
workload at a time: the largest hold gigabytes.
"""
import numpy as np
import pytest
import torch

import oracle
from kv_cache_attention_amd import binding as kb
from kv_cache_attention_amd import workloads
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu

NAMES = list(workloads.CONFIGS)
_HELD = {}


def _inputs(name):
    """(case, host inputs with never-attended slots poisoned, device copies)."""
    if name not in _HELD:
        _HELD.clear()
        torch.cuda.empty_cache()
        case = workloads.CONFIGS[name]
        inp = workloads.make_inputs(case)
        n_poison = gh.poison_unattended(case, inp)
        print(f"{name}: inputs drawn, {n_poison} never-attended slots poisoned", flush=True)
        _HELD[name] = (case, inp, gh.to_device(inp))
    return _HELD[name]


def _oracle(case, inp, q):
    """float64 [batch, q_len, Hq, D], every row.  Hundreds of rows per sequence (a
    prefill chunk) take the matrix form of the definition, the others the C oracle."""
    args = (case, q, inp["k_cache"], inp["v_cache"], inp["block_table"], inp["seq_lens"])
    kw = dict(k_scale=inp["k_scale"], v_scale=inp["v_scale"], tree_mask=inp["tree_mask"])
    if case.q_len > 64:
        return oracle.decode_matmul_np(*args, **kw)
    return oracle.decode(*args, **kw)


def _run(case, d, q, layout):
    h = kb.KVAttn.for_case(case, layout=layout)
    out = gh.run(case, d, layout=layout, q=q, handle=h)
    plan = h.plan(case.q_len, case.mask_mode, case.n_sink, case.window)
    h.close()
    return out, plan


@pytest.mark.parametrize("name", NAMES)
@pytest.mark.parametrize("q_scale", [1.0, 8.0])
def test_full_size_every_row(name, q_scale):
    case, inp, d = _inputs(name)
    print(f"full-size case={name} q_scale={q_scale}", flush=True)
    q = inp["q"] if q_scale == 1.0 else (inp["q"].float() * q_scale).to(inp["q"].dtype)
    ref = _oracle(case, inp, q)
    qd = q.to(d["q"].device)
    for layout in ("head_major", "token_major"):
        out, plan = _run(case, d, qd, layout)
        max_abs, rel = gh.check(out, ref, case.dtype, f"{name}/{layout}/q x {q_scale}")
        print(f"{name} {layout}: rows={ref.shape[0] * ref.shape[1] * ref.shape[2]} "
              f"max_abs={max_abs:.3g} rel={rel:.3g} plan={plan}", flush=True)


def _v_rows(case, inp, slots):
    """V of the listed flat slots as float64 [n, Hkv, D] (8-bit caches dequantised)."""
    vflat = inp["v_cache"].reshape(-1, case.num_kv_heads, case.head_dim)
    v = oracle.to_f64(vflat.index_select(0, torch.as_tensor(slots)))
    if inp["v_scale"] is not None:
        v = v * oracle.to_f64(inp["v_scale"])[None, :, None]
    return v


def _rows_attended(case, inp, b):
    """Flat slots of every new row of sequence b, from the oracle's enumerator."""
    words = oracle.tree_words(inp["tree_mask"]) if inp["tree_mask"] is not None else None
    return [oracle.attended(case, inp["block_table"], inp["seq_lens"], b, i,
                            int(words[b, i]) if words is not None else 0)[1]
            for i in range(case.q_len)]


@pytest.mark.parametrize("name", NAMES)
def test_full_size_q_zero_gives_mean_of_attended_values(name):
    """q = 0: all scores equal, so each row is the arithmetic mean of V over exactly the
    positions it attends (StreamingLLM article, "The softmax problem": equal scores get
    equal weights).  Pins the attended set of every row through the whole numeric path."""
    case, inp, d = _inputs(name)
    print(f"full-size q=0 case={name}", flush=True)
    g = case.group
    ref = np.zeros((case.batch, case.q_len, case.num_q_heads, case.head_dim))
    for b in range(case.batch):
        rows = _rows_attended(case, inp, b)
        # causal rows attend prefixes of the last row's list: one running sum serves all
        causal = case.mask_mode == "causal" and all(
            np.array_equal(sl, rows[-1][:sl.size]) for sl in rows)
        union = rows[-1] if causal else np.unique(np.concatenate(rows))
        if union.size == 0:
            continue
        v = _v_rows(case, inp, union)
        csum = np.cumsum(v, axis=0) if causal else None
        for i, sl in enumerate(rows):
            if sl.size == 0:
                continue
            if causal:
                mean = csum[sl.size - 1] / sl.size
            else:
                mean = v[np.searchsorted(union, sl)].mean(axis=0)
            ref[b, i] = np.repeat(mean, g, axis=0)
    qz = torch.zeros_like(d["q"])
    out, _ = _run(case, d, qz, "head_major")
    gh.check(out, ref, case.dtype, f"{name}/q=0")


@pytest.mark.parametrize("name", NAMES)
def test_full_size_gather_is_bit_exact(name):
    """kvattn_debug_gather (the decode kernels' own span, mask and slot code) lists, for
    every new row of the full-size workload, exactly the flat slots the oracle's
    enumerator lists, in the same order."""
    case, inp, d = _inputs(name)
    print(f"full-size gather case={name}", flush=True)
    rows = [_rows_attended(case, inp, b) for b in range(case.batch)]
    max_slots = max(1, max(len(s) for r in rows for s in r))
    h = kb.KVAttn.for_case(case)
    if case.mask_mode == "tree":
        slots, counts = h.debug_gather_tree(d["block_table"], d["seq_lens"], case.q_len,
                                            d["tree_mask"], max_slots)
    else:
        slots, counts = h.debug_gather(d["block_table"], d["seq_lens"], case.q_len,
                                       case.mask_mode, case.n_sink, case.window, max_slots)
    slots, counts = slots.cpu().numpy(), counts.cpu().numpy()
    h.close()
    for b in range(case.batch):
        for i in range(case.q_len):
            ref = rows[b][i]
            assert counts[b, i] == len(ref), (name, b, i, counts[b, i], len(ref))
            assert np.array_equal(slots[b, i, :len(ref)], ref), (name, b, i)
