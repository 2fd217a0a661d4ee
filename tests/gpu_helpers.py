"""Shared pieces of the GPU tests: poisoning never-attended slots, running the library
through its C ABI, and the acceptance comparison against the oracle."""
import numpy as np
import torch

import oracle
from kv_cache_attention_amd import binding as kb

# max-abs bars per dtype, plus the normalised-error bars that keep near-uniform
# softmax outputs (tiny |out|) from passing vacuously
MAX_ABS = {"f32": 1e-5, "f16": 5e-3, "bf16": 2e-2}
REL_L2 = {"f32": 1e-6, "f16": 2e-3, "bf16": 1e-2}


def attended_union_slots(case, inp):
    """Flat slots any new row of any sequence attends (from the oracle's enumerator)."""
    used = set()
    words = oracle.tree_words(inp["tree_mask"]) if inp.get("tree_mask") is not None else None
    for b in range(case.batch):
        for i in range(case.q_len):
            bits = int(words[b, i]) if words is not None else 0
            _, slots = oracle.attended(case, inp["block_table"], inp["seq_lens"], b, i, bits)
            used.update(slots.tolist())
    return used


def poison_unattended(case, inp):
    """Fill every K/V slot no row attends with NaN (in place; any device)."""
    used = attended_union_slots(case, inp)
    kc, vc = inp["k_cache"], inp["v_cache"]
    n_slots = kc.shape[0] * kc.shape[1]
    mask = torch.ones(n_slots, dtype=torch.bool)
    if used:
        mask[torch.as_tensor(sorted(used), dtype=torch.int64)] = False
    idx = mask.nonzero().view(-1).to(kc.device)
    if idx.numel():
        for c in (kc, vc):
            if c.dtype == torch.float8_e4m3fn:  # E4M3 NaN code S.1111.111
                c.view(torch.uint8).view(n_slots, *c.shape[2:]).index_fill_(0, idx, 0x7F)
            else:
                c.view(n_slots, *c.shape[2:]).index_fill_(0, idx, float("nan"))
    return int(idx.numel())


def to_device(inp, device="cuda"):
    out = {}
    for k, v in inp.items():
        out[k] = v.to(device) if isinstance(v, torch.Tensor) else v
    return out


def to_head_major(case, t):
    if case.cache_mode == "paged":
        return t.permute(0, 2, 1, 3).contiguous()   # [blocks, Hkv, bs, D]
    return t.permute(0, 2, 1, 3).contiguous()       # [B, Hkv, S, D]


def run(case, dinp, layout="token_major", split_len=0, q=None, handle=None):
    """Decode through the C ABI; returns the output tensor (on the device)."""
    h = handle or kb.KVAttn.for_case(case, layout=layout)
    if split_len:
        h.set_split_len(split_len)
    if getattr(case, "kv_dtype", None) == "fp8":
        h.set_kv_scales(dinp["k_scale"], dinp["v_scale"])
    kc, vc = dinp["k_cache"], dinp["v_cache"]
    if layout == "head_major":
        kc, vc = to_head_major(case, kc), to_head_major(case, vc)
    if case.mask_mode == "tree":
        out = h.decode_tree(dinp["q"] if q is None else q, kc, vc, dinp["block_table"],
                            dinp["seq_lens"], case.q_len, dinp["tree_mask"])
    else:
        out = h.decode(dinp["q"] if q is None else q, kc, vc, dinp["block_table"],
                       dinp["seq_lens"], case.q_len, case.mask_mode, case.n_sink, case.window)
    torch.cuda.synchronize()
    return out


def check(got, ref, dtype, what=""):
    """Acceptance: finite, max-abs within the dtype bar, normalised L2 within its bar."""
    g = got.detach().float().cpu().double().numpy() if isinstance(got, torch.Tensor) else got
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    err = np.abs(g - ref)
    max_abs = float(err.max()) if err.size else 0.0
    nrm = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(g - ref) / nrm) if nrm > 0 else float(np.linalg.norm(g))
    assert max_abs <= MAX_ABS[dtype], f"{what}: max-abs {max_abs:.3g} > {MAX_ABS[dtype]}"
    assert rel <= REL_L2[dtype], f"{what}: rel-L2 {rel:.3g} > {REL_L2[dtype]}"
    return max_abs, rel
