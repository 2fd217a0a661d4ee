"""GPU parity at the workloads' full sizes (the five, the 8-bit-cache versions of
three of them, token-tree verification and chunked prefill), in the launch configuration
the benchmark times (automatic plan, head-major caches): sampled output rows against
the oracle computed row by row, plus NaN poison in never-attended slots and the sharp
(q x 8) variant of each."""
import numpy as np
import pytest
import torch

import oracle
from kv_cache_attention_amd import binding as kb
from kv_cache_attention_amd import workloads
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu


def _sample_rows(case, n=40, seed=0):
    rng = np.random.default_rng(seed)
    rows = {(b, case.q_len - 1, h) for b in range(case.batch) for h in (0, case.num_q_heads - 1)}
    rows |= {(b, 0, 0) for b in range(case.batch)}
    n = min(n, case.batch * case.q_len * case.num_q_heads)
    while len(rows) < n:
        rows.add((int(rng.integers(case.batch)), int(rng.integers(case.q_len)),
                  int(rng.integers(case.num_q_heads))))
    return np.array(sorted(rows), dtype=np.int32)


@pytest.mark.parametrize("name", list(workloads.CONFIGS))
@pytest.mark.parametrize("q_scale", [1.0, 8.0])
def test_full_size_sampled_rows(name, q_scale):
    case = workloads.CONFIGS[name]
    print(f"full-size case={name} q_scale={q_scale}", flush=True)
    d = workloads.make_inputs(case, device="cuda")
    if q_scale != 1.0:
        d["q"] = (d["q"].float() * q_scale).to(d["q"].dtype)
    host_meta = {"block_table": d["block_table"].cpu() if d["block_table"] is not None else None,
                 "seq_lens": d["seq_lens"].cpu(), "k_cache": d["k_cache"], "v_cache": d["v_cache"],
                 "tree_mask": d["tree_mask"].cpu() if d["tree_mask"] is not None else None}
    n_poison = gh.poison_unattended(case, host_meta)
    h = kb.KVAttn.for_case(case, layout="head_major")
    out = gh.run(case, d, layout="head_major", handle=h)
    rows = _sample_rows(case)
    ref = oracle.decode_rows(case, d["q"], d["k_cache"], d["v_cache"], host_meta["block_table"],
                             host_meta["seq_lens"], rows, k_scale=d["k_scale"],
                             v_scale=d["v_scale"], tree_mask=host_meta["tree_mask"])
    got = out.float().cpu().numpy()[rows[:, 0], rows[:, 1], rows[:, 2]].astype(np.float64)
    max_abs, rel = gh.check(got, ref, case.dtype, name)
    print(f"{name}: rows={len(rows)} poisoned={n_poison} max_abs={max_abs:.3g} rel={rel:.3g} "
          f"plan={h.plan(case.q_len, case.mask_mode, case.n_sink, case.window)}", flush=True)
    assert torch.isfinite(out.float()).all()
