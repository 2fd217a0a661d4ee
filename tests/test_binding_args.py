"""The binding checks every tensor against the handle's shape before a pointer reaches
the library, which cannot see sizes (CPU only: the checks are host logic)."""
import pytest
import torch

from kv_cache_attention_amd import binding as kb


def _chk(**kw):
    base = dict(dtype="bf16", kv_dtype=None, num_q_heads=8, num_kv_heads=2, head_dim=128,
                cache_mode="contiguous", capacity=256, block_size=16, num_blocks=0,
                layout="token_major")
    base.update(kw)
    return kb.ArgCheck(**base)


def _t(*shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype)


def _step(c, batch=3, q_len=2, **kw):
    c.step(batch, q_len, on_device=False, **kw)


def test_matching_tensors_pass():
    c = _chk()
    _step(c, q=_t(3, 2, 8, 128), out=_t(3, 2, 8, 128),
          caches=(("k_cache", _t(3, 256, 2, 128)), ("v_cache", _t(4, 256, 2, 128))),
          seq_lens=_t(3, dtype=torch.int32), new_rows=(("k_new", _t(3, 2, 2, 128)),))
    h = _chk(layout="head_major")
    _step(h, caches=(("k_cache", _t(3, 2, 256, 128)),))
    p = _chk(cache_mode="paged", num_blocks=40, capacity=256)
    _step(p, caches=(("k_cache", _t(40, 16, 2, 128)),), block_table=_t(3, 16, dtype=torch.int32))
    ph = _chk(cache_mode="paged", num_blocks=40, capacity=256, layout="head_major")
    _step(ph, caches=(("k_cache", _t(40, 2, 16, 128)),), block_table=_t(5, 16, dtype=torch.int32))
    _step(c, tree_mask=_t(3, 2, dtype=torch.int64))
    f8 = _chk(kv_dtype="fp8", dtype="f16")
    _step(f8, caches=(("k_cache", _t(3, 256, 2, 128, dtype=torch.float8_e4m3fn)),))


@pytest.mark.parametrize("kw, what", [
    (dict(q=lambda: _t(2, 2, 8, 128)), "q"),                  # fewer sequences than the batch
    (dict(q=lambda: _t(3, 1, 8, 128)), "q"),                  # q_len
    (dict(q=lambda: _t(3, 2, 4, 128)), "q"),                  # query heads
    (dict(q=lambda: _t(3, 2, 8, 64)), "q"),                   # head_dim
    (dict(q=lambda: _t(3, 2, 8, 128, dtype=torch.float16)), "q"),
    (dict(out=lambda: _t(3, 2, 8, 128).t() if False else _t(3, 2, 8, 128)[:, :, :, ::2]), "out"),
    (dict(caches=lambda: (("k_cache", _t(2, 256, 2, 128)),)), "k_cache"),
    (dict(caches=lambda: (("v_cache", _t(3, 128, 2, 128)),)), "v_cache"),  # capacity
    (dict(caches=lambda: (("k_cache", _t(3, 2, 256, 128)),)), "k_cache"),  # wrong layout
    (dict(seq_lens=lambda: _t(2, dtype=torch.int32)), "seq_lens"),
    (dict(seq_lens=lambda: _t(3, dtype=torch.int64)), "seq_lens"),
    (dict(new_rows=lambda: (("k_new", _t(3, 2, 8, 128)),)), "k_new"),     # query heads, not KV
    (dict(tree_mask=lambda: _t(3, 1, dtype=torch.int64)), "tree_mask"),
    (dict(block_table=lambda: _t(3, 16, dtype=torch.int32)), "block_table"),  # not paged
])
def test_mismatches_are_rejected(kw, what):
    c = _chk()
    args = {k: v() for k, v in kw.items()}
    with pytest.raises(ValueError, match=what):
        _step(c, **args)


def test_paged_pool_and_table_must_match():
    p = _chk(cache_mode="paged", num_blocks=40, capacity=256)
    with pytest.raises(ValueError, match="k_cache"):   # a different pool size
        _step(p, caches=(("k_cache", _t(41, 16, 2, 128)),), block_table=_t(3, 16, dtype=torch.int32))
    with pytest.raises(ValueError, match="block_table"):
        _step(p, block_table=_t(3, 15, dtype=torch.int32))
    with pytest.raises(ValueError, match="block_table"):
        _step(p, seq_lens=_t(3, dtype=torch.int32))


def test_host_tensors_are_rejected_for_device_calls():
    c = _chk()
    with pytest.raises(ValueError, match="device"):
        c.step(3, 2, q=_t(3, 2, 8, 128))
