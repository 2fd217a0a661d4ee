"""Seeded synthetic inputs for one decode step of attention over a KV cache.

This module only draws numbers and lays them out; it holds none of the
attention arithmetic, no slot mapping and no masking.  Both the oracle side
(tests) and the library side (tests, bench) take their inputs from here.

Workload shapes follow the decode settings the source pages discuss:
  * a 7B-style model with 32 query / 32 KV heads of width 128 in fp16
    ("KV cache math" section of the nextadmin.net lesson on the KV cache and
    Flash Attention, and the "KV-cache memory bottleneck" section of the
    dothoosh.com StreamingLLM article);
  * speculative verification of 1 accepted + 4 draft tokens against a GQA
    model (dothoosh.com speculative-decoding article, "parallel verification"
    and "verify phase");
  * a StreamingLLM cache of 4 sink tokens plus a 4,092-token window (StreamingLLM
    article, "The StreamingLLM solution");
  * a 100,000-token context paged in 16-token blocks through a page table
    (lesson, "PagedAttention - the KV cache as virtual memory").

Draw order (fixed, so a seed names one input set): integer structure first
(sequence lengths, block permutation, token trees) from torch's CPU generator
seeded with the case's seed; then Q, K, V as float32 standard normals; then the
value scale (and the optional boost of K at position 0); then the cast to the
storage dtype.  The normals of tensor n (0 = Q, 1 = K, 2 = V) are drawn in
chunks of 2^22 consecutive elements, chunk c from its own CPU generator seeded
with (seed << 16) | (n << 14) | c (a 32-bit seed: torch's CPU generator keeps
only the low 32 bits), so the values are the same on every machine and a
gigabyte cache is drawn by several host threads at once.  An 8-bit KV cache (kv_dtype "fp8", OCP
E4M3) casts K and V per KV head: scale = max |x| / 448 over that head's slots
(the largest finite E4M3 magnitude), code = round-to-nearest-even(x / scale);
the scales (float32 [Hkv]) travel with the inputs as k_scale, v_scale.

Layouts (row-major, head_dim innermost):
  q, out            [batch, q_len, num_q_heads, head_dim]
  contiguous / ring [batch, capacity, num_kv_heads, head_dim]
  paged             [num_blocks, block_size, num_kv_heads, head_dim]
  block_table       int32 [batch, capacity // block_size]
  seq_lens          int32 [batch]
"""
from __future__ import annotations

import concurrent.futures as cf
import dataclasses
import os
from dataclasses import dataclass
from typing import Optional, Tuple

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16,
          "fp8": torch.float8_e4m3fn}
E4M3_MAX = 448.0


@dataclass(frozen=True)
class Case:
    name: str
    seed: int
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str                      # "f32" | "f16" | "bf16"
    cache_mode: str                 # "contiguous" | "paged" | "ring"
    capacity: int                   # slots per sequence (paged: blocks_per_seq * block_size)
    q_len: int = 1
    mask_mode: str = "causal"       # "causal" | "sink_window" | "tree"
    n_sink: int = 0
    window: int = 0
    block_size: int = 16
    num_blocks: int = 0             # paged pool size
    seq_lens: Optional[Tuple[int, ...]] = None      # fixed lengths, or
    seq_len_range: Optional[Tuple[int, int]] = None  # inclusive uniform integer range
    value_scale: float = 1.0
    k0_boost: float = 1.0           # K at logical position 0 multiplied by this
    kv_dtype: Optional[str] = None  # cache element type when it differs from dtype ("fp8")

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def rows(self) -> int:
        return self.q_len * self.group

    @property
    def blocks_per_seq(self) -> int:
        return self.capacity // self.block_size

    def replace(self, **kw) -> "Case":
        return dataclasses.replace(self, **kw)


# The five workloads of the decode-attention path, at full size.
TINY = Case("tiny", seed=1, batch=1, num_q_heads=4, num_kv_heads=4, head_dim=64,
            dtype="f32", cache_mode="contiguous", capacity=256, seq_lens=(256,),
            value_scale=1.0)
DECODE_7B = Case("decode_7b", seed=2, batch=16, num_q_heads=32, num_kv_heads=32,
                 head_dim=128, dtype="f16", cache_mode="contiguous", capacity=4096,
                 seq_len_range=(1024, 4096), value_scale=0.5)
SPEC_VERIFY = Case("spec_verify", seed=3, batch=8, num_q_heads=64, num_kv_heads=8,
                   head_dim=128, dtype="bf16", cache_mode="contiguous", capacity=8192,
                   q_len=5, seq_lens=(8192,) * 8, value_scale=0.5)
SINK_WINDOW = Case("sink_window", seed=4, batch=4, num_q_heads=32, num_kv_heads=32,
                   head_dim=128, dtype="f16", cache_mode="ring", capacity=32768,
                   mask_mode="sink_window", n_sink=4, window=4092,
                   seq_lens=(32768, 36000, 100000, 1000000), value_scale=0.5,
                   k0_boost=4.0)
PAGED_100K = Case("paged_100k", seed=5, batch=2, num_q_heads=32, num_kv_heads=8,
                  head_dim=128, dtype="bf16", cache_mode="paged", capacity=100000,
                  block_size=16, num_blocks=12500, seq_lens=(100000, 100000),
                  value_scale=0.5)

# The same shapes with an 8-bit (E4M3) K/V cache and per-KV-head scales.
DECODE_7B_FP8 = DECODE_7B.replace(name="decode_7b_fp8", seed=6, kv_dtype="fp8")
SINK_WINDOW_FP8 = SINK_WINDOW.replace(name="sink_window_fp8", seed=7, kv_dtype="fp8")
PAGED_100K_FP8 = PAGED_100K.replace(name="paged_100k_fp8", seed=8, kv_dtype="fp8")
# speculative verification (40 rows per KV head: the matrix-core path) with an 8-bit cache
SPEC_VERIFY_FP8 = SPEC_VERIFY.replace(name="spec_verify_fp8", seed=11, kv_dtype="fp8")

# Token-tree verification: the verify step with 8 draft tokens per sequence arranged
# as a seeded random tree (8 x GQA 8 = 64 rows per KV head).
TREE_VERIFY = SPEC_VERIFY.replace(name="tree_verify", seed=9, q_len=8, mask_mode="tree")

# Chunked prefill: a chunk of 512 new tokens per sequence against a 7,680-token cached
# prefix (GQA 4: 2,048 rows per KV head, eight 256-row blocks of the prefill kernel).
CHUNKED_PREFILL = Case("chunked_prefill", seed=10, batch=4, num_q_heads=32, num_kv_heads=8,
                       head_dim=128, dtype="bf16", cache_mode="contiguous", capacity=8192,
                       q_len=512, seq_lens=(8192,) * 4, value_scale=0.5)

# The same chunk over a paged cache (16-token pages, the pool shuffled over the batch).
CHUNKED_PREFILL_PAGED = CHUNKED_PREFILL.replace(name="chunked_prefill_paged", seed=12,
                                                cache_mode="paged", block_size=16,
                                                num_blocks=2048)

CONFIGS = {c.name: c for c in (TINY, DECODE_7B, SPEC_VERIFY, SINK_WINDOW, PAGED_100K,
                               DECODE_7B_FP8, SINK_WINDOW_FP8, PAGED_100K_FP8, SPEC_VERIFY_FP8,
                               TREE_VERIFY, CHUNKED_PREFILL, CHUNKED_PREFILL_PAGED)}


def tree_words_from_parents(parents) -> list:
    """Mask words of a token tree given each node's parent (-1: a child of the last
    cached token; parents precede their children): bit j of node i's word is set iff
    node j is node i or one of its ancestors."""
    words = []
    for i, par in enumerate(parents):
        assert par < i
        words.append((words[par] if par >= 0 else 0) | (1 << i))
    return words


def draw_tree(q_len: int, g: torch.Generator) -> list:
    """A seeded random tree of q_len draft tokens: node 0 hangs off the cached prefix,
    node j > 0 off a node drawn uniformly from 0 .. j - 1; returns the parents."""
    return [-1] + [int(torch.randint(0, j, (1,), generator=g)) for j in range(1, q_len)]


def cache_shape(case: Case) -> Tuple[int, ...]:
    if case.cache_mode == "paged":
        return (case.num_blocks, case.block_size, case.num_kv_heads, case.head_dim)
    return (case.batch, case.capacity, case.num_kv_heads, case.head_dim)


CHUNK = 1 << 22  # elements per generator stream


def _chunk_seed(seed: int, tensor: int, chunk: int) -> int:
    assert 0 <= seed < (1 << 16) and 0 <= tensor < 4 and 0 <= chunk < (1 << 14)
    return (seed << 16) | (tensor << 14) | chunk


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _normals(shape, seed: int, tensor: int, pool) -> torch.Tensor:
    """float32 standard normals of `shape`: chunk c of the flat tensor from the CPU
    generator seeded with _chunk_seed(seed, tensor, c)."""
    n = int(np.prod(shape))
    x = torch.empty(n, dtype=torch.float32)

    def fill(c):
        g = torch.Generator("cpu").manual_seed(_chunk_seed(seed, tensor, c))
        x[c * CHUNK:min(n, (c + 1) * CHUNK)].normal_(generator=g)

    list(pool.map(fill, range((n + CHUNK - 1) // CHUNK)))
    return x.view(shape)


def _cast(x: torch.Tensor, dt: torch.dtype, pool) -> torch.Tensor:
    """x.to(dt), chunk by chunk on the worker threads (round to nearest even)."""
    if dt == torch.float32:
        return x
    flat = x.reshape(-1)
    out = torch.empty(flat.shape, dtype=dt)

    def cast(c):
        sl = slice(c * CHUNK, min(flat.numel(), (c + 1) * CHUNK))
        out[sl] = flat[sl].to(dt)

    list(pool.map(cast, range((flat.numel() + CHUNK - 1) // CHUNK)))
    return out.view(x.shape)


def make_inputs(case: Case, device: str = "cpu") -> dict:
    """Draw one input set for `case` on the host (the same values on every machine),
    then move it to `device`.  Returns a dict of tensors plus "case"."""
    g_cpu = torch.Generator("cpu").manual_seed(case.seed)

    # 1. integer structure
    if case.seq_lens is not None:
        assert len(case.seq_lens) == case.batch
        seq_lens = torch.tensor(case.seq_lens, dtype=torch.int32)
    else:
        lo, hi = case.seq_len_range
        seq_lens = torch.randint(lo, hi + 1, (case.batch,), generator=g_cpu,
                                 dtype=torch.int64).to(torch.int32)
    block_table = None
    if case.cache_mode == "paged":
        need = case.batch * case.blocks_per_seq
        assert case.capacity % case.block_size == 0 and need <= case.num_blocks
        perm = torch.randperm(case.num_blocks, generator=g_cpu)
        block_table = perm[:need].view(case.batch, case.blocks_per_seq).to(torch.int32).contiguous()
    tree_mask = None
    if case.mask_mode == "tree":
        # one tree per sequence, as int64 words (bit 63 would be the sign bit)
        words = [tree_words_from_parents(draw_tree(case.q_len, g_cpu)) for _ in range(case.batch)]
        tree_mask = torch.tensor(np.array(words, dtype=np.uint64).view(np.int64))

    # 2. values (float32 standard normals)
    qshape = (case.batch, case.q_len, case.num_q_heads, case.head_dim)
    dt = DTYPES[case.dtype]
    kvdt = case.kv_dtype or case.dtype
    out = {"k_scale": None, "v_scale": None}
    with cf.ThreadPoolExecutor(_workers()) as pool:
        for n, (name, shape) in enumerate((("q", qshape), ("k_cache", cache_shape(case)),
                                           ("v_cache", cache_shape(case)))):
            x = _normals(shape, case.seed, n, pool)
            # 3. scale
            if case.value_scale != 1.0:
                x.mul_(case.value_scale)
            if name == "k_cache" and case.k0_boost != 1.0:
                # Logical position 0 of each sequence.  Contiguous and ring caches
                # keep position 0 in the sequence's first slot (sink tokens are
                # never evicted); a paged cache keeps it at offset 0 of the block
                # the first page-table entry names.
                if case.cache_mode == "paged":
                    for b in range(case.batch):
                        x[int(block_table[b, 0]), 0].mul_(case.k0_boost)
                else:
                    x[:, 0].mul_(case.k0_boost)
            # 4. cast
            if name != "q" and kvdt == "fp8":
                # per KV head (dim 2 of every cache layout): scale = amax / 448
                amax = x.abs().amax(dim=tuple(d for d in range(x.dim()) if d != 2))
                sc = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax)).to(torch.float32)
                x.div_(sc.view(1, 1, -1, 1))
                out[name] = _cast(x, torch.float8_e4m3fn, pool)
                out["k_scale" if name == "k_cache" else "v_scale"] = sc
            else:
                out[name] = _cast(x, dt, pool)
            del x
    for k in ("q", "k_cache", "v_cache", "k_scale", "v_scale"):
        if out[k] is not None:
            out[k] = out[k].to(device)
    out["seq_lens"] = seq_lens.to(device)
    out["block_table"] = block_table.to(device) if block_table is not None else None
    out["tree_mask"] = tree_mask.to(device) if tree_mask is not None else None
    out["case"] = case
    return out


def small_prefill_variants():
    """Reduced chunked-prefill cases: 100 new rows x GQA 4 (400 rows per KV head, seven
    blocks of 64 with a ragged last one) on a contiguous cache, one sequence shorter than
    its chunk; 80 rows x GQA 4 on a paged cache; 70 rows without GQA at head_dim 64 in
    f16 (a full block of 64 and a ragged one of 6); 100 rows on the StreamingLLM ring
    with its sink/window mask (the window rolling across the chunk)."""
    sv = small_variants()
    return {
        "prefill_small": CHUNKED_PREFILL.replace(name="prefill_small", batch=2, num_q_heads=8,
                                                 num_kv_heads=2, capacity=700, q_len=100,
                                                 seq_lens=(700, 60), seed=41),
        "prefill_paged": sv["paged_small"].replace(name="prefill_paged", q_len=80,
                                                   seq_lens=(1600, 500, 81), seed=42),
        "prefill_d64": CHUNKED_PREFILL.replace(name="prefill_d64", batch=2, num_q_heads=4,
                                               num_kv_heads=4, head_dim=64, dtype="f16",
                                               capacity=600, q_len=70, seq_lens=(600, 333),
                                               seed=43),
        "prefill_ring": sv["sink_window_small"].replace(name="prefill_ring", q_len=100,
                                                        seed=44),
    }


def small_tree_variants():
    """Reduced token-tree verification cases: 5 and 8 draft tokens with GQA 8 (40 and
    64 rows per KV head) and 7 on a paged cache with GQA 4 (28 rows; all three on the
    split-KV matrix-core kernel), 6 tokens without GQA (vector-ALU kernel), wide trees
    of 40 and 64 tokens with GQA 8 (320 and 512 rows: the prefill kernel's 256-row
    blocks, one of them ragged) and of 30 tokens on a paged cache (120 rows: two
    64-row blocks of the split-KV kernel), and sequences shorter than their tree."""
    sv = small_variants()
    base = sv["spec_verify_small"].replace(mask_mode="tree")
    return {
        "tree_small": base.replace(name="tree_small", seed=31),
        "tree_small_q8": base.replace(name="tree_small_q8", q_len=8, seed=32),
        "tree_short": base.replace(name="tree_short", q_len=8, seq_lens=(1000, 3, 8), seed=33),
        "tree_valu": sv["decode_7b_small"].replace(name="tree_valu", mask_mode="tree",
                                                   q_len=6, seq_len_range=(1, 1200), seed=34),
        "tree_paged": sv["paged_small"].replace(name="tree_paged", mask_mode="tree", q_len=7,
                                                seed=35),
        "tree_wide": base.replace(name="tree_wide", q_len=40, seed=36),
        "tree_q64": base.replace(name="tree_q64", q_len=64, seq_lens=(1000, 64, 40), seed=37),
        "tree_wide_paged": sv["paged_small"].replace(name="tree_wide_paged", mask_mode="tree",
                                                     q_len=30, seed=38),
    }


def small_fp8_variants():
    """Reduced cases with an 8-bit K/V cache: the reduced decode, ring and paged cases,
    a paged case with q_len 5 (per-row causal masks, 20 rows per KV head) and the
    reduced verify case (40 rows per KV head); the last two take the matrix cores."""
    sv = small_variants()
    return {
        "spec_verify_small_fp8": sv["spec_verify_small"].replace(name="spec_verify_small_fp8",
                                                                 kv_dtype="fp8", seed=27),
        "decode_7b_small_fp8": sv["decode_7b_small"].replace(name="decode_7b_small_fp8",
                                                             kv_dtype="fp8", seed=22),
        "sink_window_small_fp8": sv["sink_window_small"].replace(name="sink_window_small_fp8",
                                                                 kv_dtype="fp8", seed=24),
        "paged_small_fp8": sv["paged_small"].replace(name="paged_small_fp8", kv_dtype="fp8",
                                                     seed=25),
        "paged_small_q5_fp8": sv["paged_small"].replace(name="paged_small_q5_fp8",
                                                        kv_dtype="fp8", q_len=5, seed=26),
    }


def small_variants():
    """Reduced cases of each workload for element-by-element checks: several
    tiles per split, ragged tails, the same structure as the full sizes."""
    return {
        "tiny": TINY,
        "decode_7b_small": DECODE_7B.replace(name="decode_7b_small", batch=5, num_q_heads=4,
                                             num_kv_heads=4, capacity=1200,
                                             seq_len_range=(1, 1200), seed=12),
        "spec_verify_small": SPEC_VERIFY.replace(name="spec_verify_small", batch=3,
                                                 num_q_heads=16, num_kv_heads=2, capacity=1000,
                                                 seq_lens=(1000, 517, 5), seed=13),
        "sink_window_small": SINK_WINDOW.replace(name="sink_window_small", batch=4,
                                                 num_q_heads=4, num_kv_heads=4, capacity=700,
                                                 n_sink=4, window=300,
                                                 seq_lens=(700, 1013, 5000, 250), seed=14),
        "paged_small": PAGED_100K.replace(name="paged_small", batch=3, num_q_heads=8,
                                          num_kv_heads=2, capacity=1600, num_blocks=310,
                                          seq_lens=(1600, 1377, 33), seed=15),
    }
