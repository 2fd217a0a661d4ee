"""Python side of the oracle (test infrastructure only; the library never imports it).

`decode*` / `attended` call the C oracle (kvattn_oracle.c).  The `*_np`
functions are an independent NumPy/PyTorch-CPU float64 twin of the same
definition, used to cross-check the C code and to state the pins:

  * Attention(Q, K, V) = softmax(Q K^T / sqrt(d)) V - "softmax problem"
    section of the dothoosh.com StreamingLLM / attention-sinks article;
  * one new query row against every cached key - "KV cache" item of the
    nextadmin.net lesson "KV cache and Flash Attention";
  * the running (max, sum) softmax across tiles gives the same result as
    the one-shot softmax - same lesson, "Flash Attention - the tiling trick"
    and implementation step 2 (tiled softmax);
  * PagedAttention: 16-token blocks and a page table from logical positions
    to physical blocks - same lesson, "PagedAttention" section;
  * StreamingLLM keeps the first 4 tokens plus the 4,092 most recent -
    StreamingLLM article, "The StreamingLLM solution".

A "problem" is any object with the attributes of a workload case
(batch, num_q_heads, num_kv_heads, head_dim, dtype, cache_mode, capacity,
q_len, mask_mode, n_sink, window, block_size); it is read by name only.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import numpy as np
import torch

DTYPE_CODES = {"f32": 0, "f16": 1, "bf16": 2, "fp8": 3}
CACHE_CODES = {"contiguous": 0, "paged": 1, "ring": 2}
MASK_CODES = {"causal": 0, "sink_window": 1, "tree": 2}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


class _Problem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in (
        "dtype", "batch", "num_q_heads", "num_kv_heads", "head_dim", "q_len",
        "cache_mode", "capacity", "block_size", "blocks_per_seq",
        "mask_mode", "n_sink", "window")] + [("scale", ctypes.c_double),
                                             ("kv_dtype", ctypes.c_int),
                                             ("k_scale", ctypes.c_void_p),
                                             ("v_scale", ctypes.c_void_p),
                                             ("tree_mask", ctypes.c_void_p)]


def load():
    """Load (building first if absent) the C oracle.  KVATTN_ORACLE_LIB names another
    build of it (the mutation test points the pins at deliberately broken copies)."""
    global _lib
    if _lib is not None:
        return _lib
    path = os.environ.get("KVATTN_ORACLE_LIB") or _LIB_PATH
    if path == _LIB_PATH and not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER(_Problem)
    vp, i32p, f64p, i64p = (ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32),
                            ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64))
    lib.oracle_decode.argtypes = [P, vp, vp, vp, i32p, i32p, f64p, ctypes.c_int]
    lib.oracle_decode.restype = ctypes.c_int
    lib.oracle_decode_rows.argtypes = [P, vp, vp, vp, i32p, i32p, i32p, ctypes.c_int64, f64p,
                                       ctypes.c_int]
    lib.oracle_decode_rows.restype = ctypes.c_int
    lib.oracle_attended.argtypes = [ctypes.c_int] * 5 + [ctypes.c_int64] + [ctypes.c_int] * 4 + [
        i32p, ctypes.c_int, ctypes.c_uint64, i64p, i64p, ctypes.c_int64]
    lib.oracle_attended.restype = ctypes.c_int64
    lib.oracle_max_threads.restype = ctypes.c_int
    lib.oracle_decode_elem.argtypes = [vp, ctypes.c_int, ctypes.c_int64]
    lib.oracle_decode_elem.restype = ctypes.c_double
    _lib = lib
    return lib


def threads() -> int:
    return load().oracle_max_threads()


def kv_dtype_of(pr) -> str:
    """Element type of the caches: the problem's kv_dtype when it has one, else dtype."""
    return getattr(pr, "kv_dtype", None) or pr.dtype


def _problem(pr, scale: float = 0.0, k_scale=None, v_scale=None, tree=None) -> _Problem:
    # k_scale / v_scale: float32 CPU tensors [num_kv_heads], tree: int64 CPU tensor
    # [batch, q_len] of mask words; kept alive by the caller
    return _Problem(DTYPE_CODES[pr.dtype], pr.batch, pr.num_q_heads, pr.num_kv_heads,
                    pr.head_dim, pr.q_len, CACHE_CODES[pr.cache_mode], pr.capacity,
                    pr.block_size, pr.capacity // pr.block_size, MASK_CODES[pr.mask_mode],
                    pr.n_sink, pr.window, float(scale), DTYPE_CODES[kv_dtype_of(pr)],
                    _ptr(k_scale), _ptr(v_scale), _ptr(tree))


def tree_words(tree_mask) -> np.ndarray:
    """Mask words as uint64 (bit j = the row attends new position j); accepts int64
    torch tensors (bit 63 as the sign) or any integer array."""
    if isinstance(tree_mask, torch.Tensor):
        return np.ascontiguousarray(_cpu(tree_mask).to(torch.int64).numpy().view(np.uint64))
    a = np.asarray(tree_mask)
    return np.ascontiguousarray(a.view(np.uint64) if a.dtype == np.int64 else a.astype(np.uint64))


def _tree(tree_mask):
    """Mask words as a contiguous int64 CPU tensor for the C oracle."""
    if tree_mask is None:
        return None
    return torch.from_numpy(tree_words(tree_mask).view(np.int64).copy())


def _scales(k_scale, v_scale):
    f = lambda t: None if t is None else _cpu(t).to(torch.float32).contiguous()
    return f(k_scale), f(v_scale)


def _cpu(t: Optional[torch.Tensor]):
    if t is None:
        return None
    t = t.detach()
    if t.device.type != "cpu":
        t = t.cpu()
    return t.contiguous()


def _ptr(t, ctype=None):
    if t is None:
        return None
    p = ctypes.c_void_p(t.data_ptr())
    return ctypes.cast(p, ctypes.POINTER(ctype)) if ctype else p


def decode(pr, q, k_cache, v_cache, block_table, seq_lens, scale: float = 0.0,
           n_threads: int = 0, k_scale=None, v_scale=None, tree_mask=None) -> np.ndarray:
    """All rows; float64 [batch, q_len, num_q_heads, head_dim].  An 8-bit cache
    (pr.kv_dtype == "fp8") takes per-KV-head dequantisation scales k_scale, v_scale;
    pr.mask_mode == "tree" takes tree_mask [batch, q_len] (uint64 words)."""
    lib = load()
    q, kc, vc, bt, sl = (_cpu(x) for x in (q, k_cache, v_cache, block_table, seq_lens))
    ks, vs = _scales(k_scale, v_scale)
    tm = _tree(tree_mask)
    out = np.zeros((pr.batch, pr.q_len, pr.num_q_heads, pr.head_dim), np.float64)
    rc = lib.oracle_decode(ctypes.byref(_problem(pr, scale, ks, vs, tm)), _ptr(q), _ptr(kc), _ptr(vc),
                           _ptr(bt, ctypes.c_int32), _ptr(sl, ctypes.c_int32),
                           out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), n_threads)
    if rc != 0:
        raise ValueError("oracle rejected the problem")
    return out


def decode_rows(pr, q, k_cache, v_cache, block_table, seq_lens, rows, scale: float = 0.0,
                n_threads: int = 0, k_scale=None, v_scale=None, tree_mask=None) -> np.ndarray:
    """Listed rows only: rows is int [n, 3] of (b, i, h); returns float64 [n, head_dim]."""
    lib = load()
    q, kc, vc, bt, sl = (_cpu(x) for x in (q, k_cache, v_cache, block_table, seq_lens))
    ks, vs = _scales(k_scale, v_scale)
    tm = _tree(tree_mask)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int32).reshape(-1, 3))
    out = np.zeros((rows.shape[0], pr.head_dim), np.float64)
    rc = lib.oracle_decode_rows(ctypes.byref(_problem(pr, scale, ks, vs, tm)), _ptr(q), _ptr(kc), _ptr(vc),
                                _ptr(bt, ctypes.c_int32), _ptr(sl, ctypes.c_int32),
                                rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                rows.shape[0],
                                out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), n_threads)
    if rc != 0:
        raise ValueError("oracle rejected the problem")
    return out


def attended(pr, block_table, seq_lens, b: int, i: int, tree_bits: int = 0):
    """(positions, flat slots) that row (b, i) attends, in increasing position order
    (mask "tree": tree_bits is the row's mask word)."""
    lib = load()
    bt, sl = _cpu(block_table), _cpu(seq_lens)
    T = int(sl[b])
    n = lib.oracle_attended(CACHE_CODES[pr.cache_mode], MASK_CODES[pr.mask_mode], b, i,
                            pr.q_len, T, pr.n_sink, pr.window, pr.capacity, pr.block_size,
                            _ptr(bt, ctypes.c_int32), pr.capacity // pr.block_size, tree_bits,
                            None, None, 0)
    pos = np.zeros(max(n, 1), np.int64)
    slots = np.zeros(max(n, 1), np.int64)
    lib.oracle_attended(CACHE_CODES[pr.cache_mode], MASK_CODES[pr.mask_mode], b, i, pr.q_len, T,
                        pr.n_sink, pr.window, pr.capacity, pr.block_size,
                        _ptr(bt, ctypes.c_int32), pr.capacity // pr.block_size, tree_bits,
                        pos.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                        slots.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), n)
    return pos[:n], slots[:n]


# ---------------------------------------------------------------------------
# NumPy / PyTorch-CPU float64 twin
# ---------------------------------------------------------------------------

def to_f64(t) -> np.ndarray:
    """Exact upcast of a stored tensor (f32 / f16 / bf16 / float8_e4m3fn) to float64
    (torch's conversion)."""
    if isinstance(t, np.ndarray):
        return t.astype(np.float64)
    return t.detach().cpu().to(torch.float64).numpy()


def attended_positions_np(mask_mode: str, T: int, q_len: int, i: int, n_sink: int,
                          window: int, tree_bits: int = 0) -> np.ndarray:
    """Positions the new row i (at T - q_len + i) attends, in increasing order.  Tree
    mask: every position before the new block, and new position T - q_len + j when
    bit j of tree_bits is set."""
    P = T - q_len + i
    p = np.arange(max(T, 0), dtype=np.int64)
    if mask_mode == "tree":
        j = p - (T - q_len)
        bit = np.array([(int(tree_bits) >> int(x)) & 1 if 0 <= x < 64 else 0 for x in j],
                       dtype=bool) if p.size else np.zeros(0, bool)
        return p[(j < 0) | bit]
    keep = p <= P
    if mask_mode == "sink_window":
        keep &= (p < n_sink) | (p > P - window)
    return p[keep]


def slot_np(cache_mode: str, b: int, p: np.ndarray, capacity: int, block_size: int,
            block_table, n_sink: int) -> np.ndarray:
    """Flat cache slot of logical positions p of sequence b."""
    p = np.asarray(p, dtype=np.int64)
    if cache_mode == "contiguous":
        return b * capacity + p
    if cache_mode == "paged":
        bt = np.asarray(block_table if isinstance(block_table, np.ndarray)
                        else block_table.cpu().numpy(), dtype=np.int64)
        return bt[b, p // block_size] * block_size + p % block_size
    r = capacity - n_sink
    return b * capacity + np.where(p < n_sink, p, n_sink + (p - n_sink) % max(r, 1))


def decode_np(pr, q, k_cache, v_cache, block_table, seq_lens, scale: float = 0.0,
              k_scale=None, v_scale=None, tree_mask=None) -> np.ndarray:
    """float64 [batch, q_len, Hq, D]; gathers only the attended slots.  8-bit caches
    are dequantised with the per-KV-head scales (torch's E4M3 conversion)."""
    D, Hq, Hkv = pr.head_dim, pr.num_q_heads, pr.num_kv_heads
    g = Hq // Hkv
    sc = scale if scale != 0.0 else 1.0 / math.sqrt(D)
    q64 = to_f64(q)
    ks = np.ones(Hkv) if k_scale is None else to_f64(k_scale.float())
    vs = np.ones(Hkv) if v_scale is None else to_f64(v_scale.float())
    kflat = k_cache.reshape(-1, Hkv, D)
    vflat = v_cache.reshape(-1, Hkv, D)
    sl = np.asarray(seq_lens.cpu() if isinstance(seq_lens, torch.Tensor) else seq_lens)
    out = np.zeros((pr.batch, pr.q_len, Hq, D))
    kv_of_h = np.arange(Hq) // g
    for b in range(pr.batch):
        for i in range(pr.q_len):
            bits = 0 if tree_mask is None else int(tree_words(tree_mask)[b, i])
            pos = attended_positions_np(pr.mask_mode, int(sl[b]), pr.q_len, i, pr.n_sink,
                                        pr.window, bits)
            if pos.size == 0:
                continue
            slots = slot_np(pr.cache_mode, b, pos, pr.capacity, pr.block_size, block_table,
                            pr.n_sink)
            idx = torch.as_tensor(slots)
            K = (to_f64(kflat.index_select(0, idx.to(kflat.device))) * ks[None, :, None])[:, kv_of_h, :]
            V = (to_f64(vflat.index_select(0, idx.to(vflat.device))) * vs[None, :, None])[:, kv_of_h, :]
            s = np.einsum("nhd,hd->hn", K, q64[b, i]) * sc
            w = np.exp(s - s.max(axis=1, keepdims=True))
            w /= w.sum(axis=1, keepdims=True)
            out[b, i] = np.einsum("hn,nhd->hd", w, V)
    return out


def decode_matmul_np(pr, q, k_cache, v_cache, block_table, seq_lens, scale: float = 0.0,
                     k_scale=None, v_scale=None, tree_mask=None) -> np.ndarray:
    """float64 [batch, q_len, Hq, D]: softmax(Q K^T / sqrt(d)) V written in matrix form
    (StreamingLLM article, "The softmax problem"), one (sequence, KV head) at a time:
    the scores of all q_len x group query rows against the sequence's attended
    positions as one float64 matrix product, the explicit boolean mask of each new row
    (-inf where it does not attend), a row-wise softmax, and one more product with V.
    Same definition as decode_np; the products are library matmuls, which makes the
    hundreds of rows of a prefill chunk affordable.  A row that attends nothing is 0."""
    D, Hq, Hkv = pr.head_dim, pr.num_q_heads, pr.num_kv_heads
    g = Hq // Hkv
    ql = pr.q_len
    sc = scale if scale != 0.0 else 1.0 / math.sqrt(D)
    ks = np.ones(Hkv) if k_scale is None else to_f64(k_scale.float())
    vs = np.ones(Hkv) if v_scale is None else to_f64(v_scale.float())
    kflat = _cpu(k_cache).reshape(-1, Hkv, D)
    vflat = _cpu(v_cache).reshape(-1, Hkv, D)
    q64 = to_f64(q)
    sl = np.asarray(seq_lens.cpu() if isinstance(seq_lens, torch.Tensor) else seq_lens)
    words = None if tree_mask is None else tree_words(tree_mask)
    out = np.zeros((pr.batch, ql, Hq, D))
    for b in range(pr.batch):
        T = int(sl[b])
        rows = [attended_positions_np(pr.mask_mode, T, ql, i, pr.n_sink, pr.window,
                                      0 if words is None else int(words[b, i]))
                for i in range(ql)]
        union = np.unique(np.concatenate(rows)) if any(r.size for r in rows) else None
        if union is None:
            continue
        mask = np.zeros((ql, union.size), bool)
        for i, r in enumerate(rows):
            mask[i, np.searchsorted(union, r)] = True
        idx = torch.as_tensor(slot_np(pr.cache_mode, b, union, pr.capacity, pr.block_size,
                                      block_table, pr.n_sink))
        Kb = kflat.index_select(0, idx)
        Vb = vflat.index_select(0, idx)
        live = mask.any(axis=1)
        for kvh in range(Hkv):
            K = to_f64(Kb[:, kvh]) * ks[kvh]
            V = to_f64(Vb[:, kvh]) * vs[kvh]
            Q = q64[b, :, kvh * g:(kvh + 1) * g, :].reshape(ql * g, D)
            S = ((Q @ K.T) * sc).reshape(ql, g, union.size)
            S = np.where(mask[:, None, :], S, -np.inf)
            S[~live] = 0.0  # rows with nothing to attend: zeroed below
            W = np.exp(S - S.max(axis=2, keepdims=True))
            W /= W.sum(axis=2, keepdims=True)
            O = (W.reshape(ql * g, union.size) @ V).reshape(ql, g, D)
            O[~live] = 0.0
            out[b, :, kvh * g:(kvh + 1) * g, :] = O
    return out


def full_causal_np(Q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """Full T x T causal attention recomputed from scratch (the O(N^2) decoder of the
    lesson's problem statement).  Q, K, V: [T, H, D] float64 -> [T, H, D]."""
    T = Q.shape[0]
    S = np.einsum("thd,shd->hts", Q, K) * scale
    S = np.where(np.tril(np.ones((T, T), bool))[None], S, -np.inf)
    S = S - S.max(axis=2, keepdims=True)
    W = np.exp(S)
    W /= W.sum(axis=2, keepdims=True)
    return np.einsum("hts,shd->thd", W, V)


def tiled_softmax_dot_np(q: np.ndarray, K: np.ndarray, V: np.ndarray, tile: int,
                         scale: float) -> np.ndarray:
    """Online softmax over key tiles (lesson, implementation step 2), with the 1/sqrt(d)
    scale of the attention formula.  q: [D], K, V: [n, D] float64 -> [D]."""
    m = -np.inf
    s = 0.0
    out = np.zeros(V.shape[1])
    for start in range(0, K.shape[0], tile):
        sc = (K[start:start + tile] @ q) * scale
        new_m = max(m, sc.max())
        old_factor = math.exp(m - new_m) if m != -np.inf else 0.0   # nothing to rescale yet
        e = np.exp(sc - new_m)
        s = s * old_factor + e.sum()
        out = out * old_factor + e @ V[start:start + tile]
        m = new_m
    return out / s


def split_merge_np(q: np.ndarray, K: np.ndarray, V: np.ndarray, n_split: int,
                   scale: float) -> np.ndarray:
    """Cut the keys into n_split contiguous pieces (some may be empty), take each piece's
    unnormalised (max, sum, weighted V), then merge with log-sum-exp weights."""
    n = K.shape[0]
    bounds = [round(n * j / n_split) for j in range(n_split + 1)]
    parts = []
    for a, z in zip(bounds[:-1], bounds[1:]):
        if z <= a:
            parts.append((-np.inf, 0.0, np.zeros(V.shape[1])))
            continue
        sc = (K[a:z] @ q) * scale
        m = sc.max()
        e = np.exp(sc - m)
        parts.append((m, e.sum(), e @ V[a:z]))
    M = max(p[0] for p in parts)
    L = sum(l * math.exp(m - M) for m, l, _ in parts if l > 0)
    acc = sum(a * math.exp(m - M) for m, l, a in parts if l > 0)
    return acc / L


def append_np(pr, k_cache, v_cache, k_new, v_new, block_table, seq_lens, n_sink: int = 0,
              num_blocks: Optional[int] = None):
    """KV append: copies of the token-major caches with row i of sequence b of
    k_new / v_new [batch, q_len, Hkv, D] written to the slot of position
    P = T_b - q_len + i - the new token's key and value written back before it is
    attended (dothoosh.com speculative-decoding article, "bypassing the memory
    bottleneck"); slots as in slot_np (contiguous; 16-token pages through the page
    table, nextadmin.net lesson "PagedAttention"; the StreamingLLM ring whose sinks
    keep their slots, "The StreamingLLM solution").  Rows without a slot are not
    written: P < 0, P >= capacity (contiguous, paged), or a page-table entry outside
    [0, num_blocks).  Stored values are copied unchanged (any element type)."""
    kc, vc = k_cache.clone(), v_cache.clone()
    Hkv, D = pr.num_kv_heads, pr.head_dim
    kf, vf = kc.view(-1, Hkv, D), vc.view(-1, Hkv, D)
    sl = [int(x) for x in (seq_lens.cpu() if isinstance(seq_lens, torch.Tensor) else seq_lens)]
    bt = None
    if pr.cache_mode == "paged":
        bt = np.asarray(block_table.cpu() if isinstance(block_table, torch.Tensor)
                        else block_table, dtype=np.int64)
    for b in range(len(sl)):
        T = max(sl[b], 0)
        for i in range(pr.q_len):
            P = T - pr.q_len + i
            if P < 0:
                continue
            if pr.cache_mode != "ring" and P >= pr.capacity:
                continue
            if pr.cache_mode == "paged":
                blk = int(bt[b, P // pr.block_size])
                if num_blocks is not None and not 0 <= blk < num_blocks:
                    continue
            slot = int(slot_np(pr.cache_mode, b, np.array([P]), pr.capacity, pr.block_size, bt,
                               n_sink)[0])
            kf[slot] = k_new[b, i]
            vf[slot] = v_new[b, i]
    return kc, vc
