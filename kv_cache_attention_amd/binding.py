"""Thin ctypes binding of libkvattn.so (include/kvattn.h).

Argument marshalling only: tensors become device pointers, the current torch
stream becomes the handle's stream, and every step of the computation runs in
the library's HIP kernels.  There is no fallback: without the built library
(or without a GPU) these calls raise.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvattn.so")

KVATTN_OK = 0
STATUS = {0: "OK", -1: "INVALID_ARG", -2: "UNSUPPORTED", -3: "CAPACITY", -4: "HIP",
          -5: "DEVICE_DATA"}
DTYPE = {"f32": 0, "f16": 1, "bf16": 2, "fp8": 3}
TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16,
               "fp8": torch.float8_e4m3fn}
CACHE = {"contiguous": 0, "paged": 1, "ring": 2}
MASK = {"causal": 0, "sink_window": 1, "tree": 2}
LAYOUT = {"token_major": 0, "head_major": 1}

EXPORTS = ("kvattn_create", "kvattn_decode", "kvattn_destroy", "kvattn_set_stream",
           "kvattn_set_batch", "kvattn_set_split_len", "kvattn_set_kv_scales", "kvattn_plan",
           "kvattn_workspace_bytes", "kvattn_last_error", "kvattn_debug_gather", "kvattn_append",
           "kvattn_append_decode", "kvattn_decode_tree", "kvattn_debug_gather_tree",
           "kvattn_check", "kvattn_stream_read", "kvattn_decode_noalloc")


class kvattn_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "dtype", "num_q_heads", "num_kv_heads", "head_dim", "max_batch", "max_q_len",
        "cache_mode", "capacity", "block_size", "num_blocks", "layout")] + [
        ("scale", ctypes.c_float), ("flags", ctypes.c_uint32), ("kv_dtype", ctypes.c_int32)]


FLAG_DETERMINISTIC = 1
FLAG_DEBUG = 2


class KVAttnError(RuntimeError):
    def __init__(self, code: int, where: str, msg: str):
        super().__init__(f"{where}: {STATUS.get(code, code)}: {msg}")
        self.code = code


_lib = None


def load() -> ctypes.CDLL:
    """Load libkvattn.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built (run kv_cache_attention_amd/build.py)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i32p = ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32)
    H = ctypes.c_void_p
    lib.kvattn_create.argtypes = [ctypes.POINTER(kvattn_config), ctypes.POINTER(H)]
    lib.kvattn_create.restype = ctypes.c_int
    lib.kvattn_decode.argtypes = [H, vp, vp, vp, vp, vp, i32, i32, i32, i32, vp]
    lib.kvattn_decode.restype = ctypes.c_int
    lib.kvattn_destroy.argtypes = [H]
    lib.kvattn_destroy.restype = None
    lib.kvattn_set_stream.argtypes = [H, vp]
    lib.kvattn_set_stream.restype = ctypes.c_int
    lib.kvattn_set_batch.argtypes = [H, i32]
    lib.kvattn_set_batch.restype = ctypes.c_int
    lib.kvattn_set_split_len.argtypes = [H, i32]
    lib.kvattn_set_split_len.restype = ctypes.c_int
    lib.kvattn_set_kv_scales.argtypes = [H, vp, vp]
    lib.kvattn_set_kv_scales.restype = ctypes.c_int
    lib.kvattn_plan.argtypes = [H, i32, i32, i32, i32, i32p, i32p, i32p]
    lib.kvattn_plan.restype = ctypes.c_int
    lib.kvattn_workspace_bytes.argtypes = [ctypes.POINTER(kvattn_config),
                                           ctypes.POINTER(ctypes.c_size_t)]
    lib.kvattn_workspace_bytes.restype = ctypes.c_int
    lib.kvattn_last_error.argtypes = []
    lib.kvattn_last_error.restype = ctypes.c_char_p
    lib.kvattn_debug_gather.argtypes = [H, vp, vp, i32, i32, i32, i32, i32, vp, vp]
    lib.kvattn_debug_gather.restype = ctypes.c_int
    lib.kvattn_decode_tree.argtypes = [H, vp, vp, vp, vp, vp, i32, vp, vp]
    lib.kvattn_decode_tree.restype = ctypes.c_int
    lib.kvattn_debug_gather_tree.argtypes = [H, vp, vp, i32, vp, i32, vp, vp]
    lib.kvattn_debug_gather_tree.restype = ctypes.c_int
    lib.kvattn_append.argtypes = [H, vp, vp, vp, vp, vp, vp, i32, i32]
    lib.kvattn_append.restype = ctypes.c_int
    lib.kvattn_append_decode.argtypes = [H, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, vp]
    lib.kvattn_append_decode.restype = ctypes.c_int
    lib.kvattn_check.argtypes = [H]
    lib.kvattn_check.restype = ctypes.c_int
    lib.kvattn_stream_read.argtypes = [vp, ctypes.c_size_t, vp, vp]
    lib.kvattn_stream_read.restype = ctypes.c_int
    lib.kvattn_decode_noalloc.argtypes = [ctypes.POINTER(kvattn_config), i32, vp, vp, vp, vp, vp,
                                          i32, i32, i32, i32, vp, vp]
    lib.kvattn_decode_noalloc.restype = ctypes.c_int
    _lib = lib
    return lib


def _check(rc: int, where: str) -> None:
    if rc != KVATTN_OK:
        raise KVAttnError(rc, where, load().kvattn_last_error().decode())


def _dev_ptr(t: Optional[torch.Tensor], name: str):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def make_config(*, dtype: str, num_q_heads: int, num_kv_heads: int, head_dim: int,
                max_batch: int, max_q_len: int, cache_mode: str, capacity: int,
                block_size: int = 16, num_blocks: int = 0, layout: str = "token_major",
                scale: float = 0.0, deterministic: bool = False,
                kv_dtype: Optional[str] = None, debug: bool = False) -> kvattn_config:
    flags = (FLAG_DETERMINISTIC if deterministic else 0) | (FLAG_DEBUG if debug else 0)
    return kvattn_config(DTYPE[dtype], num_q_heads, num_kv_heads, head_dim, max_batch, max_q_len,
                         CACHE[cache_mode], capacity, block_size, num_blocks, LAYOUT[layout],
                         scale, flags, DTYPE[kv_dtype] if kv_dtype else 0)


# ------------------------------------------------------------ same names as the C ABI

def kvattn_create(cfg: kvattn_config) -> ctypes.c_void_p:
    h = ctypes.c_void_p()
    _check(load().kvattn_create(ctypes.byref(cfg), ctypes.byref(h)), "kvattn_create")
    return h


def kvattn_decode(h, q, k_cache, v_cache, block_table, seq_lens, q_len: int, mask_mode: int,
                  n_sink: int, window: int, out) -> None:
    _check(load().kvattn_decode(h, _dev_ptr(q, "q"), _dev_ptr(k_cache, "k_cache"),
                                _dev_ptr(v_cache, "v_cache"), _dev_ptr(block_table, "block_table"),
                                _dev_ptr(seq_lens, "seq_lens"), q_len, mask_mode, n_sink, window,
                                _dev_ptr(out, "out")), "kvattn_decode")


def kvattn_decode_tree(h, q, k_cache, v_cache, block_table, seq_lens, q_len: int, tree_mask,
                       out) -> None:
    _check(load().kvattn_decode_tree(h, _dev_ptr(q, "q"), _dev_ptr(k_cache, "k_cache"),
                                     _dev_ptr(v_cache, "v_cache"),
                                     _dev_ptr(block_table, "block_table"),
                                     _dev_ptr(seq_lens, "seq_lens"), q_len,
                                     _dev_ptr(tree_mask, "tree_mask"), _dev_ptr(out, "out")),
           "kvattn_decode_tree")


def kvattn_debug_gather_tree(h, block_table, seq_lens, q_len: int, tree_mask, max_slots: int,
                             slots_out, counts_out) -> None:
    _check(load().kvattn_debug_gather_tree(h, _dev_ptr(block_table, "block_table"),
                                           _dev_ptr(seq_lens, "seq_lens"), q_len,
                                           _dev_ptr(tree_mask, "tree_mask"), max_slots,
                                           _dev_ptr(slots_out, "slots_out"),
                                           _dev_ptr(counts_out, "counts_out")),
           "kvattn_debug_gather_tree")


def kvattn_append(h, k_new, v_new, k_cache, v_cache, block_table, seq_lens, q_len: int,
                  n_sink: int) -> None:
    _check(load().kvattn_append(h, _dev_ptr(k_new, "k_new"), _dev_ptr(v_new, "v_new"),
                                _dev_ptr(k_cache, "k_cache"), _dev_ptr(v_cache, "v_cache"),
                                _dev_ptr(block_table, "block_table"), _dev_ptr(seq_lens, "seq_lens"),
                                q_len, n_sink), "kvattn_append")


def kvattn_append_decode(h, q, k_new, v_new, k_cache, v_cache, block_table, seq_lens, q_len: int,
                         mask_mode: int, n_sink: int, window: int, out) -> None:
    _check(load().kvattn_append_decode(
        h, _dev_ptr(q, "q"), _dev_ptr(k_new, "k_new"), _dev_ptr(v_new, "v_new"),
        _dev_ptr(k_cache, "k_cache"), _dev_ptr(v_cache, "v_cache"),
        _dev_ptr(block_table, "block_table"), _dev_ptr(seq_lens, "seq_lens"), q_len, mask_mode,
        n_sink, window, _dev_ptr(out, "out")), "kvattn_append_decode")


def kvattn_destroy(h) -> None:
    load().kvattn_destroy(h)


def kvattn_set_stream(h, stream: int) -> None:
    _check(load().kvattn_set_stream(h, ctypes.c_void_p(stream)), "kvattn_set_stream")


def kvattn_set_batch(h, batch: int) -> None:
    _check(load().kvattn_set_batch(h, batch), "kvattn_set_batch")


def kvattn_set_split_len(h, split_len: int) -> None:
    _check(load().kvattn_set_split_len(h, split_len), "kvattn_set_split_len")


def kvattn_set_kv_scales(h, k_scale, v_scale) -> None:
    if k_scale is None or v_scale is None:
        raise ValueError("k_scale and v_scale are required")
    for name, t in (("k_scale", k_scale), ("v_scale", v_scale)):
        if t.dtype != torch.float32:
            raise ValueError(f"{name} must be float32")
    _check(load().kvattn_set_kv_scales(h, _dev_ptr(k_scale, "k_scale"), _dev_ptr(v_scale, "v_scale")),
           "kvattn_set_kv_scales")


def kvattn_plan(h, q_len: int, mask_mode: int, n_sink: int, window: int):
    ns, sl, kern = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _check(load().kvattn_plan(h, q_len, mask_mode, n_sink, window, ctypes.byref(ns),
                              ctypes.byref(sl), ctypes.byref(kern)), "kvattn_plan")
    return ns.value, sl.value, kern.value


def kvattn_workspace_bytes(cfg: kvattn_config) -> int:
    n = ctypes.c_size_t()
    _check(load().kvattn_workspace_bytes(ctypes.byref(cfg), ctypes.byref(n)),
           "kvattn_workspace_bytes")
    return n.value


def kvattn_last_error() -> str:
    return load().kvattn_last_error().decode()


def kvattn_check(h) -> None:
    _check(load().kvattn_check(h), "kvattn_check")


def kvattn_decode_noalloc(cfg: kvattn_config, batch: int, q, k_cache, v_cache, block_table,
                          seq_lens, q_len: int, mask_mode: int, n_sink: int, window: int, out,
                          stream: int) -> None:
    _check(load().kvattn_decode_noalloc(ctypes.byref(cfg), batch, _dev_ptr(q, "q"),
                                        _dev_ptr(k_cache, "k_cache"), _dev_ptr(v_cache, "v_cache"),
                                        _dev_ptr(block_table, "block_table"),
                                        _dev_ptr(seq_lens, "seq_lens"), q_len, mask_mode, n_sink,
                                        window, _dev_ptr(out, "out"), ctypes.c_void_p(stream)),
           "kvattn_decode_noalloc")


def kvattn_stream_read(buf, sink, stream: int) -> None:
    """Enqueue a plain streaming read of the whole (contiguous, device) tensor `buf`."""
    if buf.nbytes % 16:
        raise ValueError("buf must hold a multiple of 16 bytes")
    _check(load().kvattn_stream_read(_dev_ptr(buf, "buf"), buf.nbytes, _dev_ptr(sink, "sink"),
                                     ctypes.c_void_p(stream)), "kvattn_stream_read")


def kvattn_debug_gather(h, block_table, seq_lens, q_len: int, mask_mode: int, n_sink: int,
                        window: int, max_slots: int, slots_out, counts_out) -> None:
    _check(load().kvattn_debug_gather(h, _dev_ptr(block_table, "block_table"),
                                      _dev_ptr(seq_lens, "seq_lens"), q_len, mask_mode, n_sink,
                                      window, max_slots, _dev_ptr(slots_out, "slots_out"),
                                      _dev_ptr(counts_out, "counts_out")), "kvattn_debug_gather")


# ------------------------------------------------------------ argument checks

class ArgCheck:
    """Shapes a handle's calls need, checked before the pointers go to the library
    (which cannot see sizes): q / out [batch, q_len, Hq, D]; caches [>= batch,
    capacity, Hkv, D] (head-major [>= batch, Hkv, capacity, D]) or the paged pool
    [num_blocks, block_size, Hkv, D] (head-major [num_blocks, Hkv, block_size, D]);
    new K/V rows [batch, q_len, Hkv, D]; seq_lens [>= batch] int32; block_table
    [>= batch, capacity / block_size] int32; tree words [>= batch, q_len] int64.
    Raises ValueError on a mismatch."""

    def __init__(self, *, dtype, kv_dtype, num_q_heads, num_kv_heads, head_dim, cache_mode,
                 capacity, block_size, num_blocks, layout):
        self.dtype, self.kv_dtype = dtype, kv_dtype or dtype
        self.num_q_heads, self.num_kv_heads, self.head_dim = num_q_heads, num_kv_heads, head_dim
        self.cache_mode, self.capacity, self.layout = cache_mode, capacity, layout
        self.block_size, self.num_blocks = block_size, num_blocks

    @staticmethod
    def tensor(name, t, dtype, shape, at_least0=True, on_device=True):
        """t (on the device when on_device), contiguous, of `dtype` and `shape` (dim 0
        at least shape[0] when at_least0, else exactly)."""
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"{name} must be a tensor")
        if on_device and not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if t.dtype != dtype:
            raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        ok = t.dim() == len(shape) and tuple(t.shape[1:]) == tuple(shape[1:]) and (
            t.shape[0] >= shape[0] if at_least0 else t.shape[0] == shape[0])
        if not ok:
            want = ("[>=%d, " % shape[0] if at_least0 else "[%d, " % shape[0]) + \
                   ", ".join(str(x) for x in shape[1:]) + "]"
            raise ValueError(f"{name} has shape {list(t.shape)}, the handle needs {want}")

    def cache_shape(self, batch):
        H, D = self.num_kv_heads, self.head_dim
        rows = (self.num_blocks, self.block_size) if self.cache_mode == "paged" else \
            (batch, self.capacity)
        if self.layout == "token_major":
            return (rows[0], rows[1], H, D)
        return (rows[0], H, rows[1], D)

    def step(self, batch, q_len, q=None, out=None, caches=(), block_table=None, seq_lens=None,
             new_rows=(), tree_mask=None, on_device=True):
        chk = lambda *a, **k: self.tensor(*a, on_device=on_device, **k)  # noqa: E731
        qshape = (batch, q_len, self.num_q_heads, self.head_dim)
        if q is not None:
            chk("q", q, TORCH_DTYPE[self.dtype], qshape)
        if out is not None:
            chk("out", out, TORCH_DTYPE[self.dtype], qshape)
        for name, t in caches:
            # a paged pool is the handle's pool; contiguous/ring hold >= batch sequences
            chk(name, t, TORCH_DTYPE[self.kv_dtype], self.cache_shape(batch),
                at_least0=self.cache_mode != "paged")
        for name, t in new_rows:
            chk(name, t, TORCH_DTYPE[self.kv_dtype], (batch, q_len, self.num_kv_heads,
                                                      self.head_dim))
        if seq_lens is not None:
            chk("seq_lens", seq_lens, torch.int32, (batch,))
        if self.cache_mode == "paged":
            if block_table is None:
                raise ValueError("a paged cache needs block_table")
            chk("block_table", block_table, torch.int32,
                (batch, self.capacity // self.block_size))
        elif block_table is not None:
            raise ValueError("block_table is for paged caches only")
        if tree_mask is not None:
            chk("tree_mask", tree_mask, torch.int64, (batch, q_len))


# ------------------------------------------------------------ convenience wrapper

class KVAttn:
    """One handle: a fixed problem shape and its workspace on the current device.

    Every tensor is checked against the handle before the call (device, dtype,
    contiguity, shape): the library takes plain pointers, so a tensor too small for
    the handle's batch, q_len, heads, head_dim, capacity or pool would be read or
    written past its end on the device.  A handle serves one stream at a time (its
    workspace holds one step): the first call binds it to the stream it runs on
    (the `stream` argument, else torch's current stream), and a later call on
    another stream raises unless `set_stream` moved the handle there first."""

    def __init__(self, *, dtype: str, num_q_heads: int, num_kv_heads: int, head_dim: int,
                 max_batch: int, max_q_len: int, cache_mode: str, capacity: int,
                 block_size: int = 16, num_blocks: int = 0, layout: str = "token_major",
                 scale: float = 0.0, deterministic: bool = False,
                 kv_dtype: Optional[str] = None, debug: bool = False):
        self.cfg = make_config(dtype=dtype, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                               head_dim=head_dim, max_batch=max_batch, max_q_len=max_q_len,
                               cache_mode=cache_mode, capacity=capacity, block_size=block_size,
                               num_blocks=num_blocks, layout=layout, scale=scale,
                               deterministic=deterministic, kv_dtype=kv_dtype, debug=debug)
        self.dtype = dtype
        self.kv_dtype = kv_dtype or dtype
        self.num_kv_heads = num_kv_heads
        self.args = ArgCheck(dtype=dtype, kv_dtype=kv_dtype, num_q_heads=num_q_heads,
                             num_kv_heads=num_kv_heads, head_dim=head_dim,
                             cache_mode=cache_mode, capacity=capacity, block_size=block_size,
                             num_blocks=num_blocks, layout=layout)
        self.batch = max_batch      # the library's initial batch
        self._stream = None         # bound at the first call (a raw hipStream_t value)
        self._scales = None  # keeps the scale tensors alive while the handle reads them
        self.h = kvattn_create(self.cfg)

    @classmethod
    def for_case(cls, case, layout: str = "token_major", max_batch: Optional[int] = None,
                 max_q_len: Optional[int] = None, deterministic: bool = False,
                 debug: bool = False) -> "KVAttn":
        return cls(dtype=case.dtype, num_q_heads=case.num_q_heads,
                   num_kv_heads=case.num_kv_heads, head_dim=case.head_dim,
                   max_batch=max_batch or case.batch, max_q_len=max_q_len or case.q_len,
                   cache_mode=case.cache_mode, capacity=case.capacity,
                   block_size=case.block_size, num_blocks=case.num_blocks, layout=layout,
                   deterministic=deterministic, kv_dtype=getattr(case, "kv_dtype", None),
                   debug=debug)

    def close(self) -> None:
        if self.h:
            kvattn_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ---- state

    def set_batch(self, batch: int) -> None:
        kvattn_set_batch(self.h, batch)
        self.batch = batch

    def set_split_len(self, split_len: int) -> None:
        kvattn_set_split_len(self.h, split_len)

    def set_kv_scales(self, k_scale, v_scale) -> None:
        for name, t in (("k_scale", k_scale), ("v_scale", v_scale)):
            if t is None or t.numel() < self.num_kv_heads:
                raise ValueError(f"{name} needs num_kv_heads = {self.num_kv_heads} values")
        kvattn_set_kv_scales(self.h, k_scale, v_scale)
        self._scales = (k_scale, v_scale)

    def set_stream(self, stream: torch.cuda.Stream) -> None:
        """Move the handle to `stream` once the work already enqueued on its current
        stream has finished (waited for here)."""
        if self._stream is not None and self._stream != stream.cuda_stream:
            torch.cuda.ExternalStream(self._stream).synchronize()
        self._stream = stream.cuda_stream
        kvattn_set_stream(self.h, self._stream)

    def _bind(self, stream: Optional[torch.cuda.Stream], device) -> None:
        st = stream if stream is not None else torch.cuda.current_stream(device)
        if self._stream is None:
            self._stream = st.cuda_stream
        elif self._stream != st.cuda_stream:
            raise ValueError("this handle is bound to another stream (its workspace serves one "
                             "step at a time); call set_stream first, or use one handle per stream")
        kvattn_set_stream(self.h, self._stream)

    def check(self) -> None:
        """Debug handles: raise KVAttnError if a step since the last check met
        device-resident arguments out of range."""
        kvattn_check(self.h)

    def plan(self, q_len: int, mask_mode: str = "causal", n_sink: int = 0, window: int = 0):
        return kvattn_plan(self.h, q_len, MASK[mask_mode], n_sink, window)

    def _out(self, q, out):
        return torch.empty_like(q) if out is None else out

    def _check_step(self, q_len, **kw):
        self.args.step(self.batch, q_len, **kw)

    # ---- steps

    def decode(self, q, k_cache, v_cache, block_table, seq_lens, q_len: int,
               mask_mode: str = "causal", n_sink: int = 0, window: int = 0, out=None,
               stream: Optional[torch.cuda.Stream] = None):
        out = self._out(q, out)
        self._check_step(q_len, q=q, out=out, caches=(("k_cache", k_cache), ("v_cache", v_cache)),
                         block_table=block_table, seq_lens=seq_lens)
        self._bind(stream, q.device)
        kvattn_decode(self.h, q, k_cache, v_cache, block_table, seq_lens, q_len, MASK[mask_mode],
                      n_sink, window, out)
        return out

    def decode_tree(self, q, k_cache, v_cache, block_table, seq_lens, q_len: int, tree_mask,
                    out=None, stream: Optional[torch.cuda.Stream] = None):
        """tree_mask: int64 device tensor [batch, q_len] of mask words (bit j = the row
        attends new position j; bit 63 is the sign bit)."""
        out = self._out(q, out)
        self._check_step(q_len, q=q, out=out, caches=(("k_cache", k_cache), ("v_cache", v_cache)),
                         block_table=block_table, seq_lens=seq_lens, tree_mask=tree_mask)
        self._bind(stream, q.device)
        kvattn_decode_tree(self.h, q, k_cache, v_cache, block_table, seq_lens, q_len, tree_mask,
                           out)
        return out

    def append(self, k_new, v_new, k_cache, v_cache, block_table, seq_lens, q_len: int,
               n_sink: int = 0, stream: Optional[torch.cuda.Stream] = None) -> None:
        """Writes the new rows k_new, v_new [batch, q_len, Hkv, D] into the caches."""
        self._check_step(q_len, caches=(("k_cache", k_cache), ("v_cache", v_cache)),
                         block_table=block_table, seq_lens=seq_lens,
                         new_rows=(("k_new", k_new), ("v_new", v_new)))
        self._bind(stream, k_new.device)
        kvattn_append(self.h, k_new, v_new, k_cache, v_cache, block_table, seq_lens, q_len, n_sink)

    def append_decode(self, q, k_new, v_new, k_cache, v_cache, block_table, seq_lens, q_len: int,
                      mask_mode: str = "causal", n_sink: int = 0, window: int = 0, out=None,
                      stream: Optional[torch.cuda.Stream] = None):
        out = self._out(q, out)
        self._check_step(q_len, q=q, out=out, caches=(("k_cache", k_cache), ("v_cache", v_cache)),
                         block_table=block_table, seq_lens=seq_lens,
                         new_rows=(("k_new", k_new), ("v_new", v_new)))
        self._bind(stream, q.device)
        kvattn_append_decode(self.h, q, k_new, v_new, k_cache, v_cache, block_table, seq_lens,
                             q_len, MASK[mask_mode], n_sink, window, out)
        return out

    # ---- test entries: the kernels' own gather code

    def _gather_out(self, q_len, max_slots, device):
        n = self.batch * q_len
        slots = torch.full((n * max(max_slots, 1),), -2, dtype=torch.int32, device=device)
        counts = torch.zeros(n, dtype=torch.int32, device=device)
        return slots, counts

    def debug_gather(self, block_table, seq_lens, q_len: int, mask_mode: str = "causal",
                     n_sink: int = 0, window: int = 0, max_slots: int = 0,
                     stream: Optional[torch.cuda.Stream] = None):
        """Slots [batch, q_len, max(max_slots, 1)] (first max_slots per row) and counts
        [batch, q_len] for the handle's current batch."""
        self._check_step(q_len, block_table=block_table, seq_lens=seq_lens)
        slots, counts = self._gather_out(q_len, max_slots, seq_lens.device)
        self._bind(stream, seq_lens.device)
        kvattn_debug_gather(self.h, block_table, seq_lens, q_len, MASK[mask_mode], n_sink, window,
                            max_slots, slots, counts)
        return slots.view(self.batch, q_len, max(max_slots, 1)), counts.view(self.batch, q_len)

    def debug_gather_tree(self, block_table, seq_lens, q_len: int, tree_mask, max_slots: int,
                          stream: Optional[torch.cuda.Stream] = None):
        self._check_step(q_len, block_table=block_table, seq_lens=seq_lens, tree_mask=tree_mask)
        slots, counts = self._gather_out(q_len, max_slots, seq_lens.device)
        self._bind(stream, seq_lens.device)
        kvattn_debug_gather_tree(self.h, block_table, seq_lens, q_len, tree_mask, max_slots,
                                 slots, counts)
        return slots.view(self.batch, q_len, max(max_slots, 1)), counts.view(self.batch, q_len)
