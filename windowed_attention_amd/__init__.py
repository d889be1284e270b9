"""Python binding of the MI355X R-SWA library (librswa.so).

Argument marshalling only: every step of the path runs in the HIP kernels behind the C ABI of
include/rswa.h. torch supplies device memory and the stream (torch's current stream unless one is
given). Importing this module fails loudly if the library has not been built.

Functions carry the C names (rswa_cache_create, rswa_append_kv, rswa_decode_attn,
rswa_prefill_attn, ...); `RswaCache` wraps the cache handle.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "librswa.so")

BF16, F32 = 0, 1
MODE_RSWA, MODE_FULL_CAUSAL = 0, 1
STATUS = {0: "RSWA_OK", -1: "RSWA_E_INVALID", -2: "RSWA_E_UNSUPPORTED", -3: "RSWA_E_CAPACITY",
          -4: "RSWA_E_OOM", -5: "RSWA_E_HIP", -6: "RSWA_E_INTERNAL"}

# Every symbol include/rswa.h declares.
EXPORTS = ("rswa_cache_plan", "rswa_cache_bytes", "rswa_cache_create", "rswa_cache_create_paged",
           "rswa_append_kv",
           "rswa_decode_attn", "rswa_decode_step", "rswa_prefill_attn", "rswa_prefill_fwd",
           "rswa_prefill_bwd", "rswa_cache_steps", "rswa_cache_info",
           "rswa_cache_set_decode_split", "rswa_cache_decode_plan", "rswa_cache_destroy",
           "rswa_cache_create_from_prefill",
           "rswa_step_graph_create", "rswa_step_graph_launch", "rswa_step_graph_destroy",
           "rswa_cache_query", "rswa_prefill_check", "rswa_prefill_bwd_noalloc",
           "rswa_status_str",
           "rswa_last_error")


class RswaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


class CacheDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
                ("mode", ctypes.c_int32), ("prefix_len", ctypes.POINTER(ctypes.c_int32)),
                ("window", ctypes.POINTER(ctypes.c_int32)),
                ("max_steps", ctypes.POINTER(ctypes.c_int32)),
                ("storage_dev", ctypes.c_void_p), ("storage_bytes", ctypes.c_uint64),
                ("prefix_paged", ctypes.c_int32)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; "
            f"g.build()'` (hipcc, gfx950). There is no fallback path.")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, u64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64, ctypes.c_float
    pi32, pi64 = ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)
    pdesc = ctypes.POINTER(CacheDesc)
    sig = {
        "rswa_cache_plan": (i32, [pdesc, pi64, pi32, ctypes.POINTER(u64)]),
        "rswa_cache_bytes": (u64, [pdesc]),
        "rswa_cache_create": (i32, [pdesc, vp, vp, vp, ctypes.POINTER(vp)]),
        "rswa_cache_create_paged": (i32, [pdesc, vp, vp, ctypes.c_int64, vp, vp,
                                          ctypes.POINTER(vp)]),
        "rswa_cache_create_from_prefill": (i32, [pdesc, vp, vp, pi32, vp, ctypes.POINTER(vp)]),
        "rswa_append_kv": (i32, [vp, vp, vp, vp, vp]),
        "rswa_decode_attn": (i32, [vp, vp, vp, i32, f32, vp, vp]),
        "rswa_decode_step": (i32, [vp, vp, vp, vp, vp, i32, f32, vp, vp]),
        "rswa_prefill_attn": (i32, [vp, vp, vp, vp, i32, vp, vp, vp, i32, i32, i32, i32, i32, f32,
                                    vp]),
        "rswa_prefill_fwd": (i32, [vp, vp, vp, vp, i32, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                   f32, vp]),
        "rswa_prefill_bwd": (i32, [vp, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp,
                                   i32, i32, i32, i32, i32, i32, f32, vp]),
        "rswa_cache_steps": (i32, [vp, pi32, vp]),
        "rswa_cache_info": (i32, [vp, ctypes.POINTER(vp), pi64, pi32]),
        "rswa_cache_set_decode_split": (i32, [vp, i32, i32]),
        "rswa_cache_decode_plan": (i32, [vp, i32, pi32, pi32]),
        "rswa_cache_destroy": (i32, [vp]),
        "rswa_step_graph_create": (i32, [vp, i32, vp, vp, vp, vp, i32, f32, ctypes.POINTER(vp)]),
        "rswa_step_graph_launch": (i32, [vp, vp]),
        "rswa_step_graph_destroy": (i32, [vp]),
        "rswa_cache_query": (i32, [vp, ctypes.POINTER(vp), pi64, pi64, pi32, pi32, vp]),
        "rswa_prefill_bwd_noalloc": (i32, [vp, vp, vp, vp, i32, vp, vp, vp, vp, vp, i32, vp, vp,
                                           vp, i32, i32, i32, i32, i32, i32, f32, vp]),
        "rswa_prefill_check": (i32, [vp]),
        "rswa_status_str": (ctypes.c_char_p, [i32]),
        "rswa_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def _check(status: int, what: str) -> None:
    if status != 0:
        detail = _lib.rswa_last_error().decode()
        raise RswaError(status, f"{what}: {STATUS.get(status, status)} ({detail})")


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return BF16
    if dt == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {dt}: use torch.bfloat16 or torch.float32")


def _torch_dtype(code: int) -> torch.dtype:
    return torch.bfloat16 if code == BF16 else torch.float32


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t: torch.Tensor | None, name: str, dtype=None, shape=None) -> ctypes.c_void_p:
    if t is None:
        return ctypes.c_void_p(None)
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _i32_array(x, n: int, name: str):
    arr = np.ascontiguousarray(np.asarray(x, dtype=np.int32).reshape(-1))
    if arr.size != n:
        raise ValueError(f"{name} must have {n} entries")
    return arr, arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _desc(prefix_len, window, max_steps, num_heads, head_dim, kv_dtype, mode, storage=None,
          paged=False):
    m = np.ascontiguousarray(np.asarray(prefix_len, dtype=np.int32).reshape(-1))
    B = m.size
    keep = [m]
    d = CacheDesc()
    d.batch, d.num_heads, d.head_dim = B, num_heads, head_dim
    d.kv_dtype, d.mode = _dtype_code(kv_dtype), mode
    d.prefix_len = m.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    if window is not None:
        w, d.window = _i32_array(window, B, "window")
        keep.append(w)
    if max_steps is not None:
        s, d.max_steps = _i32_array(max_steps, B, "max_steps")
        keep.append(s)
    if storage is not None:
        d.storage_dev = storage.data_ptr()
        d.storage_bytes = storage.numel() * storage.element_size()
    d.prefix_paged = int(bool(paged))
    return d, keep


def rswa_cache_plan(prefix_len, window=None, max_steps=None, *, num_heads=16, head_dim=128,
                    kv_dtype=torch.bfloat16, mode=MODE_RSWA, paged=False):
    """Host-only layout: (seq_offset elements [B] int64, rows [B] int32, storage bytes)."""
    d, keep = _desc(prefix_len, window, max_steps, num_heads, head_dim, kv_dtype, mode,
                    paged=paged)
    B = d.batch
    off = np.zeros(max(B, 1), dtype=np.int64)
    rows = np.zeros(max(B, 1), dtype=np.int32)
    nbytes = ctypes.c_uint64(0)
    _check(_lib.rswa_cache_plan(ctypes.byref(d), off.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                ctypes.byref(nbytes)), "rswa_cache_plan")
    return off[:B], rows[:B], int(nbytes.value)


def rswa_cache_bytes(prefix_len, window=None, max_steps=None, *, num_heads=16, head_dim=128,
                     kv_dtype=torch.bfloat16, mode=MODE_RSWA, paged=False) -> int:
    d, keep = _desc(prefix_len, window, max_steps, num_heads, head_dim, kv_dtype, mode,
                    paged=paged)
    return int(_lib.rswa_cache_bytes(ctypes.byref(d)))


class RswaCache:
    """A batch of B decode sequences: static prefix rows plus an n-slot ring per sequence
    (mode MODE_RSWA) or a growing cache (MODE_FULL_CAUSAL).

    With `pool_k`, `pool_v` ([pool_rows][H][D]) and `prefix_table` (int32 [sum m_b], device) the
    prefixes are not copied: sequence b's prefix token j is pool row prefix_table[M_b + j]
    (rswa_cache_create_paged); prefix_k / prefix_v must then be None. The pools must stay alive
    and unchanged while the cache is used (the object keeps a reference).

    With `prefill_k`, `prefill_v` ([total][H][D]) and `cu_seqlens` (host sequence of B + 1 ints)
    the cache is filled from a packed prefill batch (rswa_cache_create_from_prefill): segment b
    holds sequence b's prefix then its outputs so far, and decoding continues after them."""

    def __init__(self, prefix_k: torch.Tensor | None, prefix_v: torch.Tensor | None, prefix_len,
                 window=None, *, mode=MODE_RSWA, max_steps=None, num_heads=16, head_dim=128,
                 kv_dtype=None, storage: torch.Tensor | None = None, pool_k=None, pool_v=None,
                 prefix_table=None, prefill_k=None, prefill_v=None, cu_seqlens=None, stream=None):
        m = np.asarray(prefix_len, dtype=np.int64).reshape(-1)
        paged = prefix_table is not None
        filled = cu_seqlens is not None
        if kv_dtype is None:
            src = pool_k if paged else (prefill_k if filled else prefix_k)
            if src is None:
                raise ValueError("kv_dtype is required when there is no prefix tensor")
            kv_dtype = src.dtype
        total_m = int(m.sum())
        if storage is not None:
            _dev(storage, "storage")
        d, keep = _desc(m, window, max_steps, num_heads, head_dim, kv_dtype, mode, storage,
                        paged=paged)
        h = ctypes.c_void_p(None)
        if filled:
            if paged or prefix_k is not None or prefix_v is not None:
                raise ValueError("a cache filled from a prefill takes prefill_k / prefill_v only")
            cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32).reshape(-1))
            if cu.size != m.size + 1:
                raise ValueError(f"cu_seqlens must have {m.size + 1} entries")
            total = int(prefill_k.shape[0])
            if cu.size and int(cu[-1]) > total:
                raise ValueError(f"cu_seqlens ends at row {int(cu[-1])} but prefill_k holds "
                                 f"{total} rows")
            shape = (total, num_heads, head_dim)
            _check(_lib.rswa_cache_create_from_prefill(
                ctypes.byref(d), _dev(prefill_k, "prefill_k", kv_dtype, shape),
                _dev(prefill_v, "prefill_v", kv_dtype, shape),
                cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), _stream(stream),
                ctypes.byref(h)), "rswa_cache_create_from_prefill")
        elif paged:
            if prefix_k is not None or prefix_v is not None:
                raise ValueError("a paged cache takes pool_k / pool_v, not prefix_k / prefix_v")
            rows = int(pool_k.shape[0])
            pshape = (rows, num_heads, head_dim)
            _check(_lib.rswa_cache_create_paged(
                ctypes.byref(d), _dev(pool_k, "pool_k", kv_dtype, pshape),
                _dev(pool_v, "pool_v", kv_dtype, pshape), rows,
                _dev(prefix_table, "prefix_table", torch.int32, (total_m,)), _stream(stream),
                ctypes.byref(h)), "rswa_cache_create_paged")
        else:
            shape = (total_m, num_heads, head_dim)
            pk = _dev(prefix_k, "prefix_k", kv_dtype, shape) if prefix_k is not None else None
            pv = _dev(prefix_v, "prefix_v", kv_dtype, shape) if prefix_v is not None else None
            _check(_lib.rswa_cache_create(ctypes.byref(d), pk or ctypes.c_void_p(None),
                                          pv or ctypes.c_void_p(None), _stream(stream),
                                          ctypes.byref(h)), "rswa_cache_create")
        self._h = h
        self._storage = storage
        self._pools = (pool_k, pool_v, prefix_table) if paged else None
        self.batch = int(m.size)
        self.num_heads = num_heads
        self.head_dim = head_dim
        self.kv_dtype = kv_dtype
        self.mode = mode
        self.prefix_len = m.astype(np.int32)

    @property
    def handle(self) -> ctypes.c_void_p:
        if self._h is None:
            raise RuntimeError("cache has been destroyed")
        return self._h

    def _bhd(self):
        return (self.batch, self.num_heads, self.head_dim)

    def append(self, k: torch.Tensor, v: torch.Tensor, active: torch.Tensor | None = None,
               stream=None) -> None:
        rswa_append_kv(self, k, v, active, stream)

    def decode(self, q: torch.Tensor, out: torch.Tensor | None = None,
               out_dtype: torch.dtype = torch.float32, scale: float = 0.0,
               active: torch.Tensor | None = None, stream=None) -> torch.Tensor:
        if out is None:
            out = torch.empty(self._bhd(), dtype=out_dtype, device=q.device)
        rswa_decode_attn(self, q, out, scale, active, stream)
        return out

    def step(self, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
             out: torch.Tensor | None = None, out_dtype: torch.dtype = torch.float32,
             scale: float = 0.0, active: torch.Tensor | None = None, stream=None) -> torch.Tensor:
        """Append (k, v) and attend with q in one launch (same result as append + decode)."""
        if out is None:
            out = torch.empty(self._bhd(), dtype=out_dtype, device=q.device)
        rswa_decode_step(self, q, k, v, out, scale, active, stream)
        return out

    def steps(self, stream=None) -> np.ndarray:
        s = np.zeros(self.batch, dtype=np.int32)
        _check(_lib.rswa_cache_steps(self.handle, s.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                     _stream(stream)), "rswa_cache_steps")
        return s

    def info(self):
        p = ctypes.c_void_p(None)
        off = np.zeros(self.batch, dtype=np.int64)
        rows = np.zeros(self.batch, dtype=np.int32)
        _check(_lib.rswa_cache_info(self.handle, ctypes.byref(p),
                                    off.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                    rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))),
               "rswa_cache_info")
        return p.value, off, rows

    def query(self, stream=None):
        """(storage pointer, K element offsets [B], V element offsets [B], rows [B], t_b [B]);
        blocks until `stream` has passed all prior work."""
        p = ctypes.c_void_p(None)
        ko = np.zeros(self.batch, dtype=np.int64)
        vo = np.zeros(self.batch, dtype=np.int64)
        rows = np.zeros(self.batch, dtype=np.int32)
        st = np.zeros(self.batch, dtype=np.int32)
        _check(_lib.rswa_cache_query(self.handle, ctypes.byref(p),
                                     ko.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                     vo.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                     rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                     st.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                     _stream(stream)), "rswa_cache_query")
        return p.value, ko, vo, rows, st

    def set_decode_split(self, chunk_rows: int = 0, grid_blocks: int = 0) -> None:
        _check(_lib.rswa_cache_set_decode_split(self.handle, chunk_rows, grid_blocks),
               "rswa_cache_set_decode_split")

    def decode_plan(self, appending: bool = True):
        """(workgroups, launches) of the next decode launch without an active mask."""
        g, n = ctypes.c_int32(0), ctypes.c_int32(0)
        _check(_lib.rswa_cache_decode_plan(self.handle, int(appending), ctypes.byref(g),
                                           ctypes.byref(n)), "rswa_cache_decode_plan")
        return g.value, n.value

    def close(self) -> None:
        if getattr(self, "_h", None) is not None:
            _check(_lib.rswa_cache_destroy(self._h), "rswa_cache_destroy")
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


def rswa_cache_create(prefix_k, prefix_v, prefix_len, window=None, **kw) -> RswaCache:
    return RswaCache(prefix_k, prefix_v, prefix_len, window, **kw)


def rswa_cache_create_from_prefill(k, v, cu_seqlens, prefix_len, window=None,
                                   **kw) -> RswaCache:
    """Cache filled from a packed prefill batch k / v ([total][H][D]): segment b of the host
    sequence cu_seqlens holds prefix_len[b] prefix rows then that sequence's outputs so far."""
    return RswaCache(None, None, prefix_len, window, prefill_k=k, prefill_v=v,
                     cu_seqlens=cu_seqlens, **kw)


def rswa_append_kv(cache: RswaCache, k: torch.Tensor, v: torch.Tensor,
                   active: torch.Tensor | None = None, stream=None) -> None:
    shape = cache._bhd()
    _check(_lib.rswa_append_kv(cache.handle, _dev(k, "k", cache.kv_dtype, shape),
                               _dev(v, "v", cache.kv_dtype, shape),
                               _dev(active, "active", torch.uint8, (cache.batch,)),
                               _stream(stream)), "rswa_append_kv")


def rswa_decode_attn(cache: RswaCache, q: torch.Tensor, out: torch.Tensor, scale: float = 0.0,
                     active: torch.Tensor | None = None, stream=None) -> None:
    shape = cache._bhd()
    _check(_lib.rswa_decode_attn(cache.handle, _dev(q, "q", cache.kv_dtype, shape),
                                 _dev(out, "out", None, shape), _dtype_code(out.dtype),
                                 ctypes.c_float(scale),
                                 _dev(active, "active", torch.uint8, (cache.batch,)),
                                 _stream(stream)), "rswa_decode_attn")


def rswa_decode_step(cache: RswaCache, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                     out: torch.Tensor, scale: float = 0.0, active: torch.Tensor | None = None,
                     stream=None) -> None:
    shape = cache._bhd()
    _check(_lib.rswa_decode_step(cache.handle, _dev(q, "q", cache.kv_dtype, shape),
                                 _dev(k, "k", cache.kv_dtype, shape),
                                 _dev(v, "v", cache.kv_dtype, shape),
                                 _dev(out, "out", None, shape), _dtype_code(out.dtype),
                                 ctypes.c_float(scale),
                                 _dev(active, "active", torch.uint8, (cache.batch,)),
                                 _stream(stream)), "rswa_decode_step")


def rswa_cache_destroy(cache: RswaCache) -> None:
    cache.close()


def rswa_prefill_attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: torch.Tensor,
                      prefix_len: torch.Tensor, window: torch.Tensor, *, out=None,
                      out_dtype: torch.dtype = torch.float32, prefix_causal: bool = False,
                      scale: float = 0.0, max_seqlen: int | None = None,
                      stream=None) -> torch.Tensor:
    """R-SWA-masked attention over packed sequences; q/k/v [total][H][D] bf16 on the device,
    cu_seqlens / prefix_len / window int32 device tensors. max_seqlen defaults to the largest
    sequence (computed on the host from cu_seqlens, which costs a device sync; the sequences are
    then also checked to fit the rows of q)."""
    total, H, D = q.shape
    nseq = prefix_len.numel()
    max_seqlen = _max_seqlen(cu_seqlens, max_seqlen, total)
    if out is None:
        out = torch.empty((total, H, D), dtype=out_dtype, device=q.device)
    shape = (total, H, D)
    _check(_lib.rswa_prefill_attn(
        _dev(q, "q", torch.bfloat16, shape), _dev(k, "k", torch.bfloat16, shape),
        _dev(v, "v", torch.bfloat16, shape), _dev(out, "out", None, shape),
        _dtype_code(out.dtype), _dev(cu_seqlens, "cu_seqlens", torch.int32, (nseq + 1,)),
        _dev(prefix_len, "prefix_len", torch.int32, (nseq,)),
        _dev(window, "window", torch.int32, (nseq,)), nseq, H, D, int(max_seqlen),
        int(bool(prefix_causal)), ctypes.c_float(scale), _stream(stream)), "rswa_prefill_attn")
    return out


class StepGraph:
    """`steps` fused decode steps of a cache captured in a HIP graph (rswa_step_graph_create).
    Before each replay, write step i's q / k / v into slot i of `q`, `k`, `v` ([steps][B][H][D]);
    the outputs land in slot i of `out`."""

    def __init__(self, cache: "RswaCache", steps: int, out_dtype: torch.dtype = torch.float32,
                 scale: float = 0.0):
        shape = (steps, cache.batch, cache.num_heads, cache.head_dim)
        dev = torch.device("cuda", torch.cuda.current_device())
        self.q = torch.zeros(shape, dtype=cache.kv_dtype, device=dev)
        self.k = torch.zeros_like(self.q)
        self.v = torch.zeros_like(self.q)
        self.out = torch.zeros(shape, dtype=out_dtype, device=dev)
        self.cache = cache
        self.steps = steps
        h = ctypes.c_void_p(None)
        _check(_lib.rswa_step_graph_create(cache.handle, steps, _dev(self.q, "q"), _dev(self.k, "k"),
                                           _dev(self.v, "v"), _dev(self.out, "out"),
                                           _dtype_code(out_dtype), ctypes.c_float(scale),
                                           ctypes.byref(h)), "rswa_step_graph_create")
        self._h = h

    def launch(self, stream=None) -> None:
        _check(_lib.rswa_step_graph_launch(self._h, _stream(stream)), "rswa_step_graph_launch")

    def close(self) -> None:
        if self._h is not None:
            torch.cuda.synchronize()
            _lib.rswa_step_graph_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _max_seqlen(cu_seqlens: torch.Tensor, max_seqlen: int | None, total: int) -> int:
    """max_seqlen as given, else the longest sequence of cu_seqlens (a host copy, which costs a
    device sync); with that copy also checks that the sequences fit the `total` rows of q/k/v,
    which the kernels cannot check."""
    if max_seqlen is not None:
        return int(max_seqlen)
    cs = cu_seqlens.cpu().numpy()
    if cs.size and int(cs[-1]) > total:
        raise ValueError(f"cu_seqlens ends at row {int(cs[-1])} but q/k/v hold {total} rows")
    return int(np.diff(cs).max()) if cs.size > 1 else 0


def rswa_prefill_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: torch.Tensor,
                     prefix_len: torch.Tensor, window: torch.Tensor, *, out=None, lse=None,
                     out_dtype: torch.dtype = torch.bfloat16, prefix_causal: bool = False,
                     scale: float = 0.0, max_seqlen: int | None = None, stream=None):
    """Training forward: rswa_prefill_attn plus the natural log-sum-exp per (token, head).
    Returns (out [total][H][D], lse [total][H] float32)."""
    total, H, D = q.shape
    nseq = prefix_len.numel()
    max_seqlen = _max_seqlen(cu_seqlens, max_seqlen, total)
    if out is None:
        out = torch.empty((total, H, D), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((total, H), dtype=torch.float32, device=q.device)
    shape = (total, H, D)
    _check(_lib.rswa_prefill_fwd(
        _dev(q, "q", torch.bfloat16, shape), _dev(k, "k", torch.bfloat16, shape),
        _dev(v, "v", torch.bfloat16, shape), _dev(out, "out", None, shape),
        _dtype_code(out.dtype), _dev(lse, "lse", torch.float32, (total, H)),
        _dev(cu_seqlens, "cu_seqlens", torch.int32, (nseq + 1,)),
        _dev(prefix_len, "prefix_len", torch.int32, (nseq,)),
        _dev(window, "window", torch.int32, (nseq,)), nseq, H, D, max_seqlen,
        int(bool(prefix_causal)), ctypes.c_float(scale), _stream(stream)), "rswa_prefill_fwd")
    return out, lse


def rswa_prefill_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
                     dout: torch.Tensor, lse: torch.Tensor, cu_seqlens: torch.Tensor,
                     prefix_len: torch.Tensor, window: torch.Tensor, *, dq=None, dk=None, dv=None,
                     work=None, grad_dtype: torch.dtype = torch.float32,
                     prefix_causal: bool = False, scale: float = 0.0,
                     max_seqlen: int | None = None, stream=None):
    """Gradients (dq, dk, dv) of the R-SWA-masked prefill; dout bf16 [total][H][D], out and lse
    from rswa_prefill_fwd. `work` ([2][H][total] float32) is a work array, allocated if absent."""
    total, H, D = q.shape
    nseq = prefix_len.numel()
    max_seqlen = _max_seqlen(cu_seqlens, max_seqlen, total)
    shape = (total, H, D)
    mk = lambda t: torch.empty(shape, dtype=grad_dtype, device=q.device) if t is None else t
    dq, dk, dv = mk(dq), mk(dk), mk(dv)
    if work is None:
        work = torch.empty((2, H, total), dtype=torch.float32, device=q.device)
    if not (dq.dtype == dk.dtype == dv.dtype):
        raise TypeError("dq, dk and dv must share one dtype")
    _check(_lib.rswa_prefill_bwd(
        _dev(q, "q", torch.bfloat16, shape), _dev(k, "k", torch.bfloat16, shape),
        _dev(v, "v", torch.bfloat16, shape), _dev(out, "out", None, shape),
        _dtype_code(out.dtype), _dev(dout, "dout", torch.bfloat16, shape),
        _dev(lse, "lse", torch.float32, (total, H)), _dev(work, "work", torch.float32, (2, H, total)),
        _dev(dq, "dq", None, shape), _dev(dk, "dk", None, shape), _dev(dv, "dv", None, shape),
        _dtype_code(dq.dtype), _dev(cu_seqlens, "cu_seqlens", torch.int32, (nseq + 1,)),
        _dev(prefix_len, "prefix_len", torch.int32, (nseq,)),
        _dev(window, "window", torch.int32, (nseq,)), nseq, total, H, D, max_seqlen,
        int(bool(prefix_causal)), ctypes.c_float(scale), _stream(stream)), "rswa_prefill_bwd")
    return dq, dk, dv


def rswa_prefill_bwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                             out: torch.Tensor, dout: torch.Tensor, lse: torch.Tensor,
                             cu_seqlens: torch.Tensor, prefix_len: torch.Tensor,
                             window: torch.Tensor, *, dq, dk, dv, prefix_causal: bool = False,
                             scale: float = 0.0, max_seqlen: int, stream=None):
    """rswa_prefill_bwd without a work array (the library's device-resident one is used); the
    gradient tensors must be given. Allocates nothing."""
    total, H, D = q.shape
    nseq = prefix_len.numel()
    shape = (total, H, D)
    if not (dq.dtype == dk.dtype == dv.dtype):
        raise TypeError("dq, dk and dv must share one dtype")
    _check(_lib.rswa_prefill_bwd_noalloc(
        _dev(q, "q", torch.bfloat16, shape), _dev(k, "k", torch.bfloat16, shape),
        _dev(v, "v", torch.bfloat16, shape), _dev(out, "out", None, shape),
        _dtype_code(out.dtype), _dev(dout, "dout", torch.bfloat16, shape),
        _dev(lse, "lse", torch.float32, (total, H)),
        _dev(dq, "dq", None, shape), _dev(dk, "dk", None, shape), _dev(dv, "dv", None, shape),
        _dtype_code(dq.dtype), _dev(cu_seqlens, "cu_seqlens", torch.int32, (nseq + 1,)),
        _dev(prefix_len, "prefix_len", torch.int32, (nseq,)),
        _dev(window, "window", torch.int32, (nseq,)), nseq, total, H, D, int(max_seqlen),
        int(bool(prefix_causal)), ctypes.c_float(scale), _stream(stream)),
        "rswa_prefill_bwd_noalloc")
    return dq, dk, dv


def rswa_prefill_check(stream=None) -> None:
    """Raise RswaError if a prefill / backward launch on the current device found bad sequence
    metadata on the device since the last check (blocks until `stream` is idle)."""
    _check(_lib.rswa_prefill_check(_stream(stream)), "rswa_prefill_check")


def status_str(code: int) -> str:
    return _lib.rswa_status_str(code).decode()
