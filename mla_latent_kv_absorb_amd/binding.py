"""Thin ctypes binding over libmla_absorb.so (declared in include/mla_absorb.h).

Argument marshalling only: shapes are read off torch tensors, outputs and workspace
are allocated with torch on the tensors' device, the call goes to the caller's
current HIP stream, and every step of the computation runs in the library's HIP
kernels.  There is no fallback: if the library cannot be loaded, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmla_absorb.so")

MLA_OK = 0
MLA_ERR_NULL = -1
MLA_ERR_SHAPE = -2
MLA_ERR_DTYPE = -3
MLA_ERR_RANGE = -4
MLA_ERR_ALIGN = -5
MLA_ERR_WORKSPACE = -6
MLA_ERR_HIP = -7
MLA_ERR_UNSUPPORTED = -8

MLA_DTYPE_F32 = 0
MLA_DTYPE_BF16 = 1

PATHS = {"auto": 0, "plain": 1, "mfma": 2}

EXPORTED = ("mla_absorb_attn", "mla_absorb_attn_noalloc", "mla_absorb_attn_ragged", "mla_absorb_attn_paged", "mla_absorb_attn_sparse",
            "mla_absorb_attn_append", "mla_absorb_attn_paged_append",
            "mla_absorb_attn_workspace_size", "mla_absorb_attn_ragged_workspace_size",
            "mla_absorb_attn_paged_workspace_size",
            "mla_absorb_attn_sparse_workspace_size", "mla_cache_append", "mla_cache_append_paged",
            "mla_expand_kv", "mla_expand_kv_workspace_size", "mla_expand_kv_append", "mla_naive_attn",
            "mla_strerror",
            "mla_last_error", "mla_timing_enable", "mla_timing_collect", "mla_kernel_name")

NUM_KERNELS = 7  # MLA_NUM_KERNELS


class AttnShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "batch", "seqlen_q", "n_heads", "kv_lora_rank", "qk_rope_head_dim", "qk_nope_head_dim",
        "v_head_dim", "cache_batch", "cache_len")]


class PagedCache(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("page_size", "num_pages", "max_pages_per_seq")]


class AttnStrides(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "q_nope_row", "q_pe_row", "out_row", "kv_batch", "kv_pos", "pe_batch", "pe_pos")]


class AttnOptions(ctypes.Structure):
    _fields_ = [("num_splits", ctypes.c_int32), ("path", ctypes.c_int32),
                ("strides", ctypes.POINTER(AttnStrides))]


class MLAError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{strerror(status)} ({status}): {detail}")
        self.status = status


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library once; raise if it is missing (nothing here falls back to another path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m mla_latent_kv_absorb_amd.build`")
    # torch ships its own copy of the HIP runtime under the same soname.  Loading torch first makes
    # the library bind to that copy, so that the library and torch share one runtime (streams,
    # current device, loaded code objects); loading the library first would put two runtimes in the
    # process, and the library's would not see torch's device selection.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    lib.mla_absorb_attn.argtypes = [vp, vp, vp, vp, vp, i64, ctypes.c_float, vp, ctypes.POINTER(AttnShape), i32,
                                    ctypes.POINTER(AttnOptions), vp, sz, vp]
    lib.mla_absorb_attn.restype = i32
    lib.mla_absorb_attn_noalloc.argtypes = [vp, vp, vp, vp, vp, i64, ctypes.c_float, vp, ctypes.POINTER(AttnShape),
                                            i32, ctypes.POINTER(AttnOptions), vp]
    lib.mla_absorb_attn_noalloc.restype = i32
    lib.mla_absorb_attn_ragged.argtypes = [vp, vp, vp, vp, vp, vp, i64, ctypes.c_float, vp, ctypes.POINTER(AttnShape),
                                           i32, ctypes.POINTER(AttnOptions), vp, sz, vp]
    lib.mla_absorb_attn_ragged.restype = i32
    lib.mla_absorb_attn_paged.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, ctypes.c_float, vp,
                                          ctypes.POINTER(AttnShape), ctypes.POINTER(PagedCache), i32,
                                          ctypes.POINTER(AttnOptions), vp, sz, vp]
    lib.mla_absorb_attn_paged.restype = i32
    lib.mla_absorb_attn_paged_workspace_size.argtypes = [ctypes.POINTER(AttnShape), i64, ctypes.POINTER(PagedCache),
                                                         i32, ctypes.POINTER(AttnOptions)]
    lib.mla_absorb_attn_paged_workspace_size.restype = sz
    lib.mla_absorb_attn_sparse.argtypes = [vp, vp, vp, vp, vp, vp, i64, vp, i64, ctypes.c_float, vp,
                                           ctypes.POINTER(AttnShape), i32, ctypes.POINTER(AttnOptions), vp, sz, vp]
    lib.mla_absorb_attn_sparse.restype = i32
    lib.mla_absorb_attn_sparse_workspace_size.argtypes = [ctypes.POINTER(AttnShape), i64, i64, i32,
                                                          ctypes.POINTER(AttnOptions)]
    lib.mla_absorb_attn_sparse_workspace_size.restype = sz
    lib.mla_cache_append.argtypes = [vp, vp, vp, ctypes.c_float, vp, i64, vp, vp, ctypes.POINTER(AttnShape), i32, vp]
    lib.mla_cache_append.restype = i32
    lib.mla_cache_append_paged.argtypes = [vp, vp, vp, ctypes.c_float, vp, i64, vp, vp, vp, ctypes.POINTER(AttnShape),
                                           ctypes.POINTER(PagedCache), i32, vp]
    lib.mla_cache_append_paged.restype = i32
    lib.mla_naive_attn.argtypes = [vp, vp, vp, vp, vp, i64, ctypes.c_float, vp, ctypes.POINTER(AttnShape), i32, i32, vp]
    lib.mla_naive_attn.restype = i32
    lib.mla_absorb_attn_workspace_size.argtypes = [ctypes.POINTER(AttnShape), i64, i32, ctypes.POINTER(AttnOptions)]
    lib.mla_absorb_attn_workspace_size.restype = sz
    lib.mla_absorb_attn_ragged_workspace_size.argtypes = [ctypes.POINTER(AttnShape), i64, i32,
                                                          ctypes.POINTER(AttnOptions)]
    lib.mla_absorb_attn_ragged_workspace_size.restype = sz
    lib.mla_expand_kv.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_float, i32, i32, vp, sz, vp]
    lib.mla_expand_kv.restype = i32
    lib.mla_expand_kv_workspace_size.argtypes = [i64, i64, i64, i64, i64, i32, i32]
    lib.mla_expand_kv_workspace_size.restype = sz
    lib.mla_expand_kv_append.argtypes = [vp, vp, vp, vp, ctypes.c_float, i64, vp, vp, vp, ctypes.POINTER(AttnShape),
                                         i32, i32, vp, sz, vp]
    lib.mla_expand_kv_append.restype = i32
    lib.mla_absorb_attn_append.argtypes = [vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp, vp, i64, ctypes.c_float,
                                           vp, ctypes.POINTER(AttnShape), i32, ctypes.POINTER(AttnOptions), vp, sz, vp]
    lib.mla_absorb_attn_append.restype = i32
    lib.mla_absorb_attn_paged_append.argtypes = [vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp, vp, vp, i64,
                                                 ctypes.c_float, vp, ctypes.POINTER(AttnShape),
                                                 ctypes.POINTER(PagedCache), i32, ctypes.POINTER(AttnOptions), vp, sz,
                                                 vp]
    lib.mla_absorb_attn_paged_append.restype = i32
    lib.mla_strerror.argtypes = [i32]
    lib.mla_strerror.restype = ctypes.c_char_p
    lib.mla_last_error.argtypes = []
    lib.mla_last_error.restype = ctypes.c_char_p
    lib.mla_timing_enable.argtypes = [ctypes.c_uint32]
    lib.mla_timing_enable.restype = i32
    lib.mla_timing_collect.argtypes = [ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_double)]
    lib.mla_timing_collect.restype = i32
    lib.mla_kernel_name.argtypes = [i32]
    lib.mla_kernel_name.restype = ctypes.c_char_p
    _lib = lib
    return lib


def strerror(status: int) -> str:
    return load().mla_strerror(status).decode()


def last_error() -> str:
    return load().mla_last_error().decode()


def timing_enable(kernel_mask: int) -> None:
    """Record HIP events around the kernels whose id bit is set (0 turns timing off)."""
    load().mla_timing_enable(kernel_mask)


def timing_collect() -> dict:
    """{kernel name: {"launches": n, "avg_us": mean duration}} since the previous collect."""
    lib = load()
    launches = (ctypes.c_int32 * NUM_KERNELS)()
    ms = (ctypes.c_double * NUM_KERNELS)()
    rc = lib.mla_timing_collect(launches, ms)
    if rc != MLA_OK:
        raise MLAError(rc, "kernel timing events failed")
    return {lib.mla_kernel_name(i).decode(): {"launches": launches[i], "avg_us": ms[i] * 1000.0 / launches[i]}
            for i in range(NUM_KERNELS) if launches[i]}


def _check(status: int) -> None:
    if status != MLA_OK:
        raise MLAError(status, last_error())


def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.float32:
        return MLA_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return MLA_DTYPE_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")


def _stream_handle(device) -> Optional[int]:
    import torch

    return torch.cuda.current_stream(device).cuda_stream


def _require_device(*ts, contiguous: bool = True) -> None:
    dev = ts[0].device
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must live on a GPU device")
        if t.device != dev:
            raise ValueError("all tensors must be on the same device")
        if contiguous and not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
        if t.dtype != ts[0].dtype:
            raise ValueError("all tensors must share one dtype")


def _shape(t, want, name: str) -> None:
    if tuple(t.shape) != tuple(want):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(want)}")


def _row_stride(t, name: str) -> int:
    """Element stride between the evenly spaced rows of a tensor whose leading dimensions all
    step by whole rows (e.g. q[..., :Dn] of a contiguous q); 0 when the rows are dense."""
    if t.stride(-1) != 1 and t.shape[-1] > 1:
        raise ValueError(f"{name}: the innermost dimension must be contiguous")
    rs = None
    step = None
    for d in range(t.dim() - 2, -1, -1):  # innermost leading dimension first
        if t.shape[d] == 1:
            continue
        if rs is None:
            rs, step = t.stride(d), t.stride(d) * t.shape[d]
        elif t.stride(d) != step:
            raise ValueError(f"{name}: rows of the leading dimensions are not evenly spaced")
        else:
            step *= t.shape[d]
    return 0 if rs is None or rs == t.shape[-1] else int(rs)


def _cache_strides(t, name: str):
    """(batch, position) element strides of a [Bmax, Tmax, D] cache view; 0 where dense."""
    if t.stride(2) != 1 and t.shape[2] > 1:
        raise ValueError(f"{name}: the innermost dimension must be contiguous")
    pos = t.stride(1) if t.shape[1] > 1 else t.shape[2]
    bat = t.stride(0) if t.shape[0] > 1 else t.shape[1] * pos
    return (0 if bat == t.shape[1] * pos and pos == t.shape[2] else int(bat), 0 if pos == t.shape[2] else int(pos))


def attn_shape(q_nope, q_pe, kv_cache, wkv_b, pe_cache=None) -> AttnShape:
    """The shape descriptor of an absorb-attention call, with every tensor's shape checked against
    it (the library only sees pointers, so a mismatch must be caught here)."""
    if q_nope.dim() != 4 or q_pe.dim() != 4 or kv_cache.dim() != 3 or wkv_b.dim() != 2:
        raise ValueError("expected q_nope [B,S,H,Dn], q_pe [B,S,H,R], kv_cache [Bmax,Tmax,C], wkv_b [H*(Dn+Dv),C]")
    B, S, H, Dn = q_nope.shape
    R = q_pe.shape[-1]
    Bmax, Tmax, C = kv_cache.shape
    _shape(q_pe, (B, S, H, R), "q_pe")
    if wkv_b.shape[1] != C:
        raise ValueError(f"wkv_b has {wkv_b.shape[1]} columns, kv_cache rows have {C}")
    if wkv_b.shape[0] % H or wkv_b.shape[0] // H <= Dn:
        raise ValueError("wkv_b rows must be n_heads * (qk_nope_head_dim + v_head_dim) with v_head_dim >= 1")
    Dv = wkv_b.shape[0] // H - Dn
    if pe_cache is not None:
        _shape(pe_cache, (Bmax, Tmax, R), "pe_cache")
    return AttnShape(B, S, H, C, R, Dn, Dv, Bmax, Tmax)


def absorb_attn_workspace_size(shape: AttnShape, end_pos: int, dtype: int, num_splits: int = 0,
                               path: str = "auto",
        strides: Optional[AttnStrides] = None) -> int:
    lib = load()
    opt = AttnOptions(num_splits, PATHS[path], None if strides is None else ctypes.pointer(strides))
    n = lib.mla_absorb_attn_workspace_size(ctypes.byref(shape), end_pos, dtype, ctypes.byref(opt))
    if n == 0 and last_error():
        raise MLAError(MLA_ERR_SHAPE, last_error())
    return int(n)


def absorb_attn_ragged_workspace_size(shape: AttnShape, max_seq_len: int, dtype: int, num_splits: int = 0,
                                      path: str = "auto",
        strides: Optional[AttnStrides] = None) -> int:
    lib = load()
    opt = AttnOptions(num_splits, PATHS[path], None if strides is None else ctypes.pointer(strides))
    n = lib.mla_absorb_attn_ragged_workspace_size(ctypes.byref(shape), max_seq_len, dtype, ctypes.byref(opt))
    if n == 0 and last_error():
        raise MLAError(MLA_ERR_SHAPE, last_error())
    return int(n)


def absorb_attn_paged_workspace_size(shape: AttnShape, max_seq_len: int, paged: PagedCache, dtype: int,
                                     num_splits: int = 0, path: str = "auto",
        strides: Optional[AttnStrides] = None) -> int:
    lib = load()
    opt = AttnOptions(num_splits, PATHS[path], None if strides is None else ctypes.pointer(strides))
    n = lib.mla_absorb_attn_paged_workspace_size(ctypes.byref(shape), max_seq_len, ctypes.byref(paged), dtype,
                                                 ctypes.byref(opt))
    if n == 0 and last_error():
        raise MLAError(MLA_ERR_SHAPE, last_error())
    return int(n)


def absorb_attn_sparse_workspace_size(shape: AttnShape, end_pos: int, topk: int, dtype: int, num_splits: int = 0,
                                      path: str = "auto",
        strides: Optional[AttnStrides] = None) -> int:
    lib = load()
    opt = AttnOptions(num_splits, PATHS[path], None if strides is None else ctypes.pointer(strides))
    n = lib.mla_absorb_attn_sparse_workspace_size(ctypes.byref(shape), end_pos, topk, dtype, ctypes.byref(opt))
    if n == 0 and last_error():
        raise MLAError(MLA_ERR_SHAPE, last_error())
    return int(n)


class AbsorbAttnCall:
    """One absorb-attention call with its arguments marshalled once.

    The tensors are validated and their pointers, the shape descriptor and the workspace are
    fixed at construction, together with the HIP stream that is current then; every call of the
    object re-issues mla_absorb_attn with them (for loops that run the same step over and over
    on the same buffers).  The object keeps the tensors alive.
    """

    def __init__(self, q_nope, q_pe, kv_cache, pe_cache, wkv_b, end_pos: int, softmax_scale: float, out=None, *,
                 num_splits: int = 0, path: str = "auto", workspace=None, seq_lens=None, block_table=None,
                 indices=None, append=None):
        """With seq_lens (an int32 tensor [B] on the same device), sequence b attends to positions
        [0, seq_lens[b]) and end_pos is the bound of the lengths (mla_absorb_attn_ragged).  With
        block_table (int32 [B, max_pages_per_seq]), kv_cache and pe_cache are page pools
        [num_pages, page_size, C / R] (mla_absorb_attn_paged; seq_lens optional).  With indices
        (int32 [B, S, topk]), each query token attends to the positions its list names
        (mla_absorb_attn_sparse; seq_lens optional).  With append = (c_kv_new [B, S, C],
        k_pe_new [B, S, R], rms_w [C], eps), every call first writes the new tokens' cache rows
        and then attends (mla_absorb_attn_append / mla_absorb_attn_paged_append)."""
        import torch

        lib = load()
        shape = attn_shape(q_nope, q_pe, kv_cache, wkv_b)
        for name, t in (("seq_lens", seq_lens), ("block_table", block_table), ("indices", indices)):
            if t is not None and (t.device != q_nope.device or t.dtype != torch.int32 or not t.is_contiguous()):
                raise ValueError(f"{name} must be a contiguous int32 tensor on the tensors' device")
        if indices is not None and (indices.dim() != 3 or tuple(indices.shape[:2]) != (shape.batch, shape.seqlen_q)):
            raise ValueError("indices must be [batch, seqlen_q, topk]")
        if seq_lens is not None and seq_lens.numel() != shape.batch:
            raise ValueError("seq_lens must hold one length per sequence")
        paged = None
        if block_table is not None:
            if block_table.dim() != 2 or block_table.shape[0] != shape.batch:
                raise ValueError("block_table must be [batch, max_pages_per_seq]")
            num_pages, page_size = kv_cache.shape[0], kv_cache.shape[1]
            _shape(pe_cache, (num_pages, page_size, shape.qk_rope_head_dim), "pe_cache (page pool)")
            for name, t in (("kv_cache", kv_cache), ("pe_cache", pe_cache)):
                if num_pages > 1 and t.stride(0) != page_size * t.stride(1):
                    raise ValueError(f"{name}: pages of a pool must follow each other at page_size rows")
            paged = PagedCache(page_size, num_pages, block_table.shape[1])
            shape.cache_batch, shape.cache_len = shape.batch, block_table.shape[1] * page_size
        else:
            _shape(pe_cache, (shape.cache_batch, shape.cache_len, shape.qk_rope_head_dim), "pe_cache")
        if out is not None:
            _shape(out, (shape.batch, shape.seqlen_q, shape.n_heads, shape.v_head_dim), "out")
        # q_nope, q_pe, the caches and out may be strided views (evenly spaced rows, contiguous
        # innermost dimension); the weight is dense
        _require_device(q_nope, q_pe, kv_cache, pe_cache, wkv_b, contiguous=False)
        _require_device(wkv_b)
        dt = _dtype_code(q_nope)
        if out is None:
            out = torch.empty((shape.batch, shape.seqlen_q, shape.n_heads, shape.v_head_dim), dtype=q_nope.dtype,
                              device=q_nope.device)
        _require_device(q_nope, out, contiguous=False)
        kv_b, kv_p = _cache_strides(kv_cache, "kv_cache")
        pe_b, pe_p = _cache_strides(pe_cache, "pe_cache")
        strides = AttnStrides(_row_stride(q_nope, "q_nope"), _row_stride(q_pe, "q_pe"), _row_stride(out, "out"),
                              kv_b, kv_p, pe_b, pe_p)
        sp = None if all(getattr(strides, f) == 0 for f, _ in AttnStrides._fields_) else strides
        opt = AttnOptions(num_splits, PATHS[path], None if sp is None else ctypes.pointer(strides))
        if indices is not None:
            if block_table is not None:
                raise ValueError("index lists over paged caches are not supported")
            if indices.dim() != 3 or tuple(indices.shape[:2]) != (shape.batch, shape.seqlen_q):
                raise ValueError("indices must be [batch, seqlen_q, topk]")
            need = absorb_attn_sparse_workspace_size(shape, end_pos, indices.shape[2], dt, num_splits, path, sp)
        elif paged is None and seq_lens is not None:
            need = absorb_attn_ragged_workspace_size(shape, end_pos, dt, num_splits, path, sp)
        elif paged is None:
            need = absorb_attn_workspace_size(shape, end_pos, dt, num_splits, path, sp)
        else:
            need = absorb_attn_paged_workspace_size(shape, end_pos, paged, dt, num_splits, path, sp)
        if append is not None:
            if indices is not None:
                raise ValueError("a fused cache append with index lists is not supported")
            c_kv_new, k_pe_new, rms_w, eps = append
            _shape(c_kv_new, (shape.batch, shape.seqlen_q, shape.kv_lora_rank), "c_kv_new")
            _shape(k_pe_new, (shape.batch, shape.seqlen_q, shape.qk_rope_head_dim), "k_pe_new")
            _shape(rms_w, (shape.kv_lora_rank,), "rms_w")
            _require_device(q_nope, c_kv_new, k_pe_new, rms_w, contiguous=False)
            _require_device(c_kv_new, k_pe_new, rms_w)
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q_nope.device)
        self.out = out
        self._keep = (q_nope, q_pe, kv_cache, pe_cache, wkv_b, out, workspace, shape, opt, strides, seq_lens,
                      block_table, paged, indices, append)
        tail = (softmax_scale, out.data_ptr(), ctypes.byref(shape), dt, ctypes.byref(opt), workspace.data_ptr(),
                workspace.numel() * workspace.element_size(), _stream_handle(q_nope.device))
        head = (q_nope.data_ptr(), q_pe.data_ptr(), kv_cache.data_ptr(), pe_cache.data_ptr(), wkv_b.data_ptr())
        lens_ptr = None if seq_lens is None else seq_lens.data_ptr()
        if append is not None:
            new = (q_nope.data_ptr(), q_pe.data_ptr(), c_kv_new.data_ptr(), k_pe_new.data_ptr(), rms_w.data_ptr(),
                   float(eps), kv_cache.data_ptr(), pe_cache.data_ptr(), wkv_b.data_ptr())
            if paged is not None:
                self._fn = lib.mla_absorb_attn_paged_append
                self._args = new + (block_table.data_ptr(), lens_ptr, end_pos, softmax_scale, out.data_ptr(),
                                    ctypes.byref(shape), ctypes.byref(paged), dt, ctypes.byref(opt),
                                    workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                    _stream_handle(q_nope.device))
            else:
                self._fn = lib.mla_absorb_attn_append
                self._args = new + (lens_ptr, end_pos) + tail
        elif indices is not None:
            self._fn = lib.mla_absorb_attn_sparse
            self._args = head + (indices.data_ptr(), indices.shape[2], lens_ptr, end_pos) + tail
        elif paged is not None:
            self._fn = lib.mla_absorb_attn_paged
            self._args = head + (block_table.data_ptr(), lens_ptr, end_pos, softmax_scale, out.data_ptr(),
                                 ctypes.byref(shape), ctypes.byref(paged), dt, ctypes.byref(opt),
                                 workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                 _stream_handle(q_nope.device))
        elif seq_lens is None:
            self._fn = lib.mla_absorb_attn
            self._args = head + (end_pos,) + tail
        else:
            self._fn = lib.mla_absorb_attn_ragged
            self._args = head + (lens_ptr, end_pos) + tail

    def __call__(self):
        _check(self._fn(*self._args))
        return self.out


def absorb_attn(q_nope, q_pe, kv_cache, pe_cache, wkv_b, end_pos: int, softmax_scale: float, out=None, *,
                num_splits: int = 0, path: str = "auto", workspace=None, seq_lens=None, block_table=None,
                indices=None, append=None):
    """MLA attention in absorb form on torch GPU tensors; returns out [B, S, H, Dv].  With
    seq_lens, a ragged batch whose lengths are bounded by end_pos; with block_table, paged caches
    (kv_cache / pe_cache are the page pools); with indices [B, S, topk], attention over the
    positions each token's list names; with append = (c_kv_new, k_pe_new, rms_w, eps), the new
    tokens' cache rows are written first, in the same call."""
    return AbsorbAttnCall(q_nope, q_pe, kv_cache, pe_cache, wkv_b, end_pos, softmax_scale, out,
                          num_splits=num_splits, path=path, workspace=workspace, seq_lens=seq_lens,
                          block_table=block_table, indices=indices, append=append)()


NOALLOC_SCRATCH_BYTES = 64 << 20  # MLA_NOALLOC_SCRATCH_BYTES


def absorb_attn_noalloc(q_nope, q_pe, kv_cache, pe_cache, wkv_b, end_pos: int, softmax_scale: float, out, *,
                        num_splits: int = 0, path: str = "auto"):
    """mla_absorb_attn_noalloc: the absorb attention of absorb_attn with the library's own scratch
    array as workspace.  `out` is the caller's (nothing is allocated here or in the library)."""
    shape = attn_shape(q_nope, q_pe, kv_cache, wkv_b, pe_cache)
    _shape(out, (shape.batch, shape.seqlen_q, shape.n_heads, shape.v_head_dim), "out")
    _require_device(q_nope, q_pe, kv_cache, pe_cache, wkv_b, out, contiguous=False)
    _require_device(wkv_b)
    kv_b, kv_p = _cache_strides(kv_cache, "kv_cache")
    pe_b, pe_p = _cache_strides(pe_cache, "pe_cache")
    strides = AttnStrides(_row_stride(q_nope, "q_nope"), _row_stride(q_pe, "q_pe"), _row_stride(out, "out"),
                          kv_b, kv_p, pe_b, pe_p)
    dense = all(getattr(strides, f) == 0 for f, _ in AttnStrides._fields_)
    opt = AttnOptions(num_splits, PATHS[path], None if dense else ctypes.pointer(strides))
    _check(load().mla_absorb_attn_noalloc(q_nope.data_ptr(), q_pe.data_ptr(), kv_cache.data_ptr(), pe_cache.data_ptr(),
                                          wkv_b.data_ptr(), end_pos, softmax_scale, out.data_ptr(),
                                          ctypes.byref(shape), _dtype_code(q_nope), ctypes.byref(opt),
                                          _stream_handle(q_nope.device)))
    return out


def cache_append(c_kv_new, k_pe_new, rms_w, eps: float, end_pos: int, kv_cache, pe_cache, *, seq_lens=None,
                 block_table=None):
    """Write the new tokens' normalised latent and rope key into the caches in place
    (mla_cache_append): positions end_pos - S + s, or seq_lens[b] - S + s with seq_lens.  With
    block_table (int32 [B, max_pages_per_seq]), kv_cache and pe_cache are page pools
    [num_pages, page_size, C / R] and end_pos is the bound of the lengths (mla_cache_append_paged)."""
    import torch

    lib = load()
    if c_kv_new.dim() != 3 or k_pe_new.dim() != 3 or kv_cache.dim() != 3:
        raise ValueError("expected c_kv_new [B,S,C], k_pe_new [B,S,R], kv_cache [Bmax,Tmax,C] (or pools)")
    B, S, C = c_kv_new.shape
    R = k_pe_new.shape[-1]
    Bmax, Tmax, _ = kv_cache.shape
    _shape(k_pe_new, (B, S, R), "k_pe_new")
    _shape(rms_w, (C,), "rms_w")
    _shape(kv_cache, (Bmax, Tmax, C), "kv_cache")
    _shape(pe_cache, (Bmax, Tmax, R), "pe_cache")
    _require_device(c_kv_new, k_pe_new, rms_w, kv_cache, pe_cache)
    shape = AttnShape(B, S, 1, C, R, 0, 0, Bmax, Tmax)
    lens_ptr = None
    if seq_lens is not None:
        if seq_lens.device != c_kv_new.device or seq_lens.dtype != torch.int32 or seq_lens.numel() != B:
            raise ValueError("seq_lens must be an int32 tensor [B] on the tensors' device")
        lens_ptr = seq_lens.data_ptr()
    if block_table is None:
        _check(lib.mla_cache_append(c_kv_new.data_ptr(), k_pe_new.data_ptr(), rms_w.data_ptr(), eps, lens_ptr,
                                    end_pos, kv_cache.data_ptr(), pe_cache.data_ptr(), ctypes.byref(shape),
                                    _dtype_code(c_kv_new), _stream_handle(c_kv_new.device)))
        return
    if (block_table.device != c_kv_new.device or block_table.dtype != torch.int32 or block_table.dim() != 2
            or block_table.shape[0] != B or not block_table.is_contiguous()):
        raise ValueError("block_table must be a contiguous int32 tensor [B, max_pages_per_seq] on the tensors' device")
    paged = PagedCache(Tmax, Bmax, block_table.shape[1])  # pools: [num_pages, page_size, .]
    _check(lib.mla_cache_append_paged(c_kv_new.data_ptr(), k_pe_new.data_ptr(), rms_w.data_ptr(), eps, lens_ptr,
                                      end_pos, block_table.data_ptr(), kv_cache.data_ptr(), pe_cache.data_ptr(),
                                      ctypes.byref(shape), ctypes.byref(paged), _dtype_code(c_kv_new),
                                      _stream_handle(c_kv_new.device)))


class NaiveAttnCall:
    """One naive-route attention call (mla_naive_attn) with its arguments marshalled once, over
    expanded keys and values: k_nope [H, Bmax, Tmax, Dn] and v [H, Bmax, Tmax, Dv] head-major,
    pe_cache [Bmax, Tmax, R].  Every call of the object re-issues it on the stream current at
    construction; the object keeps the tensors alive."""

    def __init__(self, q_nope, q_pe, k_nope, v, pe_cache, end_pos: int, softmax_scale: float, out=None, *,
                 path: str = "auto"):
        import torch

        lib = load()
        if q_nope.dim() != 4 or q_pe.dim() != 4 or k_nope.dim() != 4 or v.dim() != 4 or pe_cache.dim() != 3:
            raise ValueError("expected q_nope/q_pe [B,S,H,.], k_nope/v [H,Bmax,Tmax,.], pe_cache [Bmax,Tmax,R]")
        B, S, H, Dn = q_nope.shape
        R = q_pe.shape[-1]
        Hk, Bmax, Tmax, Dk = k_nope.shape
        Dv = v.shape[-1]
        _shape(q_pe, (B, S, H, R), "q_pe")
        if Hk != H or Dk != Dn or tuple(v.shape[:3]) != (H, Bmax, Tmax) or tuple(pe_cache.shape) != (Bmax, Tmax, R):
            raise ValueError("k_nope / v / pe_cache shapes disagree with the query")
        if out is not None:
            _shape(out, (B, S, H, Dv), "out")
        _require_device(q_nope, q_pe, k_nope, v, pe_cache)
        if out is None:
            out = torch.empty((B, S, H, Dv), dtype=q_nope.dtype, device=q_nope.device)
        _require_device(q_nope, out)
        shape = AttnShape(B, S, H, 0, R, Dn, Dv, Bmax, Tmax)
        self.out = out
        self._keep = (q_nope, q_pe, k_nope, v, pe_cache, out, shape)
        self._fn = lib.mla_naive_attn
        self._args = (q_nope.data_ptr(), q_pe.data_ptr(), k_nope.data_ptr(), v.data_ptr(), pe_cache.data_ptr(),
                      end_pos, softmax_scale, out.data_ptr(), ctypes.byref(shape), _dtype_code(q_nope), PATHS[path],
                      _stream_handle(q_nope.device))

    def __call__(self):
        _check(self._fn(*self._args))
        return self.out


def naive_attn(q_nope, q_pe, k_nope, v, pe_cache, end_pos: int, softmax_scale: float, out=None, *,
               path: str = "auto"):
    """Naive-route attention over expanded keys and values (mla_naive_attn); see NaiveAttnCall.
    Returns out [B, S, H, Dv]."""
    return NaiveAttnCall(q_nope, q_pe, k_nope, v, pe_cache, end_pos, softmax_scale, out, path=path)()


def expand_kv_workspace_size(n_tokens: int, n_heads: int, kv_lora_rank: int, qk_nope_head_dim: int,
                             v_head_dim: int, dtype: int, path: str = "auto") -> int:
    lib = load()
    n = lib.mla_expand_kv_workspace_size(n_tokens, n_heads, kv_lora_rank, qk_nope_head_dim, v_head_dim, dtype,
                                         PATHS[path])
    if n == 0 and last_error():
        raise MLAError(MLA_ERR_SHAPE, last_error())
    return int(n)


def expand_kv(c_kv, rms_w, wkv_b, n_heads: int, qk_nope_head_dim: int, v_head_dim: int, eps: float = 1e-6,
              k_nope=None, v=None, *, path: str = "auto", workspace=None) -> Tuple["object", "object"]:
    """Latent KV expansion with split; returns (k_nope [H, T, Dn], v [H, T, Dv])."""
    import torch

    lib = load()
    if c_kv.dim() != 2:
        raise ValueError("c_kv must be [n_tokens, kv_lora_rank]")
    T, C = c_kv.shape
    _shape(rms_w, (C,), "rms_w")
    _shape(wkv_b, (n_heads * (qk_nope_head_dim + v_head_dim), C), "wkv_b")
    if k_nope is not None:
        _shape(k_nope, (n_heads, T, qk_nope_head_dim), "k_nope")
    if v is not None:
        _shape(v, (n_heads, T, v_head_dim), "v")
    _require_device(c_kv, rms_w, wkv_b)
    if k_nope is None:
        k_nope = torch.empty((n_heads, T, qk_nope_head_dim), dtype=c_kv.dtype, device=c_kv.device)
    if v is None:
        v = torch.empty((n_heads, T, v_head_dim), dtype=c_kv.dtype, device=c_kv.device)
    _require_device(c_kv, k_nope, v)
    dt = _dtype_code(c_kv)
    need = expand_kv_workspace_size(T, n_heads, C, qk_nope_head_dim, v_head_dim, dt, path)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=c_kv.device)
    ws_ptr = workspace.data_ptr() if need else None
    ws_bytes = workspace.numel() * workspace.element_size() if need else 0
    rc = lib.mla_expand_kv(c_kv.data_ptr(), rms_w.data_ptr(), wkv_b.data_ptr(), k_nope.data_ptr(), v.data_ptr(),
                           T, n_heads, C, qk_nope_head_dim, v_head_dim, eps, dt, PATHS[path], ws_ptr, ws_bytes,
                           _stream_handle(c_kv.device))
    _check(rc)
    return k_nope, v


class ExpandAppendCall:
    """One naive-route cache append (mla_expand_kv_append) with its arguments marshalled once: the
    new tokens' keys and values, expanded through wkv_b, into the full-width head-major caches
    k_cache [H, Bmax, Tmax, Dn] / v_cache [H, Bmax, Tmax, Dv] at positions end_pos - S + s, and
    their rope keys into pe_cache [Bmax, Tmax, R] (k_pe_new and pe_cache: both or neither).  Every
    call of the object re-issues the append on the stream current at construction."""

    def __init__(self, c_kv_new, k_pe_new, rms_w, wkv_b, eps: float, end_pos: int, k_cache, v_cache, pe_cache, *,
                 path: str = "auto", workspace=None):
        import torch

        lib = load()
        if c_kv_new.dim() != 3 or k_cache.dim() != 4 or v_cache.dim() != 4:
            raise ValueError("expected c_kv_new [B,S,C], k_cache [H,Bmax,Tmax,Dn], v_cache [H,Bmax,Tmax,Dv]")
        if (k_pe_new is None) != (pe_cache is None):
            raise ValueError("k_pe_new and pe_cache go together")
        B, S, C = c_kv_new.shape
        H, Bmax, Tmax, Dn = k_cache.shape
        Dv = v_cache.shape[3]
        R = k_pe_new.shape[-1] if k_pe_new is not None else (pe_cache.shape[-1] if pe_cache is not None else 64)
        _shape(rms_w, (C,), "rms_w")
        _shape(wkv_b, (H * (Dn + Dv), C), "wkv_b")
        _shape(v_cache, (H, Bmax, Tmax, Dv), "v_cache")
        tensors = [c_kv_new, rms_w, wkv_b, k_cache, v_cache]
        if k_pe_new is not None:
            _shape(k_pe_new, (B, S, R), "k_pe_new")
            _shape(pe_cache, (Bmax, Tmax, R), "pe_cache")
            tensors += [k_pe_new, pe_cache]
        _require_device(*tensors)
        dt = _dtype_code(c_kv_new)
        shape = AttnShape(B, S, H, C, R, Dn, Dv, Bmax, Tmax)
        need = expand_kv_workspace_size(B * S, H, C, Dn, Dv, dt, path)
        if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
            workspace = torch.empty(need, dtype=torch.uint8, device=c_kv_new.device)
        self._keep = (c_kv_new, k_pe_new, rms_w, wkv_b, k_cache, v_cache, pe_cache, workspace, shape)
        self._fn = lib.mla_expand_kv_append
        self._args = (c_kv_new.data_ptr(), None if k_pe_new is None else k_pe_new.data_ptr(), rms_w.data_ptr(),
                      wkv_b.data_ptr(), eps, end_pos, k_cache.data_ptr(), v_cache.data_ptr(),
                      None if pe_cache is None else pe_cache.data_ptr(), ctypes.byref(shape), dt, PATHS[path],
                      workspace.data_ptr() if need else None,
                      workspace.numel() * workspace.element_size() if need else 0, _stream_handle(c_kv_new.device))

    def __call__(self):
        _check(self._fn(*self._args))


def expand_kv_append(c_kv_new, k_pe_new, rms_w, wkv_b, eps: float, end_pos: int, k_cache, v_cache, pe_cache, *,
                     path: str = "auto", workspace=None):
    """The naive path's cache append (mla_expand_kv_append), in place; see ExpandAppendCall."""
    ExpandAppendCall(c_kv_new, k_pe_new, rms_w, wkv_b, eps, end_pos, k_cache, v_cache, pe_cache, path=path,
                     workspace=workspace)()
