"""C-ABI checks that need no GPU: the library loads, exports what include/mla_absorb.h declares,
and rejects bad arguments before any HIP call (so these calls never touch a device)."""
import ctypes
import os
import re

import pytest

from mla_latent_kv_absorb_amd import binding as B

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "mla_absorb.h")

# Fake, 16-byte-aligned device addresses.  Every call below fails validation before any kernel
# could be enqueued, so they are never dereferenced.
P = [0x7f0000000000 + i * 0x100000000 for i in range(8)]


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        import __graft_entry__

        __graft_entry__.build()
    return B.load()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?(?:char\s*\*|size_t|int32_t)\s*\**\s*(mla_\w+)\s*\(", text, re.M)))


def test_header_declares_the_binding_names():
    assert declared_functions() == sorted(B.EXPORTED)


def test_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_strerror_covers_codes(lib):
    for code in range(0, -9, -1):
        assert B.strerror(code) and B.strerror(code) != "unknown status"
    assert B.strerror(-99) == "unknown status"


def shape(**kw):
    d = dict(batch=2, seqlen_q=1, n_heads=128, kv_lora_rank=512, qk_rope_head_dim=64, qk_nope_head_dim=128,
             v_head_dim=128, cache_batch=2, cache_len=4096)
    d.update(kw)
    return B.AttnShape(*[d[f] for f, _ in B.AttnShape._fields_])


def call_attn(lib, s, end_pos=4096, dtype=B.MLA_DTYPE_BF16, ptrs=None, ws=P[7], ws_bytes=1 << 40, scale=0.07,
              opt=None):
    p = list(P[:6]) if ptrs is None else ptrs
    o = ctypes.byref(opt) if opt is not None else None
    return lib.mla_absorb_attn(p[0], p[1], p[2], p[3], p[4], end_pos, scale, p[5], ctypes.byref(s), dtype, o, ws,
                               ws_bytes, None)


def test_workspace_size_query(lib):
    n = B.absorb_attn_workspace_size(shape(), 4096, B.MLA_DTYPE_BF16)
    assert n > 0
    n32 = B.absorb_attn_workspace_size(shape(n_heads=4, kv_lora_rank=64, qk_rope_head_dim=16, qk_nope_head_dim=32,
                                             v_head_dim=32, batch=1, cache_batch=1, cache_len=128), 128,
                                       B.MLA_DTYPE_F32)
    assert n32 > 0
    bad = lib.mla_absorb_attn_workspace_size(ctypes.byref(shape(batch=3)), 4096, B.MLA_DTYPE_BF16, None)
    assert bad == 0 and "batch" in B.last_error()


@pytest.mark.parametrize("kw,end_pos,code,needle", [
    (dict(batch=3), 4096, B.MLA_ERR_RANGE, "batch"),
    ({}, 4097, B.MLA_ERR_RANGE, "end_pos"),
    ({}, 0, B.MLA_ERR_RANGE, "end_pos"),
    (dict(seqlen_q=5), 4, B.MLA_ERR_RANGE, "seqlen_q"),
    (dict(n_heads=0), 4096, B.MLA_ERR_SHAPE, "n_heads"),
    (dict(kv_lora_rank=-1), 4096, B.MLA_ERR_SHAPE, "kv_lora_rank"),
    (dict(kv_lora_rank=500), 4096, B.MLA_ERR_ALIGN, "multiples"),
])
def test_attn_shape_errors(lib, kw, end_pos, code, needle):
    assert call_attn(lib, shape(**kw), end_pos=end_pos) == code
    assert needle in B.last_error()


def test_attn_pointer_errors(lib):
    s = shape()
    for i in range(6):
        p = list(P[:6])
        p[i] = None
        assert call_attn(lib, s, ptrs=p) == B.MLA_ERR_NULL
        p[i] = P[i] + 2
        assert call_attn(lib, s, ptrs=p) == B.MLA_ERR_ALIGN
    assert lib.mla_absorb_attn(*P[:5], 4096, 0.07, P[5], None, B.MLA_DTYPE_BF16, None, P[7], 1 << 40,
                               None) == B.MLA_ERR_NULL


def test_attn_dtype_scale_and_options(lib):
    s = shape()
    assert call_attn(lib, s, dtype=7) == B.MLA_ERR_DTYPE
    assert call_attn(lib, s, scale=0.0) == B.MLA_ERR_SHAPE
    assert call_attn(lib, s, scale=float("nan")) == B.MLA_ERR_SHAPE
    assert call_attn(lib, s, opt=B.AttnOptions(-1, 0)) == B.MLA_ERR_SHAPE
    assert call_attn(lib, s, opt=B.AttnOptions(0, 9)) == B.MLA_ERR_UNSUPPORTED
    fp32 = shape(n_heads=4, kv_lora_rank=64, qk_rope_head_dim=16, qk_nope_head_dim=32, v_head_dim=32)
    assert call_attn(lib, fp32, dtype=B.MLA_DTYPE_F32, end_pos=128,
                     opt=B.AttnOptions(0, B.PATHS["mfma"])) == B.MLA_ERR_UNSUPPORTED


def test_attn_workspace_errors(lib):
    s = shape()
    need = B.absorb_attn_workspace_size(s, 4096, B.MLA_DTYPE_BF16)
    assert call_attn(lib, s, ws=None) == B.MLA_ERR_WORKSPACE
    assert call_attn(lib, s, ws_bytes=need - 1) == B.MLA_ERR_WORKSPACE
    assert call_attn(lib, s, ws=P[7] + 8) == B.MLA_ERR_ALIGN
    # workspace on top of kv_cache
    assert call_attn(lib, s, ws=P[2] + 4096) == B.MLA_ERR_WORKSPACE


def test_attn_out_alias(lib):
    p = list(P[:6])
    p[5] = P[2] + 1024  # out inside kv_cache
    assert call_attn(lib, shape(), ptrs=p) == B.MLA_ERR_SHAPE
    assert "overlaps" in B.last_error()


def call_expand(lib, T=64, H=128, C=512, Dn=128, Dv=128, eps=1e-6, dtype=B.MLA_DTYPE_BF16, ptrs=None, path=0,
                ws=None, ws_bytes=None):
    p = list(P[:5]) if ptrs is None else ptrs
    if ws is None:
        ws = P[6]
    if ws_bytes is None:
        ws_bytes = 1 << 30
    return lib.mla_expand_kv(p[0], p[1], p[2], p[3], p[4], T, H, C, Dn, Dv, eps, dtype, path, ws, ws_bytes, None)


def test_expand_errors(lib):
    assert call_expand(lib, T=0) == B.MLA_ERR_SHAPE
    assert call_expand(lib, C=511) == B.MLA_ERR_ALIGN
    assert call_expand(lib, dtype=3) == B.MLA_ERR_DTYPE
    assert call_expand(lib, eps=-1.0) == B.MLA_ERR_SHAPE
    assert call_expand(lib, path=5) == B.MLA_ERR_UNSUPPORTED
    for i in range(5):
        p = list(P[:5])
        p[i] = None
        assert call_expand(lib, ptrs=p) == B.MLA_ERR_NULL
        p[i] = P[i] + 4
        assert call_expand(lib, ptrs=p) == B.MLA_ERR_ALIGN
    p = list(P[:5])
    p[4] = P[3] + 64  # v inside k_nope
    assert call_expand(lib, ptrs=p) == B.MLA_ERR_SHAPE
    assert call_expand(lib, dtype=B.MLA_DTYPE_F32, C=64, H=4, Dn=32, Dv=32, path=B.PATHS["mfma"]) == \
        B.MLA_ERR_UNSUPPORTED


def test_expand_workspace(lib):
    need = lib.mla_expand_kv_workspace_size(64, 128, 512, 128, 128, B.MLA_DTYPE_BF16, B.PATHS["mfma"])
    assert need >= 64 * 512 * 2
    assert lib.mla_expand_kv_workspace_size(64, 128, 512, 128, 128, B.MLA_DTYPE_BF16, B.PATHS["plain"]) == 0
    assert lib.mla_expand_kv_workspace_size(0, 128, 512, 128, 128, B.MLA_DTYPE_BF16, 0) == 0 and B.last_error()
    assert call_expand(lib, ws=None, ws_bytes=0, path=B.PATHS["mfma"]) == B.MLA_ERR_WORKSPACE
    assert call_expand(lib, ws_bytes=need - 1, path=B.PATHS["mfma"]) == B.MLA_ERR_WORKSPACE
    assert call_expand(lib, ws=P[6] + 4, path=B.PATHS["mfma"]) == B.MLA_ERR_ALIGN
    assert call_expand(lib, ws=P[0], path=B.PATHS["mfma"]) == B.MLA_ERR_WORKSPACE  # overlaps c_kv


def call_expand_append(lib, s, end_pos=4096, eps=1e-6, dtype=B.MLA_DTYPE_BF16, ptrs=None, path=0, ws=P[7],
                       ws_bytes=1 << 40):
    p = list(P[:7]) if ptrs is None else ptrs
    return lib.mla_expand_kv_append(p[0], p[1], p[2], p[3], eps, end_pos, p[4], p[5], p[6], ctypes.byref(s), dtype,
                                    path, ws, ws_bytes, None)


def test_expand_append_argument_errors(lib):
    s = shape(seqlen_q=512)
    assert lib.mla_expand_kv_append(*P[:4], 1e-6, 4096, *P[4:7], None, B.MLA_DTYPE_BF16, 0, P[7], 1 << 40,
                                    None) == B.MLA_ERR_NULL
    assert call_expand_append(lib, s, end_pos=4097) == B.MLA_ERR_RANGE
    assert call_expand_append(lib, s, end_pos=511) == B.MLA_ERR_RANGE  # S > end_pos
    assert call_expand_append(lib, shape(batch=3)) == B.MLA_ERR_RANGE
    assert call_expand_append(lib, shape(n_heads=0)) == B.MLA_ERR_SHAPE
    assert call_expand_append(lib, s, eps=-1.0) == B.MLA_ERR_SHAPE
    assert call_expand_append(lib, s, dtype=4) == B.MLA_ERR_DTYPE
    assert call_expand_append(lib, s, path=9) == B.MLA_ERR_UNSUPPORTED
    assert call_expand_append(lib, shape(kv_lora_rank=500)) == B.MLA_ERR_ALIGN
    assert call_expand_append(lib, shape(qk_rope_head_dim=4)) == B.MLA_ERR_ALIGN
    # the rope rows go together: a rope source without a rope cache (and the reverse) is refused
    for i in (1, 6):
        p = list(P[:7])
        p[i] = None
        assert call_expand_append(lib, s, ptrs=p) == B.MLA_ERR_NULL and "k_pe_new" in B.last_error()
    for i in (0, 2, 3, 4, 5):
        p = list(P[:7])
        p[i] = None
        assert call_expand_append(lib, s, ptrs=p) == B.MLA_ERR_NULL
    for i in range(7):
        p = list(P[:7])
        p[i] = P[i] + 2
        assert call_expand_append(lib, s, ptrs=p) == B.MLA_ERR_ALIGN
    # the caches must not overlap each other, the new rows or the workspace
    p = list(P[:7])
    p[5] = P[4] + 4096  # v_cache inside k_cache
    assert call_expand_append(lib, s, ptrs=p) == B.MLA_ERR_SHAPE
    p = list(P[:7])
    p[6] = P[0] + 1024  # pe_cache inside c_kv_new
    assert call_expand_append(lib, s, ptrs=p) == B.MLA_ERR_SHAPE
    need = lib.mla_expand_kv_workspace_size(2 * 512, 128, 512, 128, 128, B.MLA_DTYPE_BF16, B.PATHS["mfma"])
    assert need >= 2 * 512 * 512 * 2
    mfma = B.PATHS["mfma"]
    assert call_expand_append(lib, s, path=mfma, ws=None, ws_bytes=0) == B.MLA_ERR_WORKSPACE
    assert call_expand_append(lib, s, path=mfma, ws_bytes=need - 1) == B.MLA_ERR_WORKSPACE
    assert call_expand_append(lib, s, path=mfma, ws=P[4] + 256) == B.MLA_ERR_WORKSPACE  # inside k_cache
    # the matrix-core kernels take bf16 and at most 2^23 cache rows per head
    assert call_expand_append(lib, s, path=mfma, dtype=B.MLA_DTYPE_F32) == B.MLA_ERR_UNSUPPORTED
    big = shape(seqlen_q=512, cache_batch=2049, cache_len=4096)
    assert call_expand_append(lib, big, path=mfma) == B.MLA_ERR_UNSUPPORTED and "rows" in B.last_error()
    # caches whose element count would overflow the size arithmetic are refused outright
    huge = shape(seqlen_q=512, n_heads=1 << 20, cache_batch=1 << 20, cache_len=1 << 20)
    assert call_expand_append(lib, huge) == B.MLA_ERR_SHAPE


def call_ragged(lib, s, lens, max_len=4096, ws=P[7], ws_bytes=1 << 40, out=None):
    p = list(P[:6])
    return lib.mla_absorb_attn_ragged(p[0], p[1], p[2], p[3], p[4], lens, max_len, 0.07, p[5] if out is None else out,
                                      ctypes.byref(s), B.MLA_DTYPE_BF16, None, ws, ws_bytes, None)


def test_ragged_argument_errors(lib):
    s = shape()
    lens = P[6]
    assert call_ragged(lib, s, None) == B.MLA_ERR_NULL and "seq_lens" in B.last_error()
    assert call_ragged(lib, s, lens + 2) == B.MLA_ERR_ALIGN and "seq_lens" in B.last_error()
    # the bound plays end_pos's role in validation
    assert call_ragged(lib, s, lens, max_len=4097) == B.MLA_ERR_RANGE
    assert call_ragged(lib, shape(seqlen_q=8), lens, max_len=4) == B.MLA_ERR_RANGE
    # outputs and workspace must not overlap the lengths (4-byte aligned is enough for them)
    assert call_ragged(lib, s, lens + 4, ws=lens - 1024) == B.MLA_ERR_WORKSPACE
    assert call_ragged(lib, s, P[5] + 64) == B.MLA_ERR_SHAPE and "seq_lens" in B.last_error()


def call_append(lib, s, end_pos=4096, ptrs=None, eps=1e-6, lens=None, dtype=B.MLA_DTYPE_BF16):
    p = list(P[:5]) if ptrs is None else ptrs
    return lib.mla_cache_append(p[0], p[1], p[2], eps, lens, end_pos, p[3], p[4], ctypes.byref(s), dtype, None)


def test_cache_append_argument_errors(lib):
    s = shape()
    assert lib.mla_cache_append(*P[:3], 1e-6, None, 4096, P[3], P[4], None, B.MLA_DTYPE_BF16, None) == B.MLA_ERR_NULL
    assert call_append(lib, s, end_pos=4097) == B.MLA_ERR_RANGE
    assert call_append(lib, shape(seqlen_q=9), end_pos=8) == B.MLA_ERR_RANGE
    assert call_append(lib, shape(batch=3)) == B.MLA_ERR_RANGE
    assert call_append(lib, s, eps=-1.0) == B.MLA_ERR_SHAPE
    assert call_append(lib, s, dtype=5) == B.MLA_ERR_DTYPE
    assert call_append(lib, shape(kv_lora_rank=500)) == B.MLA_ERR_ALIGN
    for i in range(5):
        p = list(P[:5])
        p[i] = None
        assert call_append(lib, s, ptrs=p) == B.MLA_ERR_NULL
        p[i] = P[i] + 2
        assert call_append(lib, s, ptrs=p) == B.MLA_ERR_ALIGN
    assert call_append(lib, s, lens=P[6] + 2) == B.MLA_ERR_ALIGN
    # the caches must not overlap each other or the new rows
    assert call_append(lib, s, ptrs=[P[0], P[1], P[2], P[3], P[3] + 4096]) == B.MLA_ERR_SHAPE
    assert call_append(lib, s, ptrs=[P[3] + 1024, P[1], P[2], P[3], P[4]]) == B.MLA_ERR_SHAPE


# new-token rows of the fused append (fake, aligned, apart from P)
A = [0x7e0000000000 + i * 0x100000000 for i in range(3)]


def call_attn_append(lib, s, end_pos=4096, ptrs=None, aptrs=None, eps=1e-6, lens=None, dtype=B.MLA_DTYPE_BF16,
                     ws=P[7], ws_bytes=1 << 40):
    p = list(P[:6]) if ptrs is None else ptrs
    a = list(A) if aptrs is None else aptrs
    return lib.mla_absorb_attn_append(p[0], p[1], a[0], a[1], a[2], eps, p[2], p[3], p[4], lens, end_pos, 0.07, p[5],
                                      ctypes.byref(s), dtype, None, ws, ws_bytes, None)


def test_attn_append_argument_errors(lib):
    s = shape()
    # the attention's own checks
    assert call_attn_append(lib, s, end_pos=4097) == B.MLA_ERR_RANGE
    assert call_attn_append(lib, shape(seqlen_q=9), end_pos=8) == B.MLA_ERR_RANGE
    assert call_attn_append(lib, s, dtype=5) == B.MLA_ERR_DTYPE
    assert call_attn_append(lib, s, ws=None) == B.MLA_ERR_WORKSPACE
    # the append's
    assert call_attn_append(lib, s, eps=-1.0) == B.MLA_ERR_SHAPE
    assert call_attn_append(lib, s, eps=float("nan")) == B.MLA_ERR_SHAPE
    for i in range(3):
        a = list(A)
        a[i] = None
        assert call_attn_append(lib, s, aptrs=a) == B.MLA_ERR_NULL
        a[i] = A[i] + 2
        assert call_attn_append(lib, s, aptrs=a) == B.MLA_ERR_ALIGN
    assert call_attn_append(lib, s, lens=P[6] + 2) == B.MLA_ERR_ALIGN
    # the caches are written: nothing else the call reads may overlap them
    assert call_attn_append(lib, s, ptrs=[P[2] + 4096, P[1], P[2], P[3], P[4], P[5]]) == B.MLA_ERR_SHAPE  # q_nope
    assert call_attn_append(lib, s, ptrs=[P[0], P[1], P[2], P[3], P[3] + 1024, P[5]]) == B.MLA_ERR_SHAPE  # wkv_b
    assert call_attn_append(lib, s, ptrs=[P[0], P[1], P[2], P[2] + 4096, P[4], P[5]]) == B.MLA_ERR_SHAPE  # pe in kv
    assert call_attn_append(lib, s, aptrs=[P[2] + 1024, A[1], A[2]]) == B.MLA_ERR_SHAPE  # new rows in kv
    assert call_attn_append(lib, s, aptrs=[A[0], A[1], P[3] + 1024]) == B.MLA_ERR_SHAPE  # rms_w in pe
    assert call_attn_append(lib, s, lens=P[2] + 1024) == B.MLA_ERR_SHAPE  # seq_lens in kv
    assert call_attn_append(lib, s, ptrs=[P[0], P[1], P[2], P[3], P[4], A[1]]) == B.MLA_ERR_SHAPE  # out on k_pe_new
    assert call_attn_append(lib, s, ws=A[0]) == B.MLA_ERR_WORKSPACE  # workspace on c_kv_new


def test_attn_paged_append_argument_errors(lib):
    s = shape()
    pg = B.PagedCache(64, 256, 64)

    def call(p=None, a=None, bt=P[6], paged=pg, lens=None, eps=1e-6):
        p = list(P[:6]) if p is None else p
        a = list(A) if a is None else a
        return lib.mla_absorb_attn_paged_append(p[0], p[1], a[0], a[1], a[2], eps, p[2], p[3], p[4], bt, lens, 4096,
                                                0.07, p[5], ctypes.byref(s), None if paged is None else ctypes.byref(paged),
                                                B.MLA_DTYPE_BF16, None, P[7], 1 << 40, None)

    assert call(paged=None) == B.MLA_ERR_NULL
    assert call(bt=None) == B.MLA_ERR_NULL
    assert call(bt=P[6] + 2) == B.MLA_ERR_ALIGN
    assert call(eps=2.0) == B.MLA_ERR_SHAPE
    assert call(bt=P[2] + 4096) == B.MLA_ERR_SHAPE  # the table inside the kv pool, which is written
    assert call(a=[A[0], P[3] + 64, A[2]]) == B.MLA_ERR_SHAPE  # new rope rows inside the pe pool


def call_naive(lib, s, end_pos=4096, ptrs=None, scale=0.07, dtype=B.MLA_DTYPE_BF16, path=B.PATHS["auto"]):
    p = list(P[:6]) if ptrs is None else ptrs
    return lib.mla_naive_attn(p[0], p[1], p[2], p[3], p[4], end_pos, scale, p[5], ctypes.byref(s), dtype, path, None)


def test_naive_attn_argument_errors(lib):
    s = shape()
    assert lib.mla_naive_attn(*P[:5], 4096, 0.07, P[5], None, B.MLA_DTYPE_BF16, 0, None) == B.MLA_ERR_NULL
    assert call_naive(lib, s, end_pos=4097) == B.MLA_ERR_RANGE
    assert call_naive(lib, s, end_pos=0) == B.MLA_ERR_RANGE
    assert call_naive(lib, shape(seqlen_q=9), end_pos=8) == B.MLA_ERR_RANGE
    assert call_naive(lib, shape(batch=3)) == B.MLA_ERR_RANGE
    assert call_naive(lib, shape(n_heads=0)) == B.MLA_ERR_SHAPE
    assert call_naive(lib, s, scale=0.0) == B.MLA_ERR_SHAPE
    assert call_naive(lib, s, scale=float("nan")) == B.MLA_ERR_SHAPE
    assert call_naive(lib, s, dtype=5) == B.MLA_ERR_DTYPE
    assert call_naive(lib, s, path=7) == B.MLA_ERR_UNSUPPORTED
    assert call_naive(lib, shape(v_head_dim=100)) == B.MLA_ERR_ALIGN
    # the matrix-core kernel is for the bf16 DeepSeek-V3 head shape only
    assert call_naive(lib, s, dtype=B.MLA_DTYPE_F32, path=B.PATHS["mfma"]) == B.MLA_ERR_UNSUPPORTED
    assert call_naive(lib, shape(qk_nope_head_dim=64), path=B.PATHS["mfma"]) == B.MLA_ERR_UNSUPPORTED
    assert call_naive(lib, shape(qk_rope_head_dim=128), path=B.PATHS["mfma"]) == B.MLA_ERR_UNSUPPORTED
    for i in range(6):
        p = list(P[:6])
        p[i] = None
        assert call_naive(lib, s, ptrs=p) == B.MLA_ERR_NULL
        p[i] = P[i] + 2
        assert call_naive(lib, s, ptrs=p) == B.MLA_ERR_ALIGN
    for i in range(5):  # out overlapping any input
        p = list(P[:6])
        p[5] = P[i] + 4096
        assert call_naive(lib, s, ptrs=p) == B.MLA_ERR_SHAPE


def call_paged(lib, s, max_len=4096, ptrs=None, bt=P[6], lens=None, pg=None, path=B.PATHS["auto"], splits=0,
               ws=P[7], ws_bytes=1 << 40):
    p = list(P[:6]) if ptrs is None else ptrs
    pg = B.PagedCache(64, 256, 64) if pg is None else pg
    opt = B.AttnOptions(splits, path)
    return lib.mla_absorb_attn_paged(p[0], p[1], p[2], p[3], p[4], bt, lens, max_len, 0.07, p[5], ctypes.byref(s),
                                     ctypes.byref(pg), B.MLA_DTYPE_BF16, ctypes.byref(opt), ws, ws_bytes, None)


def test_paged_argument_errors(lib):
    s = shape()
    opt = B.AttnOptions(0, 0)
    assert lib.mla_absorb_attn_paged(*P[:5], P[6], None, 4096, 0.07, P[5], ctypes.byref(s), None, B.MLA_DTYPE_BF16,
                                     ctypes.byref(opt), P[7], 1 << 40, None) == B.MLA_ERR_NULL
    assert call_paged(lib, s, bt=None) == B.MLA_ERR_NULL
    assert call_paged(lib, s, bt=P[6] + 2) == B.MLA_ERR_ALIGN
    assert call_paged(lib, s, lens=P[6] + 4096 + 2) == B.MLA_ERR_ALIGN
    assert call_paged(lib, s, pg=B.PagedCache(0, 256, 64)) == B.MLA_ERR_SHAPE
    assert call_paged(lib, s, pg=B.PagedCache(64, 0, 64)) == B.MLA_ERR_SHAPE
    assert call_paged(lib, s, pg=B.PagedCache(64, 256, 0)) == B.MLA_ERR_SHAPE
    # capacity max_pages_per_seq * page_size bounds max_seq_len; shape's cache fields are not used
    assert call_paged(lib, s, max_len=4097) == B.MLA_ERR_RANGE
    assert call_paged(lib, shape(cache_batch=1, cache_len=1), max_len=4097) == B.MLA_ERR_RANGE
    assert call_paged(lib, s, max_len=0) == B.MLA_ERR_RANGE
    # the matrix-core kernels need a power-of-two page of at least 32 positions
    for bad in (16, 48, 100):
        pg = B.PagedCache(bad, 4096, 4096 // bad + 1)
        assert call_paged(lib, s, pg=pg, path=B.PATHS["mfma"]) == B.MLA_ERR_UNSUPPORTED
    # out, workspace, block_table and seq_lens must not overlap
    assert call_paged(lib, s, bt=P[5] + 64) == B.MLA_ERR_SHAPE
    assert call_paged(lib, s, bt=P[7] + 64) == B.MLA_ERR_WORKSPACE
    assert call_paged(lib, s, lens=P[5] + 64) == B.MLA_ERR_SHAPE
    assert call_paged(lib, s, ws_bytes=16) == B.MLA_ERR_WORKSPACE


def test_paged_workspace_and_split_plan(lib):
    s = shape(batch=32)
    pg = B.PagedCache(64, 32 * 64, 64)
    # at the decode shape the paged size is that of the ragged (balanced) contiguous plan, which
    # provides more split slots than the uniform plan; a forced split count is not balanced
    dense = B.absorb_attn_workspace_size(shape(batch=32, cache_batch=32), 4096, B.MLA_DTYPE_BF16)
    ragged = B.absorb_attn_ragged_workspace_size(shape(batch=32, cache_batch=32), 4096, B.MLA_DTYPE_BF16)
    assert B.absorb_attn_paged_workspace_size(s, 4096, pg, B.MLA_DTYPE_BF16) == ragged > dense
    assert B.absorb_attn_ragged_workspace_size(shape(batch=32, cache_batch=32), 4096, B.MLA_DTYPE_BF16, num_splits=8) \
        == B.absorb_attn_workspace_size(shape(batch=32, cache_batch=32), 4096, B.MLA_DTYPE_BF16, num_splits=8)
    # the plain path plans the same with or without lengths
    assert B.absorb_attn_ragged_workspace_size(shape(batch=32, cache_batch=32), 4096, B.MLA_DTYPE_BF16,
                                               path="plain") == \
        B.absorb_attn_workspace_size(shape(batch=32, cache_batch=32), 4096, B.MLA_DTYPE_BF16, path="plain")
    # one split over 16384 positions spans more pages of 32 than a workgroup keeps: refused on the
    # matrix-core path, planned with more splits by default
    one = shape(batch=1, seqlen_q=512, n_heads=128, cache_batch=1, cache_len=16384)
    pg32 = B.PagedCache(32, 512, 512)
    with pytest.raises(B.MLAError):
        B.absorb_attn_paged_workspace_size(one, 16384, pg32, B.MLA_DTYPE_BF16, num_splits=1, path="mfma")
    ws = {p: B.absorb_attn_paged_workspace_size(one, 16384, B.PagedCache(p, 16384 // p, 16384 // p),
                                                B.MLA_DTYPE_BF16, path="mfma") for p in (32, 64, 128)}
    assert ws[32] > ws[64] > ws[128] == B.absorb_attn_ragged_workspace_size(one, 16384, B.MLA_DTYPE_BF16, path="mfma")


def call_sparse(lib, s, end_pos=4096, ptrs=None, idx=P[6], topk=2048, lens=None, path=B.PATHS["auto"], splits=0,
                ws=P[7], ws_bytes=1 << 40):
    p = list(P[:6]) if ptrs is None else ptrs
    opt = B.AttnOptions(splits, path)
    return lib.mla_absorb_attn_sparse(p[0], p[1], p[2], p[3], p[4], idx, topk, lens, end_pos, 0.07, p[5],
                                      ctypes.byref(s), B.MLA_DTYPE_BF16, ctypes.byref(opt), ws, ws_bytes, None)


def test_sparse_argument_errors(lib):
    s = shape()
    assert call_sparse(lib, s, idx=None) == B.MLA_ERR_NULL
    assert call_sparse(lib, s, idx=P[6] + 2) == B.MLA_ERR_ALIGN
    assert call_sparse(lib, s, lens=P[6] + (1 << 20) + 2) == B.MLA_ERR_ALIGN
    assert call_sparse(lib, s, topk=0) == B.MLA_ERR_SHAPE
    assert call_sparse(lib, s, topk=(1 << 24) + 1) == B.MLA_ERR_SHAPE
    assert call_sparse(lib, s, end_pos=4097) == B.MLA_ERR_RANGE
    assert call_sparse(lib, shape(seqlen_q=9), end_pos=8) == B.MLA_ERR_RANGE
    # a matrix-core workgroup's 128 rows must be the heads of one token
    assert call_sparse(lib, shape(seqlen_q=2, n_heads=64), path=B.PATHS["mfma"]) == B.MLA_ERR_UNSUPPORTED
    assert call_sparse(lib, shape(seqlen_q=1, n_heads=192), path=B.PATHS["mfma"]) == B.MLA_ERR_UNSUPPORTED
    # a forced split may hold at most 256 list entries on the matrix-core path
    assert call_sparse(lib, s, splits=1, topk=257, path=B.PATHS["mfma"]) == B.MLA_ERR_UNSUPPORTED
    # out, workspace, indices and seq_lens must not overlap
    assert call_sparse(lib, s, idx=P[5] + 64) == B.MLA_ERR_SHAPE
    assert call_sparse(lib, s, idx=P[7] + 64) == B.MLA_ERR_WORKSPACE
    assert call_sparse(lib, s, ws_bytes=16) == B.MLA_ERR_WORKSPACE
    for i in range(6):
        p = list(P[:6])
        p[i] = None
        assert call_sparse(lib, s, ptrs=p) == B.MLA_ERR_NULL


def test_sparse_workspace_plan(lib):
    # splits cut the list entries: 2048 entries of 32 decode tokens plan like 2048 positions
    s = shape(batch=32, cache_batch=32)
    assert B.absorb_attn_sparse_workspace_size(s, 4096, 2048, B.MLA_DTYPE_BF16) == \
        B.absorb_attn_workspace_size(s, 2048, B.MLA_DTYPE_BF16)
    # one token with a long list: at least topk / 256 splits on the matrix-core path
    one = shape(batch=1, seqlen_q=1, cache_batch=1, cache_len=65536)
    few = B.absorb_attn_sparse_workspace_size(one, 65536, 256, B.MLA_DTYPE_BF16, path="mfma")
    many = B.absorb_attn_sparse_workspace_size(one, 65536, 65536, B.MLA_DTYPE_BF16, path="mfma")
    assert many > few


def call_append_paged(lib, s, max_len=4096, ptrs=None, bt=P[6], lens=None, pg=None, eps=1e-6):
    p = list(P[:5]) if ptrs is None else ptrs
    pg = B.PagedCache(64, 256, 64) if pg is None else pg
    return lib.mla_cache_append_paged(p[0], p[1], p[2], eps, lens, max_len, bt, p[3], p[4], ctypes.byref(s),
                                      ctypes.byref(pg), B.MLA_DTYPE_BF16, None)


def test_cache_append_paged_argument_errors(lib):
    s = shape()
    assert lib.mla_cache_append_paged(*P[:3], 1e-6, None, 4096, P[6], P[3], P[4], ctypes.byref(s), None,
                                      B.MLA_DTYPE_BF16, None) == B.MLA_ERR_NULL
    assert call_append_paged(lib, s, bt=None) == B.MLA_ERR_NULL
    assert call_append_paged(lib, s, bt=P[6] + 2) == B.MLA_ERR_ALIGN
    assert call_append_paged(lib, s, pg=B.PagedCache(0, 256, 64)) == B.MLA_ERR_SHAPE
    assert call_append_paged(lib, s, pg=B.PagedCache(64, 0, 64)) == B.MLA_ERR_SHAPE
    assert call_append_paged(lib, s, max_len=4097) == B.MLA_ERR_RANGE
    assert call_append_paged(lib, shape(seqlen_q=9), max_len=8) == B.MLA_ERR_RANGE
    assert call_append_paged(lib, s, eps=-1.0) == B.MLA_ERR_SHAPE
    # the pools must not overlap the table or each other
    assert call_append_paged(lib, s, bt=P[3] + 64) == B.MLA_ERR_SHAPE
    assert call_append_paged(lib, s, ptrs=[P[0], P[1], P[2], P[3], P[3] + 4096]) == B.MLA_ERR_SHAPE
    for i in range(5):
        p = list(P[:5])
        p[i] = None
        assert call_append_paged(lib, s, ptrs=p) == B.MLA_ERR_NULL


# ------------------------------------------------------------------------------- strides

def strides(**kw):
    d = {f: 0 for f, _ in B.AttnStrides._fields_}
    d.update(kw)
    return B.AttnStrides(*[d[f] for f, _ in B.AttnStrides._fields_])


@pytest.mark.parametrize("kw,code,needle", [
    (dict(q_nope_row=100), B.MLA_ERR_SHAPE, "q_nope_row"),   # narrower than a row
    (dict(q_pe_row=60), B.MLA_ERR_SHAPE, "q_pe_row"),
    (dict(out_row=-128), B.MLA_ERR_SHAPE, "out_row"),
    (dict(kv_pos=511), B.MLA_ERR_SHAPE, "kv_pos"),
    (dict(pe_pos=63), B.MLA_ERR_SHAPE, "pe_pos"),
    (dict(kv_batch=-1), B.MLA_ERR_SHAPE, "kv_batch"),
    (dict(q_nope_row=196), B.MLA_ERR_ALIGN, "q_nope_row"),  # 392 bytes: rows off 16-byte boundaries
    (dict(kv_pos=516), B.MLA_ERR_ALIGN, "kv_pos"),
    (dict(pe_batch=4 * 64 + 4), B.MLA_ERR_ALIGN, "pe_batch"),
    (dict(q_pe_row=1 << 41), B.MLA_ERR_SHAPE, "q_pe_row"),
])
def test_attn_stride_errors(lib, kw, code, needle):
    st = strides(**kw)
    opt = B.AttnOptions(0, 0, ctypes.pointer(st))
    assert call_attn(lib, shape(), opt=opt) == code
    assert needle in B.last_error()
    # the size query validates the same way
    assert lib.mla_absorb_attn_workspace_size(ctypes.byref(shape()), 4096, B.MLA_DTYPE_BF16, ctypes.byref(opt)) == 0


def test_attn_strided_extents_in_overlap_checks(lib):
    """Overlap checks use the extents the strides imply: a row stride that spreads out's 256 rows
    over 2^33 elements reaches into the next tensor (the fake pointers are 4 GiB apart)."""
    p = list(P[:6])
    p[5] = P[0] - (1 << 20)  # out just below q_nope: dense it ends 64 KiB later, well before q_nope
    # (ws=None: the call still fails validation, at the workspace, after the overlap checks, so
    # nothing is ever launched on these fake pointers)
    assert call_attn(lib, shape(), ptrs=p, ws=None) == B.MLA_ERR_WORKSPACE
    st = strides(out_row=1 << 25)
    opt = B.AttnOptions(0, 0, ctypes.pointer(st))
    assert call_attn(lib, shape(), ptrs=p, opt=opt) == B.MLA_ERR_SHAPE
    assert "out overlaps q_nope" in B.last_error()
    # a combined [Bmax, Tmax, 576] cache (kv and pe interleaved): inputs may overlap each other
    st = strides(kv_pos=576, pe_pos=576, q_nope_row=192, q_pe_row=192)
    opt = B.AttnOptions(0, 0, ctypes.pointer(st))
    q = list(P[:6])
    q[1], q[3] = q[0] + 256, q[2] + 1024
    rc = call_attn(lib, shape(), ptrs=q, opt=opt, ws=None)
    assert rc == B.MLA_ERR_WORKSPACE  # validation got past shapes, strides and overlaps


def test_binding_rejects_mismatched_shapes():
    """The binding checks every tensor's shape against the call's sizes before it touches a device
    (the library sees only pointers); CPU tensors suffice, since the shape checks come first."""
    import torch

    bf = torch.bfloat16
    q_nope = torch.zeros(2, 1, 4, 128, dtype=bf)
    q_pe = torch.zeros(2, 1, 4, 64, dtype=bf)
    kv = torch.zeros(2, 64, 512, dtype=bf)
    pe = torch.zeros(2, 64, 64, dtype=bf)
    w = torch.zeros(4 * 256, 512, dtype=bf)
    cases = [
        (dict(q_pe=torch.zeros(2, 1, 3, 64, dtype=bf)), "q_pe"),
        (dict(pe_cache=torch.zeros(2, 64, 32, dtype=bf)), "pe_cache"),
        (dict(pe_cache=torch.zeros(2, 60, 64, dtype=bf)), "pe_cache"),
        (dict(wkv_b=torch.zeros(4 * 256, 256, dtype=bf)), "wkv_b"),
        (dict(wkv_b=torch.zeros(4 * 128, 512, dtype=bf)), "wkv_b"),
        (dict(out=torch.zeros(2, 1, 4, 64, dtype=bf)), "out"),
        (dict(indices=torch.zeros(2, 2, 8, dtype=torch.int32)), "indices"),
    ]
    for kw, needle in cases:
        args = dict(q_nope=q_nope, q_pe=q_pe, kv_cache=kv, pe_cache=pe, wkv_b=w)
        extra = {k: kw.pop(k) for k in ("out", "indices") if k in kw}
        args.update(kw)
        with pytest.raises(ValueError, match=needle):
            B.absorb_attn(args["q_nope"], args["q_pe"], args["kv_cache"], args["pe_cache"], args["wkv_b"], 64, 0.07,
                          **extra)
    with pytest.raises(ValueError, match="rms_w"):
        B.expand_kv(torch.zeros(16, 512, dtype=bf), torch.zeros(256, dtype=bf), w, 4, 128, 128)
    with pytest.raises(ValueError, match="wkv_b"):
        B.expand_kv(torch.zeros(16, 512, dtype=bf), torch.zeros(512, dtype=bf), w, 8, 128, 128)
    with pytest.raises(ValueError, match="k_nope"):
        B.expand_kv(torch.zeros(16, 512, dtype=bf), torch.zeros(512, dtype=bf), w, 4, 128, 128,
                    k_nope=torch.zeros(4, 15, 128, dtype=bf))
    with pytest.raises(ValueError, match="v"):
        B.expand_kv(torch.zeros(16, 512, dtype=bf), torch.zeros(512, dtype=bf), w, 4, 128, 128,
                    v=torch.zeros(4, 16, 64, dtype=bf))
    with pytest.raises(ValueError, match="rms_w"):
        B.cache_append(torch.zeros(2, 1, 512, dtype=bf), torch.zeros(2, 1, 64, dtype=bf), torch.zeros(64, dtype=bf),
                       1e-6, 8, kv, pe)
    with pytest.raises(ValueError, match="pe_cache"):
        B.cache_append(torch.zeros(2, 1, 512, dtype=bf), torch.zeros(2, 1, 64, dtype=bf),
                       torch.zeros(512, dtype=bf), 1e-6, 8, kv, torch.zeros(2, 64, 32, dtype=bf))
    with pytest.raises(ValueError, match="out"):
        B.naive_attn(q_nope, q_pe, torch.zeros(4, 2, 64, 128, dtype=bf), torch.zeros(4, 2, 64, 128, dtype=bf), pe, 64,
                     0.07, out=torch.zeros(2, 1, 4, 100, dtype=bf))


def test_binding_row_strides():
    """Views whose rows are evenly spaced give their row stride; dense tensors give 0."""
    import torch

    q = torch.zeros(2, 3, 4, 192)
    assert B._row_stride(q[..., :128], "q_nope") == 192
    assert B._row_stride(q[..., 128:], "q_pe") == 192
    assert B._row_stride(q, "q") == 0
    assert B._row_stride(q[:1, :1, :1, :128], "one row") == 0
    with pytest.raises(ValueError, match="evenly spaced"):
        B._row_stride(q[:, :2], "q")
    with pytest.raises(ValueError, match="evenly spaced"):
        B._row_stride(torch.zeros(2, 4, 3, 64).transpose(1, 2), "q")
    cache = torch.zeros(3, 10, 576)
    assert B._cache_strides(cache[..., :512], "kv") == (5760, 576)
    assert B._cache_strides(cache[..., 512:], "pe") == (5760, 576)
    assert B._cache_strides(torch.zeros(3, 10, 512), "kv") == (0, 0)
    assert B._cache_strides(torch.zeros(4, 10, 512)[:3], "kv") == (0, 0)
    assert B._cache_strides(torch.zeros(3, 12, 512)[:, :10], "kv") == (6144, 0)
