"""CPU oracle for MLA absorb attention and latent-KV expansion.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, links or runs
this module: only the tests, the smoke check and the benchmark's CPU-baseline
leg use it.  It shares no code with the HIP kernels.

Everything here is plain NumPy in float64 by default (``dtype=np.float32`` is
accepted for the fp32 equivalence checks).  Library matmuls serve as the
contraction steps; there is no blocking, fusion or reordering beyond the
definitions below.

Sources (the pages):
  [MLA] "Naive vs Absorb Attention Implementations in DeepSeek-V3: MLA
        Optimization Guide" (instagit.com).  Sections "Memory Layout and Cache
        Structure" (cache shapes), "Computational Patterns and Projection
        Handling" (naive and absorb computations) and the FAQ entry on whether
        switching implementation changes the output (it does not).
  [EXP] "Latent KV expansion with split" (kernelindex.com, operation 064):
        RMSNorm over the 512-wide latent, linear projection to
        n_heads * (qk_nope_head_dim + v_head_dim), reshape, transpose, split.

Readings adopted where the pages are silent (each is listed in the design doc):
  * A softmax over cache positions, after scaling and masking, sits between
    the scores and the value sum (no snippet prints it; "attention" implies it).
  * For more than one query token per sequence, query s sits at absolute
    position end_pos - S + s and sees cache positions t <= that position.
  * wkv_b is a Linear weight [H*(Dn+Dv), C]; viewed per head as [H, Dn+Dv, C],
    the first Dn rows of each head are W_UK and the last Dv rows are W_UV.
  * In the naive route the rope key pe[b, t, :] is shared by every head and is
    appended to each head's no-rope key.
  * kv_cache holds the already-normalised latent; the absorb route does not
    normalise.  The expansion normalises raw c_kv with
    x / sqrt(mean(x^2) + eps) * w, eps inside the square root.
  * The softmax scale multiplies the sum of both score terms.
  * A ragged batch (each sequence with its own length) takes the page's slice
    [:bsz, :end_pos] per sequence: sequence b attends to positions
    [0, seq_lens[b]) with its queries at seq_lens[b] - S + s.
  * A paged cache (the DeepSeek Sparse Attention explainer's paged attention /
    KV-cache pages) is storage only: position t of sequence b is row
    t % page_size of page block_table[b, t // page_size]; the attention is that
    of the ragged batch over the rows the pages spell out.
  * Sparse attention over a selected set of positions (the same explainer's
    fine-grained sparse attention over the spans a pre-selector keeps): query
    token (b, s) attends to the cache positions its index list names, shared by
    all heads; an entry counts only if 0 <= idx <= the token's own position, each
    counting entry is one term of the softmax (a repeated entry counts twice), and
    a token with no counting entry gets output 0.
"""
from __future__ import annotations

from typing import Iterable, List, Sequence, Tuple

import numpy as np

__all__ = [
    "split_wkv_b",
    "allowed_positions",
    "masked_softmax",
    "absorb_attention",
    "naive_kv",
    "naive_attention",
    "attention_over_kv",
    "attention_partial",
    "merge_partials",
    "absorb_attention_rows",
    "absorb_attention_ragged",
    "paged_gather",
    "absorb_attention_paged",
    "absorb_attention_sparse",
    "rms_norm",
    "expand_kv",
    "cache_append",
    "cache_append_paged",
]


def _as(x, dtype):
    return np.asarray(x, dtype=dtype)


def split_wkv_b(wkv_b, n_heads: int, qk_nope_head_dim: int, v_head_dim: int):
    """Per-head key and value up-projections held in wkv_b ([MLA] "Absorb Path Execution").

    wkv_b is [H*(Dn+Dv), C].  Head h owns rows h*(Dn+Dv) .. (h+1)*(Dn+Dv)-1; the
    first Dn of them map the latent to the head's no-rope key (W_UK[h], [Dn, C]),
    the remaining Dv map it to the head's value (W_UV[h], [Dv, C]).
    """
    rows, C = wkv_b.shape
    if rows != n_heads * (qk_nope_head_dim + v_head_dim):
        raise ValueError("wkv_b rows do not match n_heads * (qk_nope_head_dim + v_head_dim)")
    per_head = wkv_b.reshape(n_heads, qk_nope_head_dim + v_head_dim, C)
    return per_head[:, :qk_nope_head_dim, :], per_head[:, qk_nope_head_dim:, :]


def allowed_positions(seqlen_q: int, end_pos: int) -> np.ndarray:
    """[S, end_pos] boolean: query s (absolute position end_pos - S + s) may see cache position t.

    With S == 1 every position in [0, end_pos) is visible (plain decode over the
    cached prefix, [MLA] "Computational Patterns").  With S > 1 the mask is causal
    inside the new chunk.
    """
    if not (1 <= seqlen_q <= end_pos):
        raise ValueError("need 1 <= seqlen_q <= end_pos")
    start_pos = end_pos - seqlen_q
    return np.arange(end_pos)[None, :] <= (start_pos + np.arange(seqlen_q))[:, None]


def masked_softmax(scores: np.ndarray, allowed: np.ndarray) -> np.ndarray:
    """Softmax over the last axis restricted to allowed positions (the rest get probability 0)."""
    z = np.where(allowed, scores, -np.inf)
    z = z - z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


def absorb_attention(q_nope, q_pe, kv_cache, pe_cache, wkv_b, end_pos: int, softmax_scale: float,
                     v_head_dim: int, dtype=np.float64, return_intermediates: bool = False):
    """Absorb-route MLA attention ([MLA] "Absorb Path Execution").

    q_nope [B,S,H,Dn], q_pe [B,S,H,R], kv_cache [Bmax,Tmax,C], pe_cache [Bmax,Tmax,R],
    wkv_b [H*(Dn+Dv), C]; attends to rows [0, B) and positions [0, end_pos) of the caches.
    Returns out [B,S,H,Dv] (and a dict of intermediates when asked).

    Steps, in the page's order:
      1. q_lat[b,s,h,:] = sum_d q_nope[b,s,h,d] * W_UK[h,d,:]          (query absorbed into the latent)
      2. score[b,s,h,t] = (q_lat[b,s,h,:].kv[b,t,:] + q_pe[b,s,h,:].pe[b,t,:]) * scale
      3. p = softmax over t (masked as in allowed_positions)
      4. o_lat[b,s,h,:] = sum_t p[b,s,h,t] * kv[b,t,:]                 (value sum in latent space)
      5. out[b,s,h,e] = sum_c o_lat[b,s,h,c] * W_UV[h,e,c]             (projection out through W_UV)
    """
    q_nope, q_pe = _as(q_nope, dtype), _as(q_pe, dtype)
    B, S, H, Dn = q_nope.shape
    R = q_pe.shape[-1]
    kv = _as(kv_cache[:B, :end_pos], dtype)
    pe = _as(pe_cache[:B, :end_pos], dtype)
    T, C = kv.shape[1], kv.shape[2]
    w_uk, w_uv = split_wkv_b(_as(wkv_b, dtype), H, Dn, v_head_dim)

    # 1. per head: [B*S, Dn] @ [Dn, C]
    q_lat = np.matmul(q_nope.transpose(2, 0, 1, 3).reshape(H, B * S, Dn), w_uk)
    q_lat = q_lat.reshape(H, B, S, C).transpose(1, 2, 0, 3)
    # 2. per sequence: [S*H, C] @ [C, T] + [S*H, R] @ [R, T]
    latent_term = np.matmul(q_lat.reshape(B, S * H, C), kv.transpose(0, 2, 1))
    rope_term = np.matmul(q_pe.reshape(B, S * H, R), pe.transpose(0, 2, 1))
    scores = ((latent_term + rope_term) * softmax_scale).reshape(B, S, H, T)
    # 3.
    p = masked_softmax(scores, allowed_positions(S, end_pos)[None, :, None, :])
    # 4. per sequence: [S*H, T] @ [T, C]
    o_lat = np.matmul(p.reshape(B, S * H, T), kv).reshape(B, S, H, C)
    # 5. per head: [B*S, C] @ [C, Dv]
    out = np.matmul(o_lat.transpose(2, 0, 1, 3).reshape(H, B * S, C), w_uv.transpose(0, 2, 1))
    out = out.reshape(H, B, S, v_head_dim).transpose(1, 2, 0, 3)
    if return_intermediates:
        return out, {"q_lat": q_lat, "scores": scores, "p": p, "o_lat": o_lat}
    return out


def naive_kv(kv_cache, wkv_b, batch: int, end_pos: int, n_heads: int, qk_nope_head_dim: int,
             v_head_dim: int, dtype=np.float64):
    """Keys and values the naive route caches ([MLA] "Naive Path Execution", "Naive
    Implementation Cache Design"): the Linear layer wkv_b applied to every cached latent
    row, reshaped per head and split into the no-rope key [B,T,H,Dn] and value [B,T,H,Dv]."""
    kv = _as(kv_cache[:batch, :end_pos], dtype)
    full = np.matmul(kv, _as(wkv_b, dtype).T)  # [B, T, H*(Dn+Dv)]
    full = full.reshape(batch, end_pos, n_heads, qk_nope_head_dim + v_head_dim)
    return full[..., :qk_nope_head_dim], full[..., qk_nope_head_dim:]


def naive_attention(q_nope, q_pe, kv_cache, pe_cache, wkv_b, end_pos: int, softmax_scale: float,
                    v_head_dim: int, dtype=np.float64, return_intermediates: bool = False):
    """Naive-route MLA attention ([MLA] "Naive Path Execution").

    Materialises per-head keys k[b,t,h,:] = concat(W_UK[h] kv[b,t], pe[b,t]) (Dn+R wide) and
    values v[b,t,h,:] = W_UV[h] kv[b,t] (Dv wide), then runs standard attention with the
    query q = concat(q_nope, q_pe).  Same masking and softmax as absorb_attention.
    """
    q_nope, q_pe = _as(q_nope, dtype), _as(q_pe, dtype)
    B, S, H, Dn = q_nope.shape
    R = q_pe.shape[-1]
    pe = _as(pe_cache[:B, :end_pos], dtype)
    T = pe.shape[1]
    k_nope, v = naive_kv(kv_cache, wkv_b, B, end_pos, H, Dn, v_head_dim, dtype)
    k = np.concatenate([k_nope, np.broadcast_to(pe[:, :, None, :], (B, T, H, R))], axis=-1)
    q = np.concatenate([q_nope, q_pe], axis=-1)
    # score[b,s,h,t] = q[b,s,h,:].k[b,t,h,:] * scale, as [B,H,S,D] @ [B,H,D,T]
    scores = np.matmul(q.transpose(0, 2, 1, 3), k.transpose(0, 2, 3, 1)) * softmax_scale
    scores = scores.transpose(0, 2, 1, 3)  # [B,S,H,T]
    p = masked_softmax(scores, allowed_positions(S, end_pos)[None, :, None, :])
    # out[b,s,h,:] = sum_t p[b,s,h,t] v[b,t,h,:], as [B,H,S,T] @ [B,H,T,Dv]
    out = np.matmul(p.transpose(0, 2, 1, 3), v.transpose(0, 2, 1, 3)).transpose(0, 2, 1, 3)
    if return_intermediates:
        return out, {"k": k, "v": v, "scores": scores, "p": p}
    return out


def attention_over_kv(q_nope, q_pe, k_nope, v, pe_cache, end_pos: int, softmax_scale: float,
                      dtype=np.float64):
    """The attention half of the naive route ([MLA] "Naive Path Execution") on keys and values
    that are already expanded: k_nope [H, Bmax, Tmax, Dn] and v [H, Bmax, Tmax, Dv] head-major
    (the layout the expansion of [EXP] writes for the caches' Bmax*Tmax rows in (b, t) order).

    Key of head h at position t: concat(k_nope[h, b, t], pe_cache[b, t]) (the rope key shared by
    every head); query: concat(q_nope[b, s, h], q_pe[b, s, h]).  Masking and softmax as in
    absorb_attention.  Returns out [B, S, H, Dv].
    """
    q = np.concatenate([_as(q_nope, dtype), _as(q_pe, dtype)], axis=-1)  # [B,S,H,Dn+R]
    B, S, H, _ = q.shape
    allowed = allowed_positions(S, end_pos)
    Dv = v.shape[-1]
    out = np.zeros((B, S, H, Dv), dtype)
    for b in range(B):
        pe = _as(pe_cache[b, :end_pos], dtype)  # [T, R]
        for h in range(H):
            k = np.concatenate([_as(k_nope[h, b, :end_pos], dtype), pe], axis=-1)  # [T, Dn+R]
            scores = np.matmul(q[b, :, h], k.T) * softmax_scale  # [S, T]
            p = masked_softmax(scores, allowed)
            out[b, :, h] = np.matmul(p, _as(v[h, b, :end_pos], dtype))
    return out


def attention_partial(q_lat, q_pe, kv_cache, pe_cache, end_pos: int, softmax_scale: float,
                      t_begin: int, t_end: int, dtype=np.float64):
    """One split of the cache positions: the online-softmax state over t in [t_begin, t_end).

    Returns (m [B,S,H], l [B,S,H], o [B,S,H,C]) with m the largest visible scaled score in
    the range (-inf when none is visible), l = sum exp(score - m) and
    o = sum exp(score - m) * kv[b,t,:] (both 0 when nothing is visible).
    """
    q_lat, q_pe = _as(q_lat, dtype), _as(q_pe, dtype)
    B, S, H, C = q_lat.shape
    R = q_pe.shape[-1]
    kv = _as(kv_cache[:B, t_begin:t_end], dtype)
    pe = _as(pe_cache[:B, t_begin:t_end], dtype)
    n = t_end - t_begin
    scores = (np.matmul(q_lat.reshape(B, S * H, C), kv.transpose(0, 2, 1))
              + np.matmul(q_pe.reshape(B, S * H, R), pe.transpose(0, 2, 1))) * softmax_scale
    scores = scores.reshape(B, S, H, n)
    vis = allowed_positions(S, end_pos)[:, t_begin:t_end][None, :, None, :]
    z = np.where(vis, scores, -np.inf)
    m = z.max(axis=-1) if n > 0 else np.full((B, S, H), -np.inf, dtype)
    any_vis = np.isfinite(m)
    e = np.where(vis, np.exp(z - np.where(any_vis, m, 0.0)[..., None]), 0.0)
    l = e.sum(axis=-1)
    o = np.matmul(e.reshape(B, S * H, n), kv).reshape(B, S, H, C)
    return m, l, o


def merge_partials(parts: Sequence[Tuple[np.ndarray, np.ndarray, np.ndarray]]) -> np.ndarray:
    """Combine split states into o_lat: with M = max_i m_i and w_i = exp(m_i - M) (0 for an
    empty split), o_lat = sum_i w_i o_i / sum_i w_i l_i."""
    ms = np.stack([p[0] for p in parts])
    M = ms.max(axis=0)
    num = 0.0
    den = 0.0
    for m, l, o in parts:
        w = np.where(np.isfinite(m), np.exp(np.where(np.isfinite(m), m - M, 0.0)), 0.0)
        num = num + w[..., None] * o
        den = den + w * l
    return num / den[..., None]


def absorb_attention_rows(q_nope, q_pe, kv_cache, pe_cache, wkv_b, end_pos: int, softmax_scale: float,
                          v_head_dim: int, rows: Iterable[Tuple[int, int, int]], dtype=np.float64):
    """absorb_attention for selected output rows (b, s, h) only; returns [len(rows), Dv].

    Each output row depends only on its own query row, its sequence's cache and its head's
    slices of wkv_b, so this evaluates the same five steps row by row (used to sample
    outputs at sizes where the full tensor is too slow on the CPU).
    """
    B, S, H, Dn = q_nope.shape
    start_pos = end_pos - S
    w_uk, w_uv = split_wkv_b(_as(wkv_b, dtype), H, Dn, v_head_dim)
    cache = {}
    res: List[np.ndarray] = []
    for b, s, h in rows:
        if b not in cache:
            cache.clear()
            cache[b] = (_as(kv_cache[b, :end_pos], dtype), _as(pe_cache[b, :end_pos], dtype))
        kv, pe = cache[b]
        q_lat = _as(q_nope[b, s, h], dtype) @ w_uk[h]
        scores = (kv @ q_lat + pe @ _as(q_pe[b, s, h], dtype)) * softmax_scale
        vis = np.arange(end_pos) <= start_pos + s
        p = masked_softmax(scores, vis)
        o_lat = p @ kv
        res.append(w_uv[h] @ o_lat)
    return np.stack(res)


def absorb_attention_ragged(q_nope, q_pe, kv_cache, pe_cache, wkv_b, seq_lens, softmax_scale: float,
                            v_head_dim: int, dtype=np.float64, rows: Iterable[Tuple[int, int, int]] = None):
    """absorb_attention for a batch whose sequences have their own lengths.

    Sequence b is absorb_attention on that sequence alone with end_pos = seq_lens[b] (the
    page's slice [:bsz, :end_pos] taken per sequence).  With `rows`, only those (b, s, h)
    outputs are evaluated (as absorb_attention_rows) and [len(rows), Dv] is returned.
    """
    B = q_nope.shape[0]
    if rows is not None:
        res = [absorb_attention_rows(q_nope[b:b + 1], q_pe[b:b + 1], kv_cache[b:b + 1], pe_cache[b:b + 1], wkv_b,
                                     int(seq_lens[b]), softmax_scale, v_head_dim, [(0, s, h)], dtype)[0]
               for b, s, h in rows]
        return np.stack(res)
    out = [absorb_attention(q_nope[b:b + 1], q_pe[b:b + 1], kv_cache[b:b + 1], pe_cache[b:b + 1], wkv_b,
                            int(seq_lens[b]), softmax_scale, v_head_dim, dtype)
           for b in range(B)]
    return np.concatenate(out, axis=0)


def paged_gather(pages, block_table, length: int, b: int, page_size: int):
    """The cache rows [0, length) of sequence b spelled out by its pages: row t is
    pages[block_table[b, t // page_size], t % page_size]."""
    t = np.arange(length)
    return pages[np.asarray(block_table)[b, t // page_size], t % page_size]


def absorb_attention_paged(q_nope, q_pe, kv_pages, pe_pages, wkv_b, block_table, seq_lens, page_size: int,
                           softmax_scale: float, v_head_dim: int, dtype=np.float64,
                           rows: Iterable[Tuple[int, int, int]] = None):
    """absorb_attention_ragged over paged caches: kv_pages [P, page_size, C], pe_pages
    [P, page_size, R], block_table [B, max_pages]; sequence b's cache is its gathered rows."""
    B = q_nope.shape[0]
    lens = [int(n) for n in seq_lens]
    T = max(lens)
    kv = np.zeros((B, T, kv_pages.shape[-1]), dtype)
    pe = np.zeros((B, T, pe_pages.shape[-1]), dtype)
    for b in range(B):
        kv[b, :lens[b]] = paged_gather(_as(kv_pages, dtype), block_table, lens[b], b, page_size)
        pe[b, :lens[b]] = paged_gather(_as(pe_pages, dtype), block_table, lens[b], b, page_size)
    return absorb_attention_ragged(q_nope, q_pe, kv, pe, wkv_b, lens, softmax_scale, v_head_dim, dtype, rows)


def absorb_attention_sparse(q_nope, q_pe, kv_cache, pe_cache, wkv_b, indices, seq_lens, softmax_scale: float,
                            v_head_dim: int, dtype=np.float64, rows: Iterable[Tuple[int, int, int]] = None):
    """Absorb-route attention over selected positions: indices [B, S, K] (int), seq_lens [B].

    Token s of sequence b sits at position seq_lens[b] - S + s; its entries idx with
    0 <= idx <= that position are the positions it attends to (in list order, repeats kept).
    Per head: q_lat = q_nope . W_UK[h]; scores over the entries (q_lat . kv[b, idx] +
    q_pe . pe[b, idx]) * scale; softmax; o_lat = sum p kv[b, idx]; out = W_UV[h] . o_lat.
    With no counting entry the output is 0.  With `rows`, [len(rows), Dv] for those (b, s, h).
    """
    q_nope, q_pe = _as(q_nope, dtype), _as(q_pe, dtype)
    B, S, H, Dn = q_nope.shape
    w_uk, w_uv = split_wkv_b(_as(wkv_b, dtype), H, Dn, v_head_dim)
    idx_all = np.asarray(indices)
    want = sorted({(b, s) for b, s, _ in rows}) if rows is not None else [(b, s) for b in range(B) for s in range(S)]
    res = {}
    for b, s in want:
        last = int(seq_lens[b]) - S + s
        idx = idx_all[b, s]
        sel = idx[(idx >= 0) & (idx <= last)]
        if sel.size == 0:
            res[(b, s)] = np.zeros((H, v_head_dim), dtype)
            continue
        kv = _as(kv_cache, dtype)[b, sel]  # [K', C]
        pe = _as(pe_cache, dtype)[b, sel]  # [K', R]
        q_lat = np.einsum("hd,hdc->hc", q_nope[b, s], w_uk)
        scores = (q_lat @ kv.T + q_pe[b, s] @ pe.T) * softmax_scale  # [H, K']
        p = masked_softmax(scores, np.ones(scores.shape, bool))
        res[(b, s)] = np.einsum("hc,hdc->hd", p @ kv, w_uv)
    if rows is not None:
        return np.stack([res[(b, s)][h] for b, s, h in rows])
    out = np.zeros((B, S, H, v_head_dim), dtype)
    for (b, s), v in res.items():
        out[b, s] = v
    return out


def rms_norm(x, w, eps: float, dtype=np.float64):
    """RMSNorm over the last axis ([EXP]): x / sqrt(mean(x^2) + eps) * w."""
    x, w = _as(x, dtype), _as(w, dtype)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * w


def expand_kv(c_kv, rms_w, wkv_b, n_heads: int, qk_nope_head_dim: int, v_head_dim: int, eps: float,
              dtype=np.float64):
    """Latent KV expansion with split ([EXP]).

    c_kv [T, C] -> RMSNorm -> y = n @ wkv_b^T [T, H*(Dn+Dv)] -> reshape [T, H, Dn+Dv]
    -> transpose [H, T, Dn+Dv] -> split into K_nope [H, T, Dn] and V [H, T, Dv].
    """
    n = rms_norm(c_kv, rms_w, eps, dtype)
    T = n.shape[0]
    y = np.matmul(n, _as(wkv_b, dtype).T)
    y = y.reshape(T, n_heads, qk_nope_head_dim + v_head_dim).transpose(1, 0, 2)
    return np.ascontiguousarray(y[..., :qk_nope_head_dim]), np.ascontiguousarray(y[..., qk_nope_head_dim:])


def cache_append(c_kv_new, k_pe_new, rms_w, eps: float, kv_cache, pe_cache, end_pos: int = None,
                 seq_lens=None, dtype=np.float64):
    """The caches after writing S new tokens per sequence ([MLA] "Memory Layout and Cache
    Structure": kv_cache holds each position's latent, pe_cache its rotary key; the latent is
    stored normalised, reading as for the absorb route).

    c_kv_new [B,S,C] raw latent, k_pe_new [B,S,R]; token s of sequence b goes to position
    end_pos - S + s (or seq_lens[b] - S + s): kv row := rms_norm(c_kv_new[b, s]), pe row :=
    k_pe_new[b, s].  Returns new arrays (the inputs are not modified); other rows are copied.
    """
    kv, pe = _as(kv_cache, dtype).copy(), _as(pe_cache, dtype).copy()
    B, S = c_kv_new.shape[0], c_kv_new.shape[1]
    n = rms_norm(c_kv_new, rms_w, eps, dtype)
    kp = _as(k_pe_new, dtype)
    for b in range(B):
        length = end_pos if seq_lens is None else int(seq_lens[b])
        for s in range(S):
            kv[b, length - S + s] = n[b, s]
            pe[b, length - S + s] = kp[b, s]
    return kv, pe


def cache_append_paged(c_kv_new, k_pe_new, rms_w, eps: float, kv_pages, pe_pages, block_table, page_size: int,
                       end_pos: int = None, seq_lens=None, dtype=np.float64):
    """cache_append into page pools (the paged layout of absorb_attention_paged): token s of
    sequence b goes to position p = end_pos - S + s (or seq_lens[b] - S + s), i.e. row
    p % page_size of page block_table[b, p // page_size].  Returns new pools."""
    kv, pe = _as(kv_pages, dtype).copy(), _as(pe_pages, dtype).copy()
    B, S = c_kv_new.shape[0], c_kv_new.shape[1]
    n = rms_norm(c_kv_new, rms_w, eps, dtype)
    kp = _as(k_pe_new, dtype)
    table = np.asarray(block_table)
    for b in range(B):
        length = end_pos if seq_lens is None else int(seq_lens[b])
        for s in range(S):
            p = length - S + s
            page, slot = table[b, p // page_size], p % page_size
            kv[page, slot] = n[b, s]
            pe[page, slot] = kp[b, s]
    return kv, pe
