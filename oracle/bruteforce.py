"""Scalar pure-Python loops for tiny shapes.

TEST INFRASTRUCTURE ONLY (see oracle/mla_oracle.py).  These loops re-derive the
attention output element by element, addressing wkv_b by explicit row number,
with no NumPy contraction, reshape or broadcast anywhere in the arithmetic.  They
are an independent check of oracle/mla_oracle.py on inputs small enough for
Python loops (a few hundred thousand multiply-adds).

Sources: "Naive vs Absorb Attention Implementations in DeepSeek-V3" (sections
"Memory Layout and Cache Structure" and "Computational Patterns and Projection
Handling"); "Latent KV expansion with split" (kernelindex.com, op 064).
"""
from __future__ import annotations

import math


def _f(x):
    return float(x)


def attention_loops(q_nope, q_pe, kv_cache, pe_cache, wkv_b, end_pos, softmax_scale, v_head_dim):
    """Standard attention with explicitly built per-head keys and values.

    For head h the key of cache position t is
        [ sum_c wkv_b[h*(Dn+Dv) + d, c] * kv[b,t,c]  for d < Dn ]  ++  pe[b,t,:]
    and its value is
        [ sum_c wkv_b[h*(Dn+Dv) + Dn + e, c] * kv[b,t,c]  for e < Dv ].
    Query s of the chunk sits at absolute position end_pos - S + s and sees t <= that.
    Returns a nested list out[b][s][h][e].
    """
    B, S, H, Dn = len(q_nope), len(q_nope[0]), len(q_nope[0][0]), len(q_nope[0][0][0])
    R = len(q_pe[0][0][0])
    C = len(kv_cache[0][0])
    Dv = v_head_dim
    stride = Dn + Dv
    start_pos = end_pos - S
    out = [[[[0.0] * Dv for _ in range(H)] for _ in range(S)] for _ in range(B)]
    for b in range(B):
        for h in range(H):
            keys, vals = [], []
            for t in range(end_pos):
                kv_row = [_f(kv_cache[b][t][c]) for c in range(C)]
                key = []
                for d in range(Dn):
                    acc = 0.0
                    for c in range(C):
                        acc += _f(wkv_b[h * stride + d][c]) * kv_row[c]
                    key.append(acc)
                key += [_f(pe_cache[b][t][r]) for r in range(R)]
                val = []
                for e in range(Dv):
                    acc = 0.0
                    for c in range(C):
                        acc += _f(wkv_b[h * stride + Dn + e][c]) * kv_row[c]
                    val.append(acc)
                keys.append(key)
                vals.append(val)
            for s in range(S):
                q = [_f(q_nope[b][s][h][d]) for d in range(Dn)] + [_f(q_pe[b][s][h][r]) for r in range(R)]
                last = start_pos + s
                logits = []
                for t in range(last + 1):
                    acc = 0.0
                    for i in range(Dn + R):
                        acc += q[i] * keys[t][i]
                    logits.append(acc * softmax_scale)
                top = max(logits)
                weights = [math.exp(z - top) for z in logits]
                total = sum(weights)
                for e in range(Dv):
                    acc = 0.0
                    for t in range(last + 1):
                        acc += weights[t] * vals[t][e]
                    out[b][s][h][e] = acc / total
    return out


def expand_loops(c_kv, rms_w, wkv_b, n_heads, qk_nope_head_dim, v_head_dim, eps):
    """Latent expansion element by element: k_nope[h][t][d] and v[h][t][e] as nested lists."""
    T, C = len(c_kv), len(c_kv[0])
    stride = qk_nope_head_dim + v_head_dim
    k_nope = [[[0.0] * qk_nope_head_dim for _ in range(T)] for _ in range(n_heads)]
    v = [[[0.0] * v_head_dim for _ in range(T)] for _ in range(n_heads)]
    for t in range(T):
        row = [_f(c_kv[t][c]) for c in range(C)]
        ms = sum(x * x for x in row) / C
        inv = 1.0 / math.sqrt(ms + eps)
        n = [row[c] * inv * _f(rms_w[c]) for c in range(C)]
        for h in range(n_heads):
            for j in range(stride):
                acc = 0.0
                for c in range(C):
                    acc += n[c] * _f(wkv_b[h * stride + j][c])
                if j < qk_nope_head_dim:
                    k_nope[h][t][j] = acc
                else:
                    v[h][t][j - qk_nope_head_dim] = acc
    return k_nope, v
