"""GPU parity: the HIP path (through the C-ABI) against the CPU oracle on the same seeded inputs.

Bar: max|gpu - ref| <= 1e-5 * max|ref| for fp32 workloads and <= 2e-2 * max|ref| for bf16
workloads, no NaN/Inf anywhere; outputs are NaN-poisoned before each call so an element the
kernels never write fails the check.
"""
import numpy as np
import pytest
import torch

from mla_latent_kv_absorb_amd.workloads import (ATTN_CONFIGS, EXPAND_CONFIGS, RAGGED_WORKLOADS, make_attn_inputs,
                                                 make_expand_inputs, ragged_workload, round_to_bf16)
from oracle import mla_oracle as O

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2}


def round_bf16(a):
    return round_to_bf16(np.asarray(a, np.float32))


def tdtype(cfg):
    return torch.float32 if cfg.dtype == "f32" else torch.bfloat16


def to_dev(x, cfg):
    return {k: torch.from_numpy(v).to("cuda").to(tdtype(cfg)) for k, v in x.items()}


def check(gpu, ref, tol, what):
    g = gpu.float().cpu().double().numpy() if isinstance(gpu, torch.Tensor) else gpu
    assert np.isfinite(g).all(), f"{what}: {int((~np.isfinite(g)).sum())} non-finite outputs"
    err = np.abs(g - ref)
    scale = np.abs(ref).max()
    worst = float(err.max() / scale)
    loc = np.unravel_index(int(err.argmax()), err.shape)
    print(f"{what}: max rel err {worst:.3e} at {loc}, mean abs err {err.mean():.3e}, max|ref| {scale:.3e}")
    assert worst <= tol, f"{what}: max abs err {err.max():.3e} = {worst:.3e} * max|ref| at {loc} > {tol}"


def run_attn(lib, cfg, t, path="auto", splits=0):
    out = torch.full((cfg.batch, cfg.seqlen_q, cfg.n_heads, cfg.v_head_dim), float("nan"), dtype=tdtype(cfg),
                     device="cuda")
    lib.absorb_attn(t["q_nope"], t["q_pe"], t["kv_cache"], t["pe_cache"], t["wkv_b"], cfg.end_pos, cfg.softmax_scale,
                    out, num_splits=splits, path=path)
    torch.cuda.synchronize()
    return out


def oracle_attn(cfg, x):
    return O.absorb_attention(x["q_nope"], x["q_pe"], x["kv_cache"], x["pe_cache"], x["wkv_b"], cfg.end_pos,
                              cfg.softmax_scale, cfg.v_head_dim)


def dsv3_small(**kw):
    base = dict(batch=2, cache_batch=3, end_pos=300, cache_len=320)
    base.update(kw)
    return ATTN_CONFIGS["dsv3_decode"].replace(**base)


# --------------------------------------------------------------------------------- tiny fp32

@pytest.mark.parametrize("path", ["plain", "auto"])
def test_tiny_f32_absorb_and_naive(gpu_lib, path):
    cfg = ATTN_CONFIGS["tiny_f32"]
    x = make_attn_inputs(cfg)
    out = run_attn(gpu_lib, cfg, to_dev(x, cfg), path=path)
    check(out, oracle_attn(cfg, x), TOL["f32"], f"tiny_f32 {path} vs absorb oracle")
    naive = O.naive_attention(x["q_nope"], x["q_pe"], x["kv_cache"], x["pe_cache"], x["wkv_b"], cfg.end_pos,
                              cfg.softmax_scale, cfg.v_head_dim)
    check(out, naive, TOL["f32"], f"tiny_f32 {path} vs naive oracle")


@pytest.mark.parametrize("splits", [1, 3, 128])
def test_tiny_f32_splits(gpu_lib, splits):
    cfg = ATTN_CONFIGS["tiny_f32"]
    x = make_attn_inputs(cfg)
    out = run_attn(gpu_lib, cfg, to_dev(x, cfg), path="plain", splits=splits)
    check(out, oracle_attn(cfg, x), TOL["f32"], f"tiny_f32 splits={splits}")


def test_tiny_f32_chunk(gpu_lib):
    cfg = ATTN_CONFIGS["tiny_f32"].replace(seqlen_q=9, end_pos=100)
    x = make_attn_inputs(cfg)
    out = run_attn(gpu_lib, cfg, to_dev(x, cfg))
    check(out, oracle_attn(cfg, x), TOL["f32"], "tiny_f32 causal chunk S=9")


@pytest.mark.parametrize("path", ["plain", "auto"])
def test_tiny_f32_expand(gpu_lib, path):
    cfg = EXPAND_CONFIGS["tiny_f32"]
    x = make_expand_inputs(cfg)
    t = to_dev(x, cfg)
    k = torch.full((cfg.n_heads, cfg.n_tokens, cfg.qk_nope_head_dim), float("nan"), device="cuda")
    v = torch.full((cfg.n_heads, cfg.n_tokens, cfg.v_head_dim), float("nan"), device="cuda")
    gpu_lib.expand_kv(t["c_kv"], t["rms_w"], t["wkv_b"], cfg.n_heads, cfg.qk_nope_head_dim, cfg.v_head_dim, cfg.eps,
                      k, v, path=path)
    torch.cuda.synchronize()
    kr, vr = O.expand_kv(x["c_kv"], x["rms_w"], x["wkv_b"], cfg.n_heads, cfg.qk_nope_head_dim, cfg.v_head_dim,
                         cfg.eps)
    check(k, kr, TOL["f32"], "tiny_f32 expand K_nope")
    check(v, vr, TOL["f32"], "tiny_f32 expand V")


# --------------------------------------------------------------------------------- bf16, DSV3 heads, small

@pytest.mark.parametrize("path", ["plain", "mfma"])
@pytest.mark.parametrize("end_pos", [1, 37, 300])
def test_bf16_decode_small(gpu_lib, path, end_pos):
    cfg = dsv3_small(end_pos=end_pos)
    x = make_attn_inputs(cfg)
    out = run_attn(gpu_lib, cfg, to_dev(x, cfg), path=path)
    check(out, oracle_attn(cfg, x), TOL["bf16"], f"bf16 decode B=2 T={end_pos} {path}")


@pytest.mark.parametrize("path", ["plain", "mfma"])
def test_bf16_chunk_small(gpu_lib, path):
    cfg = dsv3_small(seqlen_q=5, end_pos=200, batch=1, cache_batch=1)
    x = make_attn_inputs(cfg)
    out = run_attn(gpu_lib, cfg, to_dev(x, cfg), path=path)
    check(out, oracle_attn(cfg, x), TOL["bf16"], f"bf16 chunk S=5 T=200 {path}")


@pytest.mark.parametrize("path", ["plain", "mfma"])
def test_bf16_expand_small(gpu_lib, path):
    cfg = EXPAND_CONFIGS["dsv3_expand"].replace(n_tokens=200)
    x = make_expand_inputs(cfg)
    t = to_dev(x, cfg)
    k = torch.full((cfg.n_heads, cfg.n_tokens, cfg.qk_nope_head_dim), float("nan"), dtype=torch.bfloat16,
                   device="cuda")
    v = torch.full_like(k, float("nan"))
    gpu_lib.expand_kv(t["c_kv"], t["rms_w"], t["wkv_b"], cfg.n_heads, cfg.qk_nope_head_dim, cfg.v_head_dim, cfg.eps,
                      k, v, path=path)
    torch.cuda.synchronize()
    kr, vr = O.expand_kv(x["c_kv"], x["rms_w"], x["wkv_b"], cfg.n_heads, cfg.qk_nope_head_dim, cfg.v_head_dim,
                         cfg.eps)
    check(k, kr, TOL["bf16"], f"bf16 expand T=200 K_nope {path}")
    check(v, vr, TOL["bf16"], f"bf16 expand T=200 V {path}")


# --------------------------------------------------------------------------------- matrix-core path

@pytest.mark.parametrize("splits", [1, 2, 3, 7, 64])
def test_mfma_forced_splits(gpu_lib, splits):
    cfg = dsv3_small(end_pos=1000, cache_len=1024)
    x = make_attn_inputs(cfg)
    out = run_attn(gpu_lib, cfg, to_dev(x, cfg), path="mfma", splits=splits)
    check(out, oracle_attn(cfg, x), TOL["bf16"], f"mfma decode T=1000 splits={splits}")


@pytest.mark.parametrize("kw", [
    dict(n_heads=16, seqlen_q=3, end_pos=130),     # 48 query rows: one partial row block
    dict(n_heads=128, seqlen_q=3, end_pos=97),     # 384 rows: three row blocks, causal
    dict(n_heads=64, seqlen_q=64, end_pos=64),     # chunk covering the whole prefix
    dict(n_heads=128, seqlen_q=1, end_pos=65),     # one position past a tile boundary
])
def test_mfma_shapes(gpu_lib, kw):
    cfg = dsv3_small(batch=2, cache_batch=2, cache_len=max(160, kw["end_pos"]), **kw)
    x = make_attn_inputs(cfg)
    out = run_attn(gpu_lib, cfg, to_dev(x, cfg), path="mfma")
    check(out, oracle_attn(cfg, x), TOL["bf16"], f"mfma {kw}")


@pytest.mark.parametrize("kw", [
    # 11 query rows per head: waves of the combine take 3, 3, 3 and 2 rows (a clamped repeat row),
    # 7 splits against batches of 4; 12 heads: workgroup counts that are not multiples of 8
    dict(batch=1, seqlen_q=11, n_heads=12, end_pos=300, splits=7),
    # 21 rows: one full 16-row group and one of 5 (2, 1, 1, 1 rows per wave); 5 splits
    dict(batch=3, seqlen_q=7, n_heads=20, end_pos=260, splits=5),
    # 2 rows with 17 splits: one row per wave, two batches of 16 splits (the second mostly repeats)
    dict(batch=2, seqlen_q=1, n_heads=40, end_pos=700, splits=17),
])
def test_mfma_combine_row_and_split_counts(gpu_lib, kw):
    kw = dict(kw)
    splits = kw.pop("splits")
    cfg = dsv3_small(cache_batch=kw["batch"], cache_len=kw["end_pos"] + 16, **kw)
    x = make_attn_inputs(cfg)
    out = run_attn(gpu_lib, cfg, to_dev(x, cfg), path="mfma", splits=splits)
    check(out, oracle_attn(cfg, x), TOL["bf16"], f"mfma {kw} splits={splits}")


def test_mfma_repeatable_bitwise(gpu_lib):
    cfg = dsv3_small(end_pos=777, cache_len=800)
    x = make_attn_inputs(cfg)
    t = to_dev(x, cfg)
    a = run_attn(gpu_lib, cfg, t, path="mfma", splits=5)
    b = run_attn(gpu_lib, cfg, t, path="mfma", splits=5)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_mfma_larger_than_tile_max_shift(gpu_lib):
    """A row whose scores grow along the cache forces the running maximum to move by far more
    than the lazy-rescale threshold several times inside one split."""
    cfg = dsv3_small(batch=1, cache_batch=1, end_pos=512, cache_len=512)
    x = make_attn_inputs(cfg)
    ramp = np.linspace(0.0, 6.0, cfg.cache_len, dtype=np.float32)[None, :, None]
    x["pe_cache"] = (x["pe_cache"] * 0.1 + ramp).astype(np.float32)
    x["q_pe"] = np.abs(x["q_pe"]) * 2.0 + 1.0
    from mla_latent_kv_absorb_amd.workloads import round_to_bf16
    x = {k: round_to_bf16(v) for k, v in x.items()}
    out = run_attn(gpu_lib, cfg, to_dev(x, cfg), path="mfma", splits=1)
    check(out, oracle_attn(cfg, x), TOL["bf16"], "mfma growing scores")


def oracle_attn_full(cfg, x, lens=None, q_block=64):
    """The oracle's absorb route for every output element, one sequence (and for S > 1 one block of
    query tokens) at a time, so that host memory stays small.  Query tokens [s0, s1) of a sequence of
    length n sit at positions n - S + s0 .. n - S + s1 - 1, so they are the absorb route of those
    tokens alone with end_pos = n - S + s1: the mask definition the chunk-rows-are-decodes pin fixes."""
    B, S = cfg.batch, cfg.seqlen_q
    out = np.empty((B, S, cfg.n_heads, cfg.v_head_dim))
    for b in range(B):
        n = cfg.end_pos if lens is None else int(lens[b])
        for s0 in range(0, S, q_block):
            s1 = min(S, s0 + q_block)
            out[b:b + 1, s0:s1] = O.absorb_attention(x["q_nope"][b:b + 1, s0:s1], x["q_pe"][b:b + 1, s0:s1],
                                                     x["kv_cache"][b:b + 1], x["pe_cache"][b:b + 1], x["wkv_b"],
                                                     n - S + s1, cfg.softmax_scale, cfg.v_head_dim)
    return out


@pytest.mark.parametrize("name", ["dsv3_decode", "long_decode", "chunk_prefill"])
def test_full_size_attention(gpu_lib, name):
    """Every output element of the full-size workload against the oracle."""
    cfg = ATTN_CONFIGS[name]
    print(f"full-size {name}: B={cfg.batch} S={cfg.seqlen_q} T={cfg.end_pos}", flush=True)
    x = make_attn_inputs(cfg)
    out = run_attn(gpu_lib, cfg, to_dev(x, cfg))
    check(out, oracle_attn_full(cfg, x), TOL["bf16"], f"{name} all outputs")


def test_full_size_fused_append(gpu_lib):
    """dsv3_decode at full size as a serving step: each sequence's new token appended in the same call
    (mla_absorb_attn_append).  Caches and output equal the two calls bit for bit, the written rows
    match the oracle's append, and every output element matches the oracle's attention over the
    appended caches."""
    cfg = ATTN_CONFIGS["dsv3_decode"]
    print(f"full-size fused append: B={cfg.batch} T={cfg.end_pos}", flush=True)
    x = make_attn_inputs(cfg)
    c_new, kp_new, w = _append_inputs(cfg, 1, 71)
    t = to_dev(x, cfg)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(torch.bfloat16)
    res = []
    for fused in (True, False):
        kv, pe = t["kv_cache"].clone(), t["pe_cache"].clone()
        out = torch.full((cfg.batch, 1, cfg.n_heads, cfg.v_head_dim), float("nan"), dtype=torch.bfloat16, device="cuda")
        if fused:
            gpu_lib.absorb_attn(t["q_nope"], t["q_pe"], kv, pe, t["wkv_b"], cfg.end_pos, cfg.softmax_scale, out,
                                append=(dev(c_new), dev(kp_new), dev(w), 1e-6))
        else:
            gpu_lib.cache_append(dev(c_new), dev(kp_new), dev(w), 1e-6, cfg.end_pos, kv, pe)
            gpu_lib.absorb_attn(t["q_nope"], t["q_pe"], kv, pe, t["wkv_b"], cfg.end_pos, cfg.softmax_scale, out)
        torch.cuda.synchronize()
        res.append((out, kv, pe))
    for a, b in zip(res[0], res[1]):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), "fused call differs from the two calls"
    kv_o, pe_o = O.cache_append(c_new, kp_new, w, 1e-6, x["kv_cache"], x["pe_cache"], end_pos=cfg.end_pos)
    g_new = res[0][1][:, cfg.end_pos - 1].float().cpu().numpy()
    check(g_new.astype(np.float64), kv_o[:, cfg.end_pos - 1], TOL["bf16"], "full-size fused append: written rows")
    x2 = dict(x, kv_cache=np.array(kv_o), pe_cache=pe_o)
    x2["kv_cache"][:, cfg.end_pos - 1] = g_new
    check(res[0][0], oracle_attn_full(cfg, x2), TOL["bf16"], "full-size fused append: all outputs")


# --------------------------------------------------------------------------------- ragged batches

def run_attn_ragged(lib, cfg, t, lens, path="auto", splits=0):
    out = torch.full((cfg.batch, cfg.seqlen_q, cfg.n_heads, cfg.v_head_dim), float("nan"), dtype=tdtype(cfg),
                     device="cuda")
    seq = torch.tensor(np.asarray(lens, np.int32), device="cuda")
    lib.absorb_attn(t["q_nope"], t["q_pe"], t["kv_cache"], t["pe_cache"], t["wkv_b"], cfg.end_pos, cfg.softmax_scale,
                    out, num_splits=splits, path=path, seq_lens=seq)
    torch.cuda.synchronize()
    return out


def poison_tails(t, lens):
    """NaN in every cache position at or past each sequence's length: none of it may reach the output."""
    for b, n in enumerate(lens):
        t["kv_cache"][b, int(n):] = float("nan")
        t["pe_cache"][b, int(n):] = float("nan")


def oracle_ragged(cfg, x, lens, rows=None):
    return O.absorb_attention_ragged(x["q_nope"], x["q_pe"], x["kv_cache"], x["pe_cache"], x["wkv_b"], lens,
                                     cfg.softmax_scale, cfg.v_head_dim, rows=rows)


@pytest.mark.parametrize("path", ["plain", "mfma"])
@pytest.mark.parametrize("seqlen_q,lens", [(1, [1, 37, 300, 64]), (5, [5, 200, 33])])
def test_ragged_small(gpu_lib, path, seqlen_q, lens):
    cfg = dsv3_small(batch=len(lens), cache_batch=len(lens) + 1, seqlen_q=seqlen_q, end_pos=max(lens) + 7,
                     cache_len=320)
    x = make_attn_inputs(cfg)
    t = to_dev(x, cfg)
    poison_tails(t, lens)
    out = run_attn_ragged(gpu_lib, cfg, t, lens, path=path)
    check(out, oracle_ragged(cfg, x, lens), TOL["bf16"], f"ragged S={seqlen_q} lens={lens} {path}")


@pytest.mark.parametrize("lens", [[4096] + [1] * 31, [1] * 31 + [4096], [64 * (i + 1) for i in range(32)]])
def test_ragged_balanced_full_heads(gpu_lib, lens):
    """The device plan at the decode head shape: one long sequence among very short ones (the
    equal-chunk plan; it takes up to four times the uniform plan's chunks), at either end of the
    chunk order, and a linear spread of lengths (the uniform splits); every output element."""
    cfg = ATTN_CONFIGS["dsv3_decode"]
    x = make_attn_inputs(cfg)
    t = to_dev(x, cfg)
    poison_tails(t, lens)
    out = run_attn_ragged(gpu_lib, cfg, t, lens)
    check(out, oracle_attn_full(cfg, x, lens=lens), TOL["bf16"], f"balanced ragged lens[0]={lens[0]}, all outputs")


@pytest.mark.parametrize("mix", ["spread", "skewed"])
@pytest.mark.parametrize("seqlen_q", [1, 3])
def test_ragged_balanced_many_sequences(gpu_lib, seqlen_q, mix):
    """More than 64 sequences: the device plan walks the lengths 64 at a time.  A spread of
    lengths up to 600 keeps the uniform splits; a skewed mix (a few at 600 among short ones)
    takes the equal-chunk plan, with the long sequences cut into several chunks."""
    rng = np.random.default_rng(11)
    B = 130
    if mix == "spread":
        lens = [int(v) for v in rng.integers(seqlen_q, 601, size=B)]
    else:
        lens = [int(v) for v in rng.integers(seqlen_q, 41, size=B)]
        for i in (3, 50, 77, 90, 120):
            lens[i] = int(rng.integers(300, 601))
    lens[7], lens[64], lens[100], lens[129] = 600, seqlen_q, 600, 257
    cfg = dsv3_small(batch=B, cache_batch=B, n_heads=16, seqlen_q=seqlen_q, end_pos=600, cache_len=640)
    x = make_attn_inputs(cfg)
    t = to_dev(x, cfg)
    poison_tails(t, lens)
    out = run_attn_ragged(gpu_lib, cfg, t, lens, path="mfma")
    check(out, oracle_ragged(cfg, x, lens), TOL["bf16"], f"ragged, {B} sequences ({mix}), S={seqlen_q}")


@pytest.mark.parametrize("splits", [0, 8, 24])
def test_ragged_empty_splits_nan_workspace(gpu_lib, splits):
    """Splits past a short sequence's end write only their statistics; the combine must not read
    their partial rows.  The workspace starts as all-ones bytes (NaN in bf16 and fp32)."""
    lens = [1, 40, 700, 999, 2]
    cfg = dsv3_small(batch=len(lens), cache_batch=len(lens), end_pos=999, cache_len=1024)
    x = make_attn_inputs(cfg)
    t = to_dev(x, cfg)
    shape = gpu_lib.attn_shape(t["q_nope"], t["q_pe"], t["kv_cache"], t["wkv_b"])
    need = gpu_lib.absorb_attn_ragged_workspace_size(shape, cfg.end_pos, gpu_lib.MLA_DTYPE_BF16, splits, "mfma")
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    out = torch.full((cfg.batch, cfg.seqlen_q, cfg.n_heads, cfg.v_head_dim), float("nan"), dtype=torch.bfloat16,
                     device="cuda")
    seq = torch.tensor(lens, dtype=torch.int32, device="cuda")
    gpu_lib.absorb_attn(t["q_nope"], t["q_pe"], t["kv_cache"], t["pe_cache"], t["wkv_b"], cfg.end_pos,
                        cfg.softmax_scale, out, num_splits=splits, path="mfma", workspace=ws, seq_lens=seq)
    torch.cuda.synchronize()
    check(out, oracle_ragged(cfg, x, lens), TOL["bf16"], f"ragged, NaN-filled workspace, splits={splits}")


@pytest.mark.parametrize("splits", [1, 3, 16])
def test_ragged_forced_splits(gpu_lib, splits):
    lens = [1, 700, 130, 999]
    cfg = dsv3_small(batch=4, cache_batch=4, end_pos=1000, cache_len=1024)
    x = make_attn_inputs(cfg)
    t = to_dev(x, cfg)
    poison_tails(t, lens)
    out = run_attn_ragged(gpu_lib, cfg, t, lens, path="mfma", splits=splits)
    check(out, oracle_ragged(cfg, x, lens), TOL["bf16"], f"ragged splits={splits}")


def test_ragged_lengths_are_clamped(gpu_lib):
    """Lengths outside [S, bound] behave as the nearest end of that range (and read nothing past it)."""
    cfg = dsv3_small(batch=3, cache_batch=3, seqlen_q=2, end_pos=150, cache_len=160)
    x = make_attn_inputs(cfg)
    t = to_dev(x, cfg)
    poison_tails(t, [150, 150, 150])
    out = run_attn_ragged(gpu_lib, cfg, t, [0, 10 ** 6, -5], path="mfma")
    check(out, oracle_ragged(cfg, x, [2, 150, 2]), TOL["bf16"], "ragged clamped lengths")


@pytest.mark.parametrize("name", RAGGED_WORKLOADS)
def test_full_size_ragged(gpu_lib, name):
    base, lens = ragged_workload(name)
    cfg = ATTN_CONFIGS[base]
    print(f"full-size {name}: B={cfg.batch} lengths {lens.min()}..{lens.max()}", flush=True)
    x = make_attn_inputs(cfg)
    t = to_dev(x, cfg)
    poison_tails(t, lens)
    out = run_attn_ragged(gpu_lib, cfg, t, lens)
    check(out, oracle_attn_full(cfg, x, lens=lens), TOL["bf16"], f"{name} all outputs")


# --------------------------------------------------------------------------------- paged caches

def to_pages(cache, lens, page_size, extra_pages, seed, table=None):
    """Scatter each sequence's rows [0, len) into distinct random pages of a NaN-filled pool (rows
    no sequence owns stay NaN, so any read of them would show in the output), or into the pages
    a given table names.  Returns the pool [num_pages, page_size, D] and block_table
    [B, max_pages] (random entries past a sequence's pages)."""
    rng = np.random.default_rng(seed)
    B, _, D = cache.shape
    need = [-(-int(n) // page_size) for n in lens]
    num_pages = sum(need) + extra_pages
    if table is None:
        ids = rng.permutation(num_pages)
        table = rng.integers(0, num_pages, (B, max(need) + 2)).astype(np.int32)
        used = 0
        for b in range(B):
            for k in range(need[b]):
                table[b, k] = ids[used]
                used += 1
    pool = np.full((num_pages, page_size, D), np.nan, np.float32)
    for b in range(B):
        for k in range(need[b]):
            n = min(page_size, int(lens[b]) - k * page_size)
            pool[table[b, k], :n] = cache[b, k * page_size:k * page_size + n]
    return pool, table


def run_attn_paged(lib, cfg, t, kvp, pep, table, bound, lens=None, path="auto", splits=0):
    out = torch.full((cfg.batch, cfg.seqlen_q, cfg.n_heads, cfg.v_head_dim), float("nan"), dtype=tdtype(cfg),
                     device="cuda")
    seq = None if lens is None else torch.tensor([int(n) for n in lens], dtype=torch.int32, device="cuda")
    lib.absorb_attn(t["q_nope"], t["q_pe"], kvp, pep, t["wkv_b"], bound, cfg.softmax_scale, out, num_splits=splits,
                    path=path, seq_lens=seq, block_table=table)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("path,page_size", [("mfma", 32), ("mfma", 64), ("mfma", 256), ("plain", 16),
                                            ("plain", 48), ("auto", 64)])
@pytest.mark.parametrize("seqlen_q", [1, 3])
def test_paged_small(gpu_lib, path, page_size, seqlen_q):
    cfg = dsv3_small(batch=3, cache_batch=3, seqlen_q=seqlen_q, end_pos=300, cache_len=320)
    if path == "plain":
        cfg = cfg.replace(n_heads=16)
    x = make_attn_inputs(cfg)
    lens = [300, 37, 161]
    kvp, table = to_pages(x["kv_cache"], lens, page_size, 3, 81 + page_size)
    pep, _ = to_pages(x["pe_cache"], lens, page_size, 3, 81 + page_size)  # same seed: same table
    t = to_dev(x, cfg)
    dev = lambda a: torch.from_numpy(a).to("cuda").to(torch.bfloat16)
    out = run_attn_paged(gpu_lib, cfg, t, dev(kvp), dev(pep), torch.from_numpy(table).to("cuda"), cfg.end_pos,
                         lens=lens, path=path)
    ref = O.absorb_attention_paged(x["q_nope"], x["q_pe"], kvp, pep, x["wkv_b"], table, lens, page_size,
                                   cfg.softmax_scale, cfg.v_head_dim)
    check(out, ref, TOL["bf16"], f"paged {path} page_size={page_size} S={seqlen_q}")


@pytest.mark.parametrize("splits", [1, 3, 7, 40])
def test_paged_forced_splits(gpu_lib, splits):
    """Split starts rounded to 32 positions; splits that end up empty; a page of 32 per tile."""
    cfg = dsv3_small(batch=2, cache_batch=2, seqlen_q=2, end_pos=290, cache_len=320)
    x = make_attn_inputs(cfg)
    lens = [290, 75]
    kvp, table = to_pages(x["kv_cache"], lens, 32, 2, 91)
    pep, _ = to_pages(x["pe_cache"], lens, 32, 2, 91)
    t = to_dev(x, cfg)
    dev = lambda a: torch.from_numpy(a).to("cuda").to(torch.bfloat16)
    out = run_attn_paged(gpu_lib, cfg, t, dev(kvp), dev(pep), torch.from_numpy(table).to("cuda"), cfg.end_pos,
                         lens=lens, path="mfma", splits=splits)
    ref = O.absorb_attention_paged(x["q_nope"], x["q_pe"], kvp, pep, x["wkv_b"], table, lens, 32,
                                   cfg.softmax_scale, cfg.v_head_dim)
    check(out, ref, TOL["bf16"], f"paged forced splits={splits}")


def test_paged_uniform_and_clamped_ids(gpu_lib):
    """No seq_lens: every sequence has max_seq_len positions.  Page ids outside the pool are
    clamped into it (here -5 -> 0 and num_pages + 3 -> num_pages - 1), on both kernel paths."""
    cfg = dsv3_small(batch=2, cache_batch=2, end_pos=256, cache_len=256)
    x = make_attn_inputs(cfg)
    table = np.array([[0, 5, 2, 7], [3, 6, 1, 4]], np.int32)  # 8 pages of 64, ids 0 and 7 in use
    kvp, _ = to_pages(x["kv_cache"], [256, 256], 64, 0, 0, table)
    pep, _ = to_pages(x["pe_cache"], [256, 256], 64, 0, 0, table)
    bad = table.copy()
    bad[table == 0] = -5
    bad[table == 7] = 11
    t = to_dev(x, cfg)
    dev = lambda a: torch.from_numpy(a).to("cuda").to(torch.bfloat16)
    ref = O.absorb_attention(x["q_nope"], x["q_pe"], x["kv_cache"], x["pe_cache"], x["wkv_b"], cfg.end_pos,
                             cfg.softmax_scale, cfg.v_head_dim)
    for path in ("mfma", "plain"):
        out = run_attn_paged(gpu_lib, cfg, t, dev(kvp), dev(pep), torch.from_numpy(bad).to("cuda"), cfg.end_pos,
                             path=path)
        check(out, ref, TOL["bf16"], f"paged uniform, clamped ids, {path}")


def test_paged_balanced_long_sequences(gpu_lib):
    """Pages of 32 (a split may span at most 255 of them, 8160 positions), automatic splits and a
    skewed ragged batch whose two long sequences exceed that span: the device plan takes equal
    chunks, with the paged chunk bound evaluated for sequences longer than it, and each chunk
    walks up to 255 page ids held in registers."""
    lens = [12000, 50, 70, 33, 9000, 64, 1, 100]
    cfg = ATTN_CONFIGS["dsv3_decode"].replace(batch=len(lens), cache_batch=len(lens), end_pos=12000,
                                              cache_len=12032)
    print(f"paged balanced: lens {lens} page 32", flush=True)
    x = make_attn_inputs(cfg)
    kvp, table = to_pages(x["kv_cache"], lens, 32, 5, 141)
    pep, _ = to_pages(x["pe_cache"], lens, 32, 5, 141)
    t = to_dev(x, cfg)
    dev = lambda a: torch.from_numpy(a).to("cuda").to(torch.bfloat16)
    out = run_attn_paged(gpu_lib, cfg, t, dev(kvp), dev(pep), torch.from_numpy(table).to("cuda"), cfg.end_pos,
                         lens=lens, path="mfma")
    ref = O.absorb_attention_paged(x["q_nope"], x["q_pe"], kvp, pep, x["wkv_b"], table, lens, 32, cfg.softmax_scale,
                                   cfg.v_head_dim)
    check(out, ref, TOL["bf16"], "paged balanced, sequences longer than one split's page span")


@pytest.mark.parametrize("name,page_size", [("dsv3_decode", 64), ("chunk_prefill", 64), ("long_decode", 256),
                                            ("ragged_decode", 64), ("skewed_decode", 64)])
def test_full_size_paged_matches_contiguous(gpu_lib, name, page_size):
    """The paged kernels read the same rows in the same order as the contiguous ones: outputs are
    bitwise equal at full size (pages in random order in a NaN-filled pool)."""
    lens = None
    if name in RAGGED_WORKLOADS:
        base, lens = ragged_workload(name)
        cfg = ATTN_CONFIGS[base]
    else:
        cfg = ATTN_CONFIGS[name]
    print(f"full-size paged {name}: B={cfg.batch} S={cfg.seqlen_q} T={cfg.end_pos} page={page_size}", flush=True)
    x = make_attn_inputs(cfg)
    t = to_dev(x, cfg)
    B, T = cfg.batch, cfg.end_pos
    npp = T // page_size
    g = torch.Generator(device="cpu")
    g.manual_seed(97)
    num_pages = B * npp + 16
    perm = torch.randperm(num_pages, generator=g)[:B * npp].to(torch.int32)
    table = perm.view(B, npp).contiguous().to("cuda")
    kvp = torch.full((num_pages, page_size, cfg.kv_lora_rank), float("nan"), dtype=torch.bfloat16, device="cuda")
    pep = torch.full((num_pages, page_size, cfg.qk_rope_head_dim), float("nan"), dtype=torch.bfloat16, device="cuda")
    kvp[table.long()] = t["kv_cache"][:B].reshape(B, npp, page_size, -1)
    pep[table.long()] = t["pe_cache"][:B].reshape(B, npp, page_size, -1)
    seq = None if lens is None else torch.tensor(lens, dtype=torch.int32, device="cuda")
    if lens is None:
        ref = run_attn(gpu_lib, cfg, t)
    else:
        ref = run_attn_ragged(gpu_lib, cfg, t, lens)
    out = run_attn_paged(gpu_lib, cfg, t, kvp, pep, table, cfg.end_pos, lens=lens)
    assert torch.isfinite(out).all(), "non-finite outputs"
    assert torch.equal(out, ref), f"paged differs from contiguous: max {float((out.float() - ref.float()).abs().max())}"


# --------------------------------------------------------------------------------- index lists

def make_lists(cfg, lens, topk, seed, empty=None):
    """Per-token lists: mostly positions the token sees, some repeats, and entries that name no
    visible position (-1, the next position, past the length, past the cache); token `empty`
    (b, s) gets only such entries."""
    rng = np.random.default_rng(seed)
    B, S = cfg.batch, cfg.seqlen_q
    idx = np.zeros((B, S, topk), np.int32)
    for b in range(B):
        for s_ in range(S):
            pos = int(lens[b]) - S + s_
            row = rng.integers(0, pos + 1, topk)
            row[rng.random(topk) < 0.05] = -1
            row[rng.random(topk) < 0.03] = pos + 1
            row[rng.random(topk) < 0.02] = cfg.cache_len + 100
            if topk > 4:
                row[3] = row[2]
            idx[b, s_] = row
    if empty is not None:
        idx[empty] = -1
        idx[empty][::2] = int(lens[empty[0]]) - S + empty[1] + 1
    return idx


def run_attn_sparse(lib, cfg, t, idx, lens=None, path="auto", splits=0):
    out = torch.full((cfg.batch, cfg.seqlen_q, cfg.n_heads, cfg.v_head_dim), float("nan"), dtype=tdtype(cfg),
                     device="cuda")
    seq = None if lens is None else torch.tensor([int(n) for n in lens], dtype=torch.int32, device="cuda")
    lib.absorb_attn(t["q_nope"], t["q_pe"], t["kv_cache"], t["pe_cache"], t["wkv_b"], cfg.end_pos,
                    cfg.softmax_scale, out, num_splits=splits, path=path, seq_lens=seq,
                    indices=torch.from_numpy(np.ascontiguousarray(idx, np.int32)).to("cuda"))
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("path", ["mfma", "plain", "auto"])
@pytest.mark.parametrize("seqlen_q,topk", [(1, 37), (1, 300), (3, 64), (1, 1)])
def test_sparse_small(gpu_lib, path, seqlen_q, topk):
    cfg = dsv3_small(batch=3, cache_batch=3, seqlen_q=seqlen_q, end_pos=300, cache_len=320)
    if path == "plain":
        cfg = cfg.replace(n_heads=16)
    x = make_attn_inputs(cfg)
    lens = [300, 41, 170]
    idx = make_lists(cfg, lens, topk, 101 + topk, empty=(1, seqlen_q - 1))
    t = to_dev(x, cfg)
    poison_tails(t, lens)
    out = run_attn_sparse(gpu_lib, cfg, t, idx, lens, path=path)
    ref = O.absorb_attention_sparse(x["q_nope"], x["q_pe"], x["kv_cache"], x["pe_cache"], x["wkv_b"], idx, lens,
                                    cfg.softmax_scale, cfg.v_head_dim)
    check(out, ref, TOL["bf16"], f"sparse {path} S={seqlen_q} topk={topk}")
    assert torch.all(out[1, seqlen_q - 1] == 0), "a token with no visible entry must give 0"


@pytest.mark.parametrize("path,splits", [("mfma", 1), ("mfma", 2), ("mfma", 5), ("mfma", 9), ("plain", 4)])
def test_sparse_forced_splits(gpu_lib, path, splits):
    """Splits over list entries (one not a multiple of 32, empty ones), with a token whose list
    names nothing visible in any split."""
    cfg = dsv3_small(batch=2, cache_batch=2, seqlen_q=1, end_pos=280, cache_len=300)
    x = make_attn_inputs(cfg)
    lens = [280, 90]
    idx = make_lists(cfg, lens, 250, 111 + splits, empty=(0, 0))
    t = to_dev(x, cfg)
    out = run_attn_sparse(gpu_lib, cfg, t, idx, lens, path=path, splits=splits)
    ref = O.absorb_attention_sparse(x["q_nope"], x["q_pe"], x["kv_cache"], x["pe_cache"], x["wkv_b"], idx, lens,
                                    cfg.softmax_scale, cfg.v_head_dim)
    check(out, ref, TOL["bf16"], f"sparse {path} splits={splits}")
    assert torch.all(out[0, 0] == 0)


@pytest.mark.parametrize("seqlen_q", [1, 4])
def test_sparse_full_list_equals_dense(gpu_lib, seqlen_q):
    """A list naming every cache position (random order; later positions masked per token) gives
    the dense causal result of mla_absorb_attn, both on the GPU."""
    cfg = dsv3_small(batch=2, cache_batch=2, seqlen_q=seqlen_q, end_pos=256, cache_len=256)
    x = make_attn_inputs(cfg)
    rng = np.random.default_rng(121)
    idx = np.stack([np.stack([rng.permutation(cfg.cache_len) for _ in range(seqlen_q)]) for _ in range(cfg.batch)])
    t = to_dev(x, cfg)
    sp = run_attn_sparse(gpu_lib, cfg, t, idx)
    dense = run_attn(gpu_lib, cfg, t)
    check(sp, dense.float().cpu().double().numpy(), TOL["bf16"], f"full list vs dense S={seqlen_q}")


@pytest.mark.parametrize("name,topk", [("dsv3_decode", 2048), ("long_decode", 2048), ("dsv3_decode", 100)])
def test_full_size_sparse(gpu_lib, name, topk):
    cfg = ATTN_CONFIGS[name]
    print(f"full-size sparse {name}: B={cfg.batch} T={cfg.end_pos} topk={topk}", flush=True)
    x = make_attn_inputs(cfg)
    rng = np.random.default_rng(131)
    idx = np.stack([np.stack([rng.choice(cfg.end_pos, topk, replace=False) for _ in range(cfg.seqlen_q)])
                    for _ in range(cfg.batch)]).astype(np.int32)
    t = to_dev(x, cfg)
    out = run_attn_sparse(gpu_lib, cfg, t, idx)
    ref = O.absorb_attention_sparse(x["q_nope"], x["q_pe"], x["kv_cache"], x["pe_cache"], x["wkv_b"], idx,
                                    [cfg.end_pos] * cfg.batch, cfg.softmax_scale, cfg.v_head_dim)
    check(out, ref, TOL["bf16"], f"{name} topk={topk} all outputs")


# --------------------------------------------------------------------------------- strided views

def strided_views(t, cfg, pad_out=64):
    """The same inputs as views of combined tensors, the way a model holds them: q_nope and q_pe
    the two parts of one [B, S, H, Dn + R] query, kv_cache and pe_cache the two parts of one
    [Bmax, Tmax, C + R] cache (with a spare position row per sequence, so the batch stride is not
    Tmax rows), and out the first Dv columns of a wider NaN-filled buffer.  Returns (views, out
    buffer); the views hold bitwise the values of t."""
    dt = t["q_nope"].dtype
    Dn, R, C = cfg.qk_nope_head_dim, cfg.qk_rope_head_dim, cfg.kv_lora_rank
    q = torch.cat([t["q_nope"], t["q_pe"]], dim=-1).contiguous()
    Bm, Tm = t["kv_cache"].shape[:2]
    cache = torch.full((Bm, Tm + 1, C + R), float("nan"), dtype=dt, device="cuda")
    cache[:, :Tm, :C] = t["kv_cache"]
    cache[:, :Tm, C:] = t["pe_cache"]
    obuf = torch.full((cfg.batch, cfg.seqlen_q, cfg.n_heads, cfg.v_head_dim + pad_out), float("nan"), dtype=dt,
                      device="cuda")
    v = dict(t, q_nope=q[..., :Dn], q_pe=q[..., Dn:], kv_cache=cache[:, :Tm, :C], pe_cache=cache[:, :Tm, C:])
    return v, obuf


@pytest.mark.parametrize("path", ["mfma", "plain"])
@pytest.mark.parametrize("seqlen_q", [1, 3])
def test_strided_views(gpu_lib, path, seqlen_q):
    """Query halves of one tensor, caches interleaved in one 576-wide cache and out as a view: the
    same result as dense tensors (bitwise), the oracle's at the bf16 bar, and out's padding
    untouched."""
    cfg = dsv3_small(seqlen_q=seqlen_q)
    if path == "plain":
        cfg = cfg.replace(n_heads=16)
    x = make_attn_inputs(cfg)
    t = to_dev(x, cfg)
    dense = run_attn(gpu_lib, cfg, t, path=path)
    v, obuf = strided_views(t, cfg)
    out = obuf[..., :cfg.v_head_dim]
    assert not out.is_contiguous() and not v["q_nope"].is_contiguous() and not v["kv_cache"].is_contiguous()
    gpu_lib.absorb_attn(v["q_nope"], v["q_pe"], v["kv_cache"], v["pe_cache"], v["wkv_b"], cfg.end_pos,
                        cfg.softmax_scale, out, path=path)
    torch.cuda.synchronize()
    assert torch.isnan(obuf[..., cfg.v_head_dim:]).all(), "a store landed in out's padding"
    assert torch.equal(out, dense), "strided views differ from dense tensors"
    check(out, oracle_attn(cfg, x), TOL["bf16"], f"strided views {path} S={seqlen_q}")


def test_strided_views_f32(gpu_lib):
    cfg = ATTN_CONFIGS["tiny_f32"]
    x = make_attn_inputs(cfg)
    t = to_dev(x, cfg)
    v, obuf = strided_views(t, cfg, pad_out=4)
    out = obuf[..., :cfg.v_head_dim]
    gpu_lib.absorb_attn(v["q_nope"], v["q_pe"], v["kv_cache"], v["pe_cache"], v["wkv_b"], cfg.end_pos,
                        cfg.softmax_scale, out)
    torch.cuda.synchronize()
    assert torch.isnan(obuf[..., cfg.v_head_dim:]).all()
    check(out, oracle_attn(cfg, x), TOL["f32"], "tiny_f32 strided views")


def test_strided_views_ragged_sparse_paged(gpu_lib):
    """Strides through the ragged, index-list and paged entry points (pools of 576-wide rows)."""
    lens = [300, 37, 161]
    cfg = dsv3_small(batch=3, cache_batch=3, seqlen_q=2, end_pos=300, cache_len=320)
    x = make_attn_inputs(cfg)
    t = to_dev(x, cfg)
    v, obuf = strided_views(t, cfg)
    out = obuf[..., :cfg.v_head_dim]
    seq = torch.tensor(lens, dtype=torch.int32, device="cuda")
    gpu_lib.absorb_attn(v["q_nope"], v["q_pe"], v["kv_cache"], v["pe_cache"], v["wkv_b"], cfg.end_pos,
                        cfg.softmax_scale, out, seq_lens=seq)
    torch.cuda.synchronize()
    assert torch.equal(out, run_attn_ragged(gpu_lib, cfg, t, lens)), "ragged: strided differs from dense"
    check(out, oracle_ragged(cfg, x, lens), TOL["bf16"], "ragged strided views")

    idx = make_lists(cfg, lens, 64, 5)
    obuf.fill_(float("nan"))
    gpu_lib.absorb_attn(v["q_nope"], v["q_pe"], v["kv_cache"], v["pe_cache"], v["wkv_b"], cfg.end_pos,
                        cfg.softmax_scale, out, seq_lens=seq, indices=torch.from_numpy(idx).to("cuda"))
    torch.cuda.synchronize()
    ref = O.absorb_attention_sparse(x["q_nope"], x["q_pe"], x["kv_cache"], x["pe_cache"], x["wkv_b"], idx, lens,
                                    cfg.softmax_scale, cfg.v_head_dim)
    check(out, ref, TOL["bf16"], "index lists, strided views")

    kvp, table = to_pages(x["kv_cache"], lens, 32, 3, 71)
    pep, _ = to_pages(x["pe_cache"], lens, 32, 3, 71)
    pool = torch.cat([torch.from_numpy(kvp), torch.from_numpy(pep)], dim=-1).to("cuda").to(torch.bfloat16)
    obuf.fill_(float("nan"))
    gpu_lib.absorb_attn(v["q_nope"], v["q_pe"], pool[..., :cfg.kv_lora_rank], pool[..., cfg.kv_lora_rank:],
                        v["wkv_b"], cfg.end_pos, cfg.softmax_scale, out, seq_lens=seq,
                        block_table=torch.from_numpy(table).to("cuda"))
    torch.cuda.synchronize()
    ref = O.absorb_attention_paged(x["q_nope"], x["q_pe"], kvp, pep, x["wkv_b"], table, lens, 32, cfg.softmax_scale,
                                   cfg.v_head_dim)
    check(out, ref, TOL["bf16"], "paged 576-wide pools, strided views")
    assert torch.isnan(obuf[..., cfg.v_head_dim:]).all()


def test_full_size_strided_views(gpu_lib):
    """dsv3_decode with q and the caches as views of combined tensors: every output element
    against the oracle."""
    cfg = ATTN_CONFIGS["dsv3_decode"]
    print(f"full-size strided views: B={cfg.batch} T={cfg.end_pos}", flush=True)
    x = make_attn_inputs(cfg)
    t = to_dev(x, cfg)
    v, obuf = strided_views(t, cfg)
    del t
    out = obuf[..., :cfg.v_head_dim]
    gpu_lib.absorb_attn(v["q_nope"], v["q_pe"], v["kv_cache"], v["pe_cache"], v["wkv_b"], cfg.end_pos,
                        cfg.softmax_scale, out)
    torch.cuda.synchronize()
    assert torch.isnan(obuf[..., cfg.v_head_dim:]).all()
    check(out, oracle_attn_full(cfg, x), TOL["bf16"], "dsv3_decode strided views, all outputs")


# --------------------------------------------------------------------------------- fp32 extensions

@pytest.mark.parametrize("seqlen_q", [1, 2])
def test_tiny_f32_extensions(gpu_lib, seqlen_q):
    """The fp32 tiny shape (plain kernels) through every extension entry point, at the fp32
    tolerance: ragged lengths, paged caches with page sizes 8 and 5, index lists, and naive
    attention over expanded keys and values."""
    cfg = ATTN_CONFIGS["tiny_f32"].replace(batch=3, cache_batch=3, seqlen_q=seqlen_q, seed=17)
    x = make_attn_inputs(cfg)
    lens = [seqlen_q, 57, cfg.cache_len]
    t = to_dev(x, cfg)
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to("cuda")
    out = run_attn_ragged(gpu_lib, cfg, t, lens, path="plain")
    check(out, oracle_ragged(cfg, x, lens), TOL["f32"], f"f32 ragged S={seqlen_q}")
    for page_size in (8, 5):
        kvp, table = to_pages(x["kv_cache"], lens, page_size, 2, 151 + page_size)
        pep, _ = to_pages(x["pe_cache"], lens, page_size, 2, 151 + page_size)
        out = run_attn_paged(gpu_lib, cfg, t, f32(kvp), f32(pep), torch.from_numpy(table).to("cuda"), cfg.end_pos,
                             lens=lens, path="plain")
        ref = O.absorb_attention_paged(x["q_nope"], x["q_pe"], kvp, pep, x["wkv_b"], table, lens, page_size,
                                       cfg.softmax_scale, cfg.v_head_dim)
        check(out, ref, TOL["f32"], f"f32 paged page_size={page_size} S={seqlen_q}")
    idx = make_lists(cfg, lens, 40, 161, empty=(0, 0))
    out = run_attn_sparse(gpu_lib, cfg, t, idx, lens, path="plain")
    ref = O.absorb_attention_sparse(x["q_nope"], x["q_pe"], x["kv_cache"], x["pe_cache"], x["wkv_b"], idx, lens,
                                    cfg.softmax_scale, cfg.v_head_dim)
    check(out, ref, TOL["f32"], f"f32 index lists S={seqlen_q}")
    kn, vn = O.naive_kv(x["kv_cache"], x["wkv_b"], cfg.cache_batch, cfg.cache_len, cfg.n_heads,
                        cfg.qk_nope_head_dim, cfg.v_head_dim)
    kh, vh = kn.transpose(2, 0, 1, 3), vn.transpose(2, 0, 1, 3)
    out = torch.full((cfg.batch, seqlen_q, cfg.n_heads, cfg.v_head_dim), float("nan"), device="cuda")
    gpu_lib.naive_attn(t["q_nope"], t["q_pe"], f32(kh), f32(vh), t["pe_cache"], cfg.end_pos, cfg.softmax_scale, out,
                       path="plain")
    torch.cuda.synchronize()
    ref = O.attention_over_kv(x["q_nope"], x["q_pe"], kh, vh, x["pe_cache"], cfg.end_pos, cfg.softmax_scale)
    check(out, ref, TOL["f32"], f"f32 naive attention S={seqlen_q}")


# --------------------------------------------------------------------------------- cache append

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("ragged", [False, True])
def test_cache_append(gpu_lib, dtype, ragged):
    """Written rows match the oracle's normalised latent and rope key; every other row is unchanged."""
    B, S, C, R, Bmax, Tmax, end_pos, eps = 3, 4, 512, 64, 4, 96, 80, 1e-6
    rng = np.random.default_rng(41)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    cast = (lambda a: a.astype(np.float32)) if dtype == "f32" else (lambda a: round_bf16(a))
    x, kp = cast(rng.normal(size=(B, S, C))), cast(rng.normal(size=(B, S, R)))
    w = cast(1.0 + 0.14 * rng.normal(size=C))
    kv0, pe0 = cast(rng.normal(size=(Bmax, Tmax, C))), cast(rng.normal(size=(Bmax, Tmax, R)))
    lens = [S, 37, end_pos] if ragged else None
    dev = lambda a: torch.from_numpy(a).to("cuda").to(tdt)
    kv, pe = dev(kv0), dev(pe0)
    seq = torch.tensor(lens, dtype=torch.int32, device="cuda") if ragged else None
    gpu_lib.cache_append(dev(x), dev(kp), dev(w), eps, end_pos, kv, pe, seq_lens=seq)
    torch.cuda.synchronize()
    kr, pr = O.cache_append(x, kp, w, eps, kv0, pe0, end_pos=end_pos, seq_lens=lens)
    new = np.zeros((Bmax, Tmax), bool)
    for b in range(B):
        n = lens[b] if ragged else end_pos
        new[b, n - S:n] = True
    g_kv, g_pe = kv.float().cpu().numpy(), pe.float().cpu().numpy()
    assert np.array_equal(g_kv[~new], kv0[~new]) and np.array_equal(g_pe[~new], pe0[~new]), "untouched rows changed"
    assert np.array_equal(g_pe[new], pr[new].astype(np.float32)), "rope rows are copied exactly"
    check(g_kv[new].astype(np.float64), kr[new], TOL[dtype], f"append {dtype} ragged={ragged} latent rows")


def test_append_then_attend(gpu_lib):
    """One decode step end to end: append each sequence's new token, then attend over the cache."""
    cfg = dsv3_small(batch=3, cache_batch=3, end_pos=200, cache_len=256)
    x = make_attn_inputs(cfg)
    rng = np.random.default_rng(43)
    c_new = round_bf16(rng.normal(size=(cfg.batch, 1, cfg.kv_lora_rank)))
    kp_new = round_bf16(rng.normal(size=(cfg.batch, 1, cfg.qk_rope_head_dim)))
    w = round_bf16(1.0 + 0.14 * rng.normal(size=cfg.kv_lora_rank))
    t = to_dev(x, cfg)
    dev = lambda a: torch.from_numpy(a).to("cuda").to(torch.bfloat16)
    gpu_lib.cache_append(dev(c_new), dev(kp_new), dev(w), 1e-6, cfg.end_pos, t["kv_cache"], t["pe_cache"])
    out = run_attn(gpu_lib, cfg, t, path="mfma")
    kv, pe = O.cache_append(c_new, kp_new, w, 1e-6, x["kv_cache"], x["pe_cache"], end_pos=cfg.end_pos)
    # the GPU attends to the bf16-rounded appended rows; the oracle rounds them the same way
    kv_b = np.array(kv)
    kv_b[:, cfg.end_pos - 1] = round_bf16(kv[:, cfg.end_pos - 1])
    ref = O.absorb_attention(x["q_nope"], x["q_pe"], kv_b, pe, x["wkv_b"], cfg.end_pos, cfg.softmax_scale,
                             cfg.v_head_dim)
    check(out, ref, TOL["bf16"], "append + attend")


@pytest.mark.parametrize("dtype,page_size,ragged", [("f32", 16, False), ("bf16", 64, True), ("bf16", 5, True)])
def test_cache_append_paged(gpu_lib, dtype, page_size, ragged):
    """Rows appended into page pools match the oracle's; every other pool row is unchanged."""
    B, S, C, R, T, eps = 3, 4, 512, 64, 192, 1e-6
    rng = np.random.default_rng(45)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    cast = (lambda a: a.astype(np.float32)) if dtype == "f32" else (lambda a: round_bf16(a))
    x, kp = cast(rng.normal(size=(B, S, C))), cast(rng.normal(size=(B, S, R)))
    w = cast(1.0 + 0.14 * rng.normal(size=C))
    npp = -(-T // page_size)
    num_pages = B * npp + 4
    table = rng.permutation(num_pages)[:B * npp].reshape(B, npp).astype(np.int32)
    kv0, pe0 = cast(rng.normal(size=(num_pages, page_size, C))), cast(rng.normal(size=(num_pages, page_size, R)))
    lens = [S, 101, T] if ragged else None
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(tdt)
    kv, pe = dev(kv0), dev(pe0)
    seq = torch.tensor(lens, dtype=torch.int32, device="cuda") if ragged else None
    gpu_lib.cache_append(dev(x), dev(kp), dev(w), eps, T, kv, pe, seq_lens=seq,
                         block_table=torch.from_numpy(table).to("cuda"))
    torch.cuda.synchronize()
    kr, pr = O.cache_append_paged(x, kp, w, eps, kv0, pe0, table, page_size, end_pos=T, seq_lens=lens)
    new = np.zeros((num_pages, page_size), bool)
    for b in range(B):
        n = lens[b] if ragged else T
        for p_ in range(n - S, n):
            new[table[b, p_ // page_size], p_ % page_size] = True
    g_kv, g_pe = kv.float().cpu().numpy(), pe.float().cpu().numpy()
    assert np.array_equal(g_kv[~new], kv0[~new]) and np.array_equal(g_pe[~new], pe0[~new]), "untouched rows changed"
    assert np.array_equal(g_pe[new], pr[new].astype(np.float32)), "rope rows are copied exactly"
    check(g_kv[new].astype(np.float64), kr[new], TOL[dtype], f"paged append {dtype} page={page_size} latent rows")


def test_append_then_attend_paged(gpu_lib):
    """One decode step over paged caches: append each sequence's new token, then paged attention."""
    cfg = dsv3_small(batch=3, cache_batch=3, end_pos=200, cache_len=256)
    x = make_attn_inputs(cfg)
    lens = [200, 77, 130]
    kvp, table = to_pages(x["kv_cache"], lens, 64, 2, 47)
    pep, _ = to_pages(x["pe_cache"], lens, 64, 2, 47)
    rng = np.random.default_rng(49)
    c_new = round_bf16(rng.normal(size=(cfg.batch, 1, cfg.kv_lora_rank)))
    kp_new = round_bf16(rng.normal(size=(cfg.batch, 1, cfg.qk_rope_head_dim)))
    w = round_bf16(1.0 + 0.14 * rng.normal(size=cfg.kv_lora_rank))
    t = to_dev(x, cfg)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to("cuda").to(torch.bfloat16)
    kv_d, pe_d, tb = dev(kvp), dev(pep), torch.from_numpy(table).to("cuda")
    seq = torch.tensor(lens, dtype=torch.int32, device="cuda")
    gpu_lib.cache_append(dev(c_new), dev(kp_new), dev(w), 1e-6, cfg.end_pos, kv_d, pe_d, seq_lens=seq, block_table=tb)
    out = run_attn_paged(gpu_lib, cfg, t, kv_d, pe_d, tb, cfg.end_pos, lens=lens, path="mfma")
    kva, pea = O.cache_append_paged(c_new, kp_new, w, 1e-6, kvp, pep, table, 64, end_pos=cfg.end_pos, seq_lens=lens)
    # the GPU attends to the bf16-rounded appended rows; the oracle rounds them the same way
    for b, n in enumerate(lens):
        page, slot = table[b, (n - 1) // 64], (n - 1) % 64
        kva[page, slot] = round_bf16(kva[page, slot])
    ref = O.absorb_attention_paged(x["q_nope"], x["q_pe"], kva, pea, x["wkv_b"], table, lens, 64, cfg.softmax_scale,
                                   cfg.v_head_dim)
    check(out, ref, TOL["bf16"], "paged append + attend")


def _append_inputs(cfg, S, seed):
    rng = np.random.default_rng(seed)
    cast = (lambda a: a.astype(np.float32)) if cfg.dtype == "f32" else round_bf16
    c_new = cast(rng.normal(size=(cfg.batch, S, cfg.kv_lora_rank)))
    kp_new = cast(rng.normal(size=(cfg.batch, S, cfg.qk_rope_head_dim)))
    w = cast(1.0 + 0.14 * rng.normal(size=cfg.kv_lora_rank))
    return c_new, kp_new, w


@pytest.mark.parametrize("dtype,S,ragged,strided,path", [
    ("bf16", 1, False, False, "mfma"), ("bf16", 5, True, False, "mfma"), ("bf16", 1, True, True, "mfma"),
    ("bf16", 130, False, False, "mfma"), ("bf16", 3, True, False, "plain"), ("f32", 3, False, False, "auto"),
    ("f32", 2, True, True, "auto")])
def test_fused_append_attend(gpu_lib, dtype, S, ragged, strided, path):
    """mla_absorb_attn_append: the caches and the output equal, bit for bit, those of the cache
    append followed by the attention call on copies of the same buffers, and the output matches the
    oracle's append followed by absorb attention."""
    if dtype == "bf16":
        cfg = dsv3_small(batch=3, cache_batch=4, seqlen_q=S, end_pos=260, cache_len=300)
    else:
        cfg = ATTN_CONFIGS["tiny_f32"].replace(batch=3, cache_batch=4, seqlen_q=S, end_pos=100, cache_len=120)
    x = make_attn_inputs(cfg)
    c_new, kp_new, w = _append_inputs(cfg, S, 61 + S)
    eps = 1e-6
    lens = [cfg.end_pos, S + 20, 150 if dtype == "bf16" else 60] if ragged else None
    t = to_dev(x, cfg)
    tdt = tdtype(cfg)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(tdt)
    seq = None if lens is None else torch.tensor(lens, dtype=torch.int32, device="cuda")

    def caches():
        if not strided:
            return t["kv_cache"].clone(), t["pe_cache"].clone()
        # rows padded to a wider stride: the appended rows must land where the attention reads
        kvw = torch.full((cfg.cache_batch, cfg.cache_len, cfg.kv_lora_rank + 64), float("nan"), dtype=tdt, device="cuda")
        pew = torch.full((cfg.cache_batch, cfg.cache_len, cfg.qk_rope_head_dim + 32), float("nan"), dtype=tdt,
                         device="cuda")
        kvw[..., :cfg.kv_lora_rank] = t["kv_cache"]
        pew[..., :cfg.qk_rope_head_dim] = t["pe_cache"]
        return kvw[..., :cfg.kv_lora_rank], pew[..., :cfg.qk_rope_head_dim]

    out_f = torch.full((cfg.batch, S, cfg.n_heads, cfg.v_head_dim), float("nan"), dtype=tdt, device="cuda")
    kv_f, pe_f = caches()
    gpu_lib.absorb_attn(t["q_nope"], t["q_pe"], kv_f, pe_f, t["wkv_b"], cfg.end_pos, cfg.softmax_scale, out_f,
                        path=path, seq_lens=seq, append=(dev(c_new), dev(kp_new), dev(w), eps))
    out_2 = torch.full_like(out_f, float("nan"))
    kv_2, pe_2 = caches()
    if strided:  # the stand-alone append takes dense caches: append into dense copies, then copy in
        kd, pd = kv_2.contiguous(), pe_2.contiguous()
        gpu_lib.cache_append(dev(c_new), dev(kp_new), dev(w), eps, cfg.end_pos, kd, pd, seq_lens=seq)
        kv_2.copy_(kd)
        pe_2.copy_(pd)
    else:
        gpu_lib.cache_append(dev(c_new), dev(kp_new), dev(w), eps, cfg.end_pos, kv_2, pe_2, seq_lens=seq)
    gpu_lib.absorb_attn(t["q_nope"], t["q_pe"], kv_2, pe_2, t["wkv_b"], cfg.end_pos, cfg.softmax_scale, out_2,
                        path=path, seq_lens=seq)
    torch.cuda.synchronize()
    what = f"fused append {dtype} S={S} ragged={ragged} strided={strided} {path}"
    assert torch.equal(kv_f.view(torch.int16 if dtype == "bf16" else torch.int32),
                       kv_2.view(torch.int16 if dtype == "bf16" else torch.int32)), f"{what}: kv_cache differs"
    assert torch.equal(pe_f.view(torch.int16 if dtype == "bf16" else torch.int32),
                       pe_2.view(torch.int16 if dtype == "bf16" else torch.int32)), f"{what}: pe_cache differs"
    assert torch.equal(out_f.view(torch.int16 if dtype == "bf16" else torch.int32),
                       out_2.view(torch.int16 if dtype == "bf16" else torch.int32)), f"{what}: out differs"
    # the oracle: append, the GPU's rounding of the written rows, then absorb attention
    kv_o, pe_o = O.cache_append(c_new, kp_new, w, eps, x["kv_cache"], x["pe_cache"], end_pos=cfg.end_pos,
                                seq_lens=lens)
    kv_o = np.array(kv_o)
    g_kv = kv_f.float().cpu().numpy()
    for b in range(cfg.batch):
        n = lens[b] if ragged else cfg.end_pos
        check(g_kv[b, n - S:n].astype(np.float64), kv_o[b, n - S:n], TOL[dtype], f"{what}: latent rows of {b}")
        kv_o[b, n - S:n] = g_kv[b, n - S:n]
    if lens is None:
        ref = O.absorb_attention(x["q_nope"], x["q_pe"], kv_o, pe_o, x["wkv_b"], cfg.end_pos, cfg.softmax_scale,
                                 cfg.v_head_dim)
    else:
        ref = O.absorb_attention_ragged(x["q_nope"], x["q_pe"], kv_o, pe_o, x["wkv_b"], lens, cfg.softmax_scale,
                                        cfg.v_head_dim)
    check(out_f, ref, TOL[dtype], what)


@pytest.mark.parametrize("dtype,page_size,S,path", [("bf16", 64, 1, "mfma"), ("bf16", 64, 4, "mfma"),
                                                    ("bf16", 32, 3, "plain"), ("f32", 16, 2, "auto")])
def test_fused_append_attend_paged(gpu_lib, dtype, page_size, S, path):
    """mla_absorb_attn_paged_append equals the paged append followed by paged attention, bit for bit."""
    if dtype == "bf16":
        cfg = dsv3_small(batch=3, cache_batch=3, seqlen_q=S, end_pos=200, cache_len=256)
        lens = [200, 77, 130]
    else:
        cfg = ATTN_CONFIGS["tiny_f32"].replace(batch=3, cache_batch=3, seqlen_q=S, end_pos=100, cache_len=112)
        lens = [100, 37, 64]
    x = make_attn_inputs(cfg)
    kvp, table = to_pages(x["kv_cache"], lens, page_size, 2, 53)
    pep, _ = to_pages(x["pe_cache"], lens, page_size, 2, 53)
    c_new, kp_new, w = _append_inputs(cfg, S, 67 + S)
    t = to_dev(x, cfg)
    tdt = tdtype(cfg)
    bits = torch.int16 if dtype == "bf16" else torch.int32
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to("cuda").to(tdt)
    tb = torch.from_numpy(table).to("cuda")
    seq = torch.tensor(lens, dtype=torch.int32, device="cuda")
    outs, pools = [], []
    for fused in (True, False):
        kv_d, pe_d = dev(kvp), dev(pep)
        out = torch.full((cfg.batch, S, cfg.n_heads, cfg.v_head_dim), float("nan"), dtype=tdt, device="cuda")
        if fused:
            gpu_lib.absorb_attn(t["q_nope"], t["q_pe"], kv_d, pe_d, t["wkv_b"], cfg.end_pos, cfg.softmax_scale, out,
                                path=path, seq_lens=seq, block_table=tb, append=(dev(c_new), dev(kp_new), dev(w), 1e-6))
        else:
            gpu_lib.cache_append(dev(c_new), dev(kp_new), dev(w), 1e-6, cfg.end_pos, kv_d, pe_d, seq_lens=seq,
                                 block_table=tb)
            gpu_lib.absorb_attn(t["q_nope"], t["q_pe"], kv_d, pe_d, t["wkv_b"], cfg.end_pos, cfg.softmax_scale, out,
                                path=path, seq_lens=seq, block_table=tb)
        torch.cuda.synchronize()
        outs.append(out)
        pools.append((kv_d, pe_d))
    for a, b in zip((outs[0],) + pools[0], (outs[1],) + pools[1]):
        # NaN rows of the pools (pages no sequence owns) compare equal bit for bit
        assert torch.equal(a.view(bits), b.view(bits)), f"fused paged append ({dtype}, {path}) differs from the two calls"
    # and the oracle: paged append, the GPU's rounding of the written rows, paged attention
    kva, pea = O.cache_append_paged(c_new, kp_new, w, 1e-6, kvp, pep, table, page_size, end_pos=cfg.end_pos,
                                    seq_lens=lens)
    g_kv = pools[0][0].float().cpu().numpy()
    for b, n in enumerate(lens):
        for p_ in range(n - S, n):
            page, slot = table[b, p_ // page_size], p_ % page_size
            kva[page, slot] = g_kv[page, slot]
    ref = O.absorb_attention_paged(x["q_nope"], x["q_pe"], kva, pea, x["wkv_b"], table, lens, page_size,
                                   cfg.softmax_scale, cfg.v_head_dim)
    check(outs[0], ref, TOL[dtype], f"fused paged append {dtype} page={page_size} S={S} {path}")


# --------------------------------------------------------------------------------- naive route

def head_major_kv(x, cfg):
    """The oracle's naive keys and values of every cache row, head-major [H, Bmax, Tmax, D], bf16-rounded."""
    kn, vn = O.naive_kv(x["kv_cache"], x["wkv_b"], cfg.cache_batch, cfg.cache_len, cfg.n_heads,
                        cfg.qk_nope_head_dim, cfg.v_head_dim)
    return round_bf16(kn.transpose(2, 0, 1, 3)), round_bf16(vn.transpose(2, 0, 1, 3))


def run_naive(lib, cfg, t, k, v, path="auto"):
    out = torch.full((cfg.batch, cfg.seqlen_q, cfg.n_heads, cfg.v_head_dim), float("nan"), dtype=torch.bfloat16,
                     device="cuda")
    lib.naive_attn(t["q_nope"], t["q_pe"], k, v, t["pe_cache"], cfg.end_pos, cfg.softmax_scale, out, path=path)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("path", ["plain", "mfma"])
@pytest.mark.parametrize("kw", [
    dict(seqlen_q=1, end_pos=300),    # decode
    dict(seqlen_q=5, end_pos=200),    # causal chunk
    dict(seqlen_q=130, end_pos=170),  # two query blocks, the second of 2 rows
    dict(seqlen_q=64, end_pos=64),    # chunk covering the whole prefix
])
def test_naive_attn(gpu_lib, path, kw):
    cfg = dsv3_small(batch=2, cache_batch=3, cache_len=320, n_heads=16, **kw)
    x = make_attn_inputs(cfg)
    kh, vh = head_major_kv(x, cfg)
    t = to_dev(x, cfg)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to("cuda").to(torch.bfloat16)
    out = run_naive(gpu_lib, cfg, t, dev(kh), dev(vh), path=path)
    ref = O.attention_over_kv(x["q_nope"], x["q_pe"], kh, vh, x["pe_cache"], cfg.end_pos, cfg.softmax_scale)
    check(out, ref, TOL["bf16"], f"naive attention {kw} {path}")


def test_naive_route_matches_absorb_on_gpu(gpu_lib):
    """The pages' FAQ invariant with both routes on the GPU: raw latents appended (normalised) into
    the cache feed the absorb route; the same latents expanded feed the naive route."""
    cfg = dsv3_small(batch=2, cache_batch=2, seqlen_q=3, end_pos=250, cache_len=256, n_heads=32)
    x = make_attn_inputs(cfg)
    rng = np.random.default_rng(61)
    raw = round_bf16(rng.normal(size=(cfg.cache_batch, cfg.cache_len, cfg.kv_lora_rank)))
    w = round_bf16(1.0 + 0.14 * rng.normal(size=cfg.kv_lora_rank))
    t = to_dev(x, cfg)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to("cuda").to(torch.bfloat16)
    # absorb route: every position appended from the raw latent (positions 0..Tmax-1)
    gpu_lib.cache_append(dev(raw), dev(np.zeros((cfg.cache_batch, cfg.cache_len, cfg.qk_rope_head_dim))), dev(w),
                         1e-6, cfg.cache_len, t["kv_cache"], torch.empty_like(t["pe_cache"]))
    a = run_attn(gpu_lib, cfg, t, path="mfma")
    # naive route: the expansion of the same raw latents, head-major [H, Bmax*Tmax, D]
    k, v = gpu_lib.expand_kv(dev(raw.reshape(-1, cfg.kv_lora_rank)), dev(w), t["wkv_b"], cfg.n_heads,
                             cfg.qk_nope_head_dim, cfg.v_head_dim, 1e-6)
    n = run_naive(gpu_lib, cfg, t, k.view(cfg.n_heads, cfg.cache_batch, cfg.cache_len, -1),
                  v.view(cfg.n_heads, cfg.cache_batch, cfg.cache_len, -1), path="mfma")
    ref = O.naive_attention(x["q_nope"], x["q_pe"], O.rms_norm(raw, w, 1e-6), x["pe_cache"], x["wkv_b"], cfg.end_pos,
                            cfg.softmax_scale, cfg.v_head_dim)
    check(a, ref, TOL["bf16"], "absorb route (GPU) vs oracle")
    check(n, ref, TOL["bf16"], "naive route (GPU) vs oracle")
    check(n, a.float().cpu().double().numpy(), TOL["bf16"], "naive route vs absorb route, both on the GPU")


def test_full_size_naive_vs_absorb_prefill(gpu_lib):
    """chunk_prefill through both routes on the GPU (expansion of the 2 x 4096 cached latents, then
    naive attention), compared with each other and with the oracle on every output element."""
    cfg = ATTN_CONFIGS["chunk_prefill"]
    print(f"full-size naive vs absorb: B={cfg.batch} S={cfg.seqlen_q} T={cfg.end_pos}", flush=True)
    x = make_attn_inputs(cfg)
    # cache rows of unit RMS (what the append step stores for unit weight), so that expanding the
    # cache with weight 1 reproduces the rows up to rounding and both routes see the same latents
    x["kv_cache"] = round_bf16(O.rms_norm(x["kv_cache"], np.ones(cfg.kv_lora_rank), 0.0))
    t = to_dev(x, cfg)
    a = run_attn(gpu_lib, cfg, t)
    k, v = gpu_lib.expand_kv(t["kv_cache"].reshape(-1, cfg.kv_lora_rank),
                             torch.ones(cfg.kv_lora_rank, dtype=torch.bfloat16, device="cuda"), t["wkv_b"],
                             cfg.n_heads, cfg.qk_nope_head_dim, cfg.v_head_dim, 0.0)
    n = run_naive(gpu_lib, cfg, t, k.view(cfg.n_heads, cfg.cache_batch, cfg.cache_len, -1),
                  v.view(cfg.n_heads, cfg.cache_batch, cfg.cache_len, -1))
    assert torch.isfinite(n).all()
    check(n, a.float().cpu().double().numpy(), TOL["bf16"], "chunk_prefill naive route vs absorb route")
    check(n, oracle_attn_full(cfg, x), TOL["bf16"], "chunk_prefill naive route, all outputs")


# ------------------------------------------------------------------ naive-route cache append

@pytest.mark.parametrize("path,dtype,S", [("mfma", "bf16", 37), ("mfma", "bf16", 3), ("mfma", "bf16", 1),
                                          ("mfma", "bf16", 200), ("plain", "bf16", 37), ("plain", "f32", 5)])
def test_expand_kv_append(gpu_lib, path, dtype, S):
    """Cache rows (h, b, end_pos - S + s) get the oracle's expansion of new token (b, s), bit for bit
    what mla_expand_kv writes for the same tokens; the rope rows are copied; every other row of the
    three caches keeps its bits.  S = 37 and 200 put sequence boundaries inside token blocks, S = 3
    and 1 several inside one 4-row store."""
    if dtype == "f32":
        H, C, R, Dn, Dv = 4, 64, 16, 32, 32
    else:
        H, C, R, Dn, Dv = 8, 512, 64, 128, 128
    B, Bmax, Tmax, end_pos, eps = 2, 3, 300, 251, 1e-6
    print(f"expand append {path} {dtype} B={B} S={S} H={H} end_pos={end_pos}", flush=True)
    rng = np.random.default_rng(71 + S)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    cast = (lambda a: np.asarray(a, np.float32)) if dtype == "f32" else round_bf16
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to("cuda").to(tdt)
    c_new, kp_new = cast(rng.normal(size=(B, S, C))), cast(rng.normal(size=(B, S, R)))
    w = cast(1.0 + 0.14 * rng.normal(size=C))
    wkv = cast(rng.normal(size=(H * (Dn + Dv), C)) / np.sqrt(C))
    k0, v0 = cast(rng.normal(size=(H, Bmax, Tmax, Dn))), cast(rng.normal(size=(H, Bmax, Tmax, Dv)))
    pe0 = cast(rng.normal(size=(Bmax, Tmax, R)))
    kc, vc, pc = dev(k0), dev(v0), dev(pe0)
    gpu_lib.expand_kv_append(dev(c_new), dev(kp_new), dev(w), dev(wkv), eps, end_pos, kc, vc, pc, path=path)
    ke, ve = gpu_lib.expand_kv(dev(c_new.reshape(-1, C)), dev(w), dev(wkv), H, Dn, Dv, eps, path=path)
    torch.cuda.synchronize()
    new = np.zeros((Bmax, Tmax), bool)
    new[:B, end_pos - S:end_pos] = True
    gk, gv, gp = (t.float().cpu().numpy() for t in (kc, vc, pc))
    assert np.array_equal(gk[:, ~new], k0[:, ~new]) and np.array_equal(gv[:, ~new], v0[:, ~new]), "untouched rows"
    assert np.array_equal(gp[~new], pe0[~new]), "untouched rope rows"
    assert np.array_equal(gp[new], kp_new.reshape(-1, R)), "rope rows are copied exactly"
    k_new, v_new = gk[:, new], gv[:, new]  # [H, B*S, D] in (b, s) order
    assert np.array_equal(k_new, ke.float().cpu().numpy()) and np.array_equal(v_new, ve.float().cpu().numpy()), \
        "appended rows differ from mla_expand_kv on the same tokens"
    kr, vr = O.expand_kv(c_new.reshape(-1, C), w, wkv, H, Dn, Dv, eps)
    check(k_new.astype(np.float64), kr, TOL[dtype], f"append {path} {dtype} S={S} K rows")
    check(v_new.astype(np.float64), vr, TOL[dtype], f"append {path} {dtype} S={S} V rows")


def test_naive_route_append_then_attend(gpu_lib):
    """One chunk step of the naive path as the pages lay it out: the caches hold full-width keys and
    values of the earlier positions; the chunk's new tokens are expanded into them, with their rope
    keys, and the naive attention reads the result.  Against the oracle's expansion and attention."""
    cfg = dsv3_small(batch=2, cache_batch=2, seqlen_q=40, end_pos=230, cache_len=256, n_heads=16)
    print(f"naive route append+attend S={cfg.seqlen_q} end_pos={cfg.end_pos}", flush=True)
    x = make_attn_inputs(cfg)
    kh, vh = head_major_kv(x, cfg)  # earlier positions' full-width rows (the new rows get overwritten)
    rng = np.random.default_rng(73)
    c_new = round_bf16(rng.normal(size=(cfg.batch, cfg.seqlen_q, cfg.kv_lora_rank)))
    kp_new = round_bf16(rng.normal(size=(cfg.batch, cfg.seqlen_q, cfg.qk_rope_head_dim)))
    w = round_bf16(1.0 + 0.14 * rng.normal(size=cfg.kv_lora_rank))
    t = to_dev(x, cfg)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to("cuda").to(torch.bfloat16)
    kc, vc = dev(kh), dev(vh)
    gpu_lib.expand_kv_append(dev(c_new), dev(kp_new), dev(w), t["wkv_b"], 1e-6, cfg.end_pos, kc, vc, t["pe_cache"])
    out = run_naive(gpu_lib, cfg, t, kc, vc, path="mfma")
    # the oracle's caches after the same append, rounded to bf16 as stored
    kr, vr = O.expand_kv(c_new.reshape(-1, cfg.kv_lora_rank), w, x["wkv_b"], cfg.n_heads, cfg.qk_nope_head_dim,
                         cfg.v_head_dim, 1e-6)
    k_ref, v_ref, pe_ref = np.array(kh), np.array(vh), np.array(x["pe_cache"])
    p0 = cfg.end_pos - cfg.seqlen_q
    k_ref[:, :cfg.batch, p0:cfg.end_pos] = round_bf16(kr).reshape(cfg.n_heads, cfg.batch, cfg.seqlen_q, -1)
    v_ref[:, :cfg.batch, p0:cfg.end_pos] = round_bf16(vr).reshape(cfg.n_heads, cfg.batch, cfg.seqlen_q, -1)
    pe_ref[:cfg.batch, p0:cfg.end_pos] = kp_new
    ref = O.attention_over_kv(x["q_nope"], x["q_pe"], k_ref, v_ref, pe_ref, cfg.end_pos, cfg.softmax_scale)
    check(out, ref, TOL["bf16"], "naive route: append the chunk, then attend")


def test_full_size_expand_append(gpu_lib):
    """chunk_prefill's naive-route append: 2 x 512 new tokens into [128, 2, 4096, 128] caches at
    positions 3584..4095; every appended element against the oracle and bit for bit against
    mla_expand_kv, and the earlier positions untouched."""
    cfg = ATTN_CONFIGS["chunk_prefill"]
    B, S, H, C, R = cfg.batch, cfg.seqlen_q, cfg.n_heads, cfg.kv_lora_rank, cfg.qk_rope_head_dim
    print(f"full-size expand append: B={B} S={S} H={H} end_pos={cfg.end_pos}", flush=True)
    rng = np.random.default_rng(79)
    c_new = round_bf16(rng.normal(size=(B, S, C)))
    kp_new = round_bf16(rng.normal(size=(B, S, R)))
    w = round_bf16(1.0 + 0.14 * rng.normal(size=C))
    wkv = round_bf16(rng.normal(size=(H * 256, C)) / np.sqrt(C))
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to("cuda").to(torch.bfloat16)
    shape_kv = (H, cfg.cache_batch, cfg.cache_len, 128)
    kc = torch.full(shape_kv, 3.0, dtype=torch.bfloat16, device="cuda")
    vc = torch.full(shape_kv, -3.0, dtype=torch.bfloat16, device="cuda")
    pc = torch.full((cfg.cache_batch, cfg.cache_len, R), 5.0, dtype=torch.bfloat16, device="cuda")
    gpu_lib.expand_kv_append(dev(c_new), dev(kp_new), dev(w), dev(wkv), 1e-6, cfg.end_pos, kc, vc, pc)
    ke, ve = gpu_lib.expand_kv(dev(c_new.reshape(-1, C)), dev(w), dev(wkv), H, 128, 128, 1e-6)
    torch.cuda.synchronize()
    p0 = cfg.end_pos - S
    assert bool((kc[:, :, :p0] == 3.0).all()) and bool((vc[:, :, :p0] == -3.0).all()) and \
        bool((pc[:, :p0] == 5.0).all()), "earlier positions changed"
    k_new = kc[:, :, p0:].reshape(H, B * S, 128)
    v_new = vc[:, :, p0:].reshape(H, B * S, 128)
    assert torch.equal(k_new, ke) and torch.equal(v_new, ve), "appended rows differ from mla_expand_kv"
    assert torch.equal(pc[:, p0:].reshape(B * S, R), dev(kp_new.reshape(-1, R))), "rope rows"
    kr, vr = O.expand_kv(c_new.reshape(-1, C), w, wkv, H, 128, 128, 1e-6)
    check(k_new, kr, TOL["bf16"], "chunk_prefill append K rows")
    check(v_new, vr, TOL["bf16"], "chunk_prefill append V rows")


def test_full_size_expand(gpu_lib):
    cfg = EXPAND_CONFIGS["dsv3_expand"]
    x = make_expand_inputs(cfg)
    t = to_dev(x, cfg)
    k = torch.full((cfg.n_heads, cfg.n_tokens, cfg.qk_nope_head_dim), float("nan"), dtype=torch.bfloat16,
                   device="cuda")
    v = torch.full_like(k, float("nan"))
    gpu_lib.expand_kv(t["c_kv"], t["rms_w"], t["wkv_b"], cfg.n_heads, cfg.qk_nope_head_dim, cfg.v_head_dim, cfg.eps,
                      k, v)
    torch.cuda.synchronize()
    # every token against the oracle, 1024 tokens at a time (each token's rows depend on it alone)
    for t0 in range(0, cfg.n_tokens, 1024):
        kr, vr = O.expand_kv(x["c_kv"][t0:t0 + 1024], x["rms_w"], x["wkv_b"], cfg.n_heads, cfg.qk_nope_head_dim,
                             cfg.v_head_dim, cfg.eps)
        check(k[:, t0:t0 + 1024], kr, TOL["bf16"], f"dsv3_expand K_nope tokens {t0}..")
        check(v[:, t0:t0 + 1024], vr, TOL["bf16"], f"dsv3_expand V tokens {t0}..")


@pytest.mark.parametrize("T", [1, 100, 257, 1000])
def test_mfma_expand_ragged(gpu_lib, T):
    cfg = EXPAND_CONFIGS["dsv3_expand"].replace(n_tokens=T, n_heads=4)
    x = make_expand_inputs(cfg)
    t = to_dev(x, cfg)
    k, v = gpu_lib.expand_kv(t["c_kv"], t["rms_w"], t["wkv_b"], cfg.n_heads, cfg.qk_nope_head_dim, cfg.v_head_dim,
                             cfg.eps, path="mfma")
    torch.cuda.synchronize()
    kr, vr = O.expand_kv(x["c_kv"], x["rms_w"], x["wkv_b"], cfg.n_heads, cfg.qk_nope_head_dim, cfg.v_head_dim,
                         cfg.eps)
    check(k, kr, TOL["bf16"], f"mfma expand T={T} K_nope")
    check(v, vr, TOL["bf16"], f"mfma expand T={T} V")
