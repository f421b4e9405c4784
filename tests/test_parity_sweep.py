"""GPU parity over a seeded sweep of shapes: batch, query length, head count, cache length and
capacity, split count and per-sequence lengths drawn at random (fixed seeds), for contiguous
caches, page pools, index lists, the naive path's append and the fused append-and-attend call, each
case through the matrix-core kernels and compared with the CPU oracle on every output element.

The fixed-shape tests pin the workloads and the edge cases one by one; this sweep covers the
combinations between them (row blocks that straddle sequences, odd causal chunks, split counts
that do not divide the length, capacities larger than the lengths)."""
import numpy as np
import pytest
import torch

from mla_latent_kv_absorb_amd.workloads import ATTN_CONFIGS, EXPAND_CONFIGS, make_attn_inputs, make_expand_inputs, \
    round_to_bf16
from oracle import mla_oracle as O

pytestmark = pytest.mark.gpu

TOL = 2e-2  # bf16 storage, fp32 accumulation: max|gpu - ref| <= TOL * max|ref|


def check(gpu, ref, what):
    g = gpu.float().cpu().double().numpy()
    assert np.isfinite(g).all(), f"{what}: non-finite outputs"
    worst = float(np.abs(g - ref).max() / np.abs(ref).max())
    print(f"{what}: max rel err {worst:.3e}", flush=True)
    assert worst <= TOL, f"{what}: {worst:.3e} > {TOL}"


def draw_attn_case(seed):
    rng = np.random.default_rng(1000 + seed)
    B = int(rng.integers(1, 6))
    S = int(rng.choice([1, 1, 2, 3, 5, 9, 17]))
    H = int(rng.choice([16, 32, 128]))
    end_pos = int(rng.integers(S, 700))
    cfg = ATTN_CONFIGS["dsv3_decode"].replace(batch=B, seqlen_q=S, n_heads=H, end_pos=end_pos,
                                              cache_len=end_pos + int(rng.integers(0, 65)),
                                              cache_batch=B + int(rng.integers(0, 3)))
    splits = int(rng.choice([0, 0, 1, 2, 3, 5, 7, 12]))
    lens = [int(n) for n in rng.integers(S, end_pos + 1, size=B)] if rng.random() < 0.3 else None
    return cfg, splits, lens


@pytest.mark.parametrize("seed", range(24))
def test_attention_sweep(gpu_lib, seed):
    cfg, splits, lens = draw_attn_case(seed)
    print(f"sweep {seed}: B={cfg.batch} S={cfg.seqlen_q} H={cfg.n_heads} end_pos={cfg.end_pos} "
          f"Tmax={cfg.cache_len} Bmax={cfg.cache_batch} splits={splits} lens={lens}", flush=True)
    x = make_attn_inputs(cfg, seed=2000 + seed)
    t = {k: torch.from_numpy(v).to("cuda").to(torch.bfloat16) for k, v in x.items()}
    out = torch.full((cfg.batch, cfg.seqlen_q, cfg.n_heads, cfg.v_head_dim), float("nan"), dtype=torch.bfloat16,
                     device="cuda")
    seq_lens = None if lens is None else torch.tensor(lens, dtype=torch.int32, device="cuda")
    gpu_lib.absorb_attn(t["q_nope"], t["q_pe"], t["kv_cache"], t["pe_cache"], t["wkv_b"], cfg.end_pos,
                        cfg.softmax_scale, out, num_splits=splits, path="mfma", seq_lens=seq_lens)
    torch.cuda.synchronize()
    if lens is None:
        ref = O.absorb_attention(x["q_nope"], x["q_pe"], x["kv_cache"], x["pe_cache"], x["wkv_b"], cfg.end_pos,
                                 cfg.softmax_scale, cfg.v_head_dim)
    else:
        ref = O.absorb_attention_ragged(x["q_nope"], x["q_pe"], x["kv_cache"], x["pe_cache"], x["wkv_b"], lens,
                                        cfg.softmax_scale, cfg.v_head_dim)
    check(out, ref, f"sweep {seed}")


@pytest.mark.parametrize("seed", range(8))
def test_expansion_append_sweep(gpu_lib, seed):
    """The naive path's append at random batch, chunk length, position and capacity: the rows
    match the oracle's expansion of the same tokens, and every other cache row keeps its bits."""
    rng = np.random.default_rng(3000 + seed)
    B, S = int(rng.integers(1, 5)), int(rng.choice([1, 2, 3, 7, 31, 33, 100, 257]))
    H = int(rng.choice([4, 8, 16]))
    end_pos = S + int(rng.integers(0, 200))
    Bmax, Tmax = B + int(rng.integers(0, 3)), end_pos + int(rng.integers(0, 40))
    print(f"append sweep {seed}: B={B} S={S} H={H} end_pos={end_pos} Bmax={Bmax} Tmax={Tmax}", flush=True)
    cfg = EXPAND_CONFIGS["dsv3_expand"].replace(n_tokens=B * S, n_heads=H)
    x = make_expand_inputs(cfg, seed=4000 + seed)
    kp = round_to_bf16(rng.normal(size=(B, S, 64)).astype(np.float32))
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to("cuda").to(torch.bfloat16)
    k0 = dev(rng.normal(size=(H, Bmax, Tmax, 128)))
    v0 = dev(rng.normal(size=(H, Bmax, Tmax, 128)))
    p0 = dev(rng.normal(size=(Bmax, Tmax, 64)))
    kc, vc, pc = k0.clone(), v0.clone(), p0.clone()
    gpu_lib.expand_kv_append(dev(x["c_kv"].reshape(B, S, -1)), dev(kp), dev(x["rms_w"]), dev(x["wkv_b"]), cfg.eps,
                             end_pos, kc, vc, pc, path="mfma")
    torch.cuda.synchronize()
    new = torch.zeros((Bmax, Tmax), dtype=torch.bool, device="cuda")
    new[:B, end_pos - S:end_pos] = True
    assert torch.equal(kc[:, ~new], k0[:, ~new]) and torch.equal(vc[:, ~new], v0[:, ~new]), "untouched rows"
    assert torch.equal(pc[~new], p0[~new]) and torch.equal(pc[new], dev(kp.reshape(-1, 64))), "rope rows"
    kr, vr = O.expand_kv(x["c_kv"], x["rms_w"], x["wkv_b"], H, 128, 128, cfg.eps)
    check(kc[:, new], kr, f"append sweep {seed} K rows")
    check(vc[:, new], vr, f"append sweep {seed} V rows")


def dev_inputs(x):
    return {k: torch.from_numpy(v).to("cuda").to(torch.bfloat16) for k, v in x.items()}


@pytest.mark.parametrize("seed", range(8))
def test_paged_sweep(gpu_lib, seed):
    """Page pools in random order at random page sizes, lengths and split counts."""
    from test_parity import run_attn_paged, to_pages

    rng = np.random.default_rng(5000 + seed)
    B = int(rng.integers(1, 5))
    S = int(rng.choice([1, 1, 2, 4]))
    H = int(rng.choice([16, 128]))
    page_size = int(rng.choice([32, 64, 128, 256]))
    lens = [int(n) for n in rng.integers(S, int(rng.integers(S, 600)) + 1, size=B)]
    bound = max(lens)  # the lengths' bound; the pools hold up to (pages per row) x page_size positions
    splits = int(rng.choice([0, 0, 1, 3, 6]))
    cfg = ATTN_CONFIGS["dsv3_decode"].replace(batch=B, seqlen_q=S, n_heads=H, end_pos=bound, cache_len=bound,
                                              cache_batch=B)
    print(f"paged sweep {seed}: B={B} S={S} H={H} page={page_size} lens={lens} splits={splits}", flush=True)
    x = make_attn_inputs(cfg, seed=6000 + seed)
    kvp, table = to_pages(x["kv_cache"], lens, page_size, 2, 7000 + seed)
    pep, _ = to_pages(x["pe_cache"], lens, page_size, 2, 7000 + seed)
    dev = lambda a: torch.from_numpy(a).to("cuda").to(torch.bfloat16)
    out = run_attn_paged(gpu_lib, cfg, dev_inputs(x), dev(kvp), dev(pep), torch.from_numpy(table).to("cuda"), bound,
                         lens=lens, path="mfma", splits=splits)
    ref = O.absorb_attention_paged(x["q_nope"], x["q_pe"], kvp, pep, x["wkv_b"], table, lens, page_size,
                                   cfg.softmax_scale, cfg.v_head_dim)
    check(out, ref, f"paged sweep {seed}")


@pytest.mark.parametrize("seed", range(8))
def test_sparse_sweep(gpu_lib, seed):
    """Index lists (with padding, repeats and entries past the visible positions) at random list
    lengths, batch sizes and split counts."""
    from test_parity import make_lists, run_attn_sparse

    rng = np.random.default_rng(8000 + seed)
    B = int(rng.integers(1, 5))
    S = int(rng.choice([1, 1, 2, 3]))
    H = 128 if S > 1 else int(rng.choice([16, 128]))
    end_pos = int(rng.integers(S + 1, 600))
    lens = [int(n) for n in rng.integers(S, end_pos + 1, size=B)]
    topk = int(rng.choice([1, 17, 64, 200, 513]))
    splits = int(rng.choice([0, 0, 1, 2, 5]))
    cfg = ATTN_CONFIGS["dsv3_decode"].replace(batch=B, seqlen_q=S, n_heads=H, end_pos=end_pos, cache_len=end_pos + 8,
                                              cache_batch=B)
    print(f"sparse sweep {seed}: B={B} S={S} H={H} topk={topk} lens={lens} splits={splits}", flush=True)
    x = make_attn_inputs(cfg, seed=9000 + seed)
    idx = make_lists(cfg, lens, topk, 9500 + seed)
    out = run_attn_sparse(gpu_lib, cfg, dev_inputs(x), idx, lens, path="mfma", splits=splits)
    ref = O.absorb_attention_sparse(x["q_nope"], x["q_pe"], x["kv_cache"], x["pe_cache"], x["wkv_b"], idx, lens,
                                    cfg.softmax_scale, cfg.v_head_dim)
    check(out, ref, f"sparse sweep {seed}")


@pytest.mark.parametrize("seed", range(12))
def test_plain_fp32_sweep(gpu_lib, seed):
    """The plain kernels (fp32, any head shape) at random widths, batch, query length, cache
    length and split count, against the oracle at the fp32 tolerance."""
    rng = np.random.default_rng(10000 + seed)
    B, S = int(rng.integers(1, 4)), int(rng.choice([1, 1, 2, 5]))
    H = int(rng.integers(1, 9))
    C, R = int(rng.choice([16, 32, 64, 96])), int(rng.choice([4, 8, 16]))
    Dn, Dv = int(rng.choice([8, 16, 32])), int(rng.choice([8, 16, 32]))
    end_pos = int(rng.integers(S, 300))
    splits = int(rng.choice([0, 1, 3, 8]))
    cfg = ATTN_CONFIGS["tiny_f32"].replace(batch=B, seqlen_q=S, n_heads=H, kv_lora_rank=C, qk_rope_head_dim=R,
                                           qk_nope_head_dim=Dn, v_head_dim=Dv, end_pos=end_pos,
                                           cache_len=end_pos + int(rng.integers(0, 20)), cache_batch=B + 1,
                                           wkv_b_var=1.0 / C)
    print(f"plain sweep {seed}: B={B} S={S} H={H} C={C} R={R} Dn={Dn} Dv={Dv} end_pos={end_pos} splits={splits}",
          flush=True)
    x = make_attn_inputs(cfg, seed=11000 + seed)
    t = {k: torch.from_numpy(v).to("cuda") for k, v in x.items()}
    out = torch.full((B, S, H, Dv), float("nan"), dtype=torch.float32, device="cuda")
    gpu_lib.absorb_attn(t["q_nope"], t["q_pe"], t["kv_cache"], t["pe_cache"], t["wkv_b"], end_pos, cfg.softmax_scale,
                        out, num_splits=splits, path="plain")
    torch.cuda.synchronize()
    ref = O.absorb_attention(x["q_nope"], x["q_pe"], x["kv_cache"], x["pe_cache"], x["wkv_b"], end_pos,
                             cfg.softmax_scale, Dv)
    g = out.cpu().double().numpy()
    worst = float(np.abs(g - ref).max() / np.abs(ref).max())
    print(f"plain sweep {seed}: max rel err {worst:.3e}", flush=True)
    assert np.isfinite(g).all() and worst <= 1e-5, f"plain sweep {seed}: {worst:.3e}"


@pytest.mark.parametrize("seed", range(8))
def test_fused_append_sweep(gpu_lib, seed):
    """mla_absorb_attn_append over seeded shapes: caches and output bit-equal to the stand-alone
    append followed by the attention call, and the output within tolerance of the oracle's append
    followed by absorb attention."""
    cfg, splits, lens = draw_attn_case(100 + seed)
    rng = np.random.default_rng(3000 + seed)
    S = cfg.seqlen_q
    print(f"fused append sweep {seed}: B={cfg.batch} S={S} H={cfg.n_heads} end_pos={cfg.end_pos} "
          f"Tmax={cfg.cache_len} Bmax={cfg.cache_batch} splits={splits} lens={lens}", flush=True)
    x = make_attn_inputs(cfg, seed=4000 + seed)
    c_new = round_to_bf16(rng.normal(size=(cfg.batch, S, cfg.kv_lora_rank)).astype(np.float32))
    kp_new = round_to_bf16(rng.normal(size=(cfg.batch, S, cfg.qk_rope_head_dim)).astype(np.float32))
    w = round_to_bf16((1.0 + 0.14 * rng.normal(size=cfg.kv_lora_rank)).astype(np.float32))
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to("cuda").to(torch.bfloat16)
    t = {k: dev(v) for k, v in x.items()}
    seq_lens = None if lens is None else torch.tensor(lens, dtype=torch.int32, device="cuda")
    res = []
    for fused in (True, False):
        kv, pe = t["kv_cache"].clone(), t["pe_cache"].clone()
        out = torch.full((cfg.batch, S, cfg.n_heads, cfg.v_head_dim), float("nan"), dtype=torch.bfloat16,
                         device="cuda")
        if fused:
            gpu_lib.absorb_attn(t["q_nope"], t["q_pe"], kv, pe, t["wkv_b"], cfg.end_pos, cfg.softmax_scale, out,
                                num_splits=splits, path="mfma", seq_lens=seq_lens,
                                append=(dev(c_new), dev(kp_new), dev(w), 1e-6))
        else:
            gpu_lib.cache_append(dev(c_new), dev(kp_new), dev(w), 1e-6, cfg.end_pos, kv, pe, seq_lens=seq_lens)
            gpu_lib.absorb_attn(t["q_nope"], t["q_pe"], kv, pe, t["wkv_b"], cfg.end_pos, cfg.softmax_scale, out,
                                num_splits=splits, path="mfma", seq_lens=seq_lens)
        torch.cuda.synchronize()
        res.append((out, kv, pe))
    for a, b in zip(res[0], res[1]):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"sweep {seed}: fused differs from two calls"
    # the oracle over the caches as the GPU wrote them (their new rows checked in the fixed tests)
    kv_g = res[0][1].float().cpu().numpy().astype(np.float64)
    pe_g = res[0][2].float().cpu().numpy().astype(np.float64)
    if lens is None:
        ref = O.absorb_attention(x["q_nope"], x["q_pe"], kv_g, pe_g, x["wkv_b"], cfg.end_pos, cfg.softmax_scale,
                                 cfg.v_head_dim)
    else:
        ref = O.absorb_attention_ragged(x["q_nope"], x["q_pe"], kv_g, pe_g, x["wkv_b"], lens, cfg.softmax_scale,
                                        cfg.v_head_dim)
    check(res[0][0], ref, f"fused append sweep {seed}")
    # and the written rows against the oracle's append
    kv_o, _ = O.cache_append(c_new, kp_new, w, 1e-6, x["kv_cache"], x["pe_cache"], end_pos=cfg.end_pos,
                             seq_lens=lens)
    for b in range(cfg.batch):
        n = cfg.end_pos if lens is None else min(max(lens[b], S), cfg.end_pos)
        g_rows = kv_g[b, n - S:n]
        o_rows = kv_o[b, n - S:n]
        assert np.abs(g_rows - o_rows).max() <= TOL * np.abs(o_rows).max(), f"sweep {seed}: appended rows of {b}"
