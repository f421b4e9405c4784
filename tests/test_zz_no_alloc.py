"""mla_absorb_attn_noalloc: the absorb attention with the library's own scratch array as workspace.

The GPU checks run the entry point through the C-ABI twice in a row, the second call smaller than
the first (the array keeps the first call's contents), and compare each output with that of
mla_absorb_attn on the same inputs (bitwise: the same kernels run) and with the oracle at the
workload's bar.  The CPU checks cover the rejections that happen before any HIP call."""
import ctypes

import numpy as np
import pytest

from mla_latent_kv_absorb_amd import binding as B
from mla_latent_kv_absorb_amd.workloads import ATTN_CONFIGS, make_attn_inputs
from oracle import mla_oracle as O

TOL = {"f32": 1e-5, "bf16": 2e-2}
P = [0x7f0000000000 + i * 0x100000000 for i in range(8)]


@pytest.fixture(scope="module")
def lib():
    return B.load()


def shape(**kw):
    d = dict(batch=2, seqlen_q=1, n_heads=128, kv_lora_rank=512, qk_rope_head_dim=64, qk_nope_head_dim=128,
             v_head_dim=128, cache_batch=2, cache_len=4096)
    d.update(kw)
    return B.AttnShape(*[d[f] for f, _ in B.AttnShape._fields_])


def call(lib, s, end_pos=4096, ptrs=None):
    p = list(P[:6]) if ptrs is None else ptrs
    return lib.mla_absorb_attn_noalloc(p[0], p[1], p[2], p[3], p[4], end_pos, 0.07, p[5], ctypes.byref(s),
                                       B.MLA_DTYPE_BF16, None, None)


def test_noalloc_rejects_before_any_hip_call(lib):
    """Calls whose workspace exceeds the array, and ordinary validation failures, are refused
    with the usual status (fake pointers: nothing may be launched)."""
    big = shape(batch=2, seqlen_q=512, cache_len=4096)  # a 512-token chunk: ~185 MB of workspace
    need = B.absorb_attn_workspace_size(big, 4096, B.MLA_DTYPE_BF16)
    assert need > B.NOALLOC_SCRATCH_BYTES
    assert call(lib, big) == B.MLA_ERR_WORKSPACE
    assert "no-allocation entry point holds" in B.last_error()
    assert call(lib, shape(batch=3)) == B.MLA_ERR_RANGE
    p = list(P[:6])
    p[0] = None
    assert call(lib, shape(), ptrs=p) == B.MLA_ERR_NULL
    p = list(P[:6])
    p[5] = P[2] + 1024
    assert call(lib, shape(), ptrs=p) == B.MLA_ERR_SHAPE


def run_both(lib_unused, cfg, x, torch):
    dt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
    t = {k: torch.from_numpy(v).to("cuda").to(dt) for k, v in x.items()}
    outs = []
    for fn in ("noalloc", "workspace"):
        out = torch.full((cfg.batch, cfg.seqlen_q, cfg.n_heads, cfg.v_head_dim), float("nan"), dtype=dt, device="cuda")
        if fn == "noalloc":
            B.absorb_attn_noalloc(t["q_nope"], t["q_pe"], t["kv_cache"], t["pe_cache"], t["wkv_b"], cfg.end_pos,
                                  cfg.softmax_scale, out)
        else:
            B.absorb_attn(t["q_nope"], t["q_pe"], t["kv_cache"], t["pe_cache"], t["wkv_b"], cfg.end_pos,
                          cfg.softmax_scale, out)
        torch.cuda.synchronize()
        outs.append(out)
    return outs


@pytest.mark.gpu
def test_noalloc_matches_workspace_entry_point():
    import torch

    if not torch.cuda.is_available():
        pytest.fail("GPU test selected but no GPU is visible")
    B.load()
    base = ATTN_CONFIGS["dsv3_decode"]
    cases = [("dsv3 decode B=8 T=1500", base.replace(batch=8, cache_batch=8, end_pos=1500, cache_len=1536)),
             ("dsv3 decode B=2 T=300 (smaller)", base.replace(batch=2, cache_batch=2, end_pos=300, cache_len=320)),
             ("tiny fp32", ATTN_CONFIGS["tiny_f32"])]
    for name, cfg in cases:
        print(f"noalloc: {name}", flush=True)
        x = make_attn_inputs(cfg)
        na, ws = run_both(None, cfg, x, torch)
        assert torch.isfinite(na).all(), f"{name}: non-finite outputs"
        assert torch.equal(na, ws), f"{name}: differs from mla_absorb_attn"
        ref = O.absorb_attention(x["q_nope"], x["q_pe"], x["kv_cache"], x["pe_cache"], x["wkv_b"], cfg.end_pos,
                                 cfg.softmax_scale, cfg.v_head_dim)
        g = na.float().cpu().double().numpy()
        err = float(np.abs(g - ref).max() / np.abs(ref).max())
        print(f"noalloc {name}: max rel err {err:.3e}")
        assert err <= TOL[cfg.dtype], f"{name}: {err}"
