"""Seeded input generators: determinism, shapes, and exact bf16 representability."""
import numpy as np
import torch

from mla_latent_kv_absorb_amd.workloads import (ATTN_CONFIGS, EXPAND_CONFIGS, bf16_bits, make_attn_inputs,
                                                 make_expand_inputs, round_to_bf16)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.005859375, 3.4e38, -1e-40], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf16_bits(x), ref)
    assert np.array_equal(round_to_bf16(x), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_tiny_shapes_and_determinism():
    cfg = ATTN_CONFIGS["tiny_f32"]
    a, b = make_attn_inputs(cfg), make_attn_inputs(cfg)
    assert a["q_nope"].shape == (1, 1, 4, 32)
    assert a["q_pe"].shape == (1, 1, 4, 16)
    assert a["kv_cache"].shape == (1, 128, 64)
    assert a["pe_cache"].shape == (1, 128, 16)
    assert a["wkv_b"].shape == (4 * 64, 64)
    for k in a:
        assert a[k].dtype == np.float32
        assert np.array_equal(a[k], b[k])
    assert abs(a["wkv_b"].std() - 1 / 8) < 0.01
    assert abs(cfg.softmax_scale - 1 / np.sqrt(48)) < 1e-12


def test_bf16_workload_values_are_representable():
    cfg = ATTN_CONFIGS["dsv3_decode"].replace(batch=2, end_pos=64, cache_len=64, cache_batch=2, n_heads=8)
    x = make_attn_inputs(cfg)
    for v in x.values():
        assert np.array_equal(round_to_bf16(v), v)
    e = make_expand_inputs(EXPAND_CONFIGS["dsv3_expand"].replace(n_tokens=16, n_heads=2))
    for v in e.values():
        assert np.array_equal(round_to_bf16(v), v)
    assert abs(float(e["rms_w"].mean()) - 1.0) < 0.05


def test_config_shapes():
    c = ATTN_CONFIGS["chunk_prefill"]
    assert (c.batch, c.seqlen_q, c.start_pos, c.end_pos) == (2, 512, 3584, 4096)
    c = ATTN_CONFIGS["long_decode"]
    assert (c.batch, c.end_pos, c.n_heads, c.kv_lora_rank, c.qk_rope_head_dim) == (4, 32768, 128, 512, 64)
    e = EXPAND_CONFIGS["dsv3_expand"]
    assert e.n_heads * (e.qk_nope_head_dim + e.v_head_dim) == 32768 and e.n_tokens == 8192
