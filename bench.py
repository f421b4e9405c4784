"""Benchmark: MLA absorb decode on one MI355X, DeepSeek-V3 decode shape.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload dsv3_decode] [--peaks]
                    [--no-extras] [--no-cpu-baseline] [--no-peaks] [--sustained-ms MS]

A step is one absorb-attention decode call (query absorption through W_UK, split-KV attention
over kv_cache + pe_cache, merge and W_UV projection) over one batch: 32 sequences x 4096 cached
positions x 128 heads, bf16.  Inputs are seeded synthetic tensors drawn on the GPU with the
workload's shapes and distributions (q, caches ~N(0,1); wkv_b ~N(0,1/512)).  To measure HBM rather
than the 256 MB Infinity Cache, the timed steps rotate over several complete input sets (about
750 MB in all), so each step's operands were last touched three steps earlier.  The timed region
starts on an idle, synchronised GPU; the host enqueues a step in about 9 us against about 65 us
of GPU work, so after the first launch the queue stays ahead of the GPU and the figure is
back-to-back GPU time (the first launch's latency is included).  No spin kernel runs ahead: a
sleeping spin let the clocks fall and cost about 4 us per step.

Prints ONE JSON line.  `value` is microseconds per step (lower is better), from timed steps that
carry no per-kernel events.  `roofline` reports the dominant kernel (the attention kernel) against
HBM bandwidth: algorithmic bytes per launch (the kv and pe cache rows it must read plus the rope
query) over its average duration, measured live by running the same timed steps again with HIP
events that the kernel's own dispatch stamps on its stream (hipExtLaunchKernel start/stop events);
those events add a queue barrier per timed dispatch, so that pass's step time is reported apart.
`cpu_baseline` times the CPU oracle (float32 NumPy, all host cores, and one core) on a bounded
sample of the same workload.  `peaks_measured` holds what simple probe kernels reach on this machine
(streaming read and copy, dense bf16 MFMA with its clock, LDS reads), and the fractions against
them stand beside the fractions against the published peaks.  `sustained` is the decode step over
a longer back-to-back run, after the chip's power management has settled its clocks.
`extras` times the other workloads the same way: long_decode, chunk_prefill, ragged_decode (the
decode batch with per-sequence lengths drawn uniformly from [256, 4096]) and skewed_decode (4 of
its sequences at 4096 positions, 28 at 64), each also under the uniform split plan for
comparison with the balanced one the library picks, paged_decode (the decode
batch with its caches in pools of 64-position pages in random order), decode_append (a serving
decode step that first writes each sequence's new token into the caches: one fused
mla_absorb_attn_append call against mla_cache_append followed by mla_absorb_attn), sparse_decode and
sparse_long_decode (the decode and long-context batches with each token attending to 2048 random
positions of its cache through an index list), chunk_prefill_naive (the same chunk through the
naive path as the pages lay it out: full-width key and value caches, into which a step expands the
2 x 512 new tokens, then attention over the caches), chunk_prefill_naive_from_latent (the naive
attention fed from the latent cache: a step expands all 2 x 4096 cached latents first),
dsv3_expand (four rotated input sets) and tiny_f32 (the fp32 decode of one sequence, 4 heads,
128 positions).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2516.6
METRIC = "MLA absorb decode µs/step, HBM GB/s & MFMA TFLOP/s as % of roofline"


def progress(msg):
    """One line per finished pass on stderr (stdout carries only the result line)."""
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def sparse_work(cfg, topk):
    """Algorithmic bytes and FLOPs of attention over index lists of topk distinct visible positions
    per query token: the listed cache rows, the lists, wkv_b, q and out."""
    B, S, H = cfg.batch, cfg.seqlen_q, cfg.n_heads
    C, R, Dn, Dv = cfg.kv_lora_rank, cfg.qk_rope_head_dim, cfg.qk_nope_head_dim, cfg.v_head_dim
    e = 2
    rows = B * S * topk
    flops = 2 * B * S * H * Dn * C + 2 * H * rows * (C + R) + 2 * H * rows * C + 2 * B * S * H * C * Dv
    return {"bytes": rows * (C + R) * e + rows * 4 + H * (Dn + Dv) * C * e + B * S * H * (Dn + R + Dv) * e,
            "flops": flops, "attn_kernel_bytes": rows * (C + R) * e + rows * 4 + B * S * H * R * e}


def attn_work(cfg, lens=None):
    """Algorithmic bytes and FLOPs of one absorb-attention call (caches [:B, :end_pos], wkv_b, q, out);
    with lens, a ragged batch (sequence b reads positions [0, lens[b]))."""
    B, S, H = cfg.batch, cfg.seqlen_q, cfg.n_heads
    C, R, Dn, Dv, T = cfg.kv_lora_rank, cfg.qk_rope_head_dim, cfg.qk_nope_head_dim, cfg.v_head_dim, cfg.end_pos
    lens = [T] * B if lens is None else [int(n) for n in lens]
    e = 2  # bf16
    cache = sum(lens) * (C + R) * e
    weights = H * (Dn + Dv) * C * e
    q = B * S * H * (Dn + R) * e
    out = B * S * H * Dv * e
    # visible (query, position) pairs per head, summed over the sequences
    pairs = sum(n - S + s + 1 for n in lens for s in range(S))
    flops = 2 * B * S * H * Dn * C + 2 * H * pairs * (C + R) + 2 * H * pairs * C + 2 * B * S * H * C * Dv
    return {"bytes": cache + weights + q + out, "flops": flops, "cache_bytes": cache,
            "attn_kernel_bytes": cache + B * S * H * R * e}


def expand_work(cfg):
    T, H, C, Dn, Dv = cfg.n_tokens, cfg.n_heads, cfg.kv_lora_rank, cfg.qk_nope_head_dim, cfg.v_head_dim
    e = 2
    return {"bytes": T * C * e + C * e + H * (Dn + Dv) * C * e + H * T * (Dn + Dv) * e,
            "flops": 2 * T * C * H * (Dn + Dv)}


def gpu_inputs(cfg, seed, torch):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)

    def draw(shape, std):
        return (torch.randn(shape, generator=g, device="cuda", dtype=torch.float32) * std).to(torch.bfloat16)

    B, S, H = cfg.batch, cfg.seqlen_q, cfg.n_heads
    return {
        "q_nope": draw((B, S, H, cfg.qk_nope_head_dim), 1.0),
        "q_pe": draw((B, S, H, cfg.qk_rope_head_dim), 1.0),
        "kv_cache": draw((cfg.cache_batch, cfg.cache_len, cfg.kv_lora_rank), 1.0),
        "pe_cache": draw((cfg.cache_batch, cfg.cache_len, cfg.qk_rope_head_dim), 1.0),
        "wkv_b": draw((H * (cfg.qk_nope_head_dim + cfg.v_head_dim), cfg.kv_lora_rank), math.sqrt(cfg.wkv_b_var)),
    }


def to_paged(x, cfg, page_size, seed, torch):
    """Move one input set's caches into page pools in a random page order; returns the table."""
    B, T = cfg.cache_batch, cfg.cache_len
    npp = T // page_size
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    table = torch.randperm(B * npp, generator=g).to(torch.int32).view(B, npp).contiguous().to("cuda")
    for key in ("kv_cache", "pe_cache"):
        pool = torch.empty((B * npp, page_size, x[key].shape[-1]), dtype=x[key].dtype, device="cuda")
        pool[table.long()] = x[key].view(B, npp, page_size, -1)
        x[key] = pool
    return table


def random_lists(cfg, topk, seed, torch):
    """topk distinct positions per query token, drawn uniformly from the visible ones (decode)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    rows = [torch.randperm(cfg.end_pos, generator=g)[:topk] for _ in range(cfg.batch * cfg.seqlen_q)]
    return torch.stack(rows).to(torch.int32).view(cfg.batch, cfg.seqlen_q, topk).contiguous().to("cuda")


def time_attn(cfg, steps, warmup, sets, torch, binding, seed=1, timed_kernels=0b010, lens=None, page_size=0,
              topk=0, num_splits=0):
    """Returns (GPU us per step, host enqueue us per step, per-kernel timing dict).  With lens, a
    ragged batch (mla_absorb_attn_ragged with the lengths in device memory, bound cfg.end_pos);
    with page_size, the caches live in page pools in random page order (mla_absorb_attn_paged);
    with topk, each token attends to topk random positions (mla_absorb_attn_sparse).  num_splits > 0
    forces the split count (0: the library's plan)."""
    inputs = [gpu_inputs(cfg, seed + 1000 * i, torch) for i in range(sets)]
    seq_lens = None if lens is None else torch.tensor([int(n) for n in lens], dtype=torch.int32, device="cuda")
    out = torch.empty((cfg.batch, cfg.seqlen_q, cfg.n_heads, cfg.v_head_dim), dtype=torch.bfloat16, device="cuda")
    shape = binding.attn_shape(inputs[0]["q_nope"], inputs[0]["q_pe"], inputs[0]["kv_cache"], inputs[0]["wkv_b"])
    lists = [random_lists(cfg, topk, seed + i, torch) if topk else None for i in range(sets)]
    if page_size:
        paged = binding.PagedCache(page_size, cfg.cache_batch * cfg.cache_len // page_size,
                                   cfg.cache_len // page_size)
        need = binding.absorb_attn_paged_workspace_size(shape, cfg.end_pos, paged, binding.MLA_DTYPE_BF16)
    elif topk:
        need = binding.absorb_attn_sparse_workspace_size(shape, cfg.end_pos, topk, binding.MLA_DTYPE_BF16)
    elif lens is not None:
        need = binding.absorb_attn_ragged_workspace_size(shape, cfg.end_pos, binding.MLA_DTYPE_BF16, num_splits)
    else:
        need = binding.absorb_attn_workspace_size(shape, cfg.end_pos, binding.MLA_DTYPE_BF16)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    tables = [to_paged(x, cfg, page_size, seed + i, torch) if page_size else None for i, x in enumerate(inputs)]
    calls = [binding.AbsorbAttnCall(x["q_nope"], x["q_pe"], x["kv_cache"], x["pe_cache"], x["wkv_b"], cfg.end_pos,
                                    cfg.softmax_scale, out, workspace=ws, seq_lens=seq_lens, block_table=tb,
                                    indices=il, num_splits=num_splits)
             for x, tb, il in zip(inputs, tables, lists)]

    def step(i):
        calls[i % sets]()

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    binding.timing_enable(timed_kernels)
    binding.timing_collect()  # drop anything recorded before the timed region
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for i in range(steps):
        step(warmup + i)
    e1.record()
    enqueue = (time.perf_counter() - t0) * 1e6 / steps
    torch.cuda.synchronize()
    kt = binding.timing_collect()
    binding.timing_enable(0)
    del inputs, calls, tables, lists
    torch.cuda.empty_cache()
    us = e0.elapsed_time(e1) * 1000.0 / steps
    progress(f"{cfg.name} lens={lens is not None} page={page_size} topk={topk} kernels={timed_kernels:#x}: {us:.2f} us/step")
    return us, enqueue, kt


def time_append_attn(cfg, steps, warmup, sets, torch, binding, fused, seed=1):
    """GPU us per serving decode step: each sequence's new token appended into the caches (its
    RMS-normalised latent and its rope key at position end_pos - 1), then absorb attention over
    [0, end_pos).  fused: one mla_absorb_attn_append call; else mla_cache_append followed by
    mla_absorb_attn."""
    import ctypes

    inputs = [gpu_inputs(cfg, seed + 1000 * i, torch) for i in range(sets)]
    g = torch.Generator(device="cuda")
    g.manual_seed(seed + 7)
    news = [(torch.randn((cfg.batch, cfg.seqlen_q, cfg.kv_lora_rank), generator=g, device="cuda").to(torch.bfloat16),
             torch.randn((cfg.batch, cfg.seqlen_q, cfg.qk_rope_head_dim), generator=g, device="cuda").to(torch.bfloat16))
            for _ in range(sets)]
    rms_w = (1.0 + 0.14 * torch.randn((cfg.kv_lora_rank,), generator=g, device="cuda")).to(torch.bfloat16)
    out = torch.empty((cfg.batch, cfg.seqlen_q, cfg.n_heads, cfg.v_head_dim), dtype=torch.bfloat16, device="cuda")
    shape = binding.attn_shape(inputs[0]["q_nope"], inputs[0]["q_pe"], inputs[0]["kv_cache"], inputs[0]["wkv_b"])
    ws = torch.empty(binding.absorb_attn_workspace_size(shape, cfg.end_pos, binding.MLA_DTYPE_BF16), dtype=torch.uint8,
                     device="cuda")
    lib = binding.load()
    steps_fn = []
    for x, (c_new, kp_new) in zip(inputs, news):
        if fused:
            steps_fn.append(binding.AbsorbAttnCall(x["q_nope"], x["q_pe"], x["kv_cache"], x["pe_cache"], x["wkv_b"],
                                                   cfg.end_pos, cfg.softmax_scale, out, workspace=ws,
                                                   append=(c_new, kp_new, rms_w, 1e-6)))
            continue
        attn = binding.AbsorbAttnCall(x["q_nope"], x["q_pe"], x["kv_cache"], x["pe_cache"], x["wkv_b"], cfg.end_pos,
                                      cfg.softmax_scale, out, workspace=ws)
        ashape = binding.AttnShape(cfg.batch, cfg.seqlen_q, 1, cfg.kv_lora_rank, cfg.qk_rope_head_dim, 0, 0,
                                   cfg.cache_batch, cfg.cache_len)
        args = (c_new.data_ptr(), kp_new.data_ptr(), rms_w.data_ptr(), 1e-6, None, cfg.end_pos,
                x["kv_cache"].data_ptr(), x["pe_cache"].data_ptr(), ctypes.byref(ashape), binding.MLA_DTYPE_BF16,
                torch.cuda.current_stream().cuda_stream)

        def two_calls(args=args, attn=attn, keep=ashape):
            rc = lib.mla_cache_append(*args)
            if rc != 0:
                raise RuntimeError(binding.last_error())
            attn()

        steps_fn.append(two_calls)
    for i in range(warmup):
        steps_fn[i % sets]()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        steps_fn[(warmup + i) % sets]()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1000.0 / steps
    del inputs, news, steps_fn
    torch.cuda.empty_cache()
    progress(f"{cfg.name} append+attend fused={fused}: {us:.2f} us/step")
    return us


def time_expand(cfg, steps, warmup, torch, binding, seed=4, sets=4, timed_kernels=0):
    """GPU us per expansion over `sets` rotated input sets (c_kv, rms_w, wkv_b) and output pairs,
    so that no call finds its operands in the Infinity Cache; with timed_kernels, also the
    per-kernel timing dict."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    ins, outs = [], []
    for _ in range(sets):
        x = torch.randn((cfg.n_tokens, cfg.kv_lora_rank), generator=g, device="cuda").to(torch.bfloat16)
        w = (1.0 + math.sqrt(cfg.rms_w_var) * torch.randn((cfg.kv_lora_rank,), generator=g, device="cuda")).to(
            torch.bfloat16)
        wk = (torch.randn((cfg.n_heads * (cfg.qk_nope_head_dim + cfg.v_head_dim), cfg.kv_lora_rank), generator=g,
                          device="cuda") * math.sqrt(cfg.wkv_b_var)).to(torch.bfloat16)
        ins.append((x, w, wk))
    for _ in range(2):  # two output pairs (537 MB each) alternate
        outs.append((torch.empty((cfg.n_heads, cfg.n_tokens, cfg.qk_nope_head_dim), dtype=torch.bfloat16, device="cuda"),
                     torch.empty((cfg.n_heads, cfg.n_tokens, cfg.v_head_dim), dtype=torch.bfloat16, device="cuda")))
    need = binding.expand_kv_workspace_size(cfg.n_tokens, cfg.n_heads, cfg.kv_lora_rank, cfg.qk_nope_head_dim,
                                            cfg.v_head_dim, binding.MLA_DTYPE_BF16)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")

    def step(i):
        x, w, wk = ins[i % sets]
        k, v = outs[i % 2]
        binding.expand_kv(x, w, wk, cfg.n_heads, cfg.qk_nope_head_dim, cfg.v_head_dim, cfg.eps, k, v, workspace=ws)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    binding.timing_enable(timed_kernels)
    binding.timing_collect()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        step(warmup + i)
    e1.record()
    torch.cuda.synchronize()
    kt = binding.timing_collect()
    binding.timing_enable(0)
    del ins, outs, ws
    torch.cuda.empty_cache()
    us = e0.elapsed_time(e1) * 1000.0 / steps
    progress(f"{cfg.name}: {us:.2f} us/step")
    return (us, kt) if timed_kernels else us


def time_tiny_f32(cfg, steps, warmup, torch, binding):
    """The tiny fp32 decode (one sequence, 4 heads, 128 positions) on the plain kernels: launch
    latency, not bandwidth, sets its time.  Inputs are the oracle tests' seeded ones."""
    from mla_latent_kv_absorb_amd.workloads import make_attn_inputs

    x = {k: torch.from_numpy(v).to("cuda") for k, v in make_attn_inputs(cfg).items()}
    call = binding.AbsorbAttnCall(x["q_nope"], x["q_pe"], x["kv_cache"], x["pe_cache"], x["wkv_b"], cfg.end_pos,
                                  cfg.softmax_scale)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1000.0 / steps
    progress(f"{cfg.name}: {us:.2f} us/step")
    return us


def naive_work(cfg):
    """Algorithmic bytes and FLOPs of the naive route's attention over expanded keys and values:
    k_nope, v and pe rows of the visible positions, q and out; scores over Dn + R, sum over Dv."""
    B, S, H = cfg.batch, cfg.seqlen_q, cfg.n_heads
    R, Dn, Dv, T = cfg.qk_rope_head_dim, cfg.qk_nope_head_dim, cfg.v_head_dim, cfg.end_pos
    e = 2
    pairs = B * sum(T - S + s + 1 for s in range(S))
    return {"bytes": (B * T * H * (Dn + Dv) + B * T * R + B * S * H * (Dn + R + Dv)) * e,
            "flops": 2 * H * pairs * (Dn + R + Dv)}


def time_naive_route(cfg, steps, warmup, torch, binding, seed=3, from_latent=False):
    """A chunk step of the naive route.  By default the naive path as the pages lay it out: the
    caches hold full-width head-major keys and values (filled once, before timing, with the
    expansion of the cached latents), and a step expands the chunk's B x S new tokens into them
    with their rope keys (mla_expand_kv_append), then attends over the caches.  With from_latent,
    a step instead expands every cached latent row (what the naive attention needs when only the
    latent cache is kept), then attends.  Returns (us per step, per-kernel timing dict)."""
    x = gpu_inputs(cfg, seed, torch)
    H, C, Dn, Dv = cfg.n_heads, cfg.kv_lora_rank, cfg.qk_nope_head_dim, cfg.v_head_dim
    B, S, R = cfg.batch, cfg.seqlen_q, cfg.qk_rope_head_dim
    rows = cfg.cache_batch * cfg.cache_len
    g = torch.Generator(device="cuda")
    g.manual_seed(seed + 7)
    w = (1.0 + 0.14 * torch.randn((C,), generator=g, device="cuda")).to(torch.bfloat16)
    k = torch.empty((H, rows, Dn), dtype=torch.bfloat16, device="cuda")
    v = torch.empty((H, rows, Dv), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((cfg.batch, cfg.seqlen_q, H, Dv), dtype=torch.bfloat16, device="cuda")
    need = binding.expand_kv_workspace_size(rows, H, C, Dn, Dv, binding.MLA_DTYPE_BF16)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    lat = x["kv_cache"].view(rows, C)
    k4, v4 = k.view(H, cfg.cache_batch, cfg.cache_len, Dn), v.view(H, cfg.cache_batch, cfg.cache_len, Dv)
    attend = binding.NaiveAttnCall(x["q_nope"], x["q_pe"], k4, v4, x["pe_cache"], cfg.end_pos, cfg.softmax_scale, out)
    if from_latent:
        def step():
            binding.expand_kv(lat, w, x["wkv_b"], H, Dn, Dv, 1e-6, k, v, workspace=ws)
            attend()
    else:
        binding.expand_kv(lat, w, x["wkv_b"], H, Dn, Dv, 1e-6, k, v, workspace=ws)  # the earlier positions
        c_new = torch.randn((B, S, C), generator=g, device="cuda").to(torch.bfloat16)
        kp_new = torch.randn((B, S, R), generator=g, device="cuda").to(torch.bfloat16)
        append = binding.ExpandAppendCall(c_new, kp_new, w, x["wkv_b"], 1e-6, cfg.end_pos, k4, v4, x["pe_cache"],
                                          workspace=ws)

        def step():
            append()
            attend()

    def timed(mask):
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        binding.timing_enable(mask)
        binding.timing_collect()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            step()
        e1.record()
        torch.cuda.synchronize()
        kt = binding.timing_collect()
        binding.timing_enable(0)
        return e0.elapsed_time(e1) * 1000.0 / steps, kt

    us, _ = timed(0)
    _, kt = timed((1 << 3) | (1 << 4) | (1 << 6))
    progress(f"{cfg.name} naive route{' from the latent cache' if from_latent else ''}: {us:.2f} us/step")
    del x, k, v, out, ws
    torch.cuda.empty_cache()
    return us, kt


def cpu_baseline(cfg, n_seq=4):
    """The CPU oracle's absorb route in float32 NumPy (BLAS-backed matmuls) on the first n_seq
    sequences of the workload, all host cores and then one core: one warm-up call, then the
    median of three timed calls, scaled to microseconds per full step (batch / n_seq)."""
    import numpy as np

    from mla_latent_kv_absorb_amd.workloads import make_attn_inputs
    from oracle import mla_oracle as O

    try:
        from threadpoolctl import threadpool_info, threadpool_limits
    except Exception:  # pragma: no cover - threadpoolctl ships with the image
        threadpool_info = threadpool_limits = None
    sub = cfg.replace(batch=n_seq, cache_batch=n_seq)
    x = make_attn_inputs(sub, seed=cfg.seed)

    def run():
        O.absorb_attention(x["q_nope"], x["q_pe"], x["kv_cache"], x["pe_cache"], x["wkv_b"], cfg.end_pos,
                           cfg.softmax_scale, cfg.v_head_dim, dtype=np.float32)

    def median_of_three():
        run()
        times = []
        for _ in range(3):
            t0 = time.perf_counter()
            run()
            times.append(time.perf_counter() - t0)
        return sorted(times)[1]

    threads = os.cpu_count() or 1
    if threadpool_info is not None:
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    t_all = median_of_three()
    t_one = None
    if threadpool_limits is not None:
        with threadpool_limits(limits=1, user_api="blas"):
            t_one = median_of_three()
    scale = cfg.batch / n_seq
    progress(f"cpu baseline: {t_all * 1e3:.1f} ms on {threads} threads, "
             f"{(t_one or 0) * 1e3:.1f} ms on 1, per {n_seq}-sequence call")
    res = {"value": round(t_all * 1e6 * scale, 1), "unit": "us/step", "cores": int(threads), "kind": "oracle",
           "sample": f"absorb route, float32 NumPy, {n_seq} of {cfg.batch} sequences (same shapes otherwise), "
                     f"median of 3 calls after 1 warm-up, scaled by {cfg.batch}/{n_seq}",
           "host_cpus": os.cpu_count()}
    if t_one is not None:
        res["single_core"] = {"value": round(t_one * 1e6 * scale, 1), "unit": "us/step", "cores": 1}
    return res


def measure_peaks(torch):
    """What this machine's HBM, matrix cores and LDS deliver to simple kernels (the probes in
    libmla_peaks.so): streaming read and copy bandwidth, dense bf16 MFMA rate with the engine clock
    it ran at, and LDS read bytes per clock per compute unit."""
    import ctypes

    from mla_latent_kv_absorb_amd import build as B

    lib = ctypes.CDLL(B.PEAKS_LIB_PATH)
    vp, i32, u64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64
    lib.mla_peak_read.argtypes = [vp, u64, vp, i32, vp]
    lib.mla_peak_copy.argtypes = [vp, vp, u64, i32, vp]
    lib.mla_peak_mfma.argtypes = [i32, i32, vp, vp, vp]
    lib.mla_peak_lds.argtypes = [i32, i32, vp, vp, vp]
    for f in (lib.mla_peak_read, lib.mla_peak_copy, lib.mla_peak_mfma, lib.mla_peak_lds):
        f.restype = i32
    stream = torch.cuda.current_stream().cuda_stream

    def timed(launch, reps):
        for _ in range(2):
            assert launch() == 0
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            assert launch() == 0
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    n = 2 << 30  # 2 GiB: far past the 256 MB Infinity Cache
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    sink = torch.zeros(1 << 20, dtype=torch.int32, device="cuda")
    blocks = 256 * 8
    t_read = timed(lambda: lib.mla_peak_read(a.data_ptr(), n, sink.data_ptr(), blocks, stream), 10)
    half = n // 2
    t_copy = timed(lambda: lib.mla_peak_copy(a.data_ptr(), a.data_ptr() + half, half, blocks, stream), 10)
    del a
    iters, mblocks = 4096, 256 * 4
    clocks = torch.zeros(2 * mblocks, dtype=torch.int64, device="cuda")
    fsink = torch.zeros(mblocks * 256, dtype=torch.float32, device="cuda")
    t_mfma = timed(lambda: lib.mla_peak_mfma(iters, mblocks, fsink.data_ptr(), clocks.data_ptr(), stream), 5)
    c = clocks.view(mblocks, 2).double()
    mhz = float((c[:, 0] / c[:, 1]).median()) * 100.0  # shader clocks per 100 MHz real-time tick
    flops = mblocks * 4 * iters * 8 * 32768
    lclocks = torch.zeros(512, dtype=torch.int64, device="cuda")
    liters = 2048
    t_lds = timed(lambda: lib.mla_peak_lds(liters, 512, sink.data_ptr(), lclocks.data_ptr(), stream), 5)
    lds_cyc = float(lclocks.double().median())
    # two workgroups per compute unit (64 KB of LDS each), each moving 4 waves x 8 x 1 KB per iteration
    lds_bpc = 2 * 4 * 8 * 1024 * liters / lds_cyc
    del clocks, fsink, lclocks, sink
    torch.cuda.empty_cache()
    res = {"read_gbs": round(n / t_read / 1e9, 1), "copy_gbs": round(2 * half / t_copy / 1e9, 1),
           "mfma_bf16_tflops": round(flops / t_mfma / 1e12, 1), "mfma_clock_mhz": round(mhz, 0),
           "lds_read_bytes_per_clk_per_cu": round(lds_bpc, 1), "lds_wall_gbs": round(512 * 4 * 8 * 1024 * liters / t_lds / 1e9, 1)}
    progress(f"peaks: {res}")
    return res


def traffic_for(kernel_src, name):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they match this source."""
    path = os.path.join(ROOT, "profiles", f"{name}_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
        sha = hashlib.sha256(open(kernel_src, "rb").read()).hexdigest()
        if rec.get("source_sha256") != sha:
            return None
        return rec.get("traffic_bytes")
    except Exception:
        return None


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="dsv3_decode")
    ap.add_argument("--sets", type=int, default=4, help="input sets rotated over (cold Infinity Cache)")
    ap.add_argument("--no-extras", action="store_true", help="skip timing the other workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peaks", action="store_true", help="skip the streaming / matrix-core / LDS peak probes")
    ap.add_argument("--profile", action="store_true",
                    help="only run --warmup + --steps steps of --workload (an attention workload, "
                         "chunk_prefill_naive, chunk_prefill_naive_from_latent or dsv3_expand) with no timing "
                         "passes, extras, probes or CPU baseline: the command rocprofv3 profiles")
    ap.add_argument("--sustained-ms", type=float, default=40.0,
                    help="length of the labelled sustained-load decode run (0 to skip)")
    ap.add_argument("--peaks", action="store_true",
                    help="only run the streaming-read, copy, matrix-core and LDS probes and print what they reach")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB, --steps times (reference "
                         "kernel of known size for scaling the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from mla_latent_kv_absorb_amd import binding
    from mla_latent_kv_absorb_amd.workloads import ATTN_CONFIGS, EXPAND_CONFIGS, RAGGED_WORKLOADS, ragged_workload

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    binding.load()  # fails loudly if the HIP library is not built
    torch.cuda.set_device(0)

    if args.peaks:
        print(json.dumps({"peaks_measured": measure_peaks(torch)}))
        return

    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20)
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "bytes_written": n, "dispatches": args.steps}))
        return

    if args.profile:
        if args.workload == "dsv3_expand":
            us = time_expand(EXPAND_CONFIGS["dsv3_expand"], args.steps, args.warmup, torch, binding)
        elif args.workload in ("chunk_prefill_naive", "chunk_prefill_naive_from_latent"):
            us, _ = time_naive_route(ATTN_CONFIGS["chunk_prefill"], args.steps, args.warmup, torch, binding,
                                     seed=ATTN_CONFIGS["chunk_prefill"].seed,
                                     from_latent=args.workload.endswith("from_latent"))
        else:
            c = ATTN_CONFIGS[args.workload]
            us, _, _ = time_attn(c, args.steps, args.warmup, min(args.sets, 2 if c.seqlen_q > 1 else args.sets),
                                 torch, binding, seed=c.seed, timed_kernels=0)
        print(json.dumps({"profile_run": args.workload, "steps": args.steps, "us_per_step": round(us, 2)}))
        return

    peaks = None if args.no_peaks else measure_peaks(torch)
    cfg = ATTN_CONFIGS[args.workload]
    work = attn_work(cfg)
    # the step time: no per-kernel events in the timed steps (each timed dispatch adds a queue
    # barrier of its own, several microseconds per kernel)
    us, enqueue_us, _ = time_attn(cfg, args.steps, args.warmup, args.sets, torch, binding, timed_kernels=0)
    # the same K steps again with the attention kernel's dispatch-stamped events: its live duration
    us_ev, _, kt = time_attn(cfg, args.steps, args.warmup, args.sets, torch, binding, timed_kernels=0b010)
    # per-kernel averages of the same workload in a third, fully instrumented pass
    _, _, kt_all = time_attn(cfg, 20, 3, args.sets, torch, binding, timed_kernels=0b111)
    gbs = work["bytes"] / (us * 1e-6) / 1e9
    tflops = work["flops"] / (us * 1e-6) / 1e12

    attn = kt.get("attn")
    roofline = None
    if attn:
        kb = work["attn_kernel_bytes"]
        ach = kb / (attn["avg_us"] * 1e-6) / 1e9
        src = os.path.join(ROOT, "mla_latent_kv_absorb_amd", "csrc", "absorb_mfma.hip")
        roofline = {"kernel": "attn_kernel", "bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic_for(src, "attn_kernel"),
                    "algorithmic_bytes": kb, "avg_us": round(attn["avg_us"], 2), "launches": attn["launches"]}
        if peaks:
            roofline["measured_peak"] = peaks["read_gbs"]
            roofline["frac_measured_peak"] = round(ach / peaks["read_gbs"], 4)

    line = {
        "metric": METRIC,
        "value": round(us, 2),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us / 1000.0, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "batch": cfg.batch, "seqlen_q": cfg.seqlen_q, "n_heads": cfg.n_heads,
                   "kv_lora_rank": cfg.kv_lora_rank, "qk_rope_head_dim": cfg.qk_rope_head_dim,
                   "qk_nope_head_dim": cfg.qk_nope_head_dim, "v_head_dim": cfg.v_head_dim,
                   "end_pos": cfg.end_pos, "input_sets_rotated": args.sets},
        "gbps": round(gbs, 1),
        "tflops": round(tflops, 2),
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "mfma_frac": round(tflops / BF16_PEAK_TFLOPS, 4),
        "algorithmic_bytes": work["bytes"],
        "algorithmic_flops": work["flops"],
        "host_enqueue_us_per_step": round(enqueue_us, 2),
        "us_per_step_with_attn_events": round(us_ev, 2),
        "roofline": roofline,
        "kernels_us": {n: round(v["avg_us"], 2) for n, v in kt_all.items()},
    }
    if peaks:
        line["peaks_measured"] = peaks
        line["hbm_frac_measured_peak"] = round(gbs / peaks["read_gbs"], 4)
        line["mfma_frac_measured_peak"] = round(tflops / peaks["mfma_bf16_tflops"], 4)
    if args.sustained_ms > 0:
        # a labelled extra: back-to-back steps for sustained_ms of GPU time (the chip's power
        # management lowers its clocks after a few milliseconds of load)
        n = max(args.steps, int(args.sustained_ms * 1000.0 / us))
        su, _, _ = time_attn(cfg, n, args.warmup, args.sets, torch, binding, timed_kernels=0)
        line["sustained"] = {"us_per_step": round(su, 2), "steps": n, "gpu_ms": round(su * n / 1000.0, 1)}

    if not args.no_extras:
        extras = {}
        for name in ("long_decode", "chunk_prefill"):
            c = ATTN_CONFIGS[name]
            w = attn_work(c)
            steps = 10 if name == "chunk_prefill" else 30
            sets = 2 if name == "chunk_prefill" else args.sets
            u, _, _ = time_attn(c, steps, 3, sets, torch, binding, seed=c.seed, timed_kernels=0)
            _, _, k = time_attn(c, steps, 3, sets, torch, binding, seed=c.seed, timed_kernels=0b111)
            extras[name] = {"us_per_step": round(u, 2), "gbps": round(w["bytes"] / (u * 1e-6) / 1e9, 1),
                            "tflops": round(w["flops"] / (u * 1e-6) / 1e12, 2),
                            "kernels_us": {n: round(v["avg_us"], 2) for n, v in k.items()}}
        for name in RAGGED_WORKLOADS:
            base, lens = ragged_workload(name)
            c = ATTN_CONFIGS[base]
            w = attn_work(c, lens)
            u, _, _ = time_attn(c, 30, 3, args.sets, torch, binding, seed=c.seed, timed_kernels=0, lens=lens)
            _, _, k = time_attn(c, 30, 3, args.sets, torch, binding, seed=c.seed, timed_kernels=0b111, lens=lens)
            # the same batch under the uniform plan: every sequence cut into the split count a batch
            # of equal lengths gets (one workgroup per compute unit, at least 128 positions a split)
            units = c.batch * -(-c.seqlen_q * c.n_heads // 128)
            uniform = max(1, min((256 + units // 2) // units, -(-c.end_pos // 128)))
            uu, _, _ = time_attn(c, 30, 3, args.sets, torch, binding, seed=c.seed, timed_kernels=0, lens=lens,
                                 num_splits=uniform)
            extras[name] = {"us_per_step": round(u, 2), "gbps": round(w["bytes"] / (u * 1e-6) / 1e9, 1),
                            "tflops": round(w["flops"] / (u * 1e-6) / 1e12, 2),
                            "lengths": [int(lens.min()), int(lens.max()), int(sum(lens))],
                            "kernels_us": {n: round(v["avg_us"], 2) for n, v in k.items()},
                            "uniform_plan": {"num_splits": uniform, "us_per_step": round(uu, 2)}}
        c = ATTN_CONFIGS["dsv3_decode"]
        w = attn_work(c)
        u, _, _ = time_attn(c, 30, 3, args.sets, torch, binding, seed=c.seed, timed_kernels=0, page_size=64)
        _, _, k = time_attn(c, 30, 3, args.sets, torch, binding, seed=c.seed, timed_kernels=0b111, page_size=64)
        extras["paged_decode"] = {"us_per_step": round(u, 2), "gbps": round(w["bytes"] / (u * 1e-6) / 1e9, 1),
                                  "page_size": 64, "kernels_us": {n: round(v["avg_us"], 2) for n, v in k.items()}}
        # a serving decode step: the new token's cache rows, then attention; fused into one call
        # (the rows written by the query-absorption kernel) against the two calls
        uf = time_append_attn(c, 30, 3, args.sets, torch, binding, fused=True)
        us2 = time_append_attn(c, 30, 3, args.sets, torch, binding, fused=False)
        extras["decode_append"] = {"fused_us_per_step": round(uf, 2), "two_calls_us_per_step": round(us2, 2)}
        for name, base in (("sparse_decode", "dsv3_decode"), ("sparse_long_decode", "long_decode")):
            c = ATTN_CONFIGS[base]
            w = sparse_work(c, 2048)
            u, _, _ = time_attn(c, 30, 3, args.sets, torch, binding, seed=c.seed, timed_kernels=0, topk=2048)
            _, _, k = time_attn(c, 30, 3, args.sets, torch, binding, seed=c.seed, timed_kernels=0b111, topk=2048)
            extras[name] = {"us_per_step": round(u, 2), "gbps": round(w["bytes"] / (u * 1e-6) / 1e9, 1),
                            "topk": 2048, "kernels_us": {n: round(v["avg_us"], 2) for n, v in k.items()},
                            "attn_gbps": round(w["attn_kernel_bytes"] / (k["attn"]["avg_us"] * 1e-6) / 1e9, 1)}
        c = ATTN_CONFIGS["chunk_prefill"]
        w = naive_work(c)
        for name, from_latent in (("chunk_prefill_naive", False), ("chunk_prefill_naive_from_latent", True)):
            u, k = time_naive_route(c, 10, 3, torch, binding, seed=c.seed, from_latent=from_latent)
            a_us = k["naive"]["avg_us"]
            extras[name] = {
                "us_per_step": round(u, 2), "kernels_us": {n: round(v["avg_us"], 2) for n, v in k.items()},
                "expanded_tokens": (c.cache_batch * c.cache_len) if from_latent else c.batch * c.seqlen_q,
                "naive_attn_tflops": round(w["flops"] / (a_us * 1e-6) / 1e12, 1),
                "naive_attn_mfma_frac": round(w["flops"] / (a_us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4),
                "naive_attn_gbps": round(w["bytes"] / (a_us * 1e-6) / 1e9, 1)}
        ec = EXPAND_CONFIGS["dsv3_expand"]
        u = time_expand(ec, 20, 3, torch, binding)
        _, k = time_expand(ec, 20, 3, torch, binding, timed_kernels=(1 << 3) | (1 << 4))
        w = expand_work(ec)
        tf = w["flops"] / (u * 1e-6) / 1e12
        extras["dsv3_expand"] = {"us_per_step": round(u, 2), "gbps": round(w["bytes"] / (u * 1e-6) / 1e9, 1),
                                 "tflops": round(tf, 2), "mfma_frac": round(tf / BF16_PEAK_TFLOPS, 4),
                                 "kernels_us": {n: round(v["avg_us"], 2) for n, v in k.items()}}
        if peaks:
            extras["dsv3_expand"]["mfma_frac_measured_peak"] = round(tf / peaks["mfma_bf16_tflops"], 4)
        tc = ATTN_CONFIGS["tiny_f32"]
        tw = attn_work(tc)
        u = time_tiny_f32(tc, 200, 20, torch, binding)
        extras["tiny_f32"] = {"us_per_step": round(u, 2), "note": "fp32, plain kernels; launch latency bound",
                              "gbps": round(tw["bytes"] * 2 / (u * 1e-6) / 1e9, 3)}
        line["extras"] = extras

    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
