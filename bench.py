#!/usr/bin/env python3
"""Benchmark of the MLA forward hot path on one MI355X.

Headline: the Kimi K2-shaped MLA prefill (B=1, T=2048, d=7168, 64 heads,
q latent 1536, kv latent 512, 128+64 query/key and 128 value widths, causal,
bf16 with fp32 softmax/accumulation), reported as algorithmic TFLOP/s of the
whole step and, for the dominant kernel, against the bf16 MFMA peak.

One step = one mla_prefill call (down-projections + norms + RoPE, up-
projections, flash attention, o_proj) on inputs already resident in HBM.
Secondary lines (same JSON object, key "secondary") time the full-cache
decode (B=64, P=1000), the absorbed latent-cache decode (B=32, P=8192), the
same over a ragged batch (B=32, per-sequence positions uniform in
[0, 8192]), a chunked prefill (512 new tokens after 3584 cached positions,
full and latent cache forms), the dense block (B=1, T=4096) with the same
weights, and a decode sweep over P in {1000, 4096, 8192, 16384} at B = 32 and
64 for both cache forms, against the HBM or MFMA roofline.  The CPU baseline times the float32 oracle on the host cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
WARM_S = 0.25                  # minimum untimed warm-up per workload, seconds
CPU_SAMPLE_S = 10.0            # minimum CPU-baseline sample, seconds
MFMA_BF16_PEAK_TFS = 2500.0    # MI355X dense bf16 MFMA, TFLOP/s

KIMI = dict(d_model=7168, n_heads=64, q_lora_rank=1536, kv_lora_rank=512, qk_nope_dim=128,
            qk_rope_dim=64, v_head_dim=128, d_ff=18432)


def prefill_kernel_flops(B, T, k=KIMI):
    """Algorithmic FLOPs per launch of each prefill kernel (2 per multiply-add;
    attention counts only the visible (causal) query/key pairs)."""
    M = B * T
    H = k["n_heads"]
    dqk = k["qk_nope_dim"] + k["qk_rope_dim"]
    n1 = k["q_lora_rank"] + k["kv_lora_rank"] + k["qk_rope_dim"]
    q_up = 2.0 * M * H * dqk * k["q_lora_rank"]
    kv_up = 2.0 * M * H * (k["qk_nope_dim"] + k["v_head_dim"]) * k["kv_lora_rank"]
    return {
        "gemm_down": 2.0 * M * n1 * k["d_model"],
        "gemm_q_up": q_up,
        "gemm_kv_up": kv_up,
        "gemm_qkv_up": q_up + kv_up,  # both up-projections in one launch
        "flash_prefill": 2.0 * H * B * (T * (T + 1) / 2) * (dqk + k["v_head_dim"]),
        "gemm_o_proj": 2.0 * M * k["d_model"] * H * k["v_head_dim"],
    }


def mla_param_count(k=KIMI):
    H = k["n_heads"]
    dqk = k["qk_nope_dim"] + k["qk_rope_dim"]
    return (k["q_lora_rank"] * k["d_model"] + k["q_lora_rank"] + H * dqk * k["q_lora_rank"]
            + (k["kv_lora_rank"] + k["qk_rope_dim"]) * k["d_model"] + k["kv_lora_rank"]
            + H * (k["qk_nope_dim"] + k["v_head_dim"]) * k["kv_lora_rank"]
            + k["d_model"] * H * k["v_head_dim"])


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary, or None when the GEMM source changed since the counters were
    taken (the summary records a hash of the source it measured)."""
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", "prefill_kimi_T2048_hbm_traffic.md")
    src = os.path.join(ROOT, "head_latent_attention_fwd_amd", "csrc", "gemm_bf16.hip")
    try:
        text = open(path).read()
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    except OSError:
        return None
    m = re.search(rf"{kernel} traffic_bytes_per_launch=(\d+) gemm_source_sha256_16=([0-9a-f]+)", text)
    if not m or m.group(2) != sha:
        return None
    return int(m.group(1))


def decode_source_hash():
    """First 16 hex digits of the SHA-256 of the decode attention kernels'
    sources (decode.hip, then latent_body.h)."""
    import hashlib
    h = hashlib.sha256()
    for f in ("decode.hip", "latent_body.h"):
        h.update(open(os.path.join(ROOT, "head_latent_attention_fwd_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def decode_traffic(form):
    """HBM bytes per launch of the decode attention kernel (read + write)
    from the committed rocprofv3 counter summary of that workload, or None
    when the decode kernels' sources changed since the counters were taken."""
    import re
    name = {"full": "decode_fullcache_B64_P1000_hbm_traffic.md",
            "latent": "decode_latentcache_B32_P8192_hbm_traffic.md"}[form]
    kern = {"full": "decode_full", "latent": "decode_latent"}[form]
    try:
        text = open(os.path.join(ROOT, "profiles", name)).read()
        sha = decode_source_hash()
    except OSError:
        return None
    m = re.search(rf"{kern} traffic_bytes_per_launch=(\d+) decode_source_sha256_16=([0-9a-f]+)", text)
    if not m or m.group(2) != sha:
        return None
    return int(m.group(1))


def achievable(torch, mla, dev, flush_buf):
    """Second denominators measured on this machine in the same run: the HBM read
    rate of the library's streaming-read yardstick over 1 GiB (four times the
    256 MB Infinity Cache; 16-byte loads, sixteen in flight per thread) and the
    bf16 dense rate of the vendor GEMM (hipBLASLt through torch.matmul) on an
    8192^3 product, each after the same clock warm-up as the workloads.  For
    reference, torch's own 1 GiB sum is timed too."""
    st = torch.cuda.current_stream()

    def rate(fn, reps):
        warm(torch, fn, 3)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(st)
        for _ in range(reps):
            fn()
        b.record(st)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e-3 / reps

    nbytes = flush_buf.numel() * flush_buf.element_size()
    sink = torch.empty(4096, dtype=torch.int32, device=dev)
    t_rd = rate(lambda: mla.mla_read_sweep(flush_buf, sink), 20)
    t_sum = rate(lambda: flush_buf.sum(), 20)
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    n = 8192
    a = torch.randn(n, n, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    b = torch.randn(n, n, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    c = torch.empty(n, n, device=dev, dtype=torch.bfloat16)
    t_mm = rate(lambda: torch.matmul(a, b, out=c), 20)
    del a, b, c
    return {"hbm_read_gbs": nbytes / t_rd / 1e9,
            "mfma_bf16_tflops": 2.0 * n ** 3 / t_mm / 1e12,
            "torch_sum_read_gbs": nbytes / t_sum / 1e9,
            "method": "HBM: mla_read_sweep over 1 GiB on the device (16-byte loads, 4096 workgroups), "
                      "20 reps; MFMA: hipBLASLt bf16 8192 x 8192 x 8192 product via torch.matmul, "
                      "20 reps; both after >= 0.25 s of warm-up, timed with HIP events"}


def make_weights(torch, dev, k, seed):
    """Synthetic N(0, 0.02^2) weights with unit gains, drawn on the device."""
    import head_latent_attention_fwd_amd as mla
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    d = mla.make_dims(k["d_model"], k["n_heads"], k["q_lora_rank"], k["kv_lora_rank"],
                      k["qk_nope_dim"], k["qk_rope_dim"], k["v_head_dim"], d_ff=k["d_ff"],
                      dtype="bf16")
    w = {}
    for name, shape in mla.weight_shapes(d).items():
        if name.startswith("g_"):
            w[name] = torch.ones(shape, dtype=torch.bfloat16, device=dev)
        else:
            w[name] = (torch.randn(shape, generator=g, device=dev, dtype=torch.float32) * 0.02).to(torch.bfloat16)
    return d, w, g


def normal_bf16(torch, shape, g, dev):
    """N(0,1) values drawn directly in bf16 on the device (no float32 copy of
    a multi-GB cache)."""
    return torch.empty(shape, dtype=torch.bfloat16, device=dev).normal_(0.0, 1.0, generator=g)


def warm(torch, fn, warmup, min_s=WARM_S):
    """Untimed warm-up: `warmup` calls, continued until the GPU has run the
    workload for at least `min_s` seconds.  The MI355X clocks settle about
    20 ms into a sustained run (a prefill step measured 670 us in the first
    batch and 543 us from the second batch on); a few-step warm-up would time
    that ramp instead of the steady state."""
    t0 = time.perf_counter()
    n = 0
    while n < warmup or time.perf_counter() - t0 < min_s:
        fn()
        n += 1
        if n % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def timed(torch, fn, steps, warmup, flush=None, samples=None):
    """Warm up, then time `steps` calls with HIP events on the current stream
    (per-step events when a cache flush runs between steps; their times are
    appended to `samples` when a list is given)."""
    if warmup > 0:
        warm(torch, fn, warmup)
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    if flush is None:
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        a.record(st)
        for _ in range(steps):
            fn()
        b.record(st)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return a.elapsed_time(b) / steps, wall
    tot = 0.0
    t0 = time.perf_counter()
    for _ in range(steps):
        flush()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(st)
        fn()
        b.record(st)
        torch.cuda.synchronize()
        e = a.elapsed_time(b)
        tot += e
        if samples is not None:
            samples.append(e)
    return tot / steps, time.perf_counter() - t0


def timed_profiled(torch, mla, fn, steps, flush=None, samples=None):
    """Time `steps` steps as they run (no per-kernel events), then time them
    again with the library's per-launch HIP events on the launch stream for
    the kernel table.  Returns (ms_per_step, wall_s, kernel_table,
    ms_per_step_with_events); with a flush, the first pass's per-step times
    go to `samples`."""
    ms, wall = timed(torch, fn, steps, 0, flush, samples)
    mla.mla_profile_summary()                  # drop anything recorded so far
    mla.mla_profile_enable(True)
    ms_ev, _ = timed(torch, fn, steps, 0, flush)
    mla.mla_profile_enable(False)
    return ms, wall, kernel_table(mla, steps), ms_ev


def per_step_stats(torch, fn, steps):
    """Median and minimum of `steps` steps, each bracketed by its own pair of
    HIP events on the current stream (a pass of its own, after the timed one)."""
    st = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in ev:
        a.record(st)
        fn()
        b.record(st)
    torch.cuda.synchronize()
    v = sorted(a.elapsed_time(b) for a, b in ev)
    return v[len(v) // 2], v[0]


def kernel_table(mla, steps):
    prof = mla.mla_profile_summary()
    return {n: {"launches": c, "avg_ms": ms / c} for n, (c, ms) in prof.items()}


def bench_prefill(torch, mla, dev, steps, warmup, k=KIMI, B=1, T=2048):
    d, w, g = make_weights(torch, dev, k, 1002)
    x = torch.randn(B, T, k["d_model"], generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    rope = mla.mla_rope_table(T, k["qk_rope_dim"], 10000.0, dev)
    out = torch.empty_like(x)
    ws = torch.empty(mla.prefill_workspace_size(d, B, T), dtype=torch.uint8, device=dev)
    fn = lambda: mla.mla_prefill(d, w, x, rope, out=out, workspace=ws)  # noqa: E731
    warm(torch, fn, warmup)
    ms, wall, kern, ms_ev = timed_profiled(torch, mla, fn, steps)
    med, mn = per_step_stats(torch, fn, steps)
    flops = prefill_kernel_flops(B, T, k)
    for n, v in kern.items():
        if n in flops:
            v["gflop"] = flops[n] / 1e9
            v["tflops"] = flops[n] / (v["avg_ms"] * 1e-3) / 1e12
    total = sum(v for n, v in flops.items() if n != "gemm_qkv_up")
    return {"ms": ms, "ms_with_kernel_events": ms_ev, "ms_median": med, "ms_min": mn, "wall_s": wall,
            "flops": total, "kernels": kern, "w": w, "d": d}


def bench_prefill_bias(torch, mla, dev, d, w, steps, warmup, k=KIMI, B=1, T=2048):
    """The headline prefill in the attention_bias variant: biases on the two
    down-projections and on o_proj, added in the kernels' epilogues.  The
    FLOP count is the headline's (the bias adds are not counted)."""
    g = torch.Generator(device=dev)
    g.manual_seed(1007)
    wb = dict(w)
    for n, shp in mla.bias_shapes(d).items():
        wb[n] = (torch.randn(shp, generator=g, device=dev, dtype=torch.float32) * 0.02).to(torch.bfloat16)
    x = torch.randn(B, T, k["d_model"], generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    rope = mla.mla_rope_table(T, k["qk_rope_dim"], 10000.0, dev)
    out = torch.empty_like(x)
    ws = torch.empty(mla.prefill_workspace_size(d, B, T), dtype=torch.uint8, device=dev)
    fn = lambda: mla.mla_prefill(d, wb, x, rope, out=out, workspace=ws)  # noqa: E731
    warm(torch, fn, warmup)
    ms, _, kern, ms_ev = timed_profiled(torch, mla, fn, steps)
    flops = sum(v for n, v in prefill_kernel_flops(B, T, k).items() if n != "gemm_qkv_up")
    return {"workload": f"Kimi K2 MLA prefill with attention_bias (q_a, kv_a and o_proj biases), bf16, B={B}, T={T}",
            "ms_per_step": ms, "ms_per_step_with_kernel_events": ms_ev,
            "tflops": flops / (ms * 1e-3) / 1e12, "kernels": kern}


def decode_extras(torch, fn, steps, samples, B):
    """Per-step statistics of the flushed steps, and the same step timed back
    to back with the Infinity Cache left as the previous step leaves it
    (labelled un-flushed: weights and part of the cache may hit in it)."""
    ex = {}
    if samples:
        v = sorted(samples)
        ex["ms_per_step_median"] = v[len(v) // 2]
        ex["ms_per_step_min"] = v[0]
    ms_warm, _ = timed(torch, fn, steps, 0)
    ex["ms_per_step_unflushed"] = ms_warm
    ex["tokens_per_s_unflushed"] = B / (ms_warm * 1e-3)
    return ex


def bench_decode_full(torch, mla, dev, d, w, steps, warmup, flush, B=64, P=1000):
    k = KIMI
    L_cap = P + 1
    g = torch.Generator(device=dev)
    g.manual_seed(1003)
    H = k["n_heads"]
    kc = normal_bf16(torch, (B, H, L_cap, 192), g, dev)
    vc = normal_bf16(torch, (B, H, L_cap, 128), g, dev)
    x = torch.randn(B, k["d_model"], generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    rope = mla.mla_rope_table(L_cap, 64, 10000.0, dev)
    out = torch.empty_like(x)
    ws = torch.empty(mla.decode_workspace_size(d, B, L_cap), dtype=torch.uint8, device=dev)
    fn = lambda: mla.mla_decode_fullcache(d, w, x, P, kc, vc, rope, out=out, workspace=ws)  # noqa: E731
    warm(torch, fn, warmup)
    samples = []
    ms, _, kern, ms_ev = timed_profiled(torch, mla, fn, steps, flush, samples)
    extras = decode_extras(torch, fn, steps, samples, B)
    L = P + 1
    cache_bytes = B * H * L * (192 + 128) * 2
    nbytes = cache_bytes + mla_param_count() * 2 + B * H * 320 * 2 + 2 * B * k["d_model"] * 2
    if "decode_full" in kern:
        kern["decode_full"]["gbs"] = cache_bytes / (kern["decode_full"]["avg_ms"] * 1e-3) / 1e9
        kern["decode_full"]["algorithmic_bytes"] = cache_bytes
        if (B, P) == (64, 1000):
            kern["decode_full"]["traffic"] = decode_traffic("full")
    del kc, vc
    return {"workload": f"MLA decode, full cache, bf16, B={B}, P={P} (L={L} keys)",
            "ms_per_step": ms, "ms_per_step_with_kernel_events": ms_ev, "tokens_per_s": B / (ms * 1e-3),
            "hbm_gbs": nbytes / (ms * 1e-3) / 1e9, "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "algorithmic_bytes": nbytes, "kernels": kern, "mall_flushed": flush is not None, **extras}


def bench_decode_latent(torch, mla, dev, d, w, steps, warmup, flush, B=32, P=8192, persistent=False):
    """Latent-cache decode step; persistent=True times the same step run as
    one cooperative kernel (mla_decode_latentcache_persistent)."""
    k = KIMI
    L_cap = P + 1
    g = torch.Generator(device=dev)
    g.manual_seed(1004)
    cc = normal_bf16(torch, (B, L_cap, 576), g, dev)
    x = torch.randn(B, k["d_model"], generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    rope = mla.mla_rope_table(L_cap, 64, 10000.0, dev)
    out = torch.empty_like(x)
    ws = torch.empty(mla.decode_workspace_size(d, B, L_cap), dtype=torch.uint8, device=dev)
    step = mla.mla_decode_latentcache_persistent if persistent else mla.mla_decode_latentcache
    fn = lambda: step(d, w, x, P, cc, rope, out=out, workspace=ws)  # noqa: E731
    warm(torch, fn, warmup)
    samples = []
    ms, _, kern, ms_ev = timed_profiled(torch, mla, fn, steps, flush, samples)
    extras = decode_extras(torch, fn, steps, samples, B)
    L = P + 1
    cache_bytes = B * L * 576 * 2
    nbytes = cache_bytes + mla_param_count() * 2 + B * 576 * 2 + 2 * B * k["d_model"] * 2
    if "decode_latent" in kern:
        kern["decode_latent"]["gbs"] = cache_bytes / (kern["decode_latent"]["avg_ms"] * 1e-3) / 1e9
        kern["decode_latent"]["algorithmic_bytes"] = cache_bytes
        if (B, P) == (32, 8192):
            kern["decode_latent"]["traffic"] = decode_traffic("latent")
    form = ", one persistent cooperative kernel" if persistent else ""
    return {"workload": f"MLA decode, absorbed latent cache, bf16, B={B}, P={P} (L={L} keys){form}",
            "ms_per_step": ms, "ms_per_step_with_kernel_events": ms_ev, "tokens_per_s": B / (ms * 1e-3),
            "hbm_gbs": nbytes / (ms * 1e-3) / 1e9, "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "algorithmic_bytes": nbytes, "kernels": kern, "mall_flushed": flush is not None, **extras}


def bench_decode_latent_ragged(torch, mla, dev, d, w, steps, warmup, flush, B=32, P_max=8192):
    """Absorbed latent decode over a ragged batch: per-sequence positions drawn
    uniformly from [0, P_max] (seeded), one decode step per call."""
    k = KIMI
    L_cap = P_max + 1
    g = torch.Generator(device=dev)
    g.manual_seed(1006)
    cc = torch.randn(B, L_cap, 576, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    x = torch.randn(B, k["d_model"], generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    import numpy as np
    pos_host = np.random.default_rng(1006).integers(0, P_max + 1, size=B)
    pos_host[0] = P_max
    pos = torch.tensor(pos_host, dtype=torch.int32, device=dev)
    rope = mla.mla_rope_table(L_cap, 64, 10000.0, dev)
    out = torch.empty_like(x)
    ws = torch.empty(mla.decode_workspace_size(d, B, L_cap), dtype=torch.uint8, device=dev)
    fn = lambda: mla.mla_decode_latentcache_ragged(d, w, x, pos, P_max, cc, rope, out=out, workspace=ws)  # noqa: E731
    warm(torch, fn, warmup)
    samples = []
    ms, _, kern, ms_ev = timed_profiled(torch, mla, fn, steps, flush, samples)
    extras = decode_extras(torch, fn, steps, samples, B)
    keys = int(pos_host.sum()) + B
    cache_bytes = keys * 576 * 2
    nbytes = cache_bytes + mla_param_count() * 2 + B * 576 * 2 + 2 * B * k["d_model"] * 2
    if "decode_latent" in kern:
        kern["decode_latent"]["gbs"] = cache_bytes / (kern["decode_latent"]["avg_ms"] * 1e-3) / 1e9
    return {"workload": f"MLA decode, absorbed latent cache, ragged batch, bf16, B={B}, positions uniform "
                        f"in [0, {P_max}] (mean {pos_host.mean():.0f}, {keys} keys in all)",
            "ms_per_step": ms, "ms_per_step_with_kernel_events": ms_ev, "tokens_per_s": B / (ms * 1e-3),
            "hbm_gbs": nbytes / (ms * 1e-3) / 1e9, "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "algorithmic_bytes": nbytes, "kernels": kern, "mall_flushed": flush is not None, **extras}


SWEEP_P = (1000, 4096, 8192, 16384)
SWEEP_B = (32, 64)


def bench_decode_sweep(torch, mla, dev, d, w, steps, warmup, flush):
    """Decode steps over the number of cached positions P (the decode mode's
    P of "Kimi K2 · Mix and project", 1,000 there) for both cache forms at
    B = 32 and 64: time per step, tokens/s and algorithmic HBM GB/s."""
    rows = []
    for form, fn in (("full", bench_decode_full), ("latent", bench_decode_latent)):
        for B in SWEEP_B:
            for P in SWEEP_P:
                log(f"[bench] decode sweep {form} B={B} P={P}")
                r = fn(torch, mla, dev, d, w, steps, warmup, flush, B=B, P=P)
                kname = "decode_full" if form == "full" else "decode_latent"
                rows.append({"form": form, "B": B, "P": P, "ms_per_step": r["ms_per_step"],
                             "tokens_per_s": r["tokens_per_s"], "hbm_gbs": r["hbm_gbs"],
                             "hbm_frac": r["hbm_frac"], "ms_per_step_median": r.get("ms_per_step_median"),
                             "ms_per_step_unflushed": r.get("ms_per_step_unflushed"),
                             "attention_kernel_gbs": r["kernels"].get(kname, {}).get("gbs")})
                torch.cuda.empty_cache()
    return {"workload": "MLA decode step over P in " + str(list(SWEEP_P)) + ", B in " + str(list(SWEEP_B)) +
                        ", both cache forms, bf16, Infinity Cache flushed before each step "
                        "(ms_per_step_unflushed: the same step back to back)",
            "points": rows}


def chunk_flops(B, T, P0, k=KIMI):
    """Algorithmic FLOPs of a chunked-prefill step: the projections of the T
    new tokens and causal attention of token t over P0 + t + 1 keys."""
    H = k["n_heads"]
    dqk = k["qk_nope_dim"] + k["qk_rope_dim"]
    proj = 2.0 * B * T * (mla_param_count(k) - k["q_lora_rank"] - k["kv_lora_rank"])
    keys = T * P0 + T * (T + 1) / 2
    return proj + 2.0 * B * H * keys * (dqk + k["v_head_dim"])


def bench_prefill_chunk(torch, mla, dev, d, w, steps, warmup, form, B=1, T=512, P0=3584):
    """Chunked prefill: T new tokens at positions P0 .. P0+T-1 against a cache
    of P0 positions (N(0,1) history), full or latent cache form."""
    k = KIMI
    L_cap = P0 + T
    g = torch.Generator(device=dev)
    g.manual_seed(1007)
    H = k["n_heads"]
    x = torch.randn(B, T, k["d_model"], generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    rope = mla.mla_rope_table(L_cap, 64, 10000.0, dev)
    out = torch.empty_like(x)
    ws = torch.empty(mla.chunk_workspace_size(d, B, T, L_cap), dtype=torch.uint8, device=dev)
    if form == "full":
        kc = torch.randn(B, H, L_cap, 192, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
        vc = torch.randn(B, H, L_cap, 128, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
        fn = lambda: mla.mla_prefill_chunk_fullcache(d, w, x, P0, kc, vc, rope, out=out, workspace=ws)  # noqa: E731
    else:
        cc = torch.randn(B, L_cap, 576, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
        fn = lambda: mla.mla_prefill_chunk_latentcache(d, w, x, P0, cc, rope, out=out, workspace=ws)  # noqa: E731
    warm(torch, fn, warmup)
    ms, _, kern, ms_ev = timed_profiled(torch, mla, fn, steps)
    flops = chunk_flops(B, T, P0)
    return {"workload": f"chunked prefill, {form} cache, bf16, B={B}, {T} new tokens at positions "
                        f"{P0}..{P0 + T - 1}",
            "ms_per_step": ms, "ms_per_step_with_kernel_events": ms_ev,
            "tflops": flops / (ms * 1e-3) / 1e12, "mfma_frac": flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFS,
            "gflop": flops / 1e9, "kernels": kern}


def bench_block(torch, mla, dev, d, w, steps, warmup, B=1, T=4096):
    k = KIMI
    g = torch.Generator(device=dev)
    g.manual_seed(1005)
    F, D = k["d_ff"], k["d_model"]
    blk = {"g_attn": torch.ones(D, dtype=torch.bfloat16, device=dev),
           "g_ffn": torch.ones(D, dtype=torch.bfloat16, device=dev)}
    for n, shp in (("w1", (F, D)), ("w3", (F, D)), ("w2", (D, F))):
        blk[n] = (torch.randn(shp, generator=g, device=dev, dtype=torch.float32) * 0.02).to(torch.bfloat16)
    x = torch.randn(B, T, D, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    rope = mla.mla_rope_table(T, 64, 10000.0, dev)
    out = torch.empty_like(x)
    ws = torch.empty(mla.block_workspace_size(d, B, T), dtype=torch.uint8, device=dev)
    fn = lambda: mla.dense_block_fwd(d, w, blk, x, rope, out=out, workspace=ws)  # noqa: E731
    warm(torch, fn, warmup)
    ms, _, kern, ms_ev = timed_profiled(torch, mla, fn, steps)
    fl = prefill_kernel_flops(B, T)
    flops = sum(v for n, v in fl.items() if n != "gemm_qkv_up") + 2.0 * B * T * D * F * 3
    fl["gemm_swiglu"] = 2.0 * B * T * D * F * 2
    fl["gemm_w2_resid"] = 2.0 * B * T * D * F
    for n, v in kern.items():
        if n in fl:
            v["tflops"] = fl[n] / (v["avg_ms"] * 1e-3) / 1e12
    return {"workload": f"dense block (RMSNorm, MLA, residual, RMSNorm, SwiGLU 18432, residual), bf16, B={B}, T={T}",
            "ms_per_step": ms, "ms_per_step_with_kernel_events": ms_ev, "tflops": flops / (ms * 1e-3) / 1e12,
            "mfma_frac": flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFS, "gflop": flops / 1e9,
            "kernels": kern}


def cpu_baseline(k=KIMI, B=1, T=2048):
    """The float32 oracle on the host cores, on the headline workload."""
    import numpy as np
    from oracle import mla_ref as ref
    from tests import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 0) for i in threadpool_info()] or [os.cpu_count() or 1])
    except Exception:  # threadpoolctl missing: report the visible cores
        threads = os.cpu_count() or 1
    dims = ref.KIMI_K2
    x, w = synth.prefill_inputs(dims, B, T, 1002, bf16=True)
    mw = ref.MLAWeights(**w)
    n = 0
    t0 = time.perf_counter()
    while n == 0 or time.perf_counter() - t0 < CPU_SAMPLE_S:
        ref.mla_prefill(dims, mw, x, dtype=np.float32)
        n += 1
    dt = (time.perf_counter() - t0) / n
    flops = sum(v for n, v in prefill_kernel_flops(B, T, k).items() if n != "gemm_qkv_up")
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "seconds_per_step": dt, "steps": n,
            "sample": f"{n} whole steps of the headline workload (B={B}, T={T}) by the NumPy oracle "
                      f"in float32, repeated for at least {CPU_SAMPLE_S:.0f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--only", choices=["prefill", "decode_full", "decode_latent", "decode_latent_persistent",
                                       "decode_latent_ragged",
                                       "prefill_bias", "chunk_full", "chunk_latent", "block", "decode_sweep",
                                       "copy"])
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    import head_latent_attention_fwd_amd as mla
    mla.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    flush_buf = torch.ones(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB, written once

    def flush():
        # A 1 GiB read sweep evicts the 256 MB Infinity Cache with clean lines,
        # as the weight reads before an attention call would.  A write sweep
        # would leave ~256 MB of dirty lines whose write-back the next kernel
        # pays for (measured: +55 us on a 302 MB read).
        flush_buf.sum()

    if args.only == "copy":
        # calibration for HBM byte counters: a plain device copy of known size
        n = 1 << 28                                 # 256 Mi bf16 = 512 MiB each way
        src = torch.empty(n, dtype=torch.bfloat16, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_each_way": n * 2, "launches": args.steps}))
        return
    if args.only and args.only != "prefill":
        d, w, _ = make_weights(torch, dev, KIMI, 1002)
        fn = {"decode_full": lambda: bench_decode_full(torch, mla, dev, d, w, args.steps, args.warmup, flush),
              "decode_latent": lambda: bench_decode_latent(torch, mla, dev, d, w, args.steps, args.warmup, flush),
              "decode_latent_persistent": lambda: bench_decode_latent(torch, mla, dev, d, w, args.steps, args.warmup,
                                                                      flush, persistent=True),
              "decode_latent_ragged": lambda: bench_decode_latent_ragged(torch, mla, dev, d, w, args.steps,
                                                                         args.warmup, flush),
              "prefill_bias": lambda: bench_prefill_bias(torch, mla, dev, d, w, args.steps, args.warmup),
              "chunk_full": lambda: bench_prefill_chunk(torch, mla, dev, d, w, args.steps, args.warmup, "full"),
              "chunk_latent": lambda: bench_prefill_chunk(torch, mla, dev, d, w, args.steps, args.warmup, "latent"),
              "block": lambda: bench_block(torch, mla, dev, d, w, args.steps, args.warmup),
              "decode_sweep": lambda: bench_decode_sweep(torch, mla, dev, d, w, args.steps, args.warmup,
                                                         flush)}[args.only]
        print(json.dumps(fn()))
        return

    log(f"[bench] prefill B=1 T=2048 steps={args.steps} warmup={args.warmup}")
    r = bench_prefill(torch, mla, dev, args.steps, args.warmup)
    kern = r["kernels"]
    gemmlike = {n: v for n, v in kern.items() if "tflops" in v}
    dom = max(gemmlike, key=lambda n: gemmlike[n]["avg_ms"])
    dv = gemmlike[dom]
    roofline = {"kernel": dom, "bound": "mfma", "achieved": dv["tflops"], "peak": MFMA_BF16_PEAK_TFS,
                "unit": "TFLOP/s", "frac": dv["tflops"] / MFMA_BF16_PEAK_TFS,
                "traffic": measured_traffic(dom),
                "avg_ms": dv["avg_ms"], "gflop_per_launch": dv["gflop"]}
    value = r["flops"] / (r["ms"] * 1e-3) / 1e12
    line = {
        "metric": "MLA prefill TFLOP/s (% MFMA peak); decode tokens/s & HBM GB/s (% peak)",
        "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": r["ms"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (N(0,1) activations, N(0,0.02^2) weights, unit gains)",
        "config": {"workload": "Kimi K2-shaped MLA prefill, bf16 (fp32 softmax/accumulate), causal",
                   "global_batch": 1, "seq_len": 2048, "d_model": 7168, "heads": 64,
                   "q_lora": 1536, "kv_lora": 512, "qk_dims": "128 nope + 64 rope", "v_dim": 128,
                   "parallelism": "none (1 GPU)"},
        "mfma_frac_step": value / MFMA_BF16_PEAK_TFS,
        "roofline": roofline,
        "ms_per_step_with_kernel_events": r["ms_with_kernel_events"],
        "ms_per_step_median": r["ms_median"], "ms_per_step_min": r["ms_min"],
        "kernels": kern,
    }
    if not args.no_secondary:
        sec = {}
        for name, fn in (("decode_fullcache", lambda: bench_decode_full(torch, mla, dev, r["d"], r["w"], max(5, args.steps // 2), 3, flush)),
                         ("decode_latentcache", lambda: bench_decode_latent(torch, mla, dev, r["d"], r["w"], max(5, args.steps // 2), 3, flush)),
                         ("decode_latentcache_persistent", lambda: bench_decode_latent(torch, mla, dev, r["d"], r["w"], max(5, args.steps // 2), 3, flush, persistent=True)),
                         ("decode_latentcache_ragged", lambda: bench_decode_latent_ragged(torch, mla, dev, r["d"], r["w"], max(5, args.steps // 2), 3, flush)),
                         ("prefill_attention_bias", lambda: bench_prefill_bias(torch, mla, dev, r["d"], r["w"], max(5, args.steps // 2), 3)),
                         ("prefill_chunk_fullcache", lambda: bench_prefill_chunk(torch, mla, dev, r["d"], r["w"], max(5, args.steps // 2), 3, "full")),
                         ("prefill_chunk_latentcache", lambda: bench_prefill_chunk(torch, mla, dev, r["d"], r["w"], max(5, args.steps // 2), 3, "latent")),
                         ("dense_block", lambda: bench_block(torch, mla, dev, r["d"], r["w"], max(3, args.steps // 4), 2)),
                         ("decode_sweep", lambda: bench_decode_sweep(torch, mla, dev, r["d"], r["w"], 5, 2, flush))):
            log(f"[bench] {name}")
            try:
                sec[name] = fn()
            except Exception as e:  # a secondary failure must not hide the headline
                sec[name] = {"error": repr(e)}
            torch.cuda.empty_cache()
        line["secondary"] = sec
    log("[bench] achievable rates (measured yardsticks)")
    try:
        ach = achievable(torch, mla, dev, flush_buf)
    except Exception as e:  # a yardstick failure must not hide the headline
        ach = {"error": repr(e)}
    line["achievable"] = ach
    if "error" not in ach:
        roofline["frac_of_achievable"] = roofline["achieved"] / ach["mfma_bf16_tflops"]
        line["mfma_frac_step_of_achievable"] = value / ach["mfma_bf16_tflops"]
        for name, v in line.get("secondary", {}).items():
            if not isinstance(v, dict):
                continue
            if "hbm_gbs" in v:
                v["hbm_frac_of_achievable"] = v["hbm_gbs"] / ach["hbm_read_gbs"]
            if "tflops" in v:
                v["mfma_frac_of_achievable"] = v["tflops"] / ach["mfma_bf16_tflops"]
            for pt in v.get("points", []):
                if "hbm_gbs" in pt:
                    pt["hbm_frac_of_achievable"] = pt["hbm_gbs"] / ach["hbm_read_gbs"]
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle, float32)")
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line))


if __name__ == "__main__":
    main()
