"""Benchmark: steady decode steps of attention-scored KV eviction on one GPU.

Workload: Llama-3.1-8B-shaped attention (32 layers, 32 query heads over 8 KV
heads, head dim 128, bf16, batch 1), 32,768-token prefill, EMA alpha 0.05
folded layer by layer, budget 3,277 tokens per KV head with 4 sinks and 32
recent tokens protected.  One step = kvev_step: append + attention over all
layers (the whole-cache kernel: one workgroup per (KV head, layer), writing
the outputs and each slot's group mass), then layer fold + selection +
compaction.  W warm-up steps run outside the timed region; the first of
them (the step that evicts the prefill down to the budget, or the first
two-tier routing event) is timed on its own and reported as first_step_ms.
Then exactly K steps are timed between two device synchronisations; inputs
are resident in HBM before the timed region.

Prints one JSON line.  ``--gpus N`` with N > 1 exits: the path runs on one
GPU.  ``--workload qevict131k`` times the two-tier window path instead
(131,072-token prefill, 205 full-precision and 819 INT2 windows per layer),
``--workload lrfu64`` the block-LRFU path (64 sequences of 4k-16k tokens,
20% block budgets).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E
# Every PROF_EVERY-th timed step is profiled (the per-kernel averages and the
# roofline come from those launches).  The step's launches record their own
# dispatch start and end into HIP events (hipExtLaunchKernelGGL), so no event
# record runs between kernels; the vector attention of the fp32 / d = 64
# path and the move, select and diagnostics launches are bracketed by event
# records instead (each about 3.7 us of GPU time).  Sampling keeps the step
# time within about 0.5% of an unprofiled run on the 32k workload.
PROF_EVERY = 15  # coprime with the tiered routing interval 8, so routing steps are sampled too


def warm_up(ctx, inputs, out, warmup):
    """Run the warm-up steps; the first one (the step whose selection evicts
    the prefill down to the budget, or the first routing event) is timed on
    its own between two device synchronisations.  Returns its milliseconds."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ctx.step(*inputs[0], out)
    torch.cuda.synchronize()
    first_ms = (time.perf_counter() - t0) * 1e3
    for t in range(1, warmup):
        ctx.step(*inputs[t], out)
    return first_ms


def timed_steps(ctx, inputs, out, first, total, prof_every=None):
    """Run steps first..total-1 between two device synchronisations, with
    HIP-event profiling of every prof_every-th step (default PROF_EVERY).
    Returns (seconds, profiled steps)."""
    import torch
    prof_every = prof_every or PROF_EVERY
    ctx.sync()
    ctx.profile(False)
    ctx.profile_reset()
    torch.cuda.synchronize()
    n_prof = 0
    t0 = time.perf_counter()
    for i, t in enumerate(range(first, total)):
        sample = i % prof_every == 0
        if sample:
            ctx.profile(True)
            n_prof += 1
        ctx.step(*inputs[t], out)
        if sample:
            ctx.profile(False)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ctx.sync()
    return dt, n_prof


def algorithmic_bytes(w, n_tokens):
    """Bytes a steady step must move (per the workload's shapes).

    K/V of the retained cache read once in every layer, q read, fp32 output
    written, appended K/V written, utility read + written, and the K/V of
    one compaction move read + written in every layer, for every sequence
    of the batch.
    """
    L, Hkv, Hq, d, B = w.n_layers, w.n_kv_heads, w.n_q_heads, w.head_dim, w.batch
    el = 4 if w.dtype == "f32" else 2
    kv = B * L * Hkv * n_tokens * 2 * d * el
    q = B * L * Hq * d * el
    out = B * L * Hq * d * 4
    app = B * L * Hkv * 2 * d * el
    state = B * Hkv * n_tokens * 4 * 2
    move = B * L * Hkv * 2 * d * el * 2
    return kv, kv + q + out + app + state + move


CSRC = os.path.join(ROOT, "decode_kv_cache_gqa_amd", "csrc")
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "attn_mfma_kernel_traffic_llama8b_32k.md")
ATTN_SOURCES = [os.path.join(CSRC, f) for f in ("attn.hip", "common.h")]
SEQ_TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "attn_seq_kernel_traffic_llama8b_32k.md")
BLK_SEQ_TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "attn_seq_kernel_traffic_lrfu64.md")
TIER_TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "tier_attn_kernel_traffic_qevict131k.md")
TIER_SOURCES = [os.path.join(CSRC, f) for f in ("tier.hip", "common.h")]
SEQ_SOURCES = [os.path.join(CSRC, f) for f in ("attn_seq.hip", "common.h")]


def measured_traffic(profile=TRAFFIC_PROFILE, sources=ATTN_SOURCES):
    """HBM bytes per attention launch from a committed counter profile, or
    None when the kernel source changed after the counters were taken."""
    import hashlib
    try:
        text = open(profile).read()
    except OSError:
        return None
    vals = dict(line.split(": ", 1) for line in text.splitlines()
                if line.startswith(("traffic_bytes_per_launch: ", "kernel_source_sha256: ")))
    h = hashlib.sha256()
    for f in sources:
        h.update(open(f, "rb").read())
    if vals.get("kernel_source_sha256", "").strip() != h.hexdigest():
        return None
    return int(vals["traffic_bytes_per_launch"])


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _timed_two_ways(segment):
    """segment(k) runs and times the k-th timed segment (k = 0, 1) of an
    oracle sample and returns its seconds per scaled step.  Segment 0 runs
    with the BLAS pools limited to one thread, segment 1 with the default
    pools.  Returns (seconds all threads, seconds one thread, threads)."""
    from threadpoolctl import threadpool_info, threadpool_limits
    with threadpool_limits(limits=1):
        one = segment(0)
    cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return segment(1), one, cores


def _baseline_record(sec_all, sec_one, cores, sample):
    return {"value": 1.0 / sec_all, "unit": "steps/s", "cores": int(cores), "kind": "oracle",
            "value_1thread": 1.0 / sec_one, "cpu_model": _cpu_model(), "sample": sample}


def cpu_baseline(w, steps=150):
    """Time the CPU oracle on a bounded sample: steady steps of ONE selection
    group at the workload's real shape (all layers, budget+1 tokens), scaled
    to the whole step.  A group is one (sequence, KV head), or one sequence
    with all its KV heads in the per-sequence mode.  Two segments of `steps`
    steps: one with one BLAS thread, one with the default threads."""
    import oracle as orc
    B = w.budget
    pooled = w.granularity == "sequence"
    if pooled:
        steps = max(steps // w.n_kv_heads, 8)
    kw = dict(budget=B, alpha_new=w.alpha_new, n_sink=w.n_sink, n_recent=w.n_recent,
              capacity=B + 2 * steps + 2, scorer=w.scorer,
              policy="cumulative" if w.policy == "cumulative" else "ema",
              refresh_interval=w.refresh_interval, score_free=w.score_free)
    if pooled:
        o = orc.PooledTokenOracle(w.n_layers, w.n_q_heads, w.n_kv_heads, w.head_dim, **kw)
        K, V = w.scaled(prefill_lens=(B,)).prefill_kv(0)
        o.prefill(0, K.float().numpy(), V.float().numpy())
        groups = w.batch
    else:
        o = orc.TokenModeOracle(w.n_layers, w.n_q_heads, w.n_kv_heads, w.head_dim, **kw)
        K, V = w.scaled(prefill_lens=(B,)).prefill_kv(0, heads=[0])
        o.prefill(0, K.float().numpy(), V.float().numpy(), heads=[0])
        groups = w.n_kv_heads * w.batch
    ins = [w.step_inputs(t, seqs=[0]) for t in range(1, 2 * steps + 2)]
    ins = [tuple(x.float().numpy() for x in s) for s in ins]
    o.decode_step(1, *ins[0], [0])
    o.evict()

    def segment(k):
        t0 = time.perf_counter()
        for t in range(2 + k * steps, 2 + (k + 1) * steps):
            o.decode_step(t, *ins[t - 1], [0])
            o.evict()
        return (time.perf_counter() - t0) / steps * groups

    sec_all, sec_one, cores = _timed_two_ways(segment)
    unit = "sequence" if pooled else "(sequence, KV head)"
    return _baseline_record(sec_all, sec_one, cores,
                            f"2 x {steps} steady steps of 1 of {groups} {unit} groups at {w.n_layers} layers x "
                            f"{B + 1} tokens, scaled x{groups}")


def tier_bytes(w, n_fp_tokens, n_q):
    """Bytes of a steady tiered step: the full-precision tokens' K/V (512 B per
    token and KV head) and the INT2 windows in every layer, plus q, the fp32
    output, the appended token and the window scores read and written.  An
    INT2 window of the fused path (32-token windows, no rotation) is read as
    its 3,072-byte record (2-bit codes of 32 x 128 keys and values, fp16
    scale and zero per key channel and per value token-group); with 8-token
    windows or the rotary mode it is read as its bf16 reconstruction
    (512 B per token and KV head)."""
    L, Hkv, Hq, d = w.n_layers, w.n_kv_heads, w.n_q_heads, w.head_dim
    W = w.window_tokens
    q_win = W * 2 * d * 2 if (W == 8 or w.rope_theta > 0) else 3072
    kv = L * Hkv * (n_fp_tokens * 2 * d * 2 + n_q * q_win)
    extra = L * Hq * d * 2 + L * Hq * d * 4 + L * Hkv * 2 * d * 2 + L * (n_fp_tokens // W + n_q) * 4 * 2
    return kv, kv + extra


def tier_footprint_record(w, fp):
    """The context's window memory against the byte budget of the review's
    section 4.3 Eq.3, B_hist = K_f M_f + K_q M_q over all layers (M_f: a
    window's full-precision K/V, M_q: its INT2 record, per KV head)."""
    W, d = w.window_tokens, w.head_dim
    rec = 1152 if W == 8 else 3072
    lh = w.n_layers * w.n_kv_heads
    m_f, m_q = W * 2 * d * 2, rec
    return {"fp_pool_bytes": fp["fp_pool"], "record_pool_bytes": fp["record_pool"],
            "staging_bytes": fp["staging"], "fp_slots": fp["fp_slots"], "record_slots": fp["record_slots"],
            "eq3_b_hist_bytes": lh * (w.fp_windows * m_f + w.int2_windows * m_q),
            "all_full_precision_bytes": lh * (-(-(w.prefill_lens[0]) // W)) * m_f}


def tier_cpu_baseline(w, steps=3):
    """The CPU oracle on one layer of the tiered workload: the first routing
    event untimed, then two segments of `steps` steady steps (one BLAS
    thread, default threads), each scaled to all layers."""
    import oracle as orc
    o = orc.TieredOracle(w.n_layers, w.n_q_heads, w.n_kv_heads, w.head_dim, k_f=w.fp_windows,
                         k_q=w.int2_windows, window=w.window_tokens, n_sink=w.n_sink,
                         n_recent=w.n_recent, capacity=w.prefill_lens[0] + 2 * steps + 2,
                         route_interval=w.route_interval)
    K, V = w.prefill_kv(0, layers=[0])
    o.prefill(K.float().numpy(), V.float().numpy(), layers=[0])
    del K, V
    ins = [tuple(x[:1, 0].float().numpy() for x in w.step_inputs(t, seqs=[0])) for t in range(1, 2 * steps + 2)]
    o.decode_step(1, *ins[0])
    o.route()

    def segment(k):
        t0 = time.perf_counter()
        for t in range(2 + k * steps, 2 + (k + 1) * steps):
            o.decode_step(t, *ins[t - 1])
            if o.routes_after(t):
                o.route()
        return (time.perf_counter() - t0) / steps * w.n_layers

    sec_all, sec_one, cores = _timed_two_ways(segment)
    return _baseline_record(sec_all, sec_one, cores,
                            f"2 x {steps} steady steps of layer 0 of {w.n_layers} after the first routing event "
                            f"({w.prefill_lens[0]}-token prefill), scaled x{w.n_layers}")


def block_cpu_baseline(w, steps=20):
    """The CPU oracle on the median-length sequence of the block workload:
    its prefill and first eviction untimed, then two segments of `steps`
    steady steps (one BLAS thread, default threads), each scaled to every
    sequence."""
    import numpy as np
    import oracle as orc
    b = int(np.argsort(w.prefill_lens)[len(w.prefill_lens) // 2])
    o = orc.BlockLRFUOracle(w.n_layers, w.n_q_heads, w.n_kv_heads, w.head_dim, alpha_new=w.alpha_new,
                            beta=w.beta, half_lives=tuple(w.region_half_lives),
                            pinned_regions=tuple(w.pinned_regions), decode_region=w.decode_region,
                            capacity=w.prefill_lens[b] + 2 * steps + 2)
    K, V = w.prefill_kv(b)
    o.prefill(b, K.float().numpy(), V.float().numpy(), w.region_labels(b), w.block_budget(b))
    del K, V
    ins = [tuple(x.float().numpy() for x in w.step_inputs(t, seqs=[b])) for t in range(1, 2 * steps + 2)]
    o.decode_step(1, *ins[0], [b])
    o.evict(1, seqs=[b])

    def segment(k):
        t0 = time.perf_counter()
        for t in range(2 + k * steps, 2 + (k + 1) * steps):
            o.decode_step(t, *ins[t - 1], [b])
            o.evict(t, seqs=[b])
        return (time.perf_counter() - t0) / steps * w.batch

    sec_all, sec_one, cores = _timed_two_ways(segment)
    return _baseline_record(sec_all, sec_one, cores,
                            f"2 x {steps} steady steps of sequence {b} ({w.prefill_lens[b]}-token prefill, the "
                            f"median) of {w.batch} after its first eviction, scaled x{w.batch}")


def run_block(args, w):
    """Steady kvev_step calls of the block-LRFU workload (all sequences each
    step; the epochs' re-admissions are not part of the timed steps)."""
    import numpy as np
    import torch
    from decode_kv_cache_gqa_amd import kvev

    total = args.warmup + args.steps
    ctx = kvev.context_for(w, max_steps=total)
    for b in range(w.batch):
        K, V = w.prefill_kv(b, device="cuda")
        ctx.prefill(b, K.contiguous(), V.contiguous(), w.region_labels(b))
        ctx.set_budget(b, w.block_budget(b))
        del K, V
    inputs = [w.step_inputs(t, device="cuda") for t in range(1, total + 1)]
    out = torch.empty((w.n_layers, w.batch, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    first_ms = warm_up(ctx, inputs, out, args.warmup)
    dt, n_prof = timed_steps(ctx, inputs, out, args.warmup, total, args.prof_every)
    names = ("open", "attn", "attn_whole", "merge", "mass", "policy", "offload")
    prof = {k: ctx.profile_read(k) for k in names}
    # "attn_whole": the whole-cache kernel over the block tables (its steps
    # need no merge), "attn": the split kernel
    whole = prof["attn_whole"][1] > 0
    assert not (whole and prof["attn"][1] > 0), "both attention kernels ran in the timed steps"
    # resident tokens read by a steady step: every resident block is full
    # except the sequence's last one (the new token's)
    n_tok = 0
    for b in range(w.batch):
        _, _, res = ctx.block_state(b)
        npos = w.prefill_lens[b] + total
        n_tok += int(res.sum()) * 16 - (-npos % 16)
    ctx.close()
    L, Hkv, Hq, d = w.n_layers, w.n_kv_heads, w.n_q_heads, w.head_dim
    kv_bytes = L * Hkv * n_tok * 2 * d * 2
    step_bytes = kv_bytes + w.batch * (L * Hq * d * 2 + L * Hq * d * 4 + L * Hkv * 2 * d * 2)
    ms_step = dt * 1e3 / args.steps
    attn_ms, attn_n = prof["attn_whole" if whole else "attn"]
    attn_avg_s = attn_ms / max(attn_n, 1) / 1e3
    attn_gbps = kv_bytes / attn_avg_s / 1e9 if attn_avg_s > 0 else None
    policy_ms = sum(prof[k][0] for k in ("merge", "mass", "policy", "offload")) / n_prof
    result = {
        "metric": "decode steps/s + KV-read GB/s (% HBM peak), incl. EMA/top-k/compaction",
        "value": round(args.steps / dt, 2), "unit": "steps/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded generator: region labels, shared heavy blocks re-targeted per epoch)",
        "config": {"workload": w.name, "layers": L, "q_heads": Hq, "kv_heads": Hkv, "head_dim": d,
                   "batch": w.batch, "prefill": [min(w.prefill_lens), max(w.prefill_lens)],
                   "block_budget_frac": w.budget_frac, "alpha_new": w.alpha_new, "beta": w.beta,
                   "offload_blocks": w.offload_blocks},
        "resident_tokens": n_tok,
        "kv_read_GBps": round(step_bytes / (dt / args.steps) / 1e9, 1),
        "pct_hbm_peak": round(100.0 * step_bytes / (dt / args.steps) / 1e9 / HBM_PEAK_GBPS, 2),
        "score_topk_compaction_share": round(policy_ms / ms_step, 4) if ms_step > 0 else None,
        "kernel_avg_us": {k: round(v[0] / max(v[1], 1) * 1e3, 3) for k, v in prof.items() if v[1]},
        "profiled_steps": n_prof,
        "first_step_ms": round(first_ms, 3),
        "roofline": {
            "bound": "hbm", "achieved": round(attn_gbps, 1) if attn_gbps else None, "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": round(attn_gbps / HBM_PEAK_GBPS, 4) if attn_gbps else None,
            # counters taken on the 64-sequence workload's whole-cache launch
            "traffic": (measured_traffic(BLK_SEQ_TRAFFIC_PROFILE, SEQ_SOURCES)
                        if whole and args.workload == "lrfu64" else None),
            "kernel": "attn_seq_kernel" if whole else "attn_mfma_kernel",
            "algorithmic_bytes_per_launch": kv_bytes,
        },
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = block_cpu_baseline(w)
    print(json.dumps(result))


def run_tier(args, w):
    import numpy as np
    import torch
    from decode_kv_cache_gqa_amd import kvev

    if args.warmup < max(w.route_interval, 1) + 1:
        # the steps before the first routing event attend every prefill window in full precision,
        # and the step after it releases the prefill staging buffers
        print(f"warmup raised to the routing interval + 1 ({w.route_interval + 1}) so that the timed "
              "steps are steady", file=sys.stderr)
        args.warmup = max(w.route_interval, 1) + 1
    total = args.warmup + args.steps
    ctx = kvev.context_for(w, max_steps=total)
    K, V = w.prefill_kv(0, device="cuda")
    ctx.prefill(0, K, V)
    del K, V
    inputs = [w.step_inputs(t, device="cuda") for t in range(1, total + 1)]
    out = torch.empty((w.n_layers, 1, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    first_ms = warm_up(ctx, inputs, out, args.warmup)
    dt, n_prof = timed_steps(ctx, inputs, out, args.warmup, total, args.prof_every)
    prof = {k: ctx.profile_read(k) for k in ("rope", "append", "attn", "merge", "mass", "route", "xfer")}
    _, tiers, _ = ctx.tier_state(0)
    fp = ctx.tier_footprint()
    npos = w.prefill_lens[0] + total
    ctx.close()
    n_fp_win = int((tiers == 0).sum())
    n_q = int((tiers == 1).sum())
    W = w.window_tokens
    n_fp_tokens = n_fp_win * W - (-npos % W)
    kv_bytes, step_bytes = tier_bytes(w, n_fp_tokens, n_q)
    ms_step = dt * 1e3 / args.steps
    attn_ms, attn_n = prof["attn"]
    attn_avg_s = attn_ms / max(attn_n, 1) / 1e3
    attn_gbps = kv_bytes / attn_avg_s / 1e9 if attn_avg_s > 0 else None
    policy_ms = sum(prof[k][0] for k in ("merge", "mass", "route", "xfer")) / n_prof
    result = {
        "metric": "decode steps/s + KV-read GB/s (% HBM peak), incl. EMA/top-k/compaction",
        "value": round(args.steps / dt, 2), "unit": "steps/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded outlier-channel / heavy-key generator, heavy keys re-targeted every 32 steps)",
        "config": {"workload": w.name, "layers": w.n_layers, "q_heads": w.n_q_heads, "kv_heads": w.n_kv_heads,
                   "head_dim": w.head_dim, "batch": 1, "prefill": w.prefill_lens[0], "window": w.window_tokens,
                   "fp_windows": w.fp_windows, "int2_windows": w.int2_windows, "n_sink": w.n_sink,
                   "n_recent": w.n_recent},
        "listed_windows": {"full_precision": n_fp_win, "int2": n_q},
        "device_footprint": tier_footprint_record(w, fp),
        "kv_read_GBps": round(step_bytes / (dt / args.steps) / 1e9, 1),
        "pct_hbm_peak": round(100.0 * step_bytes / (dt / args.steps) / 1e9 / HBM_PEAK_GBPS, 2),
        "score_topk_compaction_share": round(policy_ms / ms_step, 4) if ms_step > 0 else None,
        "kernel_avg_us": {k: round(v[0] / max(v[1], 1) * 1e3, 3) for k, v in prof.items() if v[1]},
        "profiled_steps": n_prof,
        "first_step_ms": round(first_ms, 3),
        "roofline": {
            "bound": "hbm", "achieved": round(attn_gbps, 1) if attn_gbps else None, "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": round(attn_gbps / HBM_PEAK_GBPS, 4) if attn_gbps else None,
            "traffic": (measured_traffic(TIER_TRAFFIC_PROFILE, TIER_SOURCES)
                        if args.workload == "qevict131k" else None), "kernel": "tier_attn_kernel",
            "algorithmic_bytes_per_launch": kv_bytes,
        },
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = tier_cpu_baseline(w)
    print(json.dumps(result))


def calibrate_stream(n_bytes=2 << 30, reps=10):
    """The HBM streaming-read ceiling: kvev_calibrate_read over a 2 GiB
    buffer (8x the last-level cache), plain and non-temporal loads, 2-16
    workgroups of 256 threads per compute unit, each configuration timed
    over `reps` launches with events on torch's stream."""
    import torch
    from decode_kv_cache_gqa_amd import kvev
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    buf = torch.ones(n_bytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(16 * cus, dtype=torch.int32, device="cuda")
    rows = []
    for nt in (0, 1):
        for bpc in (2, 4, 8, 16):
            blocks = bpc * cus
            for _ in range(2):
                kvev.calibrate_read(buf, nt, blocks, sink)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                kvev.calibrate_read(buf, nt, blocks, sink)
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1000.0 / reps
            rows.append({"nontemporal": nt, "blocks_per_cu": bpc, "us": round(us, 2),
                         "TBps": round(n_bytes / us / 1e6, 3)})
    best = max(rows, key=lambda r: r["TBps"])
    print(json.dumps({"calibration": "stream_read", "bytes": n_bytes, "cus": cus, "reps": reps,
                      "results": rows, "best": best}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", default="llama8b_32k")
    ap.add_argument("--prof-every", type=int, default=PROF_EVERY,
                    help="profile every N-th timed step (HIP events around its launches)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 256 MiB device-to-device copy (counter calibration)")
    ap.add_argument("--calibrate-stream", action="store_true",
                    help="only time the library's streaming read of a 2 GiB buffer (the HBM read ceiling)")
    args = ap.parse_args()
    args.warmup = max(args.warmup, 1)  # the first step is timed on its own inside the warm-up
    if args.gpus != 1:
        print(f"bench.py: this path runs on one GPU; --gpus {args.gpus} is not supported",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from decode_kv_cache_gqa_amd import kvev, synth

    if args.calibrate_copy:
        n = 256 << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "copy", "bytes_read": n, "bytes_written": n, "launches": 4}))
        return

    if args.calibrate_stream:
        return calibrate_stream()

    w = synth.workload(args.workload)
    if w.policy == "tiered_int2":
        return run_tier(args, w)
    if w.policy == "lrfu_block":
        return run_block(args, w)
    total = args.warmup + args.steps
    dev = "cuda"
    ctx = kvev.context_for(w, max_steps=total)
    for b in range(w.batch):
        K, V = w.prefill_kv(b, device=dev)
        ctx.prefill(b, K, V)
        del K, V
    inputs = [w.step_inputs(t, device=dev) for t in range(1, total + 1)]
    out = torch.empty((w.n_layers, w.batch, w.n_q_heads, w.head_dim), dtype=torch.float32,
                      device=dev)
    torch.cuda.synchronize()

    first_ms = warm_up(ctx, inputs, out, args.warmup)
    dt, n_prof = timed_steps(ctx, inputs, out, args.warmup, total, args.prof_every)
    prof = {k: ctx.profile_read(k) for k in ("attn", "attn_whole", "post", "move", "diag")}
    diag = None
    if w.diag_topk > 0:
        import numpy as np
        # rank-trace statistics over the whole run, averaged over the groups
        gs = ctx.diag_read()
        mean = lambda key, den: float(np.mean([g[key] / max(g[den], 1) for g in gs]))
        diag = {"k": w.diag_topk, "steps": gs[0]["steps"],
                "raw_churn": mean("sum_raw_churn", "pairs"),
                "util_churn": mean("sum_util_churn", "pairs"),
                "raw_util_jaccard": mean("sum_raw_util_jaccard", "steps"),
                "raw_top_evicted": mean("sum_raw_top_evicted", "steps"),
                "selection_churn": mean("sum_selection_churn", "pairs")}
    ctx.close()

    n_tok = w.budget + 1
    kv_bytes, step_bytes = algorithmic_bytes(w, n_tok)
    # the library names the attention launches by kernel: "attn_whole" for
    # the whole-cache kernel, "attn" for the split kernel
    whole = prof["attn_whole"][1] > 0
    assert not (whole and prof["attn"][1] > 0), "both attention kernels ran in the timed steps"
    attn_kernel = ("attn_seq_kernel" if whole else "attn_mfma_kernel") if w.dtype == "bf16" and w.head_dim == 128 \
        else "attn_valu_kernel"
    ms_step = dt * 1e3 / args.steps
    steps_s = args.steps / dt
    attn_ms, attn_n = prof["attn_whole" if whole else "attn"]
    attn_avg_s = attn_ms / max(attn_n, 1) / 1e3
    attn_gbps = kv_bytes / attn_avg_s / 1e9 if attn_avg_s > 0 else None
    policy_ms = sum(prof[k][0] for k in ("post", "move", "diag")) / n_prof
    result = {
        "metric": "decode steps/s + KV-read GB/s (% HBM peak), incl. EMA/top-k/compaction",
        "value": round(steps_s, 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded outlier-channel / heavy-key generator)",
        "config": {"workload": w.name, "layers": w.n_layers, "q_heads": w.n_q_heads,
                   "kv_heads": w.n_kv_heads, "head_dim": w.head_dim, "batch": w.batch,
                   "prefill": w.prefill_lens[0], "budget": w.budget, "n_sink": w.n_sink,
                   "n_recent": w.n_recent, "alpha_new": w.alpha_new, "scorer": w.scorer,
                   "granularity": w.granularity, "diag_topk": w.diag_topk},
        "kv_read_GBps": round(step_bytes / (dt / args.steps) / 1e9, 1),
        "pct_hbm_peak": round(100.0 * step_bytes / (dt / args.steps) / 1e9 / HBM_PEAK_GBPS, 2),
        "score_topk_compaction_share": round(policy_ms / ms_step, 4) if ms_step > 0 else None,
        "kernel_avg_us": {k: round(v[0] / max(v[1], 1) * 1e3, 3) for k, v in prof.items() if v[1]},
        "profiled_steps": n_prof,
        "first_step_ms": round(first_ms, 3),
        "roofline": {
            "bound": "hbm",
            "achieved": round(attn_gbps, 1) if attn_gbps else None,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(attn_gbps / HBM_PEAK_GBPS, 4) if attn_gbps else None,
            # the committed counters were taken on the 32k workload only
            "traffic": (measured_traffic(*((SEQ_TRAFFIC_PROFILE, SEQ_SOURCES) if whole else ()))
                        if args.workload == "llama8b_32k" else None),
            "kernel": attn_kernel,
            "algorithmic_bytes_per_launch": kv_bytes,
        },
    }
    if diag is not None:
        result["diagnostics"] = diag
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
