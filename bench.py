"""Benchmark: DSA decode queries/s at 128K context, k = 2048, on one MI355X.

One step = one dsa_forward call (lightning indexer -> top-k -> sparse MLA
attention + split combine) over the long-context decode batch: 16 sequences
of 131072 tokens, one query token each, 64x128 FP8 indexer, 128 heads over
576-wide latent rows, 2% planted far keys.  Inputs are synthetic, seeded and
resident in HBM before timing starts.

Cache state.  A decoding model runs this step once per layer, each layer over
its own caches, so a layer's keys are never in L2 or the 256 MB MALL when its
step starts.  The benchmark reproduces that with REPLICAS copies of the
per-layer tensors (index keys, latent KV, queries) used in rotation: between
two uses of one copy, the others stream several GB through the caches.  The
steps run back to back on one stream, as a model's layers do.

Prints one JSON line.  `roofline` covers the dominant kernel (the indexer,
bound by HBM), timed with HIP events on the stream it runs on; `cpu_baseline`
times the float64 CPU oracle on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FP8_PEAK_TFLOPS = 5033.0
BF16_PEAK_TFLOPS = 2517.0
REPLICAS = 4

# HBM traffic of one indexer launch on the 128K decode batch, from two
# rocprofv3 --pmc passes (FETCH_SIZE, WRITE_SIZE) over this script with
# --copy-calibration, each scaled by counter/true bytes of a plain 256 MiB
# device copy in the same pass.  Valid only for the kernel sources they were
# taken on (hash below); otherwise the field is reported as null.
TRAFFIC = {
    "sources_sha256": "5351d7d2401fe9d357b182341292a5dd73e8f9e31745fcf393af6cc1f6153df9",
    # FETCH_SIZE 135763.5 KiB/launch x 1.99981 (copy: 131084.2 KiB counted for 262144 KiB read)
    "fetch_bytes": 278017797,
    # WRITE_SIZE 8192.0 KiB/launch x 1.0 (copy: 262144 KiB counted for 262144 KiB written)
    "write_bytes": 8388608,
}
# the indexer kernel's device code (launch.h holds host declarations only)
TRAFFIC_SOURCES = ("sparse_attention_long_03_amd/csrc/indexer.hip", "sparse_attention_long_03_amd/csrc/indexer_math.h",
                   "sparse_attention_long_03_amd/csrc/common.h")


def sources_hash():
    h = hashlib.sha256()
    for rel in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="decode128k")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the CPU-oracle sample")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--kl", action="store_true",
                    help="with --config train64k_chunk4k: time the indexer's KL training signal instead of the "
                         "attention backward")
    ap.add_argument("--kl-dense", action="store_true",
                    help="with a decode config: time the dense warm-up's KL target over every position")
    ap.add_argument("--proj", action="store_true",
                    help="time the indexer projection (hidden states -> FP8 query + scale, head weights, index key)")
    ap.add_argument("--crossover", action="store_true",
                    help="time the masked dense attention against the sparse gather over context lengths")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run plain 256 MiB device copies (reference dispatches for HBM counters)")
    return ap.parse_args()


def algorithmic_bytes(x):
    """Bytes (and flops) the method must move per forward, per kernel.

    indexer: per visible (query, key) pair the FP8 key row and its scale are
    read and one fp32 logit is written; per query the FP8 query, its scale and
    the head weights are read.  top-k: the logits are read and k indices
    written.  attention: per selected row the 576 bf16 latent values and the
    index are read; per query the 128x576 bf16 query is read and the 128x512
    bf16 output written."""
    c = x.cfg
    n = (x.pos.long() + 1).sum().item()                      # visible (query, key) pairs
    T = x.T
    idx_bytes = n * (c.D_I + 4) + n * 4 + T * (c.H_I * c.D_I + 4 + 4 * c.H_I)
    sel = sum(min(int(p) + 1, c.k) for p in x.pos.tolist())   # selected rows
    topk_bytes = n * 4 + T * c.k * 4
    attn_bytes = sel * (c.D * 2 + 4) + T * c.H * c.D * 2 + T * c.H * c.d_v * 2
    idx_flops = 2 * n * c.H_I * c.D_I
    attn_flops = 2 * sel * c.H * (c.D + c.d_v)
    return dict(n_pairs=n, selected=sel, indexer=idx_bytes, topk=topk_bytes, attn=attn_bytes,
                indexer_flops=idx_flops, attn_flops=attn_flops)


def replicas(x, n):
    """n copies of the per-layer tensors (same values, distinct memory)."""
    out = [x]
    for _ in range(n - 1):
        out.append(dataclasses.replace(x, iq8=x.iq8.clone(), iqs=x.iqs.clone(), iw=x.iw.clone(), q=x.q.clone(),
                                       ik8=x.ik8.clone(), iks=x.iks.clone(), kv=x.kv.clone()))
    return out


def timed_rotation(fns, n, stream):
    """Runs fns[i % len(fns)] for i < n back to back on `stream`; returns the
    per-launch durations (ms) from HIP events recorded around each call."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(evs):
        a.record(stream)
        fns[i % len(fns)]()
        b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def batch_rotation(fns, n, stream):
    """Runs fns[i % len(fns)] for i < n back to back on `stream` between one
    pair of HIP events; returns the mean duration per launch (ms).  Unlike an
    event pair around every launch, this adds no marker packets between the
    kernels, so it matches a profiler's per-kernel time up to the launch gaps."""
    import torch
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for i in range(n):
        fns[i % len(fns)]()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n


def mean(xs):
    return sum(xs) / len(xs)


def median(xs):
    return sorted(xs)[len(xs) // 2]


def _host_rows(x, b, n, cache):
    """Logical rows 0..n-1 of sequence b of a cache (contiguous or paged), on the host."""
    import torch
    if x.block_table is None:
        return cache[b, :n].cpu()
    pos = torch.arange(n, device=cache.device)
    pages = x.block_table[b].long()[pos // 64]
    return cache[pages, pos % 64].cpu()


def cpu_baseline(x, budget_s, rows=None, extrapolate_to=None):
    """Float64 oracle on the host cores, one query at a time (cycling over
    `rows`, by default every query of the batch) until the time budget is
    spent.  BLAS threads are set to the process's CPU affinity count, which is
    what `cores` reports.  With `extrapolate_to` (prefill), the rows are a
    uniform sample of the queries and the rate is extrapolated: the sample's
    mean time per query stands for every query's.  A sequence's caches are
    copied to the host (untimed) the first time one of its queries runs."""
    import numpy as np
    import oracle as O
    from sparse_attention_long_03_amd import inputs as I
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_limits
    except Exception:
        threadpool_limits = None
    c = x.cfg
    rows = list(range(x.T)) if rows is None else list(rows)
    seq_cache = {}

    def host_seq(b, n):
        if b not in seq_cache or seq_cache[b][0] < n:
            L = max(n, int(x.seq_lens[b]))
            seq_cache[b] = (L, _host_rows(x, b, L, x.ik8).numpy(), _host_rows(x, b, L, x.iks).numpy().astype(np.float64),
                            I.bf16_bits(_host_rows(x, b, L, x.kv)))
        return seq_cache[b]

    done, dt = 0, 0.0
    ctx = threadpool_limits(cores) if threadpool_limits is not None else None
    try:
        while dt <= budget_s:
            t = rows[done % len(rows)]
            b, n = int(x.seq_id[t]), int(x.pos[t]) + 1
            _, k8, ks, kv = host_seq(b, n)
            q8, qs, w = x.iq8[t].cpu().numpy(), float(x.iqs[t]), x.iw[t].cpu().numpy().astype(np.float64)
            q = I.bf16_bits(x.q[t:t + 1])
            ts = time.perf_counter()
            lg = O.indexer_logits_row(q8, qs, w, k8[:n], ks[:n])
            sel = O.topk_select(lg.astype(np.float32), n, c.k)
            O.sparse_mla_attention(q, kv[None, :n], sel[None], np.zeros(1, int), c.scale, c.d_v)
            dt += time.perf_counter() - ts
            done += 1
    finally:
        if ctx is not None:
            ctx.restore_original_limits()
    rate = done / dt
    if extrapolate_to is None:
        sample = (f"{done} queries of the same workload, cycling over its {len(rows)} query rows (indexer over all "
                  f"of each row's keys, top-k, attention), float64 NumPy oracle, {dt:.1f} s")
        unit = "queries/s"
    else:
        sample = (f"{done} query rows of a uniform sample of {len(rows)} of the workload's {extrapolate_to} (indexer "
                  f"over all of each row's keys, top-k, attention), float64 NumPy oracle, {dt:.1f} s; extrapolated: "
                  f"the sample's mean time per row stands for every row's")
        unit = "tokens/s"
    return {"value": round(rate, 3), "unit": unit, "cores": cores, "kind": "oracle", "sample": sample}


def cache_write_timing(x, n_launch, stream):
    """dsa_cache_write of one new token per query (its FP8 index key and
    latent row) at the query's position: mean time and algorithmic GB/s
    (fp32 key + bf16 row read; FP8 key + scale + row written)."""
    import torch
    from sparse_attention_long_03_amd import binding as B
    c = x.cfg
    g = torch.Generator(device="cuda").manual_seed(99)
    k_new = torch.randn((x.T, c.D_I), generator=g, device="cuda")
    kv_new = torch.randn((x.T, c.D), generator=g, device="cuda").to(torch.bfloat16)
    q = B.queries(x.seq_id, x.pos, c.B, x.max_len)
    lay = B.paged_layout(x.block_table, x.kv.shape[0], c.page_size) if x.block_table is not None \
        else B.contiguous_layout(x.kv.shape[1])
    fn = lambda: B.dsa_cache_write(q, lay, c.D_I, k_new, kv_new, x.ik8, x.iks, x.kv)
    timed_rotation([fn], 2, stream)
    ts = mean(timed_rotation([fn], n_launch, stream))
    nbytes = x.T * (c.D_I * 4 + c.D * 2 + c.D_I + 4 + c.D * 2)
    return round(ts * 1e3, 2), round(nbytes / (ts * 1e-3) / 1e9, 1)


def workload_name(cfg):
    if cfg.kind == "decode":
        return (f"{cfg.name}: decode, B={cfg.B} sequences x L={cfg.L} tokens, 1 query token each, indexer "
                f"{cfg.H_I}x{cfg.D_I} FP8, top-k={cfg.k}, MLA-MQA {cfg.H} heads x 576 (512+64 rope)"
                + (f", {cfg.planted_frac:.0%} planted far keys" if cfg.planted_frac > 0 else ""))
    if cfg.kind == "ragged":
        return (f"{cfg.name}: B={cfg.B} sequences, lengths uniform in [{cfg.min_len},{cfg.L}], paged KV "
                f"(page {cfg.page_size}), 1-2 query tokens each, top-k={cfg.k}")
    return cfg.name


def bench_prefill(args, cfg):
    """Prefill: every token of one sequence is a causal query.  dsa_forward
    takes its many-token branch (indexer fused with the selection, no logits
    stored), then the sparse attention.  Both are bound by the matrix cores,
    so the roofline is the fused kernel's FP8 TFLOP/s."""
    import torch
    from sparse_attention_long_03_amd import binding as B
    from sparse_attention_long_03_amd import inputs as I
    from sparse_attention_long_03_amd.path import DSAPath

    x = I.make_inputs(cfg, "cuda")
    p = DSAPath(x)
    p.ws(B.DSA_OP_FORWARD)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        p.forward()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        p.forward()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps

    k = cfg.k
    idx = torch.empty((x.T, k), dtype=torch.int32, device="cuda")
    sel_ws = B.workspace(B.dsa_workspace_bytes(B.DSA_OP_INDEXER_TOPK, x.T, x.max_len, 0, k))
    fused = lambda: B.dsa_indexer_topk(p.q, p.layout, cfg.H_I, cfg.D_I, x.iq8, x.iqs, x.iw, x.ik8, x.iks, k, idx,
                                       sel_ws)
    n_launch = max(args.steps, 5)
    timed_rotation([fused, lambda: p.attn(idx)], 2, stream)
    fused_ts = timed_rotation([fused], n_launch, stream)
    attn_ts = timed_rotation([lambda: p.attn(idx)], n_launch, stream)
    fused_avg, attn_avg = mean(fused_ts), mean(attn_ts)
    step_ts = timed_rotation([p.forward], max(args.steps, 5), stream)
    cw_us, cw_gbs = cache_write_timing(x, n_launch, stream)  # last: it overwrites the caches

    pairs = (x.pos.long() + 1).sum().item()
    sel = sum(min(int(q) + 1, k) for q in x.pos.tolist())
    idx_flops = 2 * pairs * cfg.H_I * cfg.D_I
    attn_flops = 2 * sel * cfg.H * (cfg.D + cfg.d_v)
    idx_tf = idx_flops / (fused_avg * 1e-3) / 1e12
    attn_tf = attn_flops / (attn_avg * 1e-3) / 1e12
    out = {
        "metric": "DSA prefill tokens/s @64K ctx, k=2048",
        "value": round(x.T / (wall_ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3 indexer / bf16 attention, fp32 accumulate",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: prefill, 1 sequence of {cfg.L} tokens, every token a causal query, "
                               f"indexer {cfg.H_I}x{cfg.D_I} FP8 fused with top-{k} (no logits stored), MLA-MQA "
                               f"{cfg.H} heads x 576", "L": cfg.L, "T": x.T, "k": k, "H_I": cfg.H_I, "D_I": cfg.D_I,
                   "H": cfg.H},
        "roofline": {"bound": "mfma", "kernel": f"indexer_topk_kernel<{cfg.H_I},{cfg.D_I}>",
                     "achieved": round(idx_tf, 1), "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(idx_tf / FP8_PEAK_TFLOPS, 4), "traffic": None,
                     "flops_per_launch": idx_flops, "avg_launch_us": round(fused_avg * 1e3, 1)},
        "p10_ms": round(sorted(step_ts)[len(step_ts) // 10], 3),
        "p90_ms": round(sorted(step_ts)[(9 * len(step_ts)) // 10], 3),
        "kernels": {"indexer_topk_ms": round(fused_avg, 3), "indexer_tflops": round(idx_tf, 1),
                    "attn_ms": round(attn_avg, 3), "attn_tflops": round(attn_tf, 1),
                    "attn_frac_bf16": round(attn_tf / BF16_PEAK_TFLOPS, 4),
                    "cache_write_us": cw_us, "cache_write_gbs": cw_gbs},
    }
    if not args.no_cpu:
        import random
        rows = random.Random(7).sample(range(x.T), 256)  # random order: any prefix is a uniform sample
        out["cpu_baseline"] = cpu_baseline(x, args.cpu_seconds, rows=rows, extrapolate_to=x.T)
    print(json.dumps(out), flush=True)


def bench_backward(args, cfg):
    """Training-step backward of the sparse attention: the last 4096 tokens
    of a 64K-token sequence as queries, each with its full top-2048
    selection (from the forward, untimed).  A step zeroes dkv and runs
    dsa_sparse_mla_attn_bwd (dq kernel, row sort, per-slot dkv, reduction).
    The dq kernel, the largest part, is also timed alone through
    dsa_sparse_mla_attn_bwd_dq: its roofline is bf16 MFMA."""
    import torch
    from sparse_attention_long_03_amd import binding as B
    from sparse_attention_long_03_amd import inputs as I
    from sparse_attention_long_03_amd.path import DSAPath

    x = I.make_inputs(cfg, "cuda")
    p = DSAPath(x)
    _, _, idx = p.forward()
    dO = I.output_grad(cfg, x.T, "cuda")
    dq, dkv = p.attn_bwd(idx, dO)
    stream = torch.cuda.current_stream()

    def step():
        dkv.zero_()
        p.attn_bwd(idx, dO, dkv=dkv)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps

    k = cfg.k
    ws = p._ws[("bwd", B.dsa_workspace_bytes(B.DSA_OP_ATTN_BWD, x.T, x.max_len, cfg.H, k))]
    dq_only = lambda: B.dsa_sparse_mla_attn_bwd_dq(p.q, p.layout, cfg.H, x.q, x.kv, idx, k, cfg.scale, p.out, p.lse,
                                                   dO, dq, ws)
    n_launch = max(args.steps, 5)
    timed_rotation([dq_only], 2, stream)
    dq_avg = mean(timed_rotation([dq_only], n_launch, stream))
    step_avg = mean(timed_rotation([step], n_launch, stream))

    sel = sum(min(int(q) + 1, k) for q in x.pos.tolist())
    # per (selected row, head): S and dq over 576, dP over 512, the stacked
    # [scale dS; P] product over 512 (dK no-rope + dV) twice, dK rope over 64
    bwd_flops = 2 * sel * cfg.H * (576 + 512 + 576 + 2 * 512 + 64)
    dq_flops = 2 * sel * cfg.H * (576 + 512 + 576)
    dq_tf = dq_flops / (dq_avg * 1e-3) / 1e12
    out = {
        "metric": "sparse MLA-MQA backward query tokens/s @64K ctx, k=2048",
        "value": round(x.T / (wall_ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 MFMA, fp32 accumulate; P, dS and per-row gradients rounded to bf16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: backward of the sparse attention for {x.T} query tokens at positions "
                               f"{cfg.L - x.T}..{cfg.L - 1} of one {cfg.L}-token sequence, top-{k} selection each, "
                               f"MLA-MQA {cfg.H} heads x 576", "L": cfg.L, "T": x.T, "k": k, "H": cfg.H},
        "roofline": {"bound": "mfma", "kernel": "sparse_mla_bwd_dq_kernel<4>", "achieved": round(dq_tf, 1),
                     "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(dq_tf / BF16_PEAK_TFLOPS, 4),
                     "traffic": None, "flops_per_launch": dq_flops, "avg_launch_us": round(dq_avg * 1e3, 1)},
        "kernels": {"dq_ms": round(dq_avg, 3), "backward_ms": round(step_avg, 3),
                    "backward_tflops": round(bwd_flops / (step_avg * 1e-3) / 1e12, 1),
                    "backward_frac_bf16": round(bwd_flops / (step_avg * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)},
    }
    print(json.dumps(out), flush=True)


def bench_kl(args, cfg):
    """The indexer's KL training signal on the training chunk: the target
    (head-mean attention probabilities of each query's top-2048, from the
    forward's lse) and the KL loss with its gradients into the indexer query,
    key and head weights.  A step zeroes dk and runs dsa_indexer_kl_target and
    dsa_indexer_kl.  The target kernel, the larger part, gathers every
    selected latent row (1152 B) per query, as the forward attention does, and
    scores it for all heads: it is bound by that gather, so its roofline is
    HBM bandwidth."""
    import torch
    from sparse_attention_long_03_amd import binding as B
    from sparse_attention_long_03_amd import inputs as I
    from sparse_attention_long_03_amd.path import DSAPath

    x = I.make_inputs(cfg, "cuda")
    p = DSAPath(x)
    _, lse, idx = p.forward()
    k = cfg.k
    target = p.kl_target(idx)
    loss, dq, dw, dk = p.indexer_kl(idx, target)
    stream = torch.cuda.current_stream()
    ws = p._ws[("kl", B.dsa_workspace_bytes(B.DSA_OP_INDEXER_KL, x.T, x.max_len, 0, k))]
    tgt_call = lambda: B.dsa_indexer_kl_target(p.q, p.layout, cfg.H, x.q, x.kv, idx, k, cfg.scale, lse, target)
    kl_call = lambda: B.dsa_indexer_kl(p.q, p.layout, cfg.H_I, cfg.D_I, x.iq8, x.iqs, x.iw, x.ik8, x.iks, idx, k,
                                       target, loss, dq, dw, dk, ws)

    def step():
        dk.zero_()
        tgt_call()
        kl_call()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    n_launch = max(args.steps, 5)
    timed_rotation([tgt_call, kl_call], 2, stream)
    tgt_avg = mean(timed_rotation([tgt_call], n_launch, stream))
    kl_avg = mean(timed_rotation([kl_call], n_launch, stream))

    sel = sum(min(int(q) + 1, k) for q in x.pos.tolist())
    tgt_flops = 2 * sel * cfg.H * cfg.D                       # scores of every head over the selected rows
    # per selected entry: its latent row, its index, its target value written;
    # per query: q (H x 576 bf16) and lse
    tgt_bytes = sel * (cfg.D * 2 + 4 + 4) + x.T * cfg.H * (cfg.D * 2 + 4)
    # per selected entry: the indexer scores twice (64 heads x 128), and the
    # dq and dk contractions (64 x 128 each)
    kl_flops = 2 * sel * cfg.H_I * cfg.D_I * 4
    tgt_tf = tgt_flops / (tgt_avg * 1e-3) / 1e12
    tgt_gbs = tgt_bytes / (tgt_avg * 1e-3) / 1e9
    out = {
        "metric": "indexer KL training signal query tokens/s @64K ctx, k=2048",
        "value": round(x.T / (wall_ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 attention scores / fp8-e4m3 indexer, fp32 accumulate; bf16 masked products",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: KL target and indexer loss/gradients for {x.T} query tokens at positions "
                               f"{cfg.L - x.T}..{cfg.L - 1} of one {cfg.L}-token sequence, top-{k} selection each, "
                               f"{cfg.H} attention heads, indexer {cfg.H_I}x{cfg.D_I}", "L": cfg.L, "T": x.T, "k": k,
                   "H": cfg.H, "H_I": cfg.H_I, "D_I": cfg.D_I},
        "roofline": {"bound": "hbm", "kernel": "kl_target_kernel", "achieved": round(tgt_gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(tgt_gbs / HBM_PEAK_GBS, 4),
                     "traffic": None, "bytes_per_launch": tgt_bytes, "avg_launch_us": round(tgt_avg * 1e3, 1)},
        "kernels": {"target_ms": round(tgt_avg, 3), "target_tflops": round(tgt_tf, 1),
                    "target_frac_bf16": round(tgt_tf / BF16_PEAK_TFLOPS, 4), "kl_ms": round(kl_avg, 3),
                    "kl_tflops": round(kl_flops / (kl_avg * 1e-3) / 1e12, 1)},
    }
    print(json.dumps(out), flush=True)


def bench_kl_dense(args, cfg):
    """The dense warm-up's KL target (dsa_indexer_kl_target_dense) over every
    position 0..pos[t] of each decode query: the dense attention's lse (first
    pass over the rows) and the head-mean probabilities (second pass).  Each
    pass reads every latent row of the query's sequence (1152 B) once, so the
    kernels are bound by HBM; four replicas of the caches rotate so that no
    launch finds its rows in the MALL."""
    import torch
    from sparse_attention_long_03_amd import binding as B
    from sparse_attention_long_03_amd import inputs as I
    from sparse_attention_long_03_amd.path import DSAPath

    x0 = I.make_inputs(I.scaled(cfg, planted_frac=0.0), "cuda")
    xs = replicas(x0, REPLICAS)
    paths = [DSAPath(x) for x in xs]
    target = torch.empty((x0.T, paths[0].ld), dtype=torch.float32, device="cuda")
    lse = torch.empty((x0.T, cfg.H), dtype=torch.float32, device="cuda")
    ws = B.workspace(B.dsa_workspace_bytes(B.DSA_OP_KL_TARGET_DENSE, x0.T, x0.max_len, cfg.H, 0))
    fns = [(lambda p=p, x=x: B.dsa_indexer_kl_target_dense(p.q, p.layout, cfg.H, x.q, x.kv, cfg.scale, target, lse,
                                                           ws)) for p, x in zip(paths, xs)]
    stream = torch.cuda.current_stream()
    timed_rotation(fns, 2 * REPLICAS, stream)
    n_launch = max(args.steps, 20)
    avg = batch_rotation(fns, n_launch, stream)
    ts = timed_rotation(fns, n_launch, stream)
    n = (x0.pos.long() + 1).sum().item()
    nbytes = 2 * n * cfg.D * 2 + n * 4 + 2 * x0.T * cfg.H * cfg.D * 2
    flops = 2 * 2 * n * cfg.H * cfg.D
    gbs = nbytes / (avg * 1e-3) / 1e9
    # the one-pass form (dsa_indexer_kl_target_dense_lse), given each replica's
    # dense lse as a dense attention forward would return it: one read of the rows
    lses = []
    for f in fns[:REPLICAS]:
        f()
        lses.append(lse.clone())
    fns1 = [(lambda p=p, x=x, l=l: B.dsa_indexer_kl_target_dense_lse(p.q, p.layout, cfg.H, x.q, x.kv, cfg.scale, l,
                                                                     target)) for p, x, l in zip(paths, xs, lses)]
    timed_rotation(fns1, 2 * REPLICAS, stream)
    avg1 = batch_rotation(fns1, n_launch, stream)
    nbytes1 = n * cfg.D * 2 + n * 4 + x0.T * cfg.H * (cfg.D * 2 + 4)
    gbs1 = nbytes1 / (avg1 * 1e-3) / 1e9
    out = {"metric": "dense warm-up KL target query tokens/s @128K ctx (every position)",
           "value": round(x0.T / (avg * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": n_launch,
           "warmup": 2 * REPLICAS, "ms_per_step": round(avg, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16 scores, fp32 softmax", "data": "synthetic",
           "config": {"workload": f"{cfg.name}: {x0.T} decode queries, target over all {x0.max_len} positions each, "
                                  f"{cfg.H} heads x 576", "T": x0.T, "L": cfg.L, "H": cfg.H},
           "roofline": {"bound": "hbm", "kernel": "kl_target_kernel<1> + kl_target_kernel<2>", "achieved": round(gbs, 1),
                        "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                        "bytes_per_launch": nbytes, "avg_launch_us": round(avg * 1e3, 1),
                        "p10_us": round(sorted(ts)[len(ts) // 10] * 1e3, 1),
                        "p90_us": round(sorted(ts)[(9 * len(ts)) // 10] * 1e3, 1)},
           "kernels": {"tflops": round(flops / (avg * 1e-3) / 1e12, 1),
                       "one_pass_given_lse_ms": round(avg1, 4), "one_pass_gbs": round(gbs1, 1),
                       "one_pass_frac_hbm": round(gbs1 / HBM_PEAK_GBS, 4), "one_pass_bytes": nbytes1}}
    print(json.dumps(out), flush=True)


def bench_crossover(args):
    """Sparse gather vs masked dense attention on the same top-2048 selection,
    prefill (every token a query) and 16-sequence decode, L = 1K .. 16K: the
    context length below which the dense variant is faster."""
    import torch
    from sparse_attention_long_03_amd import inputs as I
    from sparse_attention_long_03_amd.path import DSAPath

    stream = torch.cuda.current_stream()
    n = max(args.steps // 5, 5)
    series = {}
    for kind, base in (("prefill", I.CONFIGS["prefill64k"]), ("decode_b16", I.CONFIGS["decode128k"])):
        pts = []
        for L in (1024, 2048, 4096, 8192, 16384):
            cfg = I.scaled(base, L=L, planted_frac=0.0)
            x = I.make_inputs(cfg, "cuda")
            p = DSAPath(x)
            idx = p.indexer_topk() if x.T >= 2048 else p.topk(p.indexer())
            out, lse = torch.empty_like(p.out), torch.empty_like(p.lse)
            sparse = lambda: p.attn(idx)
            dense = lambda: p.dense_attn(idx, out, lse)
            timed_rotation([sparse, dense], 4, stream)
            ts = mean(timed_rotation([sparse], n, stream))
            td = mean(timed_rotation([dense], n, stream))
            pts.append({"L": L, "T": x.T, "sparse_ms": round(ts, 4), "dense_ms": round(td, 4),
                        "rows_gathered": sum(min(int(q) + 1, cfg.k) for q in x.pos.tolist()),
                        "rows_dense": int((x.pos.long() + 1).sum().item())})
            del x, p, idx, out, lse
            torch.cuda.empty_cache()
        faster = [pt["L"] for pt in pts if pt["dense_ms"] < pt["sparse_ms"]]
        series[kind] = {"points": pts, "dense_faster_up_to_L": max(faster) if faster else None}
    print(json.dumps({"metric": "masked dense vs sparse attention time, same top-2048 selection", "unit": "ms",
                      "n_gpus": 1, "data": "synthetic", "series": series}), flush=True)


def bench_projection(args):
    """The indexer's inputs from hidden states (dsa_indexer_project): per
    token, q = Wq h (64 heads x 128, then FP8 with a per-token scale),
    w = Ww h and the token's index key k = Wk h, from bf16 h and weights.
    The hidden width is 7168 (the pages leave d open; this is the width of
    the model family they describe).  Decode (16 tokens) streams the 120 MB
    of weights: bound by HBM, with four weight replicas in rotation so that no
    launch finds them in the 256 MB MALL (one per layer in a model).  A
    4096-token chunk is bound by the bf16 matrix cores."""
    import torch
    from sparse_attention_long_03_amd import binding as B

    d, H_I, D_I = 7168, 64, 128
    N = H_I * D_I + H_I + D_I
    stream = torch.cuda.current_stream()
    g = torch.Generator(device="cuda").manual_seed(5)
    mk = lambda *shape, s=1.0: (torch.randn(shape, generator=g, device="cuda") * s).to(torch.bfloat16)
    weights = [(mk(H_I * D_I, d, s=d ** -0.5), mk(H_I, d, s=d ** -0.5), mk(D_I, d, s=d ** -0.5))
               for _ in range(REPLICAS)]
    res = {}
    n_launch = max(args.steps, 20)
    for T in (16, 4096):
        h = mk(T, d)
        q8 = torch.empty((T, H_I, D_I), dtype=torch.uint8, device="cuda")
        qs = torch.empty((T,), dtype=torch.float32, device="cuda")
        w = torch.empty((T, H_I), dtype=torch.float32, device="cuda")
        k = torch.empty((T, D_I), dtype=torch.float32, device="cuda")
        ws = B.workspace(B.dsa_workspace_bytes(B.DSA_OP_INDEXER_PROJ, T, d, H_I, D_I))
        fns = [(lambda wq=wq, ww=ww, wk=wk: B.dsa_indexer_project(d, H_I, D_I, h, wq, ww, wk, q8, qs, w, k, ws))
               for wq, ww, wk in weights]
        timed_rotation(fns, 2 * REPLICAS, stream)
        avg = batch_rotation(fns, n_launch, stream)
        ts = timed_rotation(fns, n_launch, stream)
        nbytes = N * d * 2 + T * d * 2 + T * (H_I * D_I + 4 + 4 * H_I + 4 * D_I)
        flops = 2 * T * d * N
        res[f"T{T}"] = {"us": round(avg * 1e3, 2), "p10_us": round(sorted(ts)[len(ts) // 10] * 1e3, 2),
                        "p90_us": round(sorted(ts)[(9 * len(ts)) // 10] * 1e3, 2),
                        "gbs": round(nbytes / (avg * 1e-3) / 1e9, 1),
                        "frac_hbm": round(nbytes / (avg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                        "tflops": round(flops / (avg * 1e-3) / 1e12, 1),
                        "frac_bf16": round(flops / (avg * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                        "bytes_per_launch": nbytes, "flops_per_launch": flops}
        del h, q8, qs, w, k, ws, fns
    dec = res["T16"]
    out = {"metric": "indexer projection tokens/s (hidden 7168 -> FP8 query 64x128 + scale, 64 weights, 128-wide key)",
           "value": round(16 / (dec["us"] * 1e-6), 1), "unit": "tokens/s", "n_gpus": 1, "steps": n_launch,
           "warmup": 2 * REPLICAS, "higher_is_better": True, "dtype": "bf16 MFMA, fp32 accumulate; FP8 query codes",
           "data": "synthetic",
           "config": {"workload": "decode step of 16 tokens (4 weight replicas in rotation) and a 4096-token chunk",
                      "d": d, "H_I": H_I, "D_I": D_I},
           "roofline": {"bound": "hbm", "kernel": "proj_gemm_kernel<16> + proj_finish_kernel<8,1024>",
                        "achieved": dec["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": dec["frac_hbm"],
                        "traffic": None, "bytes_per_launch": dec["bytes_per_launch"], "avg_launch_us": dec["us"]},
           "points": res}
    print(json.dumps(out), flush=True)


def stream_copy_gbs():
    """Measured device-to-device copy bandwidth on this GPU: a 1 GiB buffer
    (four times the 256 MB MALL) copied with torch, read + written bytes over
    the mean HIP-event time of 5 copies."""
    import torch
    n = 1 << 28  # int32 elements: 1 GiB
    src = torch.ones(n, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(5)]
    for a, b in ev:
        a.record()
        dst.copy_(src)
        b.record()
    torch.cuda.synchronize()
    ms = mean([a.elapsed_time(b) for a, b in ev])
    del src, dst
    torch.cuda.empty_cache()
    return 2 * 4 * n / (ms * 1e-3) / 1e9


def forward_graph_timing(fwd, steps, stream):
    """The same decode steps launched from HIP graphs: one graph per replica,
    each holding one dsa_forward, replayed in rotation for exactly `steps`
    steps between two synchronisations.  Returns microseconds per step."""
    import torch
    graphs = []
    for f in fwd:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            f()
        graphs.append(g)
    torch.cuda.synchronize()
    for i in range(2 * len(graphs)):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    us = (time.perf_counter() - t0) * 1e6 / steps
    stream.synchronize()
    return us


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the DSA path runs on one GPU: --gpus must be 1 (how it would shard over several "
                                   "GPUs is described, not implemented)"}))
        sys.exit(2)
    import torch
    from sparse_attention_long_03_amd import binding as B
    from sparse_attention_long_03_amd import inputs as I
    from sparse_attention_long_03_amd.path import DSAPath

    torch.cuda.set_device(0)
    if args.crossover:
        bench_crossover(args)
        return
    if args.proj:
        bench_projection(args)
        return
    cfg = I.CONFIGS[args.config]
    if cfg.kind == "prefill":
        bench_prefill(args, cfg)
        return
    if cfg.name == "train64k_chunk4k":
        if args.kl:
            bench_kl(args, cfg)
        else:
            bench_backward(args, cfg)
        return
    if args.kl_dense:
        bench_kl_dense(args, cfg)
        return
    x0 = I.make_inputs(cfg, "cuda")
    xs = replicas(x0, REPLICAS)
    paths = [DSAPath(x) for x in xs]
    for p in paths[1:]:
        p._ws = paths[0]._ws  # one workspace, as in a model's layer loop
    for p in paths:
        p.ws(B.DSA_OP_FORWARD)
    stream = torch.cuda.current_stream()
    fwd = [p.forward for p in paths]
    torch.cuda.synchronize()

    # warmup, then exactly `steps` dsa_forward calls back to back (wall clock
    # between two synchronisations; per-step HIP events alongside)
    for i in range(args.warmup):
        fwd[i % REPLICAS]()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        fwd[i % REPLICAS]()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps

    # per-kernel launches, same launch configuration as inside dsa_forward
    n_launch = max(args.steps, 20)
    logits = [p.new_logits() for p in paths]
    idx = torch.empty((x0.T, cfg.k), dtype=torch.int32, device="cuda")
    topk_ws = B.workspace(B.dsa_workspace_bytes(B.DSA_OP_TOPK, x0.T, logits[0].shape[1], 0, cfg.k))
    idx_fns = [(lambda p=p, lg=lg: p.indexer(lg)) for p, lg in zip(paths, logits)]
    topk_fns = [(lambda p=p, lg=lg: B.dsa_topk(lg, p.valid_len, lg.shape[1], cfg.k, idx, topk_ws))
                for p, lg in zip(paths, logits)]
    attn_fns = [(lambda p=p: p.attn(p.idx)) for p in paths]
    timed_rotation(idx_fns + topk_fns + attn_fns, 3 * REPLICAS, stream)  # warm every launch path
    # means from one event pair around each batch of back-to-back launches;
    # per-launch event pairs (which add ~3 us of markers to each) only for the median
    idx_avg = batch_rotation(idx_fns, n_launch, stream)
    topk_avg = batch_rotation(topk_fns, n_launch, stream)
    attn_avg = batch_rotation(attn_fns, n_launch, stream)
    step_avg = batch_rotation(fwd, n_launch, stream)
    idx_ts = timed_rotation(idx_fns, n_launch, stream)
    step_ts = timed_rotation(fwd, n_launch, stream)
    graph_us = forward_graph_timing(fwd, args.steps, stream)
    copy_gbs = stream_copy_gbs()
    cw_us, cw_gbs = cache_write_timing(xs[1], n_launch, stream)  # on a replica not used below

    if args.copy_calibration:
        src = torch.ones(1 << 26, dtype=torch.int32, device="cuda")  # 256 MiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    ab = algorithmic_bytes(x0)
    idx_gbs = ab["indexer"] / (idx_avg * 1e-3) / 1e9
    value = x0.T / (wall_ms * 1e-3)
    traffic = None
    if TRAFFIC["sources_sha256"] is not None and TRAFFIC["sources_sha256"] == sources_hash() \
            and cfg.name == "decode128k":
        traffic = TRAFFIC["fetch_bytes"] + TRAFFIC["write_bytes"]
    out = {
        "metric": ("DSA decode queries/s @128K ctx, k=2048 (+indexer TFLOP/s, sparse-attn GB/s)"
                   if cfg.name == "decode128k" else
                   f"DSA decode queries/s, {cfg.name}, k={cfg.k} (+indexer TFLOP/s, sparse-attn GB/s)"),
        "value": round(value, 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 4),
        "p10_ms": round(sorted(step_ts)[len(step_ts) // 10], 4),
        "p90_ms": round(sorted(step_ts)[(9 * len(step_ts)) // 10], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3 indexer / bf16 attention, fp32 accumulate",
        "data": "synthetic",
        "config": {"workload": workload_name(cfg), "B": cfg.B, "L": cfg.L, "T": x0.T, "k": cfg.k, "H_I": cfg.H_I,
                   "D_I": cfg.D_I, "H": cfg.H, "paged": cfg.paged},
        "roofline": {"bound": "hbm", "kernel": f"indexer_kernel<{cfg.H_I},{cfg.D_I},{'false' if cfg.paged else 'true'}>", "achieved": round(idx_gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(idx_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "stream_copy_gbs": round(copy_gbs, 1),
                     "frac_of_stream_copy": round(idx_gbs / copy_gbs, 4), "bytes_per_launch": ab["indexer"],
                     "avg_launch_us": round(idx_avg * 1e3, 2),
                     "median_launch_us_event_pairs": round(median(idx_ts) * 1e3, 2)},
        "kernels": {
            "indexer_us": round(idx_avg * 1e3, 2),
            "indexer_tflops": round(ab["indexer_flops"] / (idx_avg * 1e-3) / 1e12, 2),
            "topk_us": round(topk_avg * 1e3, 2),
            "topk_gbs": round(ab["topk"] / (topk_avg * 1e-3) / 1e9, 1),
            "attn_us": round(attn_avg * 1e3, 2),
            "attn_gbs": round(ab["attn"] / (attn_avg * 1e-3) / 1e9, 1),
            "attn_tflops": round(ab["attn_flops"] / (attn_avg * 1e-3) / 1e12, 2),
            "forward_event_us": round(step_avg * 1e3, 2),
            "forward_graph_us": round(graph_us, 2),
            "cache_write_us": cw_us,
            "cache_write_gbs": cw_gbs,
        },
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(x0, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
