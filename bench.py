#!/usr/bin/env python3
"""Benchmark: speculative rounds on the 7B-shape bf16 workload, one MI355X.

A timed step is one full speculative round over the batch: K draft steps, verify-input
assembly, ONE target verify pass over K+1 positions, and the fused accept / resample /
bonus step with cache roll-back.  Inputs are synthetic and seeded: random-init weights
of the named shapes (N(0, 0.02^2), bf16), context ids uniform over the vocabulary,
prefilled through the library before timing.  All inputs are resident in HBM when the
timed region starts.

Output: one JSON line.  value = emitted tokens per second over the whole job (accepted
drafts plus the resampled or bonus token of every row, summed over rows).  The
roofline object covers the dominant kernel (the weight-streaming GEMM), timed live with
HIP events on its launch stream over the timed rounds.
"""
import argparse
import gc
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# HBM traffic of the dominant kernel, from rocprofv3 FETCH_SIZE / WRITE_SIZE runs of
# `bench.py --verify-only` scaled by the same counters on a copy of known size; used
# only while the kernel sources still hash to the value recorded with the figures.
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "gemm_verify_7b_b1_k5_traffic.md")
GEMM_SOURCES = ["speculative_decoding_forward_amd/csrc/gemm.hip",
                "speculative_decoding_forward_amd/csrc/common.h",
                "speculative_decoding_forward_amd/csrc/gemm.h",
                "speculative_decoding_forward_amd/csrc/kv_layout.h",
                "speculative_decoding_forward_amd/csrc/act_layout.h",
                "speculative_decoding_forward_amd/build_lib.py"]  # the compile flags


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # 200 rounds: tokens per round vary round to round (one row at B = 1), and 20 rounds
    # left the mean tokens/s uncertain by about 10%; 200 rounds of the 7B shape take 1.3 s
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="7b", choices=["tiny", "small", "7b", "70b", "accept"],
                    help="model workloads run full speculative rounds; 'accept' times the "
                         "fused accept / resample step alone on synthetic logits")
    ap.add_argument("--batch", type=int, default=None)
    ap.add_argument("--K", type=int, default=None)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--sweep", action="store_true",
                    help="K x batch sweep on the 7B shape (one JSON line per point, then a "
                         "summary line); --steps timed rounds per point")
    ap.add_argument("--sweep-batches", default="1,2,4,8,16,32,64")
    ap.add_argument("--sweep-K", default="1,2,3,4,5,6,7,8")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-summaries", action="store_true",
                    help="headline line only: skip the batch-8 and other-workload summaries")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--verify-only", action="store_true",
                    help="target model only: prefill, then --steps eager verify passes "
                         "(each rolled back); for counter runs of the verify GEMMs")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="copy MIB MiB device-to-device three times and exit (known bytes "
                         "for scaling the HBM counters)")
    return ap.parse_args()


def gemm_source_hash():
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic():
    """Bytes per GEMM launch from the committed counter summary, or None when it is absent
    or was taken on other kernel sources."""
    try:
        with open(TRAFFIC_SUMMARY) as fh:
            text = fh.read()
    except OSError:
        return None
    src = re.search(r"kernel_sources_sha256:\s*([0-9a-f]+)", text)
    val = re.search(r"traffic_bytes_per_launch:\s*([0-9.]+)", text)
    if not src or not val or src.group(1) != gemm_source_hash():
        return None
    return float(val.group(1))


def gemm_bytes_per_verify(shape, R):
    """Algorithmic bytes of the weight GEMMs of one forward over R rows: every weight
    once and the activation rows read; outputs: q / K / V / FFN activations in the
    element type (QKV, up), the residual rows read and written in fp32 plus the next
    product's input bf16(x * g) and its per-16-column sums of squares (O-proj, down; the
    last down writes x * g in fp32 for the normalise pass instead), fp32 logits (LM
    head).  Normalised products inside the layers also read their rows' sums of
    squares."""
    d, F, V, L = shape.d_model, shape.d_ffn, shape.vocab, shape.n_layers
    e = shape.elt_bytes()
    ffn_in = 2 * F if shape.ffn_kind == "swiglu" else F
    ss = R * (d // 16) * 4
    resid_out = R * d * 4 * 2 + R * d * e + ss
    last_out = R * d * 4 * 3 + ss
    # (N, K, input bytes, output bytes) of qkv, O-proj, up, down
    gemms = [(3 * d, d, R * d * e + ss, R * 3 * d * e), (d, d, R * d * e, resid_out),
             (ffn_in, d, R * d * e + ss, R * F * e), (d, F, R * F * e, resid_out)]
    total, n = 0, 0
    for N, K, a_in, out in gemms:
        total += L * (N * K * e + a_in + out)
        n += L
    total += last_out - resid_out
    total += V * d * e + R * d * e + R * V * 4
    n += 1
    return total, n


def verify_bytes(shape, B, K, lens):
    """Algorithmic bytes of one verify call: weights once, gathered embedding rows, KV
    read (context + new positions) and write, logits."""
    d, L = shape.d_model, shape.n_layers
    e = shape.elt_bytes()
    M = B * (K + 1)
    w = shape.n_params() - shape.vocab * d      # all weights but the embedding table
    w_bytes = w * e - (2 * L + 1) * d * (e - 4)  # norm gains are fp32
    kv_read = sum(L * 2 * (int(l) + K + 1) * d * e for l in lens)
    kv_write = B * L * 2 * (K + 1) * d * e
    return w_bytes + M * d * e + kv_read + kv_write + M * shape.vocab * 4


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_round_seconds(wl, K, target_seconds):
    """Seconds of one round of one row for the oracle (numpy, float64) on this host,
    from a bounded sample: one round's work on the first layer of the target and of the
    draft, the LM heads and the accept step, repeated for about target_seconds, the
    per-layer part scaled to the full depth.  Returns (seconds, repetitions)."""
    import dataclasses

    from oracle import model as omodel
    from oracle import philox, sampling
    from speculative_decoding_forward_amd import synth

    t_shape = dataclasses.replace(wl.target, n_layers=1)
    d_shape = dataclasses.replace(wl.draft, n_layers=1)
    Wt = synth.weights_to_numpy(synth.make_weights(t_shape, seed=0, device="cpu"))
    Wd = synth.weights_to_numpy(synth.make_weights(d_shape, seed=0, model_id=1, device="cpu"))
    ctx = wl.ctx

    def cache(shape):
        c = omodel.KVCache(shape, 1, ctx + K + 2)
        fill = synth.kv_fill(shape, 1, ctx + K + 2, ctx, seed=0).float().numpy()
        c.fill(fill, [ctx])
        return c

    tc, dc = cache(t_shape), cache(d_shape)
    rng = np.random.default_rng(0)
    new = rng.integers(0, wl.target.vocab, (1, K + 1))
    reps, t_target, t_draft, t_acc = 0, 0.0, 0.0, 0.0
    t_start = time.perf_counter()
    while reps == 0 or time.perf_counter() - t_start < target_seconds:
        tc.len[:] = ctx
        dc.len[:] = ctx
        t0 = time.perf_counter()
        plog = omodel.forward(t_shape, Wt, tc, new)
        t1 = time.perf_counter()
        qlog = np.concatenate([omodel.forward(d_shape, Wd, dc, new[:, j:j + 1])
                               for j in range(K)], axis=1)
        t2 = time.perf_counter()
        sampling.accept_resample_logits(
            plog[0].astype(np.float32), qlog[0].astype(np.float32), new[0, :K],
            philox.uniform(0, reps, np.arange(K), 0, 1),
            philox.uniform(0, reps, np.arange(K + 1), 0, 2), wl.temperature, wl.top_k,
            wl.top_p)
        t3 = time.perf_counter()
        t_target += t1 - t0
        t_draft += t2 - t1
        t_acc += t3 - t2
        reps += 1
    t_target, t_draft, t_acc = t_target / reps, t_draft / reps, t_acc / reps
    # a 1-layer forward = embed + 1 layer + head; the head-only time separates the part
    # that the layer count multiplies
    tc.len[:] = ctx
    dc.len[:] = ctx
    t0 = time.perf_counter()
    omodel.forward(t_shape, Wt, tc, new, layers=0)
    th = time.perf_counter() - t0
    t0 = time.perf_counter()
    for j in range(K):
        omodel.forward(d_shape, Wd, dc, new[:, j:j + 1], layers=0)
    dh = time.perf_counter() - t0
    return ((t_target - th) * wl.target.n_layers + th +
            (t_draft - dh) * wl.draft.n_layers + dh + t_acc), reps


def cpu_verify_seconds(wl, K):
    """Seconds of one oracle verify forward (K+1 new tokens, one row, at the workload's
    context) and the repetitions behind it: the first layer of the target timed, the
    layer part scaled to the full depth (the tiny model runs whole)."""
    import dataclasses

    from oracle import model as omodel
    from speculative_decoding_forward_amd import synth

    L = wl.target.n_layers
    shape = wl.target if L <= 2 else dataclasses.replace(wl.target, n_layers=1)
    W = synth.weights_to_numpy(synth.make_weights(shape, seed=0, device="cpu"))
    c = omodel.KVCache(shape, 1, wl.ctx + K + 2)
    c.fill(synth.kv_fill(shape, 1, wl.ctx + K + 2, wl.ctx, seed=0).float().numpy(), [wl.ctx])
    new = np.random.default_rng(0).integers(0, shape.vocab, (1, K + 1))
    reps, t = 0, 0.0
    while reps < 2 or (t < 1.0 and reps < 20):
        c.len[:] = wl.ctx
        t0 = time.perf_counter()
        omodel.forward(shape, W, c, new)
        t += time.perf_counter() - t0
        reps += 1
    t /= reps
    if shape is wl.target:
        return t, reps
    c.len[:] = wl.ctx
    t0 = time.perf_counter()
    omodel.forward(shape, W, c, new, layers=0)
    th = time.perf_counter() - t0
    return (t - th) * L + th, reps


def cpu_accept_seconds():
    """Seconds of one oracle accept / resample call over the accept-only workload
    (B = 32 rows, K = 8, V = 32000, T = 0.8)."""
    from oracle import philox, sampling
    from speculative_decoding_forward_amd import synth

    B, K, T = 32, 8, 0.8
    p, q = synth.vocab_logits(0, B, K, 32000, 2.0, 0.5)
    xt = np.zeros((B, K), dtype=np.int64)
    t0 = time.perf_counter()
    for b in range(B):
        sampling.accept_resample_logits(p[b], q[b], xt[b], philox.uniform(0, 0, np.arange(K), b, 1),
                                        philox.uniform(0, 0, np.arange(K + 1), b, 2), T, 0, 1.0)
    return time.perf_counter() - t0


def cpu_items(K=5):
    """The oracle's verify forward per workload and its accept step, on numpy's default
    BLAS threads and on one thread (seconds per call; the 70B and 7B figures scale one
    timed layer to the full depth)."""
    from threadpoolctl import threadpool_limits

    from speculative_decoding_forward_amd import synth

    out = {}
    for threads in ("all", "one"):
        res = {}
        ctx = threadpool_limits(limits=1, user_api="blas") if threads == "one" else None
        try:
            if ctx:
                ctx.__enter__()
            for name in ("tiny", "small", "7b", "70b"):
                wl = synth.WORKLOADS[name]
                s, reps = cpu_verify_seconds(wl, wl.K if name != "7b" else K)
                res[f"verify_{name}_s"] = s
            res["accept_b32_k8_s"] = cpu_accept_seconds()
        finally:
            if ctx:
                ctx.__exit__(None, None, None)
        out[threads] = res
    out["note"] = ("oracle seconds per call: one verify forward over K+1 tokens at each "
                   "workload's context (one row; small, 7B and 70B from one timed layer scaled "
                   "to the full depth), and one accept step over the 32 x 9 x 32000 workload")
    return out


def cpu_baseline(wl, B, K, tokens_per_round, target_seconds):
    """The oracle as it stands timed on this host's cores on a bounded sample of the same
    workload (cpu_round_seconds), twice: with numpy's BLAS on its default threads (the
    value) and on one thread; both scaled to B rows at the GPU's measured tokens per
    round."""
    from threadpoolctl import threadpool_info, threadpool_limits

    blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
    threads = max([p.get("num_threads", 1) for p in blas] or [1])
    half = target_seconds / 2
    s_all, reps_all = cpu_round_seconds(wl, K, half)
    with threadpool_limits(limits=1, user_api="blas"):
        s_one, reps_one = cpu_round_seconds(wl, K, half)
    return {
        "value": tokens_per_round / (s_all * B), "unit": "tokens/s", "cores": threads,
        "kind": "oracle",
        "sample": (f"{reps_all} repetitions of one round's work on 1 target layer + 1 draft "
                   f"layer (+ heads, accept step) at context {wl.ctx}, K={K}, one row; "
                   f"per-layer time scaled to {wl.target.n_layers}+{wl.draft.n_layers} "
                   f"layers and {B} rows; numpy float64 on {threads} BLAS threads; "
                   f"{s_all * B:.2f} s per full round"),
        "single_thread": {"value": tokens_per_round / (s_one * B), "cores": 1,
                          "repetitions": reps_one, "seconds_per_round": s_one * B},
        "cpu_model": cpu_model(),
        "host_cpus_visible": len(os.sched_getaffinity(0)),
    }


def verify_only(args, wl):
    """Target model only: prefill the context, then --steps eager verify passes over K+1
    new tokens per row, each rolled back so every pass sees the same cache length."""
    import torch

    from speculative_decoding_forward_amd import binding, synth

    B = args.batch or wl.batch
    K = args.K or wl.K
    dev = "cuda"
    W = synth.make_weights(wl.target, seed=args.seed, model_id=synth.TARGET, device=dev)
    m = binding.Model(wl.target, W)
    del W
    max_len = wl.ctx + 2 * (K + 1) + 2
    kv = binding.KVCache(wl.target, B, max_len, dev)
    ws = m.workspace(B, 64, max_len, device=dev)
    ctx = synth.context_ids(args.seed, B, wl.ctx, wl.target.vocab)
    lg = torch.empty((B, 64, wl.target.vocab), device=dev)
    for s0 in range(0, wl.ctx, 64):
        tok = torch.from_numpy(np.ascontiguousarray(ctx[:, s0:s0 + 64]).astype(np.int32)).to(dev)
        binding.verify_forward(m, kv, tok, lg[:, :tok.shape[1]].contiguous(), ws)
    torch.cuda.synchronize()
    base = kv.len.clone()
    new = torch.from_numpy(synth.context_ids(args.seed + 1, B, K + 1, wl.target.vocab)
                           .astype(np.int32)).to(dev)
    logits = torch.empty((B, K + 1, wl.target.vocab), device=dev)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        binding.verify_forward(m, kv, new, logits, ws)
        kv.rollback(base)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    print(json.dumps({"mode": "verify-only", "workload": args.workload, "batch": B, "K": K,
                      "passes": args.steps, "ms_per_pass": dt / args.steps * 1e3,
                      "kernel_sources_sha256": gemm_source_hash()}))


def accept_only(args, emit=True):
    """The accept / resample step alone: target logits [B, K+1, V] ~ N(0, 2^2), draft
    logits = target + N(0, 0.5^2), temperature 0.8, top-k and top-p off, draft tokens
    drawn from the processed draft rows (input synthesis, outside the timed region).
    A step is one spec_accept_resample call over the batch; the roofline is that of the
    vocab kernel, which reads every logit row once.  Calls rotate over N_SETS seeded input
    sets (8 x 69.6 MB at the default shape, more than the 256 MB memory-side cache), so
    the rows come from HBM."""
    import torch

    from speculative_decoding_forward_amd import binding, synth

    B = args.batch or 32
    K = args.K or 8
    V = 32000
    knobs = (0.8, 0, 1.0)
    dev = "cuda"
    N_SETS = 8
    sets = []
    g = torch.Generator(device=dev)
    g.manual_seed(args.seed)
    for k in range(N_SETS):
        p, q = synth.vocab_logits(args.seed + k, B, K, V, 2.0, 0.5)
        P = torch.from_numpy(p).to(dev)
        Q = torch.from_numpy(q).to(dev)
        probs = torch.softmax(Q.double() / knobs[0], dim=-1).reshape(B * K, V)
        X = torch.multinomial(probs, 1, generator=g).reshape(B, K).to(torch.int32).contiguous()
        del probs
        sets.append((P, Q, X))
    out = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
    n_out = torch.empty((B,), dtype=torch.int32, device=dev)
    st = torch.empty((B,), dtype=torch.int32, device=dev)
    ws = binding.accept_workspace(B, K)
    for r in range(max(args.warmup, N_SETS)):
        P, Q, X = sets[r % N_SETS]
        binding.accept_resample(P, Q, X, knobs, args.seed, r, out, n_out, st, ws)
    torch.cuda.synchronize()
    n_sum = torch.zeros((B,), dtype=torch.int64, device=dev)
    n_sum += n_out  # the accumulation's first use (kernel code load) before the clock
    n_sum.zero_()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i, (a, b) in enumerate(ev):
        P, Q, X = sets[i % N_SETS]
        a.record(stream)
        binding.accept_resample(P, Q, X, knobs, args.seed, args.warmup + i, out, n_out, st, ws)
        b.record(stream)
        n_sum += n_out
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    call_ms = np.array([a.elapsed_time(b) for a, b in ev])
    tokens = int(n_sum.sum().item())
    assert int((st != 0).sum().item()) == 0
    vb = (B * (K + 1) * V + B * K * V) * 4  # every logit row read once
    c_med = float(np.median(call_ms))
    achieved = vb / (c_med / 1e3) / 1e9
    res = {
        "metric": "accepted tokens/s + vocab-kernel HBM GB/s (% of peak), accept/resample alone",
        "value": tokens / wall, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic: N(0,2^2) target logits, draft = target + N(0,0.5^2), "
                f"{N_SETS} input sets rotated",
        "config": {"workload": "accept/resample alone", "batch": B, "K": K, "vocab": V,
                   "temperature": knobs[0], "top_k": 0, "top_p": 1.0},
        "call_ms_median": c_med,
        "tokens_per_row_per_call": tokens / (B * args.steps),
        "roofline": {"bound": "hbm", "kernel": "k_accept_rows + k_select (one call)",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "bytes_per_call": vb},
    }
    if emit:
        print(json.dumps(res))
    return res


AR_STEPS = 8  # single-token steps per graph of the plain-decoding baseline


def ar_ms_per_token(binding, torch, model, kv, ws, B, V, knobs, seed, tok0, n_rep):
    """Plain autoregressive decoding on the same kernels: a graph of AR_STEPS one-token
    steps of `model` (forward + sample, the draft-step entry point) that rolls the cache
    back at its end, replayed n_rep times between HIP events; returns the median ms per
    token step.  Step 0 runs at two rows (room for two pending tokens), the rest at one."""
    i32 = dict(dtype=torch.int32, device="cuda")
    xt = torch.zeros((B, AR_STEPS), **i32)
    ql = torch.zeros((B, AR_STEPS, V), dtype=torch.float32, device="cuda")
    n_in = torch.ones(B, **i32)
    saved = kv.len.clone()

    def body():
        for j in range(AR_STEPS):
            binding.draft_step(model, kv, tok0, n_in, j, knobs, seed, 0, xt, ql, ws)
        kv.rollback(saved)

    body()  # eager pass: code loading, outside the measurement
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        body()
    g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n_rep)]
    for a, b in ev:
        a.record(stream)
        g.replay()
        b.record(stream)
    torch.cuda.synchronize()
    assert torch.equal(kv.len, saved)
    return float(np.median([a.elapsed_time(b) for a, b in ev])) / AR_STEPS


def speedup_formula(alpha, K, c):
    """Expected wall-time improvement ([LENS] "How much faster in practice?")."""
    e = (1 - alpha ** (K + 1)) / (1 - alpha) if alpha < 1 else K + 1
    return e / (K * c + 1)


def sweep(args):
    """Where speculation stops paying and which K is best, per batch size: the 7B-shape
    models built once, one prefilled context per batch size, and for every K a fresh
    round driver on the same caches rolled back to the context.  Each point: graph-
    replayed rounds timed as in the main bench, alpha, plain decoding at that batch size,
    and the tokens/s the measured round time would give at the pages' alpha = 0.8."""
    import torch

    from speculative_decoding_forward_amd import binding, rounds, synth

    wl = synth.WORKLOADS["7b"]
    knobs = (wl.temperature, wl.top_k, wl.top_p)
    V = wl.target.vocab
    Bs = [int(x) for x in args.sweep_batches.split(",")]
    Ks = [int(x) for x in args.sweep_K.split(",")]
    Wt = synth.make_weights(wl.target, seed=args.seed, model_id=synth.TARGET, device="cuda")
    Wd = synth.make_weights(wl.draft, seed=args.seed, model_id=synth.DRAFT, device="cuda")
    tm, dm = binding.Model(wl.target, Wt), binding.Model(wl.draft, Wd)
    del Wt, Wd
    torch.cuda.empty_cache()
    warm, steps = 2, args.steps
    summary = []
    for B in Bs:
        max_len = wl.ctx + (warm + steps + 3) * (max(Ks) + 1) + AR_STEPS
        caches = (binding.KVCache(wl.target, B, max_len), binding.KVCache(wl.draft, B, max_len))
        ctx = synth.context_ids(args.seed, B, wl.ctx, V)
        base = rounds.SpecDecoder(wl.target, None, wl.draft, None, B, 1, max_len, knobs,
                                  seed=args.seed, models=(tm, dm), caches=caches)
        base.prefill(ctx)
        torch.cuda.synchronize()
        lt0, ld0 = caches[0].len.clone(), caches[1].len.clone()
        tok0 = base.pending.clone()
        t_ar = ar_ms_per_token(binding, torch, tm, caches[0], base.ws_t, B, V, knobs, args.seed,
                               tok0, 6)
        d_ar = ar_ms_per_token(binding, torch, dm, caches[1], base.ws_d, B, V, knobs, args.seed,
                               tok0, 6)
        ar_tps = B / (t_ar / 1e3)
        pts = []
        for K in Ks:
            caches[0].len.copy_(lt0)
            caches[1].len.copy_(ld0)
            dec = rounds.SpecDecoder(wl.target, None, wl.draft, None, B, K, max_len, knobs,
                                     seed=args.seed, models=(tm, dm), caches=caches)
            dec.pending.copy_(tok0)
            dec.n_pending.fill_(1)
            for r in range(warm):
                dec.step(r)
            dec.set_round(warm)
            dec.capture()
            n_hist = torch.zeros((steps, B), dtype=torch.int32, device="cuda")
            dec.replay()
            n_hist[0] += dec.n_out
            n_hist.zero_()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i in range(steps):
                dec.replay()
                n_hist[i] += dec.n_out
            torch.cuda.synchronize()
            wall = time.perf_counter() - t0
            hist = n_hist.cpu().numpy().astype(np.int64)
            assert hist.min() >= 1
            acc = hist - 1
            alpha = acc.sum() / max(1, acc.sum() + (acc < K).sum())
            round_s = wall / steps
            e08 = (1 - 0.8 ** (K + 1)) / (1 - 0.8)
            pt = {"sweep_point": True, "batch": B, "K": K, "tokens_per_s": hist.sum() / wall,
                  "ms_per_round": round_s * 1e3, "tokens_per_round_per_row": hist.mean(),
                  "alpha_measured": float(alpha), "autoregressive_tokens_per_s": ar_tps,
                  "c_measured": d_ar / t_ar,
                  "speedup_measured": hist.sum() / wall / ar_tps,
                  "speedup_formula": speedup_formula(float(alpha), K, d_ar / t_ar),
                  "projected_at_alpha_0.8_tokens_per_s": B * e08 / round_s,
                  "projected_speedup_at_alpha_0.8": B * e08 / round_s / ar_tps}
            print(json.dumps(pt), flush=True)
            pts.append(pt)
            del dec
        c = d_ar / t_ar
        best_formula_K = max(range(1, 17), key=lambda k: speedup_formula(0.8, k, c))
        best = max(pts, key=lambda q: q["projected_at_alpha_0.8_tokens_per_s"])
        summary.append({"batch": B, "autoregressive_tokens_per_s": ar_tps, "c_measured": c,
                        "best_K_at_alpha_0.8": best["K"],
                        "best_projected_speedup_at_alpha_0.8":
                            best["projected_speedup_at_alpha_0.8"],
                        "formula_best_K_at_alpha_0.8_and_measured_c": best_formula_K,
                        "pays_at_alpha_0.8": best["projected_speedup_at_alpha_0.8"] > 1.0,
                        "best_measured_K": max(pts, key=lambda q: q["tokens_per_s"])["K"],
                        "best_measured_speedup": max(q["speedup_measured"] for q in pts)})
        del base, caches
        torch.cuda.empty_cache()
    print(json.dumps({"sweep_summary": summary, "workload": "7b-shape, context 2048, T=0.8, "
                      "top-p 0.95, random-init models"}))


def device_copy_GBps(mib=1024, reps=10):
    """Context for the roofline: the HBM rate of torch's device-to-device copy of `mib` MiB
    (bytes read + bytes written over the median event-timed copy)."""
    import torch

    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for a, b in ev:
        a.record()
        dst.copy_(src)
        b.record()
    torch.cuda.synchronize()
    ms = float(np.median([a.elapsed_time(b) for a, b in ev]))
    del src, dst
    torch.cuda.empty_cache()
    return 2 * n * 4 / (ms / 1e3) / 1e9


def build_models(wl, seed, dev="cuda"):
    """Target and draft of a workload, each tensor generated on the device, loaded into
    the model's store and released (peak memory: the stores plus one tensor)."""
    import torch

    from speculative_decoding_forward_amd import binding, synth

    models = []
    for shape, mid in ((wl.target, synth.TARGET), (wl.draft, synth.DRAFT)):
        m = binding.Model(shape, None, device=dev)
        for nm in shape.weight_names():
            w = synth.make_weight(shape, nm, seed=seed, model_id=mid, device=dev)
            m.load_weight(nm, w)
            del w
        models.append(m)
    torch.cuda.synchronize()
    return models


def run_rounds(wl, B, K, steps, warmup, seed, models, timed_extra=0, with_ar=True,
               gemm_timing=True):
    """Speculative rounds of a workload on one GPU: prefill, `warmup` eager rounds, one
    round captured as a HIP graph and replayed `steps` times between two synchronisations
    (the timed region), then -- outside it -- the verify pass alone, the verify GEMMs'
    and attention's event-timed launches, plain decoding on the same kernels, and
    `timed_extra` more replays for a steadier tokens/s.  Returns the measurements."""
    import torch

    from speculative_decoding_forward_amd import binding, rounds, synth

    knobs = (wl.temperature, wl.top_k, wl.top_p)
    dev = "cuda"
    rounds_total = warmup + 1 + steps + timed_extra
    max_len = wl.ctx + (rounds_total + 1) * (K + 1) + 2 + AR_STEPS
    dec = rounds.SpecDecoder(wl.target, None, wl.draft, None, B, K, max_len, knobs, seed=seed,
                             models=models)
    ctx = synth.context_ids(seed, B, wl.ctx, wl.target.vocab)
    dec.prefill(ctx)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    for r in range(warmup):
        dec.step(r)
    torch.cuda.synchronize()
    # one round captured as a HIP graph, numbered by the device round counter; one replay
    # and the token accumulation run once before the clock starts (a kernel's first use
    # loads its code, which is not part of a round); per-round counts land in row i of
    # n_hist (one elementwise add per round)
    dec.set_round(warmup)
    dec.capture()
    n_hist = torch.zeros((steps + timed_extra, B), dtype=torch.int32, device=dev)
    dec.replay()
    n_hist[0] += dec.n_out
    n_hist.zero_()
    len_start = dec.tkv.len.cpu().numpy().astype(np.float64)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        dec.replay()
        n_hist[i] += dec.n_out
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    len_end = dec.tkv.len.cpu().numpy().astype(np.float64)
    extra = None
    if timed_extra:
        t1 = time.perf_counter()
        for i in range(steps, steps + timed_extra):
            dec.replay()
            n_hist[i] += dec.n_out
        torch.cuda.synchronize()
        extra = time.perf_counter() - t1
    hist_all = n_hist.cpu().numpy().astype(np.int64)
    if timed_extra:
        extra = {"rounds": timed_extra, "tokens": int(hist_all[steps:].sum()),
                 "tokens_per_s": float(hist_all[steps:].sum() / extra)}
    hist = hist_all[:steps]
    assert hist_all.min() >= 1, "a row emitted nothing (row status set)"
    tokens = int(hist.sum())

    # verify-pass latency: a graph of [verify-input assembly, verify pass] replayed with
    # events around each replay, and after each, outside the events, a graph rolling the
    # cache back to the pre-verify lengths
    saved_len = dec.tkv.len.clone()
    vg = torch.cuda.CUDAGraph()
    with torch.cuda.graph(vg):
        dec.verify_phase()
    rg = torch.cuda.CUDAGraph()
    with torch.cuda.graph(rg):
        dec.tkv.rollback(saved_len)
    dec.tkv.rollback(saved_len)
    vg.replay()
    rg.replay()
    torch.cuda.synchronize()
    n_v = max(10, min(64, steps))
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n_v)]
    for a, b in ev:
        a.record(stream)
        vg.replay()
        b.record(stream)
        rg.replay()
    torch.cuda.synchronize()
    verify_ms = np.array([a.elapsed_time(b) for a, b in ev])
    lens_v = saved_len.cpu().numpy().astype(np.float64)
    out = {}
    if gemm_timing:
        # the verify pass's weight-streaming GEMMs and attention, timed by HIP events
        # attached to their own dispatch packets over eager verify passes
        n_meas = max(4, min(20, steps // 2))
        torch.cuda.synchronize()
        binding.timing_enable(True)
        binding.timing_read()
        for _ in range(n_meas):
            dec.verify_phase()
            dec.tkv.rollback(saved_len)
        torch.cuda.synchronize()
        binding.timing_enable(False)
        gemm_ms, gemm_n, attn_ms, attn_n = binding.timing_read()
        gb_v, gn_v = gemm_bytes_per_verify(wl.target, B * (K + 1))
        assert gemm_n == n_meas * gn_v, (gemm_n,)
        gemm_avg_s = gemm_ms / 1e3 / gemm_n
        achieved = gb_v / gn_v / gemm_avg_s / 1e9
        out.update(gemm_avg_bytes=gb_v / gn_v, gemm_avg_s=gemm_avg_s, gemm_achieved=achieved,
                   gemm_n=gemm_n, gemm_ms_per_pass=gemm_ms / n_meas,
                   attn_ms_per_pass=attn_ms / n_meas,
                   attn_kv_GBps=sum(wl.target.n_layers * 2 * (l + K + 1) * wl.target.d_model *
                                    wl.target.elt_bytes() for l in lens_v) / (attn_ms / n_meas / 1e3) / 1e9)
    acc_counts = hist - 1
    accepted = int(acc_counts.sum())
    rejections = int((acc_counts < K).sum())
    alpha_hat = accepted / max(1, accepted + rejections)
    e_tokens_iid = (1 - alpha_hat ** (K + 1)) / (1 - alpha_hat) if alpha_hat < 1 else K + 1
    vb = verify_bytes(wl.target, B, K, lens_v)
    v_med = float(np.median(verify_ms))
    out.update(tokens=tokens, wall=wall, hist=hist, len_start=len_start, len_end=len_end,
               verify_ms=verify_ms, v_med=v_med, vb=vb, alpha=alpha_hat, e_iid=e_tokens_iid,
               extra=extra)
    if with_ar:
        tok0 = torch.full((B, 2), -1, dtype=torch.int32, device=dev)
        tok0[:, 0] = dec.pending[:, 0]
        n_ar = max(6, min(steps, 20))
        t_ar = ar_ms_per_token(binding, torch, dec.target, dec.tkv, dec.ws_t, B,
                               wl.target.vocab, knobs, seed, tok0, n_ar)
        d_ar = ar_ms_per_token(binding, torch, dec.draft, dec.dkv, dec.ws_d, B,
                               wl.target.vocab, knobs, seed, tok0, n_ar)
        out.update(t_ar=t_ar, d_ar=d_ar, ar_bytes=verify_bytes(wl.target, B, 0, len_end))
    del dec, vg, rg
    torch.cuda.empty_cache()
    return out


def summary_line(wl, B, K, r, steps):
    """The compact per-workload figures of a run_rounds() result."""
    d = {"workload": wl.name, "batch": B, "K": K, "context": wl.ctx,
         "tokens_per_s": r["tokens"] / r["wall"], "ms_per_round": r["wall"] / steps * 1e3,
         "rounds": steps, "alpha_measured": r["alpha"],
         "tokens_per_round_per_row": r["tokens"] / (B * steps),
         "verify_ms_median": r["v_med"], "verify_bytes": r["vb"],
         "verify_frac_of_peak": r["vb"] / (r["v_med"] / 1e3) / 1e9 / HBM_PEAK_GBS}
    if "gemm_achieved" in r:
        d.update(gemm_GBps=r["gemm_achieved"], gemm_frac_of_peak=r["gemm_achieved"] / HBM_PEAK_GBS,
                 gemm_avg_launch_us=r["gemm_avg_s"] * 1e6,
                 attention_ms_per_pass=r["attn_ms_per_pass"],
                 attention_frac_of_peak=r["attn_kv_GBps"] / HBM_PEAK_GBS)
    if "t_ar" in r:
        c = r["d_ar"] / r["t_ar"]
        d.update(autoregressive_tokens_per_s=B / (r["t_ar"] / 1e3), c_measured=c,
                 speedup_measured=(r["tokens"] / r["wall"]) / (B / (r["t_ar"] / 1e3)),
                 speedup_formula=speedup_formula(r["alpha"], K, c))
    e08 = (1 - 0.8 ** (K + 1)) / (1 - 0.8)
    d["projected_tokens_per_s_at_alpha_0.8"] = B * e08 / (r["wall"] / steps)
    return d


def guarded(fn, *a, **kw):
    """A summary that must never cost the headline line: its result, or its error."""
    import torch
    try:
        return fn(*a, **kw)
    except Exception as exc:  # noqa: BLE001 -- reported in the JSON line
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        return {"error": f"{type(exc).__name__}: {exc}"[:300]}


def workload_summary(name, B, K, steps, warmup, seed):
    import torch

    from speculative_decoding_forward_amd import synth

    wl = synth.WORKLOADS[name]
    models = build_models(wl, seed)
    r = run_rounds(wl, B, K, steps, warmup, seed, models, gemm_timing=wl.target.dtype == "bf16")
    del models
    gc.collect()
    torch.cuda.empty_cache()
    return summary_line(wl, B, K, r, steps)


def accept_summary(seed):
    class A:
        pass
    a = A()
    a.batch, a.K, a.seed, a.steps, a.warmup = None, None, seed, 200, 3
    return accept_only(a, emit=False)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the path "
              "shards by batch row with no exchange, so run one process per GPU.",
              file=sys.stderr)
        sys.exit(2)
    import torch

    from speculative_decoding_forward_amd import synth

    assert torch.cuda.is_available(), "no GPU"
    if args.calibrate_copy:
        n = args.calibrate_copy * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_read": n * 4, "bytes_written": n * 4}))
        return
    if args.workload == "accept":
        accept_only(args)
        return
    if args.sweep:
        sweep(args)
        return
    wl = synth.WORKLOADS[args.workload]
    if args.verify_only:
        verify_only(args, wl)
        return
    B = args.batch or wl.batch
    K = args.K or wl.K
    torch.manual_seed(args.seed)
    models = build_models(wl, args.seed)
    r = run_rounds(wl, B, K, args.steps, args.warmup, args.seed, models, timed_extra=200,
                   gemm_timing=wl.target.dtype == "bf16")
    tokens, wall = r["tokens"], r["wall"]
    round_s = wall / args.steps
    t_ar, d_ar = r["t_ar"], r["d_ar"]
    c_hat = d_ar / t_ar
    ar_tps = B / (t_ar / 1e3)
    formula = r["e_iid"] / (K * c_hat + 1)
    e08 = (1 - 0.8 ** (K + 1)) / (1 - 0.8)
    vb, v_med, verify_ms = r["vb"], r["v_med"], r["verify_ms"]
    res = {
        "metric": "accepted tokens/s + verify-pass HBM GB/s (% of peak), 7B-shape bf16, K=5",
        "value": tokens / wall,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.target.dtype == "bf16" else "f32",
        "data": "synthetic: seeded random-init weights (N(0,0.02^2)), uniform context ids",
        "config": {"workload": f"{args.workload}-shape speculative rounds: target "
                               f"L{wl.target.n_layers} d{wl.target.d_model} F{wl.target.d_ffn} "
                               f"{wl.target.ffn_kind} V{wl.target.vocab}, draft "
                               f"L{wl.draft.n_layers} d{wl.draft.d_model} F{wl.draft.d_ffn}",
                   "batch": B, "K": K, "context": wl.ctx, "temperature": wl.temperature,
                   "top_p": wl.top_p, "parallelism": "1 GPU"},
        "verify_ms_median": v_med,
        "verify_ms_p10_p90": [float(np.percentile(verify_ms, 10)),
                              float(np.percentile(verify_ms, 90))],
        "verify_GBps": vb / (v_med / 1e3) / 1e9,
        "verify_frac_of_peak": vb / (v_med / 1e3) / 1e9 / HBM_PEAK_GBS,
        "verify_bytes": vb,
        "tokens_per_round_per_row": tokens / (B * args.steps),
        "alpha_measured": r["alpha"],
        "tokens_per_round_at_alpha_iid": r["e_iid"],
        "autoregressive": {
            "what": "plain decoding on the same kernels: one-token target steps (forward + "
                    "sample), graph of 8 steps, median of HIP-event-timed replays",
            "target_ms_per_token": t_ar, "tokens_per_s": ar_tps,
            "draft_ms_per_token": d_ar, "c_measured": c_hat,
            "speedup_measured": (tokens / wall) / ar_tps,
            "speedup_formula_at_measured_alpha_c": formula,
            "bandwidth_ceiling_tokens_per_s": B * HBM_PEAK_GBS * 1e9 / r["ar_bytes"],
            "bytes_per_token_step": r["ar_bytes"],
        },
        "projected_at_alpha_0.8": {
            "note": "context, not measured: the measured round time with the tokens per "
                    "round that alpha = 0.8 would give",
            "tokens_per_s": B * e08 / round_s,
            "speedup_vs_measured_autoregressive": B * e08 / round_s / ar_tps,
        },
        "verify_attention_ms": r["attn_ms_per_pass"],
        "verify_attention_frac_of_peak": r["attn_kv_GBps"] / HBM_PEAK_GBS,
        "verify_gemm_ms": r["gemm_ms_per_pass"],
        "roofline": {"bound": "hbm",
                     "kernel": "k_gemm_bf16 (verify-pass weight-streaming GEMM, 4 per layer "
                               "+ LM head)",
                     "achieved": r["gemm_achieved"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": r["gemm_achieved"] / HBM_PEAK_GBS, "traffic": recorded_traffic(),
                     "bytes_per_launch": r["gemm_avg_bytes"],
                     "avg_launch_us": r["gemm_avg_s"] * 1e6, "launches": r["gemm_n"],
                     "kernel_sources_sha256": gemm_source_hash()},
    }
    res["device_copy_GBps"] = guarded(device_copy_GBps)
    if r["extra"]:
        res["tokens_per_s_over_more_rounds"] = dict(
            r["extra"], note="context: the same graph replayed right after the timed rounds "
                             "(tokens per round vary round to round at B = 1)")
    if not args.no_summaries and args.workload == "7b" and B == 1:
        # batch 8 on the same models (its rows add KV reads and GEMM rows, not weights)
        res["b8"] = guarded(lambda: summary_line(wl, 8, K, run_rounds(
            wl, 8, K, max(20, args.steps), 2, args.seed, models), max(20, args.steps)))
        # the other draft lengths of the headline workload, batch 1, on the same models
        n_k = max(20, min(args.steps, 60))
        res["other_K"] = {f"K{k}": guarded(lambda k=k: summary_line(
            wl, 1, k, run_rounds(wl, 1, k, n_k, 2, args.seed, models), n_k)) for k in (3, 7)}
    del models
    gc.collect()
    torch.cuda.empty_cache()
    if not args.no_summaries and args.workload == "7b" and B == 1:
        res["other_configs"] = {
            "tiny": guarded(workload_summary, "tiny", 1, 4, 32, 2, args.seed),
            "small": guarded(workload_summary, "small", 1, 4, 100, 2, args.seed),
            "accept": guarded(accept_summary, args.seed),
            "70b": guarded(workload_summary, "70b", 1, 4, 20, 2, args.seed),
        }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl, B, K, tokens / args.steps, args.cpu_seconds)
        if not args.no_summaries:
            res["cpu_baseline"]["per_call"] = guarded(cpu_items, K)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
