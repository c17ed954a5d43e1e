#!/usr/bin/env python3
"""Decode benchmark of the routed-expert MoE layer on one MI355X.

Workload (default): 48 MoE layers of 512 experts, top-8, hidden 2048, expert
FFN 1024, 4-bit blocks; batch-1 decode over 256 steps with Zipf(1.1) expert
popularity; an HBM pool of 256 slots per layer (half the experts) seeded from
a routing-frequency table; cold experts read zero-copy from pinned host RAM;
the cache step runs between decode steps.

A step is one decode token through all 48 layers (routing, lookup + stamps +
miss record, gate/up GEMV + SwiGLU, down GEMV + weighted combine added into
a residual buffer), followed by the host cache step (promotions). Every
(step, layer) has its own N(0, 1) input, as the router logits are drawn
independently of the activations; inputs of 32 distinct steps are resident
in HBM and reused cyclically (the logits of all 256 steps are resident). The
timed region replays a HIP graph of the 48-layer forward per step.

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0      # MI355X HBM3E
# HBM bytes per launch of the roofline kernel (gemv_route_gateup_kernel<64,1,4,1>, hot picks), from two rocprofv3
# counter runs (FETCH_SIZE x2.0 + WRITE_SIZE x1.0, scaled by a 1 GiB copy) over launches that served 7.167 hot picks
# each (16.91 MB algorithmic); the summary and commands are under profiles/. Set to None when the kernel changes.
ROOFLINE_TRAFFIC = {"bytes_per_launch": 17120226, "algorithmic_bytes_per_launch": 16908288}
PCIE_PEAK_GBPS = 64.0       # PCIe Gen5 x16, one direction
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA; fp16 (what the grouped GEMM runs) has the same rate
METRIC = "MoE-layer decode tokens/s + effective weight GB/s vs HBM/PCIe roofline"
# decode batches of 1..7 tokens: 1 = one launch per layer where the shape allows it, 2 = two launches
DECODE_LAUNCHES = 2


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def setup_ctx(moe, wl, slots, stream, host_alloc, layers=None, progress=True, capture_picks=None, pool="layer",
              max_prefill_tokens=0, swaps=(0, 0), cold_exec=0, cpu_threads=0, budget=None, reserve=0, timing=None):
    """slots per layer; pool="global" gives one pool of the same total size to all layers. budget/reserve:
    the pool's capacity rule instead (budget -1: free HBM minus reserve; both: the smaller). timing: a dict
    that receives the seconds spent creating the context (pinning the host arena, allocating the pool) and
    registering the weights (generating them, repacking into pinned memory)."""
    from workload import frequency_table, layer_weights

    L = wl.n_layers if layers is None else layers
    t0 = time.time()
    ctx = moe.moe_create(L, wl.n_experts, wl.top_k, wl.hidden, wl.ffn,
                         pool_budget_bytes=L * slots * wl.expert_bytes if budget is None else int(budget),
                         reserve_bytes=int(reserve), window_tokens=wl.window,
                         admit_misses=wl.admit_misses, max_batch_tokens=wl.tokens,
                         max_prefill_tokens=max_prefill_tokens, host_alloc=host_alloc,
                         host_sets=min(wl.weight_layers, L), stream=stream, capture_picks=capture_picks,
                         pool_mode=moe.MOE_POOL_GLOBAL if pool == "global" else moe.MOE_POOL_PER_LAYER,
                         swaps_per_step=swaps[0], swap_lead=swaps[1], cold_exec=cold_exec, cpu_threads=cpu_threads,
                         decode_launches=DECODE_LAUNCHES)
    t1 = time.time()
    buf = None
    gen_s = 0.0
    for layer in range(min(wl.weight_layers, L)):  # layer l reads host set l % weight_layers
        tg = time.time()
        buf = layer_weights(wl, layer, out=buf)
        gen_s += time.time() - tg
        moe.moe_register_layer(ctx, layer, *buf)
        if progress and (layer % 8 == 7 or layer == min(wl.weight_layers, L) - 1):
            log(f"registered host set {layer + 1}/{min(wl.weight_layers, L)} ({time.time() - t1:.1f} s)")
    if timing is not None:
        info = moe.moe_get_info(ctx)
        timing.update(create_s=round(t1 - t0, 2), register_s=round(time.time() - t1 - gen_s, 2),
                      generate_weights_s=round(gen_s, 2), pinned_GB=round(info["host_bytes"] / 1e9, 2),
                      pool_GB=round(info["pool_bytes"] / 1e9, 2))
    freq = frequency_table(wl)[:L]
    return ctx, freq


def run_steps(moe, ctx, n, step_fn, stats_acc=None):
    for i in range(n):
        step_fn(i)
        st = moe.moe_cache_step(ctx)
        if stats_acc is not None:
            for k_, v in st.items():
                stats_acc[k_] = stats_acc.get(k_, 0) + v


def kernel_pass(moe, torch, wl, slots, layers, steps, stream, host_alloc, logits_all, x_all, capture_picks=None):
    """Time the forward kernels on a small context (all hot or all cold)."""
    ctx, freq = setup_ctx(moe, wl, slots, stream, host_alloc, layers=layers, progress=False,
                          capture_picks=capture_picks)
    moe.moe_seed(ctx, freq)
    T, H = wl.tokens, wl.hidden
    res = torch.empty((T, H), dtype=torch.float32, device="cuda")
    with torch.cuda.stream(stream):
        moe.moe_profile(ctx, 1)

        def step(i):
            res.zero_()
            for layer in range(layers):
                moe.moe_forward(ctx, layer, T, x_all[i % x_all.shape[0], layer], logits_all[i % wl.steps, layer], res,
                                flags=moe.MOE_ACCUMULATE)

        run_steps(moe, ctx, steps, step)
        prof = moe.moe_profile(ctx, 0)
    moe.moe_destroy(ctx)
    return prof


PREFILL_WORKLOADS = ("prefill-e512k8-h2048f1024-t4096", "large-e256k8-h4096f1536-t12288")


def fp16_gemm_ceiling(torch, n=8192, reps=20):
    """TFLOP/s of a plain fp16 n^3 GEMM by the vendor library (hipBLASLt through torch.matmul): the matrix
    rate this chip sustains under a GEMM load, at the clock it holds there. A reference beside the spec peak,
    not part of the MoE path."""
    a = torch.randn(n, n, dtype=torch.float16, device="cuda")
    b = torch.randn(n, n, dtype=torch.float16, device="cuda")
    for _ in range(3):
        a @ b
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        a @ b
    torch.cuda.synchronize()
    return 2.0 * n ** 3 * reps / (time.perf_counter() - t0) / 1e12


def prefill_cpu_baseline(wl, weights, x_np, z_np, seconds):
    """The oracle on the host cores over the first tokens of the same prompt, same layer (fp64)."""
    import numpy as np

    import oracle

    oracle.lib()
    g, u, d = weights
    threads = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
    spent, tokens, chunk = 0.0, 0, 16
    while spent < seconds and tokens < wl.tokens:
        xs = x_np[tokens:tokens + chunk].astype(np.float64)
        zs = np.ascontiguousarray(z_np[tokens:tokens + chunk])
        ids, _ = oracle.route(zs, wl.top_k)
        experts = {int(e): (g[e], u[e], d[e]) for e in np.unique(ids)}
        t0 = time.perf_counter()
        oracle.moe_layer(wl.n_experts, wl.top_k, wl.hidden, wl.ffn, experts, xs, logits=zs)
        spent += time.perf_counter() - t0
        tokens += xs.shape[0]
    return dict(value=round(tokens / spent, 2), unit="tokens/s", cores=threads, kind="oracle",
                sample=f"first {tokens} of the {wl.tokens} prompt tokens through the layer (fp64 oracle, "
                       f"{spent:.1f} s of oracle time)")


def _timed_prefill(moe, torch, wl, stream, host_alloc, slots, x, z, weights, reps):
    """Mean time and kernel profile of `reps` prompt passes of layer 0 with `slots` pool slots."""
    from workload import frequency_table

    T = wl.tokens
    ctx = moe.moe_create(1, wl.n_experts, wl.top_k, wl.hidden, wl.ffn, pool_budget_bytes=slots * wl.expert_bytes,
                         max_batch_tokens=1, max_prefill_tokens=T, host_alloc=host_alloc, host_sets=1, stream=stream)
    moe.moe_register_layer(ctx, 0, *weights)
    moe.moe_seed(ctx, frequency_table(wl))
    y = torch.empty_like(x)
    with torch.cuda.stream(stream):
        moe.moe_prefill(ctx, 0, T, x, z, y)  # warm-up
        moe.moe_profile(ctx, 1)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            moe.moe_prefill(ctx, 0, T, x, z, y)
        torch.cuda.synchronize()
        elapsed = (time.perf_counter() - t0) / reps
        prof = moe.moe_profile(ctx, 0)
    moe.moe_destroy(ctx)
    n = max(prof["prefill_passes"], 1)
    return elapsed, {k_: v_ / n for k_, v_ in prof.items() if k_.startswith("prefill_")}


def prefill_pass(moe, torch, wl, stream, host_alloc, reps=3, gemm_ceiling=None, cpu_seconds=0.0):
    """A prompt pass of one layer at the workload's pool share, end to end, with the roofline of what bounds
    it: the staging copy of the non-resident experts over PCIe, or the grouped GEMMs. The GEMMs are also timed
    alone, in the same pass with every expert resident: in the staged pass they run beside the gather kernel,
    whose PCIe reads hold up the memory pipelines of the CUs they share, so their launch times there are not
    their own."""
    import numpy as np

    from workload import activations, layer_weights, zipf_logits

    T, H, F, E = wl.tokens, wl.hidden, wl.ffn, wl.n_experts
    weights = layer_weights(wl, 0)
    x_np = activations(wl, 0, tokens=T)
    z_np = np.ascontiguousarray(zipf_logits(wl, steps=1, tokens=T)[0, 0])
    x = torch.from_numpy(x_np).cuda()
    z = torch.from_numpy(z_np).cuda()
    elapsed, prof = _timed_prefill(moe, torch, wl, stream, host_alloc, wl.slots, x, z, weights, reps)
    alone_s, alone = _timed_prefill(moe, torch, wl, stream, host_alloc, E, x, z, weights, reps)
    pairs = prof["prefill_pairs"]
    staged_bytes = prof["prefill_staged"] * wl.expert_bytes
    prep_ms, gu_ms, dn_ms = alone["prefill_prep_ms"], alone["prefill_gateup_ms"], alone["prefill_down_ms"]
    tflops = 6.0 * pairs * H * F / ((prep_ms + gu_ms + dn_ms) * 1e-3) / 1e12
    gemm_roofline = {"bound": "mfma", "achieved": round(tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel": "grouped_gemm_kernel (gate/up + down, fp16 MFMA; time includes the scale "
                               "transposition before them; timed with every expert resident), algorithmic "
                               "flops 6*H*F per pair",
                     "mfma_flops_per_algorithmic_flop": 1,
                     "measured_fp16_gemm_ceiling": gemm_ceiling and round(gemm_ceiling, 1),
                     "frac_of_measured_ceiling": gemm_ceiling and round(tflops / gemm_ceiling, 4)}
    staging_gbps = staged_bytes / elapsed / 1e9
    stage_ms = prof["prefill_stage_ms"]
    pcie_ceiling = moe.moe_measure_read_bandwidth(None, 1 << 30, reps=3, host_coherent=True)
    if staged_bytes / (pcie_ceiling * 1e9) > 0.5 * elapsed and stage_ms > 0:
        copy_gbps = staged_bytes / (stage_ms * 1e-3) / 1e9
        roofline = {"bound": "pcie", "achieved": round(copy_gbps, 2), "peak": PCIE_PEAK_GBPS, "unit": "GB/s",
                    "frac": round(copy_gbps / PCIE_PEAK_GBPS, 4), "traffic": None,
                    "kernel": "stage_experts_kernel (the staged experts read zero-copy over PCIe into HBM, in "
                              "chunks on a stream of its own): staged bytes / the staging span on that stream, "
                              "start of the first chunk to end of the last",
                    "stage_ms": round(stage_ms, 3),
                    "measured_zero_copy_ceiling": round(pcie_ceiling, 2),
                    "frac_of_measured_ceiling": round(copy_gbps / pcie_ceiling, 4),
                    "whole_pass_GBps": round(staging_gbps, 2)}
    else:
        roofline = gemm_roofline
    return {
        "workload": wl.name, "tokens_per_s": round(T / elapsed, 1), "ms_per_pass": round(elapsed * 1e3, 3),
        "staged_experts": int(prof["prefill_staged"]), "staged_GB": round(staged_bytes / 1e9, 3),
        "staging_GBps": round(staging_gbps, 2), "tiles": int(prof["prefill_tiles"]),
        "gemm_alone": {"ms_per_pass": round(alone_s * 1e3, 3), "scale_transpose_ms": round(prep_ms, 4),
                       "gateup_gemm_ms": round(gu_ms, 4), "down_gemm_ms": round(dn_ms, 4),
                       "roofline": gemm_roofline},
        "roofline": roofline,
        "cpu_baseline": prefill_cpu_baseline(wl, weights, x_np, z_np, cpu_seconds) if cpu_seconds > 0 else None,
    }


def request_pass(moe, torch, ctx, wl, freq, stream, prompt_tokens, decode_tokens, replay, xs, x_all):
    """A prompt pass through every layer, then decode tokens, without and with preheat.

    The request's expert popularity is the workload's Zipf law over a fresh
    permutation (epoch 1), which the seeding frequency table (epoch 0) has not
    seen; prompt and decode are one run of token clocks of that law. Each
    variant starts from the seeded pool. With preheat, every layer's prompt
    pass is followed by moe_preheat of that layer (at most the layer's slot
    share). Decode replays the same forward as the main timed region.
    """
    import numpy as np

    from workload import activations, zipf_logits

    P, D, L, E = prompt_tokens, decode_tokens, wl.n_layers, wl.n_experts
    wr = wl.with_(epoch_base=1)
    xp = torch.from_numpy(activations(wr, 0, tokens=P)).cuda()  # one prompt input serves every layer
    yp = torch.empty_like(xp)
    zp = torch.empty((L, P, E), dtype=torch.float32, device="cuda")
    zd = torch.empty((D, L, 1, E), dtype=torch.float32, device="cuda")
    for layer in range(L):
        lz = zipf_logits(wr, layers=[layer], steps=1, tokens=P + D)[0, 0]
        zp[layer].copy_(torch.from_numpy(lz[:P]))
        zd[:, layer, 0].copy_(torch.from_numpy(np.ascontiguousarray(lz[P:])))
    x_steps = x_all.shape[0]
    out = {"prompt_tokens": P, "decode_tokens": D,
           "popularity": f"Zipf({wl.zipf_s}) over a permutation the frequency table has not seen"}
    with torch.cuda.stream(stream):
        for preheat in (False, True):
            moe.moe_seed(ctx, freq)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            t_pre, admitted = 0.0, 0
            for layer in range(L):
                moe.moe_prefill(ctx, layer, P, xp, zp[layer], yp)  # synchronises
                if preheat:
                    t1 = time.perf_counter()
                    admitted += moe.moe_preheat(ctx, layer, wl.slots)
                    t_pre += time.perf_counter() - t1
            prompt_s = time.perf_counter() - t0
            acc = {}
            torch.cuda.synchronize()
            t2 = time.perf_counter()
            run_steps(moe, ctx, D, lambda i: (xs.copy_(x_all[i % x_steps]), replay(zd[i])), acc)
            torch.cuda.synchronize()
            dec_s = time.perf_counter() - t2
            r = {"decode_tokens_per_s": round(D / dec_s, 2), "hit_rate": round(
                acc["hits"] / max(acc["hits"] + acc["misses"], 1), 4),
                 "admissions_per_step": round(acc["admissions"] / D, 3),
                 "prompt_tokens_per_s": round(P / prompt_s, 1), "prompt_s": round(prompt_s, 3)}
            if preheat:
                r.update(preheated_experts=admitted, preheat_ms=round(t_pre * 1e3, 1))
            out["with_preheat" if preheat else "without_preheat"] = r
            log(f"prompt {P} then decode {D}, preheat={preheat}: {r}")
    out["decode_gain"] = round(out["with_preheat"]["decode_tokens_per_s"] /
                               out["without_preheat"]["decode_tokens_per_s"], 4)
    del zp, zd, xp, yp
    return out


def host_cold_pass(moe, torch, wl, stream, host_alloc, pool, x_all, logits_all, steps, warmup, swap_lead=1,
                   cpu_threads=0):
    """The same decode with the cold picks computed by the host threads (eager launches: the hand-off is not
    capturable), swap lead 1 (promotions are pinned-to-HBM copies here: no cold read to capture)."""
    T, L = wl.tokens, wl.n_layers
    ctx, freq = setup_ctx(moe, wl, wl.slots, stream, host_alloc, progress=False, capture_picks=0, pool=pool,
                          swaps=(0, swap_lead), cold_exec=moe.MOE_COLD_CPU, cpu_threads=cpu_threads)
    info = moe.moe_get_info(ctx)
    x_steps = x_all.shape[0]
    res = torch.zeros((T, wl.hidden), dtype=torch.float32, device="cuda")
    xv = [[x_all[s, layer] for layer in range(L)] for s in range(x_steps)]
    zv = [[logits_all[s, layer] for layer in range(L)] for s in range(wl.steps)]

    def step(i):
        res.zero_()
        for layer in range(L):
            moe.moe_forward(ctx, layer, T, xv[i % x_steps][layer], zv[i % wl.steps][layer], res,
                            flags=moe.MOE_ACCUMULATE)

    moe.moe_seed(ctx, freq)
    with torch.cuda.stream(stream):
        run_steps(moe, ctx, warmup, step)
        moe.moe_seed(ctx, freq)
        torch.cuda.synchronize()
        moe.moe_profile(ctx, 0)
        acc = {}
        t0 = time.perf_counter()
        run_steps(moe, ctx, steps, step, acc)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        host = moe.moe_profile(ctx, -1)
    moe.moe_destroy(ctx)
    passes = max(host["host_expert_passes"], 1)
    return {
        "tokens_per_s": round(steps * T / elapsed, 2), "ms_per_step": round(elapsed / steps * 1e3, 4),
        "hit_rate": round(acc["hits"] / max(acc["hits"] + acc["misses"], 1), 4), "swap_lead": swap_lead,
        "threads": info["host_threads"], "isa": {1: "scalar", 2: "avx2", 3: "avx512"}.get(info["host_isa"]),
        "compute_us_per_expert_pass": round(host["host_compute_ms"] / passes * 1e3, 2),
        "wait_us_per_forward": round(host["host_wait_ms"] / max(host["host_forwards"], 1) * 1e3, 2),
        # weight bytes of the cold experts the host threads read / time computing them
        "weight_GBps": round(passes * wl.expert_bytes / max(host["host_compute_ms"], 1e-9) / 1e6, 1),
        "launch": "eager"}


LARGE_WORKLOADS = ("large-e256k8-h4096f1536-l60-b1", "large-e256k8-h4096f1536-l60-b32")


LARGE_POOL_CAP = 160e9       # the large model's HBM pool cap ...
LARGE_RESERVE = 16e9         # ... after a reservation for the KV cache and dense weights


def large_pass(moe, torch, stream, host_alloc, steps=32, warmup=4):
    """The 60-layer, 256-expert model at decode batch 1 and 32 on one context (pool capped at 160 GB after a
    16 GB reservation: min(160e9, free HBM - 16e9), 251 slots per layer; batch 32 takes the grouped path).
    HIP graph per step, as the main run."""
    import numpy as np

    from workload import WORKLOADS, frequency_table, step_activations, zipf_logits

    wl1, wl32 = (WORKLOADS[n] for n in LARGE_WORKLOADS)
    setup = {}
    ctx, _ = setup_ctx(moe, wl32, wl32.slots, stream, host_alloc, progress=False, budget=LARGE_POOL_CAP,
                       reserve=LARGE_RESERVE, timing=setup)
    info = moe.moe_get_info(ctx)
    out = {"pool": {"rule": "min(160e9, free HBM - 16e9)", "free_GB_at_sizing": round(info["free_bytes_at_sizing"] / 1e9, 2),
                    "budget_GB": round(info["pool_budget_bytes"] / 1e9, 2), "slots_per_layer": info["slots_per_layer"]},
           "setup": setup}
    log(f"large model pool: {out['pool']}")
    L, H, E = wl32.n_layers, wl32.hidden, wl32.n_experts
    try:
        for wl in (wl1, wl32):
            T = wl.tokens
            freq = frequency_table(wl)  # each workload's own popularity
            logits = torch.from_numpy(zipf_logits(wl, steps=steps)).cuda()
            x_all = torch.from_numpy(np.stack([step_activations(wl, s) for s in range(4)])).cuda()
            xs = torch.zeros((L, T, H), dtype=torch.float32, device="cuda")
            zs = torch.zeros((L, T, E), dtype=torch.float32, device="cuda")
            res = torch.zeros((T, H), dtype=torch.float32, device="cuda")
            moe.moe_seed(ctx, freq)
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.stream(stream):
                with torch.cuda.graph(graph, stream=stream):
                    for layer in range(L):
                        moe.moe_forward(ctx, layer, T, xs[layer], zs[layer], res, flags=moe.MOE_ACCUMULATE)

                def step(i):
                    xs.copy_(x_all[i % 4])
                    zs.copy_(logits[i % steps])
                    res.zero_()
                    graph.replay()

                run_steps(moe, ctx, warmup, step)
                moe.moe_seed(ctx, freq)
                torch.cuda.synchronize()
                acc = {}
                t0 = time.perf_counter()
                run_steps(moe, ctx, steps, step, acc)
                torch.cuda.synchronize()
                elapsed = time.perf_counter() - t0
            distinct_gbps = acc["distinct_experts"] * wl.expert_bytes / elapsed / 1e9
            out[wl.name] = {"tokens_per_s": round(steps * T / elapsed, 2),
                            "ms_per_step": round(elapsed / steps * 1e3, 3),
                            "hit_rate": round(acc["hits"] / max(acc["hits"] + acc["misses"], 1), 4),
                            "path": "grouped by expert" if T >= 8 else "one GEMV pass per pick",
                            "distinct_experts_per_layer_step": round(acc["distinct_experts"] / (steps * L), 2),
                            # bytes of the distinct (layer, expert) pairs each step read / time: the weight bytes
                            # the step has to move at least (tokens picking one expert share its read)
                            "distinct_weight_GBps": round(distinct_gbps, 1),
                            "distinct_frac_of_hbm": round(distinct_gbps / HBM_PEAK_GBPS, 4),
                            "cold_experts_per_layer_step": round(acc["distinct_cold_experts"] / (steps * L), 3),
                            "admissions_per_step": round(acc["admissions"] / steps, 2),
                            "promotion_GB_over_pcie_per_step": round(acc["copied_pcie_bytes"] / steps / 1e9, 4)}
            log(f"{wl.name}: {out[wl.name]}")
            del graph, logits, x_all, xs, zs, res
    finally:
        moe.moe_destroy(ctx)
    return out


POLICY_WORKLOAD = "policy-e512k8-h2048f1024-l48-rot512"


def policy_pass(moe, torch, stream, host_alloc, warmup=8):
    """The cache-policy workload end to end (2048 decode steps of 48 layers, popularity permutation re-drawn
    every 512 tokens, 40 % pool, admission on the second miss within 64 tokens), from the seeded pool and, as
    the ablation, from an empty one (moe_seed with no table). HIP graph per step, cache step between steps,
    as the main run. Each run starts at step 0 of the workload."""
    import numpy as np

    from workload import WORKLOADS, step_activations, zipf_logits

    wl = WORKLOADS[POLICY_WORKLOAD]
    L, T, H, E = wl.n_layers, wl.tokens, wl.hidden, wl.n_experts
    setup = {}
    ctx, freq = setup_ctx(moe, wl, wl.slots, stream, host_alloc, progress=False, timing=setup)
    out = {"workload": wl.name, "steps": wl.steps, "slots_per_layer": wl.slots, "setup": setup}
    try:
        logits = torch.from_numpy(zipf_logits(wl)).cuda()                      # [2048][L][1][E]
        x_all = torch.from_numpy(np.stack([step_activations(wl, s) for s in range(16)])).cuda()
        xs = torch.zeros((L, T, H), dtype=torch.float32, device="cuda")
        zs = torch.zeros((L, T, E), dtype=torch.float32, device="cuda")
        res = torch.zeros((T, H), dtype=torch.float32, device="cuda")
        moe.moe_seed(ctx, freq)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            with torch.cuda.graph(graph, stream=stream):
                for layer in range(L):
                    moe.moe_forward(ctx, layer, T, xs[layer], zs[layer], res, flags=moe.MOE_ACCUMULATE)

            def step(i):
                xs.copy_(x_all[i % 16])
                zs.copy_(logits[i])
                res.zero_()
                graph.replay()

            for seeded in (True, False):
                moe.moe_seed(ctx, freq)
                run_steps(moe, ctx, warmup, step)
                moe.moe_seed(ctx, freq if seeded else None)
                torch.cuda.synchronize()
                acc = {}
                t0 = time.perf_counter()
                run_steps(moe, ctx, wl.steps, step, acc)
                torch.cuda.synchronize()
                elapsed = time.perf_counter() - t0
                r = {"tokens_per_s": round(wl.steps * T / elapsed, 2), "ms_per_step": round(elapsed / wl.steps * 1e3, 4),
                     "hit_rate": round(acc["hits"] / max(acc["hits"] + acc["misses"], 1), 4),
                     "admissions_per_step": round(acc["admissions"] / wl.steps, 3),
                     "promotion_GB_over_pcie": round(acc["copied_pcie_bytes"] / 1e9, 3)}
                log(f"policy workload, {'seeded' if seeded else 'no seed'}: {r}")
                if seeded:
                    out.update(r)
                else:
                    out["no_seed"] = r
        out["seed_gain"] = round(out["tokens_per_s"] / out["no_seed"]["tokens_per_s"], 4)
        del graph, logits, x_all, xs, zs, res
    finally:
        moe.moe_destroy(ctx)
    return out


def cpu_baseline(wl, seconds, logits):
    """The oracle on the host cores: decode tokens through all layers, fp64."""
    import numpy as np

    import oracle
    from workload import activations, expert_weights

    oracle.lib()
    threads = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
    spent = 0.0
    tokens = 0
    step = 0
    while spent < seconds and step < wl.steps:
        for layer in range(wl.n_layers):
            x = activations(wl, step, layer=layer).astype(np.float64)
            z = logits[step, layer]
            ids, _ = oracle.route(z, wl.top_k)
            experts = {int(e): expert_weights(wl, layer, int(e)) for e in np.unique(ids)}
            t0 = time.perf_counter()
            oracle.moe_layer(wl.n_experts, wl.top_k, wl.hidden, wl.ffn, experts, x, logits=z)
            spent += time.perf_counter() - t0
        tokens += wl.tokens
        step += 1
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return dict(value=tokens / spent, unit="tokens/s", cores=threads, kind="oracle",
                sample=f"first {tokens} decode tokens through all {wl.n_layers} layers (fp64 oracle, "
                       f"{spent:.1f} s of oracle time; weight generation excluded)", cpu_model=model)


def pcie_reads():
    """The workload of the PCIe read counters: (1) calibration, read_stream_kernel over 256 MiB of pinned host
    memory (one untimed and two timed launches); (2) a cold-only decode of the 512-expert top-8 hidden 2048 /
    ffn 1024 shape, empty pool, batch 1, 2 layers x 8 steps, capture off (every gate/up and down launch serves 8
    cold picks); (3) its 4096-token prompt pass with an empty pool (every used expert staged over PCIe)."""
    import numpy as np
    import torch

    import moe_expert_offload_gemv_amd as moe
    from workload import WORKLOADS, activations, layer_weights, zipf_logits

    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        g = moe.moe_measure_read_bandwidth(None, 256 << 20, reps=2, host_coherent=True)
        log(f"calibration: 3 launches x 268435456 B pinned zero-copy, {g:.2f} GB/s")
        wl = WORKLOADS["decode-e512k8-h2048f1024-l48-b1"]
        E, k, H, F = wl.n_experts, wl.top_k, wl.hidden, wl.ffn
        ctx = moe.moe_create(2, E, k, H, F, pool_budget_bytes=0, max_batch_tokens=1, host_sets=1, capture_picks=0,
                             stream=stream)
        moe.moe_register_layer(ctx, 0, *layer_weights(wl, 0))
        moe.moe_seed(ctx, None)
        z = torch.from_numpy(zipf_logits(wl, layers=[0, 1], steps=8)).cuda()
        x = torch.from_numpy(np.stack([activations(wl, s) for s in range(8)])).cuda()
        y = torch.zeros((1, H), dtype=torch.float32, device="cuda")
        picks = 0
        for s in range(8):
            for layer in range(2):
                moe.moe_forward(ctx, layer, 1, x[s], z[s, layer], y, flags=moe.MOE_ACCUMULATE)
            picks += moe.moe_cache_step(ctx)["misses"]
        torch.cuda.synchronize()
        moe.moe_destroy(ctx)
        log(f"cold decode: 16 forwards, {picks} cold picks")
        wlp = WORKLOADS["prefill-e512k8-h2048f1024-t4096"]
        T = wlp.tokens
        ctx = moe.moe_create(1, E, k, H, F, pool_budget_bytes=0, max_batch_tokens=1, max_prefill_tokens=T,
                             host_sets=1, stream=stream)
        moe.moe_register_layer(ctx, 0, *layer_weights(wlp, 0))
        moe.moe_seed(ctx, None)
        xp = torch.from_numpy(activations(wlp, 0, tokens=T)).cuda()
        zp = torch.from_numpy(np.ascontiguousarray(zipf_logits(wlp, steps=1, tokens=T)[0, 0])).cuda()
        yp = torch.empty_like(xp)
        moe.moe_prefill(ctx, 0, T, xp, zp, yp)
        torch.cuda.synchronize()
        moe.moe_destroy(ctx)
        log("prompt pass: 4096 tokens, every used expert staged")


def main():
    global DECODE_LAUNCHES
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--workload", default="decode-e512k8-h2048f1024-l48-b1")
    ap.add_argument("--eager", action="store_true", help="launch per step instead of replaying a HIP graph")
    ap.add_argument("--host-alloc", choices=["coherent", "noncoherent"], default="coherent")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-side-passes", action="store_true")
    ap.add_argument("--pool", choices=["layer", "global"], default="layer",
                    help="slots per layer, or one pool of the same total size shared by all layers")
    ap.add_argument("--slots", type=int, default=0, help="pool slots per layer (0: the workload's)")
    ap.add_argument("--capture-picks", type=int, default=-1,
                    help="picks per layer whose cold reads are kept for promotion (-1: top_k, 0: off)")
    ap.add_argument("--swaps-per-step", type=int, default=0, help="admissions per cache step (0: no limit)")
    ap.add_argument("--swap-lead", type=int, default=0,
                    help="cache steps an admission waits for its copy before its table entry flips")
    ap.add_argument("--cold-exec", choices=["gpu", "cpu"], default="gpu",
                    help="cold picks read zero-copy by the GPU, or computed by host threads (eager launches)")
    ap.add_argument("--cpu-threads", type=int, default=0, help="host threads for --cold-exec cpu (0: all CPUs of the affinity mask but two)")
    ap.add_argument("--profile-steps", type=int, default=64, help="steps of the kernel-timing pass")
    ap.add_argument("--decode-launches", type=int, choices=[1, 2], default=DECODE_LAUNCHES,
                    help="decode batches of 1..7 tokens: 1 one launch per layer, 2 two launches")
    ap.add_argument("--prefill-only", action="store_true",
                    help="only run the two prompt passes (one line of JSON each; for counter runs)")
    ap.add_argument("--prompt-tokens", type=int, default=12288,
                    help="prompt length of the prompt-then-decode pass (0: skip it)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 4 times (the reference for counter scaling)")
    ap.add_argument("--pcie-reads", action="store_true",
                    help="only run the PCIe counter workload: a pinned-memory read of known size, a cold-only decode "
                         "and a staged prompt pass (for rocprofv3 --pmc runs)")
    args = ap.parse_args()
    DECODE_LAUNCHES = args.decode_launches
    if args.copy_calibration:
        import torch

        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copied 4 x 1 GiB")
        return
    if args.pcie_reads:
        pcie_reads()
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path shards per GPU with no "
              f"exchange, so a multi-GPU figure is N independent copies of this one.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import moe_expert_offload_gemv_amd as moe
    from workload import WORKLOADS, step_activations, zipf_logits

    if args.prefill_only:
        host_alloc = moe.MOE_HOST_NONCOHERENT if args.host_alloc == "noncoherent" else moe.MOE_HOST_COHERENT
        stream = torch.cuda.Stream()
        for name in PREFILL_WORKLOADS:
            print(json.dumps(prefill_pass(moe, torch, WORKLOADS[name], stream, host_alloc,
                                          gemm_ceiling=fp16_gemm_ceiling(torch),
                                          cpu_seconds=0.0 if args.no_cpu_baseline else 10.0)), flush=True)
        return

    wl = WORKLOADS[args.workload]
    host_alloc = moe.MOE_HOST_NONCOHERENT if args.host_alloc == "noncoherent" else moe.MOE_HOST_COHERENT
    T, L, H, E, k = wl.tokens, wl.n_layers, wl.hidden, wl.n_experts, wl.top_k
    B = wl.expert_bytes
    log(f"workload {wl.name}: L={L} E={E} k={k} H={H} F={wl.ffn} T={T} slots={wl.slots} "
        f"expert={B} B host sets={wl.weight_layers} pinned={wl.weight_layers * E * B / 1e9:.1f} GB "
        f"pool={L * wl.slots * B / 1e9:.1f} GB")

    stream = torch.cuda.Stream()
    t_setup = time.time()
    log(f"creating the context: pinning {wl.weight_layers * E * B / 1e9:.1f} GB of host memory")
    if args.slots:
        wl = wl.with_(slots=args.slots)
    prompt_tokens = 0 if args.no_side_passes else args.prompt_tokens
    cold_exec = moe.MOE_COLD_CPU if args.cold_exec == "cpu" else moe.MOE_COLD_GPU
    if cold_exec == moe.MOE_COLD_CPU:
        args.eager = True  # the host hand-off is not capturable
    setup = {}
    ctx, freq = setup_ctx(moe, wl, wl.slots, stream, host_alloc,
                          capture_picks=None if args.capture_picks < 0 else args.capture_picks, pool=args.pool,
                          max_prefill_tokens=prompt_tokens, swaps=(args.swaps_per_step, args.swap_lead),
                          cold_exec=cold_exec, cpu_threads=args.cpu_threads, timing=setup)
    info = moe.moe_get_info(ctx)
    if cold_exec == moe.MOE_COLD_CPU:
        log(f"cold picks on {info['host_threads']} host threads (isa code {info['host_isa']})")
    logits_np = zipf_logits(wl)
    logits_all = torch.from_numpy(logits_np).cuda()                       # [steps][L][T][E]
    x_steps = min(wl.steps, 32)
    x_all = torch.from_numpy(np.stack([step_activations(wl, s) for s in range(x_steps)])).cuda()  # [32][L][T][H]
    xs = torch.zeros((L, T, H), dtype=torch.float32, device="cuda")
    zs = torch.zeros((L, T, E), dtype=torch.float32, device="cuda")
    res = torch.zeros((T, H), dtype=torch.float32, device="cuda")
    t_seed = time.time()
    moe.moe_seed(ctx, freq)
    setup["seed_s"] = round(time.time() - t_seed, 2)
    setup["total_s"] = round(time.time() - t_setup, 2)
    log(f"setup {setup}")

    def forward_all():
        for layer in range(L):
            moe.moe_forward(ctx, layer, T, xs[layer], zs[layer], res, flags=moe.MOE_ACCUMULATE)

    graph = None
    if not args.eager:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            with torch.cuda.graph(graph, stream=stream):
                forward_all()

    def step(i):
        s = i % wl.steps
        xs.copy_(x_all[s % x_steps])
        zs.copy_(logits_all[s])
        res.zero_()
        if graph is not None:
            graph.replay()
        else:
            forward_all()

    with torch.cuda.stream(stream):
        run_steps(moe, ctx, args.warmup, step)
        moe.moe_seed(ctx, freq)  # the timed region starts from the seeded pool at step 0
        torch.cuda.synchronize()
        moe.moe_profile(ctx, 0)  # kernel timing off; host-thread counters start here
        acc = {}
        t0 = time.perf_counter()
        run_steps(moe, ctx, args.steps, step, acc)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
    host = moe.moe_profile(ctx, -1) if cold_exec == moe.MOE_COLD_CPU else None
    tokens = args.steps * T
    tps = tokens / elapsed
    log(f"timed: {args.steps} steps in {elapsed * 1e3:.1f} ms -> {tps:.1f} tokens/s; stats {acc}")

    # kernel timing over the same steps, eager launches bracketed by HIP events on the context stream
    with torch.cuda.stream(stream):
        moe.moe_seed(ctx, freq)
        moe.moe_profile(ctx, 1)
        prof_steps = min(args.steps, args.profile_steps)
        t1 = time.perf_counter()
        run_steps(moe, ctx, prof_steps, lambda i: (xs.copy_(x_all[i % x_steps]), zs.copy_(
            logits_all[i % wl.steps]), res.zero_(), forward_all()))
        t_prof = time.perf_counter() - t1
        prof = moe.moe_profile(ctx, 0)
    fw = max(prof["forwards"], 1)
    gu_bytes = prof["gateup_bytes_per_pick"]
    pick_bytes = gu_bytes + prof["down_bytes_per_pick"]
    one_launch = prof["layer_forwards"] == prof["forwards"] and prof["forwards"] > 0
    if one_launch:
        # one launch per layer, timed as a hot launch (routing, lookup, gate/up and down of the hot picks)
        # and a cold one (the cold picks, then the combine)
        hot_gu_us = prof["hot_layer_ms"] / fw * 1e3
        hot_gu_bytes = prof["hot_picks"] * pick_bytes / fw
        cold_rate = prof["cold_picks"] * pick_bytes / max(prof["cold_layer_ms"], 1e-9) / 1e6
        cold_dn_rate = None
        roof_kernel = ("decode_layer_kernel, hot launch (routing + slot lookup + gate/up + SwiGLU + down of the hot "
                       "picks from the HBM pool, one launch per layer)")
        pcie_kernel = "decode_layer_kernel, cold launch (zero-copy reads of pinned host memory, then the combine)"
    else:
        hot_gu_us = prof["hot_gateup_ms"] / fw * 1e3
        hot_gu_bytes = prof["hot_picks"] * gu_bytes / fw
        cold_rate = prof["cold_picks"] * gu_bytes / max(prof["cold_gateup_ms"], 1e-9) / 1e6
        cold_dn_rate = prof["cold_picks"] * prof["down_bytes_per_pick"] / max(prof["cold_down_ms"], 1e-9) / 1e6
        roof_kernel = ("gemv_route_gateup_kernel, hot picks (routing + slot lookup + gate/up + SwiGLU from the HBM "
                       "pool; the launch includes the routing)")
        pcie_kernel = "gemv_route_gateup_kernel, cold picks (zero-copy reads of pinned host memory)"
    achieved = hot_gu_bytes / (hot_gu_us * 1e-6) / 1e9
    log(f"kernel timing ({prof_steps} eager steps, {prof_steps * T / t_prof:.1f} tokens/s): {prof}")

    request = None
    if prompt_tokens > 0 and T == 1:
        request = request_pass(moe, torch, ctx, wl, freq, stream, prompt_tokens, 256,
                               lambda z: (zs.copy_(z), res.zero_(), graph.replay() if graph is not None
                                          else forward_all()), xs, x_all)
    moe.moe_destroy(ctx)

    result = {
        "metric": METRIC,
        "value": round(tps, 3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "layers": L, "experts": E, "top_k": k, "hidden": H, "ffn": wl.ffn,
                   "tokens_per_step": T, "pool_slots_per_layer": wl.slots, "weights": "q4 blocks (18 B / 32)",
                   "host_alloc": args.host_alloc, "host_weight_sets": wl.weight_layers,
                   "capture_picks": (0 if args.cold_exec == "cpu" else wl.top_k) if args.capture_picks < 0
                   else args.capture_picks,
                   "pool": args.pool, "swaps_per_step": args.swaps_per_step, "swap_lead": args.swap_lead,
                   "cold_exec": args.cold_exec, "host_threads": info["host_threads"],
                   "launch": "eager" if args.eager else "hip-graph",
                   "decode_launches_per_layer": DECODE_LAUNCHES},
        # outside the timed region: pinning and allocating, weight generation, registration, seeding
        "setup": setup,
        "effective_weight_GBps": round((acc["hot_bytes"] + acc["cold_bytes"]) / elapsed / 1e9, 2),
        "hot_GBps_over_step": round(acc["hot_bytes"] / elapsed / 1e9, 2),
        "cold_GBps_over_step": round(acc["cold_bytes"] / elapsed / 1e9, 2),
        "hit_rate": round(acc["hits"] / max(acc["hits"] + acc["misses"], 1), 4),
        "admissions_per_step": round(acc["admissions"] / args.steps, 3),
        # promotions copied from the HBM capture of their cold reads vs from pinned memory (PCIe)
        "promotion_GB": round(acc["copied_bytes"] / 1e9, 3),
        "promotion_GB_over_pcie": round(acc["copied_pcie_bytes"] / 1e9, 3),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": ROOFLINE_TRAFFIC and int(ROOFLINE_TRAFFIC["bytes_per_launch"]),
                     "traffic_over_algorithmic": ROOFLINE_TRAFFIC and round(
                         ROOFLINE_TRAFFIC["bytes_per_launch"] / ROOFLINE_TRAFFIC["algorithmic_bytes_per_launch"], 3),
                     "kernel": roof_kernel,
                     "avg_launch_us": round(hot_gu_us, 2), "bytes_per_launch": int(hot_gu_bytes)},
        "pcie": ({"cold_layer_GBps": round(cold_rate, 2)} if one_launch else
                 {"cold_gateup_GBps": round(cold_rate, 2), "cold_down_GBps": round(cold_dn_rate, 2)}) | {
                 "peak": PCIE_PEAK_GBPS, "frac": round(cold_rate / PCIE_PEAK_GBPS, 4), "kernel": pcie_kernel},
        # route is 0 where the routing runs inside the gate/up launches (logits given, E <= 512); with one
        # launch per layer only hot_layer and cold_layer are nonzero
        "per_layer_us": {k_: round(prof[k_ + "_ms"] / fw * 1e3, 2)
                         for k_ in ("route", "hot_gateup", "hot_down", "cold_gateup", "cold_down", "hot_layer",
                                    "cold_layer")},
    }

    if not args.no_side_passes:
        side = min(4, L)
        cap = None if args.capture_picks < 0 else args.capture_picks
        hot = kernel_pass(moe, torch, wl, E, side, 32, stream, host_alloc, logits_all, x_all, cap)
        cold = kernel_pass(moe, torch, wl, 0, side, 8, stream, host_alloc, logits_all, x_all, cap)

        def rate(p, ms_key, picks_key, bytes_key):
            return p[picks_key] * p[bytes_key] / max(p[ms_key], 1e-9) / 1e6  # bytes / ms -> GB/s

        def side(p, tag, peak):
            keys = ("route", "hot_gateup", "hot_down", "cold_gateup", "cold_down", "hot_layer", "cold_layer")
            out = {"per_layer_us": {k_: round(p[k_ + "_ms"] / p["forwards"] * 1e3, 2) for k_ in keys}}
            if p["layer_forwards"]:
                p = dict(p, pick_bytes=p["gateup_bytes_per_pick"] + p["down_bytes_per_pick"])
                r = rate(p, tag + "_layer_ms", tag + "_picks", "pick_bytes")
                out["layer_GBps"] = round(r, 2)
            else:
                r = rate(p, tag + "_gateup_ms", tag + "_picks", "gateup_bytes_per_pick")
                out["gateup_GBps"] = round(r, 2)
                out["down_GBps"] = round(rate(p, tag + "_down_ms", tag + "_picks", "down_bytes_per_pick"), 2)
            out["frac_of_" + ("hbm" if tag == "hot" else "pcie")] = round(r / peak, 4)
            return out

        result["kernels_all_hot"] = side(hot, "hot", HBM_PEAK_GBPS)
        result["kernels_all_cold"] = side(cold, "cold", PCIE_PEAK_GBPS)
        # DMA ceiling: pinned host -> HBM copy of 1 GiB
        src = torch.empty(1 << 30, dtype=torch.uint8, pin_memory=True)
        dst = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst.copy_(src, non_blocking=True)
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        for _ in range(3):
            dst.copy_(src, non_blocking=True)
        torch.cuda.synchronize()
        result["pcie_dma_h2d_GBps"] = round(3 * (1 << 30) / (time.perf_counter() - t2) / 1e9, 2)
        del src, dst
        # read ceilings of a plain 128-bit streaming kernel: 8 GiB of HBM, 1 GiB of pinned host memory zero-copy
        buf = torch.empty(8 << 30, dtype=torch.uint8, device="cuda")
        hbm_ceiling = moe.moe_measure_read_bandwidth(buf, reps=5)
        del buf
        result["ceilings"] = {
            "hbm_stream_read_GBps": round(hbm_ceiling, 1),
            "zero_copy_read_GBps": {
                k_: round(moe.moe_measure_read_bandwidth(None, 1 << 30, reps=3, host_coherent=c_), 2)
                for k_, c_ in (("coherent", True), ("noncoherent", False))},
            "dma_h2d_GBps": result["pcie_dma_h2d_GBps"],
            "spec": {"hbm_GBps": HBM_PEAK_GBPS, "pcie_GBps": PCIE_PEAK_GBPS}}
        if result.get("roofline") and result["roofline"].get("unit") == "GB/s":
            result["roofline"]["frac_of_measured_ceiling"] = round(result["roofline"]["achieved"] / hbm_ceiling, 4)
        log(f"side passes: hot {result['kernels_all_hot']} cold {result['kernels_all_cold']} "
            f"dma {result['pcie_dma_h2d_GBps']} GB/s")

    if host is not None:
        hb = host["host_expert_passes"] * B  # weight bytes read (tokens sharing an expert share the pass)
        result["host_threads"] = {
            "threads": info["host_threads"], "isa": {1: "scalar", 2: "avx2", 3: "avx512"}.get(info["host_isa"]),
            "forwards": host["host_forwards"], "expert_passes": host["host_expert_passes"],
            "picks": host["host_picks"],
            "wait_us_per_forward": round(host["host_wait_ms"] / max(host["host_forwards"], 1) * 1e3, 2),
            "compute_us_per_forward": round(host["host_compute_ms"] / max(host["host_forwards"], 1) * 1e3, 2),
            "compute_us_per_expert_pass": round(host["host_compute_ms"] / max(host["host_expert_passes"], 1) * 1e3,
                                                2),
            # weight bytes of the cold picks / time computing them
            "weight_GBps": round(hb / max(host["host_compute_ms"], 1e-9) / 1e6, 1)}
        log(f"host threads: {result['host_threads']}")
    if request is not None:
        result["prompt_then_decode"] = request
    if not args.no_side_passes and cold_exec == moe.MOE_COLD_GPU and T == 1:
        # the method's other way to serve misses, same workload, measured here (a context of its own)
        result["cold_picks_on_host_threads"] = host_cold_pass(moe, torch, wl, stream, host_alloc, args.pool, x_all,
                                                              logits_all, args.steps, args.warmup,
                                                              cpu_threads=args.cpu_threads)
        log(f"host-thread cold picks: {result['cold_picks_on_host_threads']}")
    if not args.no_side_passes and wl.name == "decode-e512k8-h2048f1024-l48-b1":
        result["policy"] = policy_pass(moe, torch, stream, host_alloc)
        result["large_model"] = large_pass(moe, torch, stream, host_alloc)
    if not args.no_side_passes:
        gemm_ceiling = fp16_gemm_ceiling(torch)
        result["prefill"] = [prefill_pass(moe, torch, WORKLOADS[name], stream, host_alloc, gemm_ceiling=gemm_ceiling,
                                          cpu_seconds=0.0 if args.no_cpu_baseline else 10.0)
                             for name in PREFILL_WORKLOADS]
        if "ceilings" in result:
            result["ceilings"]["fp16_gemm_TFLOPs"] = round(gemm_ceiling, 1)
        log(f"prefill: {result['prefill']}")

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds, logits_np)
        log(f"cpu baseline: {result['cpu_baseline']}")

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
