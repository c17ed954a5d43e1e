"""Parity at the full sizes of the evaluation workloads, in the launch
configuration bench.py times (a HIP graph of every layer's forward, each adding its output into one
residual buffer, replayed per step, then the cache step).

Policy state is compared bit for bit with the oracle's simulation at every
step (statistics and miss log) and at checkpoints (all slot tables and
stamps); layer outputs are compared with the oracle's fp64 chain on sampled
steps (per token: max abs error over max abs value below 2e-3).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import moe_expert_offload_gemv_amd as moe  # noqa: E402
import oracle  # noqa: E402
from tests._gpu import (TOL, GraphDecode, oracle_layers, oracle_policy, tile_edge_tokens,  # noqa: E402
                        token_rel_err)
from workload import WORKLOADS, activations, step_activations, zipf_logits  # noqa: E402

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def _check_tables(g: GraphDecode, pol):
    wl = g.wl
    tabs = pol.tables()
    for layer in range(wl.n_layers):
        assert np.array_equal(moe.moe_get_slot_table(g.d.ctx, layer, wl.n_experts), tabs["table"][layer]), layer
        assert np.array_equal(moe.moe_get_stamps(g.d.ctx, layer, g.d.S), tabs["stamps"][layer]), layer


def _run(wl, steps, sample_steps, table_every, max_batch=None, sample_rows=None, cold_exec=moe.MOE_COLD_GPU,
         swaps=(0, 0)):
    g = GraphDecode(wl, max_batch=max_batch, cold_exec=cold_exec, swaps=swaps)
    try:
        return _steps(g, wl, steps, sample_steps, table_every, sample_rows, swaps)
    finally:
        g.close()


def _steps(g, wl, steps, sample_steps, table_every, sample_rows, swaps=(0, 0)):
    pol = oracle_policy(wl, wl.slots, swaps_per_step=swaps[0], swap_lead=swaps[1])
    logits = zipf_logits(wl, steps=steps)
    worst = 0.0
    hits = misses = 0
    for step in range(steps):
        xs = step_activations(wl, step)
        st = g.step(xs, logits[step])
        for layer in range(wl.n_layers):
            pol.forward(layer, oracle.route(logits[step, layer], wl.top_k)[0])
        so = pol.step()
        for key in ("hits", "misses", "admissions", "evictions", "tokens"):
            assert st[key] == so[key], (step, key, st, so)
        assert np.array_equal(moe.moe_get_miss_log(g.d.ctx), pol.last_log()), step
        hits += st["hits"]
        misses += st["misses"]
        if step % table_every == table_every - 1 or step == steps - 1:
            _check_tables(g, pol)
        if step in sample_steps:
            # sample_steps: a set of steps (every layer) or step -> layers (None: every layer)
            layers = sample_steps.get(step) if isinstance(sample_steps, dict) else None
            layers = list(range(wl.n_layers)) if layers is None else list(layers)
            rows = list(range(wl.tokens)) if sample_rows is None else sample_rows
            got = g.layer_outputs()
            ref = oracle_layers(wl, xs[:, rows], logits[step][:, rows], layers=layers)
            for li, layer in enumerate(layers):
                err = token_rel_err(got[layer][rows], ref[li])
                worst = max(worst, err)
                assert err < TOL, (step, layer, err)
    assert np.array_equal(moe.moe_get_counts(g.d.ctx, wl.n_layers, wl.n_experts), pol.counts())
    return worst, hits / max(hits + misses, 1)


def test_decode_48_layers_512_experts_all_256_steps():
    wl = WORKLOADS["decode-e512k8-h2048f1024-l48-b1"]
    worst, hit_rate = _run(wl, wl.steps, sample_steps={0, 131, 255}, table_every=32)
    print(f"worst layer error {worst:.2e}, hit rate {hit_rate:.4f}")
    assert 0.85 < hit_rate < 0.95


def test_decode_48_layers_cold_picks_on_host_threads():
    # the bench's host-thread configuration: eager launches, swap lead 1, 8
    # swaps per step; most forwards have no cold pick and do not wait for the
    # host, so later forwards overtake the host's reading of the mailbox
    wl = WORKLOADS["decode-e512k8-h2048f1024-l48-b1"]
    worst, hit_rate = _run(wl, 96, sample_steps={0, 50, 95}, table_every=16, cold_exec=moe.MOE_COLD_CPU,
                           swaps=(8, 1))
    print(f"worst layer error {worst:.2e}, hit rate {hit_rate:.4f}")


def test_policy_2048_steps_with_rotation():
    wl = WORKLOADS["policy-e512k8-h2048f1024-l48-rot512"]
    # outputs before and after rotations (every 512 tokens), every layer
    worst, hit_rate = _run(wl, wl.steps, sample_steps={0, 600, 1300, 2047}, table_every=128)
    print(f"worst layer error {worst:.2e}, hit rate {hit_rate:.4f}")


def test_large_model_batch_1():
    wl = WORKLOADS["large-e256k8-h4096f1536-l60-b1"]
    _run(wl, 48, sample_steps={47}, table_every=16)


def test_large_model_batch_32():
    wl = WORKLOADS["large-e256k8-h4096f1536-l60-b32"]
    # every row of the batch; every layer at the last step, a third of them (all 20 host weight sets) earlier
    worst, _ = _run(wl, 24, sample_steps={0: range(0, 60, 3), 11: range(1, 60, 3), 23: None}, table_every=8)
    print(f"worst layer error {worst:.2e}")


@pytest.mark.parametrize("name", ["prefill-e512k8-h2048f1024-t4096", "large-e256k8-h4096f1536-t12288"])
def test_prefill_full_size(name):
    from tests._gpu import Decode

    wl = WORKLOADS[name]
    T = wl.tokens
    d = Decode(wl, max_batch=1, max_prefill=T)
    try:
        x32 = activations(wl, 0, tokens=T)
        z = zipf_logits(wl, steps=1, tokens=T)[0, 0]
        x = torch.from_numpy(x32).cuda()
        y = torch.empty_like(x)
        moe.moe_prefill(d.ctx, 0, T, x, torch.from_numpy(np.ascontiguousarray(z)).cuda(), y)
        if T <= 4096:
            rows = np.arange(T)
        else:
            # the first and last row of every (expert, tile), whichever tile height the pass took, and random rows
            ids_all, _ = oracle.route(z, wl.top_k)
            edges = tile_edge_tokens(ids_all)
            rest = np.setdiff1d(np.arange(T), edges)
            extra = np.random.default_rng(1).choice(rest, size=max(0, 2048 - edges.size // 2), replace=False)
            rows = np.union1d(edges, extra)
        ids, _ = oracle.route(z[rows], wl.top_k)
        y_ref, _, _ = oracle.moe_layer(wl.n_experts, wl.top_k, wl.hidden, wl.ffn, d.experts(0, ids),
                                       x32[rows].astype(np.float64), logits=z[rows])
        err = token_rel_err(y.cpu().numpy()[rows], y_ref)
        print(name, f"{rows.size} rows, worst token error {err:.2e}")
        assert rows.size >= min(T, 2048)
        assert err < TOL
    finally:
        d.close()


def test_pool_capacity_from_free_hbm_minus_reserve():
    """The large model's pool from the capacity rule: free HBM at sizing minus a 16 GB reserve, and the
    same capped at 160 GB; S = min(E, budget / (L * expert bytes))."""
    wl = WORKLOADS["large-e256k8-h4096f1536-l60-b1"]
    L, E, B = wl.n_layers, wl.n_experts, wl.expert_bytes
    reserve = 16 * 10**9
    for cap in (-1, 160 * 10**9):
        free_before, _ = torch.cuda.mem_get_info()
        ctx = moe.moe_create(L, E, wl.top_k, wl.hidden, wl.ffn, pool_budget_bytes=cap, reserve_bytes=reserve,
                             max_batch_tokens=1, host_sets=1)
        try:
            info = moe.moe_get_info(ctx)
            free = info["free_bytes_at_sizing"]
            # only the small device state and the capture blocks come before the sizing
            assert free_before - 8 * 10**9 < free <= free_before, (free_before, free)
            budget = free - reserve if cap < 0 else min(cap, free - reserve)
            assert info["pool_budget_bytes"] == budget
            assert info["slots_per_layer"] == min(E, budget // (L * B))
            assert info["pool_bytes"] == L * info["slots_per_layer"] * B
            print(f"cap {cap}: free {free / 1e9:.1f} GB, budget {budget / 1e9:.1f} GB, "
                  f"{info['slots_per_layer']} slots per layer")
            if cap > 0 and free - reserve >= cap:
                assert info["slots_per_layer"] == wl.slots  # 251 of 256 at 160 GB
        finally:
            moe.moe_destroy(ctx)
