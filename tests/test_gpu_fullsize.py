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
from tests._gpu import TOL, GraphDecode, oracle_layers, oracle_policy, token_rel_err  # noqa: E402
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
            rows = list(range(wl.tokens)) if sample_rows is None else sample_rows
            got = g.layer_outputs()
            ref = oracle_layers(wl, xs[:, rows], logits[step][:, rows])
            for layer in range(wl.n_layers):
                err = token_rel_err(got[layer][rows], ref[layer])
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
    worst, hit_rate = _run(wl, wl.steps, sample_steps={600}, table_every=128)
    print(f"worst layer error {worst:.2e}, hit rate {hit_rate:.4f}")


def test_large_model_batch_1():
    wl = WORKLOADS["large-e256k8-h4096f1536-l60-b1"]
    _run(wl, 48, sample_steps={47}, table_every=16)


def test_large_model_batch_32():
    wl = WORKLOADS["large-e256k8-h4096f1536-l60-b32"]
    _run(wl, 24, sample_steps={23}, table_every=8, sample_rows=[0, 31])


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
        rows = np.random.default_rng(1).choice(T, size=24, replace=False)
        ids, _ = oracle.route(z[rows], wl.top_k)
        y_ref, _, _ = oracle.moe_layer(wl.n_experts, wl.top_k, wl.hidden, wl.ffn, d.experts(0, ids),
                                       x32[rows].astype(np.float64), logits=z[rows])
        err = token_rel_err(y.cpu().numpy()[rows], y_ref)
        print(name, "sampled token error", err)
        assert err < TOL
    finally:
        d.close()
