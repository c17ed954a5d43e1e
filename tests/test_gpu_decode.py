"""GPU parity of the decode path through the C ABI against the oracle.

Routing ids, miss logs, slot tables, stamps, counts and step statistics are
compared bit for bit with the oracle's step-by-step policy simulation; layer
outputs within 2e-3 of the oracle's fp64 result (per token, max abs error
over max abs value).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import moe_expert_offload_gemv_amd as moe  # noqa: E402
import oracle  # noqa: E402
from tests._gpu import TOL, Decode, oracle_policy, token_rel_err  # noqa: E402
from workload import WORKLOADS, Workload, activations, router_weights, step_activations, zipf_logits  # noqa: E402

pytestmark = pytest.mark.gpu


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _compare_policy(d: Decode, pol, st_gpu, st_orc, layers):
    wl = d.wl
    for key in ("hits", "misses", "admissions", "evictions", "tokens"):
        assert st_gpu[key] == st_orc[key], (key, st_gpu, st_orc)
    assert st_gpu["hot_bytes"] == st_orc["hits"] * d.B and st_gpu["cold_bytes"] == st_orc["misses"] * d.B
    tabs = pol.tables()
    for layer in layers:
        assert np.array_equal(moe.moe_get_slot_table(d.ctx, layer, wl.n_experts), tabs["table"][layer]), layer
        group = 0 if d.pool == "global" else layer
        assert np.array_equal(moe.moe_get_stamps(d.ctx, layer, d.S), tabs["stamps"][group]), layer
    assert np.array_equal(moe.moe_get_miss_log(d.ctx), pol.last_log())


def _run_decode(wl: Workload, slots: int, check_every: int, seed=True, host_alloc=moe.MOE_HOST_COHERENT,
                capture_picks=None, copies=None, pool="layer", swaps=(0, 0), cold_exec=moe.MOE_COLD_GPU,
                cpu_threads=0, repeats=None):
    """repeats: a list that receives, per step, how many admissions took a slot that an earlier admission
    of the same step (same pool) had already taken."""
    d = Decode(wl, slots=slots, seed=seed, host_alloc=host_alloc, capture_picks=capture_picks, pool=pool,
               swaps_per_step=swaps[0], swap_lead=swaps[1], cold_exec=cold_exec, cpu_threads=cpu_threads)
    if cold_exec == moe.MOE_COLD_CPU:
        info = moe.moe_get_info(d.ctx)
        print("host threads", info["host_threads"], "isa code", info["host_isa"])
        assert info["host_threads"] >= 1 and info["host_isa"] >= 1
    pol = oracle_policy(wl, slots, seed=seed, pool=pool, swaps_per_step=swaps[0], swap_lead=swaps[1])
    logits = zipf_logits(wl)
    L, T, k, H = wl.n_layers, wl.tokens, wl.top_k, wl.hidden
    y = torch.empty((T, H), dtype=torch.float32, device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    worst = 0.0
    for step in range(wl.steps):
        check = step % check_every == 0
        for layer in range(L):
            x32 = activations(wl, step, layer=layer)
            x = _dev(x32)
            z = logits[step, layer]
            moe.moe_forward(d.ctx, layer, T, x, _dev(z), y, ids, w)
            ids_h = ids.cpu().numpy()
            ids_o, w_o = oracle.route(z, k)
            assert np.array_equal(ids_h, ids_o), (step, layer)
            np.testing.assert_allclose(w.cpu().numpy(), w_o, rtol=2e-6, atol=1e-7)
            pol.forward(layer, ids_o)
            if check:
                y_ref, _, _ = oracle.moe_layer(wl.n_experts, k, H, wl.ffn, d.experts(layer, ids_o),
                                               x32.astype(np.float64), logits=z)
                err = token_rel_err(y.cpu().numpy(), y_ref)
                worst = max(worst, err)
                assert err < TOL, (step, layer, err)
        st_g = moe.moe_cache_step(d.ctx)
        st_o = pol.step()
        _compare_policy(d, pol, st_g, st_o, range(L))
        if repeats is not None:
            adm = pol.last_admissions()
            keys = [(0 if pool == "global" else int(a[0]), int(a[2])) for a in adm]
            repeats.append(len(keys) - len(set(keys)))
        assert 0 <= st_g["copied_pcie_bytes"] <= st_g["copied_bytes"] == st_o["admissions"] * d.B
        if copies is not None:
            copies["copied"] = copies.get("copied", 0) + st_g["copied_bytes"]
            copies["pcie"] = copies.get("pcie", 0) + st_g["copied_pcie_bytes"]
    assert np.array_equal(moe.moe_get_counts(d.ctx, L, wl.n_experts), pol.counts())
    d.close()
    return worst


def test_tiny_layer_router_in_the_loop():
    wl = WORKLOADS["tiny-e8k2-h256f512-t4"]
    d = Decode(wl)
    moe.moe_register_router(d.ctx, 0, router_weights(wl, 0))  # allowed after seed: no weights move
    x32 = activations(wl, 0)
    y = torch.empty((4, 256), dtype=torch.float32, device="cuda")
    ids = torch.empty((4, 2), dtype=torch.int32, device="cuda")
    w = torch.empty((4, 2), dtype=torch.float32, device="cuda")
    moe.moe_forward(d.ctx, 0, 4, _dev(x32), None, y, ids, w)
    W = router_weights(wl, 0)
    g, u, dn = d.weights[0]
    y_ref, ids_ref, w_ref = oracle.moe_layer(8, 2, 256, 512, {e: (g[e], u[e], dn[e]) for e in range(8)},
                                             x32.astype(np.float64), w_router=W, x32=x32)
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    np.testing.assert_allclose(w.cpu().numpy(), w_ref, rtol=2e-6)
    assert token_rel_err(y.cpu().numpy(), y_ref) < TOL
    st = moe.moe_cache_step(d.ctx)
    assert st["misses"] == 0 and st["hits"] == 8 and st["admissions"] == 0 and st["tokens"] == 4
    assert moe.moe_get_miss_log(d.ctx).size == 0
    # logits handed in give the same result
    z = oracle.router_logits(x32, W)
    y2 = torch.empty_like(y)
    moe.moe_forward(d.ctx, 0, 4, _dev(x32), _dev(z), y2)
    assert torch.equal(y, y2)
    d.close()


REDUCED = Workload("decode-e64k8-h2048f1024-l4-b1-rot16", 101, 4, 64, 8, 2048, 1024, tokens=1, steps=40,
                   zipf_s=1.1, slots=26, rotation=16)


def test_decode_reduced_layers_bit_exact_policy():
    copies = {}
    worst = _run_decode(REDUCED, slots=26, check_every=8, copies=copies)
    print("worst token error", worst, "promotion bytes", copies)
    # batch 1 with logits: every cold pick captured its bytes, so no promotion
    # crossed PCIe a second time
    assert copies["copied"] > 0 and copies["pcie"] == 0


@pytest.mark.parametrize("capture_picks", [None, 0])
def test_promotions_every_miss_checked_every_step(capture_picks):
    # admit on the first miss: every step promotes, and every step's outputs
    # are checked, so an expert copied from its capture block (or from pinned
    # memory with capture off) is read from its new slot right away
    wl = REDUCED.with_(name="decode-e64k8-h2048f1024-l4-b1-admit1", steps=10, admit_misses=1)
    copies = {}
    _run_decode(wl, slots=26, check_every=1, capture_picks=capture_picks, copies=copies)
    assert copies["copied"] > 0
    assert copies["pcie"] == (0 if capture_picks is None else copies["copied"]), copies


def test_cold_start_admit_every_miss_many_copies_per_step():
    # every slot free and every miss admitted: the first steps admit dozens of
    # experts per layer, evicting some of their own newcomers again, so the
    # cache step's copies span several launches and repeat slots
    wl = Workload("decode-e64k8-h256f512-l3-b16-admit1", 108, 3, 64, 8, 256, 512, tokens=16, steps=6, zipf_s=0.9,
                  slots=24, rotation=5, admit_misses=1)
    _run_decode(wl, slots=24, check_every=1, seed=False)


def test_decode_batch_of_five_tokens():
    wl = Workload("decode-e64k8-h2048f1024-l2-b5", 102, 2, 64, 8, 2048, 1024, tokens=5, steps=12, zipf_s=1.1,
                  slots=20, rotation=20)
    _run_decode(wl, slots=20, check_every=3)


def test_decode_other_shapes_ragged_lanes():
    # hidden 4096 (two blocks per lane), ffn 1536 (48 blocks: 16 lanes x 3)
    wl = Workload("decode-e16k4-h4096f1536-l2-b3", 103, 2, 16, 4, 4096, 1536, tokens=3, steps=6, zipf_s=1.0,
                  slots=6)
    _run_decode(wl, slots=6, check_every=2)


# (E, k, H, F, tokens, slots): every routing path and lane layout the launches choose between
_SWEEP = [
    (3, 1, 256, 256, 1, 1),         # the smallest: one pick, one slot, 8 blocks per row (8 lanes x 1)
    (130, 3, 768, 512, 2, 40),      # E not a multiple of 64; 24 blocks per row (8 lanes x 3)
    (512, 8, 256, 256, 1, 100),     # the largest E the fused routing takes
    (64, 8, 1024, 3072, 1, 20),     # down rows of 96 blocks (32 lanes x 3)
    (33, 8, 512, 1024, 7, 12),      # the largest batch of the fused path
    (40, 5, 2048, 768, 9, 16),      # a grouped batch with an odd k
    (700, 4, 256, 256, 1, 100),     # E past the fused routing: the routing kernel
    (24, 12, 6144, 256, 2, 8),      # k > 8 (top-k by rounds); 192 blocks per row (64 lanes x 3)
    (20, 6, 1024, 1536, 12, 8),     # a grouped batch on the matrix cores, 72 picks over 20 experts
    (8, 8, 512, 512, 3, 4),         # k = E: every expert picked by every token
    (64, 4, 512, 512, 256, 16),     # the largest batch a context takes (grouped, 1024 picks)
]


@pytest.mark.parametrize("i", range(len(_SWEEP)))
def test_decode_shape_sweep(i):
    E, k, H, F, T, slots = _SWEEP[i]
    wl = Workload(f"sweep-e{E}k{k}-h{H}f{F}-b{T}", 300 + i, 2, E, k, H, F, tokens=T, steps=4, zipf_s=1.0,
                  slots=slots)
    _run_decode(wl, slots=slots, check_every=1)


def test_forced_cold_every_pick_over_pcie():
    wl = Workload("decode-e32k8-h2048f1024-l2-b2-cold", 104, 2, 32, 8, 2048, 1024, tokens=2, steps=6, zipf_s=1.1)
    _run_decode(wl, slots=0, check_every=2)


def test_noncoherent_pinned_arena():
    wl = Workload("decode-e32k8-h2048f1024-l2-b1-nc", 105, 2, 32, 8, 2048, 1024, tokens=1, steps=8, zipf_s=1.1,
                  slots=12)
    _run_decode(wl, slots=12, check_every=4, host_alloc=moe.MOE_HOST_NONCOHERENT)


def test_cold_start_without_seed():
    wl = Workload("decode-e32k4-h256f512-l3-b2-noseed", 106, 3, 32, 4, 256, 512, tokens=2, steps=40, zipf_s=1.1,
                  slots=8, rotation=30)
    _run_decode(wl, slots=8, check_every=10, seed=False)


def test_full_pool_never_misses():
    wl = Workload("decode-e16k4-h256f512-l2-b3-full", 107, 2, 16, 4, 256, 512, tokens=3, steps=5, zipf_s=1.1,
                  slots=16)
    d = Decode(wl)
    logits = zipf_logits(wl)
    y = torch.empty((3, 256), dtype=torch.float32, device="cuda")
    for step in range(5):
        x = _dev(activations(wl, step))
        for layer in range(2):
            moe.moe_forward(d.ctx, layer, 3, x, _dev(logits[step, layer]), y)
        st = moe.moe_cache_step(d.ctx)
        assert st["misses"] == 0 and st["hits"] == 2 * 3 * 4
    d.close()


def test_accumulate_in_place():
    wl = Workload("decode-e16k4-h256f512-l1-b2-acc", 108, 1, 16, 4, 256, 512, tokens=2, zipf_s=1.1, slots=8)
    d = Decode(wl)
    z = _dev(zipf_logits(wl)[0, 0])
    x = _dev(activations(wl, 0))
    y = torch.empty_like(x)
    moe.moe_forward(d.ctx, 0, 2, x, z, y)
    x2 = x.clone()
    moe.moe_forward(d.ctx, 0, 2, x2, z, x2, flags=moe.MOE_ACCUMULATE)
    torch.testing.assert_close(x2, x + y, rtol=0, atol=0)
    d.close()


def test_graph_capture_replays_match_eager():
    wl = Workload("decode-e64k8-h2048f1024-l3-b1-graph", 109, 3, 64, 8, 2048, 1024, tokens=1, steps=10,
                  zipf_s=1.1, slots=24, rotation=4)
    s = torch.cuda.Stream()
    eager = Decode(wl, stream=s)
    graph = Decode(wl, stream=s)
    logits = zipf_logits(wl)
    L, H = wl.n_layers, wl.hidden
    xs = torch.zeros((L, 1, H), dtype=torch.float32, device="cuda")
    zs = torch.zeros((L, 1, wl.n_experts), dtype=torch.float32, device="cuda")
    ys = [torch.zeros((1, H), dtype=torch.float32, device="cuda") for _ in range(L)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for layer in range(L):
                moe.moe_forward(graph.ctx, layer, 1, xs[layer], zs[layer], ys[layer])
    pol = oracle_policy(wl, 24)
    for step in range(wl.steps):
        with torch.cuda.stream(s):
            xs.copy_(_dev(step_activations(wl, step)))
            zs.copy_(_dev(logits[step]))
            g.replay()
            st_g = moe.moe_cache_step(graph.ctx)
            ye = torch.empty((1, H), dtype=torch.float32, device="cuda")
            for layer in range(L):
                xe = _dev(activations(wl, step, layer=layer))
                moe.moe_forward(eager.ctx, layer, 1, xe, _dev(logits[step, layer]), ye)
                assert torch.equal(ye, ys[layer]), (step, layer)
                pol.forward(layer, oracle.route(logits[step, layer], wl.top_k)[0])
            st_e = moe.moe_cache_step(eager.ctx)
        s.synchronize()
        st_o = pol.step()
        assert st_g == st_e
        _compare_policy(graph, pol, st_g, st_o, range(L))
    eager.close()
    graph.close()


def test_error_codes():
    wl = Workload("decode-e16k4-h256f512-l2-b2-err", 110, 2, 16, 4, 256, 512, tokens=2, zipf_s=1.1, slots=4)
    d = Decode(wl, seed=None)
    x = torch.zeros((2, 256), dtype=torch.float32, device="cuda")
    z = torch.zeros((2, 16), dtype=torch.float32, device="cuda")
    y = torch.zeros_like(x)

    def code(fn, *a, **kw):
        with pytest.raises(moe.MoeError) as ei:
            fn(*a, **kw)
        return ei.value.code

    assert code(moe.moe_forward, d.ctx, 0, 2, x, z, y) == moe.MOE_E_STATE  # before seed
    assert code(moe.moe_cache_step, d.ctx) == moe.MOE_E_STATE
    moe.moe_seed(d.ctx, d.freq)
    g = d.weights[0]
    assert code(moe.moe_register_layer, d.ctx, 0, *g) == moe.MOE_E_STATE  # after seed
    assert code(moe.moe_forward, d.ctx, 2, 2, x, z, y) == moe.MOE_E_INVAL  # layer out of range
    assert code(moe.moe_forward, d.ctx, 0, 3, x, z, y) == moe.MOE_E_INVAL  # more tokens than max_batch
    assert code(moe.moe_forward, d.ctx, 0, 0, x, z, y) == moe.MOE_E_INVAL
    assert code(moe.moe_forward, d.ctx, 0, 2, x, z, x) == moe.MOE_E_INVAL  # alias without accumulate
    xb = torch.zeros(2 * 256 + 1, dtype=torch.float32, device="cuda")[1:].view(2, 256)
    assert code(moe.moe_forward, d.ctx, 0, 2, xb, z, y) == moe.MOE_E_INVAL  # misaligned
    assert code(moe.moe_forward, d.ctx, 0, 2, x, None, y) == moe.MOE_E_INVAL  # no router
    assert "router" in moe.moe_last_error(d.ctx)
    # cache step inside a capture
    s = torch.cuda.Stream()
    d2 = Decode(wl, stream=s)
    cg = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(cg, stream=s):
            x.mul_(1.0)
            rc = moe.lib().moe_cache_step(d2.ctx, None)
            rc_seed = moe.lib().moe_seed(d2.ctx, None)
    assert rc == moe.MOE_E_CAPTURING and rc_seed == moe.MOE_E_CAPTURING
    d2.close()
    # a pool larger than the device
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_create(64, 4096, 4, 4096, 4096, pool_budget_bytes=1 << 50)  # 7.4 TB pool
    assert ei.value.code in (moe.MOE_E_NOMEM,)
    d.close()


def test_shared_host_sets():
    # 5 layers over 2 pinned host sets: layer l reads set l % 2 (weights of layer l % 2)
    wl = Workload("decode-e32k8-h2048f1024-l5-b2-sets", 111, 5, 32, 8, 2048, 1024, tokens=2, steps=10, zipf_s=1.1,
                  slots=10, rotation=5, distinct_layers=2)
    _run_decode(wl, slots=10, check_every=3)


@pytest.mark.parametrize("launches", [1, 2])
def test_kernel_timing_hook(launches):
    wl = Workload("decode-e32k8-h2048f1024-l3-b2-prof", 112, 3, 32, 8, 2048, 1024, tokens=2, steps=4, zipf_s=1.1,
                  slots=12)
    d = Decode(wl, decode_launches=launches)
    logits = zipf_logits(wl)
    y = torch.empty((2, 2048), dtype=torch.float32, device="cuda")
    moe.moe_profile(d.ctx, 1)
    tot = {"hits": 0, "misses": 0}
    for step in range(wl.steps):
        x = _dev(activations(wl, step))
        for layer in range(3):
            moe.moe_forward(d.ctx, layer, 2, x, _dev(logits[step, layer]), y)
        st = moe.moe_cache_step(d.ctx)
        tot["hits"] += st["hits"]
        tot["misses"] += st["misses"]
    prof = moe.moe_profile(d.ctx, 0)
    assert prof["forwards"] == 3 * wl.steps
    assert prof["hot_picks"] == tot["hits"] and prof["cold_picks"] == tot["misses"]
    assert tot["hits"] + tot["misses"] == wl.steps * 3 * 2 * 8
    if launches == 2:
        for key in ("hot_gateup_ms", "hot_down_ms", "cold_gateup_ms", "cold_down_ms"):
            assert prof[key] > 0, key
        assert prof["layer_forwards"] == 0 and prof["hot_layer_ms"] == 0 and prof["cold_layer_ms"] == 0
    else:  # one launch per layer: timed as a hot and a cold launch
        assert prof["layer_forwards"] == 3 * wl.steps
        assert prof["hot_layer_ms"] > 0 and prof["cold_layer_ms"] > 0
        for key in ("hot_gateup_ms", "hot_down_ms", "cold_gateup_ms", "cold_down_ms"):
            assert prof[key] == 0, key
    assert prof["route_ms"] == 0  # with logits the gate/up launches route by themselves
    assert prof["gateup_bytes_per_pick"] + prof["down_bytes_per_pick"] == wl.expert_bytes
    # a router chain runs (and is timed) in its own launch
    tiny = WORKLOADS["tiny-e8k2-h256f512-t4"]
    dt = Decode(tiny)
    moe.moe_register_router(dt.ctx, 0, router_weights(tiny, 0))
    moe.moe_profile(dt.ctx, 1)
    yt = torch.empty((4, 256), dtype=torch.float32, device="cuda")
    moe.moe_forward(dt.ctx, 0, 4, _dev(activations(tiny, 0)), None, yt)
    moe.moe_cache_step(dt.ctx)
    assert moe.moe_profile(dt.ctx, 0)["route_ms"] > 0
    dt.close()
    # timing on: the forward refuses graph capture
    s = torch.cuda.Stream()
    d2 = Decode(wl, stream=s)
    moe.moe_profile(d2.ctx, 1)
    g = torch.cuda.CUDAGraph()
    xs = torch.zeros((2, 2048), dtype=torch.float32, device="cuda")
    zs = torch.zeros((2, 32), dtype=torch.float32, device="cuda")
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            xs.mul_(1.0)
            rc = moe.lib().moe_forward(d2.ctx, 0, 2, xs.data_ptr(), zs.data_ptr(), xs.data_ptr(), None, None,
                                       moe.MOE_ACCUMULATE)
    assert rc == moe.MOE_E_CAPTURING
    d2.close()
    d.close()


def test_global_pool_bit_exact_policy():
    # one pool of 104 slots (the memory of 26 per layer) shared by the 4 layers:
    # admissions evict whichever layer's expert holds the oldest stamp
    copies = {}
    worst = _run_decode(REDUCED.with_(name="decode-e64k8-h2048f1024-l4-b1-global"), slots=104, check_every=5,
                        pool="global", copies=copies)
    print("worst token error", worst, "promotion bytes", copies)
    assert copies["copied"] > 0 and copies["pcie"] == 0


def test_global_pool_cold_start_batch():
    wl = Workload("decode-e32k4-h256f512-l3-b2-global", 113, 3, 32, 4, 256, 512, tokens=2, steps=30, zipf_s=1.1,
                  slots=8, rotation=20)
    _run_decode(wl, slots=24, check_every=6, seed=False, pool="global")


@pytest.mark.parametrize("capture_picks,budget,lead", [(0, 3, 1), (None, 3, 1), (0, 0, 2), (None, 0, 2)])
def test_swap_budget_and_lead_bit_exact(capture_picks, budget, lead):
    # admit on the first miss, so every step wants more swaps than the budget
    # allows; every step's outputs are checked, so a slot read before its copy
    # landed (pinned copies run on the swap stream beside the next steps) shows
    wl = REDUCED.with_(name="decode-e64k8-h2048f1024-l4-b1-swaps", steps=14, admit_misses=1)
    copies = {}
    _run_decode(wl, slots=26, check_every=1, capture_picks=capture_picks, copies=copies, swaps=(budget, lead))
    assert copies["copied"] > 0
    assert copies["pcie"] == (0 if capture_picks is None else copies["copied"]), copies


def test_swap_lead_global_pool_window_admission():
    _run_decode(REDUCED.with_(name="decode-e64k8-h2048f1024-l4-b1-global-lead"), slots=104, check_every=4,
                pool="global", capture_picks=0, swaps=(4, 1))


# ---------------------------------------------------------------------------
# cold picks computed by the host threads (cold_exec = MOE_COLD_CPU)

@pytest.mark.parametrize("cpu_threads", [0, 3])
def test_cold_picks_on_host_threads_bit_exact_policy(cpu_threads):
    # every step's outputs checked: cold picks come from the host's answer,
    # hot ones from the GPU, summed in pick order
    wl = REDUCED.with_(name="decode-e64k8-h2048f1024-l4-b1-hostcold", steps=16)
    copies = {}
    _run_decode(wl, slots=26, check_every=1, copies=copies, cold_exec=moe.MOE_COLD_CPU, cpu_threads=cpu_threads)
    # nothing was captured: every promotion is a copy from pinned memory
    assert copies["copied"] > 0 and copies["pcie"] == copies["copied"]


def test_cold_picks_on_host_threads_batch_shared_experts():
    # five tokens per step: tokens that picked the same cold expert share one
    # pass of the host threads over its weights
    wl = Workload("decode-e64k8-h2048f1024-l2-b5-hostcold", 102, 2, 64, 8, 2048, 1024, tokens=5, steps=8,
                  zipf_s=1.1, slots=20, rotation=20)
    _run_decode(wl, slots=20, check_every=1, cold_exec=moe.MOE_COLD_CPU)


def test_cold_picks_on_host_threads_global_pool_swap_lead_cold_start():
    wl = Workload("decode-e32k4-h256f512-l3-b2-hostcold", 113, 3, 32, 4, 256, 512, tokens=2, steps=24, zipf_s=1.1,
                  slots=8, rotation=12)
    _run_decode(wl, slots=24, check_every=3, seed=False, pool="global", swaps=(3, 1), cold_exec=moe.MOE_COLD_CPU)


def test_cold_picks_on_host_threads_accumulate_and_errors():
    wl = Workload("decode-e32k4-h256f512-l1-b3-hostcold", 114, 1, 32, 4, 256, 512, tokens=3, steps=1, zipf_s=1.1,
                  slots=0)
    d = Decode(wl, slots=0, cold_exec=moe.MOE_COLD_CPU, cpu_threads=2)  # every pick cold
    x32 = activations(wl, 0)
    z = zipf_logits(wl)[0, 0]
    y0 = np.random.default_rng(1).standard_normal((3, 256)).astype(np.float32)
    y = _dev(y0)
    moe.moe_forward(d.ctx, 0, 3, _dev(x32), _dev(z), y, flags=moe.MOE_ACCUMULATE)
    ids, _ = oracle.route(z, 4)
    y_ref, _, _ = oracle.moe_layer(32, 4, 256, 512, d.experts(0, ids), x32.astype(np.float64), logits=z)
    assert token_rel_err(y.cpu().numpy() - y0, y_ref) < TOL
    st = moe.moe_cache_step(d.ctx)
    assert st["misses"] == 12 and st["hits"] == 0
    # the hand-off needs logits
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_forward(d.ctx, 0, 3, _dev(x32), None, y)
    assert ei.value.code == moe.MOE_E_INVAL
    # and is not capturable
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    xd, zd = _dev(x32), _dev(z)
    d2 = Decode(wl, slots=0, cold_exec=moe.MOE_COLD_CPU, cpu_threads=2, stream=s)
    with torch.cuda.stream(s):
        g.capture_begin()
        rc = moe.lib().moe_forward(d2.ctx, 0, 3, xd.data_ptr(), zd.data_ptr(), y.data_ptr(), None, None, 0)
        g.capture_end()
    assert rc == moe.MOE_E_CAPTURING
    d2.close()
    d.close()
    # capture of cold reads has nothing to capture with host threads
    with pytest.raises(moe.MoeError):
        moe.moe_create(1, 32, 4, 256, 512, 0, cold_exec=moe.MOE_COLD_CPU, capture_picks=4)


# ---------------------------------------------------------------------------
# grouped decode: batches of 8 tokens or more read each expert's weights once

@pytest.mark.parametrize("tokens", [8, 12])
def test_grouped_batch_bit_exact_policy(tokens):
    wl = Workload(f"decode-e64k8-h2048f1024-l2-b{tokens}-grouped", 115, 2, 64, 8, 2048, 1024, tokens=tokens, steps=10,
                  zipf_s=1.1, slots=20, rotation=40)
    copies = {}
    _run_decode(wl, slots=20, check_every=1, copies=copies)
    assert copies["copied"] > 0  # promotions happen (from pinned memory: the grouped path captures nothing)


def test_grouped_batch_global_pool_cold_start_swap_lead():
    wl = Workload("decode-e32k4-h256f512-l3-b16-grouped", 116, 3, 32, 4, 256, 512, tokens=16, steps=16, zipf_s=0.9,
                  slots=8, rotation=24)
    _run_decode(wl, slots=24, check_every=2, seed=False, pool="global", swaps=(4, 1))


@pytest.mark.gpu
def test_read_bandwidth_ceilings():
    """The streaming-read measurement aid: HBM from a device buffer, PCIe from
    pinned host memory in both coherence modes; bad arguments rejected on the host."""
    buf = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    hbm = moe.moe_measure_read_bandwidth(buf, reps=2)
    assert 100.0 < hbm < 20000.0, hbm
    for coherent in (True, False):
        pcie = moe.moe_measure_read_bandwidth(None, 16 << 20, reps=1, host_coherent=coherent)
        assert 1.0 < pcie < 200.0, (coherent, pcie)
    with pytest.raises(moe.MoeError):
        moe.moe_measure_read_bandwidth(None, 15, reps=1)  # not a multiple of 16
    with pytest.raises(moe.MoeError):
        moe.moe_measure_read_bandwidth(buf, reps=0)


@pytest.mark.gpu
@pytest.mark.parametrize("E,k", [(64, 8), (96, 12), (600, 6), (8, 2)])
def test_routing_exact_ties_and_signed_zeros(E, k):
    """Every top-k path: the sorting-network top-8 of the fused launch (k <= 8,
    E <= 512), its rounds (k > 8) and the routing kernel (E > 512), on logits
    full of exact ties and signed zeros. Ids bit-exact against the oracle
    (larger logit first, equal logits lower id first, -0 equal to +0); weights
    and outputs within tolerance."""
    T, H, F = 4, 256, 512
    wl = Workload(f"route-ties-e{E}k{k}", 117, 1, E, k, H, F, tokens=T, steps=1, zipf_s=1.1, slots=E // 2)
    d = Decode(wl, slots=E // 2)
    rng = np.random.default_rng(1000 * E + k)
    z = (np.round(rng.standard_normal((T, E)) * 2.0) / 2.0).astype(np.float32)  # steps of 0.5: many ties
    z[0, : k + 3] = 3.0  # more equal maxima than picks
    z[1] = -np.abs(z[1]) - 0.5
    z[1, ::5], z[1, 2::5] = -0.0, 0.0  # the largest values are signed zeros
    z[3] = 1.0  # every logit equal
    x32 = activations(wl, 0)
    y = torch.empty((T, H), dtype=torch.float32, device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    moe.moe_forward(d.ctx, 0, T, _dev(x32), _dev(z), y, ids, w)
    ids_ref, w_ref = oracle.route(z, k)
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    np.testing.assert_allclose(w.cpu().numpy(), w_ref, rtol=2e-6)
    g, u, dn = d.weights[0]
    y_ref, _, _ = oracle.moe_layer(E, k, H, F, {int(e): (g[e], u[e], dn[e]) for e in np.unique(ids_ref)},
                                   x32.astype(np.float64), logits=z)
    assert token_rel_err(y.cpu().numpy(), y_ref) < TOL
    d.close()


def test_fused_path_slot_taken_twice_in_one_step_copies_from_capture():
    # 4 tokens (the fused routing + gate/up path), every pick may capture, every miss admitted, 3 slots per
    # layer: a step admits more experts than a layer has slots, so one copy list holds two transfers to one
    # slot (only the later one must land), and every promotion copies a capture block, none crosses PCIe
    wl = Workload("decode-e32k4-h256f512-l2-b4-admit1-s3", 117, 2, 32, 4, 256, 512, tokens=4, steps=8,
                  zipf_s=0.6, slots=3, admit_misses=1)
    copies, repeats = {}, []
    _run_decode(wl, slots=3, check_every=1, capture_picks=16, copies=copies, repeats=repeats)
    print("repeated slots per step", repeats, "promotion bytes", copies)
    assert sum(repeats) > 0
    assert copies["copied"] > 0 and copies["pcie"] == 0


def test_second_forward_of_a_layer_in_a_step_leaves_no_stale_capture():
    # A fused forward captures expert 3 (cold, second miss) into capture block 0; a second forward of the
    # same layer in the same step (8 tokens: routed by the routing kernel) puts expert 5 at pick 0, and 5 is
    # admitted by its second miss. Its promotion must not copy block 0 (expert 3's bytes) into 5's slot.
    E, k, H, F = 16, 2, 256, 512
    wl = Workload("decode-e16k2-h256f512-l1-twice", 118, 1, E, k, H, F, tokens=8, zipf_s=1.1, slots=4)
    d = Decode(wl, slots=4, seed=False, max_batch=8, capture_picks=8 * k)
    try:
        def logits(rows):
            z = np.zeros((len(rows), E), np.float32)
            for t, (a, b) in enumerate(rows):
                z[t, a], z[t, b] = 10.0, 9.0
            return z

        def forward(rows, step):
            z = logits(rows)
            x32 = activations(wl, step, tokens=len(rows))
            y = torch.empty((len(rows), H), dtype=torch.float32, device="cuda")
            moe.moe_forward(d.ctx, 0, len(rows), _dev(x32), _dev(z), y)
            return x32, z, y

        forward([(3, 5)], 0)
        st = moe.moe_cache_step(d.ctx)
        assert st["misses"] == 2 and st["admissions"] == 0
        forward([(3, 7)], 1)                                  # 3 captured at pick 0
        forward([(5, 9)] + [(10 + t % 6, 2) for t in range(7)], 2)  # same layer, same step: pick 0 is 5
        st = moe.moe_cache_step(d.ctx)
        table = moe.moe_get_slot_table(d.ctx, 0, E)
        assert table[5] >= 0 and table[3] < 0, table
        x32, z, y = forward([(5, 3)], 3)                      # 5 from its new slot
        y_ref, _, _ = oracle.moe_layer(E, k, H, F, d.experts(0, [5, 3]), x32.astype(np.float64), logits=z)
        err = token_rel_err(y.cpu().numpy(), y_ref)
        assert err < TOL, err
    finally:
        d.close()


def test_grouped_cold_experts_staged_then_promoted_from_capture():
    # 16 tokens at hidden 2048 / ffn 1024 take the grouped matrix-core path; every miss is admitted and
    # every cold group has a capture block, so each cold expert crosses PCIe once (staged into its block
    # before its products) and every promotion copies that block: no promotion bytes over PCIe, and the
    # promoted experts are read from their new slots by the next step, checked every step
    wl = Workload("decode-e64k8-h2048f1024-l2-b16-stage", 120, 2, 64, 8, 2048, 1024, tokens=16, steps=6,
                  zipf_s=0.8, slots=16, admit_misses=1)
    copies = {}
    _run_decode(wl, slots=16, check_every=1, capture_picks=16 * 8, copies=copies)
    print("promotion bytes", copies)
    assert copies["copied"] > 0 and copies["pcie"] == 0


@pytest.mark.gpu
@pytest.mark.parametrize("E,k,H,F,T,slots", [(64, 8, 2048, 1024, 1, 24), (64, 8, 2048, 1024, 3, 24),
                                            (16, 4, 4096, 1536, 2, 6), (32, 4, 256, 512, 7, 10),
                                            (8, 2, 256, 512, 4, 3)])
def test_one_launch_layer_matches_two_launches_bitwise(E, k, H, F, T, slots):
    """The one-launch layer kernel (gate/up and down work-groups in one grid, the down ones waiting on
    a device counter) against the two-launch path on the same inputs: picks, weights, outputs (every
    forward, MOE_ACCUMULATE on odd layers), tables, stamps and miss logs bit-identical, hot and cold
    picks mixed, captures on; the first step also against the oracle."""
    wl = Workload(f"layer-ab-e{E}k{k}-h{H}f{F}-b{T}", 121, 2, E, k, H, F, tokens=T, steps=5, zipf_s=1.0,
                  slots=slots)
    one = Decode(wl, slots=slots, decode_launches=1)
    two = Decode(wl, slots=slots, decode_launches=2)
    logits = zipf_logits(wl)
    outs = {}
    try:
        for step in range(wl.steps):
            for layer in range(wl.n_layers):
                x32 = activations(wl, step, layer=layer)
                flags = moe.MOE_ACCUMULATE if layer % 2 else 0
                base = torch.from_numpy(activations(wl, step + 100, layer=layer)).cuda()
                for name, d in (("one", one), ("two", two)):
                    y = base.clone()
                    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
                    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
                    moe.moe_forward(d.ctx, layer, T, _dev(x32), _dev(logits[step, layer]), y, ids, w, flags=flags)
                    outs[name] = (y.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy())
                for a, b in zip(outs["one"], outs["two"]):
                    assert np.array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                                          b.view(np.uint32) if b.dtype == np.float32 else b), (step, layer)
                if step == 0:
                    ids_o, _ = oracle.route(logits[step, layer], k)
                    y_ref, _, _ = oracle.moe_layer(E, k, H, F, one.experts(layer, ids_o), x32.astype(np.float64),
                                                   logits=logits[step, layer])
                    y_one = outs["one"][0] - (base.cpu().numpy() if flags else 0)
                    assert token_rel_err(y_one, y_ref) < TOL, (layer, token_rel_err(y_one, y_ref))
            s1, s2 = moe.moe_cache_step(one.ctx), moe.moe_cache_step(two.ctx)
            assert s1 == s2, (step, s1, s2)
            for layer in range(wl.n_layers):
                assert np.array_equal(moe.moe_get_slot_table(one.ctx, layer, E), moe.moe_get_slot_table(two.ctx, layer, E))
                assert np.array_equal(moe.moe_get_stamps(one.ctx, layer, slots), moe.moe_get_stamps(two.ctx, layer, slots))
            assert np.array_equal(moe.moe_get_miss_log(one.ctx), moe.moe_get_miss_log(two.ctx))
            assert s1["misses"] > 0 or step > 0
    finally:
        one.close()
        two.close()


@pytest.mark.gpu
def test_one_launch_layer_wait_bound_is_reported():
    # A wait bound of one poll, every pick cold (an empty pool: gate/up reads cross PCIe, tens of
    # microseconds): the down work-groups give up at once, go on, and the cache step reports it. Every
    # kernel still ends; the counters are cleared by the step that reports the error.
    wl = Workload("layer-bound-e32k8-h2048f1024", 122, 1, 32, 8, 2048, 1024, tokens=1, steps=1, zipf_s=1.0,
                  slots=4)
    d = Decode(wl, slots=4, seed=False, decode_launches=1, decode_sync_polls=1)
    try:
        z = zipf_logits(wl)[0, 0]
        y = torch.empty((1, 2048), dtype=torch.float32, device="cuda")
        moe.moe_forward(d.ctx, 0, 1, _dev(activations(wl, 0)), _dev(z), y)
        with pytest.raises(moe.MoeError) as ei:
            moe.moe_cache_step(d.ctx)
        assert ei.value.code == moe.MOE_E_HIP and "gave up waiting" in str(ei.value)
    finally:
        d.close()
    # a default bound on the same work is exact
    d = Decode(wl, slots=4, seed=False, decode_launches=1)
    try:
        x32 = activations(wl, 0)
        moe.moe_forward(d.ctx, 0, 1, _dev(x32), _dev(z), y)
        moe.moe_cache_step(d.ctx)
        ids_o, _ = oracle.route(z, 8)
        y_ref, _, _ = oracle.moe_layer(32, 8, 2048, 1024, d.experts(0, ids_o), x32.astype(np.float64), logits=z)
        assert token_rel_err(y.cpu().numpy(), y_ref) < TOL
    finally:
        d.close()


@pytest.mark.gpu
@pytest.mark.parametrize("T", [1, 5])
def test_decode_activations_of_mixed_magnitude(T):
    """Decode activations far from unit scale: rows scaled by 1e3 and 1e-4, single huge values inside a
    block of small ones, blocks of exact zeros and of subnormal values. Every output within the tolerance
    of the oracle (fp64), on hot and cold picks."""
    E, k, H, F = 32, 8, 2048, 1024
    wl = Workload(f"decode-mixed-e{E}k{k}-b{T}", 123, 1, E, k, H, F, tokens=T, steps=1, zipf_s=1.0, slots=16)
    d = Decode(wl, slots=16)
    try:
        rng = np.random.default_rng(77 + T)
        x32 = activations(wl, 0)
        x32[0] *= 1e3
        if T > 1:
            x32[1] *= 1e-4
            x32[2, ::32] = 5e4           # one huge value per block, the rest N(0, 1)
            x32[3, 64:256] = 0.0         # whole blocks of zeros
            x32[4, :32] = rng.standard_normal(32).astype(np.float32) * 1e-40  # subnormal block
        z = zipf_logits(wl)[0, 0]
        y = torch.empty((T, H), dtype=torch.float32, device="cuda")
        moe.moe_forward(d.ctx, 0, T, _dev(x32), _dev(z), y)
        ids_o, _ = oracle.route(z, k)
        y_ref, _, _ = oracle.moe_layer(E, k, H, F, d.experts(0, ids_o), x32.astype(np.float64), logits=z)
        err = token_rel_err(y.cpu().numpy(), y_ref)
        print("mixed-magnitude decode error", err)
        assert err < TOL, err
        st = moe.moe_cache_step(d.ctx)
        assert st["hits"] > 0 and st["misses"] > 0, st
    finally:
        d.close()
