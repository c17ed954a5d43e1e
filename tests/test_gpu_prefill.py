"""GPU parity of the prompt pass (sort by expert, staging, fp16-MFMA grouped
GEMMs, combine) through the C ABI against the oracle, and its neutrality
towards the cache policy."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import moe_expert_offload_gemv_amd as moe  # noqa: E402
import oracle  # noqa: E402
from tests._gpu import TOL, Decode, token_rel_err  # noqa: E402
from workload import WORKLOADS, Workload, activations, router_weights, zipf_logits  # noqa: E402

pytestmark = pytest.mark.gpu


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _prefill_check(wl: Workload, slots: int, sample=None, flags=0, pool="layer", seed=True, x_scale=None):
    """x_scale: a factor for every activation, or an array of one factor per token."""
    d = Decode(wl, slots=slots, max_batch=1, max_prefill=wl.tokens, pool=pool, seed=seed)
    T, H = wl.tokens, wl.hidden
    x32 = activations(wl, 0, tokens=T)
    if x_scale is not None:
        x32 = (x32 * np.asarray(x_scale, np.float32).reshape(-1, 1)).astype(np.float32)
    z = zipf_logits(wl, steps=1, tokens=T)[0, 0]
    x = _dev(x32)
    y = _dev(np.full((T, H), 0.25, np.float32)) if flags else torch.empty((T, H), dtype=torch.float32, device="cuda")
    tbl0 = [moe.moe_get_slot_table(d.ctx, layer, wl.n_experts) for layer in range(wl.n_layers)]
    moe.moe_profile(d.ctx, 1)
    moe.moe_prefill(d.ctx, 0, T, x, _dev(z), y, flags)
    prof = moe.moe_profile(d.ctx, 0)
    yh = y.cpu().numpy().astype(np.float64)
    if flags:
        yh -= 0.25
    rows = np.arange(T) if sample is None else np.random.default_rng(0).choice(T, size=sample, replace=False)
    ids, _ = oracle.route(z[rows], wl.top_k)
    y_ref, ids_ref, _ = oracle.moe_layer(wl.n_experts, wl.top_k, H, wl.ffn, d.experts(0, ids), x32[rows].astype(
        np.float64), logits=z[rows])
    err = token_rel_err(yh[rows], y_ref)
    print(f"{wl.name}: worst token error {err:.2e}")
    assert err < TOL, err
    # policy neutral: tables, stamps, counts, clock untouched
    for layer in range(wl.n_layers):
        assert np.array_equal(moe.moe_get_slot_table(d.ctx, layer, wl.n_experts), tbl0[layer])
        assert d.S == 0 or not moe.moe_get_stamps(d.ctx, layer, d.S).any()
    assert not moe.moe_get_counts(d.ctx, wl.n_layers, wl.n_experts).any()
    assert moe.moe_get_info(d.ctx)["clock"] == 1
    assert prof["prefill_passes"] == 1 and prof["prefill_pairs"] == T * wl.top_k
    assert (prof["prefill_stage_ms"] > 0) == (prof["prefill_staged"] > 0)
    d.close()
    return err, prof


def test_prefill_small_ragged_tiles_with_staging():
    wl = Workload("prefill-e16k4-h256f512-t37", 201, 1, 16, 4, 256, 512, tokens=37, zipf_s=1.1)
    err, prof = _prefill_check(wl, slots=8)
    assert prof["prefill_staged"] > 0
    print("err", err, prof)


# (E, k, H, F, tokens, slots): ragged tiles, the routing paths, the lane layouts of the decode kernels the
# context shares
_SWEEP = [
    (3, 1, 256, 256, 1, 1),       # one token, one pick
    (130, 3, 768, 512, 65, 40),   # E not a multiple of 64, a 65-row expert at most
    (64, 8, 1024, 3072, 20, 20),  # K of the down GEMM 3072
    (24, 12, 6144, 256, 33, 8),   # k > 8, K of the gate/up GEMM 6144
    (700, 4, 256, 256, 50, 100),  # E past the fused routing
    (8, 8, 512, 512, 40, 4),      # k = E: every expert picked by every token
]


@pytest.mark.parametrize("i", range(len(_SWEEP)))
def test_prefill_shape_sweep(i):
    E, k, H, F, T, slots = _SWEEP[i]
    wl = Workload(f"pf-sweep-e{E}k{k}-h{H}f{F}-t{T}", 320 + i, 1, E, k, H, F, tokens=T, zipf_s=1.0)
    _prefill_check(wl, slots=slots)


def test_prefill_many_tiles_per_expert():
    wl = Workload("prefill-e8k2-h256f512-t1000", 202, 1, 8, 2, 256, 512, tokens=1000, zipf_s=1.1)
    err, prof = _prefill_check(wl, slots=3, sample=200)
    assert prof["prefill_tiles"] > 8


def test_prefill_dma_staging_beside_long_gemms():
    # one staged expert against ~7000 pairs of resident ones: the copy hides
    # behind the GEMMs, so it goes to the DMA engines instead of the gather kernel
    wl = Workload("prefill-e8k2-h256f512-t4000", 208, 1, 8, 2, 256, 512, tokens=4000, zipf_s=1.1)
    err, prof = _prefill_check(wl, slots=7, sample=160)
    assert prof["prefill_staged"] == 1


def test_prefill_cold_pool_more_misses_than_staging_blocks():
    # cold start: every slot free, so all 16 experts miss but only E - S = 8
    # staging blocks exist; the other 8 are read zero-copy beside the gathers
    wl = Workload("prefill-e16k4-h256f512-t100-coldpool", 209, 1, 16, 4, 256, 512, tokens=100, zipf_s=0.6)
    err, prof = _prefill_check(wl, slots=8, seed=False)
    assert prof["prefill_staged"] == 8


def test_prefill_most_experts_the_layout_allows():
    # E = 4096: the counting sort's per-chunk counters fill 16 KiB of LDS, and
    # ~500 staged experts go through all eight gather chunks
    wl = Workload("prefill-e4096k8-h256f512-t64", 210, 1, 4096, 8, 256, 512, tokens=64, zipf_s=0.8)
    err, prof = _prefill_check(wl, slots=64)
    assert prof["prefill_staged"] > 8 * 16


def test_prefill_decode_shape():
    wl = Workload("prefill-e64k8-h2048f1024-t300", 203, 1, 64, 8, 2048, 1024, tokens=300, zipf_s=1.1)
    _prefill_check(wl, slots=26, sample=48)


def test_prefill_wide_shape_all_resident():
    wl = Workload("prefill-e16k8-h4096f1536-t90", 204, 1, 16, 8, 4096, 1536, tokens=90, zipf_s=1.0)
    err, prof = _prefill_check(wl, slots=16, sample=24)
    assert prof["prefill_staged"] == 0


def test_prefill_all_cold_and_accumulate():
    wl = Workload("prefill-e16k4-h256f512-t20-cold", 205, 1, 16, 4, 256, 512, tokens=20, zipf_s=1.1)
    err, prof = _prefill_check(wl, slots=0, flags=moe.MOE_ACCUMULATE)
    assert prof["prefill_staged"] == len(set(oracle.route(zipf_logits(wl, steps=1, tokens=20)[0, 0], 4)[0].ravel()))


def test_prefill_router_in_the_loop_matches_decode():
    wl = WORKLOADS["tiny-e8k2-h256f512-t4"]
    d = Decode(wl, max_batch=4, max_prefill=4)
    moe.moe_register_router(d.ctx, 0, router_weights(wl, 0))
    x = _dev(activations(wl, 0))
    y1 = torch.empty_like(x)
    y2 = torch.empty_like(x)
    moe.moe_prefill(d.ctx, 0, 4, x, None, y1)
    moe.moe_forward(d.ctx, 0, 4, x, None, y2)
    # two different kernels on the same routing: the fp32 GEMV and the grouped
    # GEMM on fp16 operands (weights and activations rounded once each, ~5e-4
    # apart at this shape), so the bar is the one both meet against the oracle
    assert token_rel_err(y1.cpu().numpy(), y2.cpu().numpy().astype(np.float64)) < TOL
    d.close()


def test_prefill_between_decode_steps_leaves_policy_identical():
    wl = Workload("decode-e32k8-h256f512-l2-b1-pf", 206, 2, 32, 8, 256, 512, tokens=1, steps=12, zipf_s=1.1,
                  slots=10, rotation=4)
    logits = zipf_logits(wl)
    xp = _dev(activations(wl, 99, tokens=50))
    zp = _dev(zipf_logits(wl, steps=1, tokens=50)[0, 1])
    yp = torch.empty_like(xp)
    runs = []
    for with_prefill in (False, True):
        d = Decode(wl, max_prefill=50)
        y = torch.empty((1, 256), dtype=torch.float32, device="cuda")
        out = []
        for step in range(wl.steps):
            x = _dev(activations(wl, step))
            for layer in range(2):
                moe.moe_forward(d.ctx, layer, 1, x, _dev(logits[step, layer]), y)
                x += y
            if with_prefill and step % 3 == 1:
                moe.moe_prefill(d.ctx, 1, 50, xp, zp, yp)
            st = moe.moe_cache_step(d.ctx)
            out.append((st, [moe.moe_get_slot_table(d.ctx, layer, 32).tolist() for layer in range(2)],
                        moe.moe_get_miss_log(d.ctx).tolist(), x.cpu().numpy().tolist()))
        runs.append(out)
        d.close()
    assert runs[0] == runs[1]


def test_prefill_with_global_pool():
    # three layers share 20 slots; layer 2's pass stages whatever the pool lacks
    wl = Workload("prefill-e16k4-h256f512-t50-global", 206, 3, 16, 4, 256, 512, tokens=50, zipf_s=1.1)
    d = Decode(wl, slots=20, max_batch=1, max_prefill=wl.tokens, pool="global")
    x32 = activations(wl, 0, tokens=50)
    z = zipf_logits(wl, steps=1, tokens=50)[0, 2]
    y = torch.empty((50, 256), dtype=torch.float32, device="cuda")
    tbl0 = moe.moe_get_slot_table(d.ctx, 2, 16)
    moe.moe_prefill(d.ctx, 2, 50, _dev(x32), _dev(z), y)
    y_ref, _, _ = oracle.moe_layer(16, 4, 256, 512, d.experts(2, oracle.route(z, 4)[0]), x32.astype(np.float64),
                                   logits=z)
    assert token_rel_err(y.cpu().numpy(), y_ref) < TOL
    assert np.array_equal(moe.moe_get_slot_table(d.ctx, 2, 16), tbl0)
    info = moe.moe_get_info(d.ctx)
    assert info["slots_per_layer"] == 20 and info["pool_bytes"] == 20 * d.B and info["staging_experts"] == 16
    d.close()


@pytest.mark.parametrize("pool", ["layer", "global"])
def test_preheat_matches_the_oracle_and_serves_decode(pool):
    from tests._gpu import oracle_policy

    wl = Workload("prefill-e32k4-h256f512-l2-preheat", 207, 2, 32, 4, 256, 512, tokens=2, steps=12, zipf_s=1.1)
    slots = 8 if pool == "layer" else 16
    d = Decode(wl, slots=slots, max_batch=2, max_prefill=60, pool=pool)
    pol = oracle_policy(wl, slots, pool=pool)
    logits = zipf_logits(wl)
    y = torch.empty((2, 256), dtype=torch.float32, device="cuda")

    def step(s, check):
        for layer in range(2):
            x32 = activations(wl, s, layer=layer)
            z = logits[s, layer]
            moe.moe_forward(d.ctx, layer, 2, _dev(x32), _dev(z), y)
            ids, _ = oracle.route(z, 4)
            pol.forward(layer, ids)
            if check:
                y_ref, _, _ = oracle.moe_layer(32, 4, 256, 512, d.experts(layer, ids), x32.astype(np.float64), logits=z)
                assert token_rel_err(y.cpu().numpy(), y_ref) < TOL
        assert moe.moe_cache_step(d.ctx)["admissions"] == pol.step()["admissions"]

    for s in range(4):
        step(s, check=False)
    # a 60-token prompt of layer 1, then preheat from its picks
    zp = zipf_logits(wl.with_(rotation=0), steps=1, tokens=60)[0, 1] * 0.5  # a flatter prompt: more cold experts
    xp = activations(wl, 0, tokens=60)
    yp = torch.empty((60, 256), dtype=torch.float32, device="cuda")
    moe.moe_prefill(d.ctx, 1, 60, _dev(xp), _dev(zp.astype(np.float32)), yp)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_preheat(d.ctx, 0, 5)
    assert ei.value.code == moe.MOE_E_STATE
    ids_p, _ = oracle.route(zp.astype(np.float32), 4)
    counts = np.bincount(ids_p.ravel(), minlength=32)
    ref = pol.preheat(1, counts, 5)
    n = moe.moe_preheat(d.ctx, 1, 5)
    assert n == len(ref) > 0
    tabs = pol.tables()
    for layer in range(2):
        assert np.array_equal(moe.moe_get_slot_table(d.ctx, layer, 32), tabs["table"][layer])
        g = 0 if pool == "global" else layer
        assert np.array_equal(moe.moe_get_stamps(d.ctx, layer, slots), tabs["stamps"][g])
    # decode goes on, reading the preheated experts from their new slots
    for s in range(4, 12):
        step(s, check=True)
        for layer in range(2):
            assert np.array_equal(moe.moe_get_slot_table(d.ctx, layer, 32), pol.tables()["table"][layer])
    d.close()


@pytest.mark.parametrize("scale", [1e3, 1e-4, "mixed"])
def test_prefill_activations_far_from_unit_scale(scale):
    # fp16 operands: each token's row is scaled by a power of two into [4, 8) before the cast and the
    # SwiGLU output by its square, so activations 1e3 or 1e-4 times N(0, 1) (h ~ 1e6 or 1e-9 unscaled, past
    # either end of fp16) keep the same relative error; "mixed" gives every token its own magnitude
    wl = Workload("prefill-e64k8-h2048f1024-t300-scaled", 211, 1, 64, 8, 2048, 1024, tokens=300, zipf_s=1.1)
    if scale == "mixed":
        scale = 10.0 ** np.random.default_rng(5).uniform(-5, 4, size=wl.tokens)
    err, prof = _prefill_check(wl, slots=26, sample=64, x_scale=scale)
    assert prof["prefill_staged"] > 0


def test_prefill_reports_values_beyond_the_fp16_operand_range():
    # block scales of 1000 (q - 8 times 1000 still fits fp16, but the SwiGLU output grows ~1e10 even after
    # the row scaling): the pass fails with MOE_E_RANGE instead of returning infinities
    wl = Workload("prefill-e8k2-h256f512-t16-range", 212, 1, 8, 2, 256, 512, tokens=16, zipf_s=1.1)
    from workload import layer_weights

    g, u, dn = (m.copy() for m in layer_weights(wl, 0))
    big = np.array([1000.0], "<f2").view(np.uint8)
    for m in (g, u, dn):  # experts 0..3 only
        m[:4, ..., 0], m[:4, ..., 1] = big[0], big[1]
    ctx = moe.moe_create(1, 8, 2, 256, 512, pool_budget_bytes=8 * wl.expert_bytes, max_batch_tokens=1,
                         max_prefill_tokens=16)
    try:
        moe.moe_register_layer(ctx, 0, g, u, dn)
        moe.moe_seed(ctx, None)
        x32 = activations(wl, 0, tokens=16)
        x = _dev(x32)
        z = zipf_logits(wl, steps=1, tokens=16)[0, 0]
        z[0, 0] = 50.0  # token 0 picks expert 0
        y = torch.empty_like(x)
        with pytest.raises(moe.MoeError) as ei:
            moe.moe_prefill(ctx, 0, 16, x, _dev(z), y)
        assert ei.value.code == moe.MOE_E_RANGE
        # a pass that routes to experts 4..7 only is valid again (the flag is cleared per pass)
        z[:, :4] = -50.0
        moe.moe_prefill(ctx, 0, 16, x, _dev(z), y)
        experts = {e: (g[e], u[e], dn[e]) for e in range(4, 8)}
        y_ref, _, _ = oracle.moe_layer(8, 2, 256, 512, experts, x32.astype(np.float64), logits=z)
        assert token_rel_err(y.cpu().numpy(), y_ref) < TOL
    finally:
        moe.moe_destroy(ctx)
