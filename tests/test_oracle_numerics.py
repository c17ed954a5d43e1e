"""Pins of the oracle's numerics to things other than itself (CPU only).

  * hand-worked Q4 blocks (tests/golden/q4_blocks.txt);
  * fp16 decoding of all 65536 bit patterns against numpy's float16;
  * a dense numpy brute force of the whole layer on tiny shapes;
  * special cases: one expert (a textbook SwiGLU MLP), all-q=8 blocks;
  * routing against a full stable sort, ties, weight sums;
  * the fp32 router logits against an exact rational fma chain.
"""
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests._brute import dense_moe, np_dequant, np_route
from workload import WORKLOADS, Workload, activations, layer_weights, router_weights, zipf_logits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "q4_blocks.txt")


def _golden_blocks():
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        name, hexs, vals = [p.strip() for p in line.split("|")]
        blk = np.frombuffer(bytes.fromhex(hexs), np.uint8)
        expect = {int(a): float(b) for a, b in (kv.split("=") for kv in vals.split())}
        yield name, blk, expect


@pytest.mark.parametrize("name,blk,expect", list(_golden_blocks()), ids=lambda v: v if isinstance(v, str) else "")
def test_dequant_hand_worked(name, blk, expect):
    assert blk.size == 18
    w = oracle.dequant_block(blk)
    for j, v in expect.items():
        assert w[j] == v, (name, j, w[j], v)


def test_half_decode_exhaustive():
    bits = np.arange(65536, dtype=np.uint32)
    ref = bits.astype(np.uint16).view(np.float16).astype(np.float64)
    got = np.array([oracle.half_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zeros keep their sign
    assert np.signbit(got[0x8000]) and not np.signbit(got[0])


def test_dequant_matrix_matches_numpy_unpacking():
    rng = np.random.default_rng(1)
    m = rng.integers(0, 256, size=(7, 3, 18), dtype=np.uint8)
    m[..., 1] &= 0x7B  # keep the scales finite
    assert np.array_equal(oracle.dequant_matrix(m), np_dequant(m))


def _tiny(E=4, k=2, H=64, F=96, T=3, seed=0):
    wl = Workload("pin", 900 + seed, 1, E, k, H, F, tokens=T, zipf_s=1.1)
    g, u, d = layer_weights(wl, 0, threads=1)
    x = activations(wl, 0).astype(np.float64)
    z = zipf_logits(wl, steps=1)[0, 0]
    return wl, g, u, d, x, z


@pytest.mark.parametrize("E,k,H,F,T", [(4, 2, 64, 96, 3), (8, 3, 32, 64, 5), (6, 6, 96, 32, 2), (5, 1, 64, 64, 4)])
def test_layer_vs_dense_brute_force(E, k, H, F, T):
    wl, g, u, d, x, z = _tiny(E, k, H, F, T, seed=E * 10 + k)
    experts = {e: (g[e], u[e], d[e]) for e in range(E)}
    y, ids, w = oracle.moe_layer(E, k, H, F, experts, x, logits=z)
    yb = dense_moe(g, u, d, x, z, k)
    ib, wb = np_route(z, k)
    assert np.array_equal(ids, ib)
    np.testing.assert_allclose(w, wb, rtol=1e-14, atol=0)
    scale = np.abs(yb).max(axis=1, keepdims=True)
    assert (np.abs(y - yb) / scale).max() < 1e-12


def test_single_expert_is_a_swiglu_mlp():
    wl, g, u, d, x, z = _tiny(E=1, k=1, H=64, F=96, T=2, seed=7)
    y, ids, w = oracle.moe_layer(1, 1, 64, 96, {0: (g[0], u[0], d[0])}, x, logits=z)
    assert ids.tolist() == [[0], [0]] and np.all(w == 1.0)
    Wg, Wu, Wd = np_dequant(g[0]), np_dequant(u[0]), np_dequant(d[0])
    for t in range(2):
        a = Wg @ x[t]
        ref = Wd @ (a * (1.0 / (1.0 + np.exp(-a))) * (Wu @ x[t]))
        assert np.abs(y[t] - ref).max() <= 1e-12 * np.abs(ref).max()


def test_all_q8_blocks_contribute_nothing():
    wl, g, u, d, x, z = _tiny(E=2, k=2, H=64, F=64, T=1, seed=3)
    d0 = d.copy()
    d0[1, :, :, 2:] = 0x88  # every q = 8 in expert 1's down matrix
    experts = {e: (g[e], u[e], d0[e]) for e in range(2)}
    y, ids, w = oracle.moe_layer(2, 2, 64, 64, experts, x, logits=z)
    y_only0, _, _ = oracle.moe_layer(2, 2, 64, 64, {0: (g[0], u[0], d[0]), 1: (g[1], u[1], d0[1])}, x, logits=z)
    pos0 = list(ids[0]).index(0)
    ye0 = oracle.expert_ffn(g[0], u[0], d[0], x[0])
    assert np.abs(y[0] - w[0, pos0] * ye0).max() <= 1e-15 * np.abs(ye0).max()
    assert np.array_equal(y, y_only0)


def test_matvec_against_numpy():
    rng = np.random.default_rng(5)
    m = rng.integers(0, 256, size=(33, 4, 18), dtype=np.uint8)
    m[..., 1] &= 0x3B
    x = rng.standard_normal(128)
    ref = np_dequant(m) @ x
    got = oracle.q4_matvec(m, x)
    assert np.abs(got - ref).max() <= 1e-12 * np.abs(ref).max()


def test_route_against_stable_sort_and_ties():
    rng = np.random.default_rng(11)
    for E, k in [(8, 2), (16, 5), (512, 8), (3, 3)]:
        z = rng.standard_normal((50, E)).astype(np.float32)
        z[:, ::3] = np.round(z[:, ::3])  # plenty of exact ties
        ids, w = oracle.route(z, k)
        ib, wb = np_route(z, k)
        assert np.array_equal(ids, ib)
        np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-12)
        np.testing.assert_allclose(w, wb, rtol=1e-13)
    ids, w = oracle.route(np.zeros((1, 6), np.float32), 4)
    assert ids.tolist() == [[0, 1, 2, 3]] and np.allclose(w, 0.25)
    # picks are listed by descending logit
    z = np.array([[0.5, 3.0, -1.0, 3.0, 2.0]], np.float32)
    ids, w = oracle.route(z, 3)
    assert ids.tolist() == [[1, 3, 4]]
    assert w[0, 0] == w[0, 1] > w[0, 2]


def _round_f32(q: Fraction) -> np.float32:
    """Nearest float32 to an exact rational, ties to even."""
    c = np.float32(float(q))
    cands = {c, np.nextafter(c, np.float32(np.inf)), np.nextafter(c, np.float32(-np.inf))}
    best = sorted(cands, key=lambda f: (abs(Fraction(float(f)) - q), int(np.frombuffer(f.tobytes(), np.uint32)[0]) & 1))
    return best[0]


def test_router_logits_are_the_fp32_fma_chain():
    wl = WORKLOADS["tiny-e8k2-h256f512-t4"]
    x = activations(wl, 0)[:2, :24]
    W = router_weights(wl, 0)[:, :24]
    z = oracle.router_logits(x, W)
    for t in range(2):
        for e in range(W.shape[0]):
            acc = np.float32(0)
            for j in range(24):
                acc = _round_f32(Fraction(float(x[t, j])) * Fraction(float(W[e, j])) + Fraction(float(acc)))
            assert z[t, e] == acc


def test_router_path_equals_given_logits():
    wl = WORKLOADS["tiny-e8k2-h256f512-t4"]
    g, u, d = layer_weights(wl, 0, threads=1)
    x32 = activations(wl, 0)
    W = router_weights(wl, 0)
    experts = {e: (g[e], u[e], d[e]) for e in range(8)}
    y1, i1, w1 = oracle.moe_layer(8, 2, 256, 512, experts, x32.astype(np.float64), w_router=W, x32=x32)
    z = oracle.router_logits(x32, W)
    y2, i2, w2 = oracle.moe_layer(8, 2, 256, 512, experts, x32.astype(np.float64), logits=z)
    assert np.array_equal(i1, i2) and np.array_equal(y1, y2) and np.array_equal(w1, w2)
    yb = dense_moe(g, u, d, x32.astype(np.float64), z, 2)
    assert (np.abs(y1 - yb).max(axis=1) / np.abs(yb).max(axis=1)).max() < 1e-12
