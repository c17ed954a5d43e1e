"""Helpers shared by the GPU tests: build a context for a workload, run
decode steps through the C ABI, and compare against the oracle."""
from __future__ import annotations

import numpy as np

import moe_expert_offload_gemv_amd as moe
import oracle
from workload import Workload, frequency_table, layer_weights

TOL = 2e-3  # per token: max |y - y_ref| / max |y_ref|


def token_rel_err(y, y_ref) -> float:
    y = np.asarray(y, np.float64).reshape(-1, y_ref.shape[-1])
    y_ref = np.asarray(y_ref, np.float64).reshape(-1, y_ref.shape[-1])
    num = np.abs(y - y_ref).max(axis=1)
    den = np.abs(y_ref).max(axis=1)
    return float((num / den).max())


class Decode:
    """A context with every layer of a workload registered.

    seed=True seeds from the workload's frequency table, False starts cold
    (moe_seed with no table), None leaves the context unseeded. pool="global"
    makes one pool of `slots` slots shared by every layer.
    """

    def __init__(self, wl: Workload, slots: int | None = None, seed=True, max_batch: int | None = None,
                 host_alloc: int = moe.MOE_HOST_COHERENT, stream=None, max_prefill: int = 0, keep_weights=True,
                 capture_picks=None, pool="layer", swaps_per_step=0, swap_lead=0, cold_exec=moe.MOE_COLD_GPU,
                 cpu_threads=0, decode_launches=0, decode_sync_polls=0):
        import torch

        self.wl = wl
        self.S = wl.slots if slots is None else slots
        self.B = wl.expert_bytes
        self.stream = stream if stream is not None else torch.cuda.current_stream()
        self.pool = pool
        budget = (1 if pool == "global" else wl.n_layers) * self.S * self.B
        self.ctx = moe.moe_create(wl.n_layers, wl.n_experts, wl.top_k, wl.hidden, wl.ffn,
                                  pool_budget_bytes=budget, window_tokens=wl.window,
                                  admit_misses=wl.admit_misses, max_batch_tokens=max_batch or max(wl.tokens, 1),
                                  max_prefill_tokens=max_prefill, host_alloc=host_alloc,
                                  host_sets=wl.distinct_layers, stream=self.stream, capture_picks=capture_picks,
                                  pool_mode=moe.MOE_POOL_GLOBAL if pool == "global" else moe.MOE_POOL_PER_LAYER,
                                  swaps_per_step=swaps_per_step, swap_lead=swap_lead, cold_exec=cold_exec,
                                  cpu_threads=cpu_threads, decode_launches=decode_launches,
                                  decode_sync_polls=decode_sync_polls)
        info = moe.moe_get_info(self.ctx)
        assert info["slots_per_layer"] == self.S, info
        self.weights = {}
        buf = None
        for layer in range(wl.weight_layers):  # layer l reads host set l % weight_layers
            buf = layer_weights(wl, layer, out=None if keep_weights else buf)
            moe.moe_register_layer(self.ctx, layer, *buf)
            if keep_weights:
                self.weights[layer] = buf
        self.freq = frequency_table(wl)
        if seed is True:
            moe.moe_seed(self.ctx, self.freq)
        elif seed is False:  # cold start: every slot free
            moe.moe_seed(self.ctx, None)

    def experts(self, layer, ids):
        g, u, d = self.weights[layer % self.wl.weight_layers]
        return {int(e): (g[e], u[e], d[e]) for e in np.unique(ids)}

    def close(self):
        if self.ctx:
            moe.moe_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def oracle_policy(wl: Workload, slots: int, seed: bool = True, pool: str = "layer", swaps_per_step=0, swap_lead=0):
    pol = oracle.Policy(wl.n_layers, wl.n_experts, slots, wl.top_k, window=wl.window, admit_misses=wl.admit_misses,
                        pool=pool, swaps_per_step=swaps_per_step, swap_lead=swap_lead)
    pol.seed(frequency_table(wl) if seed else None)
    return pol


class GraphDecode:
    """The decode step as bench.py runs it: one HIP graph of the L-layer
    forward, every layer adding its output into one residual buffer
    (MOE_ACCUMULATE), replayed per step, then the cache step. With
    snapshots the graph also copies the residual after every layer, so each
    layer's output is the difference of two snapshots. With cold_exec CPU
    (not capturable) the same launches run eagerly each step, as bench.py
    runs that mode."""

    def __init__(self, wl: Workload, snapshots: bool = True, max_batch: int | None = None,
                 cold_exec=moe.MOE_COLD_GPU, swaps=(0, 0)):
        import torch

        self.torch = torch
        self.wl = wl
        self.stream = torch.cuda.Stream()
        self.d = Decode(wl, stream=self.stream, max_batch=max_batch or wl.tokens, keep_weights=False,
                        cold_exec=cold_exec, swaps_per_step=swaps[0], swap_lead=swaps[1])
        L, T, H, E = wl.n_layers, wl.tokens, wl.hidden, wl.n_experts
        self.xs = torch.zeros((L, T, H), dtype=torch.float32, device="cuda")
        self.zs = torch.zeros((L, T, E), dtype=torch.float32, device="cuda")
        self.res = torch.zeros((T, H), dtype=torch.float32, device="cuda")
        self.snap = torch.zeros((L, T, H), dtype=torch.float32, device="cuda") if snapshots else None

        def forward_all():
            for layer in range(L):
                moe.moe_forward(self.d.ctx, layer, T, self.xs[layer], self.zs[layer], self.res,
                                flags=moe.MOE_ACCUMULATE)
                if snapshots:
                    self.snap[layer].copy_(self.res)

        self.forward_all = forward_all
        self.graph = None
        if cold_exec == moe.MOE_COLD_GPU:
            self.graph = torch.cuda.CUDAGraph()
            with torch.cuda.stream(self.stream):
                with torch.cuda.graph(self.graph, stream=self.stream):
                    forward_all()

    def step(self, xs_step, logits_step):
        torch = self.torch
        with torch.cuda.stream(self.stream):
            self.xs.copy_(torch.from_numpy(np.ascontiguousarray(xs_step)).cuda())
            self.zs.copy_(torch.from_numpy(np.ascontiguousarray(logits_step)).cuda())
            self.res.zero_()
            if self.graph is not None:
                self.graph.replay()
            else:
                self.forward_all()
            st = moe.moe_cache_step(self.d.ctx)
        return st

    def layer_outputs(self):
        """fp64 [L][T][H]: each layer's output of the last replay."""
        s = self.snap.cpu().numpy().astype(np.float64)
        prev = np.concatenate([np.zeros_like(s[:1]), s[:-1]], axis=0)
        return s - prev

    def close(self):
        self.d.close()


def picked_weights(wl: Workload, layer: int, ids) -> dict:
    """expert id -> (gate, up, down) for the experts in ids, regenerated on a thread pool."""
    from concurrent.futures import ThreadPoolExecutor

    from workload import expert_weights

    todo = [int(e) for e in np.unique(ids)]
    with ThreadPoolExecutor(max(1, min(16, len(todo)))) as ex:
        mats = list(ex.map(lambda e: expert_weights(wl, layer, e), todo))
    return dict(zip(todo, mats))


def oracle_layers(wl: Workload, xs_step, logits_step, layers=None):
    """fp64 outputs [len(layers)][T][H] of the layers of one step through the
    oracle (every layer when layers is None), regenerating the picked experts' weights."""
    out = []
    for layer in range(wl.n_layers) if layers is None else layers:
        z = logits_step[layer]
        ids, _ = oracle.route(z, wl.top_k)
        y, _, _ = oracle.moe_layer(wl.n_experts, wl.top_k, wl.hidden, wl.ffn, picked_weights(wl, layer, ids),
                                   np.asarray(xs_step[layer], np.float64), logits=z)
        out.append(y)
    return np.stack(out)


def tile_edge_tokens(ids: np.ndarray, tile_rows=(64, 128)) -> np.ndarray:
    """Tokens of the first and last pair of every (expert, tile) of a prompt pass, for each tile height:
    the pairs (token t, pick i) numbered t * k + i, stably sorted by expert, cut per expert into tiles."""
    k = ids.shape[1]
    flat = ids.reshape(-1)
    order = np.argsort(flat, kind="stable")
    counts = np.bincount(flat, minlength=int(flat.max()) + 1)
    starts = np.concatenate([[0], np.cumsum(counts)[:-1]])
    pos = []
    for bm in tile_rows:
        for e in np.nonzero(counts)[0]:
            for m0 in range(0, int(counts[e]), bm):
                first = starts[e] + m0
                pos += [first, first + min(bm, int(counts[e]) - m0) - 1]
    return np.unique(order[np.asarray(pos, np.int64)] // k)
