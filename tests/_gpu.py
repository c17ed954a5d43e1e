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
    (moe_seed with no table), None leaves the context unseeded.
    """

    def __init__(self, wl: Workload, slots: int | None = None, seed=True, max_batch: int | None = None,
                 host_alloc: int = moe.MOE_HOST_COHERENT, stream=None, max_prefill: int = 0, keep_weights=True):
        import torch

        self.wl = wl
        self.S = wl.slots if slots is None else slots
        self.B = wl.expert_bytes
        self.stream = stream if stream is not None else torch.cuda.current_stream()
        self.ctx = moe.moe_create(wl.n_layers, wl.n_experts, wl.top_k, wl.hidden, wl.ffn,
                                  pool_budget_bytes=wl.n_layers * self.S * self.B, window_tokens=wl.window,
                                  admit_misses=wl.admit_misses, max_batch_tokens=max_batch or max(wl.tokens, 1),
                                  max_prefill_tokens=max_prefill, host_alloc=host_alloc,
                                  host_sets=wl.distinct_layers, stream=self.stream)
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


def oracle_policy(wl: Workload, slots: int, seed: bool = True):
    pol = oracle.Policy(wl.n_layers, wl.n_experts, slots, wl.top_k, window=wl.window, admit_misses=wl.admit_misses)
    pol.seed(frequency_table(wl) if seed else None)
    return pol
