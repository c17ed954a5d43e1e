"""Seeded synthetic workloads for the routed-expert MoE layer.

Every array is drawn from numpy's PCG64 keyed by
SeedSequence(ROOT_SEED, spawn_key=(purpose, ...)), so any expert, layer,
step or token batch can be regenerated on its own, in any order, on any
machine.

What is drawn (the shapes and distributions of the pages' workloads; no
trained model or dataset is used):
  * expert weights in the canonical 4-bit block format: per 32-weight block an
    fp16 scale d drawn from U(0.001, 0.01) in fp64 and rounded to fp16 (round
    to nearest even), and 16 bytes of uniformly random nibbles (q uniform on
    0..15); the block is d (little endian) followed by the 16 bytes, element j
    in the low nibble of byte j and element j+16 in its high nibble;
  * router weights N(0, 0.02^2) fp32 (tiny workload) and activations N(0, 1)
    fp32, one independent draw per (step, layer);
  * router logits with Zipf(s) expert popularity: for layer l and epoch r a
    permutation maps popularity rank -> expert, and the logit of expert e is
    ln p(rank(e)) + Gumbel(0, 1), computed in fp64 and stored as fp32;
  * a routing-frequency table per layer: pick counts of a 1024-token warm-up
    drawn as a multinomial over the epoch-0 popularity.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT_SEED = 20261202

# purpose keys
_P_WEIGHT = 1
_P_ROUTER = 2
_P_X = 3
_P_PERM = 4
_P_GUMBEL = 5
_P_FREQ = 6

QBLOCK = 32
BLOCK_BYTES = 18


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(ROOT_SEED, spawn_key=tuple(int(k) for k in key))))


def expert_bytes(hidden: int, ffn: int) -> int:
    """Bytes of gate + up + down of one expert in the canonical format."""
    return 3 * hidden * ffn // QBLOCK * BLOCK_BYTES


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int                 # numeric id used in seed keys
    n_layers: int
    n_experts: int
    top_k: int
    hidden: int
    ffn: int
    tokens: int              # tokens per decode step, or per prefill pass
    steps: int = 1           # decode steps
    zipf_s: float = 0.0      # 0: logits come from the router instead
    zipf_s_alt: float = 0.0  # > 0: odd layers use this exponent instead (layers of unequal skew)
    slots: int = 0           # pool slots per layer
    rotation: int = 0        # re-draw the popularity permutation every this many tokens (0: never)
    epoch_base: int = 0      # popularity epoch of token clock 1 (the frequency table is always epoch 0)
    window: int = 64
    admit_misses: int = 2
    warmup_tokens: int = 1024
    distinct_layers: int = 0  # layers with their own weights; 0 = all
    prefill: bool = False
    meta: dict = field(default_factory=dict, compare=False, hash=False)

    @property
    def expert_bytes(self) -> int:
        return expert_bytes(self.hidden, self.ffn)

    @property
    def weight_layers(self) -> int:
        return self.distinct_layers or self.n_layers

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The workloads of the method's evaluation, named by what they are.
WORKLOADS = {
    w.name: w
    for w in [
        # single MoE layer, router in the loop, every expert resident
        Workload("tiny-e8k2-h256f512-t4", 1, 1, 8, 2, 256, 512, tokens=4, steps=1, slots=8),
        # batch-1 decode, 48 layers, half the experts in HBM; 32 distinct host
        # weight sets (58 GB pinned: the host allows about 66 GiB of pinned memory)
        Workload("decode-e512k8-h2048f1024-l48-b1", 2, 48, 512, 8, 2048, 1024, tokens=1, steps=256,
                 zipf_s=1.1, slots=256, distinct_layers=32),
        # one layer of the same shape, 4096-token prompt pass, half the experts resident
        Workload("prefill-e512k8-h2048f1024-t4096", 3, 1, 512, 8, 2048, 1024, tokens=4096, zipf_s=1.1,
                 slots=256, prefill=True),
        # 2048 decode steps, popularity permutation re-drawn every 512 tokens, 40% pool
        Workload("policy-e512k8-h2048f1024-l48-rot512", 4, 48, 512, 8, 2048, 1024, tokens=1, steps=2048,
                 zipf_s=1.1, slots=204, rotation=512, distinct_layers=32),
        # 60 layers of 256 experts (hidden 4096, ffn 1536): 163 GB of experts, 251 slots per layer;
        # 20 distinct host weight sets (54 GB pinned)
        Workload("large-e256k8-h4096f1536-l60-b1", 5, 60, 256, 8, 4096, 1536, tokens=1, steps=256,
                 zipf_s=1.0, slots=251, distinct_layers=20),
        Workload("large-e256k8-h4096f1536-l60-b32", 6, 60, 256, 8, 4096, 1536, tokens=32, steps=256,
                 zipf_s=1.0, slots=251, distinct_layers=20),
        Workload("large-e256k8-h4096f1536-t12288", 7, 1, 256, 8, 4096, 1536, tokens=12288, zipf_s=1.0,
                 slots=251, prefill=True),
        # the decode shape with layers of unequal skew (even layers Zipf 1.4, odd 0.7) and a quarter of
        # the experts in HBM: where one pool shared by all layers can move slots between layers
        Workload("decode-e512k8-h2048f1024-l48-b1-mixedzipf", 8, 48, 512, 8, 2048, 1024, tokens=1, steps=256,
                 zipf_s=1.4, zipf_s_alt=0.7, slots=128, distinct_layers=32),
    ]
}


# ---------------------------------------------------------------------------
# weights


def q4_matrix(rng: np.random.Generator, rows: int, k: int, out: np.ndarray | None = None) -> np.ndarray:
    """rows x k weights as canonical blocks: uint8 [rows][k/32][18] (written into out if given)."""
    assert k % QBLOCK == 0
    nb = rows * (k // QBLOCK)
    d = rng.uniform(0.001, 0.01, size=nb).astype("<f2")
    qs = rng.bit_generator.random_raw(nb * 2).view(np.uint8).reshape(nb, 16)
    blk = np.empty((nb, BLOCK_BYTES), dtype=np.uint8) if out is None else out.reshape(nb, BLOCK_BYTES)
    blk[:, :2] = d.view(np.uint8).reshape(nb, 2)
    blk[:, 2:] = qs
    return blk.reshape(rows, k // QBLOCK, BLOCK_BYTES)


def _expert_key(wl: Workload, layer: int, expert: int):
    return (_P_WEIGHT, wl.hidden, wl.ffn, wl.n_experts, layer % wl.weight_layers, expert)


def expert_weights(wl: Workload, layer: int, expert: int, out=None):
    """(gate [F][H/32][18], up [F][H/32][18], down [H][F/32][18]) of one expert.

    Keyed by the layer shape, so workloads of the same shape share weights.
    """
    base = _expert_key(wl, layer, expert)
    o = (None, None, None) if out is None else out
    gate = q4_matrix(_rng(*base, 0), wl.ffn, wl.hidden, o[0])
    up = q4_matrix(_rng(*base, 1), wl.ffn, wl.hidden, o[1])
    down = q4_matrix(_rng(*base, 2), wl.hidden, wl.ffn, o[2])
    return gate, up, down


def layer_weights(wl: Workload, layer: int, out=None, experts=None, threads: int = 0):
    """All experts of a layer: (gate [E][F][H/32][18], up [...], down [E][H][F/32][18]).

    With experts given, only those rows of the output are filled.
    """
    E, H, F = wl.n_experts, wl.hidden, wl.ffn
    if out is None:
        gate = np.empty((E, F, H // QBLOCK, BLOCK_BYTES), np.uint8)
        up = np.empty_like(gate)
        down = np.empty((E, H, F // QBLOCK, BLOCK_BYTES), np.uint8)
    else:
        gate, up, down = out
    todo = [int(e) for e in (range(E) if experts is None else experts)]

    def one(e):
        expert_weights(wl, layer, e, out=(gate[e], up[e], down[e]))

    nthreads = min(len(todo), threads or _default_threads())
    if nthreads <= 1:
        for e in todo:
            one(e)
    else:  # numpy drops the GIL while filling, so threads scale
        with ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(one, todo))
    return gate, up, down


def _default_threads() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def router_weights(wl: Workload, layer: int) -> np.ndarray:
    """fp32 [E][H] ~ N(0, 0.02^2)."""
    return _rng(_P_ROUTER, wl.wid, layer).normal(0.0, 0.02, size=(wl.n_experts, wl.hidden)).astype(np.float32)


def activations(wl: Workload, step: int = 0, tokens: int | None = None, layer: int = 0) -> np.ndarray:
    """fp32 [T][H] ~ N(0, 1): the input of one layer in one decode step (or of a prefill pass).

    Every (step, layer) has its own input, like the router logits, which are
    drawn independently of the activations too.
    """
    T = wl.tokens if tokens is None else tokens
    return _rng(_P_X, wl.wid, step, layer).standard_normal((T, wl.hidden)).astype(np.float32)


def step_activations(wl: Workload, step: int, layers=None) -> np.ndarray:
    """fp32 [L][T][H]: the inputs of every layer of one decode step."""
    layers = range(wl.n_layers) if layers is None else layers
    return np.stack([activations(wl, step, layer=layer) for layer in layers])


# ---------------------------------------------------------------------------
# routing inputs


def zipf_popularity(n: int, s: float) -> np.ndarray:
    """p(rank) proportional to (rank+1)^-s, ranks 0..n-1 (fp64, sums to 1)."""
    p = np.arange(1, n + 1, dtype=np.float64) ** (-float(s))
    return p / p.sum()


def rank_permutation(wl: Workload, layer: int, epoch: int) -> np.ndarray:
    """int64 [E]: perm[rank] = expert holding that popularity rank."""
    return _rng(_P_PERM, wl.wid, layer, epoch).permutation(wl.n_experts)


def _epoch_log_popularity(wl: Workload, layer: int, epoch: int) -> np.ndarray:
    """fp64 [E]: ln p(rank(e)) for each expert e in the given epoch."""
    perm = rank_permutation(wl, layer, epoch)
    s = wl.zipf_s_alt if (wl.zipf_s_alt > 0 and layer % 2 == 1) else wl.zipf_s
    logp = np.log(zipf_popularity(wl.n_experts, s))
    out = np.empty(wl.n_experts, np.float64)
    out[perm] = logp
    return out


def zipf_logits(wl: Workload, layers=None, steps=None, tokens: int | None = None) -> np.ndarray:
    """fp32 [steps][len(layers)][T][E] router logits with Zipf(s) popularity.

    Token i of step s has clock t = 1 + s*T + i; with a rotation period R the
    popularity permutation of epoch epoch_base + (t-1)//R applies.
    """
    assert wl.zipf_s > 0, "workload draws its logits from a router"
    layers = range(wl.n_layers) if layers is None else list(layers)
    T = wl.tokens if tokens is None else tokens
    n_steps = wl.steps if steps is None else steps
    E = wl.n_experts
    out = np.empty((n_steps, len(layers), T, E), np.float32)
    t = 1 + np.arange(n_steps)[:, None] * T + np.arange(T)[None, :]
    epochs = wl.epoch_base + ((t - 1) // wl.rotation if wl.rotation else np.zeros_like(t))
    for li, layer in enumerate(layers):
        g = _rng(_P_GUMBEL, wl.wid, layer).gumbel(0.0, 1.0, size=(n_steps, T, E))
        for ep in np.unique(epochs):
            mask = epochs == ep
            g[mask] += _epoch_log_popularity(wl, layer, int(ep))[None, :]
        out[:, li] = g.astype(np.float32)
    return out


def frequency_table(wl: Workload) -> np.ndarray:
    """uint32 [L][E]: warm-up pick counts per expert (multinomial over epoch-0 popularity)."""
    L, E = wl.n_layers, wl.n_experts
    out = np.zeros((L, E), np.uint32)
    for layer in range(L):
        if wl.zipf_s > 0:
            p = np.exp(_epoch_log_popularity(wl, layer, 0))
        else:
            p = np.full(E, 1.0 / E)
        out[layer] = _rng(_P_FREQ, wl.wid, layer).multinomial(wl.warmup_tokens * wl.top_k, p / p.sum())
    return out
