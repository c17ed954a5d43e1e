"""CPU oracle of the routed-expert MoE layer and its expert cache.

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg import this package. The GPU library neither imports nor
links it, and it shares no code with the GPU library.

The arithmetic lives in moe_oracle.c (fp64, plain loops, see its header for
what each function computes and where the pages define it); this module only
loads it with ctypes and marshals numpy arrays.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle_moe.so")

_u8p = np.ctypeslib.ndpointer(np.uint8, flags="C_CONTIGUOUS")
_f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS")
_u32p = np.ctypeslib.ndpointer(np.uint32, flags="C_CONTIGUOUS")
_u64p = np.ctypeslib.ndpointer(np.uint64, flags="C_CONTIGUOUS")
_i64p = np.ctypeslib.ndpointer(np.int64, flags="C_CONTIGUOUS")


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (fp64, no FMA contraction, OpenMP over rows)."""
    if force or not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(_SRC):
        tmp = LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
             "-fvisibility=hidden", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = C.CDLL(LIB_PATH)
        L.orc_half_to_double.argtypes = [C.c_uint16]
        L.orc_half_to_double.restype = C.c_double
        L.orc_dequant_block.argtypes = [_u8p, _f64p]
        L.orc_dequant_matrix.argtypes = [_u8p, C.c_int64, C.c_int64, _f64p]
        L.orc_q4_matvec.argtypes = [_u8p, C.c_int64, C.c_int64, _f64p, _f64p]
        L.orc_router_logits.argtypes = [_f32p, _f32p, C.c_int32, C.c_int32, C.c_int32, _f32p]
        L.orc_route.argtypes = [_f32p, C.c_int32, C.c_int32, _i32p, _f64p]
        L.orc_expert_ffn.argtypes = [_u8p, _u8p, _u8p, C.c_int32, C.c_int32, _f64p, _f64p]
        L.orc_moe_layer.argtypes = [C.c_int32] * 5 + [C.c_void_p] * 3 + [C.c_void_p, C.c_void_p, C.c_void_p,
                                                                          _f64p, _f64p, _i32p, _f64p]
        L.orc_moe_layer.restype = C.c_int
        L.orc_policy_new.argtypes = [C.c_int32] * 6 + [C.c_int64, C.c_int32]
        L.orc_policy_new.restype = C.c_void_p
        L.orc_policy_free.argtypes = [C.c_void_p]
        L.orc_policy_set_swaps.argtypes = [C.c_void_p, C.c_int32, C.c_int32]
        L.orc_policy_preheat.argtypes = [C.c_void_p, C.c_int32, C.c_void_p, C.c_int32, C.c_void_p]
        L.orc_policy_preheat.restype = C.c_int32
        L.orc_policy_seed.argtypes = [C.c_void_p, C.c_void_p]
        L.orc_policy_forward.argtypes = [C.c_void_p, C.c_int32, C.c_int32, _i32p]
        L.orc_policy_forward.restype = C.c_int
        L.orc_policy_step.argtypes = [C.c_void_p, _i64p]
        L.orc_policy_tables.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p]
        L.orc_policy_last_log.argtypes = [C.c_void_p, C.c_void_p, C.c_int64]
        L.orc_policy_last_log.restype = C.c_int64
        L.orc_policy_last_admissions.argtypes = [C.c_void_p, C.c_void_p, C.c_int64]
        L.orc_policy_last_admissions.restype = C.c_int64
        L.orc_policy_counts.argtypes = [C.c_void_p, _u32p]
        L.orc_policy_clock.argtypes = [C.c_void_p]
        L.orc_policy_clock.restype = C.c_uint32
        _lib = L
    return _lib


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


# --- numerics ---------------------------------------------------------------

def half_to_double(h: int) -> float:
    return lib().orc_half_to_double(int(h) & 0xFFFF)


def dequant_block(blk) -> np.ndarray:
    out = np.empty(32, np.float64)
    lib().orc_dequant_block(_c(blk, np.uint8).reshape(-1), out)
    return out


def dequant_matrix(m: np.ndarray) -> np.ndarray:
    """uint8 [rows][k/32][18] -> fp64 [rows][k]."""
    rows, nb = m.shape[0], m.shape[1]
    out = np.empty((rows, nb * 32), np.float64)
    lib().orc_dequant_matrix(_c(m, np.uint8).reshape(-1), rows, nb * 32, out)
    return out


def q4_matvec(m: np.ndarray, x) -> np.ndarray:
    rows, nb = m.shape[0], m.shape[1]
    y = np.empty(rows, np.float64)
    lib().orc_q4_matvec(_c(m, np.uint8).reshape(-1), rows, nb * 32, _c(x, np.float64), y)
    return y


def router_logits(x32: np.ndarray, w_router: np.ndarray) -> np.ndarray:
    x32 = _c(x32, np.float32)
    T, H = x32.shape
    E = w_router.shape[0]
    z = np.empty((T, E), np.float32)
    lib().orc_router_logits(x32, _c(w_router, np.float32), T, E, H, z)
    return z


def route(z: np.ndarray, k: int):
    """z fp32 [T][E] (or [E]) -> ids int32 [T][k], w fp64 [T][k]."""
    z = _c(z, np.float32)
    z2 = z.reshape(-1, z.shape[-1])
    T, E = z2.shape
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    for t in range(T):
        it, wt = ids[t], w[t]
        lib().orc_route(np.ascontiguousarray(z2[t]), E, k, it, wt)
    return ids.reshape(z.shape[:-1] + (k,)), w.reshape(z.shape[:-1] + (k,))


def expert_ffn(gate, up, down, x) -> np.ndarray:
    F, nbh = gate.shape[0], gate.shape[1]
    H = nbh * 32
    y = np.empty(H, np.float64)
    lib().orc_expert_ffn(_c(gate, np.uint8).reshape(-1), _c(up, np.uint8).reshape(-1),
                         _c(down, np.uint8).reshape(-1), H, F, _c(x, np.float64), y)
    return y


def moe_layer(E: int, k: int, H: int, F: int, experts, x, logits=None, w_router=None, x32=None):
    """One MoE layer for T tokens.

    experts: mapping expert id -> (gate, up, down) canonical uint8 arrays
    (only the picked experts are needed). x fp64 [T][H]; logits fp32 [T][E]
    or None with w_router fp32 [E][H] and x32 fp32 [T][H] (router in fp32).
    Returns (y fp64 [T][H], ids int32 [T][k], w fp64 [T][k]).
    """
    x = _c(x, np.float64)
    T = x.shape[0]
    keep = []
    ptrs = [(C.c_void_p * E)() for _ in range(3)]
    for e, mats in experts.items():
        for m in range(3):
            a = _c(mats[m], np.uint8)
            keep.append(a)
            ptrs[m][int(e)] = a.ctypes.data
    y = np.empty((T, H), np.float64)
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    lg = None if logits is None else _c(logits, np.float32)
    wr = None if w_router is None else _c(w_router, np.float32)
    xs = None if x32 is None else _c(x32, np.float32)
    rc = lib().orc_moe_layer(T, E, k, H, F, C.cast(ptrs[0], C.c_void_p), C.cast(ptrs[1], C.c_void_p),
                             C.cast(ptrs[2], C.c_void_p),
                             None if lg is None else lg.ctypes.data, None if wr is None else wr.ctypes.data,
                             None if xs is None else xs.ctypes.data, x, y, ids, w)
    if rc != 0:
        raise KeyError("a picked expert's weights were not supplied")
    return y, ids, w


# --- cache policy -------------------------------------------------------------

class Policy:
    """Step-by-step simulation of the expert cache (see moe_oracle.c)."""

    def __init__(self, n_layers, n_experts, slots, top_k, window=64, admit_misses=2, log_capacity=1 << 20,
                 pool="layer", swaps_per_step=0, swap_lead=0):
        """slots: per layer (pool="layer") or in the one pool all layers share (pool="global").
        swaps_per_step: admissions allowed per step (0: any); swap_lead: steps an admission waits
        before its table entry flips (0: at once)."""
        assert pool in ("layer", "global")
        self.L, self.E, self.S, self.k = n_layers, n_experts, slots, top_k
        self.pool = pool
        self.groups = 1 if pool == "global" else n_layers
        self._p = lib().orc_policy_new(n_layers, n_experts, slots, top_k, window, admit_misses, log_capacity,
                                       1 if pool == "global" else 0)
        lib().orc_policy_set_swaps(self._p, swaps_per_step, swap_lead)

    def __del__(self):
        if getattr(self, "_p", None):
            lib().orc_policy_free(self._p)
            self._p = None

    def seed(self, freq=None):
        f = None if freq is None else _c(freq, np.uint32)
        lib().orc_policy_seed(self._p, None if f is None else f.ctypes.data)

    def forward(self, layer: int, ids) -> None:
        ids = _c(ids, np.int32).reshape(-1, self.k)
        if lib().orc_policy_forward(self._p, layer, ids.shape[0], ids) != 0:
            raise OverflowError("miss log capacity exceeded")

    def step(self) -> dict:
        s = np.zeros(5, np.int64)
        lib().orc_policy_step(self._p, s)
        return dict(hits=int(s[0]), misses=int(s[1]), admissions=int(s[2]), evictions=int(s[3]),
                    tokens=int(s[4]))

    def preheat(self, layer: int, counts, max_experts: int) -> np.ndarray:
        """Admit the cold experts a prompt pass of `layer` used (counts [E]: its pairs per expert);
        returns the admission records int32 [n][5] as last_admissions."""
        c = _c(counts, np.uint32)
        out = np.empty((max(min(max_experts, self.S), 1), 5), np.int32)
        n = lib().orc_policy_preheat(self._p, layer, c.ctypes.data, max_experts, out.ctypes.data)
        return out[:n]

    def tables(self):
        """table [L][E] (slot in the layer's pool, -1 cold); per pool [groups][S]: owner (expert or -1),
        owner_layer (layer or -1), stamps; last_miss [L][E]. groups = L per layer, 1 global."""
        tbl = np.empty((self.L, self.E), np.int32)
        own = np.empty((self.groups, max(self.S, 1)), np.int32)
        st = np.empty((self.groups, max(self.S, 1)), np.uint32)
        lm = np.empty((self.L, self.E), np.uint32)
        lib().orc_policy_tables(self._p, tbl.ctypes.data, own.ctypes.data, st.ctypes.data, lm.ctypes.data)
        own = own[:, :self.S]
        return dict(table=tbl, owner=np.where(own < 0, -1, own % self.E), owner_layer=np.where(own < 0, -1, own // self.E),
                    stamps=st[:, :self.S], last_miss=lm)

    def last_log(self) -> np.ndarray:
        n = lib().orc_policy_last_log(self._p, None, 0)
        out = np.empty(max(n, 1), np.uint64)
        lib().orc_policy_last_log(self._p, out.ctypes.data, n)
        return out[:n]

    def last_admissions(self) -> np.ndarray:
        """int32 [n][5]: (layer, expert, slot, evicted layer, evicted expert; -1 when the slot was free),
        in walk order."""
        n = lib().orc_policy_last_admissions(self._p, None, 0)
        out = np.empty((max(n, 1), 5), np.int32)
        lib().orc_policy_last_admissions(self._p, out.ctypes.data, n)
        return out[:n]

    def counts(self) -> np.ndarray:
        out = np.empty((self.L, self.E), np.uint32)
        lib().orc_policy_counts(self._p, out)
        return out

    @property
    def clock(self) -> int:
        return int(lib().orc_policy_clock(self._p))
