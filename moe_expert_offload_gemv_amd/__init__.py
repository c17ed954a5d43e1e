"""Python binding of libmoe_offload.so (include/moe_offload.h).

Argument marshalling only: every step of the MoE layer runs in the HIP
kernels and the host runtime of the shared library. Device buffers are torch
cuda tensors (passed by data_ptr()); host buffers are numpy arrays. The
functions keep the C names and raise MoeError on a negative return code.
If the library has not been built this module raises on first use; there is
no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "libmoe_offload.so")

MOE_OK = 0
MOE_E_INVAL = -1
MOE_E_NOMEM = -2
MOE_E_HIP = -3
MOE_E_STATE = -4
MOE_E_CAPTURING = -5
MOE_E_RANGE = -6
MOE_Q4_32_F16 = 1
MOE_ACCUMULATE = 1
MOE_MAX_SWAP_LEAD = 8
MOE_STATIC_SCRATCH_BYTES = 16777216
MOE_COLD_GPU = 0
MOE_COLD_CPU = 1
MOE_HOST_COHERENT = 0
MOE_HOST_NONCOHERENT = 1
MOE_POOL_PER_LAYER = 0
MOE_POOL_GLOBAL = 1

EXPORTED = [
    "moe_expert_bytes", "moe_create", "moe_destroy", "moe_register_layer", "moe_register_router", "moe_seed",
    "moe_forward", "moe_prefill", "moe_cache_step", "moe_get_info", "moe_get_slot_table", "moe_get_stamps",
    "moe_get_miss_log", "moe_get_counts", "moe_last_error", "moe_profile", "moe_preheat", "moe_measure_read_bandwidth",
    "moe_forward_static_scratch",
]


class moe_config(C.Structure):
    _fields_ = [
        ("n_layers", C.c_int32), ("n_experts", C.c_int32), ("top_k", C.c_int32), ("hidden", C.c_int32),
        ("ffn", C.c_int32), ("quant", C.c_int32), ("pool_budget_bytes", C.c_int64), ("reserve_bytes", C.c_int64),
        ("window_tokens", C.c_int32), ("admit_misses", C.c_int32), ("max_batch_tokens", C.c_int32),
        ("max_prefill_tokens", C.c_int32), ("device", C.c_int32), ("host_alloc", C.c_int32),
        ("host_sets", C.c_int32), ("stream", C.c_void_p), ("capture_picks", C.c_int32), ("pool_mode", C.c_int32),
        ("swaps_per_step", C.c_int32), ("swap_lead", C.c_int32), ("cold_exec", C.c_int32),
        ("cpu_threads", C.c_int32), ("decode_launches", C.c_int32), ("decode_sync_polls", C.c_int32),
    ]


class moe_info(C.Structure):
    _fields_ = [(n, C.c_int64) for n in ("slots_per_layer", "expert_bytes", "pool_bytes", "host_bytes",
                                        "staging_experts", "clock", "steps", "host_threads", "host_isa",
                                        "pool_budget_bytes", "free_bytes_at_sizing")]


class moe_step_stats(C.Structure):
    _fields_ = [(n, C.c_int64) for n in ("step", "tokens", "hits", "misses", "admissions", "evictions",
                                        "hot_bytes", "cold_bytes", "copied_bytes", "copied_pcie_bytes",
                                        "distinct_experts", "distinct_cold_experts")]

    def as_dict(self):
        return {n: int(getattr(self, n)) for n, _ in self._fields_}


class moe_profile_stats(C.Structure):
    _fields_ = [("forwards", C.c_int64), ("route_ms", C.c_double), ("hot_gateup_ms", C.c_double),
                ("hot_down_ms", C.c_double), ("cold_gateup_ms", C.c_double), ("cold_down_ms", C.c_double),
                ("hot_picks", C.c_int64), ("cold_picks", C.c_int64), ("gateup_bytes_per_pick", C.c_int64),
                ("down_bytes_per_pick", C.c_int64), ("prefill_passes", C.c_int64),
                ("prefill_gateup_ms", C.c_double), ("prefill_down_ms", C.c_double), ("prefill_pairs", C.c_int64),
                ("prefill_tiles", C.c_int64), ("prefill_staged", C.c_int64), ("prefill_prep_ms", C.c_double),
                ("prefill_stage_ms", C.c_double), ("host_forwards", C.c_int64),
                ("host_expert_passes", C.c_int64), ("host_picks", C.c_int64), ("host_wait_ms", C.c_double),
                ("host_compute_ms", C.c_double), ("layer_forwards", C.c_int64), ("hot_layer_ms", C.c_double),
                ("cold_layer_ms", C.c_double)]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


class MoeError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


_lib = None


def lib():
    """The loaded shared library (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with python -m moe_expert_offload_gemv_amd.build")
        L = C.CDLL(LIB_PATH)
        vp, i32, i64, u32 = C.c_void_p, C.c_int32, C.c_int64, C.c_uint32
        sig = {
            "moe_expert_bytes": (i64, [i32, i32]),
            "moe_create": (C.c_int, [C.POINTER(moe_config), C.POINTER(vp)]),
            "moe_destroy": (C.c_int, [vp]),
            "moe_register_layer": (C.c_int, [vp, i32, vp, vp, vp]),
            "moe_register_router": (C.c_int, [vp, i32, vp]),
            "moe_seed": (C.c_int, [vp, vp]),
            "moe_forward": (C.c_int, [vp, i32, i32, vp, vp, vp, vp, vp, u32]),
            "moe_forward_static_scratch": (C.c_int, [vp, i32, i32, vp, vp, vp, vp, vp, u32]),
            "moe_prefill": (C.c_int, [vp, i32, i32, vp, vp, vp, u32]),
            "moe_cache_step": (C.c_int, [vp, C.POINTER(moe_step_stats)]),
            "moe_get_info": (C.c_int, [vp, C.POINTER(moe_info)]),
            "moe_get_slot_table": (C.c_int, [vp, i32, vp]),
            "moe_get_stamps": (C.c_int, [vp, i32, vp]),
            "moe_get_miss_log": (C.c_int, [vp, vp, i64, C.POINTER(i64)]),
            "moe_get_counts": (C.c_int, [vp, vp]),
            "moe_last_error": (C.c_char_p, [vp]),
            "moe_profile": (C.c_int, [vp, i32, C.POINTER(moe_profile_stats)]),
            "moe_preheat": (C.c_int, [vp, i32, i32, C.POINTER(i32)]),
            "moe_measure_read_bandwidth": (C.c_int, [vp, i64, i32, i32, vp, C.POINTER(C.c_double)]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


def _check(ctx, rc: int) -> None:
    if rc != MOE_OK:
        msg = lib().moe_last_error(ctx) if ctx else b""
        raise MoeError(rc, (msg or b"").decode(errors="replace"))


def _dptr(t):
    """Device address of a torch cuda tensor (None -> NULL)."""
    if t is None:
        return None
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("device arguments must be contiguous cuda tensors")
    return t.data_ptr()


def _hptr(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data


# ---------------------------------------------------------------------------

def moe_expert_bytes(hidden: int, ffn: int) -> int:
    return int(lib().moe_expert_bytes(hidden, ffn))


def moe_create(n_layers, n_experts, top_k, hidden, ffn, pool_budget_bytes, reserve_bytes=0, window_tokens=64,
               admit_misses=2, max_batch_tokens=64, max_prefill_tokens=0, device=0, host_alloc=MOE_HOST_COHERENT,
               host_sets=0, stream=None, capture_picks=None, pool_mode=0, swaps_per_step=0, swap_lead=0,
               cold_exec=MOE_COLD_GPU, cpu_threads=0, decode_launches=0, decode_sync_polls=0):
    """Returns an opaque context handle.

    stream: a torch.cuda.Stream, a raw hipStream_t int, or None for torch's
    current stream on the device (0, the null stream, is a valid handle).
    capture_picks: None for top_k (one token's picks per layer; 0 with cold_exec=MOE_COLD_CPU), 0 for off.
    cold_exec: MOE_COLD_GPU (zero-copy reads of cold experts) or MOE_COLD_CPU (host threads compute them).
    pool_mode: MOE_POOL_PER_LAYER (slots per layer) or MOE_POOL_GLOBAL (one pool for all layers).
    swaps_per_step: admissions per cache step (0: no limit); swap_lead: cache steps an admission waits
    for its copy before its table entry flips (0: at once).
    decode_launches: 1 for one launch per layer where the decode shape allows it, 0 or 2 for two (the default).
    decode_sync_polls: bound of the one-launch down work-groups' wait (0: the default, 2^20 polls).
    """
    if capture_picks is None:
        capture_picks = 0 if cold_exec == MOE_COLD_CPU else top_k
    if stream is None:
        stream = 0
        try:
            import torch

            if torch.cuda.is_available():
                stream = torch.cuda.current_stream(device).cuda_stream
        except ImportError:
            pass
    elif not isinstance(stream, int):
        stream = stream.cuda_stream
    cfg = moe_config(n_layers, n_experts, top_k, hidden, ffn, MOE_Q4_32_F16, pool_budget_bytes, reserve_bytes,
                     window_tokens, admit_misses, max_batch_tokens, max_prefill_tokens, device, host_alloc,
                     host_sets, stream, capture_picks, pool_mode, swaps_per_step, swap_lead, cold_exec, cpu_threads,
                     decode_launches, decode_sync_polls)
    out = C.c_void_p()
    rc = lib().moe_create(C.byref(cfg), C.byref(out))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_create: " + (lib().moe_last_error(None) or b"").decode(errors="replace"))
    return out.value


def moe_destroy(ctx) -> None:
    _check(None, lib().moe_destroy(ctx))


def moe_register_layer(ctx, layer: int, gate, up, down) -> None:
    g, gp = _hptr(gate, np.uint8)
    u, up_ = _hptr(up, np.uint8)
    d, dp = _hptr(down, np.uint8)
    _check(ctx, lib().moe_register_layer(ctx, layer, gp, up_, dp))


def moe_register_router(ctx, layer: int, w_router) -> None:
    w, wp = _hptr(w_router, np.float32)
    _check(ctx, lib().moe_register_router(ctx, layer, wp))


def moe_seed(ctx, freq=None) -> None:
    if freq is None:
        _check(ctx, lib().moe_seed(ctx, None))
    else:
        f, fp = _hptr(freq, np.uint32)
        _check(ctx, lib().moe_seed(ctx, fp))


def moe_forward(ctx, layer: int, n_tokens: int, x, logits, y, ids=None, w=None, flags: int = 0) -> None:
    _check(ctx, lib().moe_forward(ctx, layer, n_tokens, _dptr(x), _dptr(logits), _dptr(y), _dptr(ids), _dptr(w),
                                  flags))


def moe_forward_static_scratch(ctx, layer: int, n_tokens: int, x, logits, y, ids=None, w=None,
                               flags: int = 0) -> None:
    _check(ctx, lib().moe_forward_static_scratch(ctx, layer, n_tokens, _dptr(x), _dptr(logits), _dptr(y),
                                                 _dptr(ids), _dptr(w), flags))


def moe_prefill(ctx, layer: int, n_tokens: int, x, logits, y, flags: int = 0) -> None:
    _check(ctx, lib().moe_prefill(ctx, layer, n_tokens, _dptr(x), _dptr(logits), _dptr(y), flags))


def moe_preheat(ctx, layer: int, max_experts: int) -> int:
    """Admit the cold experts the last prompt pass (of `layer`) used; returns how many were admitted."""
    n = C.c_int32(0)
    _check(ctx, lib().moe_preheat(ctx, layer, max_experts, C.byref(n)))
    return int(n.value)


def moe_cache_step(ctx) -> dict:
    s = moe_step_stats()
    _check(ctx, lib().moe_cache_step(ctx, C.byref(s)))
    return s.as_dict()


def moe_get_info(ctx) -> dict:
    s = moe_info()
    _check(ctx, lib().moe_get_info(ctx, C.byref(s)))
    return {n: int(getattr(s, n)) for n, _ in s._fields_}


def moe_get_slot_table(ctx, layer: int, n_experts: int) -> np.ndarray:
    out = np.empty(n_experts, np.int32)
    _check(ctx, lib().moe_get_slot_table(ctx, layer, out.ctypes.data))
    return out


def moe_get_stamps(ctx, layer: int, slots: int) -> np.ndarray:
    out = np.zeros(max(slots, 1), np.uint32)
    _check(ctx, lib().moe_get_stamps(ctx, layer, out.ctypes.data))
    return out[:slots]


def moe_get_miss_log(ctx) -> np.ndarray:
    n = C.c_int64()
    _check(ctx, lib().moe_get_miss_log(ctx, None, 0, C.byref(n)))
    out = np.empty(max(n.value, 1), np.uint64)
    _check(ctx, lib().moe_get_miss_log(ctx, out.ctypes.data, n.value, C.byref(n)))
    return out[: n.value]


def moe_get_counts(ctx, n_layers: int, n_experts: int) -> np.ndarray:
    out = np.empty((n_layers, n_experts), np.uint32)
    _check(ctx, lib().moe_get_counts(ctx, out.ctypes.data))
    return out


def moe_profile(ctx, enable: int = -1) -> dict:
    s = moe_profile_stats()
    _check(ctx, lib().moe_profile(ctx, enable, C.byref(s)))
    return s.as_dict()


def moe_measure_read_bandwidth(buf=None, nbytes: int = 0, reps: int = 3, host_coherent: bool = True,
                               stream=None) -> float:
    """GB/s of a plain 128-bit streaming read kernel: over the cuda tensor buf
    (HBM), or with buf None over nbytes of pinned host memory the library
    allocates (zero-copy over PCIe). A measurement aid, not the MoE path."""
    import torch

    if buf is not None:
        nbytes = buf.numel() * buf.element_size()
    s = stream if stream is not None else torch.cuda.current_stream()
    out = C.c_double(0.0)
    rc = lib().moe_measure_read_bandwidth(_dptr(buf), int(nbytes), int(reps), 1 if host_coherent else 0,
                                          s.cuda_stream, C.byref(out))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_measure_read_bandwidth failed")
    return out.value


def moe_last_error(ctx) -> str:
    return (lib().moe_last_error(ctx) or b"").decode(errors="replace")
