"""The C-ABI library loads and exports every function include/moe_offload.h
declares (CPU only: no compute call needs a GPU here)."""
import ctypes
import os
import re

import pytest

import moe_expert_offload_gemv_amd as moe
from workload import expert_bytes

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_offload.h")


def _declared():
    txt = open(HEADER).read()
    return re.findall(r"^MOE_API\s+[\w\s\*]+?\b(moe_\w+)\s*\(", txt, flags=re.M)


def test_header_declares_the_boundary():
    names = _declared()
    assert set(names) == set(moe.EXPORTED)
    for need in ("moe_create", "moe_register_layer", "moe_seed", "moe_forward", "moe_cache_step", "moe_prefill"):
        assert need in names


def test_library_exports_every_declared_symbol():
    if not os.path.exists(moe.LIB_PATH):
        pytest.fail(f"{moe.LIB_PATH} not built (run __graft_entry__.build())")
    lib = ctypes.CDLL(moe.LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name


def test_expert_bytes_host_helper():
    for H, F in [(256, 512), (2048, 1024), (4096, 1536)]:
        assert moe.moe_expert_bytes(H, F) == expert_bytes(H, F)
    assert moe.moe_expert_bytes(100, 512) == -1


def test_create_rejects_bad_config_without_touching_a_gpu():
    # argument validation happens before any device call
    bad = dict(n_layers=1, n_experts=8, top_k=9, hidden=256, ffn=512, pool_budget_bytes=0)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_create(**bad)
    assert ei.value.code == moe.MOE_E_INVAL
    with pytest.raises(moe.MoeError):
        moe.moe_create(n_layers=1, n_experts=8, top_k=2, hidden=100, ffn=512, pool_budget_bytes=0)
    with pytest.raises(moe.MoeError):
        moe.moe_create(n_layers=1, n_experts=5000, top_k=2, hidden=256, ffn=512, pool_budget_bytes=0)
    with pytest.raises(moe.MoeError):  # more than 2^26 prompt pairs per pass
        moe.moe_create(n_layers=1, n_experts=8, top_k=2, hidden=256, ffn=512, pool_budget_bytes=0,
                       max_prefill_tokens=(1 << 25) + 1)


def test_binding_constants_match_the_header():
    txt = open(HEADER).read()
    defines = dict(re.findall(r"^#define\s+(MOE_\w+)\s+(-?\d+)", txt, flags=re.M))
    assert defines, "no constants found"
    for name, value in defines.items():
        assert getattr(moe, name) == int(value), name


def _struct_fields(name):
    txt = open(HEADER).read()
    body = re.search(r"typedef struct \{([^{}]*)\}\s*" + name + r";", txt).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    return re.findall(r"\b(\w+)\s*;", body)


@pytest.mark.parametrize("name", ["moe_config", "moe_info", "moe_step_stats", "moe_profile_stats"])
def test_binding_structs_mirror_the_header(name):
    assert [f for f, _ in getattr(moe, name)._fields_] == _struct_fields(name)


def test_create_rejects_bad_pool_mode_and_capture():
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_create(n_layers=1, n_experts=8, top_k=2, hidden=256, ffn=512, pool_budget_bytes=0, pool_mode=7)
    assert ei.value.code == moe.MOE_E_INVAL
    with pytest.raises(moe.MoeError):
        moe.moe_create(n_layers=1, n_experts=8, top_k=2, hidden=256, ffn=512, pool_budget_bytes=0,
                       max_batch_tokens=1, capture_picks=3)
