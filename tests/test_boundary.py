"""The C-ABI boundary without a GPU: the library loads, exports every symbol
include/moe_fp8.h declares, plans buffer sizes, and rejects bad arguments
synchronously (validation runs before anything touches the device, so these
calls are safe on a host without a GPU)."""
import ctypes
import os
import re

import pytest

import fp8_block_quantized_group_amd as moe
import moe_synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_fp8.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(moe.LIB_PATH):
        from fp8_block_quantized_group_amd import build
        build.build()
    return moe.load_library()


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\*\s]+?\b(moe_\w+)\s*\(", text, re.M)))


def test_header_declares_the_boundary():
    names = _declared()
    for n in ("moe_stage", "moe_grouped_gemm_w13", "moe_act_requant", "moe_grouped_gemm_w2",
              "moe_topk_reduce", "moe_forward", "moe_workspace_size", "moe_last_error"):
        assert n in names
    assert set(names) == set(moe.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for n in _declared():
        assert hasattr(lib, n), n


def _status(fn, *args):
    return fn(*args)


def test_sizes_follow_the_problem(lib):
    for name, cfg in moe_synth.CONFIGS.items():
        p = moe.Problem.from_config(cfg)
        s = moe.sizes(p)
        assert s["slots"] == cfg.T * cfg.top_k
        if cfg.layout == "batched":
            assert s["stage_rows"] == cfg.E * cfg.max_tokens == s["expert_rows"]
        else:
            assert s["stage_rows"] == cfg.T and s["expert_rows"] == cfg.T * cfg.top_k
        G = cfg.K // 128
        assert s["x_sf_row"] == (4 * ((G + 3) // 4) if cfg.act_quant == "ue8m0" else G)
        assert s["tile_m"] in (16, 32, 64, 128, 192, 256)
        ws = moe.workspace_size(p)
        gate_up = s["expert_rows"] * 2 * cfg.N * 2
        assert ws >= gate_up + s["expert_rows"] * cfg.N


@pytest.mark.parametrize("field,value,status", [
    ("hidden", 100, -1), ("hidden", 0, -1), ("intermediate", 200, -1),
    ("num_experts", 0, -2), ("num_experts", 2000, -2), ("top_k", 0, -1),
    ("layout", 7, -1), ("num_tokens", -1, -1), ("act_quant", 5, -1),
])
def test_invalid_problem_rejected(lib, field, value, status):
    kw = dict(num_tokens=16, hidden=256, intermediate=512, num_experts=4, top_k=2)
    kw[field] = value
    p = moe.Problem(**kw)
    with pytest.raises(moe.MoeError) as ei:
        moe.sizes(p)
    assert ei.value.status == status
    assert lib.moe_last_error().decode()


def test_batched_needs_max_tokens(lib):
    p = moe.Problem(16, 256, 512, 4, 2, layout=moe.LAYOUT_BATCHED, max_tokens_per_expert=0)
    with pytest.raises(moe.MoeError):
        moe.sizes(p)


def _fake(addr=1 << 20):
    return ctypes.c_void_p(addr)


def test_call_validation_before_launch(lib):
    p = moe.Problem(16, 256, 512, 4, 2).c()
    V = _fake()
    # null hidden states
    st = lib.moe_forward(ctypes.byref(p), None, None, V, V, None, None, V, V, V, V, V, V,
                         1 << 30, None)
    assert st == -1 and "hidden" in lib.moe_last_error().decode()
    # misaligned output
    st = lib.moe_forward(ctypes.byref(p), V, None, V, V, None, None, V, V, V, V,
                         _fake((1 << 20) + 2), V, 1 << 30, None)
    assert st == -1 and "aligned" in lib.moe_last_error().decode()
    # workspace too small
    st = lib.moe_forward(ctypes.byref(p), V, None, V, V, None, None, V, V, V, V, V, V, 16, None)
    assert st == -3
    # bf16 activations are a staging-only scheme
    pb = moe.Problem(16, 256, 512, 4, 2, act_quant=moe.Q_BF16).c()
    st = lib.moe_forward(ctypes.byref(pb), V, None, V, V, None, None, V, V, V, V, V, V,
                         1 << 30, None)
    assert st == -2
    # batched layout without expert_num_tokens
    pbt = moe.Problem(16, 256, 512, 4, 2, layout=moe.LAYOUT_BATCHED,
                      max_tokens_per_expert=8).c()
    st = lib.moe_forward(ctypes.byref(pbt), V, None, V, V, None, None, V, V, V, V, V, V,
                         1 << 30, None)
    assert st == -1 and "expert_num_tokens" in lib.moe_last_error().decode()
    # x_sf given for bf16 staging
    r = moe._Routing(V, V, V, V, V)
    st = lib.moe_stage(ctypes.byref(pb), V, None, V, V, None, None, V, V, V, V,
                       ctypes.byref(r), V, 1 << 20, None)
    assert st == -1 and "x_sf" in lib.moe_last_error().decode()


def test_empty_batch_is_a_noop(lib):
    p = moe.Problem(0, 256, 512, 4, 2).c()
    assert lib.moe_forward(ctypes.byref(p), None, None, None, None, None, None, None, None,
                           None, None, None, None, 0, None) == 0
    assert lib.moe_stage(ctypes.byref(p), None, None, None, None, None, None, None, None, None,
                         None, None, None, 0, None) == 0
    assert lib.moe_last_error().decode() == ""
