"""GPU parity of the activations other than SiLU(gate)*up (GELU, its tanh
form, and the _no_mul SiLU / GELU / GELU-tanh / ReLU^2 whose w13 has N rows)
against the oracle, through the C ABI: the activation kernel in isolation on
the oracle's gate_up, the fused w13 epilogue against the unfused pair (bit
for bit), and the whole layer in every layout, including the indexed one."""
import dataclasses
import os

import numpy as np
import pytest
import torch

import fp8_block_quantized_group_amd as moe
import moe_synth
from oracle import moe_oracle as O
from parity_util import (abs_gemm_cfg, check_bf16_act_chain, check_bf16_close, check_output,
                         check_requant, check_requant_chain, to_dev, to_np)
from test_gpu_parity import SENTINEL_BF16, SENTINEL_U8, gpu  # noqa: F401

pytestmark = pytest.mark.gpu


def _cfg(name, act, **kw):
    base = dict(T=300, E=5, top_k=3, K=384, N=384, seed=51, pad_frac=0.07)
    base.update(kw)
    return moe_synth.custom(name=name, activation=act, **base)


CASES = {f"{a}": _cfg(a, a) for a in ("gelu", "gelu_tanh", "silu_no_mul", "gelu_no_mul",
                                       "gelu_tanh_no_mul", "relu2_no_mul")}
CASES.update({
    "gelu_tanh_fp32": _cfg("gelu_tanh_fp32", "gelu_tanh", act_quant="fp32", seed=52),
    "relu2_bf16": _cfg("relu2_bf16", "relu2_no_mul", act_quant="bf16", seed=53),
    "gelu_bf16": _cfg("gelu_bf16", "gelu", act_quant="bf16", seed=54),
    "gelu_mx": _cfg("gelu_mx", "gelu", act_quant="mxfp8", weight_quant="mxfp8", seed=55),
    "silu_no_mul_mx4": _cfg("silu_no_mul_mx4", "silu_no_mul", act_quant="mxfp8",
                            weight_quant="mxfp4", seed=56),
    "gelu_no_mul_batched": _cfg("gelu_no_mul_batched", "gelu_no_mul", T=250, E=4, top_k=2,
                                N=256, seed=57, pad_frac=0.0, layout="batched",
                                max_tokens=160),
    # the clamped SwiGLU forms, with limits inside the gate_up range (about
    # N(0, 0.4) here) so that every clamp is active on a good share of the
    # values; the last two with their default limit 7 (no clamp reached)
    "silu_clamp": _cfg("silu_clamp", "silu", act_limit=0.3, seed=58),
    "swigluoai": _cfg("swigluoai", "swigluoai", act_limit=0.4, seed=59),
    "swiglustep": _cfg("swiglustep", "swiglustep", act_limit=0.1, seed=60),
    "swigluoai_mx4": _cfg("swigluoai_mx4", "swigluoai", act_limit=0.4, act_quant="mxfp8",
                          weight_quant="mxfp4", seed=61),
    "swiglustep_bf16": _cfg("swiglustep_bf16", "swiglustep", act_limit=0.1, act_quant="bf16",
                            seed=62),
    "silu_clamp_fp32_batched": _cfg("silu_clamp_fp32_batched", "silu", act_limit=0.3, T=250,
                                    E=4, top_k=2, N=256, seed=63, pad_frac=0.0,
                                    layout="batched", max_tokens=160, act_quant="fp32"),
    "swigluoai_default": _cfg("swigluoai_default", "swigluoai", seed=64),
    "swiglustep_default": _cfg("swiglustep_default", "swiglustep", seed=65),
})

_CACHE = {}


def case(name):
    if name not in _CACHE:
        cfg = CASES[name]
        inp = moe_synth.make_inputs(cfg, "cpu")
        h = O.host_inputs(inp)
        _CACHE[name] = (cfg, h, inp, O.forward(h))
    cfg, h, inp, ref = _CACHE[name]
    dev = {k: (v.to("cuda") if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    return cfg, h, dev, ref


def valid_rows(cfg, ref):
    if cfg.layout == "batched":
        return np.concatenate([np.arange(e * cfg.max_tokens, e * cfg.max_tokens + int(c))
                               for e, c in enumerate(ref["counts"])]).astype(np.int64)
    return np.arange(int(ref["offsets"][-1]))


def w13_abs(cfg, h, ref):
    """The oracle's w13 GEMM on absolute values (the MFMA error scale)."""
    vr = valid_rows(cfg, ref)
    out = np.zeros((len(ref["gate_up"]), cfg.w13_rows))
    rows_of = {}
    if cfg.layout == "batched":
        for e, c in enumerate(ref["counts"]):
            rows_of[e] = np.arange(e * cfg.max_tokens, e * cfg.max_tokens + int(c))
    else:
        for e in range(cfg.E):
            rows_of[e] = np.arange(int(ref["offsets"][e]), int(ref["offsets"][e + 1]))
    for e, rows in rows_of.items():
        if len(rows) == 0:
            continue
        a_rows = rows if cfg.layout == "batched" else ref["row_src"][rows]
        x_sf = None if ref["x_sf"] is None else ref["x_sf"][a_rows]
        out[rows] = abs_gemm_cfg(cfg, ref["x_q"][a_rows], x_sf, h["w13"][e], h["w13_sf"][e])
    return out[vr]


def stage(cfg, dev):
    p = moe.Problem.from_config(cfg)
    bufs = moe.alloc_stage_outputs(p)
    moe.stage(p, dev["hidden"], dev["topk_ids"], dev["topk_weights"], bufs, dev["is_padding"],
              dev["expert_num_tokens"], dev["eplb"])
    return p, bufs


def a2_buffers(cfg, p):
    s = moe.sizes(p)
    rows = s["padded_rows"]
    if cfg.act_quant == "bf16":
        return (torch.full((rows, cfg.N), SENTINEL_BF16, dtype=torch.int16,
                           device="cuda").view(torch.bfloat16), None)
    return (torch.full((rows, cfg.N), SENTINEL_U8, dtype=torch.uint8, device="cuda"),
            torch.zeros((rows, s["a2_sf_row"]), dtype=moe.scale_dtype(p), device="cuda"))


@pytest.mark.parametrize("name", list(CASES))
def test_activation_isolated(gpu, name):
    """moe_act_requant on the oracle's own gate_up (routing from the GPU's
    stage, which the stage tests prove bit-exact)."""
    cfg, h, dev, ref = case(name)
    p, bufs = stage(cfg, dev)
    s = moe.sizes(p)
    vr = valid_rows(cfg, ref)
    gu = np.full((s["expert_rows"], cfg.w13_rows), 0x7FC0, np.uint16)   # NaN outside
    gu[vr] = ref["gate_up"][vr]
    a2_q, a2_sf = a2_buffers(cfg, p)
    moe.act_requant(p, to_dev(gu), bufs, a2_q, a2_sf)
    torch.cuda.synchronize()
    untouched = np.setdiff1d(np.arange(s["expert_rows"]), vr)
    if cfg.act_quant == "bf16":
        got = to_np(a2_q)
        check_bf16_close(got[vr], ref["a2_q"][vr], f"{name} activation (bf16)")
        assert np.all(got[untouched] == SENTINEL_BF16)
        return
    got_q, got_sf = to_np(a2_q), to_np(a2_sf)
    h32 = O.act_f32(ref["gate_up"][vr], cfg.N, cfg.activation, cfg.act_limit)
    check_requant(got_q[vr], got_sf[vr], ref["a2_q"][vr], ref["a2_sf"][vr], h32,
                  O.act_e8m0(cfg), f"{name} activation", O.act_group(cfg))
    assert np.all(got_q[untouched] == SENTINEL_U8)


@pytest.mark.parametrize("name", list(CASES))
def test_layer_chain_and_forward(gpu, name):
    """stage -> w13 -> activation -> w2 -> reduce through the separate calls,
    checked step by step against the oracle; moe_forward gives the same
    bits."""
    cfg, h, dev, ref = case(name)
    p, bufs = stage(cfg, dev)
    s = moe.sizes(p)
    vr = valid_rows(cfg, ref)
    gate_up = torch.full((s["expert_rows"], cfg.w13_rows), SENTINEL_BF16, dtype=torch.int16,
                         device="cuda").view(torch.bfloat16)
    moe.grouped_gemm_w13(p, bufs["x_q"], bufs["x_sf"], bufs, dev["w13"], dev["w13_sf"], gate_up)
    a2_q, a2_sf = a2_buffers(cfg, p)
    moe.act_requant(p, gate_up, bufs, a2_q, a2_sf)
    down = torch.empty((s["expert_rows"], cfg.K), dtype=torch.bfloat16, device="cuda")
    moe.grouped_gemm_w2(p, a2_q, a2_sf, bufs, dev["w2"], dev["w2_sf"], down)
    out = torch.empty((cfg.T, cfg.K), dtype=torch.bfloat16, device="cuda")
    moe.topk_reduce(p, down, bufs["slot_row"], bufs["topk_w"], out)
    torch.cuda.synchronize()
    s_abs = w13_abs(cfg, h, ref)
    if cfg.act_quant == "bf16":
        check_bf16_act_chain(to_np(a2_q)[vr], ref["a2_q"][vr], ref["gate_up"][vr], s_abs,
                             f"{name} a2 (chain)", cfg.activation, cfg.act_limit)
    else:
        check_requant_chain(to_np(a2_q)[vr], to_np(a2_sf)[vr], ref["a2_q"][vr],
                            ref["a2_sf"][vr], ref["gate_up"][vr], s_abs, O.act_e8m0(cfg),
                            f"{name} a2 (chain)", O.act_group(cfg), cfg.activation,
                            limit=cfg.act_limit)
    check_output(to_np(out), ref["out"], f"{name} chained output")
    layer = moe.MoeLayer(p, dev["w13"], dev["w13_sf"], dev["w2"], dev["w2_sf"])
    fwd = layer(dev["hidden"], dev["topk_ids"], dev["topk_weights"], None, dev["is_padding"],
                dev["expert_num_tokens"], dev["eplb"])
    torch.cuda.synchronize()
    assert torch.equal(fwd.view(torch.int16), out.view(torch.int16)), name


@pytest.mark.parametrize("tile_m", [16, 64, 128, 256])
@pytest.mark.parametrize("name", [n for n, c in CASES.items() if c.gated])
def test_fused_epilogue_equals_chain(gpu, name, tile_m, monkeypatch):
    monkeypatch.setenv("MOE_TILE_M", str(tile_m))
    cfg, h, dev, ref = case(name)
    if cfg.act_quant == "bf16" and tile_m > 128:
        pytest.skip("bf16 activation tiles are at most 128 rows (LDS)")
    p, bufs = stage(cfg, dev)
    s = moe.sizes(p)
    vr = valid_rows(cfg, ref)
    gate_up = torch.empty((s["expert_rows"], cfg.w13_rows), dtype=torch.bfloat16, device="cuda")
    moe.grouped_gemm_w13(p, bufs["x_q"], bufs["x_sf"], bufs, dev["w13"], dev["w13_sf"], gate_up)
    want_q, want_sf = a2_buffers(cfg, p)
    moe.act_requant(p, gate_up, bufs, want_q, want_sf)
    got_q, got_sf = a2_buffers(cfg, p)
    moe.grouped_gemm_w13_act(p, bufs["x_q"], bufs["x_sf"], bufs, dev["w13"], dev["w13_sf"],
                             got_q, got_sf)
    torch.cuda.synchronize()
    g, w = to_np(got_q), to_np(want_q)
    assert np.array_equal(g[vr], w[vr]), (name, tile_m)
    if got_sf is not None:
        assert np.array_equal(to_np(got_sf)[vr].view(np.uint8), to_np(want_sf)[vr].view(np.uint8))
    untouched = np.setdiff1d(np.arange(s["expert_rows"]), vr)
    assert np.all(g[untouched] == (SENTINEL_BF16 if cfg.act_quant == "bf16" else SENTINEL_U8))


def test_fused_call_rejects_no_mul(gpu):
    cfg, h, dev, ref = case("relu2_no_mul")
    p, bufs = stage(cfg, dev)
    a2_q, a2_sf = a2_buffers(cfg, p)
    with pytest.raises(moe.MoeError) as ei:
        moe.grouped_gemm_w13_act(p, bufs["x_q"], bufs["x_sf"], bufs, dev["w13"], dev["w13_sf"],
                                 a2_q, a2_sf)
    assert ei.value.status == -2


@pytest.mark.parametrize("name", ["gelu", "silu_no_mul", "relu2_bf16", "gelu_mx"])
def test_indexed_layout_other_activations(gpu, name):
    """moe_forward in the indexed layout equals the contiguous one bit for bit
    (the _no_mul ones run the indexed w13 GEMM into a sorted-order gate_up
    and the activation kernel over the padded rows)."""
    cfg, h, dev, ref = case(name)
    p = moe.Problem.from_config(cfg)
    layer = moe.MoeLayer(p, dev["w13"], dev["w13_sf"], dev["w2"], dev["w2_sf"])
    base = layer(dev["hidden"], dev["topk_ids"], dev["topk_weights"], None, dev["is_padding"])
    for bs in (16, 64):
        os.environ["MOE_TILE_M"] = str(bs)
        try:
            pi = moe.Problem.from_config(dataclasses.replace(cfg, layout="indexed"))
            li = moe.MoeLayer(pi, dev["w13"], dev["w13_sf"], dev["w2"], dev["w2_sf"])
            out = li(dev["hidden"], dev["topk_ids"], dev["topk_weights"], None,
                     dev["is_padding"])
            torch.cuda.synchronize()
        finally:
            del os.environ["MOE_TILE_M"]
        assert torch.equal(out.view(torch.int16), base.view(torch.int16)), (name, bs)
    check_output(to_np(base), ref["out"], f"{name} output")
