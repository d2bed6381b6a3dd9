"""Parity at the workloads' full sizes (the five block-fp8 ones, the MX and
bf16-activation variants and the indexed-layout DeepSeek-V3 prefill), in
the launch configuration the benchmark times (moe_forward, same tile
height).

The oracle cannot run these layers whole, so it checks what it can compute
piece by piece: the complete routing layout and EPLB load (cheap), the
quantized hidden rows of a sample of tokens, and for a few sampled tokens
every row of the chain (gate_up, a2, down) and the token's output row.
Intermediates come from the separate entry points, whose final output must
equal moe_forward's bit for bit.
"""
import numpy as np
import pytest
import torch

import fp8_block_quantized_group_amd as moe
import moe_synth
from oracle import moe_oracle as O
from parity_util import (abs_gemm_cfg, check_bf16_act_chain, check_gemm, check_output,
                         check_requant_chain, to_np)
from test_gpu_parity import check_schedule, run_chain, run_forward

pytestmark = pytest.mark.gpu

FULL = ["tiny", "mixtral", "dsv3_prefill", "dsv3_decode", "qwen3", "dsv3_prefill_mxfp8",
        "dsv3_prefill_mxfp4", "qwen3_bf16", "dsv3_prefill_indexed"]


def _host_light(inp):
    """Host copies of everything except the weights (those stay on the GPU;
    the oracle copies single experts when it needs them)."""
    h = {}
    for k, v in inp.items():
        if k in ("w13", "w13_sf", "w2", "w2_sf"):
            h[k] = v
        elif k == "eplb" and v is not None:
            h[k] = {k2: O._np(v2) for k2, v2 in v.items()}
        elif k == "cfg":
            h[k] = v
        else:
            h[k] = O._np(v)
    return h


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled(name):
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    cfg = moe_synth.ALL_CONFIGS[name]
    print(f"\n[fullsize] {name}: generating inputs", flush=True)
    inp = moe_synth.make_inputs(cfg, "cuda")
    torch.cuda.synchronize()
    print(f"[fullsize] {name}: running the layer", flush=True)
    chain = run_chain(cfg, inp)
    out = run_forward(cfg, inp)
    assert torch.equal(out.view(torch.int16), chain["out"].view(torch.int16))
    h = _host_light(inp)
    st = O.stage_routing_only(h)
    bufs = chain["bufs"]
    # routing layout, complete and bit-exact
    assert np.array_equal(to_np(bufs["topk_idx"]), st["ids"])
    assert np.array_equal(to_np(bufs["topk_w"]).view(np.uint32), st["weights"].view(np.uint32))
    assert np.array_equal(to_np(bufs["expert_num_tokens"]), st["counts"])
    assert np.array_equal(to_np(bufs["slot_row"]).reshape(cfg.T, cfg.top_k), st["slot_row"])
    T_valid = cfg.T - (int(h["is_padding"].sum()) if h["is_padding"] is not None else 0)
    assert int(st["counts"].sum()) == T_valid * cfg.top_k
    if cfg.layout != "batched":
        assert np.array_equal(to_np(bufs["expert_offsets"]), st["offsets"])
        M = int(st["offsets"][-1])
        assert np.array_equal(to_np(bufs["row_src"])[:M], st["row_src"])
    if cfg.eplb:
        assert np.array_equal(to_np(inp["eplb"]["expert_load"]), st["load"])
    counts = st["counts"] if cfg.layout != "batched" else np.minimum(st["counts"], cfg.max_tokens)
    bases = ([e * cfg.max_tokens for e in range(cfg.E)] if cfg.layout == "batched"
             else st["offsets"][:-1])
    check_schedule(bufs["tile_list"], counts, moe.sizes(moe.Problem.from_config(cfg)), cfg.E,
                   bases)
    # quantized hidden rows of a token sample, bit-exact
    rng = np.random.default_rng(cfg.seed + 100)
    ue, grp = O.act_e8m0(cfg), O.act_group(cfg)
    hid = h["hidden"].reshape(-1, cfg.K)
    if cfg.layout == "batched":
        live = np.concatenate([np.arange(e * cfg.max_tokens, e * cfg.max_tokens + int(c))
                               for e, c in enumerate(st["counts"])])
    else:
        live = np.arange(cfg.T)
    rows = np.sort(rng.choice(live, min(256, live.size), replace=False))
    xq = to_np(bufs["x_q"][torch.from_numpy(rows).cuda()])
    if cfg.act_quant == "bf16":
        assert np.array_equal(xq, hid[rows]) and bufs["x_sf"] is None   # staging copy
    else:
        q_ref, s_ref = O.quantize_groups(O.bf16_to_f64(hid[rows]).astype(np.float32), ue, grp)
        xsf = to_np(bufs["x_sf"][torch.from_numpy(rows).cuda()])
        assert np.array_equal(xq, q_ref)
        if ue:
            assert np.array_equal(xsf, O.pack_ue8m0_rows(s_ref))
        else:
            assert np.array_equal(xsf.view(np.uint32), s_ref.view(np.uint32))
    # a few whole tokens through the oracle
    routed = np.flatnonzero((st["slot_row"] >= 0).any(axis=1))
    tokens = sorted(set(rng.choice(routed, min(3, routed.size), replace=False).tolist()))
    print(f"[fullsize] {name}: oracle on tokens {tokens}", flush=True)
    ref = O.forward_tokens(h, tokens, st)
    gate_up, a2_q, down = (to_np(chain[k]) for k in ("gate_up", "a2_q", "down"))
    a2_sf = None if chain["a2_sf"] is None else to_np(chain["a2_sf"])
    for r, info in ref["rows"].items():
        e = info["expert"]
        s_abs = abs_gemm_cfg(cfg, info["x_q"][None],
                             None if info["x_sf"] is None else info["x_sf"][None],
                             O._np(inp["w13"][e]), O._np(inp["w13_sf"][e]))
        check_gemm(gate_up[r:r + 1], info["gate_up"][None], s_abs, f"{name} gate_up row {r}")
        if cfg.act_quant == "bf16":
            check_bf16_act_chain(a2_q[r:r + 1], info["a2_q"][None], info["gate_up"][None],
                                 s_abs, f"{name} a2 row {r}")
        else:
            check_requant_chain(a2_q[r:r + 1], a2_sf[r:r + 1], info["a2_q"][None],
                                info["a2_sf"][None], info["gate_up"][None], s_abs, ue,
                                f"{name} a2 row {r}", grp)
        check_output(down[r:r + 1], info["down"][None], f"{name} down row {r}")
    got = to_np(out)[tokens]
    want = np.stack([ref["out"][t] for t in tokens])
    rel, mx = check_output(got, want, f"{name} output rows {tokens}")
    print(f"[fullsize] {name}: sampled rel_frobenius={rel:.3e}", flush=True)
