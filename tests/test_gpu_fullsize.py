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
                         check_requant_chain, to_dev, to_np)
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
    # whole tokens through the oracle: one routed to the hottest expert (the
    # most m-tiles, and the deepest schedule chunks), one routed to the
    # expert with the fewest rows (a single m-tile), and random ones
    tokens = sample_tokens(st, rng)
    print(f"[fullsize] {name}: oracle on tokens {tokens}", flush=True)
    ref = O.forward_tokens(h, tokens, st)
    gate_up, a2_q, down = (to_np(chain[k]) for k in ("gate_up", "a2_q", "down"))
    a2_sf = None if chain["a2_sf"] is None else to_np(chain["a2_sf"])
    rows = sorted(ref["rows"])
    # w2 alone, to its element bound: the oracle's a2 rows replace the GPU's
    # in a copy of the chain's a2, the GPU's w2 GEMM runs on that copy, and
    # those rows' outputs are held to the oracle's down rows (the oracle
    # never takes a GPU intermediate as input)
    q_rows = np.stack([ref["rows"][r]["a2_q"] for r in rows])
    s_rows = None if a2_sf is None else np.stack([ref["rows"][r]["a2_sf"] for r in rows])
    idx = torch.tensor(rows, dtype=torch.int64, device="cuda")
    a2_q_in = chain["a2_q"].clone()
    a2_q_in[idx] = to_dev(q_rows)
    a2_sf_in = None
    if s_rows is not None:
        a2_sf_in = chain["a2_sf"].clone()
        a2_sf_in[idx] = to_dev(O.pack_ue8m0_rows(s_rows) if ue and grp == 128 else s_rows)
    down_in = torch.empty_like(chain["down"])
    moe.grouped_gemm_w2(moe.Problem.from_config(cfg), a2_q_in, a2_sf_in, bufs, inp["w2"],
                        inp["w2_sf"], down_in)
    torch.cuda.synchronize()
    down_in = to_np(down_in)
    gu_got, gu_want, gu_abs, dn_got, dn_want, dn_abs = [], [], [], [], [], []
    for i, r in enumerate(rows):
        info = ref["rows"][r]
        e = info["expert"]
        w13e, w13s = O._np(inp["w13"][e]), O._np(inp["w13_sf"][e])
        w2e, w2s = O._np(inp["w2"][e]), O._np(inp["w2_sf"][e])
        gu_abs.append(abs_gemm_cfg(cfg, info["x_q"][None],
                                   None if info["x_sf"] is None else info["x_sf"][None],
                                   w13e, w13s)[0])
        gu_got.append(gate_up[r])
        gu_want.append(info["gate_up"])
        dn_abs.append(abs_gemm_cfg(cfg, q_rows[i:i + 1],
                                   None if s_rows is None else s_rows[i:i + 1], w2e, w2s)[0])
        dn_got.append(down_in[r])
        dn_want.append(info["down"])
    gu_got, gu_want, gu_abs = np.stack(gu_got), np.stack(gu_want), np.stack(gu_abs)
    f13 = check_gemm(gu_got, gu_want, gu_abs, f"{name} gate_up rows {rows}")
    f2 = check_gemm(np.stack(dn_got), np.stack(dn_want), np.stack(dn_abs),
                    f"{name} down rows {rows} (w2 on the oracle's a2)")
    a2_want = np.stack([ref["rows"][r]["a2_q"] for r in rows])
    if cfg.act_quant == "bf16":
        fa = check_bf16_act_chain(a2_q[rows], a2_want, gu_want, gu_abs, f"{name} a2 rows")
    else:
        sf_want = np.stack([ref["rows"][r]["a2_sf"] for r in rows])
        fa = check_requant_chain(a2_q[rows], a2_sf[rows], a2_want, sf_want, gu_want, gu_abs, ue,
                                 f"{name} a2 rows", grp)
    check_output(down[rows], np.stack([ref["rows"][r]["down"] for r in rows]),
                 f"{name} down rows (oracle chain)")
    got = to_np(out)[tokens]
    want = np.stack([ref["out"][t] for t in tokens])
    rel, mx = check_output(got, want, f"{name} output rows {tokens}")
    print(f"[fullsize] {name}: {len(rows)} rows; differing gate_up {f13:.3%}, down {f2:.3%}, "
          f"a2 {fa:.3%}; sampled output rel_frobenius={rel:.3e}", flush=True)


def sample_tokens(st, rng, n_random=3):
    """A token of the hottest expert, a token of the least loaded routed
    expert (a single m-tile wherever some expert fits in one), and n_random
    other routed tokens."""
    ids, counts = st["ids"], st["counts"]
    routed_slots = st["slot_row"] >= 0
    routed = np.flatnonzero(routed_slots.any(axis=1))
    picks = []
    hot = int(np.argmax(counts))
    live = np.flatnonzero(counts > 0)
    cold = int(live[np.argmin(counts[live])])
    for e in (hot, cold):
        t_of_e = np.flatnonzero(((ids == e) & routed_slots).any(axis=1))
        picks.append(int(rng.choice(t_of_e)))
    rest = np.setdiff1d(routed, picks)
    picks += rng.choice(rest, min(n_random, rest.size), replace=False).tolist()
    return sorted(set(int(t) for t in picks))
