"""GPU parity of the indexed experts layout (moe_align_block_size, the
gather / scatter GEMMs on the block map and moe_fused_mul_sum) against the
oracle's align_block_size / forward_indexed, through the C ABI.

The block map is integer work: compared bit for bit.  Per row the indexed
GEMMs run the contiguous layout's arithmetic, so their a2 / down rows (both
in (token, slot) order) and the fused mul-sum must equal the contiguous
chain's bits exactly; the layer output is also checked against the oracle's
indexed forward.  Rows of unrouted slots in a2 and down carry a sentinel that
must survive.  w2 also runs on a block map of another block size, as the
experts do when their w2 tuning picks one.
"""
import dataclasses
import os

import numpy as np
import pytest
import torch

import fp8_block_quantized_group_amd as moe
import moe_synth
from oracle import moe_oracle as O
from parity_util import check_output, to_np
from test_gpu_parity import (SENTINEL_BF16, SENTINEL_U8, SMALL, case, gpu, problem,  # noqa: F401
                             run_chain, stage_on_gpu, tile160_ok)

pytestmark = pytest.mark.gpu

# the contiguous-routing configs of the small set (the block map needs them)
NAMES = [n for n, c in SMALL.items() if c.layout != "batched"]


def _block_sizes(cfg):
    return [16, 32, 64, 128] + ([160] if tile160_ok(cfg) else []) + \
        ([] if cfg.act_quant == "bf16" else [192, 256])


def run_indexed(cfg, dev, bs, bs2=None):
    """stage -> align -> w13+act (indexed) -> w2 (indexed, on a block map of
    block size bs2, default bs) -> fused mul-sum."""
    p, bufs = stage_on_gpu(cfg, dev)
    ix = moe.alloc_indexed(p, bs)
    ix["sorted_ids"].fill_(-5)
    ix["expert_ids"].fill_(-5)
    moe.align_block_size(p, bufs["topk_idx"], bufs, ix)
    ix2 = ix
    if bs2 is not None and bs2 != bs:
        ix2 = moe.alloc_indexed(p, bs2)
        moe.align_block_size(p, bufs["topk_idx"], bufs, ix2)
    rows = cfg.T * cfg.top_k
    if cfg.act_quant == "bf16":
        a2_q = torch.full((rows, cfg.N), SENTINEL_BF16, dtype=torch.int16,
                          device="cuda").view(torch.bfloat16)
        a2_sf = None
    else:
        a2_q = torch.full((rows, cfg.N), SENTINEL_U8, dtype=torch.uint8, device="cuda")
        a2_sf = torch.full((rows, moe.sizes(p)["a2_sf_row"]), 0x7F,
                           dtype=moe.scale_dtype(p), device="cuda")
    moe.grouped_gemm_w13_act_indexed(p, bufs["x_q"], bufs["x_sf"], ix, dev["w13"],
                                     dev["w13_sf"], a2_q, a2_sf)
    down = torch.full((rows, cfg.K), SENTINEL_BF16, dtype=torch.int16,
                      device="cuda").view(torch.bfloat16)
    moe.grouped_gemm_w2_indexed(p, a2_q, a2_sf, ix2, dev["w2"], dev["w2_sf"], down)
    out = torch.empty((cfg.T, cfg.K), dtype=torch.bfloat16, device="cuda")
    moe.fused_mul_sum(p, down, bufs["topk_idx"], bufs["topk_w"], out)
    torch.cuda.synchronize()
    return {"bufs": bufs, "ix": ix, "a2_q": a2_q, "a2_sf": a2_sf, "down": down, "out": out}


def _u16(t):
    return to_np(t.view(torch.int16)).view(np.uint16) if t.dtype == torch.bfloat16 else to_np(t)


@pytest.mark.parametrize("name", NAMES)
def test_align_block_size_bit_exact(gpu, name):
    cfg, h, dev, ref = case(name)
    for bs in _block_sizes(cfg):
        r = run_indexed(cfg, dev, bs)
        sid, eid, P = O.align_block_size(ref["ids"], cfg.E, bs)
        got_P = int(r["ix"]["num_tokens_padded"].item())
        assert got_P == P, (name, bs, got_P, P)
        assert np.array_equal(to_np(r["ix"]["sorted_ids"])[:P], sid), (name, bs)
        assert np.array_equal(to_np(r["ix"]["expert_ids"])[:P // bs], eid), (name, bs)
        # nothing past the padded total is written
        assert np.all(to_np(r["ix"]["sorted_ids"])[P:] == -5)
        assert np.all(to_np(r["ix"]["expert_ids"])[P // bs:] == -5)


@pytest.mark.parametrize("name", NAMES)
def test_indexed_layer_matches_contiguous_and_oracle(gpu, name):
    cfg, h, dev, ref = case(name)
    chain = run_chain(cfg, dev)
    slot_row = to_np(chain["bufs"]["slot_row"]).reshape(-1)
    c_a2 = _u16(chain["a2_q"])
    c_sf = None if chain["a2_sf"] is None else to_np(chain["a2_sf"])
    c_down = _u16(chain["down"])
    c_out = _u16(chain["out"])
    numel = cfg.T * cfg.top_k
    routed = np.flatnonzero(slot_row >= 0)
    unrouted = np.flatnonzero(slot_row < 0)
    sizes = _block_sizes(cfg)
    for n_bs, bs in enumerate(sizes):
        # w2 on its own block map (another block size) every other time
        bs2 = sizes[(n_bs + 1) % len(sizes)] if n_bs % 2 else bs
        r = run_indexed(cfg, dev, bs, bs2)
        P = int(r["ix"]["num_tokens_padded"].item())
        sid = to_np(r["ix"]["sorted_ids"])[:P]
        assert np.array_equal(np.sort(sid[sid < numel]), routed)
        # a2 row s is the contiguous a2 row of slot s, bit for bit
        a2 = _u16(r["a2_q"])
        assert np.array_equal(a2[routed], c_a2[slot_row[routed]]), (name, bs, "a2")
        if c_sf is not None:
            assert np.array_equal(to_np(r["a2_sf"])[routed], c_sf[slot_row[routed]]), \
                (name, bs, "a2_sf")
        sent = SENTINEL_BF16 if cfg.act_quant == "bf16" else SENTINEL_U8
        assert np.all(a2[unrouted] == sent), (name, bs, "unrouted rows written")
        # down row s (token, slot order) is the contiguous down row of that slot
        down = _u16(r["down"])
        assert np.array_equal(down[routed], c_down[slot_row[routed]]), (name, bs, "down")
        assert np.all(down[unrouted] == SENTINEL_BF16), (name, bs, "unrouted rows written")
        # the fused mul-sum sums the same values in the same order as the reduce
        assert np.array_equal(_u16(r["out"]), c_out), (name, bs, "out")
    ref_ix = O.forward_indexed(h, 64)
    check_output(_u16(r["out"]), ref_ix["out"], f"{name} indexed layer vs oracle")
    check_output(down[routed], ref_ix["down"][routed], f"{name} indexed down vs oracle")


@pytest.mark.parametrize("name", NAMES)
def test_fused_mul_sum_isolated(gpu, name):
    """On the oracle's own down rows (token, slot order) and repacked ids."""
    cfg, h, dev, ref = case(name)
    p = problem(cfg)
    numel = cfg.T * cfg.top_k
    rng = np.random.default_rng(7)
    down = O.bf16_round(rng.standard_normal((numel, cfg.K)))
    ids = np.asarray(ref["ids"], np.int64)
    w = np.asarray(ref["weights"], np.float32)
    expect = O.fused_mul_sum(down, ids, w, cfg.E)
    out = torch.empty((cfg.T, cfg.K), dtype=torch.bfloat16, device="cuda")
    moe.fused_mul_sum(p, torch.from_numpy(down.view(np.int16)).cuda().view(torch.bfloat16),
                      torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda(), out)
    torch.cuda.synchronize()
    # fp32 accumulation of top_k products vs the fp64 sum, each rounded once
    # to bf16: apart by at most one bf16 step of the result plus the fp32
    # error bound k * 2^-24 * sum |w * down|
    g, e = O.bf16_to_f64(_u16(out)), O.bf16_to_f64(expect)
    ok = (ids >= 0) & (ids < cfg.E)
    mag = np.einsum("tj,tjc->tc", np.abs(w.astype(np.float64)) * ok,
                    np.abs(O.bf16_to_f64(down)).reshape(cfg.T, cfg.top_k, cfg.K))
    bound = np.abs(e) * 2.0 ** -7 + 2.0 ** -133 + cfg.top_k * 2.0 ** -24 * mag * 2
    assert np.all(np.abs(g - e) <= bound), name
    assert np.all(g[~ok.any(axis=1)] == 0)


def test_forward_indexed_layout(gpu):
    """moe_forward with layout INDEXED equals the contiguous moe_forward bit
    for bit, at every block size it can choose."""
    for name in ("ragged", "skewed", "mx4_skewed", "bf16_ragged"):
        cfg, h, dev, ref = case(name)
        chain = run_chain(cfg, dev)
        cfg_ix = dataclasses.replace(cfg, layout="indexed")
        for bs in (_block_sizes(cfg)[0], 64, 128):
            os.environ["MOE_TILE_M"] = str(bs)
            try:
                p = problem(cfg_ix)
                assert p.layout == moe.LAYOUT_INDEXED and moe.sizes(p)["tile_m"] == bs
                layer = moe.MoeLayer(p, dev["w13"], dev["w13_sf"], dev["w2"], dev["w2_sf"])
                if dev["eplb"] is not None:
                    dev["eplb"]["expert_load"].zero_()
                out = layer(dev["hidden"], dev["topk_ids"], dev["topk_weights"], None,
                            dev["is_padding"], dev["expert_num_tokens"], dev["eplb"])
                torch.cuda.synchronize()
            finally:
                del os.environ["MOE_TILE_M"]
            assert np.array_equal(_u16(out), _u16(chain["out"])), (name, bs)


def test_indexed_degenerate_routing(gpu):
    """Every slot unrouted (no blocks at all), one token, and every expert
    holding exactly one slot (every block mostly padding)."""
    cases = []
    cfg = moe_synth.custom(name="ix_none", T=24, E=3, top_k=2, K=256, N=256, seed=41)
    inp = moe_synth.make_inputs(cfg, "cpu")
    inp["topk_ids"] = torch.full_like(inp["topk_ids"], -1)
    cases.append((cfg, inp))
    cfg = moe_synth.custom(name="ix_one", T=1, E=6, top_k=3, K=256, N=256, seed=42)
    cases.append((cfg, moe_synth.make_inputs(cfg, "cpu")))
    cfg = moe_synth.custom(name="ix_spread", T=16, E=64, top_k=4, K=256, N=384, seed=43)
    inp = moe_synth.make_inputs(cfg, "cpu")
    inp["topk_ids"] = torch.arange(64, dtype=torch.int32).reshape(16, 4)
    cases.append((cfg, inp))
    for cfg, inp in cases:
        h = O.host_inputs(inp)
        dev = {k: (v.to("cuda") if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
        for bs in (16, 128):
            r = run_indexed(cfg, dev, bs)
            sid, eid, P = O.align_block_size(O.stage(h)["ids"], cfg.E, bs)
            assert int(r["ix"]["num_tokens_padded"].item()) == P
            assert np.array_equal(to_np(r["ix"]["sorted_ids"])[:P], sid)
            assert np.array_equal(to_np(r["ix"]["expert_ids"])[:P // bs], eid)
            ref = O.forward_indexed(h, bs)
            check_output(_u16(r["out"]), ref["out"], f"{cfg.name} bs={bs}")
            if P == 0:
                assert np.all(_u16(r["out"]) == 0)
