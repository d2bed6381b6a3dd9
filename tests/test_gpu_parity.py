"""GPU parity of every step of the layer against the CPU oracle, through the
C ABI (libmoe_fp8.so), at sizes the oracle runs in seconds that still span
several GEMM tiles and ragged tails.

Each step is first run in isolation on the oracle's own inputs for that
step (so an upstream difference cannot hide a bug), then the whole layer is
run end to end.  Masked rows of the batched layout and rows past an expert's
count are poisoned with NaN codes / infinite scales on input and a sentinel
on output, so reading or writing them fails the test.
"""
import os

import numpy as np
import pytest
import torch

import fp8_block_quantized_group_amd as moe
import moe_synth
from oracle import moe_oracle as O
from parity_util import (abs_gemm_cfg, check_bf16_act_chain, check_bf16_close, check_gemm,
                         check_output, check_requant, check_requant_chain, to_dev, to_np)

pytestmark = pytest.mark.gpu

SENTINEL_BF16 = 0x7FBF          # a NaN pattern no kernel produces
SENTINEL_U8 = 0xA5

SMALL = {
    "tiny": moe_synth.CONFIGS["tiny"],
    "ragged": moe_synth.custom(name="ragged", T=300, E=5, top_k=3, K=384, N=384, seed=21,
                               pad_frac=0.07),
    "batched": moe_synth.custom(name="batched", T=250, E=4, top_k=2, K=384, N=256, seed=22,
                                layout="batched", max_tokens=160),
    "eplb_fp32": moe_synth.custom(name="eplb_fp32", T=200, E=7, top_k=4, K=256, N=384,
                                  seed=23, act_quant="fp32", num_logical=5),
    "skewed": moe_synth.custom(name="skewed", T=400, E=16, top_k=4, K=256, N=256, seed=24,
                               routing="zipf", zipf_s=1.1, pad_frac=0.05),
    # MX scheme pair (kMxfp8Static, kMxfp8Dynamic): 32-column E8M0 scales
    "mx_ragged": moe_synth.custom(name="mx_ragged", T=300, E=5, top_k=3, K=384, N=384,
                                  seed=25, pad_frac=0.07, act_quant="mxfp8",
                                  weight_quant="mxfp8"),
    "mx_batched": moe_synth.custom(name="mx_batched", T=250, E=4, top_k=2, K=384, N=256,
                                   seed=26, layout="batched", max_tokens=160,
                                   act_quant="mxfp8", weight_quant="mxfp8"),
    # (kFp8Static128BlockSym, None): unquantized bf16 activations
    "bf16_ragged": moe_synth.custom(name="bf16_ragged", T=300, E=5, top_k=3, K=384, N=384,
                                    seed=29, pad_frac=0.07, act_quant="bf16"),
    "bf16_batched": moe_synth.custom(name="bf16_batched", T=250, E=4, top_k=2, K=384, N=256,
                                     seed=30, layout="batched", max_tokens=160,
                                     act_quant="bf16"),
    # (kMxfp4Static, kMxfp8Dynamic): e2m1 weights
    "mx4_ragged": moe_synth.custom(name="mx4_ragged", T=300, E=5, top_k=3, K=384, N=384,
                                   seed=27, pad_frac=0.07, act_quant="mxfp8",
                                   weight_quant="mxfp4"),
    # zipf-skewed routing with fp32 scales and in the batched layout: experts
    # of a few rows next to experts of several 128-row tiles
    "skewed_fp32": moe_synth.custom(name="skewed_fp32", T=400, E=16, top_k=4, K=256, N=256,
                                    seed=31, routing="zipf", zipf_s=1.1, pad_frac=0.05,
                                    act_quant="fp32"),
    "skewed_batched": moe_synth.custom(name="skewed_batched", T=400, E=8, top_k=2, K=512,
                                       N=256, seed=32, layout="batched", max_tokens=400,
                                       routing="zipf", zipf_s=1.1),
    "mx4_skewed": moe_synth.custom(name="mx4_skewed", T=400, E=16, top_k=4, K=256, N=256,
                                   seed=28, routing="zipf", zipf_s=1.1, act_quant="mxfp8",
                                   weight_quant="mxfp4"),
}


# Mid-size configs: K and N between 1152 and 2048, so each GEMM runs 9-16
# k-steps.  Every LDS ring depth (2, 3 and 4 slots) wraps several times and
# both slots of the MX weight-scale panel (which alternate every 4 k-steps)
# are used; N = 1152 (hidden K = 1152 for w2's output) takes the 128-column
# w2 tiles, 2048 the 256-column ones.  Run at tile heights 16, 128 and 256
# (128 at most for bf16 activations) with every routed row compared.
MID = {
    "mid_ue8m0": moe_synth.custom(name="mid_ue8m0", T=320, E=6, top_k=3, K=2048, N=1152,
                                  seed=41, routing="zipf", zipf_s=1.1, pad_frac=0.05),
    "mid_fp32": moe_synth.custom(name="mid_fp32", T=320, E=7, top_k=3, K=1152, N=2048,
                                 seed=42, act_quant="fp32", num_logical=5),
    "mid_mxfp8": moe_synth.custom(name="mid_mxfp8", T=320, E=6, top_k=3, K=2048, N=1152,
                                  seed=43, routing="zipf", zipf_s=1.1, pad_frac=0.05,
                                  act_quant="mxfp8", weight_quant="mxfp8"),
    "mid_mxfp4": moe_synth.custom(name="mid_mxfp4", T=320, E=6, top_k=3, K=1152, N=2048,
                                  seed=44, routing="zipf", zipf_s=1.1, act_quant="mxfp8",
                                  weight_quant="mxfp4"),
    "mid_bf16": moe_synth.custom(name="mid_bf16", T=320, E=6, top_k=3, K=2048, N=1152,
                                 seed=45, routing="zipf", zipf_s=1.1, pad_frac=0.05,
                                 act_quant="bf16"),
    "mid_batched": moe_synth.custom(name="mid_batched", T=320, E=4, top_k=2, K=1152,
                                    N=2048, seed=46, layout="batched", max_tokens=384,
                                    routing="zipf", zipf_s=1.1),
}
# w2 reductions of N >= 8192 split in two (split-K): N = 8192 (64 k-steps)
MID.update({
    "split_ue8m0": moe_synth.custom(name="split_ue8m0", T=200, E=4, top_k=2, K=512, N=8192,
                                    seed=47, routing="zipf", zipf_s=1.1, pad_frac=0.05),
    "split_mxfp8": moe_synth.custom(name="split_mxfp8", T=200, E=4, top_k=2, K=512, N=8192,
                                    seed=48, act_quant="mxfp8", weight_quant="mxfp8"),
    "split_bf16": moe_synth.custom(name="split_bf16", T=200, E=4, top_k=2, K=512, N=8192,
                                   seed=49, act_quant="bf16"),
    "split_batched": moe_synth.custom(name="split_batched", T=200, E=4, top_k=2, K=512,
                                      N=8192, seed=50, layout="batched", max_tokens=160),
})
# 128-row tiles (about 96 rows per expert) with Zipf skew: the heaviest
# experts exceed 128 rows and go to the second (256-row) tile list
TALL = {
    "tall_ue8m0": moe_synth.custom(name="tall_ue8m0", T=256, E=8, top_k=3, K=1024, N=1024,
                                   seed=52, routing="zipf", zipf_s=1.1, pad_frac=0.05),
    "tall_fp32": moe_synth.custom(name="tall_fp32", T=256, E=8, top_k=3, K=1024, N=1024,
                                  seed=53, routing="zipf", zipf_s=1.1, act_quant="fp32"),
    "tall_mxfp4": moe_synth.custom(name="tall_mxfp4", T=256, E=8, top_k=3, K=1024, N=1024,
                                   seed=54, routing="zipf", zipf_s=1.1, act_quant="mxfp8",
                                   weight_quant="mxfp4"),
    "tall_batched": moe_synth.custom(name="tall_batched", T=256, E=8, top_k=3, K=1024,
                                     N=1024, seed=55, layout="batched", max_tokens=256,
                                     routing="zipf", zipf_s=1.1),
}
MID.update(TALL)
MID_TILES = [16, 128, 256]


def tile160_ok(cfg):
    """160-row tiles run the block scheme with per-128 fp8 activations only."""
    return cfg.act_quant in ("ue8m0", "fp32") and cfg.weight_quant == "fp8_block128"


# the 160-row tiles (a 3-slot ring beside a shortened weight-scale panel)
# on every mid-size config of the block scheme
MID_CASES = [(n, t) for n in MID for t in MID_TILES
             if not (MID[n].act_quant == "bf16" and t > 128) and n not in TALL] + \
    [(n, 160) for n in MID if tile160_ok(MID[n]) and n not in TALL]
CASES = {**SMALL, **MID}


@pytest.fixture(scope="session")
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    moe.load_library()
    return torch.device("cuda:0")


_CACHE = {}


def case(name):
    """(cfg, host inputs, device inputs, oracle forward) for a small config."""
    if name not in _CACHE:
        cfg = CASES[name]
        inp = moe_synth.make_inputs(cfg, "cpu")
        h = O.host_inputs(inp)
        ref = O.forward(h)
        _CACHE[name] = (cfg, h, inp, ref)
    cfg, h, inp, ref = _CACHE[name]
    dev = {}
    for k, v in inp.items():
        if isinstance(v, torch.Tensor):
            dev[k] = v.to("cuda")
        elif k == "eplb" and v is not None:
            dev[k] = {k2: v2.to("cuda") if isinstance(v2, torch.Tensor) and k2 != "replica_of"
                      else v2 for k2, v2 in v.items()}
        else:
            dev[k] = v
    return cfg, h, dev, ref


def problem(cfg):
    return moe.Problem.from_config(cfg)


def valid_rows(cfg, ref):
    """Row indices holding routed data (the rest are masked)."""
    if cfg.layout == "batched":
        return np.concatenate([np.arange(e * cfg.max_tokens, e * cfg.max_tokens + int(c))
                               for e, c in enumerate(ref["counts"])]).astype(np.int64)
    return np.arange(int(ref["offsets"][-1]))


def stage_on_gpu(cfg, dev):
    p = problem(cfg)
    bufs = moe.alloc_stage_outputs(p)
    if dev["eplb"] is not None:
        dev["eplb"]["expert_load"].zero_()
    moe.stage(p, dev["hidden"], dev["topk_ids"], dev["topk_weights"], bufs,
              dev["is_padding"], dev["expert_num_tokens"], dev["eplb"])
    torch.cuda.synchronize()
    return p, bufs


def host_tile_list(counts, tile_m, n_entries, bases, max_tiles):
    """Every (expert, m0) tile in plain expert order, one group per expert,
    all in the main list (a tall list, if the plan has one, stays empty:
    count 0) -- test plumbing: the GEMM must not depend on the order or the
    split the routing step emits.  bases: each expert's first row in the
    GEMM's row space."""
    E = len(counts)
    tl = np.zeros(n_entries, np.int32)
    info = tl[4:4 + 8 * max_tiles].reshape(max_tiles, 8)
    groups = tl[4 + 8 * max_tiles:]
    pos = 0
    for e, c in enumerate(counts):
        groups[e] = pos
        first, n = pos, -(-int(c) // tile_m)
        for m0 in range(0, int(c), tile_m):
            info[pos] = (e, m0, first, n, int(c), int(bases[e]), first, 0)
            pos += 1
    groups[E] = pos
    tl[0], tl[1] = pos, E
    return tl


def expected_schedule(tiles_per_expert):
    """The documented schedule: chunks of at most S = max(8, ceil(n / 1024))
    m-tiles per expert, sorted by size (full chunks first in expert order,
    then remainders r by the class floor(8r / S) descending, ties by expert),
    dealt in rounds of 8 to the bins ranked by (tiles so far, bin index),
    bins concatenated.
    Returns the (expert, m-tile index) sequence and the group sizes."""
    n = int(sum(tiles_per_expert))
    S = max(8, -(-n // 1024))
    full = [(e, j * S, S) for e, t in enumerate(tiles_per_expert) for j in range(t // S)]
    rem = sorted(((e, (t // S) * S, t % S) for e, t in enumerate(tiles_per_expert) if t % S),
                 key=lambda c: (-(c[2] * 8 // S), c[0]))
    chunks = full + rem
    load, bins = [0] * 8, [[] for _ in range(8)]
    for r0 in range(0, len(chunks), 8):
        rank = sorted(range(8), key=lambda x: (load[x], x))
        for i, ch in enumerate(chunks[r0:r0 + 8]):
            bins[rank[i]].append(ch)
            load[rank[i]] += ch[2]
    seq, sizes = [], []
    for b in bins:
        for e, m, c in b:
            seq += [(e, m + t) for t in range(c)]
            sizes.append(c)
    return seq, sizes


def oracle_routing(p, cfg, ref):
    """Device routing arrays built from the oracle's layout."""
    s = moe.sizes(p)
    slots = max(s["slots"], 1)
    row_src = np.zeros(slots, np.int32)
    row_src[:len(ref["row_src"])] = ref["row_src"]
    return {
        "expert_num_tokens": to_dev(ref["counts"].astype(np.int32)),
        "expert_offsets": to_dev(ref["offsets"].astype(np.int32)),
        "row_src": to_dev(row_src),
        "slot_row": to_dev(ref["slot_row"].reshape(-1).astype(np.int32)),
        "tile_list": to_dev(host_tile_list(
            ref["counts"], s["tile_m"], s["tile_list"],
            [e * cfg.max_tokens for e in range(cfg.E)] if cfg.layout == "batched"
            else ref["offsets"][:-1], s["max_tiles"])),
    }


_ABS = {}


def gemm_abs(cfg, h, ref, which):
    """S_abs per output element (the oracle's GEMM on absolute values), for
    the GEMM tolerance; rows laid out like the oracle's intermediates."""
    key = (cfg.name, which)
    if key in _ABS:
        return _ABS[key]
    ue = O.act_e8m0(cfg)
    cols = 2 * cfg.N if which == "w13" else cfg.K
    out = np.zeros((ref["gate_up"].shape[0], cols))
    for e, c in enumerate(ref["counts"]):
        c = int(c)
        if c == 0:
            continue
        if cfg.layout == "batched":
            rows = np.arange(e * cfg.max_tokens, e * cfg.max_tokens + c)
            a_rows = rows
        else:
            lo = int(ref["offsets"][e])
            rows = np.arange(lo, lo + c)
            a_rows = ref["row_src"][rows]
        if which == "w13":
            x_sf = None if ref["x_sf"] is None else ref["x_sf"][a_rows]
            out[rows] = abs_gemm_cfg(cfg, ref["x_q"][a_rows], x_sf,
                                     h["w13"][e], h["w13_sf"][e])
        else:
            a2_sf = None if ref["a2_sf"] is None else ref["a2_sf"][rows]
            out[rows] = abs_gemm_cfg(cfg, ref["a2_q"][rows], a2_sf,
                                     h["w2"][e], h["w2_sf"][e])
    _ABS[key] = out
    return out


def poisoned(arr, rows, value):
    """Copy with every row not in `rows` set to `value`."""
    out = np.full_like(arr, value)
    out[rows] = arr[rows]
    return out


def sf_poison(ue8m0):
    return 255 if ue8m0 else np.float32(np.inf)


# ---------------------------------------------------------------------------
# step 1: the group quantizer, exhaustively over bf16
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("scheme", ["ue8m0", "fp32", "mxfp8"])
def test_stage_quant_every_bf16_value(gpu, scheme):
    """Every finite bf16 value alone in its group and packed densely, for the
    per-128 UE8M0 / fp32 schemes and the per-32 MXFP8 scheme: codes and
    scales bit-exact."""
    ue8m0 = scheme != "fp32"
    group = 32 if scheme == "mxfp8" else 128
    act = {"ue8m0": moe.Q_FP8_UE8M0, "fp32": moe.Q_FP8_F32, "mxfp8": moe.Q_MXFP8}[scheme]
    wq = moe.W_MXFP8 if scheme == "mxfp8" else moe.W_FP8_BLOCK128
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = np.isfinite(O.bf16_to_f64(bits))
    vals = bits[finite]
    n = vals.size
    # (a) each value alone in its group: every amax the exponent rule can see
    alone = np.zeros((n, 128), np.uint16)
    alone[:, 5] = vals
    # (b) dense groups: 128 consecutive values share one scale
    dense = np.zeros(((n + 127) // 128) * 128, np.uint16)
    dense[:n] = vals
    dense = dense.reshape(-1, 128)
    for x in (alone, dense):
        rows = x.shape[0]
        p = moe.Problem(rows, 128, 128, 1, 1, act_quant=act, weight_quant=wq)
        bufs = moe.alloc_stage_outputs(p)
        ids = torch.zeros((rows, 1), dtype=torch.int32, device="cuda")
        w = torch.ones((rows, 1), dtype=torch.float32, device="cuda")
        moe.stage(p, to_dev(x), ids, w, bufs)
        torch.cuda.synchronize()
        q_ref, s_ref = O.quantize_groups(O.bf16_to_f64(x).astype(np.float32), ue8m0, group)
        assert np.array_equal(to_np(bufs["x_q"]), q_ref)
        sf = to_np(bufs["x_sf"])
        if ue8m0:
            assert np.array_equal(sf, O.pack_ue8m0_rows(s_ref))
        else:
            assert np.array_equal(sf.view(np.uint32), s_ref.view(np.uint32))


# ---------------------------------------------------------------------------
# step 1-2 on the configs: staging + routing, bit-exact
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", list(SMALL))
def test_stage_and_route_bit_exact(gpu, name):
    cfg, h, dev, ref = case(name)
    p, bufs = stage_on_gpu(cfg, dev)
    ue = O.act_e8m0(cfg)
    rows = valid_rows(cfg, ref) if cfg.layout == "batched" else np.arange(cfg.T)
    assert np.array_equal(to_np(bufs["x_q"])[rows], ref["x_q"][rows])
    if cfg.act_quant == "bf16":
        assert bufs["x_sf"] is None and ref["x_sf"] is None
    elif ue:
        sf = to_np(bufs["x_sf"])[rows]
        assert np.array_equal(sf, O.pack_ue8m0_rows(ref["x_sf"][rows]))
    else:
        sf = to_np(bufs["x_sf"])[rows]
        assert np.array_equal(sf.view(np.uint32), ref["x_sf"][rows].view(np.uint32))
    assert np.array_equal(to_np(bufs["topk_idx"]), ref["ids"])
    assert np.array_equal(to_np(bufs["topk_w"]).view(np.uint32), ref["weights"].view(np.uint32))
    assert np.array_equal(to_np(bufs["expert_num_tokens"]), ref["counts"])
    M = int(ref["offsets"][-1])
    if cfg.layout != "batched":
        assert np.array_equal(to_np(bufs["expert_offsets"]), ref["offsets"])
        assert np.array_equal(to_np(bufs["row_src"])[:M], ref["row_src"])
    assert np.array_equal(to_np(bufs["slot_row"]).reshape(cfg.T, cfg.top_k), ref["slot_row"])
    if cfg.eplb:
        assert np.array_equal(to_np(dev["eplb"]["expert_load"]), ref["load"])
    bases = ([e * cfg.max_tokens for e in range(cfg.E)] if cfg.layout == "batched"
             else ref["offsets"][:-1])
    check_schedule(bufs["tile_list"], ref["counts"], moe.sizes(p), cfg.E, bases)


def _check_one_list(tl, tiles, bm, max_tiles, counts, bases, tile0):
    """One tile list: every listed expert's tiles exactly once, in the
    documented XCD-balanced order, groups of consecutive m-tiles of one
    expert, and each tile's information (group, expert rows, first row, the
    expert's first block of the indexed block map: tile0)."""
    n, G = int(tl[0]), int(tl[1])
    assert tl[2] == 0 and tl[3] == 0
    info = tl[4:4 + 8 * n].reshape(n, 8)
    seq, sizes = expected_schedule(tiles)
    assert [(int(e), int(m0) // bm) for e, m0 in info[:, :2]] == seq
    assert np.all(info[:, 1] % bm == 0)
    groups = tl[4 + 8 * max_tiles:4 + 8 * max_tiles + G + 1]
    assert G == len(sizes) and groups[0] == 0 and groups[-1] == n
    assert list(np.diff(groups)) == sizes
    for g in range(G):
        seg = info[groups[g]:groups[g + 1]]
        assert np.all(seg[:, 0] == seg[0, 0])
        assert list(seg[:, 1]) == list(range(int(seg[0, 1]), int(seg[0, 1]) + len(seg) * bm, bm))
        assert np.all(seg[:, 2] == groups[g]) and np.all(seg[:, 3] == len(seg))
        e = int(seg[0, 0])
        assert np.all(seg[:, 4] == int(counts[e])) and np.all(seg[:, 5] == int(bases[e]))
        # the expert's first block of the indexed layout's block map (block
        # size tile_m: every expert's blocks counted, in both lists)
        assert np.all(seg[:, 6] == tile0[e]) and np.all(seg[:, 7] == 0)


def check_schedule(tile_list, counts, s, E, bases):
    """The tile schedule.  With a tall list (s["tall_tile_m"] != 0) the
    experts of more than tile_m rows are scheduled there in tiles of
    tall_tile_m rows and the others in the main list; otherwise every expert
    is in the main list."""
    tl = to_np(tile_list)
    bm, tall = s["tile_m"], s["tall_tile_m"]
    heavy = [tall != 0 and int(c) > bm for c in counts]
    blocks = [-(-int(c) // bm) for c in counts]
    tile0 = np.concatenate([[0], np.cumsum(blocks)[:-1]])
    _check_one_list(tl, [0 if h else b for b, h in zip(blocks, heavy)], bm,
                    s["max_tiles"], counts, bases, tile0)
    if tall:
        off = s["tall_list_offset"]
        assert off % 4 == 0 and off >= 4 + 9 * s["max_tiles"] + E
        _check_one_list(tl[off:], [-(-int(c) // tall) if h else 0 for c, h in zip(counts, heavy)],
                        tall, s["max_tiles_tall"], counts, bases, tile0)


def test_stage_bf16_copy(gpu):
    cfg, h, dev, ref = case("ragged")
    p = moe.Problem.from_config(cfg, act_quant=moe.Q_BF16)
    bufs = moe.alloc_stage_outputs(p)
    moe.stage(p, dev["hidden"], dev["topk_ids"], dev["topk_weights"], bufs, dev["is_padding"])
    torch.cuda.synchronize()
    assert torch.equal(bufs["x_q"].view(torch.int16), dev["hidden"].view(torch.int16))
    assert np.array_equal(to_np(bufs["topk_idx"]), ref["ids"])


# ---------------------------------------------------------------------------
# steps 3-6 in isolation, on the oracle's inputs
# ---------------------------------------------------------------------------

def _gemm_isolated(cfg, h, dev, ref, which):
    p = problem(cfg)
    s = moe.sizes(p)
    ue = O.act_e8m0(cfg)
    routing = oracle_routing(p, cfg, ref)
    vr = valid_rows(cfg, ref)
    bf = cfg.act_quant == "bf16"
    poison = 0x7FC0 if bf else 0x7F            # bf16 NaN / e4m3 NaN outside the counts
    if which == "w13":
        arows = (np.arange(s["stage_rows"]) if cfg.layout != "batched" else vr)
        a_q = poisoned(ref["x_q"], arows, poison)
        a_sf = None
        if not bf:
            a_sf = O.pack_ue8m0_rows(ref["x_sf"]) if ue else ref["x_sf"]
            a_sf = poisoned(a_sf, arows, sf_poison(ue))
        cols = 2 * cfg.N
        want = ref["gate_up"]
    else:
        a_q = np.full((s["expert_rows"], cfg.N), poison, ref["a2_q"].dtype)
        a_q[vr] = ref["a2_q"][vr]
        a_sf = None
        if not bf:
            a_sf = O.pack_ue8m0_rows(ref["a2_sf"]) if ue else ref["a2_sf"]
            a_sf = poisoned(a_sf, vr, sf_poison(ue))
        cols = cfg.K
        want = ref["down"]
    out = torch.full((s["expert_rows"], cols), SENTINEL_BF16, dtype=torch.int16,
                     device="cuda").view(torch.bfloat16)
    w = dev["w13"] if which == "w13" else dev["w2"]
    w_sf = dev["w13_sf"] if which == "w13" else dev["w2_sf"]
    fn = moe.grouped_gemm_w13 if which == "w13" else moe.grouped_gemm_w2
    fn(p, to_dev(a_q), None if a_sf is None else to_dev(a_sf), routing, w, w_sf, out)
    torch.cuda.synchronize()
    got = to_np(out)
    frac = check_gemm(got[vr], want[vr], gemm_abs(cfg, h, ref, which)[vr], f"{cfg.name} {which}")
    print(f"{cfg.name} {which}: {frac:.3%} of bf16 outputs differ from the oracle's")
    untouched = np.setdiff1d(np.arange(s["expert_rows"]), vr)
    assert np.all(got[untouched] == SENTINEL_BF16), "rows outside the experts' counts written"


@pytest.mark.parametrize("name", list(SMALL))
def test_gemm_w13_isolated(gpu, name):
    cfg, h, dev, ref = case(name)
    _gemm_isolated(cfg, h, dev, ref, "w13")


@pytest.mark.parametrize("name", list(SMALL))
def test_gemm_w2_isolated(gpu, name):
    cfg, h, dev, ref = case(name)
    _gemm_isolated(cfg, h, dev, ref, "w2")


@pytest.mark.parametrize("name", list(SMALL))
def test_act_requant_isolated(gpu, name):
    cfg, h, dev, ref = case(name)
    p = problem(cfg)
    s = moe.sizes(p)
    ue = O.act_e8m0(cfg)
    vr = valid_rows(cfg, ref)
    gu = np.full((s["expert_rows"], 2 * cfg.N), 0x7FC0, np.uint16)   # NaN outside
    gu[vr] = ref["gate_up"][vr]
    routing = oracle_routing(p, cfg, ref)
    if cfg.act_quant == "bf16":
        # unquantized: h rounded to bf16, within one bf16 unit of the oracle's
        # (fp32 exp / reciprocal vs fp64, then one rounding each)
        a2 = torch.full((s["expert_rows"], cfg.N), SENTINEL_BF16, dtype=torch.int16,
                        device="cuda").view(torch.bfloat16)
        moe.act_requant(p, to_dev(gu), routing, a2, None)
        torch.cuda.synchronize()
        got = to_np(a2)
        check_bf16_close(got[vr], ref["a2_q"][vr], f"{name} act bf16")
        untouched = np.setdiff1d(np.arange(s["expert_rows"]), vr)
        assert np.all(got[untouched] == SENTINEL_BF16)
        return
    a2_q = torch.full((s["expert_rows"], cfg.N), SENTINEL_U8, dtype=torch.uint8, device="cuda")
    a2_sf = (torch.zeros((s["expert_rows"], s["a2_sf_row"]), dtype=torch.uint8, device="cuda")
             if ue else torch.zeros((s["expert_rows"], s["a2_sf_row"]), dtype=torch.float32,
                                    device="cuda"))
    moe.act_requant(p, to_dev(gu), routing, a2_q, a2_sf)
    torch.cuda.synchronize()
    got_q, got_sf = to_np(a2_q), to_np(a2_sf)
    h32 = O.silu_mul_f32(ref["gate_up"][vr], cfg.N)
    grp = O.act_group(cfg)
    check_requant(got_q[vr], got_sf[vr], ref["a2_q"][vr], ref["a2_sf"][vr], h32, ue,
                  f"{name} act_requant", grp)
    if ue:
        G = cfg.N // grp
        assert np.all(got_sf[vr][:, G:] == 0), "pad bytes of the scale rows must be zero"
    untouched = np.setdiff1d(np.arange(s["expert_rows"]), vr)
    assert np.all(got_q[untouched] == SENTINEL_U8)


@pytest.mark.parametrize("tile_m", [16, 32, 64, 128, 160, 192, 256])
@pytest.mark.parametrize("name", list(SMALL))
def test_gemm_w13_act_fused_equals_chain(gpu, name, tile_m, monkeypatch):
    """The fused w13 + activation call against the two calls it replaces, on
    the oracle's staged inputs (rows outside the counts poisoned): a2 codes and
    scales bit-identical on every routed row, nothing written elsewhere.  The
    unfused pair is itself checked against the oracle above; the fused path
    additionally against the oracle's a2 through check_requant_chain."""
    monkeypatch.setenv("MOE_TILE_M", str(tile_m))
    if CASES[name].act_quant == "bf16" and tile_m > 128:
        pytest.skip("bf16 activation tiles are at most 128 rows (LDS)")
    if tile_m == 160 and not tile160_ok(CASES[name]):
        pytest.skip("160-row tiles: block scheme with per-128 fp8 activations only")
    _fused_equals_chain(name, tile_m)


def _fused_equals_chain(name, tile_m):
    cfg, h, dev, ref = case(name)
    p = problem(cfg)
    s = moe.sizes(p)
    assert s["tile_m"] == tile_m
    ue = O.act_e8m0(cfg)
    routing = oracle_routing(p, cfg, ref)
    vr = valid_rows(cfg, ref)
    arows = (np.arange(s["stage_rows"]) if cfg.layout != "batched" else vr)
    if cfg.act_quant == "bf16":
        rows = s["expert_rows"]
        a_q = to_dev(poisoned(ref["x_q"], arows, 0x7FC0))
        gate_up = torch.empty((rows, 2 * cfg.N), dtype=torch.bfloat16, device="cuda")
        moe.grouped_gemm_w13(p, a_q, None, routing, dev["w13"], dev["w13_sf"], gate_up)
        want = torch.full((rows, cfg.N), SENTINEL_BF16, dtype=torch.int16,
                          device="cuda").view(torch.bfloat16)
        moe.act_requant(p, gate_up, routing, want, None)
        got = torch.full((rows, cfg.N), SENTINEL_BF16, dtype=torch.int16,
                         device="cuda").view(torch.bfloat16)
        moe.grouped_gemm_w13_act(p, a_q, None, routing, dev["w13"], dev["w13_sf"], got, None)
        torch.cuda.synchronize()
        g, w = to_np(got), to_np(want)
        assert np.array_equal(g[vr], w[vr]), f"{name} tile {tile_m}: fused bf16 a2 differs"
        untouched = np.setdiff1d(np.arange(rows), vr)
        assert np.all(g[untouched] == SENTINEL_BF16), "fused call wrote rows outside the counts"
        check_bf16_act_chain(g[vr], ref["a2_q"][vr], ref["gate_up"][vr],
                             gemm_abs(cfg, h, ref, "w13")[vr], f"{name} fused tile {tile_m}")
        return
    a_q = to_dev(poisoned(ref["x_q"], arows, 0x7F))
    a_sf = O.pack_ue8m0_rows(ref["x_sf"]) if ue else ref["x_sf"]
    a_sf = to_dev(poisoned(a_sf, arows, sf_poison(ue)))
    rows, G = s["expert_rows"], cfg.N // O.act_group(cfg)
    sf_dtype = torch.uint8 if ue else torch.float32

    gate_up = torch.empty((rows, 2 * cfg.N), dtype=torch.bfloat16, device="cuda")
    moe.grouped_gemm_w13(p, a_q, a_sf, routing, dev["w13"], dev["w13_sf"], gate_up)
    want_q = torch.full((rows, cfg.N), SENTINEL_U8, dtype=torch.uint8, device="cuda")
    want_sf = torch.zeros((rows, s["a2_sf_row"]), dtype=sf_dtype, device="cuda")
    moe.act_requant(p, gate_up, routing, want_q, want_sf)

    got_q = torch.full((rows, cfg.N), SENTINEL_U8, dtype=torch.uint8, device="cuda")
    got_sf = torch.full((rows, s["a2_sf_row"]), SENTINEL_U8, dtype=torch.uint8,
                        device="cuda").view(sf_dtype) if ue else \
        torch.full((rows, s["a2_sf_row"]), float("nan"), dtype=torch.float32, device="cuda")
    moe.grouped_gemm_w13_act(p, a_q, a_sf, routing, dev["w13"], dev["w13_sf"], got_q, got_sf)
    torch.cuda.synchronize()
    gq, gs, wq, ws = to_np(got_q), to_np(got_sf), to_np(want_q), to_np(want_sf)
    assert np.array_equal(gq[vr], wq[vr]), f"{name} tile {tile_m}: fused a2 codes differ"
    if ue:
        assert np.array_equal(gs[vr], ws[vr]), f"{name} tile {tile_m}: fused exponents differ"
        assert np.all(gs[vr][:, G:] == 0), "pad bytes of the scale rows must be zero"
    else:
        assert np.array_equal(gs[vr].view(np.uint32), ws[vr].view(np.uint32)), \
            f"{name} tile {tile_m}: fused fp32 scales differ"
    untouched = np.setdiff1d(np.arange(rows), vr)
    assert np.all(gq[untouched] == SENTINEL_U8), "fused call wrote rows outside the counts"
    if ue:
        assert np.all(gs[untouched] == SENTINEL_U8)
    else:
        assert np.all(np.isnan(gs[untouched]))
    check_requant_chain(gq[vr], gs[vr], ref["a2_q"][vr], ref["a2_sf"][vr], ref["gate_up"][vr],
                        gemm_abs(cfg, h, ref, "w13")[vr], ue, f"{name} fused tile {tile_m}",
                        O.act_group(cfg))


@pytest.mark.parametrize("name", list(SMALL))
def test_topk_reduce_isolated(gpu, name):
    cfg, h, dev, ref = case(name)
    p = problem(cfg)
    s = moe.sizes(p)
    vr = valid_rows(cfg, ref)
    down = np.full((s["expert_rows"], cfg.K), 0x7FC0, np.uint16)     # NaN outside
    down[vr] = ref["down"][vr]
    out = torch.empty((cfg.T, cfg.K), dtype=torch.bfloat16, device="cuda")
    moe.topk_reduce(p, to_dev(down), to_dev(ref["slot_row"].astype(np.int32)),
                    to_dev(ref["weights"]), out)
    torch.cuda.synchronize()
    check_bf16_close(to_np(out), ref["out"], f"{name} reduce")


# ---------------------------------------------------------------------------
# the whole layer
# ---------------------------------------------------------------------------

def run_chain(cfg, dev):
    """moe_stage -> w13 -> act_requant -> w2 -> reduce through the separate
    entry points; returns every intermediate."""
    p, bufs = stage_on_gpu(cfg, dev)
    s = moe.sizes(p)
    ue = O.act_e8m0(cfg)
    gate_up = torch.full((s["expert_rows"], 2 * cfg.N), SENTINEL_BF16, dtype=torch.int16,
                         device="cuda").view(torch.bfloat16)
    moe.grouped_gemm_w13(p, bufs["x_q"], bufs["x_sf"], bufs, dev["w13"], dev["w13_sf"], gate_up)
    if cfg.act_quant == "bf16":
        a2_q = torch.full((s["expert_rows"], cfg.N), SENTINEL_BF16, dtype=torch.int16,
                          device="cuda").view(torch.bfloat16)
        a2_sf = None
    else:
        a2_q = torch.full((s["expert_rows"], cfg.N), SENTINEL_U8, dtype=torch.uint8,
                          device="cuda")
        a2_sf = torch.zeros((s["expert_rows"], s["a2_sf_row"]),
                            dtype=torch.uint8 if ue else torch.float32, device="cuda")
    moe.act_requant(p, gate_up, bufs, a2_q, a2_sf)
    down = torch.full((s["expert_rows"], cfg.K), SENTINEL_BF16, dtype=torch.int16,
                      device="cuda").view(torch.bfloat16)
    moe.grouped_gemm_w2(p, a2_q, a2_sf, bufs, dev["w2"], dev["w2_sf"], down)
    out = torch.empty((cfg.T, cfg.K), dtype=torch.bfloat16, device="cuda")
    moe.topk_reduce(p, down, bufs["slot_row"], bufs["topk_w"], out)
    torch.cuda.synchronize()
    return {"bufs": bufs, "gate_up": gate_up, "a2_q": a2_q, "a2_sf": a2_sf, "down": down,
            "out": out}


def run_forward(cfg, dev):
    p = problem(cfg)
    layer = moe.MoeLayer(p, dev["w13"], dev["w13_sf"], dev["w2"], dev["w2_sf"])
    if dev["eplb"] is not None:
        dev["eplb"]["expert_load"].zero_()
    out = layer(dev["hidden"], dev["topk_ids"], dev["topk_weights"], None, dev["is_padding"],
                dev["expert_num_tokens"], dev["eplb"])
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("name", list(SMALL))
def test_forward_end_to_end(gpu, name):
    _forward_end_to_end(name)


def _forward_end_to_end(name):
    cfg, h, dev, ref = case(name)
    ue = O.act_e8m0(cfg)
    chain = run_chain(cfg, dev)
    vr = valid_rows(cfg, ref)
    if cfg.act_quant == "bf16":
        frac = check_bf16_act_chain(to_np(chain["a2_q"])[vr], ref["a2_q"][vr],
                                    ref["gate_up"][vr], gemm_abs(cfg, h, ref, "w13")[vr],
                                    f"{name} a2 (chain)")
    else:
        frac = check_requant_chain(to_np(chain["a2_q"])[vr], to_np(chain["a2_sf"])[vr],
                                   ref["a2_q"][vr], ref["a2_sf"][vr], ref["gate_up"][vr],
                                   gemm_abs(cfg, h, ref, "w13")[vr], ue, f"{name} a2 (chain)",
                                   O.act_group(cfg))
    print(f"{name}: {frac:.3%} of a2 codes differ at the end of the GPU chain")
    check_output(to_np(chain["out"]), ref["out"], f"{name} chained output")
    out = run_forward(cfg, dev)
    check_output(to_np(out), ref["out"], f"{name} moe_forward output")
    # moe_forward runs the fused w13 + activation call, bit-identical to the
    # unfused pair of the chain: identical bits; and it is deterministic
    assert torch.equal(out.view(torch.int16), chain["out"].view(torch.int16))
    out2 = run_forward(cfg, dev)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    if cfg.eplb:
        assert np.array_equal(to_np(dev["eplb"]["expert_load"]), ref["load"])
    if cfg.pad_frac > 0:
        pad = h["is_padding"].astype(bool)
        assert np.all(to_np(out)[pad] == 0)


@pytest.mark.parametrize("tile_m", [16, 32, 64, 128, 160, 192, 256])
def test_every_tile_height(gpu, tile_m, monkeypatch):
    monkeypatch.setenv("MOE_TILE_M", str(tile_m))
    for name in ("ragged", "batched"):
        cfg, h, dev, ref = case(name)
        assert moe.sizes(problem(cfg))["tile_m"] == tile_m
        chain = run_chain(cfg, dev)
        vr = valid_rows(cfg, ref)
        check_gemm(to_np(chain["gate_up"])[vr], ref["gate_up"][vr],
                   gemm_abs(cfg, h, ref, "w13")[vr], f"{name} gate_up tile_m={tile_m}")
        check_output(to_np(chain["out"]), ref["out"], f"{name} out tile_m={tile_m}")


# ---------------------------------------------------------------------------
# mid-size configs (9-16 k-steps per GEMM) at three tile heights
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name,tile_m", MID_CASES)
def test_mid_stage_route_and_act(gpu, name, tile_m, monkeypatch):
    """Staging and routing bit-exact (the schedule for this tile height), and
    the activation step in isolation on the oracle's gate_up."""
    monkeypatch.setenv("MOE_TILE_M", str(tile_m))
    assert moe.sizes(problem(MID[name]))["tile_m"] == tile_m
    test_stage_and_route_bit_exact(gpu, name)
    if tile_m == MID_TILES[0]:
        test_act_requant_isolated(gpu, name)


@pytest.mark.parametrize("name,tile_m", MID_CASES)
def test_mid_gemms_isolated(gpu, name, tile_m, monkeypatch):
    """Both GEMMs on the oracle's inputs, every routed row against the
    oracle, nothing written outside the experts' rows."""
    monkeypatch.setenv("MOE_TILE_M", str(tile_m))
    cfg, h, dev, ref = case(name)
    assert moe.sizes(problem(cfg))["tile_m"] == tile_m
    _gemm_isolated(cfg, h, dev, ref, "w13")
    _gemm_isolated(cfg, h, dev, ref, "w2")


@pytest.mark.parametrize("name,tile_m", MID_CASES)
def test_mid_fused_equals_chain(gpu, name, tile_m, monkeypatch):
    monkeypatch.setenv("MOE_TILE_M", str(tile_m))
    _fused_equals_chain(name, tile_m)


@pytest.mark.parametrize("name,tile_m", MID_CASES)
def test_mid_forward_end_to_end(gpu, name, tile_m, monkeypatch):
    monkeypatch.setenv("MOE_TILE_M", str(tile_m))
    _forward_end_to_end(name)


@pytest.mark.parametrize("name", ["mid_ue8m0", "mid_fp32", "mid_bf16", "mid_batched",
                                  "split_ue8m0"])
def test_k_rotation_forced(gpu, name, monkeypatch):
    """The GEMMs with the k-step rotation forced on (by default it runs only
    where the weight rows are a multiple of 4 KB, which these configs' rows
    are not): both GEMMs on the oracle's inputs, every routed row; the fused
    w13 equal to the unfused pair bit for bit at two tile heights (they share
    the rotation key); the forward output within its bound."""
    monkeypatch.setenv("MOE_KROT", "1")
    cfg, h, dev, ref = case(name)
    _gemm_isolated(cfg, h, dev, ref, "w13")
    _gemm_isolated(cfg, h, dev, ref, "w2")
    for t in (16, 128):
        monkeypatch.setenv("MOE_TILE_M", str(t))
        _fused_equals_chain(name, t)
    monkeypatch.delenv("MOE_TILE_M")
    check_output(to_np(run_forward(cfg, dev)), ref["out"], f"{name} rotated output")


@pytest.mark.parametrize("ksplit", [1, 2, 4])
@pytest.mark.parametrize("name", ["mid_fp32", "mid_mxfp4", "split_ue8m0", "split_batched"])
def test_w2_split_k(gpu, name, ksplit, monkeypatch):
    """w2 with its reduction forced into 1, 2 or 4 ranges (MOE_KSPLIT): every
    routed row within the GEMM bound of the oracle, nothing written outside
    the experts' rows, the same bits on a second call (the partials are
    added in split order, whichever split finishes last), and the whole
    layer through moe_forward within the output bound."""
    monkeypatch.setenv("MOE_KSPLIT", str(ksplit))
    cfg, h, dev, ref = case(name)
    p = problem(cfg)
    expect = ksplit if cfg.N // 128 >= 4 * ksplit else max(1, ksplit // 2)
    assert (moe.w2_workspace_size(p) > 0) == (expect > 1)
    _gemm_isolated(cfg, h, dev, ref, "w2")
    s = moe.sizes(p)
    vr = valid_rows(cfg, ref)
    ue = O.act_e8m0(cfg)
    a_q = to_dev(ref["a2_q"])
    a_sf = None if ref["a2_sf"] is None else to_dev(
        O.pack_ue8m0_rows(ref["a2_sf"]) if ue and O.act_group(cfg) == 128 else ref["a2_sf"])
    routing = oracle_routing(p, cfg, ref)
    ws = moe.alloc_w2_workspace(p)
    outs = []
    for _ in range(2):
        down = torch.full((s["expert_rows"], cfg.K), SENTINEL_BF16, dtype=torch.int16,
                          device="cuda").view(torch.bfloat16)
        moe.grouped_gemm_w2(p, a_q, a_sf, routing, dev["w2"], dev["w2_sf"], down, ws)
        torch.cuda.synchronize()
        outs.append(to_np(down)[vr])
    assert np.array_equal(outs[0], outs[1]), f"{name} split {ksplit}: not deterministic"
    check_output(to_np(run_forward(cfg, dev)), ref["out"], f"{name} split {ksplit} output")


@pytest.mark.parametrize("name,tile_m", [("mid_ue8m0", "128"), ("tall_ue8m0", None),
                                         ("tall_fp32", None), ("tall_batched", None)])
def test_w2_paired_tiles(gpu, name, tile_m, monkeypatch):
    """w2 at 128-row tiles takes two neighbouring 256-column n-tiles per
    block by default (MOE_PAIR): on the oracle's a2 every routed row is
    within the GEMM bound, and the bits equal those of one n-tile per block,
    for the GEMM alone and through moe_forward."""
    if tile_m is None:
        monkeypatch.delenv("MOE_TILE_M", raising=False)
    else:
        monkeypatch.setenv("MOE_TILE_M", tile_m)
    monkeypatch.delenv("MOE_TALL", raising=False)
    cfg, h, dev, ref = case(name)
    p = problem(cfg)
    s = moe.sizes(p)
    assert s["tile_m"] == 128 and cfg.K % 512 == 0 and cfg.act_quant in ("ue8m0", "fp32")
    ue = O.act_e8m0(cfg)
    vr = valid_rows(cfg, ref)
    a_q = to_dev(ref["a2_q"])
    a_sf = to_dev(O.pack_ue8m0_rows(ref["a2_sf"]) if ue else ref["a2_sf"])
    routing = oracle_routing(p, cfg, ref)
    got = {}
    for v in ("1", "0"):
        monkeypatch.setenv("MOE_PAIR", v)
        down = torch.full((s["expert_rows"], cfg.K), SENTINEL_BF16, dtype=torch.int16,
                          device="cuda").view(torch.bfloat16)
        moe.grouped_gemm_w2(p, a_q, a_sf, routing, dev["w2"], dev["w2_sf"], down)
        torch.cuda.synchronize()
        got[v] = (to_np(down), to_np(run_forward(cfg, dev)))
    untouched = np.setdiff1d(np.arange(s["expert_rows"]), vr)
    assert np.all(got["1"][0][untouched] == SENTINEL_BF16), "paired w2 wrote rows outside"
    check_gemm(got["1"][0][vr], ref["down"][vr], gemm_abs(cfg, h, ref, "w2")[vr],
               f"{name} paired w2")
    assert np.array_equal(got["1"][0], got["0"][0]), f"{name}: paired w2 bits differ"
    assert np.array_equal(got["1"][1], got["0"][1]), f"{name}: paired layer bits differ"


# ---------------------------------------------------------------------------
# the second (tall) tile list at the default tile height
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", list(TALL))
def test_tall_list(gpu, name, monkeypatch):
    """Experts above 128 rows in 256-row tiles of a second list, whose GEMM
    launches run on a second stream alongside the main list's (moe_forward,
    the GEMM entry points) or after them (moe_forward_static).  The routing
    writes both lists bit-exact; the chain and moe_forward match the oracle;
    the bits equal those with one list (MOE_TALL=0) and moe_forward_static's."""
    monkeypatch.delenv("MOE_TILE_M", raising=False)
    monkeypatch.delenv("MOE_TALL", raising=False)
    cfg, h, dev, ref = case(name)
    s = moe.sizes(problem(cfg))
    assert s["tile_m"] == 128 and s["tall_tile_m"] == 256
    counts = ref["counts"] if cfg.layout != "batched" else np.minimum(ref["counts"],
                                                                      cfg.max_tokens)
    assert (counts > 128).any() and ((counts > 0) & (counts <= 128)).any()
    test_stage_and_route_bit_exact(gpu, name)
    _fused_equals_chain(name, 128)
    _forward_end_to_end(name)
    out = run_forward(cfg, dev)
    monkeypatch.setenv("MOE_TALL", "0")
    assert moe.sizes(problem(cfg))["tall_tile_m"] == 0
    one = run_forward(cfg, dev)
    monkeypatch.delenv("MOE_TALL")
    assert torch.equal(out.view(torch.int16), one.view(torch.int16)), f"{name}: one list differs"
    p = problem(cfg)
    st = torch.empty_like(out)
    moe.forward_static(p, dev["hidden"], dev["topk_ids"], dev["topk_weights"], dev["w13"],
                       dev["w13_sf"], dev["w2"], dev["w2_sf"], st, is_padding=dev["is_padding"],
                       expert_num_tokens=dev["expert_num_tokens"])
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), st.view(torch.int16)), f"{name}: static differs"


TALL_INDEXED = moe_synth.custom(name="tall_indexed", T=256, E=8, top_k=3, K=1024, N=1024,
                                seed=56, routing="zipf", zipf_s=1.1, pad_frac=0.05,
                                layout="indexed")


def test_w2_paired_tiles_indexed(gpu, monkeypatch):
    """The indexed layout's moe_forward, whose w2 takes two 256-column
    n-tiles per 128-row block by default (MOE_PAIR): the output within the
    bound, and the same bits with the pairs off."""
    monkeypatch.delenv("MOE_TILE_M", raising=False)
    monkeypatch.delenv("MOE_TALL", raising=False)
    cfg = TALL_INDEXED
    CASES.setdefault(cfg.name, cfg)
    _, h, dev, ref = case(cfg.name)
    assert moe.sizes(problem(cfg))["tile_m"] == 128 and cfg.K % 512 == 0
    outs = {}
    for v in ("1", "0"):
        monkeypatch.setenv("MOE_PAIR", v)
        outs[v] = to_np(run_forward(cfg, dev))
    check_output(outs["1"], ref["out"], "tall_indexed paired w2")
    assert np.array_equal(outs["1"], outs["0"]), "indexed layer: paired w2 bits differ"


def test_tall_list_indexed(gpu, monkeypatch):
    """The indexed layout with the tall list: 256-row tiles cover 256
    positions of a heavy expert's segment of the 128-block map (never the
    next expert's).  moe_forward matches the oracle, equals the one-list
    run (MOE_TALL=0) and moe_forward_static bit for bit."""
    monkeypatch.delenv("MOE_TILE_M", raising=False)
    monkeypatch.delenv("MOE_TALL", raising=False)
    cfg = TALL_INDEXED
    CASES.setdefault(cfg.name, cfg)
    _, h, dev, ref = case(cfg.name)
    p = problem(cfg)
    s = moe.sizes(p)
    assert p.layout == moe.LAYOUT_INDEXED and s["tile_m"] == 128 and s["tall_tile_m"] == 256
    counts = ref["counts"]
    assert (counts > 128).any() and ((counts > 0) & (counts <= 128)).any()
    out = run_forward(cfg, dev)
    check_output(to_np(out), ref["out"], "tall_indexed moe_forward output")
    monkeypatch.setenv("MOE_TALL", "0")
    one = run_forward(cfg, dev)
    monkeypatch.delenv("MOE_TALL")
    assert torch.equal(out.view(torch.int16), one.view(torch.int16)), "one list differs"
    st = torch.empty_like(out)
    moe.forward_static(p, dev["hidden"], dev["topk_ids"], dev["topk_weights"], dev["w13"],
                       dev["w13_sf"], dev["w2"], dev["w2_sf"], st, is_padding=dev["is_padding"],
                       expert_num_tokens=dev["expert_num_tokens"])
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), st.view(torch.int16)), "static differs"


# ---------------------------------------------------------------------------
# degenerate inputs
# ---------------------------------------------------------------------------

def _layer_out(cfg, inp):
    dev = {k: (v.to("cuda") if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    return to_np(run_forward(cfg, dev))


def test_empty_batch_noop(gpu):
    p = moe.Problem(0, 256, 512, 4, 2)
    out = torch.full((1, 256), 3, dtype=torch.bfloat16, device="cuda")
    moe.forward(p, out, torch.zeros((1, 2), dtype=torch.int32, device="cuda"),
                torch.zeros((1, 2), device="cuda"), out, out, out, out, out,
                torch.empty(256, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    assert torch.all(out == 3)


def test_all_tokens_padding_or_unrouted(gpu):
    cfg = moe_synth.custom(name="pad_all", T=40, E=3, top_k=2, K=256, N=256, seed=31)
    inp = moe_synth.make_inputs(cfg, "cpu")
    inp["is_padding"] = torch.ones(cfg.T, dtype=torch.uint8)
    assert np.all(_layer_out(cfg, inp) == 0)
    inp["is_padding"] = None
    ids = inp["topk_ids"].clone()
    ids[:, 0] = -1
    ids[:, 1] = cfg.E + 5                 # out of range: unrouted, not an error
    inp["topk_ids"] = ids
    assert np.all(_layer_out(cfg, inp) == 0)


def test_single_token_and_invalid_ids(gpu):
    cfg = moe_synth.custom(name="one", T=1, E=6, top_k=3, K=256, N=256, seed=32)
    inp = moe_synth.make_inputs(cfg, "cpu")
    h = O.host_inputs(inp)
    check_output(_layer_out(cfg, inp), O.forward(h)["out"], "single token")
    cfg2 = moe_synth.custom(name="invalid", T=64, E=6, top_k=3, K=256, N=256, seed=33)
    inp2 = moe_synth.make_inputs(cfg2, "cpu")
    ids = inp2["topk_ids"].clone()
    ids[::3, 1] = -7
    ids[1::5, 2] = 99
    inp2["topk_ids"] = ids
    h2 = O.host_inputs(inp2)
    check_output(_layer_out(cfg2, inp2), O.forward(h2)["out"], "invalid ids")


def test_batched_empty_slabs_and_garbage(gpu):
    cfg = moe_synth.custom(name="slabs", T=30, E=6, top_k=1, K=256, N=256, seed=34,
                           layout="batched", max_tokens=48)
    inp = moe_synth.make_inputs(cfg, "cpu")
    # route every token to experts 1 and 4 only: the other slabs are empty
    inp["topk_ids"] = torch.where(torch.arange(cfg.T)[:, None] % 2 == 0,
                                  torch.tensor(1), torch.tensor(4)).to(torch.int32)
    inp.update(moe_synth._stage_batched(cfg, inp["tokens"], inp["topk_ids"], "cpu"))
    h = O.host_inputs(inp)
    check_output(_layer_out(cfg, inp), O.forward(h)["out"], "batched with empty slabs")


@pytest.mark.parametrize("indexed", [False, True])
def test_reduce_many_tokens(gpu, indexed):
    """70 000 tokens, past a 65 535 grid-y limit: the reduce puts tokens on
    its one-dimensional grid.  moe_topk_reduce (slot rows, 5 % unrouted) and
    moe_fused_mul_sum ((token, slot) rows, invalid ids unrouted) against the
    oracle's reduce, every token."""
    T, k, K, E = 70000, 2, 384, 4
    rng = np.random.default_rng(61)
    M = T * k
    down = O.bf16_round(rng.standard_normal((M, K)))
    w = rng.random((T, k)).astype(np.float32)
    p = moe.Problem(T, K, 256, E, k)
    out = torch.empty((T, K), dtype=torch.bfloat16, device="cuda")
    if indexed:
        ids = rng.integers(0, E, (T, k)).astype(np.int64)
        ids[rng.random((T, k)) < 0.05] = -1
        slot_row = np.where(ids >= 0, np.arange(M).reshape(T, k), -1)
        moe.fused_mul_sum(p, to_dev(down), to_dev(ids), to_dev(w), out)
    else:
        slot_row = rng.permutation(M).reshape(T, k).astype(np.int32)
        slot_row[rng.random((T, k)) < 0.05] = -1
        moe.topk_reduce(p, to_dev(down), to_dev(slot_row), to_dev(w), out)
    torch.cuda.synchronize()
    check_bf16_close(to_np(out), O.topk_reduce(down, slot_row, w), f"reduce of {T} tokens")


def test_expert_count_multiple_of_tile(gpu, monkeypatch):
    """Counts landing exactly on tile boundaries (no ragged tail)."""
    monkeypatch.setenv("MOE_TILE_M", "32")
    cfg = moe_synth.custom(name="exact", T=128, E=4, top_k=1, K=256, N=256, seed=35)
    inp = moe_synth.make_inputs(cfg, "cpu")
    inp["topk_ids"] = (torch.arange(cfg.T) // 32).to(torch.int32)[:, None].contiguous()
    h = O.host_inputs(inp)
    check_output(_layer_out(cfg, inp), O.forward(h)["out"], "exact tiles")
