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


def _param_counts():
    """Parameter count of every function include/moe_fp8.h declares."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    out = {}
    for m in re.finditer(r"\b(moe_\w+)\s*\(([^)]*)\)\s*;", text):
        params = m.group(2).strip()
        out[m.group(1)] = 0 if params in ("", "void") else params.count(",") + 1
    return out


def test_binding_signatures_match_the_header(lib):
    # every export has a ctypes signature of the header's arity (a missing
    # one makes ctypes truncate pointers to 32-bit ints)
    counts = _param_counts()
    assert set(counts) == set(moe.EXPORTS)
    for name, n in counts.items():
        argtypes = getattr(lib, name).argtypes
        assert argtypes is not None, name
        assert len(argtypes) == n, (name, len(argtypes), n)


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
    for name, cfg in moe_synth.MX_CONFIGS.items():
        p = moe.Problem.from_config(cfg)
        s = moe.sizes(p)
        assert s["x_sf_row"] == cfg.K // 32 and s["a2_sf_row"] == cfg.N // 32
        assert s["tile_m"] in (16, 32, 64, 128, 160, 192, 256)
        ws = moe.workspace_size(p)
        # staged x_q, the w2 input a2 and the bf16 down projection coexist
        # (the fused w13 call reads x_q while it writes a2)
        x_q = s["stage_rows"] * cfg.K
        a2 = s["expert_rows"] * cfg.N
        down = s["expert_rows"] * cfg.K * 2
        assert ws >= x_q + a2 + down


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


def test_scheme_pairs(lib):
    # (weight, activation) pairs of the experts' supported-scheme list that
    # this library implements; the rest are rejected before any launch
    base = dict(num_tokens=16, hidden=256, intermediate=512, num_experts=4, top_k=2)
    for wq in (moe.W_MXFP8, moe.W_MXFP4):
        s = moe.sizes(moe.Problem(**base, act_quant=moe.Q_MXFP8, weight_quant=wq))
        assert s["x_sf_row"] == 256 // 32 and s["a2_sf_row"] == 512 // 32
    for act, wq, status in [(moe.Q_FP8_UE8M0, moe.W_MXFP8, -2), (moe.Q_FP8_F32, moe.W_MXFP8, -2),
                            (moe.Q_MXFP8, moe.W_FP8_BLOCK128, -2), (moe.Q_FP8_UE8M0, moe.W_MXFP4, -2),
                            (moe.Q_MXFP8, 7, -1), (9, moe.W_MXFP8, -1)]:
        with pytest.raises(moe.MoeError) as ei:
            moe.sizes(moe.Problem(**base, act_quant=act, weight_quant=wq))
        assert ei.value.status == status, (act, wq)


def test_large_token_counts(lib):
    """Token counts far past 65 535 (a grid-y limit) are valid: the reduce
    puts tokens on its one-dimensional grid.  A count whose staged
    activations would pass the 3.5 GiB buffer limit (32-bit buffer offsets)
    is rejected by every call before anything is enqueued -- here
    moe_topk_reduce and moe_forward with fake pointers, which a launch would
    fault on."""
    assert moe.sizes(moe.Problem(1 << 20, 2048, 512, 4, 1))["slots"] == 1 << 20
    big = moe.Problem((1 << 21) + 8, 2048, 512, 4, 1)
    with pytest.raises(moe.MoeError) as ei:
        moe.sizes(big)
    assert ei.value.status == -2 and "3.5 GiB" in lib.moe_last_error().decode()
    V = _fake()
    st = lib.moe_topk_reduce(ctypes.byref(big.c()), V, V, V, V, None)
    assert st == -2 and "3.5 GiB" in lib.moe_last_error().decode()
    st = lib.moe_forward(ctypes.byref(big.c()), V, None, V, V, None, None, V, V, V, V, V, V,
                         1 << 62, None)
    assert st == -2 and "3.5 GiB" in lib.moe_last_error().decode()


def test_static_forward_rejects_oversized_problems(lib):
    """moe_forward_static checks the problem's workspace against its static
    array before it touches the device (so this runs without a GPU)."""
    p = moe.Problem.from_config(moe_synth.CONFIGS["dsv3_prefill"])
    assert moe.workspace_size(p) > moe.STATIC_SCRATCH_BYTES
    V = _fake()
    st = lib.moe_forward_static(ctypes.byref(p.c()), V, None, V, V, None, None, V, V, V, V, V,
                                None)
    assert st == -3 and "static scratch" in lib.moe_last_error().decode()
    # a DeepSeek-V3-shaped decode batch fits
    assert moe.workspace_size(moe.Problem.from_config(moe_synth.CONFIGS["dsv3_decode"])) < \
        moe.STATIC_SCRATCH_BYTES // 4
    hdr = open(HEADER).read()
    assert f"MOE_STATIC_SCRATCH_BYTES ({moe.STATIC_SCRATCH_BYTES >> 20}u << 20)" in hdr


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
    # bf16 activations pair only with block fp8 weights
    pbm = moe.Problem(16, 256, 512, 4, 2, act_quant=moe.Q_BF16, weight_quant=moe.W_MXFP8).c()
    st = lib.moe_forward(ctypes.byref(pbm), V, None, V, V, None, None, V, V, V, V, V, V,
                         1 << 30, None)
    assert st == -2
    pb = moe.Problem(16, 256, 512, 4, 2, act_quant=moe.Q_BF16).c()
    # batched layout without expert_num_tokens
    pbt = moe.Problem(16, 256, 512, 4, 2, layout=moe.LAYOUT_BATCHED,
                      max_tokens_per_expert=8).c()
    st = lib.moe_forward(ctypes.byref(pbt), V, None, V, V, None, None, V, V, V, V, V, V,
                         1 << 30, None)
    assert st == -1 and "expert_num_tokens" in lib.moe_last_error().decode()
    # EPLB remapping needs the contiguous routing: batched slabs are already
    # per physical expert
    e = moe._Eplb(V, 1, V, 2, None, None, None)
    st = lib.moe_forward(ctypes.byref(pbt), V, V, V, V, None, ctypes.byref(e), V, V, V, V, V, V,
                         1 << 30, None)
    assert st == -2 and "EPLB" in lib.moe_last_error().decode()
    st = lib.moe_forward(ctypes.byref(p), V, None, V, V, None, ctypes.byref(e), V, V, V, V, V, V,
                         16, None)
    assert st == -3, "the contiguous layout accepts eplb (then fails on the small workspace)"
    # x_sf given for bf16 staging
    r = moe._Routing(V, V, V, V, V)
    st = lib.moe_stage(ctypes.byref(pb), V, None, V, V, None, None, V, V, V, V,
                       ctypes.byref(r), V, 1 << 20, None)
    assert st == -1 and "x_sf" in lib.moe_last_error().decode()
    # the fused w13 + activation call needs its fp8 outputs
    st = lib.moe_grouped_gemm_w13_act(ctypes.byref(p), V, V, ctypes.byref(r), V, V, None, V,
                                      None)
    assert st == -1 and "a2_q" in lib.moe_last_error().decode()
    st = lib.moe_grouped_gemm_w13_act(ctypes.byref(p), V, V, ctypes.byref(r), V, V, V,
                                      _fake((1 << 20) + 2), None)
    assert st == -1 and "a2_sf" in lib.moe_last_error().decode()
    # bf16 activations carry no scales
    st = lib.moe_grouped_gemm_w13_act(ctypes.byref(pb), V, V, ctypes.byref(r), V, V, V, None,
                                      None)
    assert st == -1 and "a_sf" in lib.moe_last_error().decode()
    st = lib.moe_grouped_gemm_w13_act(ctypes.byref(pb), V, None, ctypes.byref(r), V, V, V, V,
                                      None)
    assert st == -1 and "a2_sf" in lib.moe_last_error().decode()


def test_empty_batch_is_a_noop(lib):
    p = moe.Problem(0, 256, 512, 4, 2).c()
    assert lib.moe_forward(ctypes.byref(p), None, None, None, None, None, None, None, None,
                           None, None, None, None, 0, None) == 0
    assert lib.moe_stage(ctypes.byref(p), None, None, None, None, None, None, None, None, None,
                         None, None, None, 0, None) == 0
    assert lib.moe_last_error().decode() == ""


def test_tall_list_sizes(lib, monkeypatch):
    """The second tile list (experts above 128 rows in 256-row tiles): where
    it applies, where it does not, and its place in the tile-list buffer."""
    monkeypatch.delenv("MOE_TILE_M", raising=False)
    monkeypatch.delenv("MOE_TALL", raising=False)
    for name, cfg in {**moe_synth.CONFIGS, **moe_synth.MX_CONFIGS,
                      **moe_synth.INDEXED_CONFIGS}.items():
        p = moe.Problem.from_config(cfg)
        s = moe.sizes(p)
        E, slots = cfg.E, cfg.T * cfg.top_k
        tall = (s["tile_m"] == 128 and cfg.act_quant != "bf16"
                and moe.w2_workspace_size(p) == 0)
        assert (s["tall_tile_m"] == 256) == tall and s["tall_tile_m"] in (0, 256), name
        main = 4 + 9 * s["max_tiles"] + E + 1
        if not tall:
            assert s["tile_list"] == main and s["tall_list_offset"] == 0, name
            continue
        off = s["tall_list_offset"]
        assert off % 4 == 0 and main <= off < main + 4, name
        cap = (E * -(-cfg.max_tokens // 256) if cfg.layout == "batched"
               else -(-slots // 256) + E)
        assert s["max_tiles_tall"] == cap, name
        assert s["tile_list"] == off + 4 + 9 * cap + E + 1, name
    # the DeepSeek-V3-shaped prefill batch has one; MOE_TALL=0 or a forced
    # tile height turns it off, MOE_TALL=1 on again
    p = moe.Problem.from_config(moe_synth.ALL_CONFIGS["dsv3_prefill"])
    assert moe.sizes(p)["tall_tile_m"] == 256
    monkeypatch.setenv("MOE_TALL", "0")
    assert moe.sizes(p)["tall_tile_m"] == 0
    monkeypatch.delenv("MOE_TALL")
    monkeypatch.setenv("MOE_TILE_M", "128")
    assert moe.sizes(p)["tall_tile_m"] == 0
    monkeypatch.setenv("MOE_TALL", "1")
    assert moe.sizes(p)["tall_tile_m"] == 256
    monkeypatch.setenv("MOE_TILE_M", "64")
    assert moe.sizes(p)["tall_tile_m"] == 0


def test_tile_height_160(lib, monkeypatch):
    """The 8-expert, 128-rows-per-expert batch with a split w2 takes 160-row
    tiles (one per expert, a 3-slot ring) in the block scheme, 192-row ones
    where 160 cannot run (MX scales, a reduction past the weight-scale
    panel); a forced MOE_TILE_M=160 is ignored there."""
    monkeypatch.delenv("MOE_TILE_M", raising=False)
    cfg = moe_synth.ALL_CONFIGS["mixtral"]
    p = moe.Problem.from_config(cfg)
    s = moe.sizes(p)
    assert s["tile_m"] == 160 and s["tall_tile_m"] == 0
    assert s["max_tiles"] == cfg.E * -(-cfg.max_tokens // 160)
    kw = dict(layout=moe.LAYOUT_BATCHED, max_tokens_per_expert=256)
    mx = moe.Problem(512, 4096, 14336, 8, 2, act_quant=moe.Q_MXFP8, weight_quant=moe.W_MXFP8,
                     **kw)
    assert moe.sizes(mx)["tile_m"] == 192
    long_k = moe.Problem(512, 24576 + 128, 14336, 8, 2, **kw)
    assert moe.sizes(long_k)["tile_m"] == 192
    # more rows per expert than a 160-row tile holds comfortably
    assert moe.sizes(moe.Problem(640, 4096, 14336, 8, 2, **kw))["tile_m"] == 192
    monkeypatch.setenv("MOE_TILE_M", "160")
    assert moe.sizes(moe.Problem(64, 4096, 1024, 8, 2))["tile_m"] == 160
    assert moe.sizes(mx)["tile_m"] == 192


def test_indexed_sizes(lib):
    # the indexed layout: sorted_ids has the padded capacity, a2 and down T*k rows
    for name, cfg in moe_synth.INDEXED_CONFIGS.items():
        p = moe.Problem.from_config(cfg)
        assert p.layout == moe.LAYOUT_INDEXED
        s = moe.sizes(p)
        bm, slots = s["tile_m"], cfg.T * cfg.top_k
        cap = (slots + min(cfg.E, slots) * (bm - 1)) // bm * bm
        assert s["padded_rows"] == cap and s["blocks"] == cap // bm
        assert s["expert_rows"] == slots
        assert moe.align_capacity(p, bm) == (cap, cap // bm)
        ws = moe.workspace_size(p)
        # a2 and down in (token, slot) order, plus the block map
        assert ws >= s["stage_rows"] * cfg.K + slots * cfg.N + slots * cfg.K * 2 + cap * 4


@pytest.mark.parametrize("T,E,k,bs,seed", [(1, 4, 1, 16, 0), (37, 8, 3, 16, 1),
                                           (300, 64, 8, 64, 2), (50, 256, 8, 256, 3),
                                           (5, 1024, 2, 128, 4)])
def test_align_capacity_bounds_the_padded_total(lib, T, E, k, bs, seed):
    # the capacity the library reports holds the oracle's padded layout for
    # any routing, including the worst case (every expert one slot)
    import numpy as np
    from oracle import moe_oracle as O
    rng = np.random.default_rng(seed)
    p = moe.Problem(T, 256, 512, E, k)
    cap, blocks = moe.align_capacity(p, bs)
    ids = np.stack([rng.permutation(E)[:k] if k <= E else rng.integers(0, E, k)
                    for _ in range(T)])
    worst = (np.arange(T * k) % E).reshape(T, k)
    for routing in (ids, worst):
        sorted_ids, expert_ids, P = O.align_block_size(routing, E, bs)
        assert P <= cap and len(expert_ids) <= blocks


def test_indexed_validation(lib):
    V = _fake()
    base = dict(num_tokens=16, hidden=256, intermediate=512, num_experts=4, top_k=2)
    p = moe.Problem(**base)
    for bs, status in [(16, 0), (256, 0), (48, -2), (0, -2), (512, -2)]:
        if status:
            with pytest.raises(moe.MoeError) as ei:
                moe.align_capacity(p, bs)
            assert ei.value.status == status
        else:
            moe.align_capacity(p, bs)
    # bf16 activations: blocks up to 128 rows
    pb = moe.Problem(**base, act_quant=moe.Q_BF16)
    moe.align_capacity(pb, 128)
    with pytest.raises(moe.MoeError):
        moe.align_capacity(pb, 256)
    # 160-row blocks: per-128 fp8 activations with block-scaled weights, and
    # reductions the 160-row tiles' weight-scale panel holds (192 k-steps)
    moe.align_capacity(p, 160)
    moe.align_capacity(moe.Problem(**base, act_quant=moe.Q_FP8_F32), 160)
    for bad in (pb, moe.Problem(**base, act_quant=moe.Q_MXFP8, weight_quant=moe.W_MXFP8),
                moe.Problem(16, 24576 + 128, 512, 4, 2)):
        with pytest.raises(moe.MoeError):
            moe.align_capacity(bad, 160)
    c = p.c()
    # batched routing has no block map
    pbat = moe.Problem(**base, layout=moe.LAYOUT_BATCHED, max_tokens_per_expert=8).c()
    st = lib.moe_align_block_size(ctypes.byref(pbat), V, None, 16, V, V, V, None)
    assert st == -2
    # a missing block-map pointer is caught before any launch
    st = lib.moe_grouped_gemm_w13_act_indexed(ctypes.byref(c), V, V, None, V, V, 16, V, V, V,
                                              V, None)
    assert st == -1 and "sorted_ids" in lib.moe_last_error().decode()
    st = lib.moe_grouped_gemm_w2_indexed(ctypes.byref(c), V, V, V, V, None, 16, V, V, V, None,
                                         0, None)
    assert st == -1 and "num_tokens_padded" in lib.moe_last_error().decode()
    st = lib.moe_grouped_gemm_w2_indexed(ctypes.byref(c), V, V, V, V, V, 24, V, V, V, None,
                                         0, None)
    assert st == -2
    st = lib.moe_fused_mul_sum(ctypes.byref(c), V, _fake((1 << 20) + 4), V, V, None)
    assert st == -1 and "topk_idx" in lib.moe_last_error().decode()
    st = lib.moe_align_block_size(ctypes.byref(c), V, None, 16, V, V, V, None)
    assert st == -1 and "routing" in lib.moe_last_error().decode()


def test_activation_validation_and_workspace(lib):
    base = dict(num_tokens=16, hidden=256, intermediate=512, num_experts=4, top_k=2)
    with pytest.raises(moe.MoeError) as ei:
        moe.sizes(moe.Problem(**base, activation=9))
    assert ei.value.status == -1
    # the clamp limit: finite and >= 0, and only for SiLU / SWIGLUOAI / SWIGLUSTEP
    for act in (0, 7, 8):
        moe.sizes(moe.Problem(**base, activation=act, act_limit=2.5))
    for limit, status in [(-1.0, -1), (float("inf"), -1), (float("nan"), -1)]:
        with pytest.raises(moe.MoeError) as ei:
            moe.sizes(moe.Problem(**base, activation=7, act_limit=limit))
        assert ei.value.status == status, limit
    for act in (1, 2, 3, 6):
        with pytest.raises(moe.MoeError) as ei:
            moe.sizes(moe.Problem(**base, activation=act, act_limit=1.0))
        assert ei.value.status == -2, act
    # the clamped SwiGLU forms are gated: w13 has 2N rows, like SiLU
    ws_silu = moe.workspace_size(moe.Problem(**base))
    assert moe.workspace_size(moe.Problem(**base, activation=7)) == ws_silu
    assert moe.workspace_size(moe.Problem(**base, activation=8, act_limit=1.0)) == ws_silu
    # _no_mul activations keep a gate_up region (T*k rows of N bf16) in the
    # forward workspace; gated ones do not
    ws_silu = moe.workspace_size(moe.Problem(**base))
    ws_gelu = moe.workspace_size(moe.Problem(**base, activation=1))
    ws_relu2 = moe.workspace_size(moe.Problem(**base, activation=6))
    assert ws_silu == ws_gelu
    assert ws_relu2 >= ws_silu + 16 * 2 * 512 * 2
    # the fused w13 call has no up half to pair for _no_mul activations: it is
    # refused before anything else is looked at
    V = _fake()
    for act, status in [(3, -2), (4, -2), (5, -2), (6, -2)]:
        c = moe.Problem(**base, activation=act).c()
        st = lib.moe_grouped_gemm_w13_act(ctypes.byref(c), V, V, None, V, V, V, V, None)
        assert st == status, act
        st = lib.moe_grouped_gemm_w13_act_indexed(ctypes.byref(c), V, V, V, V, V, 16, V, V, V,
                                                  V, None)
        assert st == status, act
