"""Batch invariance of the layer on the GPU: a token's output bits do not
depend on the batch it runs in ("vllm.model_executor.layers.fused_moe.
experts.fused_humming_moe", HummingExpertsBase._supports_batch_invariance
returns True and the experts' compute config carries use_batch_invariant).

Why it holds here: every element of every step is produced by the same
operations in the same order whatever the tile height, the column-tile width
and the other rows of its tile -- staging and the activation quantize one
row's groups; each GEMM output is one lane's chain of 128-deep MFMA block
products promoted (or, for the MX schemes, accumulated by the MFMA itself)
in ascending k order (a w2 whose reduction is split -- a choice made from
N alone -- adds its ranges' fp32 partials in range order); the reduce sums
a token's slots in ascending order.
So a token run alone (16-row tiles), inside a small batch (16- or 32-row
tiles) and inside a large one (its default tiles, and 128- and 256-row
tiles forced) must give identical bits.  The test also runs the tokens in reverse order,
which changes every expert's row order.
"""
import numpy as np
import pytest
import torch

import fp8_block_quantized_group_amd as moe
import moe_synth

pytestmark = pytest.mark.gpu

SCHEMES = {
    "ue8m0": dict(act_quant="ue8m0"),
    # N = 8192: w2 splits its reduction in two (the split depends on N only)
    "ue8m0_split": dict(act_quant="ue8m0", N=8192, K=512),
    "fp32": dict(act_quant="fp32"),
    # K = N = 4096: weight rows of 4 KB, so both GEMMs rotate their k-step
    # order (keyed by expert and output columns, never by the batch)
    "ue8m0_krot": dict(act_quant="ue8m0", K=4096, N=4096),
    "mxfp8": dict(act_quant="mxfp8", weight_quant="mxfp8"),
    "mxfp4": dict(act_quant="mxfp8", weight_quant="mxfp4"),
    "bf16": dict(act_quant="bf16"),
}


def _forward(cfg, inp, sel=None, tile_m=None, monkeypatch=None):
    """moe_forward over the tokens ``sel`` (all if None), in that order."""
    if tile_m is not None:
        monkeypatch.setenv("MOE_TILE_M", str(tile_m))
    else:
        monkeypatch.delenv("MOE_TILE_M", raising=False)
    idx = torch.arange(cfg.T, device="cuda") if sel is None else \
        torch.as_tensor(sel, device="cuda", dtype=torch.int64)
    T = int(idx.numel())
    p = moe.Problem(T, cfg.K, cfg.N, cfg.E, cfg.top_k,
                    act_quant=moe.Problem.from_config(cfg).act_quant,
                    weight_quant=moe.Problem.from_config(cfg).weight_quant)
    got_tile = moe.sizes(p)["tile_m"]
    layer = moe.MoeLayer(p, inp["w13"], inp["w13_sf"], inp["w2"], inp["w2_sf"])
    out = layer(inp["hidden"][idx].contiguous(), inp["topk_ids"][idx].contiguous(),
                inp["topk_weights"][idx].contiguous())
    torch.cuda.synchronize()
    return out.view(torch.int16).cpu().numpy(), got_tile


@pytest.mark.parametrize("scheme", list(SCHEMES))
def test_token_bits_independent_of_batch(scheme, monkeypatch):
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    # 384 tokens x top-2 over 6 experts: 128 rows per expert on average
    sizes = dict(K=1024, N=1024)
    sizes.update({k: v for k, v in SCHEMES[scheme].items() if k in ("K", "N")})
    cfg = moe_synth.custom(name=f"invariance_{scheme}", T=384, E=6, top_k=2, seed=51, **sizes,
                           **{k: v for k, v in SCHEMES[scheme].items() if k not in ("K", "N")})
    inp = moe_synth.make_inputs(cfg, "cuda")
    full, tile = _forward(cfg, inp, monkeypatch=monkeypatch)
    # a split w2 at 128 rows per expert: 160-row tiles (block scheme)
    assert tile == (160 if cfg.N >= 8192 else 128), tile
    # the same batch with other tile heights
    tall = 64 if cfg.act_quant == "bf16" else 256
    for other in (128, tall):
        full2, tile2 = _forward(cfg, inp, tile_m=other, monkeypatch=monkeypatch)
        assert tile2 == other
        assert np.array_equal(full, full2), f"{scheme}: {tile}- and {other}-row tiles differ"
    # reversed token order: every expert's rows come in another order
    rev, _ = _forward(cfg, inp, sel=np.arange(cfg.T)[::-1].copy(), monkeypatch=monkeypatch)
    assert np.array_equal(rev[::-1], full), f"{scheme}: reversed batch differs"
    # tokens alone (16-row tiles) and a 40-token slice (small tiles)
    rng = np.random.default_rng(7)
    ids = inp["topk_ids"].cpu().numpy()
    counts = np.bincount(ids.reshape(-1), minlength=cfg.E)
    hot = np.flatnonzero((ids == np.argmax(counts)).any(axis=1))
    picks = sorted(set([int(rng.choice(hot))] + rng.choice(cfg.T, 4, replace=False).tolist()))
    for t in picks:
        one, tile1 = _forward(cfg, inp, sel=[t], monkeypatch=monkeypatch)
        assert tile1 == 16
        assert np.array_equal(one[0], full[t]), f"{scheme}: token {t} alone differs"
    lo = int(rng.integers(0, cfg.T - 40))
    part, tile3 = _forward(cfg, inp, sel=np.arange(lo, lo + 40), monkeypatch=monkeypatch)
    assert tile3 in (16, 32), tile3
    assert np.array_equal(part, full[lo:lo + 40]), f"{scheme}: 40-token slice differs"
    print(f"{scheme}: tokens {picks} alone, a 40-token slice, {tile}/128/{tall}-row tiles and "
          f"the reversed batch give identical bits")
