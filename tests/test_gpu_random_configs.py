"""Seeded random small workloads, end to end against the oracle.

The hand-picked configs of test_gpu_parity each exercise a known corner;
these draw the corners' combinations instead: every scheme pair (UE8M0 and
fp32 per-128 scales, MXFP8 and MXFP4 weights with MXFP8 activations, bf16
activations), the contiguous, batched and indexed layouts, 1-320 tokens,
1-40 experts, top-k 1-8, hidden and intermediate sizes of 1-12 scale groups,
uniform or Zipf routing, padding tokens, EPLB replicas (contiguous and indexed
layouts: the batched layout takes physical ids), and a forced tile
height (MOE_TILE_M) or w2 split (MOE_KSPLIT) on top; every fifth of the
later draws is shaped (about 100 rows per expert, Zipf) to put its heavy
experts in the second, 256-row tile list.  A forced tile height
the problem cannot take is ignored by the library (its own choice then
runs), so the draw needs no filter.  Each config is checked through
test_gpu_parity's end-to-end path where it applies (staging and routing
feed the unfused chain, its a2 within the end-of-chain bar, the output
within the benchmark spec's bound, moe_forward bit-identical to the chain and
deterministic); the indexed layout through moe_forward against the oracle.
"""
import numpy as np
import pytest
import torch

import fp8_block_quantized_group_amd as moe
import moe_synth
import test_gpu_parity as P
from parity_util import check_output, to_np
from test_gpu_parity import gpu  # noqa: F401  (the session fixture)

pytestmark = pytest.mark.gpu

SCHEMES = [("ue8m0", "fp8_block128"), ("fp32", "fp8_block128"), ("mxfp8", "mxfp8"),
           ("mxfp8", "mxfp4"), ("bf16", "fp8_block128")]
LAYOUTS = ["contiguous", "batched", "indexed"]
N_CONFIGS = 60


def _draw(i):
    """Config i and the environment it runs under (seeded, independent of
    the other draws)."""
    rng = np.random.default_rng(7000 + i)
    act, wq = SCHEMES[i % len(SCHEMES)]
    layout = LAYOUTS[(i // len(SCHEMES)) % len(LAYOUTS)]
    E = int(rng.integers(1, 41))
    top_k = int(rng.integers(1, min(E, 8) + 1))
    T = int(rng.integers(1, 321))
    K = 128 * int(rng.integers(1, 13))
    N = 128 * int(rng.integers(1, 13))
    tall = i >= 30 and i % 5 == 0 and act != "bf16" and layout != "batched"
    if tall:
        # about 100 rows per expert with Zipf skew at the default tile height:
        # 128-row tiles, and the experts above 128 rows in the 256-row list
        E = int(rng.integers(4, 13))
        top_k = int(rng.integers(2, 5))
        T = min(320, int(round(100 * E / top_k)))
    kw = dict(name=f"rand{i}", T=T, E=E, top_k=top_k, K=K, N=N, seed=7000 + i, layout=layout,
              act_quant=act, weight_quant=wq)
    if tall or (E > 2 and rng.random() < 0.5):
        kw.update(routing="zipf", zipf_s=1.1)
    if layout == "batched":
        kw["max_tokens"] = T                     # an expert gets each token at most once
    elif rng.random() < 0.5:
        kw["pad_frac"] = 0.07
    if layout != "batched" and E >= 4 and rng.random() < 0.5:
        # EPLB replicas of distinct logical experts; top_k of them per token
        kw["num_logical"] = max(top_k, E - int(rng.integers(1, E // 2 + 1)))
    env = {}
    r = rng.random()
    if tall:
        pass
    elif r < 0.4:
        env["MOE_TILE_M"] = str(int(rng.choice([16, 32, 64, 128, 160, 192, 256])))
    elif r < 0.6:
        env["MOE_KSPLIT"] = str(int(rng.choice([2, 4])))
    return moe_synth.custom(**kw), env


@pytest.mark.parametrize("i", range(N_CONFIGS))
def test_random_config(gpu, i, monkeypatch):
    cfg, env = _draw(i)
    for k in ("MOE_TILE_M", "MOE_KSPLIT", "MOE_TALL", "MOE_KROT"):
        monkeypatch.delenv(k, raising=False)
    for k, v in env.items():
        monkeypatch.setenv(k, v)
    print(f"rand{i}: T={cfg.T} E={cfg.E} k={cfg.top_k} K={cfg.K} N={cfg.N} {cfg.layout} "
          f"{cfg.act_quant}/{cfg.weight_quant} {cfg.routing} pad={cfg.pad_frac} "
          f"logical={cfg.num_logical} env={env} tile={moe.sizes(P.problem(cfg))['tile_m']}",
          flush=True)
    P.CASES[cfg.name] = cfg
    if cfg.layout != "indexed":
        P._forward_end_to_end(cfg.name)
        return
    _, h, dev, ref = P.case(cfg.name)
    out = P.run_forward(cfg, dev)
    check_output(to_np(out), ref["out"], f"{cfg.name} moe_forward output")
    if cfg.eplb:
        assert np.array_equal(to_np(dev["eplb"]["expert_load"]), ref["load"])
    again = P.run_forward(cfg, dev)
    assert torch.equal(out.view(torch.int16), again.view(torch.int16)), "not deterministic"
    if cfg.pad_frac > 0:
        assert np.all(to_np(out)[h["is_padding"].astype(bool)] == 0)
