"""Workloads at the limits the boundary accepts, end to end against the oracle.

Small token counts keep the oracle fast; the sizes sit on the edges the host
validation and the kernels' fixed capacities define: 1024 experts (the
routing scan's one-block width), a top-k of 32 (four groups of the reduce's
8-slot loads), hidden and intermediate sizes of 32768 (256 k-steps: the
block scheme's full weight-scale panel; a 32768-long w2 reduction split in
two), K = 24576 at 160-row tiles (the last reduction length their shortened
weight-scale panel holds) and one group past it (the forced height is then
refused and the default tile runs), and the same long reductions with MX and
bf16 activations.  Each runs through test_gpu_parity's end-to-end path:
staging and routing bit-exact into the unfused chain, a2 within the
end-of-chain bar, the output within the benchmark spec's bound, moe_forward
bit-identical to the chain and deterministic.
"""
import pytest

import fp8_block_quantized_group_amd as moe
import moe_synth
import test_gpu_parity as P
from test_gpu_parity import gpu  # noqa: F401  (the session fixture)

pytestmark = pytest.mark.gpu

LIMITS = {
    "lim_e1024": (dict(T=96, E=1024, top_k=8, K=128, N=128, seed=81), {}),
    "lim_k32": (dict(T=64, E=64, top_k=32, K=256, N=256, seed=82, pad_frac=0.07), {}),
    "lim_hidden": (dict(T=8, E=2, top_k=1, K=32768, N=128, seed=83), {}),
    "lim_inter": (dict(T=8, E=2, top_k=2, K=128, N=32768, seed=84), {}),
    "lim_t160_edge": (dict(T=40, E=2, top_k=2, K=24576, N=256, seed=85), {"MOE_TILE_M": "160"}),
    "lim_t160_past": (dict(T=40, E=2, top_k=2, K=24704, N=256, seed=86), {"MOE_TILE_M": "160"}),
    "lim_mx_hidden": (dict(T=8, E=2, top_k=2, K=32768, N=256, seed=87, act_quant="mxfp8",
                           weight_quant="mxfp4"), {}),
    "lim_bf16_inter": (dict(T=8, E=2, top_k=2, K=256, N=16384, seed=88, act_quant="bf16"), {}),
}


@pytest.mark.parametrize("name", list(LIMITS))
def test_limit_config(gpu, name, monkeypatch):
    kw, env = LIMITS[name]
    for k in ("MOE_TILE_M", "MOE_KSPLIT", "MOE_TALL", "MOE_KROT"):
        monkeypatch.delenv(k, raising=False)
    for k, v in env.items():
        monkeypatch.setenv(k, v)
    cfg = moe_synth.custom(name=name, **kw)
    s = moe.sizes(P.problem(cfg))
    if name == "lim_t160_edge":
        assert s["tile_m"] == 160
    if name == "lim_t160_past":
        assert s["tile_m"] != 160
    print(f"{name}: tile {s['tile_m']}, w2 workspace {moe.w2_workspace_size(P.problem(cfg))} B",
          flush=True)
    P.CASES[name] = cfg
    P._forward_end_to_end(name)
