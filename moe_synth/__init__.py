"""Seeded synthetic inputs for the fp8 block-quantized MoE expert layer.

This module is the one piece shared by the CPU oracle and the HIP path: it
draws the layer's inputs and holds none of the layer's own arithmetic (no
activation quantization, no routing layout, no GEMM, no reduce).

What it draws, per workload (the shapes the vLLM API pages' MoE layer is
called with: ``hidden_states [T, K]``, ``topk_ids``/``topk_weights [T, top_k]``,
fused gate/up weights ``w13 [E, 2N, K]`` and down weights ``w2 [E, K, N]``
with 128x128 fp32 block scales, "Fused MoE utilities for Humming",
``HummingExpertsBase.get_buffer_metas`` and the ``kFp8Static128BlockSym``
weight scheme):

* hidden states: fp32 N(0, 1) rounded to bf16 by torch's own cast;
* router: iid N(0, 1) logits over the logical experts, top-k, softmax over
  the k chosen logits (fp32); a Zipf(s) skew is drawn as
  ``log p(expert) + Gumbel(0, 1)`` logits, which makes top-k a draw without
  replacement proportional to p;
* padding: an exact fraction of token positions, picked by a seeded
  permutation; those tokens keep valid-looking ids and weights, so the
  staging step has to unroute them itself;
* weights: fp32 N(0, 0.02) per expert, quantized per 128x128 block to fp8
  e4m3fn with scale ``amax / 448`` by torch's ``float8_e4m3fn`` cast (the
  pages show no weight quantizer; this is only a way to get realistic codes);
* batched-masked staging: each expert's routed tokens, in ascending
  (token, slot) order, copied into ``[E, max_tokens, K]``; rows past the
  count are filled with bf16 NaN / +-Inf / +-3e38 garbage;
* expert-parallel load balancing state: a seeded set of logical experts gets
  a second physical replica whose weights are copies of the original.

Every tensor is drawn on ``device`` by a torch generator seeded from
``(seed, stream)``; a CPU draw and a GPU draw with the same seed differ, so a
test always hands the oracle host copies of the very tensors the GPU used.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

# Independent random streams, one generator per input.
_STREAMS = ("hidden", "logits", "gumbel", "expert_perm", "padding", "w13",
            "w2", "garbage", "replicas")


@dataclasses.dataclass(frozen=True)
class MoeConfig:
    """One synthetic workload.  Sizes follow the usual MoE notation:
    T tokens, E physical experts (E_log logical), top_k, hidden K,
    intermediate N."""
    name: str
    T: int
    E: int
    top_k: int
    K: int
    N: int
    seed: int
    layout: str = "contiguous"          # "contiguous" | "batched" | "indexed"
    max_tokens: int = 0                 # batched layout: rows per expert slab
    act_quant: str = "ue8m0"            # "ue8m0" | "fp32" (128-groups) | "mxfp8" (32-groups) | "bf16"
    weight_quant: str = "fp8_block128"  # "fp8_block128" | "mxfp8" | "mxfp4"
    routing: str = "uniform"            # "uniform" | "zipf"
    zipf_s: float = 1.1
    pad_frac: float = 0.0
    num_logical: int = 0                # >0: EPLB with E - num_logical replicas
    weight_std: float = 0.02
    # "silu" | "gelu" | "gelu_tanh" | "swigluoai" | "swiglustep" (gated: w13
    # has 2N rows, gate then up) | "silu_no_mul" | "gelu_no_mul" |
    # "gelu_tanh_no_mul" | "relu2_no_mul" (w13 has N rows, the activation
    # applies to all of them)
    activation: str = "silu"
    # clamp limit of the gated SwiGLU forms (0: none for SiLU, the default
    # for SWIGLUOAI / SWIGLUSTEP)
    act_limit: float = 0.0

    @property
    def gated(self) -> bool:
        return not self.activation.endswith("_no_mul")

    @property
    def w13_rows(self) -> int:
        return 2 * self.N if self.gated else self.N

    @property
    def E_log(self) -> int:
        return self.num_logical if self.num_logical else self.E

    @property
    def eplb(self) -> bool:
        return self.num_logical > 0


# The five workloads the layer is sized for.
CONFIGS = {
    "tiny": MoeConfig("tiny", T=16, E=4, top_k=2, K=256, N=512, seed=1),
    "mixtral": MoeConfig("mixtral", T=512, E=8, top_k=2, K=4096, N=14336,
                         seed=2, layout="batched", max_tokens=256),
    "dsv3_prefill": MoeConfig("dsv3_prefill", T=4096, E=256, top_k=8, K=7168,
                              N=2048, seed=3, routing="zipf", zipf_s=1.1,
                              pad_frac=0.05),
    "dsv3_decode": MoeConfig("dsv3_decode", T=64, E=256, top_k=8, K=7168,
                             N=2048, seed=4),
    "qwen3": MoeConfig("qwen3", T=16384, E=144, top_k=8, K=4096, N=1536,
                       seed=5, act_quant="fp32", num_logical=128),
}


# The same DeepSeek-V3-shaped prefill batch with the MX scheme pairs the
# Humming experts accept: (kMxfp8Static weights, kMxfp8Dynamic activations)
# and (kMxfp4Static, kMxfp8Dynamic); plus small cases for parity tests.
MX_CONFIGS = {
    "dsv3_prefill_mxfp8": MoeConfig("dsv3_prefill_mxfp8", T=4096, E=256, top_k=8, K=7168,
                                    N=2048, seed=6, routing="zipf", zipf_s=1.1,
                                    pad_frac=0.05, act_quant="mxfp8", weight_quant="mxfp8"),
    "dsv3_prefill_mxfp4": MoeConfig("dsv3_prefill_mxfp4", T=4096, E=256, top_k=8, K=7168,
                                    N=2048, seed=7, routing="zipf", zipf_s=1.1,
                                    pad_frac=0.05, act_quant="mxfp8", weight_quant="mxfp4"),
}

# The Qwen3-shaped batch with unquantized bf16 activations (the staging copy
# variant, carried through the layer with the (kFp8Static128BlockSym, None)
# scheme pair).
BF16_CONFIGS = {
    "qwen3_bf16": MoeConfig("qwen3_bf16", T=16384, E=144, top_k=8, K=4096, N=1536,
                            seed=5, act_quant="bf16", num_logical=128),
}

# The DeepSeek-V3-shaped prefill batch (the same inputs: same seed) run
# through the indexed experts' block map instead of the contiguous rows.
INDEXED_CONFIGS = {
    "dsv3_prefill_indexed": MoeConfig("dsv3_prefill_indexed", T=4096, E=256, top_k=8, K=7168,
                                      N=2048, seed=3, routing="zipf", zipf_s=1.1,
                                      pad_frac=0.05, layout="indexed"),
}

ALL_CONFIGS = {**CONFIGS, **MX_CONFIGS, **BF16_CONFIGS, **INDEXED_CONFIGS}


def _gen(device, seed: int, stream: str) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1_000_003 + _STREAMS.index(stream) * 7919 + 17)
    return g


def _quantize_weight_blocks(w: torch.Tensor):
    """fp32 [R, C] -> (fp8 codes uint8 [R, C], fp32 scales [R/128, C/128]),
    scale = block amax / 448, codes from torch's e4m3fn cast."""
    R, C = w.shape
    blocks = w.view(R // 128, 128, C // 128, 128)
    amax = blocks.abs().amax(dim=(1, 3))
    scale = (amax / 448.0).to(torch.float32)
    q = (blocks / scale[:, None, :, None]).to(torch.float8_e4m3fn)
    return q.view(R, C).view(torch.uint8), scale


# e2m1 magnitudes by 3-bit code (OCP MX fp4: 1 sign, 2 exponent, 1 mantissa bit)
_E2M1 = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def _quantize_weight_mx(w: torch.Tensor, fp4: bool):
    """fp32 [R, C] -> MX codes + E8M0 scales per 32 consecutive columns, with
    the OCP MX shared-exponent rule: exponent = floor(log2(block amax)) minus
    the element format's largest exponent (8 for e4m3, 2 for e2m1), elements
    rounded to nearest and saturated.  e4m3: codes uint8 [R, C]; e2m1: two
    codes per byte, column 2j in the low nibble, uint8 [R, C/2].  Scales uint8
    [R, C/32] (2^(byte - 127))."""
    R, C = w.shape
    blocks = w.view(R, C // 32, 32)
    amax = blocks.abs().amax(dim=2)
    emax = 2 if fp4 else 8
    shared = torch.floor(torch.log2(amax.clamp_min(2.0 ** -120))) - emax
    shared = shared.clamp(-127, 127)
    v = blocks / torch.exp2(shared)[:, :, None]
    if not fp4:
        q = v.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).view(R, C)
    else:
        mags = torch.tensor(_E2M1, device=w.device)
        mid = (mags[1:] + mags[:-1]) / 2
        code = torch.bucketize(v.abs().clamp(max=6.0), mid).to(torch.uint8)
        code = code | ((v < 0).to(torch.uint8) << 3)
        code = code.view(R, C)
        q = code[:, 0::2] | (code[:, 1::2] << 4)
    return q.contiguous(), (shared + 127).to(torch.uint8)


def _draw_weights(cfg: MoeConfig, device, which: str):
    """w13 [E_log, 2N (N without gating), K] or w2 [E_log, K, N] codes + scales, one expert at a
    time so the fp32 draw never exceeds one expert.  fp8_block128: e4m3 codes
    and fp32 scales per 128x128 block; mxfp8 / mxfp4: MX codes and E8M0
    scales per row and 32 columns."""
    g = _gen(device, cfg.seed, which)
    rows, cols = (cfg.w13_rows, cfg.K) if which == "w13" else (cfg.K, cfg.N)
    if cfg.weight_quant == "fp8_block128":
        q = torch.empty((cfg.E_log, rows, cols), dtype=torch.uint8, device=device)
        s = torch.empty((cfg.E_log, rows // 128, cols // 128), dtype=torch.float32,
                        device=device)
    else:
        fp4 = cfg.weight_quant == "mxfp4"
        q = torch.empty((cfg.E_log, rows, cols // 2 if fp4 else cols), dtype=torch.uint8,
                        device=device)
        s = torch.empty((cfg.E_log, rows, cols // 32), dtype=torch.uint8, device=device)
    for e in range(cfg.E_log):
        w = torch.randn((rows, cols), generator=g, device=device,
                        dtype=torch.float32) * cfg.weight_std
        if cfg.weight_quant == "fp8_block128":
            q[e], s[e] = _quantize_weight_blocks(w)
        else:
            q[e], s[e] = _quantize_weight_mx(w, cfg.weight_quant == "mxfp4")
    return q, s


def _route(cfg: MoeConfig, device):
    """Router stand-in: (topk_ids int32 [T, k], topk_weights fp32 [T, k])."""
    T, El, k = cfg.T, cfg.E_log, cfg.top_k
    logits = torch.randn((T, El), generator=_gen(device, cfg.seed, "logits"),
                         device=device, dtype=torch.float32)
    if cfg.routing == "zipf":
        ranks = torch.arange(1, El + 1, device=device, dtype=torch.float64)
        p_rank = ranks.pow(-cfg.zipf_s)
        p_rank = p_rank / p_rank.sum()
        perm = torch.randperm(El, generator=_gen(device, cfg.seed, "expert_perm"),
                              device=device)
        p = torch.empty(El, dtype=torch.float64, device=device)
        p[perm] = p_rank
        u = torch.rand((T, El), generator=_gen(device, cfg.seed, "gumbel"),
                       device=device, dtype=torch.float64)
        u = u.clamp_min(1e-300)
        gumbel = -torch.log(-torch.log(u))
        logits = (torch.log(p)[None, :] + gumbel).to(torch.float32)
    top_vals, top_ids = torch.topk(logits, k, dim=1, largest=True, sorted=True)
    weights = torch.softmax(top_vals, dim=1).to(torch.float32)
    return top_ids.to(torch.int32).contiguous(), weights.contiguous()


def _padding(cfg: MoeConfig, device) -> Optional[torch.Tensor]:
    if cfg.pad_frac <= 0.0:
        return None
    n_pad = int(math.floor(cfg.pad_frac * cfg.T))
    perm = torch.randperm(cfg.T, generator=_gen(device, cfg.seed, "padding"),
                          device=device)
    pad = torch.zeros(cfg.T, dtype=torch.uint8, device=device)
    pad[perm[:n_pad]] = 1
    return pad


def _eplb_tables(cfg: MoeConfig, device):
    """Physical experts 0..E_log-1 are the logical ones; physical E_log+i is
    a second replica of a seeded distinct logical expert."""
    El, n_rep = cfg.E_log, cfg.E - cfg.E_log
    perm = torch.randperm(El, generator=_gen("cpu", cfg.seed, "replicas"))
    replicated = perm[:n_rep].tolist()
    l2p = torch.full((El, 2), -1, dtype=torch.int32)
    l2p[:, 0] = torch.arange(El, dtype=torch.int32)
    count = torch.ones(El, dtype=torch.int32)
    for i, le in enumerate(replicated):
        l2p[le, 1] = El + i
        count[le] = 2
    return {
        "l2p": l2p.to(device),
        "replica_count": count.to(device),
        "replica_of": torch.tensor(replicated, dtype=torch.int64),
        "expert_load": torch.zeros(cfg.E, dtype=torch.int32, device=device),
        "record": torch.ones(1, dtype=torch.int32, device=device),
        "num_unpadded": torch.tensor([cfg.T], dtype=torch.int32, device=device),
    }


def _garbage_bf16(shape, device, seed: int) -> torch.Tensor:
    """bf16 NaN, +-Inf and +-3e38 patterns for rows nobody may read."""
    pats = torch.tensor([0x7FC0, 0xFFC0, 0x7F80, 0xFF80, 0x7F62, 0xFF62],
                        dtype=torch.int32)
    idx = torch.randint(0, len(pats), shape,
                        generator=_gen("cpu", seed, "garbage"))
    return pats[idx].to(torch.int16).view(torch.bfloat16).to(device)


def make_inputs(cfg: MoeConfig, device="cpu") -> dict:
    """Draw every input of one workload on ``device``.

    Returns a dict of tensors:
      hidden        bf16 [T, K] (contiguous) or [E, max_tokens, K] (batched)
      tokens        bf16 [T, K], the token-order hidden states
      topk_ids      int32 [T, top_k] (logical ids)
      topk_weights  fp32 [T, top_k]
      is_padding    uint8 [T] or None
      expert_num_tokens  int32 [E] (batched layout only)
      eplb          dict of tables or None
      w13, w13_sf   uint8 [E, 2N, K], fp32 [E, 2N/128, K/128]
      w2, w2_sf     uint8 [E, K, N],  fp32 [E, K/128, N/128]
    """
    device = torch.device(device)
    tokens = torch.randn((cfg.T, cfg.K), generator=_gen(device, cfg.seed, "hidden"),
                         device=device, dtype=torch.float32).to(torch.bfloat16)
    topk_ids, topk_weights = _route(cfg, device)
    is_padding = _padding(cfg, device)
    w13, w13_sf = _draw_weights(cfg, device, "w13")
    w2, w2_sf = _draw_weights(cfg, device, "w2")
    eplb = None
    if cfg.eplb:
        eplb = _eplb_tables(cfg, device)
        src = eplb["replica_of"].to(device)
        w13 = torch.cat([w13, w13[src]], dim=0)
        w13_sf = torch.cat([w13_sf, w13_sf[src]], dim=0)
        w2 = torch.cat([w2, w2[src]], dim=0)
        w2_sf = torch.cat([w2_sf, w2_sf[src]], dim=0)

    out = {
        "cfg": cfg, "tokens": tokens, "hidden": tokens,
        "topk_ids": topk_ids, "topk_weights": topk_weights,
        "is_padding": is_padding, "expert_num_tokens": None, "eplb": eplb,
        "w13": w13.contiguous(), "w13_sf": w13_sf.contiguous(),
        "w2": w2.contiguous(), "w2_sf": w2_sf.contiguous(),
    }
    if cfg.layout == "batched":
        out.update(_stage_batched(cfg, tokens, topk_ids, device))
    return out


def _stage_batched(cfg: MoeConfig, tokens, topk_ids, device) -> dict:
    """Dispatcher stand-in for the batched-experts format: expert e's routed
    tokens, in ascending (token, slot) order, fill rows 0..count-1 of slab e."""
    ids = topk_ids.to("cpu").to(torch.int64)
    T, k = ids.shape
    slab = _garbage_bf16((cfg.E, cfg.max_tokens, cfg.K), "cpu", cfg.seed)
    counts = torch.zeros(cfg.E, dtype=torch.int32)
    tok_cpu = tokens.to("cpu")
    src_rows = [[] for _ in range(cfg.E)]
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            if 0 <= e < cfg.E:
                src_rows[e].append(t)
    for e in range(cfg.E):
        n = len(src_rows[e])
        if n > cfg.max_tokens:
            raise ValueError(f"expert {e} got {n} rows > max_tokens {cfg.max_tokens}")
        counts[e] = n
        if n:
            slab[e, :n] = tok_cpu[torch.tensor(src_rows[e])]
    return {"hidden": slab.to(device), "expert_num_tokens": counts.to(device)}


def custom(name="custom", **kw) -> MoeConfig:
    """A workload with explicit sizes (tests use these for ragged cases)."""
    return MoeConfig(name=name, **kw)
