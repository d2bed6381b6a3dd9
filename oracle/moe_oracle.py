"""CPU oracle for the fp8 block-quantized MoE expert layer.

TEST INFRASTRUCTURE ONLY.  A plain, slow, obviously correct numpy model of
what the layer computes.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import it; the product path
never does, and this file shares no code, table or constant generator with
the HIP library.

Sources (all from the vLLM API documentation pages on the subject):
  [STAGE]  "vllm.model_executor.layers.fused_moe.prepare_megamoe":
           ``_quantize_fp8_groups``, ``_store_topk``, ``_pack_bytes``,
           ``_eplb_kernel_args``, ``prepare_megamoe_inputs``.
  [HUM]    "vllm.model_executor.layers.fused_moe.experts.fused_humming_moe"
           (pull-request 58588 build): ``BatchedHummingGroupedExperts.apply``,
           ``HummingGroupedExperts.apply``, ``HummingExpertsBase``
           (``process_input``, ``get_buffer_metas``,
           ``_supports_quant_scheme``).
  [HUM2]   the same module on the latest-docs page: the activation list of
           ``_supports_activation`` and the activation buffer widths of
           ``get_buffer_metas``.

Schemes: unquantized bf16 activations with block fp8 weights (the
(kFp8Static128BlockSym, None) pair; staging copies the hidden states, the w2
input is silu(gate)*up rounded to bf16); block fp8 (kFp8Static128BlockSym
weights with 128x128 fp32 scales,
kFp8Dynamic128Sym activations with UE8M0 or fp32 per-128 scales) and MX
(kMxfp8Static / kMxfp4Static weights with one E8M0 scale per row and 32
columns, kMxfp8Dynamic activations: the staging quantizer with 32-column
groups and E8M0 scales, which [STAGE] ``_resolve_hidden_quant`` maps to
GROUP_K = 32, USE_UE8M0).

Number formats.  bf16 -> fp64 and e4m3fn -> fp64 are exact.  fp32 steps are
numpy float32 operations (IEEE binary32, round to nearest even).  Block
partial sums of fp8 products are exact in fp64 (products of two e4m3fn
values have at most 8 significant bits and lie in [2^-18, 2^17.6], so a sum
of 128 of them needs fewer than 45 bits).

Readings of points the pages leave open (each one is listed, with its
reason, in the design notes):
  * all of the group quantizer runs in fp32 after an exact bf16 -> fp32 upcast;
  * fp32 divisions are correctly rounded; values are scaled as ``x * (1/s)``;
  * fp32 -> e4m3fn rounds to nearest even and saturates to +-448;
  * UE8M0 scale bytes are stored one per group, ``4*ceil(G/4)`` bytes per
    row (byte-identical to little-endian packing four per int32), pad 0;
  * w13 rows [0, N) are the gate projection, rows [N, 2N) the up projection;
  * SiLU(gate)*up stays fp32 and is quantized directly (no bf16 rounding);
  * gate_up and down are rounded once to bf16 (nearest even);
  * padding tokens are unrouted (id -1, weight 0); ids outside [0, E) are
    unrouted; an expert's rows are ordered by ascending (token, slot);
  * expert replica choice under EPLB is ``token mod replica_count`` (parity
    unpinned: the pages do not show ``eplb_map_and_record``'s body; only the
    invariants it must satisfy are tested);
  * activations other than SiLU (named on the pages, formulas not shown)
    take their standard definitions; gated ones read w13's 2N columns as
    gate then up, the _no_mul ones act on all N columns of a w13 with N rows
    (the w2 input width is N in both cases);
  * the clamped SwiGLU forms, named on the pages without bodies or
    constants (parity unpinned: only the properties of this reading are
    tested): SiLU with a clamp limit L (the experts' gemm1_clamp_limit)
    is silu(min(g, L)) * clamp(u, -L, L); SWIGLUSTEP is
    min(silu(g), L) * clamp(u, -L, L); SWIGLUOAI is
    (clamp(u, -L, L) + 1) * g' * sigmoid(1.702 g') with g' = min(g, L);
    L defaults to 7 for the last two;
  * MX: the w2 input (SiLU(gate)*up) is quantized like the staged hidden
    states, 32-column groups with E8M0 scales (Humming's own input quantizer
    is not shown); E8M0 byte e means 2^(e-127); e2m1 codes are packed two per
    byte, even column in the low nibble.
"""
from __future__ import annotations

import math

import numpy as np

GROUP = 128          # quantization group along K (and along N for w2's input)
FP8_MAX = 448.0      # largest finite e4m3fn value


# ---------------------------------------------------------------------------
# Codecs
# ---------------------------------------------------------------------------

def _e4m3fn_table() -> np.ndarray:
    """Value of every e4m3fn byte (OCP 8-bit float, 'fn' variant: exponent
    bias 7, 3 mantissa bits, subnormals m*2^-9, no infinities, S.1111.111 is
    NaN).  [STAGE] stores quantized hidden states as ``tl.float8e4nv``,
    which is this format."""
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        exp = (code >> 3) & 0xF
        man = code & 0x7
        if exp == 0xF and man == 0x7:
            vals[code] = np.nan
        elif exp == 0:
            vals[code] = sign * man * 2.0 ** -9
        else:
            vals[code] = sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)
    return vals


E4M3_VALUES = _e4m3fn_table()
_POS_FINITE = E4M3_VALUES[:0x7F]          # codes 0x00..0x7E, increasing


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    return E4M3_VALUES[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(v) -> np.ndarray:
    """fp32 values -> e4m3fn codes: nearest representable value, ties to the
    even code (even mantissa), magnitudes above 448 saturate to 448, NaN ->
    NaN; the sign is kept (-0 -> 0x80)."""
    v = np.asarray(v, dtype=np.float32)
    a = np.abs(v).astype(np.float64).ravel()
    hi = np.searchsorted(_POS_FINITE, a, side="left")      # first value >= a
    hi_c = np.minimum(hi, 0x7E)
    lo_c = np.maximum(hi - 1, 0)
    d_lo = a - _POS_FINITE[lo_c]
    d_hi = _POS_FINITE[hi_c] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi_c % 2 == 0))
    code = np.where(pick_hi, hi_c, lo_c)
    code = np.where(hi == 0, 0, code)                       # a == 0
    code = np.where(hi > 0x7E, 0x7E, code)                  # saturate
    code = np.where(np.isnan(a), 0x7F, code).astype(np.uint8)
    sign = (np.signbit(v.ravel())).astype(np.uint8) << 7
    return (code | sign).reshape(v.shape)


def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact fp64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def bf16_round(x) -> np.ndarray:
    """fp64 -> bf16 bit patterns, one rounding to nearest even (8 significant
    bits; the fp32 exponent range, with subnormals below 2^-126)."""
    x = np.asarray(x, dtype=np.float64)
    mant, exp = np.frexp(x)                    # x = mant * 2^exp, |mant| in [0.5, 1)
    normal = np.abs(x) >= 2.0 ** -126
    q_norm = np.ldexp(np.rint(np.ldexp(mant, 8)), exp - 8)
    q_sub = np.ldexp(np.rint(np.ldexp(x, 133)), -133)
    q = np.where(normal, q_norm, q_sub)
    q = np.where(np.abs(q) > 3.3895313892515355e38, np.copysign(np.inf, x), q)
    q = np.where(np.isnan(x), np.nan, q)
    bits = (q.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return bits


def ue8m0_decode(e) -> np.ndarray:
    """UE8M0 scale byte e -> 2^(e-127)."""
    return np.ldexp(1.0, np.asarray(e, dtype=np.int64) - 127)


# ---------------------------------------------------------------------------
# O2: per-128-group fp8 quantization  [STAGE, _quantize_fp8_groups]
# ---------------------------------------------------------------------------

def ceil_log2(s) -> np.ndarray:
    """ceil(log2 s) for positive fp32 s, exactly: frexp writes s = m * 2^x
    with m in [0.5, 1), so log2 s lies in [x - 1, x) and equals x - 1 only
    when m = 0.5 (s is a power of two).  Infinite or NaN s gives a value
    above every clamp (the largest scale)."""
    s = np.asarray(s, dtype=np.float64)
    m, x = np.frexp(np.where(np.isfinite(s), s, 1.0))
    c = np.where(m == 0.5, x - 1, x).astype(np.int64)
    return np.where(np.isfinite(s), c, 1 << 20)


def quantize_groups(x32, ue8m0: bool, group: int = GROUP):
    """Quantize rows of fp32 values in groups of ``group`` consecutive columns
    (128 for the block scheme, 32 for MXFP8; any divisor of 128 for [STAGE]).

    Per group, in fp32: amax = max|x|, amax = max(amax, 1e-4),
    s = amax / 448 (one correctly rounded fp32 division).  UE8M0: the scale
    is s rounded up to the next power of two, 2^c with c = ceil(log2 s),
    whose biased exponent e = c + 127 is clamped to [1, 254]; the quantizing
    scale is 2^(e-127) and the stored value is the byte e.  fp32: the
    quantizing scale is s itself and the stored value is s.  Values are
    x * (1/scale) converted to e4m3fn.

    Returns (codes uint8 [rows, C], stored scales: uint8 [rows, G] exponents
    or float32 [rows, G]).
    """
    x32 = np.asarray(x32, dtype=np.float32)
    rows, cols = x32.shape
    assert cols % group == 0
    g = x32.reshape(rows, cols // group, group)
    amax = np.max(np.abs(g), axis=2)
    amax = np.maximum(amax, np.float32(1.0e-4))
    s = (amax / np.float32(FP8_MAX)).astype(np.float32)
    if ue8m0:
        e = np.clip(ceil_log2(s) + 127, 1, 254)
        qscale = np.ldexp(np.float32(1.0), e - 127).astype(np.float32)
        stored = e.astype(np.uint8)
    else:
        qscale = s
        stored = s
    recip = (np.float32(1.0) / qscale).astype(np.float32)
    v = (g * recip[:, :, None]).astype(np.float32)
    codes = e4m3_encode(v).reshape(rows, cols)
    return codes, stored


# ---------------------------------------------------------------------------
# MX element formats (OCP Microscaling: E8M0 scales, e4m3 / e2m1 elements)
# ---------------------------------------------------------------------------

E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
                        -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0])


def e2m1_decode(nibbles) -> np.ndarray:
    """4-bit e2m1 codes (sign bit 3, exponent bits 2..1 with bias 1, mantissa
    bit 0; exponent 0 is subnormal: 0.5 * mantissa) -> fp64."""
    return E2M1_VALUES[np.asarray(nibbles, dtype=np.int64) & 0xF]


def unpack_fp4(packed) -> np.ndarray:
    """uint8 [..., C/2] -> nibbles [..., C]: column 2j is byte j's low nibble."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out


def scale_values(stored, ue8m0: bool) -> np.ndarray:
    """Stored activation scales -> their exact fp64 values."""
    return ue8m0_decode(stored) if ue8m0 else np.asarray(stored, np.float64)


def pack_ue8m0_rows(exps) -> np.ndarray:
    """[rows, G] exponent bytes -> [rows, 4*ceil(G/4)] bytes, pad bytes 0.
    Little-endian int32 words with byte j at bits 8j hold the same bytes
    ([STAGE, _pack_bytes])."""
    exps = np.asarray(exps, dtype=np.uint8)
    rows, G = exps.shape
    out = np.zeros((rows, 4 * ((G + 3) // 4)), dtype=np.uint8)
    out[:, :G] = exps
    return out


# ---------------------------------------------------------------------------
# O3: routing repack  [STAGE, _store_topk and _eplb_kernel_args]
# ---------------------------------------------------------------------------

def repack_topk(topk_ids, topk_weights, is_padding=None, eplb=None,
                num_physical=None):
    """Routing ids -> int64 (padding tokens -> -1), weights -> fp32 (padding
    tokens -> 0).  With expert-replica tables, a logical id in
    [0, num_logical) becomes ``l2p[id, t mod replica_count[id]]``; when the
    record flag is set, every mapped id of a token t < num_unpadded adds one
    to ``expert_load[id]``.

    Returns (ids int64 [T, k], weights fp32 [T, k], load int32 [E] or None).
    """
    ids = np.asarray(topk_ids).astype(np.int64).copy()
    w = np.asarray(topk_weights, dtype=np.float32).copy()
    T, k = ids.shape
    if is_padding is not None:
        pad = np.asarray(is_padding).astype(bool)
        ids[pad, :] = -1
        w[pad, :] = 0.0
    load = None
    if eplb is not None:
        l2p = np.asarray(eplb["l2p"], dtype=np.int64)
        count = np.asarray(eplb["replica_count"], dtype=np.int64)
        num_logical = l2p.shape[0]
        record = int(np.asarray(eplb["record"]).ravel()[0]) != 0
        num_unpadded = int(np.asarray(eplb["num_unpadded"]).ravel()[0])
        load = np.zeros(num_physical, dtype=np.int32)
        for t in range(T):
            for j in range(k):
                lid = ids[t, j]
                if 0 <= lid < num_logical:
                    pid = l2p[lid, t % count[lid]]
                    ids[t, j] = pid
                    if record and t < num_unpadded and 0 <= pid < num_physical:
                        load[pid] += 1
    return ids, w, load


# ---------------------------------------------------------------------------
# O4: per-expert counts, offsets and the row permutation
#     [HUM, HummingGroupedExperts.apply: moe_prepare_scatter / moe_permute]
# ---------------------------------------------------------------------------

def route_layout(ids, E: int, max_tokens: int = 0):
    """Group routed (token, slot) pairs by expert.

    Rows of expert e are its slots in ascending flat order t*k + j.
    Contiguous layout: row = offsets[e] + rank.  Batched-masked layout
    (max_tokens > 0): row = e * max_tokens + rank.

    Returns dict: counts int32 [E], offsets int32 [E+1], row_src int32 [M]
    (token of each contiguous row), slot_row int32 [T, k] (-1: unrouted).
    """
    ids = np.asarray(ids, dtype=np.int64)
    T, k = ids.shape
    flat = ids.ravel()
    valid = (flat >= 0) & (flat < E)
    key = np.where(valid, flat, E)
    order = np.argsort(key, kind="stable")
    counts = np.bincount(flat[valid], minlength=E).astype(np.int32)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    M = int(offsets[-1])
    sorted_slots = order[:M]
    row_src = (sorted_slots // k).astype(np.int32)
    slot_row = np.full(T * k, -1, dtype=np.int64)
    if max_tokens:
        rank = np.arange(M) - offsets[flat[sorted_slots]]
        slot_row[sorted_slots] = flat[sorted_slots] * max_tokens + rank
    else:
        slot_row[sorted_slots] = np.arange(M)
    return {
        "counts": counts,
        "offsets": offsets.astype(np.int32),
        "row_src": row_src,
        "slot_row": slot_row.reshape(T, k).astype(np.int32),
    }


def align_block_size(ids, E: int, block_size: int):
    """The indexed experts' alignment ([HUM] HummingIndexedExperts
    .prepare_humming_moe_kwargs calls moe_align_block_size; its body is not
    on the pages, this is the plainest reading): each expert's routed flat
    slot indices t*k + j in ascending order, the segment padded with the
    sentinel T*k up to a multiple of block_size, experts in id order; the
    expert id of every block; the padded total.  Invalid ids are ignored.

    Returns (sorted_ids int32 [P], expert_ids int32 [P / block_size], P)."""
    ids = np.asarray(ids, dtype=np.int64)
    T, k = ids.shape
    flat = ids.ravel()
    numel = T * k
    sorted_ids, expert_ids = [], []
    for e in range(E):
        slots = np.flatnonzero(flat == e)
        if slots.size == 0:
            continue
        padded = -(-slots.size // block_size) * block_size
        seg = np.full(padded, numel, dtype=np.int64)
        seg[:slots.size] = slots
        sorted_ids.append(seg)
        expert_ids += [e] * (padded // block_size)
    sorted_ids = (np.concatenate(sorted_ids) if sorted_ids else np.zeros(0, np.int64))
    return sorted_ids.astype(np.int32), np.asarray(expert_ids, dtype=np.int32), int(sorted_ids.size)


def fused_mul_sum(down_bits, ids, weights, E: int) -> np.ndarray:
    """out[t] = bf16(sum over slots j ascending with a valid id of
    weights[t, j] * down[t*k + j]) — down in (token, slot) row order, as the
    indexed experts' moe_fused_mul_sum reads it.  fp64 accumulation."""
    ids = np.asarray(ids, dtype=np.int64)
    T, k = ids.shape
    down = bf16_to_f64(down_bits).reshape(T, k, -1)
    acc = np.zeros((T, down.shape[2]), dtype=np.float64)
    for j in range(k):
        ok = (ids[:, j] >= 0) & (ids[:, j] < E)
        acc[ok] += np.asarray(weights, np.float64)[ok, j:j + 1] * down[ok, j]
    return bf16_round(acc)


# ---------------------------------------------------------------------------
# O5 / O7: block-scaled fp8 GEMM   [HUM, humming_forward on w13 and w2 with
# the (kFp8Static128BlockSym weight, kFp8Dynamic128Sym activation) scheme]
# ---------------------------------------------------------------------------

def block_scaled_gemm_f64(a_codes, a_scale, w_codes, w_scale) -> np.ndarray:
    """out[m, n] = sum_b a_scale[m, b] * w_scale[n // 128, b]
                          * sum_{c in block b} a[m, c] * w[n, c]

    a_codes uint8 [m, C] (e4m3fn), a_scale fp64 [m, C/128],
    w_codes uint8 [n, C], w_scale fp32 [n/128, C/128].  Result in fp64
    before the bf16 rounding; the inner block sums are exact.
    """
    a = e4m3_decode(a_codes)
    w = e4m3_decode(w_codes)
    m, C = a.shape
    n = w.shape[0]
    G = C // GROUP
    a_b = a.reshape(m, G, GROUP).transpose(1, 0, 2)          # [G, m, 128]
    w_b = w.reshape(n, G, GROUP).transpose(1, 2, 0)          # [G, 128, n]
    partial = np.matmul(a_b, w_b)                            # [G, m, n], exact
    ws = np.repeat(np.asarray(w_scale, np.float64), GROUP, axis=0)  # [n, G]
    out = np.zeros((m, n), dtype=np.float64)
    for b in range(G):
        out += partial[b] * np.asarray(a_scale, np.float64)[:, b:b + 1] * ws[None, :, b]
    return out


def mx_gemm_f64(a_codes, a_exps, w_codes, w_exps, fp4: bool) -> np.ndarray:
    """out[m, n] = sum_b 2^(ea[m, b] - 127) * 2^(ew[n, b] - 127)
                          * sum_{c in block b} a[m, c] * w[n, c]
    over 32-column blocks b (the MX scheme pairs (kMxfp8Static or
    kMxfp4Static, kMxfp8Dynamic) of [HUM, _supports_quant_scheme]).

    a_codes uint8 [m, C] e4m3fn, a_exps uint8 [m, C/32]; w_codes uint8 [n, C]
    e4m3fn or [n, C/2] packed e2m1 (fp4), w_exps uint8 [n, C/32].  Result in
    fp64; the block sums are exact (at most 8-bit products, 32 terms).
    """
    a = e4m3_decode(a_codes)
    w = e2m1_decode(unpack_fp4(w_codes)) if fp4 else e4m3_decode(w_codes)
    m, C = a.shape
    n = w.shape[0]
    G = C // 32
    a_b = a.reshape(m, G, 32).transpose(1, 0, 2)            # [G, m, 32]
    w_b = w.reshape(n, G, 32).transpose(1, 2, 0)            # [G, 32, n]
    partial = np.matmul(a_b, w_b)                           # [G, m, n], exact
    sa = ue8m0_decode(a_exps)                               # [m, G]
    sw = ue8m0_decode(w_exps)                               # [n, G]
    out = np.zeros((m, n), dtype=np.float64)
    for b in range(G):
        out += partial[b] * sa[:, b:b + 1] * sw[None, :, b]
    return out


def bf16_gemm_f64(a_bits, w_codes, w_scale) -> np.ndarray:
    """out[m, n] = sum_b w_scale[n // 128, b] * sum_{c in block b} a[m, c] * w[n, c]
    with bf16 activations (the (kFp8Static128BlockSym, None) scheme pair).

    a_bits uint16 [m, C] (bf16), w_codes uint8 [n, C] (e4m3fn), w_scale fp32
    [n/128, C/128].  Result in fp64; each product is exact, the sums are
    fp64 sums."""
    a = bf16_to_f64(a_bits)
    w = e4m3_decode(w_codes)
    m, C = a.shape
    n = w.shape[0]
    G = C // GROUP
    a_b = a.reshape(m, G, GROUP).transpose(1, 0, 2)          # [G, m, 128]
    w_b = w.reshape(n, G, GROUP).transpose(1, 2, 0)          # [G, 128, n]
    partial = np.matmul(a_b, w_b)                            # [G, m, n]
    ws = np.repeat(np.asarray(w_scale, np.float64), GROUP, axis=0)  # [n, G]
    out = np.zeros((m, n), dtype=np.float64)
    for b in range(G):
        out += partial[b] * ws[None, :, b]
    return out


# ---------------------------------------------------------------------------
# scheme selection
# ---------------------------------------------------------------------------

def act_group(cfg) -> int:
    """Activation quantization group: 32 for MXFP8, else 128."""
    return 32 if cfg.act_quant == "mxfp8" else GROUP


def act_e8m0(cfg) -> bool:
    """Activation scales are E8M0 exponent bytes (else fp32)."""
    return cfg.act_quant in ("ue8m0", "mxfp8")


def expert_gemm(cfg, a_codes, a_stored, w, w_sf) -> np.ndarray:
    """One expert's GEMM in the workload's scheme (fp64, before rounding).
    bf16 activations: a_codes holds their bits and a_stored is unused."""
    if cfg.act_quant == "bf16":
        return bf16_gemm_f64(a_codes, w, w_sf)
    if cfg.weight_quant == "fp8_block128":
        return block_scaled_gemm_f64(a_codes, scale_values(a_stored, act_e8m0(cfg)), w, w_sf)
    return mx_gemm_f64(a_codes, a_stored, w, w_sf, fp4=cfg.weight_quant == "mxfp4")


# ---------------------------------------------------------------------------
# O6: activation, re-quantized  [HUM, process_input('w2', activation=...);
# HUM2, HummingExpertsBase._supports_activation and get_buffer_metas: the
# activation list, and the w2 input width N for gated activations, the whole
# w13 output for the _NO_MUL ones]
# ---------------------------------------------------------------------------

def _erf(x: np.ndarray) -> np.ndarray:
    return np.vectorize(math.erf, otypes=[np.float64])(x)


# The activation functions by name.  The pages list them (the activation
# enum members the experts accept) without their formulas; these are the
# standard definitions: SiLU x*sigmoid(x); GELU x*Phi(x) with the exact
# normal CDF; GELU_TANH its tanh approximation with sqrt(2/pi) and 0.044715;
# RELU2 max(x, 0)^2.
ACT_FUNCS = {
    "silu": lambda x: x / (1.0 + np.exp(-x)),
    "gelu": lambda x: 0.5 * x * (1.0 + _erf(x / math.sqrt(2.0))),
    "gelu_tanh": lambda x: 0.5 * x * (1.0 + np.tanh(math.sqrt(2.0 / math.pi)
                                                    * (x + 0.044715 * x ** 3))),
    "relu2": lambda x: np.maximum(x, 0.0) ** 2,
}
GATED = ("silu", "gelu", "gelu_tanh", "swigluoai", "swiglustep")
NO_MUL = ("silu_no_mul", "gelu_no_mul", "gelu_tanh_no_mul", "relu2_no_mul")
SWIGLU_DEFAULT_LIMIT = 7.0
SWIGLUOAI_ALPHA = 1.702


def gated_act(activation: str, g, u, limit: float = 0.0):
    """h = F(g, u) for a gated activation with gate g and up u (fp64).
    ``limit`` > 0 clamps as described in the module docstring (SiLU: only
    when given; SWIGLUOAI / SWIGLUSTEP: 7 when 0)."""
    if activation in ("gelu", "gelu_tanh") or (activation == "silu" and limit <= 0):
        return ACT_FUNCS[activation](g) * u
    L = limit if limit > 0 else SWIGLU_DEFAULT_LIMIT
    uc = np.clip(u, -L, L)
    if activation == "silu":
        return ACT_FUNCS["silu"](np.minimum(g, L)) * uc
    if activation == "swiglustep":
        return np.minimum(ACT_FUNCS["silu"](g), L) * uc
    assert activation == "swigluoai", activation
    gc = np.minimum(g, L)
    return (uc + 1.0) * gc / (1.0 + np.exp(-SWIGLUOAI_ALPHA * gc))


def act_f32(gate_up_bits, N: int, activation: str = "silu", limit: float = 0.0) -> np.ndarray:
    """The w2 input before quantization, in fp64 rounded once to fp32.
    Gated: bf16 [rows, 2N] -> h = F(g, u) with g = columns [0, N) and
    u = columns [N, 2N).  _no_mul: bf16 [rows, N] -> h = f(x)."""
    gu = bf16_to_f64(gate_up_bits)
    if activation in GATED:
        h = gated_act(activation, gu[:, :N], gu[:, N:2 * N], limit)
    else:
        assert activation in NO_MUL, activation
        h = ACT_FUNCS[activation[:-len("_no_mul")]](gu[:, :N])
    return h.astype(np.float32)


def silu_mul_f32(gate_up_bits, N: int) -> np.ndarray:
    return act_f32(gate_up_bits, N, "silu")


def act_requant(gate_up_bits, N: int, ue8m0: bool, group: int = GROUP,
                activation: str = "silu", limit: float = 0.0):
    return quantize_groups(act_f32(gate_up_bits, N, activation, limit), ue8m0, group)


def act_bf16(gate_up_bits, N: int, activation: str = "silu", limit: float = 0.0):
    """Unquantized w2 input: h (fp32, as above) rounded once to bf16 (the
    c_dtype of the activation buffer)."""
    return bf16_round(act_f32(gate_up_bits, N, activation, limit).astype(np.float64))


def act_step(cfg, gate_up_bits):
    """The w2 input in the workload's scheme: (codes or bf16 bits, scales or
    None)."""
    act = getattr(cfg, "activation", "silu")
    limit = getattr(cfg, "act_limit", 0.0)
    if cfg.act_quant == "bf16":
        return act_bf16(gate_up_bits, cfg.N, act, limit), None
    return act_requant(gate_up_bits, cfg.N, act_e8m0(cfg), act_group(cfg), act, limit)


# ---------------------------------------------------------------------------
# O8: top-k weighted reduce  [HUM, HummingGroupedExperts.apply: moe_unpermute;
# HummingIndexedExperts.apply: moe_fused_mul_sum; router weight applied after
# w2 since apply_router_weight_on_input is False]
# ---------------------------------------------------------------------------

def topk_reduce(down_bits, slot_row, weights) -> np.ndarray:
    """out[t] = bf16(sum over slots j with slot_row[t, j] >= 0, ascending j,
    of weights[t, j] * down[slot_row[t, j]]), accumulated in fp64."""
    slot_row = np.asarray(slot_row, dtype=np.int64)
    T, k = slot_row.shape
    down = bf16_to_f64(down_bits)
    acc = np.zeros((T, down.shape[1]), dtype=np.float64)
    for j in range(k):
        r = slot_row[:, j]
        ok = r >= 0
        acc[ok] += np.asarray(weights, np.float64)[ok, j:j + 1] * down[r[ok]]
    return bf16_round(acc)


# ---------------------------------------------------------------------------
# The whole layer
# ---------------------------------------------------------------------------

def _np(x):
    if x is None:
        return None
    if hasattr(x, "detach"):
        x = x.detach().to("cpu")
        if str(x.dtype) == "torch.bfloat16":
            return x.view(__import__("torch").int16).numpy().view(np.uint16)
        return x.numpy()
    return np.asarray(x)


def host_inputs(inp: dict) -> dict:
    """Host numpy copies of a generator input dict (bf16 as uint16 bits)."""
    out = {}
    for key, val in inp.items():
        if key == "eplb" and val is not None:
            out[key] = {k2: _np(v2) for k2, v2 in val.items()}
        elif key == "cfg":
            out[key] = val
        else:
            out[key] = _np(val)
    return out


def stage(h: dict):
    """Steps 1-2: quantize the hidden rows that will be read, repack the
    routing and build the expert layout."""
    cfg = h["cfg"]
    ue8m0, grp = act_e8m0(cfg), act_group(cfg)
    ids, w, load = repack_topk(h["topk_ids"], h["topk_weights"], h["is_padding"],
                               h["eplb"], num_physical=cfg.E)
    batched = cfg.layout == "batched"
    lay = route_layout(ids, cfg.E, cfg.max_tokens if batched else 0)
    hid = np.asarray(h["hidden"]).reshape(-1, cfg.K)
    if batched:
        # only rows below each slab's count exist; the rest are never read
        valid_rows = np.concatenate(
            [np.arange(e * cfg.max_tokens, e * cfg.max_tokens + int(c))
             for e, c in enumerate(np.asarray(h["expert_num_tokens"]))]
            + [np.zeros(0, dtype=np.int64)]).astype(np.int64)
    else:
        valid_rows = np.arange(hid.shape[0])
    if cfg.act_quant == "bf16":
        # staging copies the hidden states unquantized ([STAGE]: no hidden_quant)
        x_q = np.zeros(hid.shape, dtype=np.uint16)
        x_q[valid_rows] = hid[valid_rows]
        return {"ids": ids, "weights": w, "load": load, "x_q": x_q, "x_sf": None, **lay}
    G = cfg.K // grp
    x_q = np.zeros(hid.shape, dtype=np.uint8)
    x_sf = np.zeros((hid.shape[0], G), dtype=np.uint8 if ue8m0 else np.float32)
    x = bf16_to_f64(hid[valid_rows]).astype(np.float32)
    x_q[valid_rows], x_sf[valid_rows] = quantize_groups(x, ue8m0, grp)
    return {"ids": ids, "weights": w, "load": load, "x_q": x_q, "x_sf": x_sf,
            **lay}


def forward(h: dict) -> dict:
    """The full layer on every row; returns every intermediate.

    Rows: contiguous layout -> M = offsets[E] permuted rows; batched layout
    -> E * max_tokens rows of which only the first counts[e] of each slab
    are computed (the rest stay 0 here and are never compared)."""
    cfg = h["cfg"]
    ue8m0, grp = act_e8m0(cfg), act_group(cfg)
    st = stage(h)
    E, N, K = cfg.E, cfg.N, cfg.K
    batched = cfg.layout == "batched"
    counts = st["counts"]
    if batched:
        given = np.asarray(h["expert_num_tokens"]).astype(np.int32)
        assert np.array_equal(given, counts), "staged counts disagree with routing"
        rows_total = E * cfg.max_tokens
    else:
        rows_total = int(st["offsets"][-1])
    bf16_act = cfg.act_quant == "bf16"
    gate_up = np.zeros((rows_total, cfg.w13_rows), dtype=np.uint16)
    a2_q = np.zeros((rows_total, N), dtype=np.uint16 if bf16_act else np.uint8)
    a2_sf = None if bf16_act else np.zeros((rows_total, N // grp),
                                           dtype=np.uint8 if ue8m0 else np.float32)
    down = np.zeros((rows_total, K), dtype=np.uint16)
    for e in range(E):
        n_e = int(counts[e])
        if n_e == 0:
            continue
        if batched:
            rows = np.arange(e * cfg.max_tokens, e * cfg.max_tokens + n_e)
            a_rows = rows
        else:
            lo = int(st["offsets"][e])
            rows = np.arange(lo, lo + n_e)
            a_rows = st["row_src"][rows]
        x_sf = None if st["x_sf"] is None else st["x_sf"][a_rows]
        gu = expert_gemm(cfg, st["x_q"][a_rows], x_sf, h["w13"][e], h["w13_sf"][e])
        gate_up[rows] = bf16_round(gu)
        q2, s2 = act_step(cfg, gate_up[rows])
        a2_q[rows] = q2
        if s2 is not None:
            a2_sf[rows] = s2
        dn = expert_gemm(cfg, q2, s2, h["w2"][e], h["w2_sf"][e])
        down[rows] = bf16_round(dn)
    out = topk_reduce(down, st["slot_row"], st["weights"])
    return {**st, "gate_up": gate_up, "a2_q": a2_q, "a2_sf": a2_sf,
            "down": down, "out": out}


def forward_indexed(h: dict, block_size: int) -> dict:
    """The layer in the indexed layout ([HUM] HummingIndexedExperts.apply and
    prepare_humming_moe_kwargs): align, w13 on the rows of sorted_ids
    (activation row = id // top_k) written to row id of an intermediate in
    (token, slot) order, the activation, w2 on that intermediate (top_k 1:
    row id) written back to row id, then the fused mul-sum.  Per row the
    arithmetic is the contiguous layout's, so the output must be identical."""
    cfg = h["cfg"]
    assert cfg.layout != "batched"
    st = stage(h)
    E, N, K, k = cfg.E, cfg.N, cfg.K, cfg.top_k
    sorted_ids, expert_ids, P = align_block_size(st["ids"], E, block_size)
    numel = cfg.T * k
    bf16_act = cfg.act_quant == "bf16"
    a2_rows = np.zeros((numel, N), dtype=np.uint16 if bf16_act else np.uint8)
    down = np.zeros((numel, K), dtype=np.uint16)
    for b, e in enumerate(expert_ids):
        pos = np.arange(b * block_size, (b + 1) * block_size)
        ids_b = sorted_ids[pos]
        live = ids_b < numel
        if not live.any():
            continue
        slots = ids_b[live]
        tokens = slots // k
        x_sf = None if st["x_sf"] is None else st["x_sf"][tokens]
        gu = bf16_round(expert_gemm(cfg, st["x_q"][tokens], x_sf, h["w13"][e], h["w13_sf"][e]))
        q2, s2 = act_step(cfg, gu)
        a2_rows[slots] = q2
        dn = expert_gemm(cfg, q2, s2, h["w2"][e], h["w2_sf"][e])
        down[slots] = bf16_round(dn)
    out = fused_mul_sum(down, st["ids"], st["weights"], E)
    return {"sorted_ids": sorted_ids, "expert_ids": expert_ids, "num_tokens_padded": P,
            "down": down, "out": out}


def forward_tokens(h: dict, tokens, st: dict | None = None) -> dict:
    """The layer for a few tokens only (for full-size workloads).

    Computes the routing layout for all tokens (cheap), then for each chosen
    token t and each of its routed slots the rows gate_up, a2 and down at the
    row the layout gives, and the token's output row.  Returns
    ``{"stage": st, "rows": {row: {...}}, "out": {t: bf16 bits [K]}}``.
    """
    cfg = h["cfg"]
    ue8m0, grp = act_e8m0(cfg), act_group(cfg)
    N, K = cfg.N, cfg.K
    if st is None:
        st = stage_routing_only(h)
    rows_info = {}
    by_expert = {}
    for t in tokens:
        for j in range(cfg.top_k):
            r = int(st["slot_row"][t, j])
            if r >= 0:
                by_expert.setdefault(int(st["ids"][t, j]), []).append((t, j, r))
    hid = h["hidden"].reshape(-1, K)
    for e, lst in sorted(by_expert.items()):
        w13, w13s, w2, w2s = h["w13"][e], h["w13_sf"][e], h["w2"][e], h["w2_sf"][e]
        if hasattr(w13, "detach"):
            w13, w13s, w2, w2s = _np(w13), _np(w13s), _np(w2), _np(w2s)
        for (t, j, r) in lst:
            a_row = r if cfg.layout == "batched" else t
            if cfg.act_quant == "bf16":
                xq, xsf = hid[a_row:a_row + 1].copy(), None
            else:
                x = bf16_to_f64(hid[a_row:a_row + 1]).astype(np.float32)
                xq, xsf = quantize_groups(x, ue8m0, grp)
            gu = bf16_round(expert_gemm(cfg, xq, xsf, w13, w13s))
            q2, s2 = act_step(cfg, gu)
            dn = bf16_round(expert_gemm(cfg, q2, s2, w2, w2s))
            rows_info[r] = {"token": t, "slot": j, "expert": e, "x_q": xq[0],
                            "x_sf": None if xsf is None else xsf[0], "gate_up": gu[0],
                            "a2_q": q2[0], "a2_sf": None if s2 is None else s2[0],
                            "down": dn[0]}
    outs = {}
    for t in tokens:
        acc = np.zeros(K, dtype=np.float64)
        for j in range(cfg.top_k):
            r = int(st["slot_row"][t, j])
            if r >= 0:
                acc += np.float64(st["weights"][t, j]) * bf16_to_f64(rows_info[r]["down"])
        outs[t] = bf16_round(acc)
    return {"stage": st, "rows": rows_info, "out": outs}


def stage_routing_only(h: dict) -> dict:
    """Routing repack and layout without quantizing any hidden row."""
    cfg = h["cfg"]
    ids, w, load = repack_topk(h["topk_ids"], h["topk_weights"], h["is_padding"],
                               h["eplb"], num_physical=cfg.E)
    lay = route_layout(ids, cfg.E, cfg.max_tokens if cfg.layout == "batched" else 0)
    return {"ids": ids, "weights": w, "load": load, **lay}
