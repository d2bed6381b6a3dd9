"""Comparison metrics and device plumbing for the GPU parity tests.

Tolerances (derived in the design notes from the arithmetic):
  * quantized bytes, scale exponents, routing metadata: bit-exact;
  * grouped-GEMM bf16 outputs: |gpu - oracle| <= one bf16 unit of the
    oracle's value + 2^-11 * S_abs, where S_abs = sum over k of
    |sa * sw * a * w| (the oracle's GEMM on absolute values).  The second
    term bounds the fp8 MFMA's own accumulation error: a measured
    v_mfma_f32_16x16x128_f8f6f4 misses the exact 128-term sum by up to
    2^-12.3 (mean 2^-15.8) of the sum of |products|; and the relative
    Frobenius difference is at most 2^-8.  At most GEMM_DIFF_CEIL of the
    bf16 outputs may differ from the oracle's at all (measured 1-2 %: the
    MFMA error moves a value across a bf16 rounding boundary only when it
    sits close to one);
  * re-quantized fp8 activations, from the oracle's own gate_up: at most
    1 ULP (sign-magnitude ordinal, +-0 equal) in at most 0.1% of elements;
    a UE8M0 exponent may differ only where amax/448 is within 2^-20
    (relative) of a power of two; fp32 scales within 2^-21 relative;
  * re-quantized fp8 activations at the end of the GPU's own chain: each
    value within half an fp8 step on each side plus the GEMM bound above
    carried through silu(g) * u; at most CHAIN_DIFF_CEIL of the codes
    differ, and at most CHAIN_MULTI_ULP_CEIL of them by more than 1 ULP
    (measured about 0.003 %: only where g or u is a sum with heavy
    cancellation, whose MFMA error bound, relative to the sum of |products|,
    spans several fp8 steps of the small result).  The pages' 1-ULP,
    0.1 % bar holds for the activation step in isolation (check_requant);
    at the end of the chain the gate_up inputs themselves already differ in
    1-2 % of elements by one bf16 unit (fp8 MFMA accumulation), and a
    2^-8 relative move flips an fp8 code (2^-3 relative steps) with
    probability about 2^-4 per moved input, so about 0.2 % of codes differ;
  * final output: relative Frobenius <= 1e-2, max |diff| <= 2e-2 * max |ref|.
"""
import numpy as np
import torch

from oracle import moe_oracle as O


def to_np(t):
    """Device or host tensor -> numpy (bf16 as uint16 bits)."""
    t = t.detach().to("cpu")
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def to_dev(a, dtype=None, device="cuda"):
    """numpy -> device tensor; uint16 arrays become bf16."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    t = torch.from_numpy(a)
    if dtype is not None:
        t = t.to(dtype)
    return t.to(device)


def bf16_ulp(x64):
    """Spacing of bf16 numbers at |x| (normal range)."""
    a = np.maximum(np.abs(x64), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(a)) - 7)


def check_bf16_close(got_bits, ref_bits, what, max_frac=0.01):
    g = O.bf16_to_f64(got_bits)
    r = O.bf16_to_f64(ref_bits)
    assert g.shape == r.shape, what
    assert np.all(np.isfinite(g)), f"{what}: non-finite values"
    d = np.abs(g - r)
    rowmax = np.abs(r).max(axis=-1, keepdims=True) if r.ndim > 1 else np.abs(r).max()
    tol = np.maximum(bf16_ulp(r), rowmax * 2.0 ** -14)
    bad = d > tol * 1.0000001
    assert not bad.any(), (f"{what}: {bad.sum()} elements beyond one bf16 unit, "
                           f"worst {d[bad].max() if bad.any() else 0}")
    frac = np.count_nonzero(d) / max(d.size, 1)
    assert frac <= max_frac, f"{what}: {frac:.4%} of elements differ"
    return frac


def fp8_ordinal(codes):
    c = codes.astype(np.int32)
    mag = c & 0x7F
    return np.where(c & 0x80, -mag, mag)


MFMA_REL = 2.0 ** -11
# ceilings on the fraction of differing elements (see the module docstring)
GEMM_DIFF_CEIL = 0.04
CHAIN_DIFF_CEIL = 0.003
CHAIN_MULTI_ULP_CEIL = 1e-4


def abs_gemm(a_codes, a_scale, w_codes, w_sf):
    """S_abs: the oracle's block-scaled GEMM on absolute values."""
    return O.block_scaled_gemm_f64(np.asarray(a_codes) & 0x7F, np.abs(a_scale),
                                   np.asarray(w_codes) & 0x7F, np.abs(np.asarray(w_sf)))


def abs_gemm_cfg(cfg, a_codes, a_stored, w_codes, w_sf):
    """S_abs in the workload's scheme: bf16 activations, block fp8 (scale
    values) or MX (E8M0 bytes on both operands; e2m1 sign bits cleared nibble
    by nibble)."""
    if cfg.act_quant == "bf16":
        return O.bf16_gemm_f64(np.asarray(a_codes) & 0x7FFF, np.asarray(w_codes) & 0x7F,
                               np.abs(np.asarray(w_sf)))
    if cfg.weight_quant == "fp8_block128":
        return abs_gemm(a_codes, O.scale_values(a_stored, O.act_e8m0(cfg)), w_codes, w_sf)
    fp4 = cfg.weight_quant == "mxfp4"
    return O.mx_gemm_f64(np.asarray(a_codes) & 0x7F, a_stored,
                         np.asarray(w_codes) & (0x77 if fp4 else 0x7F), w_sf, fp4)


def within_rate(count, size, rate):
    """count <= what a rate ceiling allows on ``size`` elements, with a
    3-sigma Poisson allowance so that a handful of sampled rows is judged by
    the same rate as a whole layer."""
    lam = rate * size
    return count <= lam + 3.0 * np.sqrt(lam)


def check_gemm(got_bits, ref_bits, s_abs, what, max_frac=GEMM_DIFF_CEIL):
    g = O.bf16_to_f64(got_bits)
    r = O.bf16_to_f64(ref_bits)
    assert g.shape == r.shape == s_abs.shape, what
    assert np.all(np.isfinite(g)), f"{what}: non-finite values"
    d = np.abs(g - r)
    tol = bf16_ulp(r) + MFMA_REL * s_abs
    bad = d > tol
    assert not bad.any(), (f"{what}: {bad.sum()} elements beyond the bound, worst excess "
                           f"{(d - tol)[bad].max():.3e}")
    den = np.linalg.norm(r)
    rel = np.linalg.norm(d) / den if den > 0 else 0.0
    assert rel <= 2.0 ** -8, f"{what}: relative Frobenius difference {rel:.3e}"
    ndiff = np.count_nonzero(d)
    frac = ndiff / max(d.size, 1)
    if max_frac is not None:
        assert within_rate(ndiff, d.size, max_frac), \
            f"{what}: {frac:.3%} of bf16 outputs differ (> {max_frac:.1%})"
    return frac


def _fp8_step(v_over_s):
    """Spacing of e4m3fn values at |v| (in scale units)."""
    return np.exp2(np.floor(np.log2(np.maximum(np.abs(v_over_s), 2.0 ** -6))) - 3)


def check_requant(got_q, got_sf, ref_q, ref_sf, ref_h32, ue8m0, what, group=128):
    """Isolation: the GPU re-quantized the oracle's own gate_up (groups of
    ``group`` columns).  <= 1 ULP in <= 0.1% of the elements."""
    rows, N = ref_q.shape
    G = N // group
    got_sf = got_sf[:, :G]
    ref_sf = ref_sf[:, :G]
    ulp = np.abs(fp8_ordinal(got_q) - fp8_ordinal(ref_q))
    if ue8m0:
        diff_e = got_sf.astype(int) != ref_sf.astype(int)
        if diff_e.any():
            amax = np.abs(ref_h32.reshape(rows, G, group)).max(axis=2).astype(np.float64)
            s = np.maximum(amax, np.float32(1e-4)) / 448.0
            near = np.abs(np.log2(s) - np.round(np.log2(s))) < 2.0 ** -20 * 1.5
            assert np.all(near[diff_e]), f"{what}: exponent differs away from a power of two"
            # those groups: compare values at the coarser of the two scales
            sv_g = np.repeat(O.scale_values(got_sf, True), group, axis=1)
            sv_r = np.repeat(O.scale_values(ref_sf, True), group, axis=1)
            vg = O.e4m3_decode(got_q) * sv_g
            vr = O.e4m3_decode(ref_q) * sv_r
            coarse = np.maximum(sv_g, sv_r)
            d = np.abs(vg - vr)
            by_value = np.where(d == 0, 0, np.where(d <= _fp8_step(vr / coarse) * coarse, 1, 2))
            ulp = np.where(np.repeat(diff_e, group, axis=1), by_value, ulp)
    else:
        rel = np.abs(got_sf.astype(np.float64) - ref_sf.astype(np.float64)) / ref_sf
        assert rel.max() <= 2.0 ** -21, f"{what}: fp32 scales differ by {rel.max():.3e}"
    assert ulp.max() <= 1, f"{what}: {np.count_nonzero(ulp > 1)} codes off by more than 1 ULP"
    frac = np.count_nonzero(ulp) / ulp.size
    assert frac <= 1e-3, f"{what}: {frac:.4%} of codes differ"
    return frac


def act_error_bound(ref_gate_up_bits, s_abs_gate_up, N, activation="silu", limit=0.0):
    """(h, dh): the oracle's h in fp64 and a bound on how far h moves when
    gate_up moves by the GEMM bound (bf16 unit + MFMA term), for the given
    activation.  SiLU uses its derivative; f(g) * u forms the largest change
    of f over [g - dg, g + dg] sampled at eight points; the clamped SwiGLU
    forms the largest change of F(g, u) over the box [g +- dg] x [u +- du]
    sampled on a 5 x 5 grid (clamps make F piecewise smooth; the grid holds
    the box's corners); both with a 25 % margin for the curvature between
    samples."""
    gu = O.bf16_to_f64(ref_gate_up_bits)
    dgu = bf16_ulp(gu) + MFMA_REL * s_abs_gate_up
    gated = activation in O.GATED
    g, dg = gu[:, :N], dgu[:, :N]
    u, du = (gu[:, N:2 * N], dgu[:, N:2 * N]) if gated else (np.ones_like(g), np.zeros_like(g))
    if activation in ("swigluoai", "swiglustep") or (activation == "silu" and limit > 0):
        F0 = O.gated_act(activation, g, u, limit)
        dh = np.zeros_like(g)
        for tg in (-1.0, -0.5, 0.0, 0.5, 1.0):
            for tu in (-1.0, -0.5, 0.0, 0.5, 1.0):
                dh = np.maximum(dh, np.abs(O.gated_act(activation, g + tg * dg, u + tu * du,
                                                       limit) - F0))
        dh = dh * 1.25 * 1.01 + np.abs(F0) * 2.0 ** -20 + 2.0 ** -40
        return F0, dh
    if activation == "silu":
        sig = 1.0 / (1.0 + np.exp(-g))
        f = g * sig
        sens = np.abs(sig * (1.0 + g * (1.0 - sig))) * dg
    else:
        fn = O.ACT_FUNCS[activation.replace("_no_mul", "")]
        f = fn(g)
        sens = np.zeros_like(g)
        for t in (-1.0, -0.75, -0.5, -0.25, 0.25, 0.5, 0.75, 1.0):
            sens = np.maximum(sens, np.abs(fn(g + t * dg) - f))
        sens *= 1.25
    dh = (sens * np.abs(u) + np.abs(f) * du + 1.1 * sens * du) * 1.01
    h = f * u
    dh += np.abs(h) * 2.0 ** -20 + 2.0 ** -40
    return h, dh


def check_requant_chain(got_q, got_sf, ref_q, ref_sf, ref_gate_up_bits, s_abs_gate_up, ue8m0,
                        what, group=128, activation="silu", max_frac=CHAIN_DIFF_CEIL,
                        limit=0.0):
    """End of the GPU's own chain: its gate_up may differ from the oracle's
    by the GEMM bound; carry that through the activation and allow half an
    fp8 step of rounding on each side.  At most ``max_frac`` of the codes
    differ and at most CHAIN_MULTI_ULP_CEIL of them, among groups where both
    sides chose the same scale, by more than 1 ULP (None: not checked).
    Returns the fraction of codes that differ."""
    rows, N = ref_q.shape
    G = N // group
    _, dh = act_error_bound(ref_gate_up_bits, s_abs_gate_up, N, activation, limit)
    sv_g = np.repeat(O.scale_values(got_sf[:, :G], ue8m0), group, axis=1)
    sv_r = np.repeat(O.scale_values(ref_sf[:, :G], ue8m0), group, axis=1)
    vg = O.e4m3_decode(got_q) * sv_g
    vr = O.e4m3_decode(ref_q) * sv_r
    assert np.all(np.isfinite(vg)), f"{what}: non-finite codes"
    bound = 0.5 * (_fp8_step(vg / sv_g) * sv_g + _fp8_step(vr / sv_r) * sv_r) + dh
    bad = np.abs(vg - vr) > bound * 1.000001
    assert not bad.any(), f"{what}: {bad.sum()} values beyond the propagated bound"
    if ue8m0:
        assert np.abs(got_sf[:, :G].astype(int) - ref_sf[:, :G].astype(int)).max() <= 1
        same = np.repeat(got_sf[:, :G] == ref_sf[:, :G], group, axis=1)
    else:
        same = np.repeat(got_sf[:, :G].view(np.uint32) == ref_sf[:, :G].view(np.uint32),
                         group, axis=1)
    multi = np.count_nonzero(same & (np.abs(fp8_ordinal(got_q) - fp8_ordinal(ref_q)) > 1))
    ndiff = np.count_nonzero(got_q != ref_q)
    frac = ndiff / got_q.size
    if max_frac is not None:
        assert within_rate(ndiff, got_q.size, max_frac), \
            f"{what}: {frac:.3%} of a2 codes differ (> {max_frac:.2%})"
        assert within_rate(multi, got_q.size, CHAIN_MULTI_ULP_CEIL), \
            f"{what}: {multi} codes ({multi / got_q.size:.4%}) more than 1 ULP apart"
    return frac


def check_bf16_act_chain(got_bits, ref_bits, ref_gate_up_bits, s_abs_gate_up, what,
                         activation="silu", limit=0.0):
    """bf16 w2 input at the end of the GPU's own chain: the GEMM bound on
    gate_up carried through the activation, plus one bf16 rounding on each
    side.  Returns the fraction of values that differ."""
    N = ref_bits.shape[1]
    h, dh = act_error_bound(ref_gate_up_bits, s_abs_gate_up, N, activation, limit)
    vg, vr = O.bf16_to_f64(got_bits), O.bf16_to_f64(ref_bits)
    assert np.all(np.isfinite(vg)), f"{what}: non-finite values"
    bound = dh + bf16_ulp(vr)
    bad = np.abs(vg - vr) > bound * 1.000001
    assert not bad.any(), f"{what}: {bad.sum()} values beyond the propagated bound"
    return np.count_nonzero(got_bits != ref_bits) / got_bits.size


def check_output(got_bits, ref_bits, what):
    g = O.bf16_to_f64(got_bits)
    r = O.bf16_to_f64(ref_bits)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    den = np.linalg.norm(r)
    rel = np.linalg.norm(g - r) / den if den > 0 else np.linalg.norm(g)
    mx = np.abs(g - r).max() if g.size else 0.0
    ref_max = np.abs(r).max() if r.size else 0.0
    assert rel <= 1e-2, f"{what}: relative Frobenius {rel:.3e}"
    assert mx <= 2e-2 * ref_max + (0 if ref_max > 0 else 1e-30), f"{what}: max abs {mx:.3e}"
    return rel, mx
