"""Pins of the CPU oracle to things other than itself.

Each test checks an oracle function against exact rational arithmetic, a
closed form, a library routine, brute force on tiny inputs, or an invariant
the vLLM pages fix ("vllm.model_executor.layers.fused_moe.prepare_megamoe":
``_quantize_fp8_groups`` / ``_store_topk``; "...experts.fused_humming_moe":
the experts' ``apply`` methods).  No GPU is needed.
"""
import bisect
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import moe_synth
from oracle import moe_oracle as O


# --------------------------------------------------------------------------
# helpers written from scratch for the pins (exact rationals)
# --------------------------------------------------------------------------

def _frac_e4m3_values():
    """The finite non-negative e4m3fn values as Fractions, code order."""
    vals = []
    for code in range(0x7F):
        e, m = code >> 3, code & 7
        if e == 0:
            vals.append(Fraction(m, 512))
        else:
            vals.append(Fraction(8 + m, 8) * Fraction(2) ** (e - 7))
    return vals


_FV = _frac_e4m3_values()


def _frac_encode(x: Fraction, negative: bool) -> int:
    """Nearest e4m3fn code by exact comparison; ties -> even code; above the
    largest finite value -> saturate."""
    a = abs(x)
    i = bisect.bisect_left(_FV, a)
    if i == 0:
        code = 0
    elif i >= len(_FV):
        code = 0x7E
    else:
        lo, hi = i - 1, i
        dl, dh = a - _FV[lo], _FV[hi] - a
        if dl < dh:
            code = lo
        elif dh < dl:
            code = hi
        else:
            code = lo if lo % 2 == 0 else hi
    return code | (0x80 if negative else 0)


def _frac_bf16(x: Fraction) -> Fraction:
    """Nearest bf16 value (8 significant bits), ties to even, normal range."""
    if x == 0:
        return Fraction(0)
    sgn = -1 if x < 0 else 1
    a = abs(x)
    e = math.floor(math.log2(a.numerator) - math.log2(a.denominator))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    q = Fraction(2) ** (e - 7)
    n = a / q
    fl = math.floor(n)
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sgn * fl * q


def _frac_f32(x: Fraction) -> Fraction:
    """Nearest binary32 value (24 significant bits), ties to even, for x in
    the normal range (the pins below keep every intermediate there)."""
    if x == 0:
        return Fraction(0)
    sgn = -1 if x < 0 else 1
    a = abs(x)
    e = math.floor(math.log2(a.numerator) - math.log2(a.denominator))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    assert -126 <= e <= 127, "outside binary32's normal range"
    q = Fraction(2) ** (e - 23)
    n = a / q
    fl = math.floor(n)
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sgn * fl * q


def _ceil_log2(r: Fraction) -> int:
    """Smallest integer j with 2^j >= r (r > 0), exactly."""
    j = math.floor(math.log2(r.numerator) - math.log2(r.denominator)) - 2
    while Fraction(2) ** j < r:
        j += 1
    while Fraction(2) ** (j - 1) >= r:
        j -= 1
    return j


# --------------------------------------------------------------------------
# e4m3fn codec
# --------------------------------------------------------------------------

def test_e4m3_table_spec_points():
    V = O.E4M3_VALUES
    assert V[0x7E] == 448.0
    assert V[0x01] == 2.0 ** -9
    assert V[0x07] == 7 * 2.0 ** -9
    assert V[0x08] == 2.0 ** -6
    assert V[0x38] == 1.0
    assert V[0x00] == 0.0 and not np.signbit(V[0x00])
    assert V[0x80] == 0.0 and np.signbit(V[0x80])
    assert np.isnan(V[0x7F]) and np.isnan(V[0xFF])
    assert np.all(np.diff(V[:0x7F]) > 0)
    assert np.array_equal(V[0x80:0xFF], -V[0x00:0x7F])
    assert np.isfinite(V).sum() == 254


def test_e4m3_table_matches_torch_decode():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    fin = np.isfinite(ref)
    assert np.array_equal(fin, np.isfinite(O.E4M3_VALUES))
    assert np.array_equal(ref[fin], O.E4M3_VALUES[fin])


def test_e4m3_encode_roundtrip_all_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = O.E4M3_VALUES[codes].astype(np.float32)
    assert np.array_equal(O.e4m3_encode(vals), codes)


def _midpoints_and_neighbours():
    v = O.E4M3_VALUES[:0x7F]
    mids = ((v[:-1] + v[1:]) / 2).astype(np.float32)        # exact in fp32
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(0))
    return np.concatenate([mids, up, dn])


def test_e4m3_encode_exact_rationals():
    rng = np.random.default_rng(11)
    logs = rng.uniform(-14, 9.2, 4000)
    xs = (rng.choice([-1, 1], 4000) * np.exp2(logs)).astype(np.float32)
    xs = np.concatenate([xs, _midpoints_and_neighbours(),
                         np.float32([448, 456, 460, 463.99, 464, 465, 1e6,
                                     2.0 ** -10, 2.0 ** -11, 3 * 2.0 ** -11, 0.0,
                                     -0.0])])
    got = O.e4m3_encode(xs)
    want = np.array([_frac_encode(Fraction(float(x)), bool(np.signbit(x)))
                     for x in xs], np.uint8)
    assert np.array_equal(got, want)


def test_e4m3_encode_matches_torch_cast_in_range():
    rng = np.random.default_rng(12)
    xs = (rng.standard_normal(200000) * np.exp2(rng.uniform(-12, 8, 200000)))
    xs = np.clip(xs, -448, 448).astype(np.float32)
    xs = np.concatenate([xs, _midpoints_and_neighbours()])
    ref = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.e4m3_encode(xs), ref)


def test_e4m3_encode_saturates_and_nan():
    xs = np.float32([449.0, 1e30, np.inf, -1e30, -np.inf, np.nan])
    got = O.e4m3_encode(xs)
    assert list(got[:5]) == [0x7E, 0x7E, 0x7E, 0xFE, 0xFE]
    assert got[5] & 0x7F == 0x7F


# --------------------------------------------------------------------------
# bf16 rounding
# --------------------------------------------------------------------------

def test_bf16_round_exact_rationals():
    rng = np.random.default_rng(13)
    xs = rng.standard_normal(3000) * np.exp2(rng.uniform(-30, 30, 3000))
    # exact ties and their neighbours: 8-bit values + half a unit
    base = rng.integers(128, 256, 500) * 2.0 ** rng.integers(-20, 20, 500)
    ties = base * (1 + 1 / 512)        # exactly half a bf16 unit above base
    xs = np.concatenate([xs, ties, np.nextafter(ties, 0), np.nextafter(ties, np.inf),
                         -ties])
    got = O.bf16_to_f64(O.bf16_round(xs))
    want = np.array([float(_frac_bf16(Fraction(float(x)))) for x in xs])
    assert np.array_equal(got, want)


def test_bf16_round_matches_torch_on_fp32_inputs():
    rng = np.random.default_rng(14)
    xs = (rng.standard_normal(100000) * np.exp2(rng.uniform(-60, 60, 100000)))
    xs = xs.astype(np.float32)
    ref = torch.from_numpy(xs).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(O.bf16_round(xs.astype(np.float64)), ref.view(np.uint16))


# --------------------------------------------------------------------------
# group quantizer  [prepare_megamoe, _quantize_fp8_groups]
# --------------------------------------------------------------------------

def _all_finite_bf16():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = O.bf16_to_f64(bits)
    keep = np.isfinite(v)
    return bits[keep], v[keep]


def test_ue8m0_exponent_closed_form_all_bf16():
    """e = 127 + ceil(log2(max(amax, 1e-4) / 448)), clamped to [1, 254],
    checked in exact rationals for every finite bf16 amax."""
    _, v = _all_finite_bf16()
    x = np.zeros((v.size, 128), np.float32)
    x[:, 0] = v
    codes, e = O.quantize_groups(x, ue8m0=True)
    floor = Fraction(float(np.float32(1e-4)))
    want = []
    for a in np.abs(v):
        A = max(Fraction(float(a)), floor)
        want.append(min(max(127 + _ceil_log2(A / 448), 1), 254))
    assert np.array_equal(e[:, 0].astype(int), np.array(want))
    # the element itself: exact power-of-two scaling, then nearest e4m3fn
    idx = np.random.default_rng(15).choice(v.size, 3000, replace=False)
    for i in idx:
        val = Fraction(float(v[i])) / Fraction(2) ** (int(e[i, 0]) - 127)
        assert codes[i, 0] == _frac_encode(val, bool(np.signbit(v[i])))
    assert np.all(codes[:, 1:] == 0)


def test_ue8m0_group_max_lands_in_top_binade():
    rng = np.random.default_rng(16)
    x = (rng.standard_normal((500, 512)) * np.exp2(rng.uniform(-10, 10, (500, 1))))
    x = x.astype(np.float32)
    codes, e = O.quantize_groups(x, ue8m0=True)
    dec = np.abs(O.e4m3_decode(codes)).reshape(500, 4, 128)
    gmax = dec.max(axis=2)
    amax = np.abs(x).reshape(500, 4, 128).max(axis=2)
    ok = amax >= 1e-4
    assert np.all(gmax[ok] >= 224) and np.all(gmax <= 448)
    assert np.all(np.abs(O.e4m3_decode(codes)) <= 448)


def test_quant_special_groups():
    x = np.zeros((3, 128), np.float32)
    x[1, 7] = 448 * 2.0 ** -5
    x[2, 3] = -448 * 2.0 ** 6
    for ue8m0 in (True, False):
        codes, s = O.quantize_groups(x, ue8m0)
        assert np.all(codes[0] == 0)
        assert codes[1, 7] == 0x7E and codes[2, 3] == 0xFE
        if ue8m0:
            assert int(s[0, 0]) == 105
            assert int(s[1, 0]) == 127 - 5 and int(s[2, 0]) == 127 + 6
        else:
            assert s[1, 0] == np.float32(2.0 ** -5) and s[2, 0] == np.float32(2.0 ** 6)


def test_fp32_scale_mode_properties():
    rng = np.random.default_rng(17)
    x = (rng.standard_normal((400, 256)) * np.exp2(rng.uniform(-8, 8, (400, 1))))
    x = x.astype(np.float32)
    codes, s = O.quantize_groups(x, ue8m0=False)
    g = x.reshape(400, 2, 128)
    amax = np.abs(g).max(axis=2)
    # the scale is amax/448 in fp32 to within one rounding
    assert np.all(np.abs(s.astype(np.float64) * 448 - amax) <= amax * 2.0 ** -23)
    # the element of largest magnitude lands on +-448
    arg = np.abs(g).argmax(axis=2)
    cg = codes.reshape(400, 2, 128)
    top = np.take_along_axis(cg, arg[:, :, None], axis=2)[:, :, 0]
    assert np.all((top & 0x7F) == 0x7E)
    # dequantized values are within half an e4m3 step (relative 2^-4) of x
    deq = O.e4m3_decode(codes).reshape(400, 2, 128) * s[:, :, None]
    err = np.abs(deq - g)
    assert np.all(err <= np.maximum(np.abs(g) * 2.0 ** -4, s[:, :, None] * 2.0 ** -10) * 1.0001)


def test_fp32_scale_mode_exact_rationals():
    """fp32 scales ([STAGE] _quantize_fp8_groups without the UE8M0 round-up,
    readings R1-R4): s = fl32(max(amax, fl32(1e-4)) / 448), then each code is
    the nearest e4m3fn value (saturating) of fl32(x * fl32(1 / s)).  Every
    step is redone here in exact rationals with its own binary32 rounding;
    groups span 2^-24 .. 2^14 in magnitude, with all-tiny groups (the 1e-4
    floor) and groups whose largest element sits a hair under a binade."""
    rng = np.random.default_rng(19)
    rows, G = 80, 3
    mag = np.exp2(rng.uniform(-24, 14, (rows, G)))
    x = rng.standard_normal((rows, G * 128)) * np.repeat(mag, 128, axis=1)
    x[5, :128] *= 1e-6                                # amax below the floor
    x[6, 128:256] = 0.0                               # an all-zero group
    x[7, 0] = np.nextafter(np.float32(448.0), np.float32(0))   # amax just under 448
    x = x.astype(np.float32)
    # rows 40-59, group 0: besides the group maximum, values whose scaled
    # product lies on or next to a midpoint between two e4m3fn values, so
    # that the binary32 rounding of x * (1/s) before the fp8 conversion
    # decides the code (ties go to the even code)
    floor = Fraction(float(np.float32(1e-4)))
    mids = [(_FV[i] + _FV[i + 1]) / 2 for i in range(len(_FV) - 1)]
    tie_rows = range(40, 60)
    for r in tie_rows:
        amax = np.float32(np.exp2(rng.uniform(-10, 10)))
        x[r, :128] = 0.0
        x[r, 0] = amax
        inv = _frac_f32(1 / _frac_f32(max(Fraction(float(amax)), floor) / 448))
        for c in range(1, 128):
            m = mids[int(rng.integers(len(mids)))]
            v = np.float32(float(m / inv))
            v = [np.nextafter(v, np.float32(0)), v, np.nextafter(v, np.float32(np.inf))][
                int(rng.integers(3))]
            x[r, c] = -v if rng.random() < 0.5 else v
    codes, s = O.quantize_groups(x, ue8m0=False)
    for r in range(rows):
        for g in range(G):
            grp = x[r, 128 * g:128 * g + 128]
            A = max(Fraction(float(np.abs(grp).max())), floor)
            s_ref = _frac_f32(A / 448)
            assert Fraction(float(s[r, g])) == s_ref, (r, g)
            inv = _frac_f32(1 / s_ref)
            cols = range(128) if (r in tie_rows and g == 0) else \
                rng.choice(128, 24, replace=False).tolist() + [int(np.abs(grp).argmax())]
            for c in cols:
                xv = Fraction(float(grp[c]))
                want = _frac_encode(_frac_f32(xv * inv) if xv != 0 else Fraction(0),
                                    bool(np.signbit(grp[c])))
                assert int(codes[r, 128 * g + c]) == want, (r, g, c)


def test_pack_bytes_matches_int32_little_endian():
    e = np.arange(1, 11, dtype=np.uint8).reshape(2, 5)
    packed = O.pack_ue8m0_rows(e)
    assert packed.shape == (2, 8)
    words = packed.view(np.int32)
    want0 = 1 | 2 << 8 | 3 << 16 | 4 << 24
    assert words[0, 0] == want0 and words[0, 1] == 5
    assert np.all(packed[:, 5:] == 0)


# --------------------------------------------------------------------------
# routing repack and layout  [prepare_megamoe, _store_topk; fused_humming_moe,
# moe_prepare_scatter / moe_permute in HummingGroupedExperts.apply]
# --------------------------------------------------------------------------

def _brute_layout(ids, E, max_tokens=0):
    T, k = ids.shape
    lists = [[] for _ in range(E)]
    for t in range(T):
        for j in range(k):
            if 0 <= ids[t, j] < E:
                lists[ids[t, j]].append((t, j))
    counts = [len(l) for l in lists]
    offs = [0]
    for c in counts:
        offs.append(offs[-1] + c)
    row_src, slot_row = [], -np.ones((T, k), np.int64)
    for e in range(E):
        for rank, (t, j) in enumerate(lists[e]):
            row_src.append(t)
            slot_row[t, j] = e * max_tokens + rank if max_tokens else offs[e] + rank
    return counts, offs, row_src, slot_row


@pytest.mark.parametrize("max_tokens", [0, 40])
def test_route_layout_brute_force(max_tokens):
    rng = np.random.default_rng(18)
    for trial in range(20):
        T, k, E = rng.integers(1, 30), rng.integers(1, 5), rng.integers(1, 9)
        ids = rng.integers(-2, E + 2, (T, k))
        lay = O.route_layout(ids, E, max_tokens)
        c, o, rs, sr = _brute_layout(ids, E, max_tokens)
        assert list(lay["counts"]) == c and list(lay["offsets"]) == o
        assert list(lay["row_src"]) == rs
        assert np.array_equal(lay["slot_row"], sr)


def test_repack_padding_and_sum_of_counts():
    rng = np.random.default_rng(19)
    T, k, E = 300, 4, 7
    ids = rng.integers(0, E, (T, k)).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    pad = (rng.random(T) < 0.1).astype(np.uint8)
    out_ids, out_w, _ = O.repack_topk(ids, w, pad)
    assert out_ids.dtype == np.int64 and out_w.dtype == np.float32
    assert np.all(out_ids[pad == 1] == -1) and np.all(out_w[pad == 1] == 0)
    assert np.array_equal(out_ids[pad == 0], ids[pad == 0])
    lay = O.route_layout(out_ids, E)
    assert lay["counts"].sum() == (pad == 0).sum() * k
    assert np.all(lay["slot_row"][pad == 1] == -1)
    # inverse maps
    for t in range(T):
        for j in range(k):
            r = lay["slot_row"][t, j]
            if r >= 0:
                assert lay["row_src"][r] == t


def test_eplb_map_invariants():
    rng = np.random.default_rng(20)
    El, extra, T, k = 12, 4, 200, 3
    l2p = -np.ones((El, 2), np.int32)
    l2p[:, 0] = np.arange(El)
    count = np.ones(El, np.int32)
    rep = rng.choice(El, extra, replace=False)
    for i, le in enumerate(rep):
        l2p[le, 1] = El + i
        count[le] = 2
    ids = rng.integers(0, El, (T, k)).astype(np.int32)
    pad = np.zeros(T, np.uint8)
    pad[:10] = 1
    eplb = {"l2p": l2p, "replica_count": count, "record": np.array([1]),
            "num_unpadded": np.array([150])}
    out, _, load = O.repack_topk(ids, np.ones((T, k), np.float32), pad, eplb,
                                 num_physical=El + extra)
    back = np.full(El + extra, -1)
    for le in range(El):
        for r in range(count[le]):
            back[l2p[le, r]] = le
    routed = out >= 0
    assert np.array_equal(back[out[routed]], ids[routed])      # logical(phys(id)) == id
    assert np.all(out[pad == 1] == -1)
    assert load.sum() == routed[:150].sum()
    want = np.bincount(out[:150][routed[:150]], minlength=El + extra)
    assert np.array_equal(load, want)
    off = O.repack_topk(ids, np.ones((T, k), np.float32), pad,
                        {**eplb, "record": np.array([0])}, num_physical=El + extra)[2]
    assert off.sum() == 0


# --------------------------------------------------------------------------
# block-scaled GEMM  [fused_humming_moe, humming_forward with 128x128 fp32
# weight block scales and per-128 activation group scales]
def test_group32_quantizer_exact_rationals():
    """32-column groups (MXFP8 activations): every group's exponent from the
    closed form in exact rationals, a sample of codes by exact nearest-even
    encoding, and the group layout (column c belongs to group c // 32)."""
    rng = np.random.default_rng(18)
    rows, cols = 60, 256
    mag = np.exp2(rng.uniform(-20, 12, (rows, cols // 32)))
    x = (rng.standard_normal((rows, cols)) * np.repeat(mag, 32, axis=1)).astype(np.float32)
    x[3, 32:64] = 0.0                                   # an all-zero group
    codes, e = O.quantize_groups(x, ue8m0=True, group=32)
    assert e.shape == (rows, cols // 32)
    floor = Fraction(float(np.float32(1e-4)))
    for r in range(rows):
        for g in range(cols // 32):
            A = max(Fraction(float(np.abs(x[r, 32 * g:32 * g + 32]).max())), floor)
            assert int(e[r, g]) == min(max(127 + _ceil_log2(A / 448), 1), 254)
    assert int(e[3, 1]) == 105 and np.all(codes[3, 32:64] == 0)
    for _ in range(3000):
        r, c = int(rng.integers(rows)), int(rng.integers(cols))
        val = Fraction(float(x[r, c])) / Fraction(2) ** (int(e[r, c // 32]) - 127)
        assert codes[r, c] == _frac_encode(val, bool(np.signbit(x[r, c])))


def test_e2m1_table_from_bit_fields():
    # OCP MX fp4: sign bit 3, two exponent bits (bias 1), one mantissa bit;
    # exponent field 0 is subnormal (0.5 * mantissa)
    for code in range(16):
        s, ex, m = code >> 3, (code >> 1) & 3, code & 1
        mag = Fraction(m, 2) if ex == 0 else Fraction(2) ** (ex - 1) * (1 + Fraction(m, 2))
        assert O.e2m1_decode(code) == (-1) ** s * float(mag)
        assert np.signbit(O.e2m1_decode(code)) == bool(s)
    assert O.e2m1_decode(0x7) == 6.0 and O.e2m1_decode(0xF) == -6.0


def test_unpack_fp4_low_nibble_first():
    got = O.unpack_fp4(np.array([[0x21, 0xF0, 0x7A]], np.uint8))
    assert got.tolist() == [[1, 2, 0, 15, 10, 7]]


def _mx_dense(codes, exps, fp4):
    """Dequantize MX operands element by element (independent of the oracle's
    GEMM): value = element * 2^(e - 127) with e the byte of column c // 32."""
    if fp4:
        nib = np.empty((codes.shape[0], codes.shape[1] * 2), np.int64)
        for c in range(nib.shape[1]):
            byte = codes[:, c // 2].astype(np.int64)
            nib[:, c] = (byte >> 4) if c % 2 else (byte & 15)
        vals = np.array([float(O.e2m1_decode(n)) for n in range(16)])[nib]
    else:
        vals = O.e4m3_decode(codes)
    scale = np.exp2(np.repeat(exps.astype(np.float64), 32, axis=1) - 127)
    return vals * scale


@pytest.mark.parametrize("fp4", [False, True])
def test_mx_gemm_equals_dense_dequantized_matmul(fp4):
    rng = np.random.default_rng(24 + fp4)
    m, n, C = 29, 96, 256
    a = _finite_codes(rng, (m, C))
    ea = rng.integers(100, 140, (m, C // 32)).astype(np.uint8)
    w = (rng.integers(0, 256, (n, C // 2)).astype(np.uint8) if fp4
         else _finite_codes(rng, (n, C)))
    ew = rng.integers(110, 130, (n, C // 32)).astype(np.uint8)
    got = O.mx_gemm_f64(a, ea, w, ew, fp4)
    want = _mx_dense(a, ea, False) @ _mx_dense(w, ew, fp4).T
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12 * np.abs(want).max())


@pytest.mark.parametrize("fp4", [False, True])
def test_mx_gemm_identity_weights(fp4):
    rng = np.random.default_rng(26)
    m, C = 12, 128
    a = _finite_codes(rng, (m, C))
    ea = rng.integers(110, 135, (m, C // 32)).astype(np.uint8)
    ew = np.full((C, C // 32), 127, np.uint8)
    if fp4:      # e2m1 code 2 is 1.0
        nib = np.zeros((C, C), np.uint8)
        nib[np.arange(C), np.arange(C)] = 2
        w = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    else:        # e4m3 code 0x38 is 1.0
        w = np.zeros((C, C), np.uint8)
        w[np.arange(C), np.arange(C)] = 0x38
    got = O.mx_gemm_f64(a, ea, w, ew, fp4)
    assert np.array_equal(got, _mx_dense(a, ea, False))


# --------------------------------------------------------------------------

def _finite_codes(rng, shape):
    c = rng.integers(0, 256, shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x38
    return c


def test_block_gemm_equals_dense_dequantized_matmul():
    rng = np.random.default_rng(21)
    m, n, C = 37, 256, 384
    a = _finite_codes(rng, (m, C))
    w = _finite_codes(rng, (n, C))
    sa = np.exp2(rng.integers(-10, 4, (m, C // 128))).astype(np.float64)
    sw = rng.uniform(0.001, 0.01, (n // 128, C // 128)).astype(np.float32)
    got = O.block_scaled_gemm_f64(a, sa, w, sw)
    A = O.e4m3_decode(a) * np.repeat(sa, 128, axis=1)
    W = O.e4m3_decode(w) * np.repeat(np.repeat(sw.astype(np.float64), 128, 0), 128, 1)
    want = A @ W.T
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12 * np.abs(want).max())


def test_block_gemm_identity_weights():
    rng = np.random.default_rng(22)
    m, C = 20, 256
    a = _finite_codes(rng, (m, C))
    sa = np.exp2(rng.integers(-6, 2, (m, 2))).astype(np.float64)
    w = np.zeros((C, C), np.uint8)
    w[np.arange(C), np.arange(C)] = 0x38
    sw = np.ones((2, 2), np.float32)
    got = O.block_scaled_gemm_f64(a, sa, w, sw)
    assert np.array_equal(got, O.e4m3_decode(a) * np.repeat(sa, 128, axis=1))


def _finite_bf16(rng, shape, scale=1.0):
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)     # truncation: any finite bf16


def test_bf16_gemm_equals_dense_dequantized_matmul():
    rng = np.random.default_rng(27)
    m, n, C = 23, 256, 384
    a = _finite_bf16(rng, (m, C), 3.0)
    w = _finite_codes(rng, (n, C))
    sw = rng.uniform(0.001, 0.01, (n // 128, C // 128)).astype(np.float32)
    got = O.bf16_gemm_f64(a, w, sw)
    A = (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    W = O.e4m3_decode(w) * np.repeat(np.repeat(sw.astype(np.float64), 128, 0), 128, 1)
    want = A @ W.T
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12 * np.abs(want).max())


def test_bf16_gemm_identity_weights():
    rng = np.random.default_rng(28)
    a = _finite_bf16(rng, (9, 256))
    w = np.zeros((256, 256), np.uint8)
    w[np.arange(256), np.arange(256)] = 0x38
    got = O.bf16_gemm_f64(a, w, np.ones((2, 2), np.float32))
    assert np.array_equal(got, (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64))


def test_act_bf16_matches_torch():
    rng = np.random.default_rng(29)
    N = 256
    gu = _finite_bf16(rng, (64, 2 * N), 2.0)
    got = O.act_bf16(gu, N)
    t = torch.from_numpy(gu.view(np.int16)).view(torch.bfloat16).float()
    want = (torch.nn.functional.silu(t[:, :N]) * t[:, N:]).to(torch.bfloat16)
    want = want.view(torch.int16).numpy().view(np.uint16)
    # fp32 silu may differ from the fp64 evaluation in its last bit, which
    # can move a bf16 rounding by one unit
    diff = np.abs(got.astype(np.int32) - want.astype(np.int32))
    assert diff.max() <= 1 and np.count_nonzero(diff) <= 0.005 * diff.size


# --------------------------------------------------------------------------
# SiLU(gate) * up and the reduce
# --------------------------------------------------------------------------

def test_silu_mul_matches_torch_and_gate_up_order():
    rng = np.random.default_rng(23)
    N = 256
    gu = rng.standard_normal((50, 2 * N)) * 3
    bits = O.bf16_round(gu)
    g64 = torch.from_numpy(O.bf16_to_f64(bits))
    ref = (torch.nn.functional.silu(g64[:, :N]) * g64[:, N:]).to(torch.float32).numpy()
    got = O.silu_mul_f32(bits, N)
    ulp = np.spacing(np.abs(ref).astype(np.float32))
    assert np.all(np.abs(got - ref) <= ulp)
    z = bits.copy()
    z[:, :N] = 0                       # gate = 0 -> silu(0) = 0 whatever up is
    assert np.all(O.silu_mul_f32(z, N) == 0)


def test_reduce_special_cases():
    rng = np.random.default_rng(24)
    T, K = 9, 256
    down = O.bf16_round(rng.standard_normal((T, K)))
    slot = np.arange(T).reshape(T, 1)
    assert np.array_equal(O.topk_reduce(down, slot, np.ones((T, 1), np.float32)), down)
    none = -np.ones((T, 3), np.int64)
    assert np.all(O.topk_reduce(down, none, np.ones((T, 3), np.float32)) == 0)
    slot2 = rng.integers(0, T, (T, 3))
    w = rng.random((T, 3)).astype(np.float32)
    want = np.einsum("tj,tjc->tc", w.astype(np.float64), O.bf16_to_f64(down)[slot2])
    assert np.array_equal(O.topk_reduce(down, slot2, w), O.bf16_round(want))


# --------------------------------------------------------------------------
# the whole layer
# --------------------------------------------------------------------------

def _dense_ffn(h, st):
    """Unquantized activations, dequantized weights, fp64: the layer the
    quantized one approximates."""
    cfg = h["cfg"]
    N = cfg.N
    x = O.bf16_to_f64(h["tokens"])
    out = np.zeros((cfg.T, cfg.K))
    for t in range(cfg.T):
        for j in range(cfg.top_k):
            e = st["ids"][t, j]
            if e < 0:
                continue
            if cfg.weight_quant == "fp8_block128":
                W13 = O.e4m3_decode(h["w13"][e]) * np.repeat(np.repeat(
                    h["w13_sf"][e].astype(np.float64), 128, 0), 128, 1)
                W2 = O.e4m3_decode(h["w2"][e]) * np.repeat(np.repeat(
                    h["w2_sf"][e].astype(np.float64), 128, 0), 128, 1)
            else:
                fp4 = cfg.weight_quant == "mxfp4"
                W13 = _mx_dense(h["w13"][e], h["w13_sf"][e], fp4)
                W2 = _mx_dense(h["w2"][e], h["w2_sf"][e], fp4)
            gu = torch.from_numpy(W13 @ x[t])
            act = _TORCH_ACT[cfg.activation](gu, N).numpy()
            out[t] += st["weights"][t, j] * (W2 @ act)
    return out


# the activations through torch's own functions (independent of the oracle)
_F = torch.nn.functional
_TORCH_ACT = {
    "silu": lambda gu, N: _F.silu(gu[..., :N]) * gu[..., N:2 * N],
    "gelu": lambda gu, N: _F.gelu(gu[..., :N]) * gu[..., N:2 * N],
    "gelu_tanh": lambda gu, N: _F.gelu(gu[..., :N], approximate="tanh") * gu[..., N:2 * N],
    "silu_no_mul": lambda gu, N: _F.silu(gu[..., :N]),
    "gelu_no_mul": lambda gu, N: _F.gelu(gu[..., :N]),
    "gelu_tanh_no_mul": lambda gu, N: _F.gelu(gu[..., :N], approximate="tanh"),
    "relu2_no_mul": lambda gu, N: _F.relu(gu[..., :N]) ** 2,
    # the clamped SwiGLU readings (limit 7), in torch's own operations
    "swiglustep": lambda gu, N: (_F.silu(gu[..., :N]).clamp(max=7.0)
                                 * gu[..., N:2 * N].clamp(-7.0, 7.0)),
    "swigluoai": lambda gu, N: ((gu[..., N:2 * N].clamp(-7.0, 7.0) + 1)
                                * gu[..., :N].clamp(max=7.0)
                                * torch.sigmoid(1.702 * gu[..., :N].clamp(max=7.0))),
}


@pytest.mark.parametrize("act", sorted(_TORCH_ACT))
def test_activation_matches_torch(act):
    """fp64 evaluation rounded once to fp32: within one fp32 unit of torch's
    float64 function rounded the same way (plus 1e-12 absolute: far in the
    negative tail 1 + tanh(y) is a few 1e-15 in one libm and 0 in another)."""
    rng = np.random.default_rng(37)
    N = 256
    width = 2 * N if act in O.GATED else N
    bits = O.bf16_round(rng.standard_normal((40, width)) * 4)
    ref = _TORCH_ACT[act](torch.from_numpy(O.bf16_to_f64(bits)), N).to(torch.float32).numpy()
    got = O.act_f32(bits, N, act)
    assert got.shape == (40, N)
    ulp = np.spacing(np.abs(ref).astype(np.float32))
    assert np.all(np.abs(got - ref) <= ulp + 1e-12), act


def test_activation_identities():
    x = np.linspace(-9, 9, 1001)
    gelu, tanh_gelu = O.ACT_FUNCS["gelu"], O.ACT_FUNCS["gelu_tanh"]
    # x * Phi(x) - (-x) * Phi(-x) = x, since Phi(x) + Phi(-x) = 1
    assert np.allclose(gelu(x) - gelu(-x), x, rtol=0, atol=1e-14)
    assert gelu(np.array([0.0]))[0] == 0 and abs(gelu(np.array([9.0]))[0] - 9) < 1e-15
    # the tanh form approximates the erf form to about 2e-4 (the published
    # approximation's accuracy)
    assert np.max(np.abs(tanh_gelu(x) - gelu(x))) < 1e-3
    assert np.all(O.ACT_FUNCS["relu2"](np.array([-2.0, 0.0, 3.0])) == [0.0, 0.0, 9.0])
    # gated with up = 1 equals the ungated form on the gate half
    rng = np.random.default_rng(38)
    N = 128
    g = O.bf16_round(rng.standard_normal((8, N)) * 3)
    one = O.bf16_round(np.ones((8, N)))
    for base in ("silu", "gelu", "gelu_tanh"):
        assert np.array_equal(O.act_f32(np.concatenate([g, one], 1), N, base),
                              O.act_f32(g, N, base + "_no_mul"))


def test_clamped_swiglu_properties():
    """The clamped SwiGLU readings (parity unpinned: the pages name them
    without bodies): a limit above every value reduces them to their
    unclamped forms; past the limits the output no longer depends on the
    clamped input; SWIGLUOAI's gate factor g * sigmoid(1.702 g) is the
    sigmoid approximation of GELU (within 0.03 of x * Phi(x), its published
    accuracy), which fixes the constant."""
    rng = np.random.default_rng(39)
    g = rng.standard_normal((6, 64)) * 4
    u = rng.standard_normal((6, 64)) * 4
    silu = O.ACT_FUNCS["silu"]
    big = 1e6
    assert np.array_equal(O.gated_act("silu", g, u, big), silu(g) * u)
    assert np.array_equal(O.gated_act("silu", g, u, 0.0), silu(g) * u)
    assert np.array_equal(O.gated_act("swiglustep", g, u, big), silu(g) * u)
    assert np.allclose(O.gated_act("swigluoai", g, u, big),
                       (u + 1) * g / (1 + np.exp(-1.702 * g)), rtol=1e-15, atol=0)
    x = np.linspace(-8, 8, 4001)
    assert np.max(np.abs(x / (1 + np.exp(-1.702 * x)) - O.ACT_FUNCS["gelu"](x))) < 0.03
    L = 1.5
    for act in ("silu", "swiglustep", "swigluoai"):
        h = O.gated_act(act, g, u, L)
        # the up input matters only inside [-L, L]
        assert np.array_equal(h, O.gated_act(act, g, np.clip(u, -L, L), L)), act
        assert np.array_equal(O.gated_act(act, g, np.full_like(u, 3 * L), L),
                              O.gated_act(act, g, np.full_like(u, L), L)), act
    # the gate is capped from above only: SiLU / SWIGLUOAI at g = L, SWIGLUSTEP
    # at silu(g) = L; far below, the output goes to zero
    for act in ("silu", "swigluoai"):
        assert np.array_equal(O.gated_act(act, np.full_like(u, 5 * L), u, L),
                              O.gated_act(act, np.full_like(u, L), u, L)), act
    gs = 2.0        # silu(2) = 1.76 > L: capped
    assert np.array_equal(O.gated_act("swiglustep", np.full_like(u, gs), u, L),
                          L * np.clip(u, -L, L))
    for act in ("silu", "swiglustep", "swigluoai"):
        assert np.max(np.abs(O.gated_act(act, np.full_like(u, -40.0), u, L))) < 1e-12
    # defaults: 7 for SWIGLUOAI / SWIGLUSTEP
    assert np.array_equal(O.gated_act("swiglustep", g, u, 0.0),
                          O.gated_act("swiglustep", g, u, 7.0))
    assert np.array_equal(O.gated_act("swigluoai", g, u, 0.0),
                          O.gated_act("swigluoai", g, u, 7.0))


@pytest.mark.parametrize("act", ["gelu", "gelu_tanh", "silu_no_mul", "gelu_no_mul",
                                 "gelu_tanh_no_mul", "relu2_no_mul", "swiglustep",
                                 "swigluoai"])
def test_tiny_layer_other_activations_track_unquantized_ffn(act):
    cfg = moe_synth.custom(T=16, E=4, top_k=2, K=256, N=512, seed=1, activation=act)
    h = O.host_inputs(moe_synth.make_inputs(cfg))
    assert h["w13"].shape[1] == (2 if cfg.gated else 1) * cfg.N
    r = O.forward(h)
    assert r["gate_up"].shape[1] == cfg.w13_rows and r["a2_q"].shape[1] == cfg.N
    ref = _dense_ffn(h, r)
    got = O.bf16_to_f64(r["out"])
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert 1e-3 < rel < 0.08, (act, rel)


def test_tiny_layer_tracks_unquantized_ffn():
    h = O.host_inputs(moe_synth.make_inputs(moe_synth.CONFIGS["tiny"]))
    r = O.forward(h)
    ref = _dense_ffn(h, r)
    got = O.bf16_to_f64(r["out"])
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert 1e-3 < rel < 0.08, rel


@pytest.mark.parametrize("wq", ["mxfp8", "mxfp4"])
def test_tiny_mx_layer_tracks_unquantized_ffn(wq):
    """MXFP8 activations with MXFP8 / MXFP4 weights: the quantized layer stays
    within a few percent of the same weights with unquantized activations,
    and is not identical to it (the activations really are quantized)."""
    cfg = moe_synth.custom(T=16, E=4, top_k=2, K=256, N=512, seed=1,
                           act_quant="mxfp8", weight_quant=wq)
    h = O.host_inputs(moe_synth.make_inputs(cfg))
    r = O.forward(h)
    assert r["x_sf"].shape == (16, 256 // 32) and r["a2_sf"].shape[1] == 512 // 32
    ref = _dense_ffn(h, r)
    got = O.bf16_to_f64(r["out"])
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert 1e-3 < rel < 0.08, rel


def test_tiny_bf16_layer_tracks_unquantized_ffn():
    """bf16 activations (staging copy, bf16 w2 input): only bf16 roundings
    separate it from the fp64 FFN with the same weights."""
    cfg = moe_synth.custom(T=16, E=4, top_k=2, K=256, N=512, seed=1, act_quant="bf16")
    h = O.host_inputs(moe_synth.make_inputs(cfg))
    r = O.forward(h)
    assert r["x_sf"] is None and r["a2_sf"] is None
    assert np.array_equal(r["x_q"], h["hidden"])
    ref = _dense_ffn(h, r)
    got = O.bf16_to_f64(r["out"])
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert 1e-4 < rel < 1e-2, rel


def test_align_block_size_brute_force():
    rng = np.random.default_rng(31)
    T, k, E, bs = 37, 3, 6, 8
    ids = rng.integers(-1, E + 1, (T, k))          # includes invalid ids
    sorted_ids, expert_ids, P = O.align_block_size(ids, E, bs)
    assert P == sorted_ids.size == expert_ids.size * bs and P % bs == 0
    pos = 0
    for e in range(E):
        slots = [t * k + j for t in range(T) for j in range(k) if ids[t, j] == e]
        if not slots:
            assert e not in expert_ids
            continue
        nb = (len(slots) + bs - 1) // bs
        assert list(sorted_ids[pos:pos + len(slots)]) == slots
        assert np.all(sorted_ids[pos + len(slots):pos + nb * bs] == T * k)
        assert list(expert_ids[pos // bs:pos // bs + nb]) == [e] * nb
        pos += nb * bs
    assert pos == P


@pytest.mark.parametrize("T,k,E,bs,seed", [(1, 1, 1, 16, 0), (50, 4, 64, 16, 1),
                                           (300, 8, 16, 128, 2), (7, 2, 300, 256, 3)])
def test_align_block_size_invariants(T, k, E, bs, seed):
    """Every routed slot appears exactly once, each block holds one expert's
    slots (ascending, routed entries before the padding), and the padded
    total is the sum of the per-expert counts rounded up to blocks."""
    rng = np.random.default_rng(seed)
    ids = rng.integers(-2, E + 2, (T, k))
    sorted_ids, expert_ids, P = O.align_block_size(ids, E, bs)
    flat = ids.ravel()
    valid = (flat >= 0) & (flat < E)
    live = sorted_ids[sorted_ids < T * k]
    assert np.array_equal(np.sort(live), np.flatnonzero(valid))
    counts = np.bincount(flat[valid], minlength=E)
    assert P == int(sum(-(-c // bs) * bs for c in counts))
    for b, e in enumerate(expert_ids):
        blk = sorted_ids[b * bs:(b + 1) * bs]
        n = int((blk < T * k).sum())
        assert n > 0                              # padding never fills a whole block
        assert np.all(blk[:n] < T * k) and np.all(blk[n:] == T * k)
        assert np.all(flat[blk[:n]] == e) and np.all(np.diff(blk[:n]) > 0)
    assert np.all(np.diff(expert_ids) >= 0)


def test_fused_mul_sum_matches_topk_reduce():
    rng = np.random.default_rng(32)
    T, k, E, K = 20, 3, 5, 64
    ids = rng.integers(-1, E, (T, k))
    w = rng.random((T, k)).astype(np.float32)
    lay = O.route_layout(ids, E)
    down_perm = O.bf16_round(rng.standard_normal((int(lay["offsets"][-1]), K)))
    down_tk = np.zeros((T * k, K), np.uint16)
    for t in range(T):
        for j in range(k):
            if lay["slot_row"][t, j] >= 0:
                down_tk[t * k + j] = down_perm[lay["slot_row"][t, j]]
    assert np.array_equal(O.fused_mul_sum(down_tk, ids, w, E),
                          O.topk_reduce(down_perm, lay["slot_row"], w))


@pytest.mark.parametrize("act", ["ue8m0", "fp32", "mxfp8", "bf16"])
def test_indexed_layout_equals_contiguous(act):
    """Same per-row arithmetic, different row placement: identical bits."""
    wq = "mxfp8" if act == "mxfp8" else "fp8_block128"
    cfg = moe_synth.custom(T=40, E=5, top_k=3, K=256, N=256, seed=33, pad_frac=0.1,
                           act_quant=act, weight_quant=wq)
    h = O.host_inputs(moe_synth.make_inputs(cfg))
    a = O.forward(h)
    for bs in (16, 64):
        b = O.forward_indexed(h, bs)
        assert np.array_equal(a["out"], b["out"])
        rows = a["slot_row"].ravel()
        ok = rows >= 0
        assert np.array_equal(b["down"][ok], a["down"][rows[ok]])


def test_layouts_and_padding_agree():
    base = dict(T=40, E=3, top_k=2, K=256, N=256, seed=9)
    hc = O.host_inputs(moe_synth.make_inputs(moe_synth.custom(**base)))
    hb = O.host_inputs(moe_synth.make_inputs(
        moe_synth.custom(**base, layout="batched", max_tokens=64)))
    rc, rb = O.forward(hc), O.forward(hb)
    assert np.array_equal(rc["out"], rb["out"])
    hp = O.host_inputs(moe_synth.make_inputs(moe_synth.custom(**base, pad_frac=0.2)))
    rp = O.forward(hp)
    pad = hp["is_padding"].astype(bool)
    assert np.all(rp["out"][pad] == 0)
    assert np.array_equal(rp["out"][~pad], rc["out"][~pad])


def test_forward_tokens_matches_forward():
    cfg = moe_synth.custom(T=30, E=5, top_k=3, K=256, N=384, seed=10,
                           act_quant="fp32", num_logical=4, pad_frac=0.1)
    h = O.host_inputs(moe_synth.make_inputs(cfg))
    full = O.forward(h)
    part = O.forward_tokens(h, [0, 7, 29])
    for t in (0, 7, 29):
        assert np.array_equal(part["out"][t], full["out"][t])
    for r, info in part["rows"].items():
        assert np.array_equal(info["gate_up"], full["gate_up"][r])
        assert np.array_equal(info["a2_q"], full["a2_q"][r])
        assert np.array_equal(info["down"], full["down"][r])
