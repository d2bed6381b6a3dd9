// Device helpers shared by the gfx950 kernels of the MoE expert layer.
//
// Number formats: bf16 in HBM, fp32 in registers, fp8 e4m3fn (OCP "fn"
// variant, max 448, no infinities) for quantized activations and weights.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kGroup = 128;        // quantization group / scale block edge
constexpr float kFp8Max = 448.0f;  // largest finite e4m3fn value

// ---- bf16 <-> fp32 --------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t packed) {
  return __uint_as_float(packed << 16);
}
__device__ __forceinline__ float bf16_hi(uint32_t packed) {
  return __uint_as_float(packed & 0xFFFF0000u);
}
// fp32 -> bf16, round to nearest even; NaN stays a quiet NaN.  One
// v_cvt_pk_bf16_f32 per pair (gfx950): checked on the GPU to give the bits of
// the integer formula -- add 0x7FFF plus the kept lsb, then truncate; a NaN
// keeps its upper bits with the quiet bit set -- for all 2^32 inputs.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return pack_bf16x2(f, 0.0f) & 0xFFFFu;
}

// ---- fp32 -> e4m3fn ---------------------------------------------------------
// The hardware converter rounds to nearest even; clamping to +-448 first
// makes out-of-range magnitudes saturate instead of becoming NaN.
__device__ __forceinline__ uint32_t f32x4_to_e4m3x4(float a, float b, float c, float d) {
  a = __builtin_amdgcn_fmed3f(a, -kFp8Max, kFp8Max);
  b = __builtin_amdgcn_fmed3f(b, -kFp8Max, kFp8Max);
  c = __builtin_amdgcn_fmed3f(c, -kFp8Max, kFp8Max);
  d = __builtin_amdgcn_fmed3f(d, -kFp8Max, kFp8Max);
  int v = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  v = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, v, true);
  return (uint32_t)v;
}

// ---- cross-lane max over a row of 16 lanes (DPP) ---------------------------
// quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror:
// after the four steps every lane of the 16-lane row holds the row maximum.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));
  v = fmaxf(v, dpp_f32<0x4E>(v));
  v = fmaxf(v, dpp_f32<0x141>(v));
  v = fmaxf(v, dpp_f32<0x140>(v));
  return v;
}

// max over a half-row of 8 lanes: the two quad steps, then row_half_mirror
__device__ __forceinline__ float row8_max(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));
  v = fmaxf(v, dpp_f32<0x4E>(v));
  v = fmaxf(v, dpp_f32<0x141>(v));
  return v;
}

// max over a quad of 4 lanes (quad_perm [1,0,3,2], [2,3,0,1])
__device__ __forceinline__ float quad_max(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));
  v = fmaxf(v, dpp_f32<0x4E>(v));
  return v;
}

// ---- the per-group scale -----------------------------------------------------
// Given the group's amax: floor it at 1e-4, divide by 448 (correctly rounded
// fp32 division), and for UE8M0 round the scale up to a power of two through
// its fp32 bit fields (exponent + 1 when the mantissa is non-zero, clamped to
// [1, 254]).  Returns the reciprocal the values are multiplied by and the
// value to store (exponent byte, or the fp32 scale's bits).
struct GroupScale {
  float recip;
  uint32_t stored;
};
template <bool UE8M0>
__device__ __forceinline__ GroupScale group_scale(float amax) {
  amax = fmaxf(amax, 1.0e-4f);
  const float s = amax / kFp8Max;
  GroupScale r;
  if (UE8M0) {
    const uint32_t bits = __float_as_uint(s);
    uint32_t e = ((bits >> 23) & 0xFFu) + ((bits & 0x7FFFFFu) != 0u ? 1u : 0u);
    e = e < 1u ? 1u : (e > 254u ? 254u : e);
    r.recip = 1.0f / __uint_as_float(e << 23);
    r.stored = e;
  } else {
    r.recip = 1.0f / s;
    r.stored = __float_as_uint(s);
  }
  return r;
}

__device__ __forceinline__ void unpack8(const uint4 v, float f[8]) {
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
  f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
  f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

// Row r of a batched-masked slab array is live iff r % max_tokens < counts[r / max_tokens].
__device__ __forceinline__ bool row_live(int64_t row, const int32_t* counts, int max_tokens) {
  if (counts == nullptr) return true;
  const int64_t e = row / max_tokens;
  return (row - e * max_tokens) < (int64_t)counts[e];
}

// The group quantizer (load_group_chunk, then quantize_group_chunk) on one
// group gid of GROUP values (128: per-128
// scales, UE8M0 bytes in rows of sf_row_len or fp32 [rows, G]; 32: MXFP8,
// E8M0 bytes in rows of G) of bf16 rows of G groups: GROUP/16 lanes per
// group, 16 values per lane from two adjacent 16-byte loads and one 16-byte
// store of codes.  The hidden states are read once, so the loads are
// non-temporal; the codes are not (the w13 GEMM re-reads them).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
// This lane's 16 values of group gid (its two adjacent 16-byte chunks).
struct GroupChunk {
  u32x4_t a, b;
};
template <int GROUP>
__device__ __forceinline__ GroupChunk load_group_chunk(const uint16_t* __restrict__ x,
                                                       int64_t gid, int lane) {
  const u32x4_t* src = reinterpret_cast<const u32x4_t*>(x + gid * GROUP) + 2 * lane;
  return GroupChunk{__builtin_nontemporal_load(src), __builtin_nontemporal_load(src + 1)};
}
// The quantizer on a loaded chunk: the group maximum across its lanes, the
// scale, the codes and the scale byte / word.
template <int GROUP, bool UE8M0>
__device__ __forceinline__ void quantize_group_chunk(const GroupChunk& c,
                                                     uint8_t* __restrict__ xq,
                                                     uint8_t* __restrict__ xsf, int64_t gid,
                                                     int lane, int G, int sf_row_len) {
  static_assert(GROUP == 128 || (GROUP == 32 && UE8M0), "per-128 groups, or MX groups of 32");
  const int64_t row = gid / G;
  const int g = (int)(gid - row * G);
  const u32x4_t a = c.a, b = c.b;
  float f[16];
  unpack8(make_uint4(a.x, a.y, a.z, a.w), f);
  unpack8(make_uint4(b.x, b.y, b.z, b.w), f + 8);
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(f[i]));
  // 8 lanes: two quad steps and row_half_mirror; 2 lanes: swap neighbours
  amax = GROUP == 128 ? row8_max(amax) : fmaxf(amax, dpp_f32<0xB1>(amax));
  const GroupScale gs = group_scale<UE8M0>(amax);
  uint4 q;
  q.x = f32x4_to_e4m3x4(f[0] * gs.recip, f[1] * gs.recip, f[2] * gs.recip, f[3] * gs.recip);
  q.y = f32x4_to_e4m3x4(f[4] * gs.recip, f[5] * gs.recip, f[6] * gs.recip, f[7] * gs.recip);
  q.z = f32x4_to_e4m3x4(f[8] * gs.recip, f[9] * gs.recip, f[10] * gs.recip, f[11] * gs.recip);
  q.w = f32x4_to_e4m3x4(f[12] * gs.recip, f[13] * gs.recip, f[14] * gs.recip, f[15] * gs.recip);
  *reinterpret_cast<uint4*>(xq + gid * GROUP + lane * 16) = q;
  if (UE8M0) {
    uint8_t* sf_row = xsf + row * sf_row_len;
    if (lane == 0) sf_row[g] = (uint8_t)gs.stored;
    // the row's trailing pad bytes (sf_row_len - G of them; 128-groups: up
    // to 3, MX rows have none) are zero
    if (GROUP == 128 && g == G - 1 && lane >= 1 && lane <= sf_row_len - G)
      sf_row[G + lane - 1] = 0;
  } else {
    if (lane == 0) reinterpret_cast<uint32_t*>(xsf + row * (int64_t)G * 4)[g] = gs.stored;
  }
}


// ---- activations ------------------------------------------------------------
// Kinds (values match moe_act_t).  Gated kinds combine the gate column g with
// its up column u; _no_mul kinds return f(g) of the single w13 output
// column.  The experts' activation list names them; the functions are the
// standard ones: SiLU g * sigmoid(g); GELU g * Phi(g) with the exact normal
// CDF; the tanh form of GELU; ReLU^2 = max(g, 0)^2.  The clamped SwiGLU
// forms (named without bodies; this library's reading), with limit L > 0:
// SiLU with a clamp limit silu(min(g, L)) * clamp(u, -L, L); SWIGLUSTEP
// min(silu(g), L) * clamp(u, -L, L); SWIGLUOAI (clamp(u, -L, L) + 1) *
// g' * sigmoid(1.702 g') with g' = min(g, L).
constexpr int kActSilu = 0;
constexpr int kActGelu = 1;
constexpr int kActGeluTanh = 2;
constexpr int kActSiluNoMul = 3;
constexpr int kActGeluNoMul = 4;
constexpr int kActGeluTanhNoMul = 5;
constexpr int kActRelu2NoMul = 6;
constexpr int kActSwigluOai = 7;
constexpr int kActSwigluStep = 8;
constexpr float kSwigluOaiAlpha = 1.702f;
constexpr bool act_is_gated(int kind) { return kind < kActSiluNoMul || kind > kActRelu2NoMul; }

__device__ __forceinline__ float silu_f32(float g) {
  const float sig = __builtin_amdgcn_rcpf(1.0f + __expf(-g));
  return g * sig;
}

// kind and limit are uniform across the launch (kernel arguments), so the
// switch is a scalar branch.  SiLU keeps the g * sigmoid(g) * u order in
// fp32.  limit: the clamp of the SwiGLU forms (> 0; for SiLU 0 = none).
__device__ __forceinline__ float apply_act(int kind, float g, float u, float limit = 0.0f) {
  switch (kind) {
    case kActSwigluOai: {
      const float gc = fminf(g, limit);
      const float uc = fminf(fmaxf(u, -limit), limit);
      const float glu = gc * __builtin_amdgcn_rcpf(1.0f + __expf(-kSwigluOaiAlpha * gc));
      return (uc + 1.0f) * glu;
    }
    case kActSwigluStep: {
      const float uc = fminf(fmaxf(u, -limit), limit);
      return fminf(silu_f32(g), limit) * uc;
    }
    case kActGelu:
    case kActGeluNoMul: {
      // 1 + erf(g / sqrt 2) as erfc(-g / sqrt 2): no cancellation for g < 0
      const float f = 0.5f * g * erfcf(-g * 0.70710678118654752f);
      return kind == kActGelu ? f * u : f;
    }
    case kActGeluTanh:
    case kActGeluTanhNoMul: {
      // (1 + tanh y) / 2 = sigmoid(2y): no cancellation for y < 0
      const float y = 0.79788456080286536f * (g + 0.044715f * g * g * g);
      const float f = g * __builtin_amdgcn_rcpf(1.0f + __expf(-2.0f * y));
      return kind == kActGeluTanh ? f * u : f;
    }
    case kActRelu2NoMul: {
      const float r = fmaxf(g, 0.0f);
      return r * r;
    }
    case kActSiluNoMul:
      return silu_f32(g);
    default: {
      if (limit > 0.0f) {
        g = fminf(g, limit);
        u = fminf(fmaxf(u, -limit), limit);
      }
      const float sig = __builtin_amdgcn_rcpf(1.0f + __expf(-g));
      return g * sig * u;
    }
  }
}

}  // namespace moe
