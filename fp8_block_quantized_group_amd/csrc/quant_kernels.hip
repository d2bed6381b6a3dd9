// Bandwidth-bound quantization kernels: hidden-state staging and the fused
// SiLU(gate)*up + re-quantization of the w2 input.
//
// Group quantizer: "vllm.model_executor.layers.fused_moe.prepare_megamoe",
// _quantize_fp8_groups (per-128 amax, 1e-4 floor, /448, UE8M0 rounding of
// the scale through its fp32 bit fields, x * (1/scale) to e4m3fn).
// Activation fused into the w2-input quantization:
// "vllm.model_executor.layers.fused_moe.experts.fused_humming_moe",
// HummingExpertsBase.process_input with activation (pull-request 58588 build).
//
// MXFP8 (kMxfp8Dynamic) is the same quantizer with 32-value groups and E8M0
// scales ("...prepare_megamoe", _resolve_hidden_quant: GROUP_K = 32).
//
// Work split: LANES = group/8 lanes per group (a 16-lane DPP row per
// 128-value group, a quad per 32-value group); each lane loads 8 bf16
// (16 bytes), the lanes reduce |x| with DPP max steps, each lane writes 8
// fp8 bytes.  A 64-lane wave covers 512 contiguous input values, so every
// load and store instruction is fully coalesced.
#include "device_common.h"
#include "kernels.h"

namespace moe {

namespace {

__device__ __forceinline__ void unpack8(const uint4 v, float f[8]) {
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
  f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
  f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

// Quantize the 8 values a lane holds (LANES consecutive lanes form one
// group), write the codes and, from the group's first lane, its scale.
template <bool UE8M0, int LANES>
__device__ __forceinline__ void quantize_store(const float f[8], int lane16, uint8_t* q_dst,
                                               uint8_t* sf_row, int g, int G, int sf_row_len) {
  static_assert(LANES == 16 || LANES == 4, "128- or 32-value groups");
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
  amax = LANES == 16 ? row16_max(amax) : quad_max(amax);
  const GroupScale gs = group_scale<UE8M0>(amax);
  uint2 q;
  q.x = f32x4_to_e4m3x4(f[0] * gs.recip, f[1] * gs.recip, f[2] * gs.recip, f[3] * gs.recip);
  q.y = f32x4_to_e4m3x4(f[4] * gs.recip, f[5] * gs.recip, f[6] * gs.recip, f[7] * gs.recip);
  *reinterpret_cast<uint2*>(q_dst) = q;
  if (UE8M0) {
    if (lane16 == 0) sf_row[g] = (uint8_t)gs.stored;
    // the row's trailing pad bytes (4*ceil(G/4) - G of them) are zero
    if (g == G - 1 && lane16 >= 1 && lane16 <= sf_row_len - G) sf_row[G + lane16 - 1] = 0;
  } else {
    if (lane16 == 0) reinterpret_cast<uint32_t*>(sf_row)[g] = gs.stored;
  }
}

// Row r of a batched-masked slab array is live iff r % max_tokens < counts[r / max_tokens].
__device__ __forceinline__ bool row_live(int64_t row, const int32_t* counts, int max_tokens) {
  if (counts == nullptr) return true;
  const int64_t e = row / max_tokens;
  return (row - e * max_tokens) < (int64_t)counts[e];
}

template <bool UE8M0, int LANES>
__global__ __launch_bounds__(256) void stage_quant_kernel(
    const uint16_t* __restrict__ x, uint8_t* __restrict__ xq, uint8_t* __restrict__ xsf,
    int64_t num_groups, int G, int sf_row_len, const int32_t* __restrict__ counts,
    int max_tokens) {
  constexpr int GROUP = 8 * LANES;
  const int64_t gid = (int64_t)blockIdx.x * (256 / LANES) + threadIdx.x / LANES;
  const int lane_g = threadIdx.x % LANES;
  if (gid >= num_groups) return;
  const int64_t row = gid / G;
  const int g = (int)(gid - row * G);
  if (!row_live(row, counts, max_tokens)) return;
  const uint4 v = reinterpret_cast<const uint4*>(x + gid * GROUP)[lane_g];
  float f[8];
  unpack8(v, f);
  uint8_t* sf_row = UE8M0 ? xsf + row * sf_row_len : xsf + row * (int64_t)G * 4;
  quantize_store<UE8M0, LANES>(f, lane_g, xq + gid * GROUP + lane_g * 8, sf_row, g, G,
                               sf_row_len);
}

// Per-128 groups (UE8M0 or fp32 scales): 8 lanes per group, 16 values per
// lane from two adjacent 16-byte loads and one 16-byte store of codes.  The
// hidden states are read once, so the loads are non-temporal; the codes are
// not (the w13 GEMM re-reads them).  Twice the bytes in flight per thread
// of the 16-lane form: 21.3 -> 19.4 us at the DSv3-shaped prefill batch
// (MALL flushed), bit-identical.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
template <bool UE8M0>
__global__ __launch_bounds__(256) void stage_quant128_kernel(
    const uint16_t* __restrict__ x, uint8_t* __restrict__ xq, uint8_t* __restrict__ xsf,
    int64_t num_groups, int G, int sf_row_len, const int32_t* __restrict__ counts,
    int max_tokens) {
  const int64_t gid = (int64_t)blockIdx.x * 32 + threadIdx.x / 8;
  const int lane8 = threadIdx.x % 8;
  if (gid >= num_groups) return;
  const int64_t row = gid / G;
  const int g = (int)(gid - row * G);
  if (!row_live(row, counts, max_tokens)) return;
  const u32x4* src = reinterpret_cast<const u32x4*>(x + gid * kGroup) + 2 * lane8;
  const u32x4 a = __builtin_nontemporal_load(src);
  const u32x4 b = __builtin_nontemporal_load(src + 1);
  float f[16];
  unpack8(make_uint4(a.x, a.y, a.z, a.w), f);
  unpack8(make_uint4(b.x, b.y, b.z, b.w), f + 8);
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(f[i]));
  amax = row8_max(amax);
  const GroupScale gs = group_scale<UE8M0>(amax);
  uint4 q;
  q.x = f32x4_to_e4m3x4(f[0] * gs.recip, f[1] * gs.recip, f[2] * gs.recip, f[3] * gs.recip);
  q.y = f32x4_to_e4m3x4(f[4] * gs.recip, f[5] * gs.recip, f[6] * gs.recip, f[7] * gs.recip);
  q.z = f32x4_to_e4m3x4(f[8] * gs.recip, f[9] * gs.recip, f[10] * gs.recip, f[11] * gs.recip);
  q.w = f32x4_to_e4m3x4(f[12] * gs.recip, f[13] * gs.recip, f[14] * gs.recip, f[15] * gs.recip);
  *reinterpret_cast<uint4*>(xq + gid * kGroup + lane8 * 16) = q;
  if (UE8M0) {
    uint8_t* sf_row = xsf + row * sf_row_len;
    if (lane8 == 0) sf_row[g] = (uint8_t)gs.stored;
    // the row's trailing pad bytes (4*ceil(G/4) - G of them) are zero
    if (g == G - 1 && lane8 >= 1 && lane8 <= sf_row_len - G) sf_row[G + lane8 - 1] = 0;
  } else {
    if (lane8 == 0) reinterpret_cast<uint32_t*>(xsf + row * (int64_t)G * 4)[g] = gs.stored;
  }
}

// bf16 staging without quantization: a masked 16-byte copy.
__global__ __launch_bounds__(256) void stage_copy_kernel(
    const uint4* __restrict__ x, uint4* __restrict__ y, int64_t num_vec, int vec_per_row,
    const int32_t* __restrict__ counts, int max_tokens) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= num_vec) return;
  if (!row_live(i / vec_per_row, counts, max_tokens)) return;
  y[i] = x[i];
}

// h = silu(gate) * up for columns [g*GROUP, (g+1)*GROUP) of the gate half
// and the same columns of the up half, then the group quantizer on h.
template <bool UE8M0, int LANES>
__global__ __launch_bounds__(256) void act_requant_kernel(
    const uint16_t* __restrict__ gu, uint8_t* __restrict__ aq, uint8_t* __restrict__ asf,
    int64_t num_groups, int N, int GN, int sf_row_len, const int32_t* __restrict__ num_rows,
    const int32_t* __restrict__ counts, int max_tokens, int act) {
  constexpr int GROUP = 8 * LANES;
  const int64_t gid = (int64_t)blockIdx.x * (256 / LANES) + threadIdx.x / LANES;
  const int lane_g = threadIdx.x % LANES;
  if (gid >= num_groups) return;
  const int64_t row = gid / GN;
  const int g = (int)(gid - row * GN);
  if (num_rows != nullptr && row >= (int64_t)*num_rows) return;
  if (!row_live(row, counts, max_tokens)) return;
  const bool gated = act_is_gated(act);
  const uint16_t* src = gu + row * (int64_t)(gated ? 2 * N : N) + g * GROUP + lane_g * 8;
  float fg[8], fu[8], h[8];
  unpack8(*reinterpret_cast<const uint4*>(src), fg);
  if (gated) unpack8(*reinterpret_cast<const uint4*>(src + N), fu);
#pragma unroll
  for (int i = 0; i < 8; ++i) h[i] = apply_act(act, fg[i], gated ? fu[i] : 0.0f);
  uint8_t* sf_row = UE8M0 ? asf + row * sf_row_len : asf + row * (int64_t)GN * 4;
  quantize_store<UE8M0, LANES>(h, lane_g, aq + row * (int64_t)N + g * GROUP + lane_g * 8,
                               sf_row, g, GN, sf_row_len);
}

// bf16 activations (no quantization): h computed as above and rounded once
// to bf16; 8 columns per thread.
__global__ __launch_bounds__(256) void act_bf16_kernel(
    const uint16_t* __restrict__ gu, uint16_t* __restrict__ out, int64_t num_vec, int N,
    const int32_t* __restrict__ num_rows, const int32_t* __restrict__ counts, int max_tokens,
    int act) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= num_vec) return;
  const int vpr = N / 8;
  const int64_t row = i / vpr;
  const int col = (int)(i - row * vpr) * 8;
  if (num_rows != nullptr && row >= (int64_t)*num_rows) return;
  if (!row_live(row, counts, max_tokens)) return;
  const bool gated = act_is_gated(act);
  const uint16_t* src = gu + row * (int64_t)(gated ? 2 * N : N) + col;
  float fg[8], fu[8], h[8];
  unpack8(*reinterpret_cast<const uint4*>(src), fg);
  if (gated) unpack8(*reinterpret_cast<const uint4*>(src + N), fu);
#pragma unroll
  for (int k = 0; k < 8; ++k) h[k] = apply_act(act, fg[k], gated ? fu[k] : 0.0f);
  *reinterpret_cast<uint4*>(out + row * (int64_t)N + col) =
      make_uint4(pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]), pack_bf16x2(h[4], h[5]),
                 pack_bf16x2(h[6], h[7]));
}

inline unsigned blocks_for(int64_t n, int per_block) {
  return (unsigned)((n + per_block - 1) / per_block);
}

}  // namespace

hipError_t launch_stage_quant(const void* x, void* xq, void* xsf, int64_t rows, int K,
                              int quant, const int32_t* counts, int max_tokens,
                              hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  if (quant == kQuantBf16) {
    const int64_t nvec = rows * (K / 8);
    stage_copy_kernel<<<blocks_for(nvec, 256), 256, 0, stream>>>(
        (const uint4*)x, (uint4*)xq, nvec, K / 8, counts, max_tokens);
  } else if (quant == kQuantMxfp8) {
    const int G = K / 32;   // K is a multiple of 128: rows of G bytes, no pad
    stage_quant_kernel<true, 4><<<blocks_for(rows * G, 64), 256, 0, stream>>>(
        (const uint16_t*)x, (uint8_t*)xq, (uint8_t*)xsf, rows * G, G, G, counts, max_tokens);
  } else {
    const int G = K / kGroup;
    const int sf_row_len = 4 * ((G + 3) / 4);
    if (quant == kQuantUe8m0)
      stage_quant128_kernel<true><<<blocks_for(rows * G, 32), 256, 0, stream>>>(
          (const uint16_t*)x, (uint8_t*)xq, (uint8_t*)xsf, rows * G, G, sf_row_len, counts,
          max_tokens);
    else
      stage_quant128_kernel<false><<<blocks_for(rows * G, 32), 256, 0, stream>>>(
          (const uint16_t*)x, (uint8_t*)xq, (uint8_t*)xsf, rows * G, G, sf_row_len, counts,
          max_tokens);
  }
  return hipGetLastError();
}

hipError_t launch_act_requant(const void* gate_up, void* aq, void* asf, int64_t rows_cap, int N,
                              int quant, const int32_t* num_rows, const int32_t* counts,
                              int max_tokens, int act, hipStream_t stream) {
  if (rows_cap == 0) return hipSuccess;
  if (quant == kQuantBf16) {
    const int64_t nvec = rows_cap * (N / 8);
    act_bf16_kernel<<<blocks_for(nvec, 256), 256, 0, stream>>>(
        (const uint16_t*)gate_up, (uint16_t*)aq, nvec, N, num_rows, counts, max_tokens, act);
    return hipGetLastError();
  }
  if (quant == kQuantMxfp8) {
    const int GN = N / 32;
    act_requant_kernel<true, 4><<<blocks_for(rows_cap * GN, 64), 256, 0, stream>>>(
        (const uint16_t*)gate_up, (uint8_t*)aq, (uint8_t*)asf, rows_cap * GN, N, GN, GN,
        num_rows, counts, max_tokens, act);
    return hipGetLastError();
  }
  const int GN = N / kGroup;
  const int sf_row_len = 4 * ((GN + 3) / 4);
  if (quant == kQuantUe8m0) {
    act_requant_kernel<true, 16><<<blocks_for(rows_cap * GN, 16), 256, 0, stream>>>(
        (const uint16_t*)gate_up, (uint8_t*)aq, (uint8_t*)asf, rows_cap * GN, N, GN,
        sf_row_len, num_rows, counts, max_tokens, act);
  } else {
    act_requant_kernel<false, 16><<<blocks_for(rows_cap * GN, 16), 256, 0, stream>>>(
        (const uint16_t*)gate_up, (uint8_t*)aq, (uint8_t*)asf, rows_cap * GN, N, GN,
        sf_row_len, num_rows, counts, max_tokens, act);
  }
  return hipGetLastError();
}

}  // namespace moe
