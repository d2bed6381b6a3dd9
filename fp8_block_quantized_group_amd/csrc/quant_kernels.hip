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
// load and store instruction is fully coalesced.  (The hidden states' fp8
// staging uses the group quantizer of device_common.h inside the routing scan's
// launch; the kernels here copy bf16 and re-quantize the w2 input of the
// unfused path.)
#include "device_common.h"
#include "kernels.h"

namespace moe {

namespace {

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
    const int32_t* __restrict__ counts, int max_tokens, int act, float limit) {
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
  for (int i = 0; i < 8; ++i) h[i] = apply_act(act, fg[i], gated ? fu[i] : 0.0f, limit);
  uint8_t* sf_row = UE8M0 ? asf + row * sf_row_len : asf + row * (int64_t)GN * 4;
  quantize_store<UE8M0, LANES>(h, lane_g, aq + row * (int64_t)N + g * GROUP + lane_g * 8,
                               sf_row, g, GN, sf_row_len);
}

// bf16 activations (no quantization): h computed as above and rounded once
// to bf16; 8 columns per thread.
__global__ __launch_bounds__(256) void act_bf16_kernel(
    const uint16_t* __restrict__ gu, uint16_t* __restrict__ out, int64_t num_vec, int N,
    const int32_t* __restrict__ num_rows, const int32_t* __restrict__ counts, int max_tokens,
    int act, float limit) {
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
  for (int k = 0; k < 8; ++k) h[k] = apply_act(act, fg[k], gated ? fu[k] : 0.0f, limit);
  *reinterpret_cast<uint4*>(out + row * (int64_t)N + col) =
      make_uint4(pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]), pack_bf16x2(h[4], h[5]),
                 pack_bf16x2(h[6], h[7]));
}

inline unsigned blocks_for(int64_t n, int per_block) {
  return (unsigned)((n + per_block - 1) / per_block);
}

__global__ __launch_bounds__(256) void zero_i32_kernel(int32_t* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

}  // namespace

hipError_t launch_zero_i32(int32_t* p, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  zero_i32_kernel<<<blocks_for(n, 256), 256, 0, stream>>>(p, n);
  return hipGetLastError();
}

hipError_t launch_stage_quant(const void* x, void* xq, void* xsf, int64_t rows, int K,
                              int quant, const int32_t* counts, int max_tokens,
                              hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  if (quant == kQuantBf16) {
    const int64_t nvec = rows * (K / 8);
    stage_copy_kernel<<<blocks_for(nvec, 256), 256, 0, stream>>>(
        (const uint4*)x, (uint4*)xq, nvec, K / 8, counts, max_tokens);
  } else {
    // fp8 staging runs inside the routing scan's launch (launch_route)
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_act_requant(const void* gate_up, void* aq, void* asf, int64_t rows_cap, int N,
                              int quant, const int32_t* num_rows, const int32_t* counts,
                              int max_tokens, int act, float act_limit, hipStream_t stream) {
  if (rows_cap == 0) return hipSuccess;
  if (quant == kQuantBf16) {
    const int64_t nvec = rows_cap * (N / 8);
    act_bf16_kernel<<<blocks_for(nvec, 256), 256, 0, stream>>>(
        (const uint16_t*)gate_up, (uint16_t*)aq, nvec, N, num_rows, counts, max_tokens, act,
        act_limit);
    return hipGetLastError();
  }
  if (quant == kQuantMxfp8) {
    const int GN = N / 32;
    act_requant_kernel<true, 4><<<blocks_for(rows_cap * GN, 64), 256, 0, stream>>>(
        (const uint16_t*)gate_up, (uint8_t*)aq, (uint8_t*)asf, rows_cap * GN, N, GN, GN,
        num_rows, counts, max_tokens, act, act_limit);
    return hipGetLastError();
  }
  const int GN = N / kGroup;
  const int sf_row_len = 4 * ((GN + 3) / 4);
  if (quant == kQuantUe8m0) {
    act_requant_kernel<true, 16><<<blocks_for(rows_cap * GN, 16), 256, 0, stream>>>(
        (const uint16_t*)gate_up, (uint8_t*)aq, (uint8_t*)asf, rows_cap * GN, N, GN,
        sf_row_len, num_rows, counts, max_tokens, act, act_limit);
  } else {
    act_requant_kernel<false, 16><<<blocks_for(rows_cap * GN, 16), 256, 0, stream>>>(
        (const uint16_t*)gate_up, (uint8_t*)aq, (uint8_t*)asf, rows_cap * GN, N, GN,
        sf_row_len, num_rows, counts, max_tokens, act, act_limit);
  }
  return hipGetLastError();
}

}  // namespace moe
