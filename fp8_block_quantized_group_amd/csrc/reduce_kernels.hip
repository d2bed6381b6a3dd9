// Top-k weighted reduce back to token order.
//
// "vllm.model_executor.layers.fused_moe.experts.fused_humming_moe":
// HummingGroupedExperts.apply ends with moe_unpermute and
// HummingIndexedExperts.apply with moe_fused_mul_sum; both return, per
// token, the router-weighted sum of the token's expert outputs (router
// weights are applied here, after w2, since apply_router_weight_on_input is
// rejected).  For the batched format the same sum is the finalize step that
// BatchedHummingGroupedExperts delegates.
//
// out[t, c] = bf16( sum_{j ascending, slot_row[t,j] >= 0} w[t,j] * down[slot_row[t,j], c] )
//
// One block of 128 threads covers 1024 columns of one token; each thread
// owns 8 columns (one 16-byte load per routed row, one 16-byte store).  The
// token's slot rows and weights are block-uniform, so they come in through
// scalar loads; the top_k row loads of a thread are independent and stay in
// flight together.
#include "device_common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kReduceThreads = 128;
constexpr int kReduceCols = kReduceThreads * 8;

// slot_row == nullptr: down rows are in (token, slot) order (the indexed
// layout's moe_fused_mul_sum); slot j of token t is row t*k + j when its
// repacked id idx[t, j] is a valid expert.
__global__ __launch_bounds__(kReduceThreads) void topk_reduce_kernel(
    const uint16_t* __restrict__ down, const int32_t* __restrict__ slot_row,
    const int64_t* __restrict__ idx, const float* __restrict__ w, uint16_t* __restrict__ out,
    int k, int K, int E) {
  const int t = blockIdx.y;
  const int c = blockIdx.x * kReduceCols + threadIdx.x * 8;
  if (c >= K) return;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const float* wt = w + (int64_t)t * k;
  for (int j = 0; j < k; ++j) {
    int r;
    if (slot_row != nullptr) {
      r = slot_row[(int64_t)t * k + j];
    } else {
      const int64_t id = idx[(int64_t)t * k + j];
      r = (id >= 0 && id < E) ? t * k + j : -1;
    }
    if (r < 0) continue;
    const float s = wt[j];
    const uint4 v = *reinterpret_cast<const uint4*>(down + (int64_t)r * K + c);
    acc[0] = fmaf(s, bf16_lo(v.x), acc[0]);
    acc[1] = fmaf(s, bf16_hi(v.x), acc[1]);
    acc[2] = fmaf(s, bf16_lo(v.y), acc[2]);
    acc[3] = fmaf(s, bf16_hi(v.y), acc[3]);
    acc[4] = fmaf(s, bf16_lo(v.z), acc[4]);
    acc[5] = fmaf(s, bf16_hi(v.z), acc[5]);
    acc[6] = fmaf(s, bf16_lo(v.w), acc[6]);
    acc[7] = fmaf(s, bf16_hi(v.w), acc[7]);
  }
  uint4 o;
  o.x = pack_bf16x2(acc[0], acc[1]);
  o.y = pack_bf16x2(acc[2], acc[3]);
  o.z = pack_bf16x2(acc[4], acc[5]);
  o.w = pack_bf16x2(acc[6], acc[7]);
  *reinterpret_cast<uint4*>(out + (int64_t)t * K + c) = o;
}

}  // namespace

hipError_t launch_topk_reduce(const void* down, const int32_t* slot_row, const float* w, void* out,
                              int T, int k, int K, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const dim3 grid((K + kReduceCols - 1) / kReduceCols, T);
  topk_reduce_kernel<<<grid, kReduceThreads, 0, stream>>>(
      (const uint16_t*)down, slot_row, nullptr, w, (uint16_t*)out, k, K, 0);
  return hipGetLastError();
}

hipError_t launch_fused_mul_sum(const void* down, const int64_t* idx, const float* w, void* out,
                                int T, int k, int K, int E, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const dim3 grid((K + kReduceCols - 1) / kReduceCols, T);
  topk_reduce_kernel<<<grid, kReduceThreads, 0, stream>>>(
      (const uint16_t*)down, nullptr, idx, w, (uint16_t*)out, k, K, E);
  return hipGetLastError();
}

}  // namespace moe
