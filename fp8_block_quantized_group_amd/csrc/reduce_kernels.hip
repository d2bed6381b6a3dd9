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
// One block of 128 threads covers 1024 columns of one token (block b: token
// b / column blocks, so the grid is one-dimensional and any token count the
// host validation accepts fits it); each thread owns 8 columns (one 16-byte load per routed row, one 16-byte store).  The
// token's slot rows and weights are block-uniform, so they come in through
// scalar loads; the row loads of a thread are issued 8 at a time so that
// they are in flight together.  Every byte is touched once, so loads and
// stores carry the non-temporal hint (measured at the DSv3-shaped prefill
// batch, MALL flushed: 120 -> 93 us).
#include "device_common.h"
#include "kernels.h"

namespace moe {

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load_nt(const uint16_t* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_nt(uint16_t* p, uint4 v) {
  const u32x4 x = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(x, reinterpret_cast<u32x4*>(p));
}

constexpr int kReduceThreads = 128;
constexpr int kReduceCols = kReduceThreads * 8;

// slot_row == nullptr: down rows are in (token, slot) order (the indexed
// layout's moe_fused_mul_sum); slot j of token t is row t*k + j when its
// repacked id idx[t, j] is a valid expert.
__global__ __launch_bounds__(kReduceThreads) void topk_reduce_kernel(
    const uint16_t* __restrict__ down, const int32_t* __restrict__ slot_row,
    const int64_t* __restrict__ idx, const float* __restrict__ w, uint16_t* __restrict__ out,
    int k, int K, int E, int col_blocks) {
  const int t = (int)(blockIdx.x / (unsigned)col_blocks);
  const int c = (int)(blockIdx.x - (unsigned)t * col_blocks) * kReduceCols + threadIdx.x * 8;
  if (c >= K) return;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const float* wt = w + (int64_t)t * k;
  // slots in groups of 8: the group's row numbers and weights first, then
  // its row loads all in flight together, then the sums in slot order
  for (int j0 = 0; j0 < k; j0 += 8) {
    int r[8];
    float s[8];
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = j0 + u;
      r[u] = -1;
      s[u] = 0.0f;
      if (j < k) {
        if (slot_row != nullptr) {
          r[u] = slot_row[(int64_t)t * k + j];
        } else {
          const int64_t id = idx[(int64_t)t * k + j];
          r[u] = (id >= 0 && id < E) ? t * k + j : -1;
        }
        s[u] = wt[j];
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (r[u] >= 0) v[u] = load_nt(down + (int64_t)r[u] * K + c);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (r[u] < 0) continue;
      acc[0] = fmaf(s[u], bf16_lo(v[u].x), acc[0]);
      acc[1] = fmaf(s[u], bf16_hi(v[u].x), acc[1]);
      acc[2] = fmaf(s[u], bf16_lo(v[u].y), acc[2]);
      acc[3] = fmaf(s[u], bf16_hi(v[u].y), acc[3]);
      acc[4] = fmaf(s[u], bf16_lo(v[u].z), acc[4]);
      acc[5] = fmaf(s[u], bf16_hi(v[u].z), acc[5]);
      acc[6] = fmaf(s[u], bf16_lo(v[u].w), acc[6]);
      acc[7] = fmaf(s[u], bf16_hi(v[u].w), acc[7]);
    }
  }
  uint4 o;
  o.x = pack_bf16x2(acc[0], acc[1]);
  o.y = pack_bf16x2(acc[2], acc[3]);
  o.z = pack_bf16x2(acc[4], acc[5]);
  o.w = pack_bf16x2(acc[6], acc[7]);
  store_nt(out + (int64_t)t * K + c, o);
}

}  // namespace

int64_t reduce_blocks(int T, int K) {
  return (int64_t)T * ((K + kReduceCols - 1) / kReduceCols);
}

hipError_t launch_topk_reduce(const void* down, const int32_t* slot_row, const float* w, void* out,
                              int T, int k, int K, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int64_t blocks = reduce_blocks(T, K);
  if (blocks >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  topk_reduce_kernel<<<dim3((unsigned)blocks), kReduceThreads, 0, stream>>>(
      (const uint16_t*)down, slot_row, nullptr, w, (uint16_t*)out, k, K, 0,
      (K + kReduceCols - 1) / kReduceCols);
  return hipGetLastError();
}

hipError_t launch_fused_mul_sum(const void* down, const int64_t* idx, const float* w, void* out,
                                int T, int k, int K, int E, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int64_t blocks = reduce_blocks(T, K);
  if (blocks >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  topk_reduce_kernel<<<dim3((unsigned)blocks), kReduceThreads, 0, stream>>>(
      (const uint16_t*)down, nullptr, idx, w, (uint16_t*)out, k, K, E,
      (K + kReduceCols - 1) / kReduceCols);
  return hipGetLastError();
}

}  // namespace moe
