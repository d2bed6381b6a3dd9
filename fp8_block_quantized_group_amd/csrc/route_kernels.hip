// Routing: top-k repack, expert-replica remap, per-expert counts, the
// stable (token, slot) -> row permutation and the M-tile schedule.
//
// Repack: "vllm.model_executor.layers.fused_moe.prepare_megamoe",
// _store_topk (ids to int64 with padding tokens -> -1, weights to fp32 with
// padding -> 0) and _eplb_kernel_args (logical -> physical replica map,
// per-physical load recording bounded by the unpadded token count).
// Counts / offsets / permutation: "...experts.fused_humming_moe",
// HummingGroupedExperts.apply (moe_prepare_scatter / moe_permute produce
// expert_offsets [E+1] and the inverse permutation; the batched format takes
// expert_num_tokens per slab).
//
// Three launches, no host synchronisation:
//   1. repack + per-block expert histogram (LDS atomics), EPLB load counts;
//   2. one block: per-expert exclusive scan over blocks, offsets, and the
//      heavy-first M-tile list for the grouped GEMMs (tiles of one expert
//      contiguous, with per-expert group offsets);
//   3. per-block stable ranks (wave ballots + LDS running counters) ->
//      row_src and slot_row.
// Rows of one expert come out in ascending flat slot order t*top_k + j, so
// the layout is deterministic.
#include "device_common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kSubRounds = kRouteChunk / kRouteThreads;

__global__ __launch_bounds__(kRouteThreads) void route_repack_hist_kernel(
    const int32_t* __restrict__ topk_ids, const float* __restrict__ topk_w,
    const uint8_t* __restrict__ is_padding, int T, int k, int E, EplbArgs eplb,
    int64_t* __restrict__ idx_out, float* __restrict__ w_out, int32_t* __restrict__ hist) {
  extern __shared__ int32_t lds[];
  int32_t* h = lds;           // [E] block histogram
  int32_t* load = lds + E;    // [E] block EPLB load
  const int tid = threadIdx.x;
  for (int i = tid; i < 2 * E; i += kRouteThreads) lds[i] = 0;
  __syncthreads();
  const bool mapped = eplb.l2p != nullptr;
  const bool record = mapped && eplb.expert_load != nullptr && eplb.record_flag != nullptr &&
                      *eplb.record_flag != 0;
  const int unpadded = (mapped && eplb.num_unpadded != nullptr) ? *eplb.num_unpadded : T;
  const int64_t total = (int64_t)T * k;
#pragma unroll
  for (int s = 0; s < kSubRounds; ++s) {
    const int64_t slot = (int64_t)blockIdx.x * kRouteChunk + s * kRouteThreads + tid;
    if (slot >= total) continue;
    const int t = (int)(slot / k);
    int64_t id = topk_ids[slot];
    float w = topk_w[slot];
    if (is_padding != nullptr && is_padding[t] != 0) {
      id = -1;
      w = 0.0f;
    }
    if (mapped && id >= 0 && id < eplb.num_logical) {
      const int c = min(eplb.replica_count[id], eplb.map_stride);
      id = c > 0 ? (int64_t)eplb.l2p[id * eplb.map_stride + t % c] : -1;
      if (record && t < unpadded && id >= 0 && id < E) atomicAdd(&load[id], 1);
    }
    idx_out[slot] = id;
    w_out[slot] = w;
    if (id >= 0 && id < E) atomicAdd(&h[id], 1);
  }
  __syncthreads();
  for (int i = tid; i < E; i += kRouteThreads) {
    hist[(int64_t)blockIdx.x * E + i] = h[i];
    if (record && load[i] != 0) atomicAdd(&eplb.expert_load[i], load[i]);
  }
}

// Inclusive scan of one value per thread over a 1024-thread block.
__device__ int block_inclusive_scan(int v, int* buf) {
  const int tid = threadIdx.x;
  buf[tid] = v;
  __syncthreads();
  for (int d = 1; d < 1024; d <<= 1) {
    const int add = tid >= d ? buf[tid - d] : 0;
    __syncthreads();
    buf[tid] += add;
    __syncthreads();
  }
  const int r = buf[tid];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(1024) void route_scan_kernel(
    int32_t* __restrict__ hist, int nblocks, int E, const int32_t* __restrict__ counts_in,
    int max_tokens, int tile_m, int max_tiles, int32_t* __restrict__ expert_num_tokens,
    int32_t* __restrict__ expert_offsets, int32_t* __restrict__ tile_list) {
  __shared__ int buf[1024];
  __shared__ int tiles[1024];
  __shared__ int order[1024];
  const int e = threadIdx.x;
  int cnt = 0;
  if (e < E) {
    // per-block bases (relative to the expert's first row)
    for (int b = 0; b < nblocks; ++b) {
      const int c = hist[(int64_t)b * E + e];
      hist[(int64_t)b * E + e] = cnt;
      cnt += c;
    }
  }
  const int incl = block_inclusive_scan(e < E ? cnt : 0, buf);
  int rows = cnt;
  if (counts_in != nullptr && e < E) rows = min(max(counts_in[e], 0), max_tokens);
  const int nt = e < E ? (rows + tile_m - 1) / tile_m : 0;
  if (e < E) {
    expert_offsets[e] = incl - cnt;
    expert_num_tokens[e] = counts_in != nullptr ? rows : cnt;
    if (e == E - 1) expert_offsets[E] = incl;
  }
  tiles[e] = nt;
  __syncthreads();
  // heavy-first order: rank by tile count descending, ties by expert id
  if (e < E) {
    int rank = 0;
    for (int o = 0; o < E; ++o) {
      const int to = tiles[o];
      rank += (to > nt || (to == nt && o < e)) ? 1 : 0;
    }
    order[rank] = e;
  }
  __syncthreads();
  const int mine = e < E ? tiles[order[e]] : 0;
  const int incl_t = block_inclusive_scan(mine, buf);
  // group e (the e-th heaviest expert) owns tiles [group_off[e], group_off[e+1])
  int32_t* group_off = tile_list + 1 + 2 * max_tiles;
  if (e < E) {
    const int ex = order[e];
    int pos = incl_t - mine;
    group_off[e] = pos;
    for (int i = 0; i < mine; ++i, ++pos) {
      tile_list[1 + 2 * pos] = ex;
      tile_list[2 + 2 * pos] = i * tile_m;
    }
    if (e == E - 1) {
      tile_list[0] = incl_t;
      group_off[E] = incl_t;
    }
  }
}

__global__ __launch_bounds__(kRouteThreads) void route_scatter_kernel(
    const int64_t* __restrict__ idx, int T, int k, int E, const int32_t* __restrict__ hist_base,
    const int32_t* __restrict__ expert_offsets, int max_tokens, int32_t* __restrict__ row_src,
    int32_t* __restrict__ slot_row) {
  extern __shared__ int32_t pos[];  // [E] next row of each expert in this block
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const bool contiguous = max_tokens == 0;
  for (int i = tid; i < E; i += kRouteThreads)
    pos[i] = (contiguous ? expert_offsets[i] : 0) + hist_base[(int64_t)blockIdx.x * E + i];
  __syncthreads();
  const int64_t total = (int64_t)T * k;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int s = 0; s < kSubRounds; ++s) {
    const int64_t slot = (int64_t)blockIdx.x * kRouteChunk + s * kRouteThreads + tid;
    const int64_t id64 = slot < total ? idx[slot] : -1;
    const bool valid = id64 >= 0 && id64 < E;
    const int id = valid ? (int)id64 : 0;
    // lanes of this wave holding the same expert id
    uint64_t same = __ballot(valid);
    for (int b = 0; b < 11; ++b) {
      const bool bit = (id >> b) & 1;
      const uint64_t m = __ballot(bit);
      same &= bit ? m : ~m;
    }
    const int before = __popcll(same & below);
    const bool leader = valid && before == 0;
    for (int w = 0; w < kRouteThreads / 64; ++w) {
      if (wave == w && valid) {
        const int base = pos[id];
        const int r = base + before;
        if (leader) pos[id] = base + __popcll(same);
        if (contiguous) {
          row_src[r] = (int)(slot / k);
          slot_row[slot] = r;
        } else {
          slot_row[slot] = r < max_tokens ? id * max_tokens + r : -1;
        }
      }
      __syncthreads();
    }
    if (!valid && slot < total) slot_row[slot] = -1;
  }
}

// Indexed layout ("...fused_humming_moe", HummingIndexedExperts: the
// outputs of moe_align_block_size, whose body the pages do not show).
// Each expert's routed slots, in the contiguous layout's row order, fill a
// segment of sorted_ids padded with numel to a multiple of the block size;
// segments follow in expert order and empty experts have none.  Every block
// scans the padded counts (E <= 1024) into LDS and places its 1024 slots;
// block 0 also writes the expert of every block, the padding and the total.
constexpr int kAlignThreads = 1024;

__global__ __launch_bounds__(kAlignThreads) void align_kernel(
    const int64_t* __restrict__ idx, const int32_t* __restrict__ slot_row,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets, int total, int E,
    int bs, int32_t* __restrict__ sorted_ids, int32_t* __restrict__ expert_ids,
    int32_t* __restrict__ num_padded) {
  __shared__ int32_t scan[kAlignThreads];
  const int t = threadIdx.x;
  const int cnt = t < E ? counts[t] : 0;
  const int pc = (cnt + bs - 1) / bs * bs;
  scan[t] = pc;
  __syncthreads();
  for (int d = 1; d < kAlignThreads; d <<= 1) {   // inclusive Hillis-Steele scan
    const int v = t >= d ? scan[t - d] : 0;
    __syncthreads();
    scan[t] += v;
    __syncthreads();
  }
  if (blockIdx.x == 0) {
    const int end = scan[t], start = end - pc;
    if (t < E) {
      for (int b = start / bs; b < end / bs; ++b) expert_ids[b] = t;
      for (int q = start + cnt; q < end; ++q) sorted_ids[q] = total;
    }
    if (t == kAlignThreads - 1) *num_padded = end;
  }
  const int slot = blockIdx.x * kAlignThreads + t;
  if (slot >= total) return;
  const int r = slot_row[slot];
  if (r < 0) return;
  const int64_t e = idx[slot];
  if (e < 0 || e >= E) return;
  sorted_ids[scan[e] - ((counts[e] + bs - 1) / bs * bs) + (r - offsets[e])] = slot;
}

}  // namespace

hipError_t launch_align(const int64_t* idx, const int32_t* slot_row, const int32_t* counts,
                        const int32_t* offsets, int T, int k, int E, int block_size,
                        int32_t* sorted_ids, int32_t* expert_ids, int32_t* num_padded,
                        hipStream_t stream) {
  const int total = T * k;
  const int blocks = total > 0 ? (total + kAlignThreads - 1) / kAlignThreads : 1;
  align_kernel<<<blocks, kAlignThreads, 0, stream>>>(idx, slot_row, counts, offsets, total, E,
                                                     block_size, sorted_ids, expert_ids,
                                                     num_padded);
  return hipGetLastError();
}

hipError_t launch_route(const int32_t* topk_ids, const float* topk_w, const uint8_t* is_padding,
                        int T, int k, int E, const EplbArgs& eplb, int64_t* idx_out,
                        float* w_out, int32_t* hist, const int32_t* counts_in, int max_tokens,
                        int tile_m, int max_tiles, int32_t* expert_num_tokens,
                        int32_t* expert_offsets, int32_t* row_src, int32_t* slot_row,
                        int32_t* tile_list, hipStream_t stream) {
  const int64_t total = (int64_t)T * k;
  const int nblocks = (int)((total + kRouteChunk - 1) / kRouteChunk);
  if (nblocks > 0) {
    route_repack_hist_kernel<<<nblocks, kRouteThreads, 2 * E * sizeof(int32_t), stream>>>(
        topk_ids, topk_w, is_padding, T, k, E, eplb, idx_out, w_out, hist);
  }
  route_scan_kernel<<<1, 1024, 0, stream>>>(hist, nblocks, E, counts_in, max_tokens, tile_m,
                                            max_tiles, expert_num_tokens, expert_offsets,
                                            tile_list);
  if (nblocks > 0) {
    route_scatter_kernel<<<nblocks, kRouteThreads, E * sizeof(int32_t), stream>>>(
        idx_out, T, k, E, hist, expert_offsets, counts_in != nullptr ? max_tokens : 0, row_src,
        slot_row);
  }
  return hipGetLastError();
}

}  // namespace moe
