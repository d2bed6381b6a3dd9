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
#include <limits.h>

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

// Inclusive scan of one value per thread over a 1024-thread block: each wave
// scans its 64 values with lane shuffles, wave 0 scans the 16 wave totals,
// every thread adds its wave's offset.  buf needs 32 ints and is free again
// when the function returns.
__device__ int block_inclusive_scan(int v, int* buf) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int t = __shfl_up(v, d);
    if (lane >= d) v += t;
  }
  if (lane == 63) buf[wave] = v;
  __syncthreads();
  if (wave == 0) {
    int w = lane < 16 ? buf[lane] : 0;
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) {
      const int t = __shfl_up(w, d);
      if (lane >= d) w += t;
    }
    if (lane < 16) buf[16 + lane] = w;
  }
  __syncthreads();
  const int r = v + (wave > 0 ? buf[16 + wave - 1] : 0);
  __syncthreads();
  return r;
}

// M-tile schedule for the grouped GEMMs.  The GEMM hands its 1-D work list
// to the 8 XCDs in 8 equal contiguous ranges (block L runs on XCD L % 8), so
// the list is ordered to give every range the same mix: each expert's
// m-tiles are cut into chunks of at most S tiles (S = 8, more only when
// there would be over 1024 chunks), the chunks sorted by size class (full
// chunks first in expert order, then the remainders r by the class
// floor(8r / S), largest first, ties by expert; for S = 8 the class is the
// size), and dealt in rounds of 8: the round's first chunk to the bin with
// the fewest tiles so far, and so on (round-based longest-processing-time).  Bins are concatenated.  Every range then holds
// about the same number of tiles (MFMA work) and of weight chunks (HBM
// bytes); a heaviest-expert-first list instead left some XCDs streaming most
// of the weights while others did most of the arithmetic.
constexpr int kChunkCap = 2048;

// role 0: per-block bases (into hist_base, which may be hist itself),
// offsets, counts and the main tile list; role 1: the tall list alone (run
// by a second block of the same launch, reading hist's counts, so hist_base
// must then be a separate array).
__device__ __forceinline__ void route_scan_body(
    int role, int32_t* __restrict__ hist, int32_t* __restrict__ hist_base, int nblocks, int E,
    const int32_t* __restrict__ counts_in, int max_tokens, const TileLists tl,
    int32_t* __restrict__ expert_num_tokens, int32_t* __restrict__ expert_offsets) {
  __shared__ int buf[1024];
  __shared__ int wcnt[16][8];      // remainder chunks per wave and size class
  __shared__ int woff[16][8];      // their first index
  __shared__ int chunk_e[kChunkCap], chunk_m[kChunkCap], chunk_n[kChunkCap];
  __shared__ int chunk_bin[kChunkCap], chunk_off[kChunkCap], chunk_idx[kChunkCap];
  __shared__ int bin_load[8], bin_cnt[8];
  __shared__ int exp_rows[1024], exp_base[1024];   // per expert: GEMM rows, first row
  __shared__ int exp_tile0[1024];                   // its first block of the block map
  const int e = threadIdx.x;
  int cnt = 0;
  if (e < E) {
    // per-block bases (relative to the expert's first row); the counts are
    // loaded 16 blocks at a time so their latencies overlap
    for (int b0 = 0; b0 < nblocks; b0 += 16) {
      int c[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) c[j] = b0 + j < nblocks ? hist[(int64_t)(b0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if (role == 0 && b0 + j < nblocks) hist_base[(int64_t)(b0 + j) * E + e] = cnt;
        cnt += c[j];
      }
    }
  }
  const int incl = block_inclusive_scan(e < E ? cnt : 0, buf);
  int rows = cnt;
  if (counts_in != nullptr && e < E) rows = min(max(counts_in[e], 0), max_tokens);
  if (role == 0 && e < E) {
    expert_offsets[e] = incl - cnt;
    expert_num_tokens[e] = counts_in != nullptr ? rows : cnt;
    if (e == E - 1) expert_offsets[E] = incl;
  }
  exp_rows[e] = rows;
  exp_base[e] = counts_in != nullptr ? e * max_tokens : incl - cnt;
  // the expert's first m-tile in expert order counting every expert's
  // tiles of tile_m rows (in both lists): its first block in the indexed
  // layout's block map when the block size is tile_m
  {
    const int nt_all = e < E ? (rows + tl.tile_m - 1) / tl.tile_m : 0;
    exp_tile0[e] = block_inclusive_scan(nt_all, buf) - nt_all;
  }
  // one list: nt m-tiles of tile_m rows for this thread's expert (0: not in
  // this list); block-uniform arguments otherwise
  auto schedule = [&](const int nt, const int tile_m, const int max_tiles,
                      int32_t* __restrict__ tile_list) {
  const int incl_nt = block_inclusive_scan(nt, buf);
  // the last thread's inclusive value is the total: broadcast it
  if (e == 1023) buf[0] = incl_nt;
  __syncthreads();
  const int total = buf[0];
  __syncthreads();
  const int S = max(8, (total + 1023) / 1024);
  const int full = nt / S, r = nt % S;
  const int fstart = block_inclusive_scan(full, buf) - full;
  if (e == 1023) bin_load[0] = fstart + full;      // F, the number of full chunks
  // remainder chunks: counting sort by size class with one ballot per class
  const int lane = e & 63, wave = e >> 6;
  const int cls = r > 0 ? (r * 8) / S : -1;
  int rank_w = 0;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const uint64_t m = __ballot(cls == c);
    if (lane == 0) wcnt[wave][c] = __popcll(m);
    if (cls == c) rank_w = __popcll(m & ((1ull << lane) - 1ull));
  }
  __syncthreads();
  const int F = bin_load[0];
  if (e < 128) {
    // first index of (wave w, class c): F, then the classes above c, then the
    // waves before w within class c
    const int w = e >> 3, c = e & 7;
    int off = F;
    for (int c2 = c + 1; c2 < 8; ++c2)
      for (int w2 = 0; w2 < 16; ++w2) off += wcnt[w2][c2];
    for (int w2 = 0; w2 < w; ++w2) off += wcnt[w2][c];
    woff[w][c] = off;
  }
  __syncthreads();
  const int ridx = cls >= 0 ? woff[wave][cls] + rank_w : 0;
  for (int j = 0; j < full; ++j) {
    chunk_e[fstart + j] = e;
    chunk_m[fstart + j] = j * S;
    chunk_n[fstart + j] = S;
  }
  if (r > 0) {
    chunk_e[ridx] = e;
    chunk_m[ridx] = full * S;
    chunk_n[ridx] = r;
  }
  const int C = F + block_inclusive_scan(r > 0 ? 1 : 0, buf);   // valid in thread 1023
  if (e == 1023) bin_cnt[0] = C;
  __syncthreads();
  const int nchunks = bin_cnt[0];
  __syncthreads();
  // round-based dealing by wave 0; lane x < 8 is bin x.  Lane y also holds
  // the size of the round's chunk y (loaded one round ahead).
  if (e < 64) {
    int load = 0, count = 0;
    const int rounds = (nchunks + 7) / 8;
    int sz = e < 8 && e < nchunks ? chunk_n[e] : 0;
    int rank = e;            // all loads 0: bin x has rank x
    bool uniform = true;     // the previous round's chunks were all one size
    for (int rd = 0; rd < rounds; ++rd) {
      const int nxt = 8 * (rd + 1) + e;
      const int sz_next = e < 8 && nxt < nchunks ? chunk_n[nxt] : 0;
      // After a round whose chunks all had one size every bin grew by the
      // same amount and the ranking stands; otherwise rank the loads again
      // (through scalar registers: no LDS round trip on this serial path).
      if (!uniform) {
        rank = 0;
#pragma unroll
        for (int y = 0; y < 8; ++y) {
          const int ly = __builtin_amdgcn_readlane(load, y);
          rank += (ly < load || (ly == load && y < e)) ? 1 : 0;
        }
      }
      // the size of this bin's chunk, and whether the round is full and of
      // one size (then the next round keeps the ranking)
      int mine = 0, smin = INT_MAX, smax = 0;
#pragma unroll
      for (int y = 0; y < 8; ++y) {
        const int sy = __builtin_amdgcn_readlane(sz, y);
        mine = rank == y ? sy : mine;
        smin = min(smin, sy);
        smax = max(smax, sy);
      }
      uniform = smin == smax && 8 * rd + 7 < nchunks;
      const int i = 8 * rd + rank;
      if (e < 8 && i < nchunks) {
        chunk_bin[i] = e;
        chunk_off[i] = load;
        chunk_idx[i] = count;
        load += mine;
        count += 1;
      }
      sz = sz_next;
    }
    if (e < 8) {
      bin_load[e] = load;
      bin_cnt[e] = count;
    }
  }
  __syncthreads();
  int32_t* info = tile_list + 4;                     // 16-byte aligned
  int32_t* group_off = tile_list + 4 + 8 * max_tiles;
  for (int i = e; i < nchunks; i += 1024) {
    const int x = chunk_bin[i];
    int tile0 = chunk_off[i], g = chunk_idx[i];
    for (int y = 0; y < x; ++y) {
      tile0 += bin_load[y];
      g += bin_cnt[y];
    }
    group_off[g] = tile0;
    const int ex = chunk_e[i], n = chunk_n[i];
    for (int t = 0; t < n; ++t) {
      // expert, first row, its group's first tile and size, the expert's
      // rows, its first row in the GEMM's row space and its first block in
      // the indexed layout's block map of tile_m-row blocks (every expert's
      // blocks counted, whichever list it is in)
      int4* d = reinterpret_cast<int4*>(info + 8 * (tile0 + t));
      d[0] = make_int4(ex, (chunk_m[i] + t) * tile_m, tile0, n);
      d[1] = make_int4(exp_rows[ex], exp_base[ex], exp_tile0[ex], 0);
    }
  }
  if (e == 0) {
    tile_list[0] = total;
    tile_list[1] = nchunks;
    tile_list[2] = 0;
    tile_list[3] = 0;
    group_off[nchunks] = total;
  }
  };
  // with a tall list, experts of more than tile_m rows go there (role 1),
  // in tiles of 2 * tile_m rows; the rest (or every expert) to the main list
  const bool in_tall = tl.tall != nullptr && e < E && rows > tl.tile_m;
  if (role == 0) {
    schedule(e < E && !in_tall ? (rows + tl.tile_m - 1) / tl.tile_m : 0, tl.tile_m,
             tl.max_tiles, tl.list);
  } else {
    const int th = 2 * tl.tile_m;
    schedule(in_tall ? (rows + th - 1) / th : 0, th, tl.max_tiles_tall, tl.tall);
  }
}

// one block per tile list (block 1: the tall list)
__global__ __launch_bounds__(1024) void route_scan_kernel(
    int32_t* __restrict__ hist, int32_t* __restrict__ hist_base, int nblocks, int E,
    const int32_t* __restrict__ counts_in, int max_tokens, const TileLists tl,
    int32_t* __restrict__ expert_num_tokens, int32_t* __restrict__ expert_offsets) {
  route_scan_body((int)blockIdx.x, hist, hist_base, nblocks, E, counts_in, max_tokens, tl,
                  expert_num_tokens, expert_offsets);
}

// The scan is one block of latency-bound work per tile list; the hidden
// states' group quantization is independent of it and bandwidth-bound.
// Block 0 (and block 1 for the tall list) runs the scan while the other
// blocks quantize, so the scan hides under the quantization's memory
// stream: one launch instead of two back to back.
// The quantizing blocks are as many as the chip holds at once (or fewer)
// and stride over the groups, 1024 / (GROUP / 16) consecutive groups per
// pass, every block making the same number of passes: no half-empty last
// wave of blocks.  Measured against torch's own bf16 -> fp8 cast of the
// same tensor (the same bytes read and written, no scales): DSv3-shaped
// prefill 20.0 us vs 20.1 us (one block per 128 groups, not striding: 21-22
// us); two or four slabs per pass with all their loads issued first were
// slower (22.2 / 23.4 us; Qwen3-shaped 45.1 / 54.0 us against 41.6 us).
template <int GROUP, bool UE8M0>
__global__ __launch_bounds__(1024) void route_scan_quant_kernel(
    int32_t* __restrict__ hist, int32_t* __restrict__ hist_base, int nblocks, int E,
    const int32_t* __restrict__ counts_in, int max_tokens, const TileLists tl,
    int32_t* __restrict__ expert_num_tokens, int32_t* __restrict__ expert_offsets,
    const uint16_t* __restrict__ x, uint8_t* __restrict__ xq, uint8_t* __restrict__ xsf,
    int64_t num_groups, int G, int sf_row_len) {
  // blocks 0 (and 1 with a tall list) build the tile lists, the rest quantize
  const int nscan = tl.tall != nullptr ? 2 : 1;
  if ((int)blockIdx.x < nscan) {
    route_scan_body((int)blockIdx.x, hist, hist_base, nblocks, E, counts_in, max_tokens, tl,
                    expert_num_tokens, expert_offsets);
    return;
  }
  constexpr int LANES = GROUP / 16;
  constexpr int GPB = 1024 / LANES;                 // groups of one pass
  const int lane = threadIdx.x % LANES;
  const int64_t stride = (int64_t)(gridDim.x - nscan) * GPB;
  for (int64_t gid = (int64_t)(blockIdx.x - nscan) * GPB + threadIdx.x / LANES; gid < num_groups;
       gid += stride) {
    if (!row_live(gid / G, counts_in, max_tokens)) continue;
    quantize_group_chunk<GROUP, UE8M0>(load_group_chunk<GROUP>(x, gid, lane), xq, xsf, gid,
                                       lane, G, sf_row_len);
  }
}

// Compute units of the current device (cached per device).
int device_cus() {
  static int cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cus[dev] = n;
  }
  return cus[dev];
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
  __shared__ int buf[32];
  const int t = threadIdx.x;
  const int cnt = t < E ? counts[t] : 0;
  const int pc = (cnt + bs - 1) / bs * bs;
  scan[t] = block_inclusive_scan(pc, buf);
  __syncthreads();
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
                        float* w_out, int32_t* hist, int32_t* hist_base,
                        const int32_t* counts_in, int max_tokens,
                        const TileLists& tl, int32_t* expert_num_tokens,
                        int32_t* expert_offsets, int32_t* row_src, int32_t* slot_row,
                        hipStream_t stream, const StageQuant* sq) {
  const int64_t total = (int64_t)T * k;
  const int nblocks = (int)((total + kRouteChunk - 1) / kRouteChunk);
  if (nblocks > 0) {
    route_repack_hist_kernel<<<nblocks, kRouteThreads, 2 * E * sizeof(int32_t), stream>>>(
        topk_ids, topk_w, is_padding, T, k, E, eplb, idx_out, w_out, hist);
  }
  if (sq != nullptr && sq->rows > 0) {
    // the hidden states' group quantization rides along with the scan
    const int G = sq->K / sq->group;
    const int64_t ng = sq->rows * G;
    // passes spread evenly over at most two 1024-thread blocks per CU (the
    // residency limit: the scan's LDS)
    const int64_t per_pass = 1024 / (sq->group / 16);
    const int64_t passes = (ng + per_pass - 1) / per_pass;
    const int nscan = tl.tall != nullptr ? 2 : 1;
    const int64_t resident = 2 * (int64_t)device_cus() - nscan;
    const int64_t rounds = (passes + resident - 1) / resident;
    const unsigned grid = (unsigned)(nscan + (passes + rounds - 1) / rounds);
    const uint16_t* x = (const uint16_t*)sq->x;
    uint8_t* xq = (uint8_t*)sq->xq;
    uint8_t* xsf = (uint8_t*)sq->xsf;
    if (sq->group == 32)
      route_scan_quant_kernel<32, true><<<grid, 1024, 0, stream>>>(
          hist, hist_base, nblocks, E, counts_in, max_tokens, tl, expert_num_tokens,
          expert_offsets, x, xq, xsf, ng, G, G);
    else if (sq->ue8m0)
      route_scan_quant_kernel<128, true><<<grid, 1024, 0, stream>>>(
          hist, hist_base, nblocks, E, counts_in, max_tokens, tl, expert_num_tokens,
          expert_offsets, x, xq, xsf, ng, G, 4 * ((G + 3) / 4));
    else
      route_scan_quant_kernel<128, false><<<grid, 1024, 0, stream>>>(
          hist, hist_base, nblocks, E, counts_in, max_tokens, tl, expert_num_tokens,
          expert_offsets, x, xq, xsf, ng, G, 4 * ((G + 3) / 4));
  } else {
    route_scan_kernel<<<tl.tall != nullptr ? 2 : 1, 1024, 0, stream>>>(
        hist, hist_base, nblocks, E, counts_in, max_tokens, tl, expert_num_tokens,
        expert_offsets);
  }
  if (nblocks > 0) {
    route_scatter_kernel<<<nblocks, kRouteThreads, E * sizeof(int32_t), stream>>>(
        idx_out, T, k, E, hist_base, expert_offsets, counts_in != nullptr ? max_tokens : 0, row_src,
        slot_row);
  }
  return hipGetLastError();
}

}  // namespace moe
