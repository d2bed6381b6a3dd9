// Internal launchers of the gfx950 kernels (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// activation quantization schemes (values match moe_quant_t)
constexpr int kQuantUe8m0 = 0;   // per-128 groups, E8M0 scale bytes
constexpr int kQuantF32 = 1;     // per-128 groups, fp32 scales
constexpr int kQuantBf16 = 2;    // unquantized copy
constexpr int kQuantMxfp8 = 3;   // per-32 groups, E8M0 scale bytes
// weight schemes (values match moe_weight_t)
constexpr int kWeightBlock128 = 0;   // e4m3, fp32 scale per 128x128 block
constexpr int kWeightMxfp8 = 1;      // e4m3, E8M0 scale per row and 32 columns
constexpr int kWeightMxfp4 = 2;      // e2m1 (two per byte), E8M0 per row and 32 columns
// GEMM scale scheme beyond the activation schemes: MXFP8 activations with
// e2m1 weights
constexpr int kSchemeMxfp8W4 = 4;

// GEMM tiles of 160 rows (block scheme only) hold the fp32 weight-scale
// panel of at most this many k-steps beside their 3-slot ring: reductions
// of up to 192 * 128 = 24576
constexpr int kTile160MaxGroups = 192;

// routing: slots handled per block of the count / scatter kernels
constexpr int kRouteChunk = 1024;
constexpr int kRouteThreads = 256;

struct EplbArgs {
  const int32_t* l2p;            // [num_logical, map_stride] or nullptr
  int map_stride;
  const int32_t* replica_count;  // [num_logical]
  int num_logical;
  int32_t* expert_load;          // [E] or nullptr
  const int32_t* record_flag;    // [1] device, or nullptr
  const int32_t* num_unpadded;   // [1] device, or nullptr
};

// Grouped GEMM problem for one launch (w13 or w2).
struct GemmArgs {
  const uint8_t* a;          // activation codes, rows of Kd bytes
  uint32_t a_bytes;          // size of the activation-code buffer (< 2^32)
  const void* a_sf;          // activation scales (UE8M0 bytes or fp32) per row
  uint32_t a_sf_bytes;       // size of the activation-scale buffer (< 2^32)
  int a_sf_stride;           // scale row length: bytes (UE8M0) or floats (fp32)
  const uint8_t* w;          // weight codes [E, Nout, Kd]
  const void* w_sf;          // weight scales: fp32 [E, Nout/128, Kd/128] (block),
                             //   E8M0 bytes [E, Nout, Kd/32] (MX)
  uint16_t* out;             // bf16 [rows, Nout] (plain GEMM)
  uint8_t* act_q;            // fused activation: fp8 [rows, Nout/2]
  uint8_t* act_sf;           //   and its per-128 scales (UE8M0 bytes or fp32)
  int act_sf_row;            //   scale row length: bytes (UE8M0) or floats (fp32)
  // [0] tile count, [1] group count, [2..3] 0, then per tile 8 ints: expert, first
  // row within the expert, first tile and size of its group (one expert's
  // consecutive m-tiles, groups in XCD-balanced order), the expert's rows,
  // its first row in the GEMM's row space (contiguous offset or slab), its
  // first block in the indexed layout's block map (blocks of the main
  // list's tile height, every expert counted), 0
  const int32_t* tile_list;
  int num_experts;
  const int32_t* row_src;    // A row gather (w13 on the contiguous layout) or nullptr
  // indexed layout (sorted_ids != nullptr): tile b is the block of BM rows
  // [b*BM, (b+1)*BM) of sorted_ids, of expert expert_ids[b]; entries not
  // below numel are padding and come after the block's routed entries.
  // row_src unused; tile_list, when given (block size = the routing's tile
  // height), orders the blocks: the schedule's tile (e, m-tile i) is block
  // first-block(e) + i; a tile of the tall list (BM = twice the block size)
  // covers positions first-block(e) * block_size + m0 + [0, rows) instead.
  const int32_t* sorted_ids;
  const int32_t* expert_ids;
  const int32_t* num_padded;       // [1] device: the padded total
  int max_blocks;                  // blocks of sorted_ids (bounds *num_padded)
  int block_size;                  // the block map's block size (indexed layout)
  int top_k;                       // w13: the routing's top_k; w2: 1
  int numel;                       // T * top_k
  int gather_sorted;               // A row = sorted_ids[pos] / top_k; else pos
  int scatter_sorted;              // output row = sorted_ids[pos] (padding skipped)
  int activation;             // ACT epilogue: a gated activation kind (moe_act_t)
  float act_limit;            //   and its clamp limit (apply_act)
  int Kd;                    // reduction length, multiple of 128
  int Nout;                  // output columns, multiple of 128
  // split-K (plain GEMM only; 1 = none): the k-steps are cut into ksplit
  // ranges of a multiple of 4 k-steps each; split s of (tile, n-tile) item q
  // stores its fp32 partial at part + (s * part_rows + row) * Nout, then
  // takes a ticket from counters[q] (q = tile * (Nout / BN) + n-tile); the
  // block that draws the last ticket adds the partials in split order,
  // rounds once to bf16 and sets the counter back to 0.  The counters must
  // be 0 at launch.
  int ksplit;
  float* part;
  int64_t part_rows;
  int32_t* counters;
  // item order inside a group of m-tiles: super-columns of sn n-tiles, each
  // walked m-tile-major (sn = 1: n-tile-major); set by the launcher
  int sn;
  // 1: 256 output columns for the unfused GEMMs' 128-row tiles whatever the
  // scheme (set when the experts above 128 rows have their own tile list)
  int wide;
  // k-step rotation key: output column c belongs to pair (c mod rot_period)
  // / 256 (the caller: Nout, or N for a gated w13 whose gate and up halves
  // share pairs; 0 = never rotate); krot (set by the launcher) turns the
  // rotation on
  int rot_period;
  int krot;
  // 1: each XCD walks its slice of the tile list in the zipper order (heavy
  // groups from the front, light ones from the back); 0: in list order
  int zip;
  // 1: plain GEMM at 128-row tiles computes two neighbouring 256-column
  // n-tiles per block (per-128 scale schemes, Nout % 512 == 0, no split;
  // otherwise ignored)
  int pair;
};

// zero n int32 (a fill kernel: safe under graph capture)
hipError_t launch_zero_i32(int32_t* p, int64_t n, hipStream_t stream);

// Staging on its own launch: the bf16 copy.  fp8 staging runs inside
// launch_route (StageQuant); here it returns hipErrorInvalidValue.
hipError_t launch_stage_quant(const void* x, void* xq, void* xsf, int64_t rows, int K, int quant,
                              const int32_t* counts, int max_tokens, hipStream_t stream);

// act: activation kind (moe_act_t); gate_up rows are 2N wide for gated
// kinds, N for the _no_mul ones
hipError_t launch_act_requant(const void* gate_up, void* aq, void* asf, int64_t rows_cap, int N,
                              int quant, const int32_t* num_rows, const int32_t* counts,
                              int max_tokens, int act, float act_limit, hipStream_t stream);

// Optional: the hidden states' group quantization run inside the routing
// scan's launch: groups of 128 (UE8M0 or fp32 scales) or 32 (MXFP8, E8M0);
// rows: staged rows ([T] or [E * max_tokens], masked by the counts).
struct StageQuant {
  const void* x;
  void* xq;
  void* xsf;
  int64_t rows;
  int K;
  int group;
  bool ue8m0;
};

// The GEMM tile schedules the routing scan writes: the main list (tiles of
// tile_m rows, capacity max_tiles) and, when tall is set, a second list of
// 2 * tile_m-row tiles that takes every expert of more than tile_m rows
// (those are then absent from the main list).  hist: the per-block expert
// histograms; hist_base: where the scan writes the per-block bases the
// scatter reads (hist itself, or a separate array of the same size when
// there is a tall list: a second block then builds it from hist's counts).
struct TileLists {
  int tile_m;
  int max_tiles;
  int32_t* list;
  int max_tiles_tall;
  int32_t* tall;      // nullptr: one list
};

hipError_t launch_route(const int32_t* topk_ids, const float* topk_w, const uint8_t* is_padding,
                        int T, int k, int E, const EplbArgs& eplb, int64_t* idx_out,
                        float* w_out, int32_t* hist, int32_t* hist_base,
                        const int32_t* counts_in, int max_tokens, const TileLists& tl, int32_t* expert_num_tokens,
                        int32_t* expert_offsets, int32_t* row_src, int32_t* slot_row,
                        hipStream_t stream, const StageQuant* sq = nullptr);

// quant: the scale scheme: an activation scheme (kQuant*; kQuantMxfp8 with
// e4m3 MX weights) or kSchemeMxfp8W4 (MXFP8 activations, e2m1 MX weights).
// act = false: out = bf16 GEMM result.  act = true (w13 only): the result's
// gate half [0, Nout/2) and up half [Nout/2, Nout) are combined into
// silu(gate) * up and quantized per group (128, or 32 for MX) into act_q /
// act_sf; nothing is written to out.
// One object per scheme (grouped_gemm.hip built with MOE_GEMM_SCHEME = SC).
template <int SC>
hipError_t launch_grouped_gemm_sc(const GemmArgs& args, int tile_m, int max_tiles, bool act,
                                  hipStream_t stream);
extern template hipError_t launch_grouped_gemm_sc<kQuantUe8m0>(const GemmArgs&, int, int, bool,
                                                               hipStream_t);
extern template hipError_t launch_grouped_gemm_sc<kQuantF32>(const GemmArgs&, int, int, bool,
                                                             hipStream_t);
extern template hipError_t launch_grouped_gemm_sc<kQuantBf16>(const GemmArgs&, int, int, bool,
                                                              hipStream_t);
extern template hipError_t launch_grouped_gemm_sc<kQuantMxfp8>(const GemmArgs&, int, int, bool,
                                                               hipStream_t);
extern template hipError_t launch_grouped_gemm_sc<kSchemeMxfp8W4>(const GemmArgs&, int, int, bool,
                                                                  hipStream_t);
inline hipError_t launch_grouped_gemm(const GemmArgs& args, int tile_m, int max_tiles, int quant,
                                      bool act, hipStream_t stream) {
  switch (quant) {
    case kQuantUe8m0: return launch_grouped_gemm_sc<kQuantUe8m0>(args, tile_m, max_tiles, act, stream);
    case kQuantF32: return launch_grouped_gemm_sc<kQuantF32>(args, tile_m, max_tiles, act, stream);
    case kQuantBf16: return launch_grouped_gemm_sc<kQuantBf16>(args, tile_m, max_tiles, act, stream);
    case kQuantMxfp8: return launch_grouped_gemm_sc<kQuantMxfp8>(args, tile_m, max_tiles, act, stream);
    case kSchemeMxfp8W4:
      return launch_grouped_gemm_sc<kSchemeMxfp8W4>(args, tile_m, max_tiles, act, stream);
    default: return hipErrorInvalidValue;
  }
}

// blocks of the reduce kernels' one-dimensional grid (must be < 2^31)
int64_t reduce_blocks(int T, int K);

hipError_t launch_topk_reduce(const void* down, const int32_t* slot_row, const float* w, void* out,
                              int T, int k, int K, hipStream_t stream);

// down rows in (token, slot) order; a slot counts when idx is in [0, E)
hipError_t launch_fused_mul_sum(const void* down, const int64_t* idx, const float* w, void* out,
                                int T, int k, int K, int E, hipStream_t stream);

// indexed layout from the contiguous routing: sorted_ids [T*k + E*(block_size-1)
// rounded down to a block multiple], expert_ids [that / block_size]
hipError_t launch_align(const int64_t* idx, const int32_t* slot_row, const int32_t* counts,
                        const int32_t* offsets, int T, int k, int E, int block_size,
                        int32_t* sorted_ids, int32_t* expert_ids, int32_t* num_padded,
                        hipStream_t stream);

}  // namespace moe
