// Host side of the C ABI: argument validation, buffer planning, tile-size
// choice and the launch sequence of the layer on one stream.
//
// Validation follows the error conditions of prepare_megamoe_inputs and
// _resolve_hidden_quant ("vllm.model_executor.layers.fused_moe.
// prepare_megamoe": hidden size a multiple of 128, matching top-k shapes,
// scale buffer present iff quantizing, an empty batch is a no-op) and the
// experts' apply() preconditions ("...experts.fused_humming_moe": batched
// format needs expert_num_tokens).  The workspace plan mirrors
// HummingExpertsBase.get_buffer_metas / prepare_buffers, minus the gate_up
// buffer the fused w13 call never materializes.  Scheme pairs follow
// HummingExpertsBase._supports_quant_scheme.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <functional>
#include <mutex>
#include <string>

#include "../../include/moe_fp8.h"
#include "kernels.h"

// Workspace of moe_forward_static: one copy per GPU, in the library's code
// object, held until the process ends.  Host code never passes this name to
// a kernel (on the host it is a stand-in, not a device address): the device
// address comes from hipGetSymbolAddress, once per device
// (static_scratch_for_current_device below).
static __device__ __align__(256) uint8_t scratch[MOE_STATIC_SCRATCH_BYTES];

namespace {

thread_local std::string g_last_error;

moe_status_t fail(moe_status_t code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
moe_status_t fail(moe_status_t code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

moe_status_t ok() {
  g_last_error.clear();
  return MOE_OK;
}

moe_status_t launch_status(hipError_t err, const char* what) {
  if (err == hipSuccess) return ok();
  return fail(MOE_ERR_LAUNCH, "%s: kernel launch failed: %s", what, hipGetErrorString(err));
}

bool aligned(const void* ptr, size_t a) { return ((uintptr_t)ptr % a) == 0; }

constexpr size_t kAlign = 256;
size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool batched(const moe_problem_t* p) { return p->layout == MOE_LAYOUT_BATCHED_MASKED; }
bool indexed(const moe_problem_t* p) { return p->layout == MOE_LAYOUT_INDEXED; }
// gated activations: w13 has 2N rows (gate, up); the _no_mul ones: N rows
bool gated(const moe_problem_t* p) {
  return p->activation < MOE_ACT_SILU_NO_MUL || p->activation > MOE_ACT_RELU2_NO_MUL;
}
// The clamp limit the kernels apply: SWIGLUOAI / SWIGLUSTEP default to 7
// when none is given; SiLU clamps only with an explicit limit; the others
// take none.
constexpr float kSwigluDefaultLimit = 7.0f;
float effective_limit(const moe_problem_t* p) {
  if (p->activation == MOE_ACT_SWIGLUOAI || p->activation == MOE_ACT_SWIGLUSTEP)
    return p->act_limit > 0.0f ? p->act_limit : kSwigluDefaultLimit;
  return p->activation == MOE_ACT_SILU ? p->act_limit : 0.0f;
}
int64_t w13_rows(const moe_problem_t* p) { return (gated(p) ? 2 : 1) * (int64_t)p->intermediate; }

// 160-row GEMM tiles: block-scaled weights with fp8 activations, both
// reductions within the tiles' weight-scale panel
bool tile160_fits(const moe_problem_t* p) {
  return (p->act_quant == MOE_Q_FP8_UE8M0 || p->act_quant == MOE_Q_FP8_F32) &&
         p->hidden / 128 <= moe::kTile160MaxGroups &&
         p->intermediate / 128 <= moe::kTile160MaxGroups;
}

// Block sizes of the indexed layout: the GEMM tile heights.
bool valid_block_size(const moe_problem_t* p, int bs) {
  if (bs == 16 || bs == 32 || bs == 64 || bs == 128) return true;
  if (bs == 160) return tile160_fits(p);
  return (bs == 192 || bs == 256) && p->act_quant != MOE_Q_BF16;
}

// Entries of sorted_ids: every routed expert pads its segment by fewer than
// bs entries, so T*k + min(E, T*k) * (bs - 1), rounded down to whole blocks.
int64_t padded_capacity(const moe_problem_t* p, int64_t bs) {
  const int64_t slots = (int64_t)p->num_tokens * p->top_k;
  const int64_t cap = slots + std::min<int64_t>(p->num_experts, slots) * (bs - 1);
  return cap / bs * bs;
}

// Split-K of the w2 GEMM: its reduction length N alone decides, so a
// token's bits never depend on the batch.  Long reductions (N >= 8192, i.e.
// 64+ k-steps) are cut in two: their GEMMs have few, long work items when
// the experts have few rows (an 8-expert batch of 128 rows per expert has
// 8 x 16 items for 256 CUs).  MOE_KSPLIT = 1 | 2 | 4 overrides it for
// tuning runs (all calls of one layer must see the same value).
int w2_ksplit(const moe_problem_t* p) {
  const int G = p->intermediate / 128;
  int s = p->intermediate >= 8192 ? 2 : 1;
  const char* env = getenv("MOE_KSPLIT");
  if (env != nullptr) {
    const int v = atoi(env);
    if (v == 1 || v == 2 || v == 4) s = v;
  }
  while (s > 1 && G < 4 * s) s /= 2;   // each split at least 4 k-steps
  return s;
}

// Activation rows per GEMM tile, from the expected rows per expert.  Rows
// per expert below 16 leave a 16-row MFMA tile mostly empty, and there the
// GEMM streams weights at HBM speed whatever the tile height, so the
// smallest tile that covers the typical expert wins.  Experts with more
// rows than one 128-row tile re-read their weights once per tile, so they
// take the tallest tile that fits the register file (256 rows): measured
// with 32 experts of 136-320 rows on average (K = 7168, N = 2048), the two
// GEMMs took 0-17 % less time with 256-row tiles than with 128-row ones,
// for the block and the MX schemes alike; at 128 rows per expert (8
// experts, N = 14336) the 128-row tiles stay ahead.
int choose_tile_m(const moe_problem_t* p) {
  const char* env = getenv("MOE_TILE_M");
  if (env != nullptr) {
    const int v = atoi(env);
    if (valid_block_size(p, v)) return v;
  }
  const double rows = (double)p->num_tokens * p->top_k / p->num_experts;
  // bf16 activation tiles take twice the LDS: at most 128 rows
  if (p->act_quant == MOE_Q_BF16 && rows > 48.0) return 128;
  // A split w2 wants few, whole-expert items: around 128 rows per expert a
  // 128-row tile leaves about half the experts a nearly empty second tile
  // (an 8-expert batch: 192 items, 384 when split = 1.5 waves of blocks for
  // 256 CUs), a 192-row tile one tile each (256 split items).  Measured on
  // the 8-expert N = 14336 batch: layer 0.453 ms (128 rows, unsplit) ->
  // 0.423 ms (192 rows, split in two).  A 192-row tile fits only a two-slot
  // ring in LDS (one k-step of weights in flight per CU); a 160-row tile,
  // where the experts' rows fit it, keeps three slots.
  if (w2_ksplit(p) > 1 && rows > 96.0 && rows <= 192.0)
    return rows <= 144.0 && tile160_fits(p) ? 160 : 192;
  if (rows <= 12.0) return 16;
  if (rows <= 24.0) return 32;
  if (rows <= 48.0) return 64;
  if (rows <= 128.0) return 128;
  return 256;
}

// Heavy experts in a second tile list.  At 128-row tiles (experts of up to
// about 128 rows on average) the experts above 128 rows re-read their
// weights once per 128-row tile; in tiles of 256 rows, launched alongside
// the 128-row tiles of the other experts on a second stream, DSv3-shaped
// prefill measured w13 1.89 -> 1.76 ms (also with MXFP4 weights: 1.52 ->
// 1.42 ms) and w2 0.99 -> 0.96 ms; the same two launches one after the
// other gained only 3 % on w13 and lost 3 % on w2 (each launch's last wave
// of blocks runs half empty).  Not for bf16 activations (128-row tiles at
// most) or a split w2 (its tickets are indexed by tile).  In the indexed
// layout a tall tile covers 256 positions of its expert's segment of the
// block map (block size 128).  A forced tile height (MOE_TILE_M) keeps one
// list; MOE_TALL = 0 | 1 turns the second list off / on where it can run.
bool use_tall(const moe_problem_t* p, int tile_m, int w2_split) {
  const bool can = tile_m == 128 && p->act_quant != MOE_Q_BF16 && w2_split == 1;
  const char* env = getenv("MOE_TALL");
  if (env != nullptr && (env[0] == '0' || env[0] == '1')) return can && env[0] == '1';
  return can && getenv("MOE_TILE_M") == nullptr;
}

moe_status_t validate_problem(const moe_problem_t* p) {
  if (p == nullptr) return fail(MOE_ERR_INVALID_ARG, "problem is NULL");
  if (p->num_tokens < 0) return fail(MOE_ERR_INVALID_ARG, "num_tokens < 0 (%d)", p->num_tokens);
  if (p->hidden <= 0 || p->hidden % 128 != 0)
    return fail(MOE_ERR_INVALID_ARG, "hidden size must be a positive multiple of 128, got %d",
                p->hidden);
  if (p->intermediate <= 0 || p->intermediate % 128 != 0)
    return fail(MOE_ERR_INVALID_ARG,
                "intermediate size must be a positive multiple of 128, got %d", p->intermediate);
  if (p->num_experts < 1 || p->num_experts > 1024)
    return fail(MOE_ERR_UNSUPPORTED, "num_experts must be in [1, 1024], got %d", p->num_experts);
  if (p->top_k < 1) return fail(MOE_ERR_INVALID_ARG, "top_k must be >= 1, got %d", p->top_k);
  if ((int64_t)p->num_tokens * p->top_k >= (int64_t)1 << 31)
    return fail(MOE_ERR_UNSUPPORTED, "num_tokens * top_k must be < 2^31");
  if (p->layout != MOE_LAYOUT_CONTIGUOUS && p->layout != MOE_LAYOUT_BATCHED_MASKED &&
      p->layout != MOE_LAYOUT_INDEXED)
    return fail(MOE_ERR_INVALID_ARG, "unknown layout %d", p->layout);
  if (batched(p) && p->max_tokens_per_expert < 1)
    return fail(MOE_ERR_INVALID_ARG, "batched layout needs max_tokens_per_expert >= 1");
  if (batched(p) && (int64_t)p->num_experts * p->max_tokens_per_expert >= (int64_t)1 << 31)
    return fail(MOE_ERR_UNSUPPORTED, "num_experts * max_tokens_per_expert must be < 2^31");
  if (p->hidden > 32768 || p->intermediate > 32768)
    return fail(MOE_ERR_UNSUPPORTED, "hidden and intermediate sizes are limited to 32768");
  {
    // activation buffers are addressed with 32-bit buffer offsets
    const int64_t rows = batched(p) ? (int64_t)p->num_experts * p->max_tokens_per_expert
                                    : (int64_t)p->num_tokens * p->top_k;
    const int64_t in_rows = batched(p) ? rows : p->num_tokens;
    const int64_t elem = p->act_quant == MOE_Q_BF16 ? 2 : 1;
    // (this also bounds T * hidden, so the reduce's one-dimensional grid of
    // T * ceil(hidden / 1024) blocks stays far below 2^31)
    if (in_rows * p->hidden * elem >= ((int64_t)7 << 29) ||
        rows * p->intermediate * elem >= ((int64_t)7 << 29))
      return fail(MOE_ERR_UNSUPPORTED, "activation buffers are limited to 3.5 GiB");
  }
  if (p->act_quant < MOE_Q_FP8_UE8M0 || p->act_quant > MOE_Q_MXFP8)
    return fail(MOE_ERR_INVALID_ARG, "unknown activation quantization %d", p->act_quant);
  if (p->weight_quant < MOE_W_FP8_BLOCK128 || p->weight_quant > MOE_W_MXFP4)
    return fail(MOE_ERR_INVALID_ARG, "unknown weight quantization %d", p->weight_quant);
  if (p->activation < MOE_ACT_SILU || p->activation > MOE_ACT_SWIGLUSTEP)
    return fail(MOE_ERR_INVALID_ARG, "unknown activation %d", p->activation);
  if (!(p->act_limit >= 0.0f) || p->act_limit > 3.0e38f)
    return fail(MOE_ERR_INVALID_ARG, "act_limit must be finite and >= 0, got %g",
                (double)p->act_limit);
  if (p->act_limit > 0.0f && p->activation != MOE_ACT_SILU &&
      p->activation != MOE_ACT_SWIGLUOAI && p->activation != MOE_ACT_SWIGLUSTEP)
    return fail(MOE_ERR_UNSUPPORTED, "activation %d takes no clamp limit", p->activation);
  // (weight, activation) pairs: block fp8 weights with per-128 or bf16
  // activations, MXFP8 or MXFP4 weights with MXFP8 activations
  const bool mx_w = p->weight_quant != MOE_W_FP8_BLOCK128;
  const bool mx_a = p->act_quant == MOE_Q_MXFP8;
  if (mx_w != mx_a || (mx_w && p->act_quant == MOE_Q_BF16))
    return fail(MOE_ERR_UNSUPPORTED,
                "weight quantization %d cannot pair with activation quantization %d",
                p->weight_quant, p->act_quant);
  return MOE_OK;
}

struct Plan {
  moe_sizes_t s;
  int64_t route_blocks;
  int64_t max_tiles;
  bool tall;                                // heavy experts in the second tile list
  size_t x_q_bytes, x_sf_bytes, a2_q_bytes, a2_sf_bytes, down_bytes;
  size_t gate_up_bytes;   // forward workspace: only for _no_mul activations
  size_t stage_ws_bytes;
  size_t hist_base_off;                     // int32 offset of the per-block bases (0: in place)
  int w2_split;                             // w2 split-K factor
  size_t w2_part_bytes, w2_counters;        // its fp32 partials, its tickets
  int64_t w2_part_rows;                     // rows of one split's partials
  size_t w2_ws_bytes;                       // both, 256-byte aligned (0: no split)
};

Plan make_plan(const moe_problem_t* p) {
  Plan pl;
  const int64_t T = p->num_tokens, k = p->top_k, E = p->num_experts;
  const int64_t K = p->hidden, N = p->intermediate;
  const int64_t GK = K / 128, GN = N / 128;
  const bool ue = p->act_quant == MOE_Q_FP8_UE8M0;
  pl.s.slots = T * k;
  pl.s.tile_m = choose_tile_m(p);
  const int64_t bm = pl.s.tile_m;
  if (batched(p)) {
    pl.s.stage_rows = E * p->max_tokens_per_expert;
    pl.s.expert_rows = pl.s.stage_rows;
    pl.max_tiles = E * ((p->max_tokens_per_expert + bm - 1) / bm);
  } else {
    pl.s.stage_rows = T;
    pl.s.expert_rows = T * k;
    pl.max_tiles = (T * k + bm - 1) / bm + E;
  }
  pl.s.padded_rows = indexed(p) ? padded_capacity(p, bm) : pl.s.expert_rows;
  pl.s.blocks = indexed(p) ? pl.s.padded_rows / bm : 0;
  // count, group count, 8 ints of per-tile information, group offsets (at
  // most one group per expert plus one per 8 tiles, so E + max_tiles + 1 is
  // a safe bound)
  pl.s.tile_list = 4 + 8 * pl.max_tiles + (E + pl.max_tiles + 1);
  pl.s.max_tiles = pl.max_tiles;
  pl.s.tall_tile_m = 0;
  pl.s.tall_list_offset = 0;
  pl.s.max_tiles_tall = 0;
  const bool mx = p->act_quant == MOE_Q_MXFP8;
  const bool bf = p->act_quant == MOE_Q_BF16;
  pl.s.x_sf_row = bf ? 0 : mx ? K / 32 : ue ? 4 * ((GK + 3) / 4) : GK;
  pl.s.a2_sf_row = bf ? 0 : mx ? N / 32 : ue ? 4 * ((GN + 3) / 4) : GN;
  pl.route_blocks = (T * k + moe::kRouteChunk - 1) / moe::kRouteChunk;
  pl.stage_ws_bytes = round_up((size_t)std::max<int64_t>(pl.route_blocks, 1) * E * 4);
  pl.hist_base_off = 0;
  const size_t elem = p->act_quant == MOE_Q_BF16 ? 2 : 1;
  pl.x_q_bytes = (size_t)pl.s.stage_rows * K * elem;
  const size_t sfb = p->act_quant == MOE_Q_FP8_F32 ? 4 : 1;
  pl.x_sf_bytes = p->act_quant == MOE_Q_BF16 ? 0 : (size_t)pl.s.stage_rows * pl.s.x_sf_row * sfb;
  pl.a2_q_bytes = (size_t)pl.s.expert_rows * N * elem;
  pl.a2_sf_bytes = p->act_quant == MOE_Q_BF16 ? 0 : (size_t)pl.s.expert_rows * pl.s.a2_sf_row * sfb;
  pl.down_bytes = (size_t)pl.s.expert_rows * K * 2;
  pl.gate_up_bytes = gated(p) ? 0 : (size_t)pl.s.expert_rows * N * 2;
  // w2 split-K: S partial rows per output row (the indexed layout writes
  // T*k rows, the others expert_rows), one ticket per (tile, n-tile) item of
  // any tile height (the most tiles: 16-row blocks)
  pl.w2_split = w2_ksplit(p);
  pl.w2_part_bytes = 0;
  pl.w2_counters = 0;
  pl.w2_part_rows = 0;
  pl.w2_ws_bytes = 0;
  if (pl.w2_split > 1) {
    const int64_t prow = std::max<int64_t>(pl.s.expert_rows, T * k);
    int64_t items = pl.max_tiles;
    if (!batched(p)) items = std::max<int64_t>(items, padded_capacity(p, 16) / 16 + E);
    pl.w2_part_rows = prow;
    pl.w2_part_bytes = (size_t)pl.w2_split * prow * K * 4;
    pl.w2_counters = (size_t)items * (K / 128);
    pl.w2_ws_bytes = round_up(pl.w2_part_bytes) + round_up(pl.w2_counters * 4);
  }
  pl.tall = use_tall(p, pl.s.tile_m, pl.w2_split);
  if (pl.tall) {
    // the per-block bases go beside the histograms, which the second scan
    // block (the tall list's) reads meanwhile
    pl.hist_base_off = pl.stage_ws_bytes / 4;
    pl.stage_ws_bytes *= 2;
    // the tall list after the main one, 16-byte aligned: tiles of twice the
    // height for experts above tile_m rows (at most one partial tile each)
    const int64_t th = 2 * bm;
    pl.s.tall_tile_m = (int32_t)th;
    pl.s.max_tiles_tall = batched(p) ? E * ((p->max_tokens_per_expert + th - 1) / th)
                                     : (T * k + th - 1) / th + E;
    pl.s.tall_list_offset = (pl.s.tile_list + 3) / 4 * 4;
    pl.s.tile_list = pl.s.tall_list_offset + 4 + 8 * pl.s.max_tiles_tall +
                     (E + pl.s.max_tiles_tall + 1);
  }
  return pl;
}

// Device addresses of the forward workspace.
struct Workspace {
  uint8_t* x_q; uint8_t* x_sf; uint8_t* a2_q; uint8_t* a2_sf; uint8_t* down; uint8_t* gate_up;
  uint8_t* w2_split;
  int64_t* idx; float* w; moe_routing_t routing; int32_t* stage_ws;
  int32_t* sorted_ids; int32_t* expert_ids; int32_t* num_padded;   // indexed layout
  size_t total;
};

// The forward pass runs w13 with the fused activation, which reads x_q while
// it writes a2: the staged activations, a2 and the bf16 down projection each
// get their own region (no gate_up buffer).
Workspace carve(const Plan& pl, const moe_problem_t* p, uint8_t* base) {
  Workspace w;
  size_t off = 0;
  auto take = [&](size_t bytes) { uint8_t* r = base + off; off += round_up(bytes); return r; };
  w.x_q = take(pl.x_q_bytes);
  w.x_sf = take(pl.x_sf_bytes);
  w.a2_q = take(pl.a2_q_bytes);
  w.a2_sf = take(pl.a2_sf_bytes);
  w.down = take(pl.down_bytes);
  w.gate_up = take(pl.gate_up_bytes);
  w.w2_split = take(pl.w2_ws_bytes);
  const size_t slots = (size_t)pl.s.slots;
  w.idx = (int64_t*)take(slots * 8);
  w.w = (float*)take(slots * 4);
  w.routing.expert_num_tokens = (int32_t*)take((size_t)p->num_experts * 4);
  w.routing.expert_offsets = (int32_t*)take((size_t)(p->num_experts + 1) * 4);
  w.routing.row_src = (int32_t*)take(std::max<size_t>(slots, 1) * 4);
  w.routing.slot_row = (int32_t*)take(std::max<size_t>(slots, 1) * 4);
  w.routing.tile_list = (int32_t*)take((size_t)pl.s.tile_list * 4);
  w.stage_ws = (int32_t*)take(pl.stage_ws_bytes);
  w.sorted_ids = (int32_t*)take((size_t)pl.s.padded_rows * 4);
  w.expert_ids = (int32_t*)take((size_t)pl.s.blocks * 4);
  w.num_padded = (int32_t*)take(indexed(p) ? 4 : 0);
  w.total = off;
  return w;
}

moe_status_t check_ptr(const void* ptr, const char* name, size_t align) {
  if (ptr == nullptr) return fail(MOE_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned(ptr, align))
    return fail(MOE_ERR_INVALID_ARG, "%s must be %zu-byte aligned", name, align);
  return MOE_OK;
}

#define CHECK(expr)                         \
  do {                                      \
    const moe_status_t _s = (expr);         \
    if (_s != MOE_OK) return _s;            \
  } while (0)

// Activation-scale pointer: required for quantized activations, NULL for bf16.
moe_status_t check_sf(const moe_problem_t* p, const void* sf, const char* name) {
  if (p->act_quant == MOE_Q_BF16) {
    if (sf != nullptr)
      return fail(MOE_ERR_INVALID_ARG, "%s must be NULL for bf16 activations", name);
    return MOE_OK;
  }
  return check_ptr(sf, name, 4);
}

moe_status_t check_routing(const moe_routing_t* r) {
  if (r == nullptr) return fail(MOE_ERR_INVALID_ARG, "routing is NULL");
  CHECK(check_ptr(r->expert_num_tokens, "routing.expert_num_tokens", 4));
  CHECK(check_ptr(r->expert_offsets, "routing.expert_offsets", 4));
  CHECK(check_ptr(r->row_src, "routing.row_src", 4));
  CHECK(check_ptr(r->slot_row, "routing.slot_row", 4));
  CHECK(check_ptr(r->tile_list, "routing.tile_list", 16));
  return MOE_OK;
}

moe_status_t check_eplb(const moe_problem_t* p, const moe_eplb_t* eplb) {
  if (eplb == nullptr) return MOE_OK;
  CHECK(check_ptr(eplb->logical_to_physical, "eplb.logical_to_physical", 4));
  CHECK(check_ptr(eplb->replica_count, "eplb.replica_count", 4));
  if (eplb->map_stride < 1) return fail(MOE_ERR_INVALID_ARG, "eplb.map_stride must be >= 1");
  if (eplb->num_logical < 1 || eplb->num_logical > p->num_experts)
    return fail(MOE_ERR_INVALID_ARG, "eplb.num_logical must be in [1, num_experts]");
  if (eplb->record_flag != nullptr && eplb->expert_load == nullptr)
    return fail(MOE_ERR_INVALID_ARG, "eplb.record_flag given without eplb.expert_load");
  return MOE_OK;
}

moe::EplbArgs eplb_args(const moe_eplb_t* eplb) {
  moe::EplbArgs a{};
  if (eplb != nullptr) {
    a.l2p = eplb->logical_to_physical;
    a.map_stride = eplb->map_stride;
    a.replica_count = eplb->replica_count;
    a.num_logical = eplb->num_logical;
    a.expert_load = eplb->expert_load;
    a.record_flag = eplb->record_flag;
    a.num_unpadded = eplb->num_unpadded_tokens;
  }
  return a;
}

moe_status_t check_stage_args(const moe_problem_t* p, const void* hidden,
                              const int32_t* counts_in, const int32_t* topk_ids,
                              const float* topk_weights, const moe_eplb_t* eplb) {
  CHECK(check_ptr(hidden, "hidden", 16));
  CHECK(check_ptr(topk_ids, "topk_ids", 4));
  CHECK(check_ptr(topk_weights, "topk_weights", 4));
  if (batched(p)) CHECK(check_ptr(counts_in, "expert_num_tokens (batched layout)", 4));
  // the replica remap is part of staging token-ordered input; batched slabs
  // come from a dispatch that already chose physical experts
  if (batched(p) && eplb != nullptr)
    return fail(MOE_ERR_UNSUPPORTED,
                "EPLB remapping needs the contiguous routing (batched slabs are per physical "
                "expert: pass physical ids and no eplb)");
  CHECK(check_eplb(p, eplb));
  return MOE_OK;
}

moe_status_t run_stage(const moe_problem_t* p, const Plan& pl, const void* hidden,
                       const int32_t* counts_in, const int32_t* topk_ids,
                       const float* topk_weights, const uint8_t* is_padding,
                       const moe_eplb_t* eplb, void* x_q, void* x_sf, int64_t* idx_out,
                       float* w_out, const moe_routing_t* r, int32_t* hist,
                       hipStream_t stream) {
  const int32_t* cin = batched(p) ? counts_in : nullptr;
  // fp8 quantization runs inside the routing scan's launch; the bf16 copy
  // launches on its own
  const bool fused = p->act_quant != MOE_Q_BF16;
  const moe::StageQuant sq{hidden, x_q, x_sf, pl.s.stage_rows, p->hidden,
                           p->act_quant == MOE_Q_MXFP8 ? 32 : 128,
                           p->act_quant != MOE_Q_FP8_F32};
  if (!fused) {
    const hipError_t err =
        moe::launch_stage_quant(hidden, x_q, x_sf, pl.s.stage_rows, p->hidden, p->act_quant,
                                cin, p->max_tokens_per_expert, stream);
    if (err != hipSuccess) return launch_status(err, "stage_quant");
  }
  const moe::TileLists tl{pl.s.tile_m, (int)pl.max_tiles, r->tile_list,
                          (int)pl.s.max_tiles_tall,
                          pl.tall ? r->tile_list + pl.s.tall_list_offset : nullptr};
  const hipError_t err = moe::launch_route(
      topk_ids, topk_weights, is_padding, p->num_tokens, p->top_k, p->num_experts,
      eplb_args(eplb), idx_out, w_out, hist, hist + pl.hist_base_off, cin,
      p->max_tokens_per_expert, tl,
      r->expert_num_tokens, r->expert_offsets, r->row_src, r->slot_row, stream,
      fused ? &sq : nullptr);
  return launch_status(err, fused ? "route + stage_quant" : "route");
}

// The indexed layout's block map (moe_align_block_size outputs).  Both
// GEMMs write their rows in (token, slot) order, row sorted_ids[position]:
// w13 reads activation row id / top_k, w2 reads w13's row id.
struct Indexed {
  const int32_t* sorted_ids;
  const int32_t* expert_ids;
  const int32_t* num_padded;
  int block_size;
};

// w13 with act: out unused, the activation goes to act_q / act_sf.  ix: the
// indexed layout (r, if given, only orders its blocks).
moe_status_t run_gemm(const moe_problem_t* p, const Plan& pl, bool w13, const void* a_q,
                      const void* a_sf, const moe_routing_t* r, const void* w, const void* w_sf,
                      void* out, hipStream_t stream, bool act = false, void* act_q = nullptr,
                      void* act_sf = nullptr, const Indexed* ix = nullptr,
                      void* split_ws = nullptr, bool tall_list = false) {
  moe::GemmArgs g{};
  g.ksplit = 1;
  if (!w13 && pl.w2_split > 1) {
    // fp32 partials, then the tickets (zeroed here: a fill kernel, so the
    // call stays capturable)
    g.ksplit = pl.w2_split;
    g.part = (float*)split_ws;
    g.part_rows = pl.w2_part_rows;
    g.counters = (int32_t*)((uint8_t*)split_ws + round_up(pl.w2_part_bytes));
    const hipError_t zerr = moe::launch_zero_i32(g.counters, (int64_t)pl.w2_counters, stream);
    if (zerr != hipSuccess) return launch_status(zerr, "grouped_gemm_w2 (split tickets)");
  }
  const size_t sfb = p->act_quant == MOE_Q_FP8_F32 ? 4 : 1;
  const size_t elem = p->act_quant == MOE_Q_BF16 ? 2 : 1;
  const int64_t cap = ix != nullptr ? padded_capacity(p, ix->block_size) : 0;
  (void)elem;
  g.a = (const uint8_t*)a_q;
  g.a_bytes = (uint32_t)(w13 ? pl.x_q_bytes : pl.a2_q_bytes);
  g.a_sf = a_sf;
  g.a_sf_stride = (int)(w13 ? pl.s.x_sf_row : pl.s.a2_sf_row);
  g.a_sf_bytes = (uint32_t)((w13 ? pl.s.stage_rows : pl.s.expert_rows) * g.a_sf_stride * sfb);
  g.w = (const uint8_t*)w;
  g.w_sf = w_sf;
  g.out = (uint16_t*)out;
  g.act_q = (uint8_t*)act_q;
  g.act_sf = (uint8_t*)act_sf;
  g.act_sf_row = (int)pl.s.a2_sf_row;
  g.num_experts = p->num_experts;
  g.wide = pl.tall ? 1 : 0;
  int tile_m = pl.s.tile_m, max_tiles = (int)pl.max_tiles;
  if (ix != nullptr) {
    g.sorted_ids = ix->sorted_ids;
    g.expert_ids = ix->expert_ids;
    g.num_padded = ix->num_padded;
    g.max_blocks = (int)(cap / ix->block_size);
    g.top_k = w13 ? p->top_k : 1;
    g.numel = p->num_tokens * p->top_k;
    g.gather_sorted = 1;
    g.scatter_sorted = 1;
    g.block_size = ix->block_size;
    tile_m = ix->block_size;
    max_tiles = g.max_blocks;
    // moe_forward hands in its routing: with blocks of the tile height the
    // GEMM takes them in the routing's XCD-balanced order (the tall list's
    // tiles cover two blocks of one expert)
    if (r != nullptr && ix->block_size == pl.s.tile_m) {
      g.tile_list = r->tile_list;
      if (tall_list) {
        g.tile_list = r->tile_list + pl.s.tall_list_offset;
        tile_m = pl.s.tall_tile_m;
        max_tiles = (int)pl.s.max_tiles_tall;
      }
    }
  } else {
    g.tile_list = r->tile_list;
    g.row_src = (w13 && !batched(p)) ? r->row_src : nullptr;
    if (tall_list) {
      g.tile_list = r->tile_list + pl.s.tall_list_offset;
      tile_m = pl.s.tall_tile_m;
      max_tiles = (int)pl.s.max_tiles_tall;
    }
  }
  // the zipper mixes heavy and light experts: not for a lone list of
  // 256-row tiles, whose experts are all heavy
  g.zip = (tile_m == 256 && !tall_list) ? 0 : 1;
  // w2 at 128-row tiles: two neighbouring n-tiles per block.  Its k-loop is
  // short where N is (16 k-steps at N = 2048), and a block's prologue and
  // epilogue, which nothing overlaps at one block per CU, are then about a
  // fifth of its time; the pair overlaps the second tile's first copies
  // with the first tile's last steps and stores (DSv3-shaped prefill
  // layer 2.796 -> 2.768 ms).  Pairs of 256-row tiles measured no better
  // (DSv3-shaped prefill +0.7 %, Qwen3-shaped within noise), so the kernel
  // takes them at 128 rows only.  MOE_PAIR = 0 | 1 overrides.
  {
    const char* env = getenv("MOE_PAIR");
    g.pair = !w13 && (env != nullptr ? env[0] == '1' : true) ? 1 : 0;
  }
  g.Kd = w13 ? p->hidden : p->intermediate;
  g.Nout = w13 ? (int)w13_rows(p) : p->hidden;
  // a gated w13's gate and up halves are keyed alike (their 256-column pairs
  // align only when N is a multiple of 256)
  g.rot_period = !(w13 && gated(p)) ? g.Nout : p->intermediate % 256 == 0 ? p->intermediate : 0;
  g.activation = p->activation;
  g.act_limit = effective_limit(p);
  const int scheme =
      p->weight_quant == MOE_W_MXFP4 ? moe::kSchemeMxfp8W4 : p->act_quant;
  const hipError_t err = moe::launch_grouped_gemm(g, tile_m, max_tiles, scheme, act, stream);
  return launch_status(err, act ? "grouped_gemm_w13_act" : w13 ? "grouped_gemm_w13" : "grouped_gemm_w2");
}

// num_rows: device row count for the contiguous / indexed layouts (nullptr:
// the expert offsets' total); the batched layout uses the slab counts.
// slot_order: the indexed layout's (token, slot)-ordered rows, all T*k of
// them (rows of unrouted slots hold whatever was there and are never read)
moe_status_t run_act(const moe_problem_t* p, const Plan& pl, const void* gate_up,
                     const moe_routing_t* r, void* a2_q, void* a2_sf, hipStream_t stream,
                     bool slot_order = false) {
  const bool b = batched(p);
  const int32_t* num_rows = b || slot_order ? nullptr : r->expert_offsets + p->num_experts;
  const hipError_t err = moe::launch_act_requant(
      gate_up, a2_q, a2_sf, pl.s.expert_rows, p->intermediate, p->act_quant, num_rows,
      b ? r->expert_num_tokens : nullptr, p->max_tokens_per_expert, p->activation,
      effective_limit(p), stream);
  return launch_status(err, "act_requant");
}

moe_status_t need_gated(const moe_problem_t* p) {
  if (gated(p)) return MOE_OK;
  return fail(MOE_ERR_UNSUPPORTED,
              "the fused w13 call pairs gate and up columns; activation %d has no up half "
              "(use the w13 GEMM and moe_act_requant)", p->activation);
}

moe_status_t run_reduce(const moe_problem_t* p, const void* down, const int32_t* slot_row,
                        const float* w, void* out, hipStream_t stream) {
  const hipError_t err = moe::launch_topk_reduce(down, slot_row, w, out, p->num_tokens, p->top_k,
                                                 p->hidden, stream);
  return launch_status(err, "topk_reduce");
}

moe_status_t run_align(const moe_problem_t* p, const int64_t* idx, const moe_routing_t* r,
                       const Indexed& ix, hipStream_t stream) {
  const hipError_t err = moe::launch_align(
      idx, r->slot_row, r->expert_num_tokens, r->expert_offsets, p->num_tokens, p->top_k,
      p->num_experts, ix.block_size, const_cast<int32_t*>(ix.sorted_ids),
      const_cast<int32_t*>(ix.expert_ids), const_cast<int32_t*>(ix.num_padded), stream);
  return launch_status(err, "align_block_size");
}

moe_status_t run_mul_sum(const moe_problem_t* p, const void* down, const int64_t* idx,
                         const float* w, void* out, hipStream_t stream) {
  const hipError_t err = moe::launch_fused_mul_sum(down, idx, w, out, p->num_tokens, p->top_k,
                                                   p->hidden, p->num_experts, stream);
  return launch_status(err, "fused_mul_sum");
}

// Device address of `scratch` on the current device, looked up on the
// first call on each device with that device current and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];

moe_status_t static_scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess)
    return fail(MOE_ERR_LAUNCH, "hipGetDevice failed: %s", hipGetErrorString(err));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MOE_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (err != hipSuccess || ptr == nullptr)
      return fail(MOE_ERR_LAUNCH, "hipGetSymbolAddress(scratch) on device %d failed: %s", dev,
                  hipGetErrorString(err));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

// The second stream of the two-list GEMM steps: one per device with two
// events, created at the first such step on that device (default priority,
// non-blocking) and kept until the process ends.  The mutex keeps one host
// thread's fork-launch-join sequence whole, since the events are shared.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  std::mutex mu;
};
std::mutex g_side_mutex;
SideStream g_side[kMaxDevices];

moe_status_t side_stream_for_current_device(SideStream** out) {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess)
    return fail(MOE_ERR_LAUNCH, "hipGetDevice failed: %s", hipGetErrorString(err));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MOE_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_side_mutex);
  SideStream& sd = g_side[dev];
  if (sd.s == nullptr) {
    hipStream_t st = nullptr;
    hipEvent_t a = nullptr, b = nullptr;
    err = hipStreamCreateWithFlags(&st, hipStreamNonBlocking);
    if (err == hipSuccess) err = hipEventCreateWithFlags(&a, hipEventDisableTiming);
    if (err == hipSuccess) err = hipEventCreateWithFlags(&b, hipEventDisableTiming);
    if (err != hipSuccess)
      return fail(MOE_ERR_LAUNCH, "second stream on device %d: %s", dev, hipGetErrorString(err));
    sd.fork = a;
    sd.join = b;
    sd.s = st;
  }
  *out = &sd;
  return MOE_OK;
}

// One GEMM step over both tile lists.  launch(tall, stream) runs one list.
// concurrent: the tall list on the second stream, forked from `stream` and
// joined back to it with events (graph capture follows the fork), the main
// list on `stream`; otherwise both on `stream`, tall list first.  With one
// list only the main launch runs.
template <class F>
moe_status_t run_lists(const Plan& pl, hipStream_t stream, bool concurrent, F&& launch) {
  if (!pl.tall) return launch(false, stream);
  if (!concurrent) {
    CHECK(launch(true, stream));
    return launch(false, stream);
  }
  SideStream* sd = nullptr;
  CHECK(side_stream_for_current_device(&sd));
  std::lock_guard<std::mutex> lock(sd->mu);
  hipError_t err = hipEventRecord(sd->fork, stream);
  if (err == hipSuccess) err = hipStreamWaitEvent(sd->s, sd->fork, 0);
  if (err != hipSuccess) return launch_status(err, "fork to the second stream");
  const moe_status_t st_tall = launch(true, sd->s);
  // join even after a failed launch, so a capturing stream is not left forked
  err = hipEventRecord(sd->join, sd->s);
  const moe_status_t st_main = launch(false, stream);
  if (err == hipSuccess) err = hipStreamWaitEvent(stream, sd->join, 0);
  if (err != hipSuccess) return launch_status(err, "join from the second stream");
  return st_tall != MOE_OK ? st_tall : st_main;
}

// Both GEMM steps over both tile lists.  A list's w2 reads only the a2 rows
// of its own experts, which its own w13 launch wrote, so each stream runs
// its list's w13 and then its w2, with one join after both: neither stream
// waits for the other between the steps.
template <class F>
moe_status_t run_lists_two_steps(const Plan& pl, hipStream_t stream, bool concurrent,
                                 F&& launch_w13, F&& launch_w2) {
  if (!pl.tall || !concurrent) {
    CHECK(run_lists(pl, stream, concurrent, launch_w13));
    return run_lists(pl, stream, concurrent, launch_w2);
  }
  SideStream* sd = nullptr;
  CHECK(side_stream_for_current_device(&sd));
  std::lock_guard<std::mutex> lock(sd->mu);
  hipError_t err = hipEventRecord(sd->fork, stream);
  if (err == hipSuccess) err = hipStreamWaitEvent(sd->s, sd->fork, 0);
  if (err != hipSuccess) return launch_status(err, "fork to the second stream");
  moe_status_t st_tall = launch_w13(true, sd->s);
  if (st_tall == MOE_OK) st_tall = launch_w2(true, sd->s);
  err = hipEventRecord(sd->join, sd->s);
  moe_status_t st_main = launch_w13(false, stream);
  if (st_main == MOE_OK) st_main = launch_w2(false, stream);
  if (err == hipSuccess) err = hipStreamWaitEvent(stream, sd->join, 0);
  if (err != hipSuccess) return launch_status(err, "join from the second stream");
  return st_tall != MOE_OK ? st_tall : st_main;
}


// The w2 call's workspace: needed (and checked) only when w2 splits.
moe_status_t check_w2_ws(const Plan& pl, const void* ws, size_t ws_bytes) {
  if (pl.w2_ws_bytes == 0) return MOE_OK;
  CHECK(check_ptr(ws, "ws (w2 split-K workspace)", 16));
  if (ws_bytes < pl.w2_ws_bytes)
    return fail(MOE_ERR_WORKSPACE, "w2 workspace too small: %zu < %zu bytes", ws_bytes,
                pl.w2_ws_bytes);
  return MOE_OK;
}

moe_status_t check_indexed(const moe_problem_t* p, const int32_t* sorted_ids,
                           const int32_t* expert_ids, const int32_t* num_padded, int bs) {
  if (batched(p))
    return fail(MOE_ERR_UNSUPPORTED, "the indexed layout needs the contiguous routing");
  if (!valid_block_size(p, bs))
    return fail(MOE_ERR_UNSUPPORTED, "block_size %d is not a GEMM tile height", bs);
  CHECK(check_ptr(sorted_ids, "sorted_ids", 4));
  CHECK(check_ptr(expert_ids, "expert_ids", 4));
  CHECK(check_ptr(num_padded, "num_tokens_padded", 4));
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_last_error(void) { return g_last_error.c_str(); }

moe_status_t moe_routing_sizes(const moe_problem_t* p, moe_sizes_t* out) {
  CHECK(validate_problem(p));
  if (out == nullptr) return fail(MOE_ERR_INVALID_ARG, "out is NULL");
  *out = make_plan(p).s;
  return ok();
}

moe_status_t moe_stage_workspace_size(const moe_problem_t* p, size_t* bytes) {
  CHECK(validate_problem(p));
  if (bytes == nullptr) return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = make_plan(p).stage_ws_bytes;
  return ok();
}

moe_status_t moe_workspace_size(const moe_problem_t* p, size_t* bytes) {
  CHECK(validate_problem(p));
  if (bytes == nullptr) return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
  const Plan pl = make_plan(p);
  *bytes = carve(pl, p, nullptr).total;
  return ok();
}

moe_status_t moe_stage(const moe_problem_t* p, const void* hidden,
                       const int32_t* expert_num_tokens_in, const int32_t* topk_ids,
                       const float* topk_weights, const uint8_t* is_padding,
                       const moe_eplb_t* eplb, void* x_q, void* x_sf, int64_t* topk_idx_out,
                       float* topk_w_out, const moe_routing_t* routing, void* ws,
                       size_t ws_bytes, void* stream) {
  CHECK(validate_problem(p));
  if (p->num_tokens == 0) return ok();
  CHECK(check_stage_args(p, hidden, expert_num_tokens_in, topk_ids, topk_weights, eplb));
  CHECK(check_ptr(x_q, "x_q", 16));
  if ((p->act_quant == MOE_Q_BF16) != (x_sf == nullptr))
    return fail(MOE_ERR_INVALID_ARG, "x_sf must be given iff the hidden states are quantized");
  if (x_sf != nullptr) CHECK(check_ptr(x_sf, "x_sf", 4));
  CHECK(check_ptr(topk_idx_out, "topk_idx_out", 8));
  CHECK(check_ptr(topk_w_out, "topk_w_out", 4));
  CHECK(check_routing(routing));
  CHECK(check_ptr(ws, "ws", 4));
  const Plan pl = make_plan(p);
  if (ws_bytes < pl.stage_ws_bytes)
    return fail(MOE_ERR_WORKSPACE, "stage workspace too small: %zu < %zu bytes", ws_bytes,
                pl.stage_ws_bytes);
  return run_stage(p, pl, hidden, expert_num_tokens_in, topk_ids, topk_weights, is_padding, eplb,
                   x_q, x_sf, topk_idx_out, topk_w_out, routing, (int32_t*)ws,
                   (hipStream_t)stream);
}

moe_status_t moe_grouped_gemm_w13(const moe_problem_t* p, const void* a_q, const void* a_sf,
                                  const moe_routing_t* routing, const void* w13,
                                  const void* w13_sf, void* gate_up, void* stream) {
  CHECK(validate_problem(p));
  if (p->num_tokens == 0) return ok();
  CHECK(check_ptr(a_q, "a_q", 16));
  CHECK(check_sf(p, a_sf, "a_sf"));
  CHECK(check_routing(routing));
  CHECK(check_ptr(w13, "w13", 16));
  CHECK(check_ptr(w13_sf, "w13_sf", 4));
  CHECK(check_ptr(gate_up, "gate_up", 16));
  const Plan pl = make_plan(p);
  return run_lists(pl, (hipStream_t)stream, true, [&](bool tall, hipStream_t st) {
    return run_gemm(p, pl, true, a_q, a_sf, routing, w13, w13_sf, gate_up, st, false, nullptr,
                    nullptr, nullptr, nullptr, tall);
  });
}

moe_status_t moe_grouped_gemm_w13_act(const moe_problem_t* p, const void* a_q, const void* a_sf,
                                      const moe_routing_t* routing, const void* w13,
                                      const void* w13_sf, void* a2_q, void* a2_sf,
                                      void* stream) {
  CHECK(validate_problem(p));
  if (p->num_tokens == 0) return ok();
  CHECK(need_gated(p));
  CHECK(check_ptr(a_q, "a_q", 16));
  CHECK(check_sf(p, a_sf, "a_sf"));
  CHECK(check_routing(routing));
  CHECK(check_ptr(w13, "w13", 16));
  CHECK(check_ptr(w13_sf, "w13_sf", 4));
  CHECK(check_ptr(a2_q, "a2_q", 16));
  CHECK(check_sf(p, a2_sf, "a2_sf"));
  const Plan pl = make_plan(p);
  return run_lists(pl, (hipStream_t)stream, true, [&](bool tall, hipStream_t st) {
    return run_gemm(p, pl, true, a_q, a_sf, routing, w13, w13_sf, nullptr, st, true, a2_q,
                    a2_sf, nullptr, nullptr, tall);
  });
}

moe_status_t moe_act_requant(const moe_problem_t* p, const void* gate_up,
                             const moe_routing_t* routing, void* a2_q, void* a2_sf,
                             void* stream) {
  CHECK(validate_problem(p));
  if (p->num_tokens == 0) return ok();
  CHECK(check_ptr(gate_up, "gate_up", 16));
  CHECK(check_routing(routing));
  CHECK(check_ptr(a2_q, "a2_q", 16));
  CHECK(check_sf(p, a2_sf, "a2_sf"));
  const Plan pl = make_plan(p);
  return run_act(p, pl, gate_up, routing, a2_q, a2_sf, (hipStream_t)stream);
}

moe_status_t moe_w2_workspace_size(const moe_problem_t* p, size_t* bytes) {
  CHECK(validate_problem(p));
  if (bytes == nullptr) return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = make_plan(p).w2_ws_bytes;
  return ok();
}

moe_status_t moe_grouped_gemm_w2(const moe_problem_t* p, const void* a2_q, const void* a2_sf,
                                 const moe_routing_t* routing, const void* w2,
                                 const void* w2_sf, void* down, void* ws, size_t ws_bytes,
                                 void* stream) {
  CHECK(validate_problem(p));
  if (p->num_tokens == 0) return ok();
  CHECK(check_ptr(a2_q, "a2_q", 16));
  CHECK(check_sf(p, a2_sf, "a2_sf"));
  CHECK(check_routing(routing));
  CHECK(check_ptr(w2, "w2", 16));
  CHECK(check_ptr(w2_sf, "w2_sf", 4));
  CHECK(check_ptr(down, "down", 16));
  const Plan pl = make_plan(p);
  CHECK(check_w2_ws(pl, ws, ws_bytes));
  return run_lists(pl, (hipStream_t)stream, true, [&](bool tall, hipStream_t st) {
    return run_gemm(p, pl, false, a2_q, a2_sf, routing, w2, w2_sf, down, st, false, nullptr,
                    nullptr, nullptr, ws, tall);
  });
}

moe_status_t moe_topk_reduce(const moe_problem_t* p, const void* down, const int32_t* slot_row,
                             const float* topk_w, void* out, void* stream) {
  CHECK(validate_problem(p));
  if (p->num_tokens == 0) return ok();
  CHECK(check_ptr(down, "down", 16));
  CHECK(check_ptr(slot_row, "slot_row", 4));
  CHECK(check_ptr(topk_w, "topk_w", 4));
  CHECK(check_ptr(out, "out", 16));
  return run_reduce(p, down, slot_row, topk_w, out, (hipStream_t)stream);
}

moe_status_t moe_align_capacity(const moe_problem_t* p, int32_t block_size,
                                int64_t* sorted_ids_len, int64_t* blocks) {
  CHECK(validate_problem(p));
  if (!valid_block_size(p, block_size))
    return fail(MOE_ERR_UNSUPPORTED, "block_size %d is not a GEMM tile height", block_size);
  if (sorted_ids_len == nullptr || blocks == nullptr)
    return fail(MOE_ERR_INVALID_ARG, "output pointer is NULL");
  *sorted_ids_len = padded_capacity(p, block_size);
  *blocks = *sorted_ids_len / block_size;
  return ok();
}

moe_status_t moe_align_block_size(const moe_problem_t* p, const int64_t* topk_idx,
                                  const moe_routing_t* routing, int32_t block_size,
                                  int32_t* sorted_ids, int32_t* expert_ids,
                                  int32_t* num_tokens_padded, void* stream) {
  CHECK(validate_problem(p));
  if (p->num_tokens == 0) return ok();
  CHECK(check_indexed(p, sorted_ids, expert_ids, num_tokens_padded, block_size));
  CHECK(check_ptr(topk_idx, "topk_idx", 8));
  CHECK(check_routing(routing));
  const Indexed ix{sorted_ids, expert_ids, num_tokens_padded, block_size};
  return run_align(p, topk_idx, routing, ix, (hipStream_t)stream);
}

moe_status_t moe_grouped_gemm_w13_act_indexed(
    const moe_problem_t* p, const void* a_q, const void* a_sf, const int32_t* sorted_ids,
    const int32_t* expert_ids, const int32_t* num_tokens_padded, int32_t block_size,
    const void* w13, const void* w13_sf, void* a2_q, void* a2_sf, void* stream) {
  CHECK(validate_problem(p));
  if (p->num_tokens == 0) return ok();
  CHECK(need_gated(p));
  CHECK(check_indexed(p, sorted_ids, expert_ids, num_tokens_padded, block_size));
  CHECK(check_ptr(a_q, "a_q", 16));
  CHECK(check_sf(p, a_sf, "a_sf"));
  CHECK(check_ptr(w13, "w13", 16));
  CHECK(check_ptr(w13_sf, "w13_sf", 4));
  CHECK(check_ptr(a2_q, "a2_q", 16));
  CHECK(check_sf(p, a2_sf, "a2_sf"));
  const Plan pl = make_plan(p);
  const Indexed ix{sorted_ids, expert_ids, num_tokens_padded, block_size};
  return run_gemm(p, pl, true, a_q, a_sf, nullptr, w13, w13_sf, nullptr, (hipStream_t)stream,
                  true, a2_q, a2_sf, &ix);
}

moe_status_t moe_grouped_gemm_w2_indexed(
    const moe_problem_t* p, const void* a2_q, const void* a2_sf, const int32_t* sorted_ids,
    const int32_t* expert_ids, const int32_t* num_tokens_padded, int32_t block_size,
    const void* w2, const void* w2_sf, void* down, void* ws, size_t ws_bytes, void* stream) {
  CHECK(validate_problem(p));
  if (p->num_tokens == 0) return ok();
  CHECK(check_indexed(p, sorted_ids, expert_ids, num_tokens_padded, block_size));
  CHECK(check_ptr(a2_q, "a2_q", 16));
  CHECK(check_sf(p, a2_sf, "a2_sf"));
  CHECK(check_ptr(w2, "w2", 16));
  CHECK(check_ptr(w2_sf, "w2_sf", 4));
  CHECK(check_ptr(down, "down", 16));
  const Plan pl = make_plan(p);
  CHECK(check_w2_ws(pl, ws, ws_bytes));
  const Indexed ix{sorted_ids, expert_ids, num_tokens_padded, block_size};
  return run_gemm(p, pl, false, a2_q, a2_sf, nullptr, w2, w2_sf, down, (hipStream_t)stream,
                  false, nullptr, nullptr, &ix, ws);
}

moe_status_t moe_fused_mul_sum(const moe_problem_t* p, const void* down, const int64_t* topk_idx,
                               const float* topk_w, void* out, void* stream) {
  CHECK(validate_problem(p));
  if (p->num_tokens == 0) return ok();
  CHECK(check_ptr(down, "down", 16));
  CHECK(check_ptr(topk_idx, "topk_idx", 8));
  CHECK(check_ptr(topk_w, "topk_w", 4));
  CHECK(check_ptr(out, "out", 16));
  return run_mul_sum(p, down, topk_idx, topk_w, out, (hipStream_t)stream);
}

}  // extern "C"

namespace {
// side: the two-list GEMM steps may use the second stream (moe_forward);
// otherwise their launches stay on the caller's stream (moe_forward_static)
moe_status_t forward_impl(const moe_problem_t* p, const void* hidden,
                          const int32_t* expert_num_tokens_in, const int32_t* topk_ids,
                          const float* topk_weights, const uint8_t* is_padding,
                          const moe_eplb_t* eplb, const void* w13, const void* w13_sf,
                          const void* w2, const void* w2_sf, void* out, void* ws,
                          size_t ws_bytes, void* stream, bool side) {
  CHECK(validate_problem(p));
  if (p->num_tokens == 0) return ok();
  CHECK(check_stage_args(p, hidden, expert_num_tokens_in, topk_ids, topk_weights, eplb));
  CHECK(check_ptr(w13, "w13", 16));
  CHECK(check_ptr(w13_sf, "w13_sf", 4));
  CHECK(check_ptr(w2, "w2", 16));
  CHECK(check_ptr(w2_sf, "w2_sf", 4));
  CHECK(check_ptr(out, "out", 16));
  CHECK(check_ptr(ws, "ws", kAlign));
  const Plan pl = make_plan(p);
  const Workspace w = carve(pl, p, (uint8_t*)ws);
  if (ws_bytes < w.total)
    return fail(MOE_ERR_WORKSPACE, "forward workspace too small: %zu < %zu bytes", ws_bytes,
                w.total);
  const hipStream_t s = (hipStream_t)stream;
  CHECK(run_stage(p, pl, hidden, expert_num_tokens_in, topk_ids, topk_weights, is_padding, eplb,
                  w.x_q, w.x_sf, w.idx, w.w, &w.routing, w.stage_ws, s));
  // gated activations: w13 with the activation fused; _no_mul ones: the w13
  // GEMM into gate_up, then the activation kernel
  if (indexed(p)) {
    const Indexed ix{w.sorted_ids, w.expert_ids, w.num_padded, pl.s.tile_m};
    CHECK(run_align(p, w.idx, &w.routing, ix, s));
    std::function<moe_status_t(bool, hipStream_t)> w2_step = [&](bool tall, hipStream_t st) {
      return run_gemm(p, pl, false, w.a2_q, w.a2_sf, &w.routing, w2, w2_sf, w.down, st, false,
                      nullptr, nullptr, &ix, w.w2_split, tall);
    };
    if (gated(p)) {
      std::function<moe_status_t(bool, hipStream_t)> w13_step = [&](bool tall, hipStream_t st) {
        return run_gemm(p, pl, true, w.x_q, w.x_sf, &w.routing, w13, w13_sf, nullptr, st, true,
                        w.a2_q, w.a2_sf, &ix, nullptr, tall);
      };
      CHECK(run_lists_two_steps(pl, s, side, w13_step, w2_step));
    } else {
      CHECK(run_lists(pl, s, side, [&](bool tall, hipStream_t st) {
        return run_gemm(p, pl, true, w.x_q, w.x_sf, &w.routing, w13, w13_sf, w.gate_up, st,
                        false, nullptr, nullptr, &ix, nullptr, tall);
      }));
      CHECK(run_act(p, pl, w.gate_up, &w.routing, w.a2_q, w.a2_sf, s, true));
      CHECK(run_lists(pl, s, side, w2_step));
    }
    CHECK(run_mul_sum(p, w.down, w.idx, w.w, out, s));
    return ok();
  }
  if (gated(p)) {
    // fused w13 + activation, then w2, per tile list
    std::function<moe_status_t(bool, hipStream_t)> w13_step = [&](bool tall, hipStream_t st) {
      return run_gemm(p, pl, true, w.x_q, w.x_sf, &w.routing, w13, w13_sf, nullptr, st, true,
                      w.a2_q, w.a2_sf, nullptr, nullptr, tall);
    };
    std::function<moe_status_t(bool, hipStream_t)> w2_step = [&](bool tall, hipStream_t st) {
      return run_gemm(p, pl, false, w.a2_q, w.a2_sf, &w.routing, w2, w2_sf, w.down, st, false,
                      nullptr, nullptr, nullptr, w.w2_split, tall);
    };
    CHECK(run_lists_two_steps(pl, s, side, w13_step, w2_step));
    CHECK(run_reduce(p, w.down, w.routing.slot_row, w.w, out, s));
    return ok();
  } else {
    CHECK(run_lists(pl, s, side, [&](bool tall, hipStream_t st) {
      return run_gemm(p, pl, true, w.x_q, w.x_sf, &w.routing, w13, w13_sf, w.gate_up, st, false,
                      nullptr, nullptr, nullptr, nullptr, tall);
    }));
    CHECK(run_act(p, pl, w.gate_up, &w.routing, w.a2_q, w.a2_sf, s));
  }
  CHECK(run_lists(pl, s, side, [&](bool tall, hipStream_t st) {
    return run_gemm(p, pl, false, w.a2_q, w.a2_sf, &w.routing, w2, w2_sf, w.down, st, false,
                    nullptr, nullptr, nullptr, w.w2_split, tall);
  }));
  CHECK(run_reduce(p, w.down, w.routing.slot_row, w.w, out, s));
  return ok();
}
}  // namespace

extern "C" {

moe_status_t moe_forward(const moe_problem_t* p, const void* hidden,
                         const int32_t* expert_num_tokens_in, const int32_t* topk_ids,
                         const float* topk_weights, const uint8_t* is_padding,
                         const moe_eplb_t* eplb, const void* w13, const void* w13_sf,
                         const void* w2, const void* w2_sf, void* out, void* ws,
                         size_t ws_bytes, void* stream) {
  return forward_impl(p, hidden, expert_num_tokens_in, topk_ids, topk_weights, is_padding, eplb,
                      w13, w13_sf, w2, w2_sf, out, ws, ws_bytes, stream, true);
}

moe_status_t moe_forward_static(const moe_problem_t* p, const void* hidden,
                                const int32_t* expert_num_tokens_in, const int32_t* topk_ids,
                                const float* topk_weights, const uint8_t* is_padding,
                                const moe_eplb_t* eplb, const void* w13, const void* w13_sf,
                                const void* w2, const void* w2_sf, void* out, void* stream) {
  CHECK(validate_problem(p));
  if (p->num_tokens == 0) return ok();
  const size_t need = carve(make_plan(p), p, nullptr).total;
  if (need > (size_t)MOE_STATIC_SCRATCH_BYTES)
    return fail(MOE_ERR_WORKSPACE,
                "moe_forward_static: this problem needs %zu workspace bytes, the static scratch "
                "holds %zu (call moe_forward with a workspace instead)",
                need, (size_t)MOE_STATIC_SCRATCH_BYTES);
  void* ws = nullptr;
  CHECK(static_scratch_for_current_device(&ws));
  return forward_impl(p, hidden, expert_num_tokens_in, topk_ids, topk_weights, is_padding, eplb,
                      w13, w13_sf, w2, w2_sf, out, ws, (size_t)MOE_STATIC_SCRATCH_BYTES, stream,
                      false);
}

}  // extern "C"
