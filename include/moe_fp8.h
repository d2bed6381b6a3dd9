/*
 * moe_fp8.h -- C ABI of the gfx950 fp8 block-quantized MoE expert layer.
 *
 * The layer, as the vLLM API documentation pages on the subject describe it:
 *   1. stage: per-128-group fp8 e4m3fn quantization of the hidden states with
 *      UE8M0 (power-of-two) or fp32 scales, and the top-k routing repack
 *      ("vllm.model_executor.layers.fused_moe.prepare_megamoe",
 *      prepare_megamoe_inputs, _quantize_fp8_groups, _store_topk);
 *   2. per-expert counts, offsets and the token -> row permutation
 *      ("vllm.model_executor.layers.fused_moe.experts.fused_humming_moe",
 *      HummingGroupedExperts.apply: moe_prepare_scatter / moe_permute;
 *      BatchedHummingGroupedExperts.apply: expert_num_tokens);
 *   3. grouped GEMM with the fused gate/up weights w13
 *      ("...experts.fused_humming_moe", HummingGroupedExperts.apply and
 *      BatchedHummingGroupedExperts.apply: the humming_forward call on the
 *      "w13" sublayer through HummingExpertsBase.process_input);
 *   4. SiLU(gate) * up re-quantized to fp8 (HummingExpertsBase.process_input
 *      with an activation);
 *   5. grouped GEMM with the down weights w2 (the same apply methods: the
 *      humming_forward call on the "w2" sublayer);
 *   6. router-weighted top-k reduce back to token order (moe_unpermute /
 *      moe_fused_mul_sum).
 *
 * Conventions for every call
 *  - Pointers named "device" are HIP device pointers; the caller allocates and
 *    owns every buffer; the library never allocates device memory, frees or
 *    synchronizes.  Work is enqueued on `stream` (a hipStream_t passed as
 *    void*, NULL = the null stream) and buffers must stay valid until it
 *    completes.  A GEMM step over two tile lists (see "Tile height") also
 *    runs one launch on a second stream the library keeps per device
 *    (created, with two events, at the first such step on the device),
 *    forked from `stream` and joined back to it by events, so work that
 *    follows on `stream` sees both launches done and a graph capture of
 *    `stream` follows the fork.
 *  - Arrays are dense row-major.  Vector-accessed buffers (hidden states, fp8
 *    codes, bf16 intermediates, weights, output) must be 16-byte aligned,
 *    scale and index arrays 4-byte aligned (int64 arrays 8-byte aligned).
 *  - Return value: MOE_OK, or a negative moe_status_t after synchronous
 *    argument validation (nothing is enqueued then); moe_last_error() gives
 *    the message.  MOE_ERR_LAUNCH reports a failed kernel launch.
 *  - num_tokens == 0 is a successful no-op (prepare_megamoe_inputs returns
 *    early for an empty batch).
 *  - Expert ids outside [0, num_experts) are treated as unrouted, never as
 *    errors.
 *
 * Formats
 *  - bf16: IEEE binary32's upper 16 bits.  fp8: OCP e4m3fn bytes.
 *  - Activation scales, MOE_Q_FP8_UE8M0: one exponent byte e per 128-group
 *    (scale 2^(e-127)), rows of 4*ceil(G/4) bytes with zero pad bytes; this is
 *    byte-identical to the pages' "four per int32" little-endian packing
 *    (_pack_bytes).  MOE_Q_FP8_F32: fp32 [rows, G].  MOE_Q_MXFP8: one
 *    exponent byte per 32-group, rows of K/32 bytes (no pad: K % 128 == 0).
 *  - Weights: w13 [E, 2N, K] fp8 codes (rows [0, N) gate, [N, 2N) up; a
 *    _NO_MUL activation: [E, N, K] and every "2N" below reads N), w2
 *    [E, K, N].  MOE_W_FP8_BLOCK128 (kFp8Static128BlockSym): fp32 block scales
 *    w13_sf [E, 2N/128, K/128], w2_sf [E, K/128, N/128], dequantized weight =
 *    code * block scale.  MOE_W_MXFP8 (kMxfp8Static): E8M0 bytes w13_sf
 *    [E, 2N, K/32], w2_sf [E, K, N/32], one per row and 32 columns,
 *    dequantized weight = code * 2^(byte-127).  MOE_W_MXFP4 (kMxfp4Static):
 *    e2m1 codes two per byte, column 2j in the low nibble: w13 [E, 2N, K/2],
 *    w2 [E, K, N/2] bytes, scales as MXFP8.
 *  - Scheme pairs (HummingExpertsBase._supports_quant_scheme): block fp8
 *    weights with UE8M0 or fp32 per-128 activations or with unquantized bf16
 *    activations (the (kFp8Static128BlockSym, None) pair: staging copies the
 *    hidden states, the w2 input is silu(gate)*up rounded to bf16, every
 *    activation-scale pointer is NULL); MXFP8 or MXFP4 weights with MXFP8
 *    activations.
 */
#ifndef MOE_FP8_H
#define MOE_FP8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1,
  MOE_ERR_UNSUPPORTED = -2,
  MOE_ERR_WORKSPACE = -3,
  MOE_ERR_LAUNCH = -4
} moe_status_t;

/* Activation quantization (w13 input and w2 input use the same scheme). */
typedef enum {
  MOE_Q_FP8_UE8M0 = 0, /* fp8 e4m3fn, per-128 power-of-two scales          */
  MOE_Q_FP8_F32 = 1,   /* fp8 e4m3fn, per-128 fp32 scales                   */
  MOE_Q_BF16 = 2,      /* bf16 activations, unquantized (no scales)          */
  MOE_Q_MXFP8 = 3      /* fp8 e4m3fn, per-32 E8M0 scales (kMxfp8Dynamic)    */
} moe_quant_t;

/* Weight quantization of w13 and w2. */
typedef enum {
  MOE_W_FP8_BLOCK128 = 0, /* e4m3fn, fp32 scale per 128x128 block           */
  MOE_W_MXFP8 = 1,        /* e4m3fn, E8M0 scale per row and 32 columns      */
  MOE_W_MXFP4 = 2         /* e2m1 (two per byte), E8M0 per row and 32 cols  */
} moe_weight_t;

/* Activation between the two GEMMs ("...experts.fused_humming_moe",
 * latest-docs page: HummingExpertsBase._supports_activation lists these and
 * apply_activation applies swiglu_limit_func for SiLU when the quant config
 * has a gemm1_clamp_limit; the pages show none of the formulas).  Standard
 * ones: SiLU g*sigmoid(g), GELU g*Phi(g) with the exact normal CDF, its tanh
 * approximation 0.5 g (1 + tanh(sqrt(2/pi) (g + 0.044715 g^3))), ReLU^2
 * max(g, 0)^2.  Gated kinds: w13 has 2N rows (gate rows first), h =
 * F(gate, up).  _NO_MUL kinds: w13 has N rows, h = f(w13 output)
 * (get_buffer_metas: the w2 input is the whole w13 output for non-gated
 * activations).  The clamped SwiGLU forms are this library's reading (their
 * bodies and constants are not on the pages), with L = act_limit:
 * SiLU with act_limit > 0: silu(min(g, L)) * clamp(up, -L, L);
 * SWIGLUSTEP: min(silu(g), L) * clamp(up, -L, L);
 * SWIGLUOAI: (clamp(up, -L, L) + 1) * g' * sigmoid(1.702 g'), g' = min(g, L);
 * for the last two act_limit 0 means L = 7. */
typedef enum {
  MOE_ACT_SILU = 0,
  MOE_ACT_GELU = 1,
  MOE_ACT_GELU_TANH = 2,
  MOE_ACT_SILU_NO_MUL = 3,
  MOE_ACT_GELU_NO_MUL = 4,
  MOE_ACT_GELU_TANH_NO_MUL = 5,
  MOE_ACT_RELU2_NO_MUL = 6,
  MOE_ACT_SWIGLUOAI = 7,
  MOE_ACT_SWIGLUSTEP = 8
} moe_act_t;

/* Expert-row layouts ("Standard" and "BatchedExperts" activation formats of
 * HummingGroupedExperts / BatchedHummingGroupedExperts, and the block map of
 * HummingIndexedExperts). */
typedef enum {
  MOE_LAYOUT_CONTIGUOUS = 0,     /* rows grouped by expert, offsets [E+1]   */
  MOE_LAYOUT_BATCHED_MASKED = 1, /* [E, max_tokens_per_expert, K] slabs     */
  MOE_LAYOUT_INDEXED = 2         /* blocks of sorted slot ids, see below    */
} moe_layout_t;

/* Problem description (host struct).  T tokens, hidden size K, intermediate
 * size N, E physical experts, top_k routed experts per token.
 * Requirements: K and N multiples of 128 (at most 32768); 1 <= E <= 1024;
 * 1 <= top_k; T * top_k < 2^31; batched layout needs
 * max_tokens_per_expert >= 1; each activation buffer (staged rows * K and
 * expert rows * N elements) under 3.5 GiB.  Every call checks these before
 * it enqueues anything (MOE_ERR_INVALID_ARG / MOE_ERR_UNSUPPORTED); no
 * launch grid then exceeds its limits (token counts ride on grid x). */
typedef struct {
  int32_t num_tokens;
  int32_t hidden;
  int32_t intermediate;
  int32_t num_experts;
  int32_t top_k;
  int32_t layout;                /* moe_layout_t */
  int32_t max_tokens_per_expert; /* batched layout only */
  int32_t act_quant;             /* moe_quant_t */
  int32_t weight_quant;          /* moe_weight_t */
  int32_t activation;            /* moe_act_t (0 = SiLU(gate) * up) */
  float act_limit;               /* clamp limit of SiLU / SWIGLUOAI /
                                    SWIGLUSTEP (>= 0; 0: none for SiLU,
                                    7 for the other two); 0 for the rest */
} moe_problem_t;

/* Expert-parallel load balancing state (optional; all device pointers).
 * A routed logical id l in [0, num_logical) becomes the physical id
 * logical_to_physical[l * map_stride + t % replica_count[l]] for token t
 * (replica_count[l] <= 0 leaves the slot unrouted); when *record_flag != 0
 * every mapped id of a token t < *num_unpadded_tokens adds one to
 * expert_load[id] (accumulated: the caller zeroes it).  From _eplb_kernel_args
 * on the prepare_megamoe page; the replica choice t % count is this
 * library's reading (the map-and-record body is not shown there). */
typedef struct {
  const int32_t* logical_to_physical; /* [num_logical, map_stride]          */
  int32_t map_stride;
  const int32_t* replica_count;       /* [num_logical]                       */
  int32_t num_logical;
  int32_t* expert_load;               /* [num_experts] or NULL               */
  const int32_t* record_flag;         /* [1] or NULL (= do not record)       */
  const int32_t* num_unpadded_tokens; /* [1] or NULL (= num_tokens)          */
} moe_eplb_t;

/* Routing layout written by moe_stage and read by the later calls (device
 * arrays, sizes from moe_routing_sizes):
 *  expert_num_tokens [E]   rows per expert (batched: the given counts)
 *  expert_offsets    [E+1] exclusive prefix of the routed counts
 *  row_src           [T*top_k] token of each contiguous row (contiguous layout)
 *  slot_row          [T*top_k] row of (token, slot), -1 when unrouted;
 *                    batched: e * max_tokens + rank (rank >= max_tokens -> -1)
 *  tile_list         [moe_sizes_t.tile_list] M-tile schedule for the GEMMs
 *                    (16-byte aligned): tile count n, group count G, two
 *                    zeros, per tile 8 ints (expert, first row within the
 *                    expert, first tile and size of its group, the expert's
 *                    rows, its first row, two zeros), then G + 1 group
 *                    offsets; a group is a run of at most 8 consecutive
 *                    m-tiles of one expert (more only for very large
 *                    batches), and the groups are ordered so that 8 equal
 *                    slices of the list hold similar work and weight bytes
 *                    (one slice per XCD).  When moe_sizes_t.tall_tile_m is
 *                    not 0, a second list of the same form starts at int32
 *                    index tall_list_offset: experts of more than tile_m
 *                    rows are scheduled there in tiles of tall_tile_m rows
 *                    (and are absent from the first list) */
typedef struct {
  int32_t* expert_num_tokens;
  int32_t* expert_offsets;
  int32_t* row_src;
  int32_t* slot_row;
  int32_t* tile_list;
} moe_routing_t;

typedef struct {
  int64_t slots;           /* T * top_k: row_src, slot_row, topk outputs     */
  int64_t tile_list;       /* int32 elements of tile_list                     */
  int64_t stage_rows;      /* rows of x_q / x_sf                              */
  int64_t expert_rows;     /* rows of gate_up / a2 / down                     */
  int64_t x_sf_row;        /* x_sf row length: bytes (UE8M0) / floats (fp32)  */
  int64_t a2_sf_row;       /* a2_sf row length, same units                    */
  int64_t padded_rows;     /* indexed: sorted_ids capacity; else expert_rows  */
  int64_t blocks;          /* indexed: expert_ids capacity; else 0            */
  int32_t tile_m;          /* activation rows per GEMM tile (indexed: the
                              block size moe_forward uses)                    */
  int32_t tall_tile_m;     /* rows per tile of the second (tall) tile list;
                              0 when there is none                            */
  int64_t max_tiles;       /* tile capacity of the first tile list            */
  int64_t tall_list_offset; /* int32 index of the tall list in tile_list      */
  int64_t max_tiles_tall;  /* its tile capacity                               */
} moe_sizes_t;

/* Tile height.  tile_m follows the expected rows per expert, T * top_k / E:
 * 16, 32 or 64 rows up to 12, 24 or 48 rows per expert, 128 up to 128, and
 * 256 above (at most 128 for bf16 activations); when w2 splits its reduction
 * (N >= 8192), 192 rows between 96 and 192 rows per expert (160 up to 144
 * rows per expert when the weights are block-scaled, the activations fp8
 * with per-128 scales and hidden and intermediate at most 24576).  At 128-row
 * tiles (fp8 or MXFP8 activations, an unsplit w2) the experts of more than
 * 128 rows go to a second tile list of 256-row tiles
 * (moe_sizes_t.tall_tile_m).  The GEMM calls that take the routing
 * (moe_grouped_gemm_w13 / _act / _w2, moe_forward, in the indexed layout's
 * moe_forward a tall tile covering two 128-blocks of one expert) then
 * launch one kernel per list: the tall list's on the library's second
 * stream beside the main list's on `stream`, or both on `stream`, tall list
 * first (moe_forward_static); the indexed entry points, which take a block
 * map, keep one launch.  The tile height never changes the results' bits.
 * MOE_KSPLIT = 1 | 2 | 4 overrides the w2 split for tuning runs (it does
 * change them: every call of one layer must see the same value).  Further
 * environment variables override the other choices for tuning runs.  MOE_TILE_M = 16 | 32 | 64 | 128 |
 * 160 | 192 | 256 (192 and 256 not for bf16, 160 only where block_size 160
 * is valid below; other values are ignored) is read by
 * every call; all calls of one layer must see the same value, since the
 * stage builds the tile schedule for the height the GEMM calls then read it
 * with; a forced height keeps one tile list.  MOE_TALL = 0 | 1 turns the
 * second list off or on (where it can run), read by every call like
 * MOE_TILE_M.  MOE_GEMM_WIDE = 0 | 1 picks 128 or 256 output columns for the
 * 128-row tiles of the unfused GEMMs (default 256; 128 for the MX schemes
 * when there is one tile list); it is read once per scale scheme, at its
 * first GEMM call, and does not change the schedule.  MOE_SN = n sets how
 * many n-tiles the GEMMs walk together inside an expert's m-tiles (default 1
 * for tiles up to 128 rows, 2 above; read once per tile shape); it changes
 * only the order of the blocks, never a result's bits.  MOE_KROT = 0 | 1
 * turns the GEMMs' k-step rotation off or on (read at every launch;
 * default on where the weight rows are a multiple of 4096 bytes long, never
 * for the MX schemes): each block starts its reduction at a k-step set by
 * its expert and its output columns, so that blocks streaming at once read
 * different offsets of their weight rows.  The start depends on neither the
 * batch nor the tile shape, but it does set the order of the fp32 additions:
 * every call of one layer must see the same value.  MOE_PAIR = 0 | 1 turns
 * off or on the w2 GEMM's two 256-column n-tiles per block at 128-row tiles
 * (default on; per-128 fp8 activations, hidden a multiple of 512, no split;
 * read at every call): the second tile's
 * first copies overlap the first tile's last k-steps and stores.  It
 * changes neither the schedule nor a result's bits. */

/* Sizes of every buffer of `p` (host only). */
moe_status_t moe_routing_sizes(const moe_problem_t* p, moe_sizes_t* out);

/* Device scratch bytes moe_stage needs (host only). */
moe_status_t moe_stage_workspace_size(const moe_problem_t* p, size_t* bytes);

/* Device workspace bytes moe_forward needs (host only).  It holds the staged
 * fp8 activations, the fp8 w2 input, the bf16 down projection, the routing
 * layout and, when w2 splits its reduction, the w2 workspace (the workspace
 * of HummingExpertsBase.prepare_buffers minus the gate_up buffer, which the
 * fused w13 call never materializes). */
moe_status_t moe_workspace_size(const moe_problem_t* p, size_t* bytes);

/* Steps 1-2.  hidden: bf16 [T, K] (contiguous) or [E, max_tokens, K]
 * (batched; only rows below expert_num_tokens_in[e] are read).
 * topk_ids int32 [T, top_k], topk_weights fp32 [T, top_k], is_padding uint8
 * [T] or NULL (padding tokens: ids -1, weights 0, never routed; their hidden
 * rows are still quantized).  expert_num_tokens_in: batched layout only,
 * int32 [E], must equal the per-expert count of topk_ids.  eplb may be NULL;
 * it needs the contiguous or indexed layout (batched slabs are per physical
 * expert, from a dispatch that already chose the replicas: pass physical
 * ids; eplb with BATCHED_MASKED -> MOE_ERR_UNSUPPORTED before any launch).
 * Outputs: x_q fp8 [rows, K] (MOE_Q_BF16: bf16 copy), x_sf (NULL for bf16),
 * topk_idx_out int64 [T, top_k], topk_w_out fp32 [T, top_k], routing.
 * ws: device scratch of moe_stage_workspace_size bytes. */
moe_status_t moe_stage(const moe_problem_t* p, const void* hidden,
                       const int32_t* expert_num_tokens_in, const int32_t* topk_ids,
                       const float* topk_weights, const uint8_t* is_padding,
                       const moe_eplb_t* eplb, void* x_q, void* x_sf, int64_t* topk_idx_out,
                       float* topk_w_out, const moe_routing_t* routing, void* ws,
                       size_t ws_bytes, void* stream);

/* Step 3 ("...experts.fused_humming_moe", HummingGroupedExperts.apply and
 * BatchedHummingGroupedExperts.apply: humming_forward on the "w13" sublayer,
 * with the weight / activation pair of HummingExpertsBase.
 * _supports_quant_scheme).
 * gate_up[r, :] = block-scaled fp8 GEMM of activation row r with
 * w13[e] for every routed row r of expert e (rows from `routing`; the
 * contiguous layout gathers x_q rows through row_src).  gate_up: bf16
 * [expert_rows, 2N]; rows past an expert's count are not written. */
moe_status_t moe_grouped_gemm_w13(const moe_problem_t* p, const void* a_q, const void* a_sf,
                                  const moe_routing_t* routing, const void* w13,
                                  const void* w13_sf, void* gate_up, void* stream);

/* Steps 3 + 4 in one pass: the w13 GEMM of moe_grouped_gemm_w13 whose result
 * never leaves the chip; each output row's gate and up halves are rounded to
 * bf16 (the gate_up buffer's precision) and turned into a2 exactly as
 * moe_act_requant would, so a2_q / a2_sf are bit-identical to that chain.
 * The pages fuse the activation into the w2-input quantization
 * (HummingExpertsBase.process_input with an activation); here it moves one
 * step earlier, into the producing GEMM.  a2_q fp8 [expert_rows, N], a2_sf per
 * the activation scheme (bf16 activations: a2_q bf16 [expert_rows, N], a2_sf
 * NULL); rows past an expert's count are not written.
 * a2_q / a2_sf must not overlap a_q / a_sf.  Gated activations only (a
 * _NO_MUL activation has no up half to pair: MOE_ERR_UNSUPPORTED; use
 * moe_grouped_gemm_w13 + moe_act_requant, as moe_forward does). */
moe_status_t moe_grouped_gemm_w13_act(const moe_problem_t* p, const void* a_q,
                                      const void* a_sf, const moe_routing_t* routing,
                                      const void* w13, const void* w13_sf, void* a2_q,
                                      void* a2_sf, void* stream);

/* Step 4: a2 = quant(h) per group (128 columns, 32 for MXFP8) with h =
 * f(gate_up[:, :N]) * gate_up[:, N:] (gated activations, SiLU by default) or
 * f(gate_up) (_NO_MUL, gate_up [expert_rows, N]), computed in fp32 and
 * quantized without an intermediate rounding.  a2_q fp8 [expert_rows, N],
 * a2_sf per the activation scheme; bf16 activations: a2_q = bf16(h)
 * [expert_rows, N], a2_sf NULL. */
moe_status_t moe_act_requant(const moe_problem_t* p, const void* gate_up,
                             const moe_routing_t* routing, void* a2_q, void* a2_sf,
                             void* stream);

/* Step 5 ("...experts.fused_humming_moe", HummingGroupedExperts.apply and
 * BatchedHummingGroupedExperts.apply: humming_forward on the "w2" sublayer,
 * fed by the activation buffer).
 * down[r, :] = block-scaled GEMM of a2 row r with w2[e] (fp8 or bf16 a2 per
 * the activation scheme); down: bf16 [expert_rows, K]; rows past an expert's
 * count are not written.
 * Split-K: when the reduction is long (N >= 8192) the k-steps are cut into
 * ranges whose fp32 partials are added in a fixed order before the one bf16
 * rounding (the experts pass a `locks` buffer to every Humming GEMM for the
 * same purpose, HummingExpertsBase).  The split depends on N alone, so a
 * token's bits do not depend on its batch.  ws: device workspace of
 * moe_w2_workspace_size bytes (fp32 partials and per-tile tickets; may be
 * NULL when that size is 0); calls sharing one ws must not overlap. */
moe_status_t moe_w2_workspace_size(const moe_problem_t* p, size_t* bytes);
moe_status_t moe_grouped_gemm_w2(const moe_problem_t* p, const void* a2_q, const void* a2_sf,
                                 const moe_routing_t* routing, const void* w2,
                                 const void* w2_sf, void* down, void* ws, size_t ws_bytes,
                                 void* stream);

/* Step 6: out[t] = bf16(sum over j ascending with slot_row[t, j] >= 0 of
 * topk_w[t, j] * down[slot_row[t, j]]); tokens with no routed slot get 0.
 * out: bf16 [T, K]. */
moe_status_t moe_topk_reduce(const moe_problem_t* p, const void* down, const int32_t* slot_row,
                             const float* topk_w, void* out, void* stream);

/* ---- Indexed layout ("...experts.fused_humming_moe",
 * HummingIndexedExperts.apply / prepare_humming_moe_kwargs).  The routed
 * (token, slot) pairs are addressed by their flat slot id t * top_k + j.
 * sorted_ids holds, expert by expert in id order, the slot ids routed to
 * that expert in ascending order, each expert's segment padded with the
 * sentinel T * top_k to a multiple of block_size (experts with no slot have
 * no segment); expert_ids[b] is the expert of block b (entries
 * [b*block_size, (b+1)*block_size)); *num_tokens_padded is the padded total.
 * The pages call moe_align_block_size without showing its body; this is the
 * plain reading (the order inside a segment is the contiguous layout's row
 * order).  block_size is a GEMM tile height: 16, 32, 64, 128, for
 * quantized activations 192 or 256, and 160 for block-scaled weights with
 * per-128 fp8 activations when hidden and intermediate are at most 24576
 * (the 160-row tiles' weight-scale panel).  These calls need the contiguous routing
 * (layout CONTIGUOUS or INDEXED; BATCHED_MASKED -> MOE_ERR_UNSUPPORTED). */

/* Capacity of sorted_ids (T*k + min(E, T*k) * (block_size - 1), rounded down
 * to whole blocks) and of expert_ids (that / block_size) (host only). */
moe_status_t moe_align_capacity(const moe_problem_t* p, int32_t block_size,
                                int64_t* sorted_ids_len, int64_t* blocks);

/* Builds the block map from moe_stage's outputs: topk_idx int64 [T, top_k]
 * and its routing (expert_num_tokens, expert_offsets and slot_row are read).
 * Outputs (device int32): sorted_ids [capacity], expert_ids [blocks],
 * num_tokens_padded [1]; entries past the padded total are not written. */
moe_status_t moe_align_block_size(const moe_problem_t* p, const int64_t* topk_idx,
                                  const moe_routing_t* routing, int32_t block_size,
                                  int32_t* sorted_ids, int32_t* expert_ids,
                                  int32_t* num_tokens_padded, void* stream);

/* Steps 3 + 4 on the block map: for every routed position q (sorted_ids[q]
 * = s < T*k), a2 row s = the fused w13 + activation of moe_grouped_gemm_w13_act
 * applied to activation row s / top_k with the weights of expert
 * expert_ids[q / block_size].  a2 is in (token, slot) order: a2_q [T*top_k,
 * N] (fp8, or bf16 for bf16 activations), a2_sf per the activation scheme
 * with T*top_k rows; rows of unrouted slots are not written.  The routed
 * entries of every block must precede its padding (as moe_align_block_size
 * writes them); *num_tokens_padded is clamped to the capacity. */
moe_status_t moe_grouped_gemm_w13_act_indexed(
    const moe_problem_t* p, const void* a_q, const void* a_sf, const int32_t* sorted_ids,
    const int32_t* expert_ids, const int32_t* num_tokens_padded, int32_t block_size,
    const void* w13, const void* w13_sf, void* a2_q, void* a2_sf, void* stream);

/* Step 5 on the block map (ws as for moe_grouped_gemm_w2): down[s] = the w2
 * GEMM of a2 row s for every routed
 * position q with s = sorted_ids[q] (the experts run w2 with top_k 1 on the
 * (token, slot)-ordered w13 output, so its block map may be another one, of
 * another block size, from moe_align_block_size on the same routing); down
 * bf16 [T*top_k, K] in (token, slot) order; rows of unrouted slots are not
 * written. */
moe_status_t moe_grouped_gemm_w2_indexed(
    const moe_problem_t* p, const void* a2_q, const void* a2_sf, const int32_t* sorted_ids,
    const int32_t* expert_ids, const int32_t* num_tokens_padded, int32_t block_size,
    const void* w2, const void* w2_sf, void* down, void* ws, size_t ws_bytes, void* stream);

/* Step 6 on the (token, slot) order (moe_fused_mul_sum): out[t] =
 * bf16(sum over j ascending with topk_idx[t, j] in [0, E) of topk_w[t, j] *
 * down[t * top_k + j]), accumulated in fp32; tokens with no routed slot get
 * 0.  out: bf16 [T, K]. */
moe_status_t moe_fused_mul_sum(const moe_problem_t* p, const void* down, const int64_t* topk_idx,
                               const float* topk_w, void* out, void* stream);

/* Steps 1-6 on one stream: the staging of prepare_megamoe_inputs
 * ("vllm.model_executor.layers.fused_moe.prepare_megamoe") followed by one
 * apply() of the experts ("...experts.fused_humming_moe",
 * HummingGroupedExperts.apply for the contiguous layout,
 * BatchedHummingGroupedExperts.apply for the batched one,
 * HummingIndexedExperts.apply for the indexed one): fused w13 + activation,
 * w2, reduce.
 * Arguments as in moe_stage plus the weights and out bf16 [T, K]; ws: device
 * workspace of moe_workspace_size bytes.  Any supported scheme pair and
 * activation (_NO_MUL ones run the w13 GEMM and the activation kernel
 * separately, through a gate_up region of the workspace).  Layout
 * INDEXED runs stage, moe_align_block_size with block size tile_m, the two
 * indexed GEMMs and moe_fused_mul_sum. */
moe_status_t moe_forward(const moe_problem_t* p, const void* hidden,
                         const int32_t* expert_num_tokens_in, const int32_t* topk_ids,
                         const float* topk_weights, const uint8_t* is_padding,
                         const moe_eplb_t* eplb, const void* w13, const void* w13_sf,
                         const void* w2, const void* w2_sf, void* out, void* ws,
                         size_t ws_bytes, void* stream);

/* moe_forward for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments and results as moe_forward (bit-identical output), without
 * ws / ws_bytes: the workspace is a static device array of
 * MOE_STATIC_SCRATCH_BYTES (64 MiB) inside the library, one per GPU, held by
 * every GPU the library runs on until the process ends; a DeepSeek-V3-shaped
 * decode batch (64 tokens, 256 experts, top-8, K 7168, N 2048) needs about
 * 9 MB of it.  The call allocates nothing and creates no stream: all its
 * launches go to `stream` (a two-list GEMM step runs its lists one after the
 * other).  A problem whose
 * moe_workspace_size exceeds the array is rejected with MOE_ERR_WORKSPACE
 * before anything is enqueued.  The array's device address is looked up on
 * the first call on each device (the current device; stream and buffers
 * must belong to it).  All calls on one GPU share its array and leave their
 * intermediates in it: calls that overlap on one GPU (other streams, other
 * threads) race and must be serialized by the caller; nothing in the array
 * needs to start at zero. */
#define MOE_STATIC_SCRATCH_BYTES (64u << 20)
moe_status_t moe_forward_static(const moe_problem_t* p, const void* hidden,
                                const int32_t* expert_num_tokens_in, const int32_t* topk_ids,
                                const float* topk_weights, const uint8_t* is_padding,
                                const moe_eplb_t* eplb, const void* w13, const void* w13_sf,
                                const void* w2, const void* w2_sf, void* out, void* stream);

/* Message of the last failed call on this thread ("" if none).  The
 * argument errors it describes follow the ValueError conditions of
 * prepare_megamoe_inputs and _resolve_hidden_quant
 * ("vllm.model_executor.layers.fused_moe.prepare_megamoe": hidden size not a
 * multiple of 128, mismatched top-k shapes, a scale buffer given or missing
 * for the scheme) and the experts' apply() preconditions (batched format
 * without expert_num_tokens); launch failures are reported as
 * MOE_ERR_LAUNCH with the HIP error string.  The pointer stays valid until
 * the next call on the same thread. */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_FP8_H */
