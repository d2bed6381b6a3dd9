// Grouped fp8 GEMM with 128x128 fp32 weight block scales and per-row,
// per-128 activation group scales, for the fused gate/up (w13) and the down
// (w2) projections of the MoE expert layer.
//
// What it computes ("vllm.model_executor.layers.fused_moe.experts.
// fused_humming_moe", humming_forward on the grouped-contiguous and the
// grouped-masked expert layouts with the kFp8Static128BlockSym weight /
// kFp8Dynamic128Sym activation pair): for each routed row r of expert e and
// output column n,
//   out[r, n] = bf16( sum_b sa[r, b] * sw[e, n/128, b] * sum_{c in block b} a[r, c] * w[e, n, c] )
//
// gfx950 mapping.
//  * One 128-deep scale block is exactly one v_mfma_f32_16x16x128_f8f6f4:
//    each k-step issues one MFMA per 16x16 sub-tile into a zeroed fp32
//    partial, then promotes it into the fp32 accumulator with
//    acc += partial * (sa * sw).
//  * The weight tile is the MFMA's A operand and the activation tile its B
//    operand, so the MFMA result is out^T: each lane owns one output row
//    (activation row) and 4*TN consecutive output columns after a fixed
//    permutation of the weight rows inside the wave tile; the epilogue then
//    writes 16-32 contiguous bytes per lane.
//  * Operand tiles travel HBM -> LDS with buffer_load_dwordx4 ... lds
//    (no register staging) through a ring of STAGES k-steps, so STAGES-1
//    k-steps (up to ~96 KB per CU) are in flight while one is multiplied.
//    The loads are issued from inline asm, so the compiler, which cannot see
//    LDS being written behind its back, neither drains the outstanding
//    loads before every fragment read nor reorders around them; the waits
//    are placed by hand (vmcnt per stage, one barrier per k-step).
//  * Activation rows past an expert's count are never loaded (whole 8-row
//    load groups are skipped, partial ones read zeros through an
//    out-of-range buffer offset) and 16-row sub-tiles without rows of the
//    expert cost no fragment reads and no MFMAs: the number of live
//    sub-tiles is a compile-time constant of the main loop, dispatched once
//    per block.  Sub-tiles are interleaved across the two wave rows so that
//    a short expert still keeps both busy.  Rows of a batched-masked slab
//    past its count are therefore never read.
//  * Work unit = (expert, BN-column weight tile, BM-row activation tile).
//    The tile list comes from the routing step, dealt into 8 XCD-balanced
//    slices; block L runs on XCD L % 8, which walks its own slice in a
//    zipper order (heavy groups from the front, light ones from the back)
//    so that matrix-bound and weight-streaming tiles run together, while
//    consecutive items still share weight or activation tiles in its L2.
//  * Cache policy: weight tiles read by a single block stream with the
//    non-temporal hint; the plain epilogue's outputs are stored
//    non-temporally (the reduce reads them once).
//  * LDS rows are 128 bytes; 16-byte chunks are XOR-swizzled per row so that
//    the fragment reads of a wave spread over the banks.
#include <stdlib.h>

#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace moe {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kRowBytes = 128;      // one k-step of a row: 128 fp8 values
constexpr uint32_t kOutOfRange = 0xF0000000u;
constexpr uint32_t kRsrcWord3 = 0x00020000u;   // raw buffer, 32-bit data format
constexpr int kMaxGroups = 256;                // reduction length <= 32768
#ifndef MOE_ZIP
#define MOE_ZIP 16
#endif
constexpr int kZip = MOE_ZIP;                  // zipper run length (work items)
constexpr int kMaxSplit = 4;                   // split-K ranges at most

// Tile geometry.  BM activation rows x BN weight rows (output columns) per
// block, NW waves arranged WN x WM, each owning a WAVE_N x WAVE_M sub-tile
// of TN x TM 16x16 MFMA tiles.  STAGES k-steps of the LDS ring.
template <int BM_, int BN_, int NW_, int STAGES_>
struct Shape {
  static constexpr int BM = BM_, BN = BN_, NW = NW_, STAGES = STAGES_;
  static constexpr int THREADS = 64 * NW;
  static constexpr int WM = BM >= 64 ? 2 : 1;        // waves along activation rows
  static constexpr int WN = NW / WM;                 // waves along weight rows
  static constexpr int WAVE_N = BN / WN;
  static constexpr int WAVE_M = BM / WM;
  static constexpr int TN = WAVE_N / 16;
  static constexpr int TM = WAVE_M / 16;
  static_assert(TN == 2 || TN == 4, "wave tile rows");
  static_assert(TM >= 1 && TM <= 8, "wave tile columns");
  static_assert(WAVE_N <= 128, "a wave's columns share one weight-scale block");
  static constexpr int LOG_4TN = TN == 4 ? 4 : 3;
  static constexpr int A_BYTES = BM * kRowBytes;
  static constexpr int B_BYTES = BN * kRowBytes;
  static constexpr int SC_WAVES = (BM + 63) / 64;          // waves that load row scales
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES + SC_WAVES * 256;
  static constexpr int NBLK = BN / 128;                    // weight-scale blocks per tile
  // the fp32 weight-scale panel after the ring: NBLK blocks of PG scales
  // (one per k-step), kMaxGroups or, where a deep ring leaves less LDS, the
  // multiples of 64 that still fit (the launcher checks Kd / 128 <= PG)
  static constexpr int PG_FIT = (160 * 1024 - STAGES * STAGE_BYTES) / (NBLK * 4) / 64 * 64;
  static constexpr int PG = PG_FIT < kMaxGroups ? PG_FIT : kMaxGroups;
  static constexpr int LDS_BYTES = STAGES * STAGE_BYTES + NBLK * PG * 4;
  // one buffer_load ... lds instruction moves 64 lanes x 16 bytes = 1 KB
  // (a tile of 160 rows: waves 0-3 issue one more than waves 4-7)
  static constexpr int A_CHUNKS = BM * 8;
  static constexpr int A_INSTR = A_CHUNKS >= THREADS ? (A_CHUNKS + THREADS - 1) / THREADS : 1;
  static constexpr int B_INSTR = BN * 8 / THREADS;
  static constexpr int BLOCKS_PER_CU = (2 * LDS_BYTES <= 160 * 1024) ? 2 : 1;
  static constexpr int MIN_WAVES_PER_EU = BLOCKS_PER_CU * NW / 4;
  static_assert(PG >= 64 && LDS_BYTES <= 160 * 1024, "LDS ring exceeds the CU's LDS");
  static_assert(B_INSTR * THREADS == BN * 8, "weight tile split");
  // most buffer loads into LDS a wave issues per k-step
  static constexpr int LMAX = A_INSTR + B_INSTR + 1;
  static_assert(3 * LMAX < 64, "vmcnt range");
};

// 16-byte chunk c of row r lives at chunk position c ^ key(r).  The keys
// make every ds_read_b128 of a fragment hit distinct 16-byte bank groups,
// both per 8-lane phase (32 banks) and per 16-lane phase (64 banks):
// activation fragments read 16 consecutive rows, weight fragments the rows
// (rho>>2) * 4TN + (rho&3) after the output-column permutation.
__device__ __forceinline__ int key_a(int r) { return (r & 6) | ((r ^ (r >> 3)) & 1); }
template <int LOG_4TN>
__device__ __forceinline__ int key_b(int r) {
  return ((r ^ (r >> (LOG_4TN + 1))) & 1) | (r & 2) | (((r >> LOG_4TN) & 1) << 2);
}
// e2m1 weight rows are 64 bytes (4 chunks) per k-step: the same requirement
// (checked on the CPU for both bank phases and both wave-tile widths)
template <int LOG_4TN>
__device__ __forceinline__ int key_w4(int r) {
  return ((r >> LOG_4TN) & 1) | ((((r >> 1) ^ (r >> (LOG_4TN + 1))) & 1) << 1);
}

// ---- LDS ring synchronisation ------------------------------------------
// The ring is filled by buffer_load ... lds issued from inline asm, so the
// compiler does not know LDS is written behind its back and neither drains
// the outstanding loads before every LDS read nor reorders around them: the
// waits below (asm with a memory clobber) are the only synchronisation.
// vmcnt counts only these loads inside the main loop (every other operand
// comes from LDS), so "at most N outstanding" means "all but the last N
// issued have landed".
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"

// Wait until at most N of this wave's LDS-bound loads are in flight and its
// own LDS reads have completed, then barrier.
template <int N>
__device__ __forceinline__ void wait_then_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"i"(N) : "memory");
#endif
}

// `after` = how many later k-steps (L loads each) may still be in flight.
// L is per wave and per block (waves skip the loads of rows an expert does
// not have), so it is dispatched to a compile-time immediate here.
template <int L>
__device__ __forceinline__ void wait_stages_l(int after) {
  if (after <= 0)
    wait_then_barrier<0>();
  else if (after == 1)
    wait_then_barrier<L>();
  else if (after == 2)
    wait_then_barrier<2 * L>();
  else
    wait_then_barrier<3 * L>();
}
// Wait until at most n (wave-uniform, <= NMAX) LDS-bound loads are in
// flight, then barrier.
template <int NMAX, int N = 0>
__device__ __forceinline__ void wait_n_then_barrier(int n) {
  if constexpr (N < NMAX) {
    if (n != N) {
      wait_n_then_barrier<NMAX, N + 1>(n);
      return;
    }
  }
  wait_then_barrier<N>();
}

template <int LMAX, int L = 0>
__device__ __forceinline__ void stage_landed(int loads_per_stage, int after) {
  if constexpr (L < LMAX) {
    if (loads_per_stage != L) {
      stage_landed<LMAX, L + 1>(loads_per_stage, after);
      return;
    }
  }
  wait_stages_l<L>(after);
}

// Raw buffer resource over [base, base + num_records): offsets at or past
// num_records read zeros.  Kept in SGPRs.
__device__ __forceinline__ v4i buffer_rsrc(const void* base, uint32_t num_records) {
  const uint64_t b = (uint64_t)base;
  return v4i{__builtin_amdgcn_readfirstlane((int)(uint32_t)b),
             __builtin_amdgcn_readfirstlane((int)((b >> 32) & 0xFFFFu)),
             __builtin_amdgcn_readfirstlane((int)num_records), (int)kRsrcWord3};
}

// HBM -> LDS: lane l's 16 (4) bytes at rsrc + voffset land at lds + 16*l (4*l).
__device__ __forceinline__ void dma16(v4i rsrc, uint32_t lds, uint32_t voffset) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               ::"s"(lds), "v"(voffset), "s"(rsrc) : "memory", "m0");
#endif
}
// Weight tiles.  stream (wave-uniform): no other block reads this tile, so
// the copy carries the non-temporal hint and leaves L2 to the tiles that
// are shared (activation rows, the weight tiles of multi-tile groups).
// Measured: DSv3-shaped decode w13 -15 %, w2 -19 %; prefill w13 -1 %, w2
// -2 %; the hint on every weight tile instead costs 1.7 % where groups of
// many m-tiles share them (Qwen3-shaped).
__device__ __forceinline__ void dma16_w(v4i rsrc, uint32_t lds, uint32_t voffset, bool stream) {
#if defined(__HIP_DEVICE_COMPILE__)
  if (stream)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
                 ::"s"(lds), "v"(voffset), "s"(rsrc) : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 ::"s"(lds), "v"(voffset), "s"(rsrc) : "memory", "m0");
#endif
}
__device__ __forceinline__ void dma4(v4i rsrc, uint32_t lds, uint32_t voffset) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               ::"s"(lds), "v"(voffset), "s"(rsrc) : "memory", "m0");
#endif
}
#pragma clang diagnostic pop

// f(integral_constant<int, v>) for a wave-uniform v in [0, N].
template <int N, class F>
__device__ __forceinline__ void with_constant(int v, F&& f) {
  if constexpr (N > 0) {
    if (v == N) {
      f(std::integral_constant<int, N>{});
      return;
    }
    with_constant<N - 1>(v, f);
  } else {
    f(std::integral_constant<int, 0>{});
  }
}

// bf16 activation rows (256 bytes per k-step): the row is stored as two
// 128-byte virtual rows v = 2r + bit 2 of the chunk, chunk
// cc = (c & 3) | (c >> 3) << 2 of v at position cc ^ key_a(v).  Read m of a
// k-step gives lane group kq chunk 4kq + m: per 16-lane pass, 16 rows at one
// chunk.  Probed on the part (SQ_LDS_BANK_CONFLICT per ds_read_b128): a
// plain 256-byte row with key r & 15 costs 4 conflict cycles per read; this
// layout none.  a16_chunk_at(r, p) = the logical chunk at position p of row r.
__device__ __forceinline__ int a16_chunk_at(int r, int p) {
  const int b = p >> 3;
  const int cc = (p & 7) ^ key_a(2 * r + b);
  return (cc & 3) | (b << 2) | ((cc >> 2) << 3);
}

// MX fp8 rows: logical 16-byte chunk c of a k-step is stored at physical
// chunk 2 (c mod 4) + (c >= 4) (before the row's XOR key), so the chunk pair
// (kq, kq + 4) the MX operand layout gives lane group kq is read from
// physical chunks (2kq, 2kq + 1) -- the block scheme's pattern, which reads
// without bank conflicts.  mx_chunk_of(p) = the logical chunk at physical p.
__device__ __forceinline__ int mx_chunk_of(int p) { return (p >> 1) | ((p & 1) << 2); }

// MX weight-scale panel: row n's 16 bytes sit at position wsc_rot(n), a
// rotation by 4 * ((n >> 4) & 3) inside each group of 16 rows.  One read of
// the panel covers the 16 rows wn*WAVE_N + 16q + r + 4i (q, r < 4): unrotated
// they are 256 bytes apart in groups of four and hit only 4 banks (4-way
// conflicts, measured as ~2e8 conflict cycles per launch); rotated, their
// positions are distinct modulo 16, so their words fall in distinct banks.
__device__ __forceinline__ int wsc_rot(int n) {
  return (n & ~15) | ((n + 4 * ((n >> 4) & 3)) & 15);
}
__device__ __forceinline__ int wsc_unrot(int pos) {
  return (pos & ~15) | ((pos - 4 * ((pos >> 4) & 3)) & 15);
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p;
}

// ACT (w13 only): the block's 256 weight rows are the gate rows j0 + [0, 128)
// and the up rows N + j0 + [0, 128) of one 128-column group j0 of h, laid
// out so that each wave holds 32 gate rows followed by the 32 matching up
// rows; the epilogue turns the result into f(gate) * up (f the gated
// activation p.activation, SiLU on the hot path), quantized per 128 columns,
// instead of storing it.
//
// SC selects the scale scheme: kQuantUe8m0 / kQuantF32 (128x128 fp32 weight
// block scales, per-128 activation scales, fp32 promotion per k-step) or
// kQuantMxfp8 (E8M0 scale per row and 32 columns on both operands, handed
// to the MFMA itself, which then accumulates across k-steps directly).
// NP: n-tiles per work item.  With NP = 2 (plain GEMM, per-128 scale
// schemes, no split) a block computes two neighbouring n-tiles of its m-tile
// in one k-loop of 2G steps: the second tile's first copies go out during
// the first tile's last k-steps, and its epilogue stores overlap them.
template <class S, int SC, bool ACT, int NP = 1>
__global__ __launch_bounds__(S::THREADS, S::MIN_WAVES_PER_EU) void grouped_gemm_kernel(
    const GemmArgs p) {
  static_assert(!ACT || (S::BN == 256 && S::WN == 4 && S::TN == 4), "fused activation tile");
  static_assert(NP == 1 || (NP == 2 && !ACT && (SC == kQuantUe8m0 || SC == kQuantF32)),
                "paired n-tiles: plain GEMM, per-128 scales");
  constexpr bool W4 = SC == kSchemeMxfp8W4;   // e2m1 weights
  constexpr bool A16 = SC == kQuantBf16;      // unquantized bf16 activations
  // activation-tile bytes per row and k-step (128 fp8 or 128 bf16 values)
  constexpr int AROW = A16 ? 2 * kRowBytes : kRowBytes;
  constexpr int AB = S::BM * AROW;
  constexpr int ACH = AROW / 16;                          // 16-byte chunks per row
  constexpr int AI = S::BM * ACH >= S::THREADS ? (S::BM * ACH + S::THREADS - 1) / S::THREADS : 1;
  constexpr int RPI = 64 / ACH;                           // rows per load instruction
  constexpr bool MX = SC == kQuantMxfp8 || W4;
  constexpr bool UE8M0 = SC == kQuantUe8m0;
  // weight-tile bytes per row and k-step (128 e4m3 or 128 e2m1 values)
  constexpr int WROW = W4 ? 64 : kRowBytes;
  constexpr int BB = S::BN * WROW;
  constexpr int BI = BB / (S::THREADS * 16);
  static_assert(BI * S::THREADS * 16 == BB, "weight tile split");
  constexpr int SC_OFF = AB + BB;            // activation-scale words of a stage
  // MX: the weight rows' E8M0 bytes of 4 k-steps (16 per row) arrive with
  // every fourth stage into one of two panel slots after the ring; the
  // block scheme keeps its fp32 weight-scale panel there instead
  constexpr int STAGE = SC_OFF + (A16 ? 0 : S::SC_WAVES * 256);
  constexpr int WSC_SLOT = S::BN * 16;
  constexpr int PANEL = MX ? 2 * WSC_SLOT : NP * S::NBLK * S::PG * 4;
  constexpr int LDS = S::STAGES * STAGE + PANEL;
  constexpr int LMAX = AI + BI + 1 + (MX ? 1 : 0);
  static_assert(LDS <= 160 * 1024 && 3 * LMAX < 64, "LDS ring / vmcnt range");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[LDS];

  // ---- which (expert, m-tile, n-tile) this block computes ----------------
  // Workgroups go to the 8 XCDs round-robin (block L to XCD L % 8).  Each
  // XCD walks its own share of the work, group by group and, inside a group
  // (one expert's consecutive m-tiles), n-tile-major: the blocks that run
  // together on one XCD share weight tiles (the group's m-tiles) and
  // activation tiles (neighbouring n-tiles) in its L2.
  // Indexed layout: tile b is block b of sorted_ids; XCD x walks the x-th of
  // 8 equal slices of the (block, n-tile) list, n-tiles innermost.  (Runs of
  // 8 blocks dealt to the XCDs in turn measured slower: they split the
  // heavy experts' blocks over more XCDs.)
  const bool indexed = p.sorted_ids != nullptr;
  const int NT = p.Nout / S::BN / NP;   // work items per m-tile (NP n-tiles each)
  // split-K: the S splits of one (tile, n-tile) item are consecutive work
  // items, so they run at about the same time (the last one's partial reads
  // then find the others' partials still in L2 / MALL)
  const int nsplit = ACT ? 1 : max(p.ksplit, 1);
  int split = 0;
  int tile, nt, e, m0, rows_here;
  bool w_once = false;   // this block is the weight tile's only reader
  int64_t base;
  // The schedule the routing step built, as a work list: this XCD's slice,
  // taken in the zipper order described below, then the (tile, n-tile) item
  // it names.  Returns false past the work.
  auto schedule_item = [&](int& t_out, int& nt_out, const int32_t*& info_out) -> bool {
    // slices of whole items: an item's splits share an XCD (and its L2)
    const int64_t work = (int64_t)p.tile_list[0] * NT * nsplit;
    const int64_t per_xcd = ((int64_t)p.tile_list[0] * NT + 7) / 8 * nsplit;
    const int64_t xcd = blockIdx.x % 8, j = blockIdx.x / 8;
    const int64_t items = min(per_xcd, work - xcd * per_xcd);   // this XCD's slice
    if (j >= items) return false;
    int64_t pos = j;   // the slice in its own order, or in the zipper order
    if (p.zip) {
      const int64_t u = j / (2 * kZip), v = j % (2 * kZip);
      pos = v < kZip ? u * kZip + v : items - 1 - (u * kZip + v - kZip);
    }
    const int64_t wls = xcd * per_xcd + pos;
    split = __builtin_amdgcn_readfirstlane((int)(wls % nsplit));
    const int64_t wl = wls / nsplit;
    const int t0 = __builtin_amdgcn_readfirstlane((int)(wl / NT));
    const int32_t* info = p.tile_list + 4 + 8 * (int64_t)t0;
    const int first = info[2], mtiles = info[3];
    const int r = (int)(wl - (int64_t)first * NT);
    // super-columns of SN n-tiles, m-tile-major inside
    const int SN = max(p.sn, 1);
    const int sc = r / (SN * mtiles);
    const int sn = min(SN, NT - sc * SN);
    const int rr = r - sc * SN * mtiles;
    nt_out = __builtin_amdgcn_readfirstlane(sc * SN + rr % sn);
    t_out = __builtin_amdgcn_readfirstlane(first + rr / sn);
    info_out = info;
    return true;
  };
  // a tile of the indexed layout's tall list (twice the block size): taken
  // from the schedule like a contiguous tile, positions in sorted_ids
  bool tall_ix = false;
  if (indexed) {
    if (p.tile_list != nullptr) {
      // moe_forward: the blocks in the schedule's XCD-balanced zipper order;
      // tile (e, m-tile i) of the schedule is block first-m-tile(e) + i
      int t = 0;
      const int32_t* info = nullptr;
      if (!schedule_item(t, nt, info)) return;
      const int t0 = (int)(info - (p.tile_list + 4)) / 8;
      if (S::BM != p.block_size) {
        // rows m0 .. of the expert's segment of sorted_ids, which starts at
        // its first block; its routed entries lead the segment, so the first
        // min(BM, count - m0) positions from m0 are all routed (and inside
        // the segment: never the next expert's)
        tall_ix = true;
        tile = t;
        e = info[0];
        m0 = info[1] + (t - t0) * S::BM;
        rows_here = min(S::BM, info[4] - m0);
        base = (int64_t)info[6] * p.block_size;
        w_once = false;
      } else {
        tile = __builtin_amdgcn_readfirstlane(info[6] + (info[1] / S::BM) + (t - t0));
        w_once = S::BM <= 160 && !W4 && info[4] <= S::BM;
      }
    } else {
      // Block order, in groups of 8 blocks: a group of one expert's blocks
      // (consecutive m-tiles of a heavy expert) is taken n-tile-major, so
      // that 8 consecutive items share a weight tile; other groups take each
      // block's n-tiles consecutively (they share its activation rows).
      const int64_t nblk = min(max(*p.num_padded, 0) / S::BM, p.max_blocks);
      const int64_t work = nblk * NT * nsplit;
      const int64_t per_xcd = (nblk * NT + 7) / 8 * nsplit;
      const int64_t wls = (int64_t)(blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
      if (blockIdx.x / 8 >= per_xcd || wls >= work) return;
      split = __builtin_amdgcn_readfirstlane((int)(wls % nsplit));
      const int64_t wl = wls / nsplit;
      const int64_t g0 = wl / (8 * NT) * 8;          // the group's first block
      const int64_t r = wl - g0 * NT;
      const bool full = g0 + 8 <= nblk;
      if (full && p.expert_ids[g0] == p.expert_ids[g0 + 7]) {
        tile = __builtin_amdgcn_readfirstlane((int)(g0 + r % 8));
        nt = __builtin_amdgcn_readfirstlane((int)(r / 8));
      } else {
        tile = __builtin_amdgcn_readfirstlane((int)(g0 + r / NT));
        nt = __builtin_amdgcn_readfirstlane((int)(r % NT));
      }
    }
    if (!tall_ix) {
      // the block's routed entries (ids below numel) lead, padding follows
      e = __builtin_amdgcn_readfirstlane(p.expert_ids[tile]);
      m0 = 0;
      base = (int64_t)tile * S::BM;
      const bool valid =
          threadIdx.x < S::BM && (uint32_t)p.sorted_ids[base + threadIdx.x] < (uint32_t)p.numel;
      rows_here = __syncthreads_count(valid);
      if ((uint32_t)e >= (uint32_t)p.num_experts) return;
    }
  } else {
    // Contiguous / batched layouts: XCD x walks the x-th of 8 equal slices
    // of the schedule the routing step built.  One scalar load of tile t0's
    // information gives its group (first tile, size), expert, rows and first
    // row; the block's tile is in the same group, so the rest follows.
    //
    // The slice lists its heaviest groups first.  Walked in that order, the
    // whole chip first runs only the heavy experts' blocks (many m-tiles
    // sharing weight tiles: bound by L2 / MALL latency, HBM mostly idle),
    // then only the light experts' blocks (weight streaming at the HBM
    // ceiling, matrix cores idle) — measured at the DSv3-shaped prefill
    // batch as two back-to-back phases of about 1 ms each.  So the blocks
    // take the slice in a zipper order instead: kZip items from its front,
    // kZip from its back (walked backwards), and so on, until front and back
    // meet.  Blocks running together on an XCD then mix both kinds, and
    // consecutive items still share a weight tile (heavy side) or an
    // activation tile (light side).  A list of alike experts (one list of
    // 256-row tiles: every expert heavy) keeps the slice's own order, which
    // leaves more of an expert's items running together (Qwen3-shaped
    // fused w13 -2.3 %; the zipper stays for the 128-row lists and the
    // tall list beside them: without it there DSv3-shaped prefill +0.3-0.8 %).
    // p.zip selects.
    int t = 0;
    const int32_t* info = nullptr;
    if (!schedule_item(t, nt, info)) return;
    const int t0 = (int)(info - (p.tile_list + 4)) / 8;
    tile = t;
    e = info[0];
    m0 = info[1] + (tile - t0) * S::BM;
    rows_here = min(S::BM, info[4] - m0);
    // (e2m1 rows are 64 bytes per k-step: two k-steps share each cache
    // line, so the hint would evict the line before its second half is
    // read — measured +8 % w13, +20 % w2 at the MXFP4 DSv3 batch)
    // Tiles of 192 / 256 rows are picked for experts with hundreds of rows,
    // whose weight tiles are shared: those shapes keep one load form (the
    // run-time choice alone cost 2-3 % on the Qwen3-shaped fused w13).  The
    // 160-row tiles hold whole experts of about 100-160 rows: there the
    // hint halved the weight stream's time per k-step (8 experts of ~128
    // rows, N = 14336: w2 0.213 -> 0.179 ms, fused w13 0.289 -> 0.253 ms;
    // without it the once-read weight lines evict the shared activation rows).
    // An expert of one m-tile is the only reader of its weight tiles; the
    // last chunk of a longer expert is not (its other chunks read the same
    // tiles), whatever that chunk's own size.
    w_once = S::BM <= 160 && !W4 && info[4] <= S::BM;
    base = info[5];
  }
  const int n0 = nt * S::BN * NP;     // first output column (plain GEMM)
  const int Nh = p.Nout / 2;            // ACT: columns of h
  const int j0 = nt * (S::BN / 2);      // ACT: first column of h

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int wn = wave % S::WN;
  const int wm = wave / S::WN;
  // k-steps of this block: all of them, or this split's range (a multiple
  // of 4 k-steps long, so the 4-k-step cadence of the MX weight-scale panel
  // and of the UE8M0 scale words starts at its first step).  Loop indices
  // below are relative to k0 (ring slots, prologue), offsets absolute.
  const int G_all = p.Kd / kGroup;
  int k0 = 0, G = G_all;
  if (nsplit > 1) {
    const int chunk = ((G_all + nsplit - 1) / nsplit + 3) & ~3;
    k0 = min(split * chunk, G_all);
    G = min(G_all, k0 + chunk) - k0;
  }
  // The block walks its G k-steps from step rot on, wrapping round (p.krot):
  // when the weight rows are a multiple of 4 KB long, blocks that stream at
  // the same k-step read the same offset of every row, which concentrates
  // the reads on a few HBM channels (a probe: 4.7 TB/s at a 4096-byte row
  // stride, 6.3 TB/s with the step order staggered per block; in the GEMMs,
  // whose blocks drift apart, it measured -1.5 % on a fused w13 of 8
  // experts at K = 4096 and -0.8 % on one of 144 experts).  rot depends
  // on the expert and on the output columns' 256-column pair only (w13:
  // counted within the gate or the up half), so the fused and the unfused
  // w13, every tile height and width, and every batch add a column's
  // k-steps in the same order.
  int rot = 0, rot1 = 0;   // rot1: the second n-tile's (NP = 2)
  if constexpr (!MX) {
    if (p.krot != 0 && G > 1) {
      const int key = ((ACT ? j0 : n0) % p.rot_period) / 256;
      rot = __builtin_amdgcn_readfirstlane((5 * key + 3 * e) % G);
      if constexpr (NP == 2) {
        const int key1 = ((n0 + S::BN) % p.rot_period) / 256;
        rot1 = __builtin_amdgcn_readfirstlane((5 * key1 + 3 * e) % G);
      }
    }
  }
  // the loop's steps: G per n-tile, NP n-tiles (steps G .. 2G-1: the second)
  const int GG = NP * G;
  // absolute k-step of the block's kb-th step
  auto kabs = [&](int kb) {
    if constexpr (NP == 2) {
      const bool h = kb >= G;
      const int r = (h ? kb - G : kb) + (h ? rot1 : rot);
      return k0 + (r >= G ? r - G : r);
    } else {
      const int r = kb + rot;
      return k0 + (r >= G ? r - G : r);
    }
  };

  // activation row of tile row m (an id that is padding gathers row T,
  // past the buffer's end: the buffer loads return zeros there)
  auto a_row_of = [&](int m) -> int64_t {
    const int64_t r = base + m0 + m;
    if (p.gather_sorted) return (int64_t)((uint32_t)p.sorted_ids[r] / (uint32_t)p.top_k);
    return p.row_src != nullptr ? (int64_t)p.row_src[r] : r;
  };
  // output row of tile row m, or -1 for a padding entry of the indexed layout
  // (which writes row sorted_ids[position], the (token, slot) order)
  auto out_row_of = [&](int m) -> int64_t {
    const int64_t r = base + m0 + m;
    if (!p.scatter_sorted) return r;
    const uint32_t id = (uint32_t)p.sorted_ids[r];
    return id < (uint32_t)p.numel ? (int64_t)id : -1;
  };

  // ---- HBM -> LDS copy plan: thread tid fills 16-byte slot i*THREADS + tid
  // The weight tile needs only the expert and the n-tile: its first k-steps
  // are issued before the activation rows are looked up (their gather loads
  // then overlap these copies).
  const uint32_t smem_base = lds_addr(smem);
  const int wave_slot = __builtin_amdgcn_readfirstlane(wave * 1024);
  const int wstride = W4 ? p.Kd / 2 : p.Kd;   // weight row bytes
  const v4i rs_b =
      ACT ? buffer_rsrc(p.w + (int64_t)e * p.Nout * wstride,
                        (uint32_t)((int64_t)p.Nout * wstride))
          : buffer_rsrc(p.w + ((int64_t)e * p.Nout + n0) * wstride,
                        (uint32_t)(NP * S::BN * wstride));
  uint32_t b_off[BI];
#pragma unroll
  for (int i = 0; i < BI; ++i) {
    const int slot = i * S::THREADS + tid;
    const int r = W4 ? slot >> 2 : slot >> 3;
    const int c = W4   ? (slot & 3) ^ key_w4<S::LOG_4TN>(r)
                  : MX ? mx_chunk_of((slot & 7) ^ key_b<S::LOG_4TN>(r))
                       : (slot & 7) ^ key_b<S::LOG_4TN>(r);
    int64_t wrow = r;
    if (ACT) {
      // tile row r = 64*w + q: gate row j0 + 32w + q (q < 32), else up row
      const int q = r & 63, w = r >> 6;
      wrow = (q < 32 ? 0 : Nh - 32) + j0 + 32 * w + q;
    }
    b_off[i] = (uint32_t)(wrow * wstride + c * 16);
  }
  auto issue_b = [&](int kb) {
    const uint32_t st = smem_base + (kb % S::STAGES) * STAGE;
#pragma unroll
    for (int i = 0; i < BI; ++i)
      dma16_w(rs_b, st + AB + i * S::THREADS * 16 + wave_slot,
              b_off[i] + (NP == 2 && kb >= G ? (uint32_t)(S::BN * wstride) : 0u) +
                  (uint32_t)kabs(kb) * WROW,
              w_once);
  };
#pragma unroll
  for (int s = 0; s < S::STAGES - 1; ++s)
    if (s < GG) issue_b(s);

  const v4i rs_a = buffer_rsrc(p.a, p.a_bytes);
  const v4i rs_s = buffer_rsrc(p.a_sf, p.a_sf_bytes);
  // A: load instruction q (64 lanes = 8 rows x 8 chunks) belongs to wave
  // q % NW; only instructions covering rows of the expert are issued (rows
  // past its count are never read; their LDS slots keep stale bytes, which
  // only ever meet output rows that are not stored).
  const int a_groups = (rows_here + RPI - 1) / RPI;
  const int a_loads = a_groups > wave ? (a_groups - wave + S::NW - 1) / S::NW : 0;
  uint32_t a_off[AI];
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    const int slot = i * S::THREADS + tid;
    // bf16 rows (16 chunks): the two-virtual-row layout of a16_chunk_at
    const int r = slot / ACH;
    const int c = A16  ? a16_chunk_at(r, slot % ACH)
                  : MX ? mx_chunk_of((slot & 7) ^ key_a(r))
                       : (slot & 7) ^ key_a(r);
    a_off[i] = (r < rows_here) ? (uint32_t)(a_row_of(r) * p.Kd * (A16 ? 2 : 1) + c * 16)
                               : kOutOfRange;
  }
  // activation scales: one 4-byte word per row and k-step (UE8M0: the word
  // holding the step's exponent byte; fp32: the scale itself; MX: the step's
  // four 32-column exponent bytes)
  const bool loads_sc = !A16 && wave < S::SC_WAVES && wave * 64 < rows_here;
  // MX weight scales: tile row wave*64 + lane's 16 bytes (4 k-steps), loaded
  // with stages kb = 0 mod 4 only
  const bool loads_wsc = MX && wave < S::BN / 64;
  const int loads_per_stage = a_loads + BI + (loads_sc ? 1 : 0);
  uint32_t sc_off = kOutOfRange;
  {
    const int r = wave * 64 + lane;
    if (loads_sc && r < rows_here)
      sc_off = (uint32_t)(a_row_of(r) * p.a_sf_stride * (SC == kQuantF32 ? 4 : 1));
  }
  const int Gw = p.Kd / 32;   // MX weight-scale bytes per row
  const v4i rs_w = MX ? buffer_rsrc((const uint8_t*)p.w_sf + (int64_t)e * p.Nout * Gw,
                                    (uint32_t)((int64_t)p.Nout * Gw))
                      : v4i{0, 0, 0, 0};
  uint32_t wsc_off = 0;
  if (MX) {
    // this lane fills panel position (wave * 64 + lane) % BN with the row
    // stored there
    const int r = wsc_unrot((wave * 64 + lane) % S::BN);
    int64_t wrow = n0 + r;
    if (ACT) {
      const int q = r & 63, w = r >> 6;
      wrow = (q < 32 ? 0 : Nh - 32) + j0 + 32 * w + q;
    }
    wsc_off = (uint32_t)(wrow * Gw);
  }
  const int wave_sc = __builtin_amdgcn_readfirstlane(wave * 256);
  // weight block scales of this tile's NBLK 128-column blocks, one per
  // k-step: wave b copies block b's G floats straight into the LDS panel
  // (no register round trip, so nothing waits on these loads here: the
  // first k-step's wait covers them)
  float* sw_panel = reinterpret_cast<float*>(smem + S::STAGES * STAGE);
  if constexpr (!MX) {
    if (wave < NP * S::NBLK) {
      const int b = wave;
      // ACT: block 0 = the gate rows' scale block, block 1 = the up rows'
      const int blk = ACT ? (b == 0 ? j0 : Nh + j0) / kGroup : n0 / kGroup + b;
      const v4i rs_p = buffer_rsrc((const uint8_t*)p.w_sf +
                                       (((int64_t)e * (p.Nout / kGroup) + blk) * G_all) * 4,
                                   (uint32_t)(G_all * 4));
      const uint32_t dst = smem_base + S::STAGES * STAGE + b * S::PG * 4;
      for (int g0 = 0; g0 < G_all; g0 += 64)
        dma4(rs_p, dst + g0 * 4, (uint32_t)((g0 + lane) * 4));
    }
  }

  // ---- per-lane MFMA fragment offsets (within a stage) -------------------
  // The 16x16x128 f8f6f4 MFMA reads lane l's 32 operand bytes as k values
  // 16*(l>>4) + [0, 16) (registers 0-3) and 64 + 16*(l>>4) + [0, 16)
  // (registers 4-7), and takes the E8M0 scale of 32-column block b from lane
  // group b: under MX, lane group kq therefore needs 16-byte chunks kq and
  // kq + 4 of the row's 128-byte k-step, which the copies place at physical
  // chunks 2kq and 2kq + 1 (mx_chunk_of).  With per-128 promotion any
  // consistent placement gives the same sum; there the logical chunks 2kq and
  // 2kq + 1 are read.  Either way every lane reads physical chunks 2kq and
  // 2kq + 1 (before the row's XOR key).
  const int rho = lane & 15;
  const int kq = lane >> 4;
  const int c0 = 2 * kq, c1 = 2 * kq + 1;
  // weight sub-tile i's row for this lane is nl0 + 4*i (same swizzle key)
  const int nl0 = wn * S::WAVE_N + (rho >> 2) * (4 * S::TN) + (rho & 3);
  // e2m1 weights: lane group kq holds k = 32kq + [0, 32), one 16-byte chunk
  const int kbw = W4 ? key_w4<S::LOG_4TN>(nl0) : key_b<S::LOG_4TN>(nl0);
  const int w_frag0 = AB + nl0 * WROW + (((W4 ? kq : c0) ^ kbw) << 4);
  const int w_frag1 = AB + nl0 * WROW + ((c1 ^ kbw) << 4);
  // activation sub-tile j of this wave holds rows 16*(j*WM + wm) + [0, 16)
  // (interleaved across the WM wave rows, so that a short expert still
  // spreads its rows over them); this lane's row is ml0 + 16*WM*j (same
  // swizzle key)
  const int ml0 = wm * 16 + rho;
  const int a_frag0 = ml0 * kRowBytes + ((c0 ^ key_a(ml0)) << 4);
  const int a_frag1 = ml0 * kRowBytes + ((c1 ^ key_a(ml0)) << 4);
  // bf16 activations: MFMA m of a k-step covers k = 32kq + 8m + [0, 8), i.e.
  // chunk 4kq + m of the row (the weight bytes 32kq + 8m + [0, 8) match)
  const int a16_v = 2 * ml0 + (kq & 1);                  // virtual row of chunk 4kq
  const int a16_frag = a16_v * 128 + ((((kq >> 1) << 2) ^ key_a(a16_v)) << 4);
  const int sc_frag = SC_OFF + ml0 * 4;
  // MX: the panel positions of weight rows nl0 + 4i (sub-tile i)
  int wsc_frag[S::TN];
#pragma unroll
  for (int i = 0; i < S::TN; ++i) wsc_frag[i] = S::STAGES * STAGE + wsc_rot(nl0 + 4 * i) * 16;
  const int scale_shift = 8 * kq;            // MX: this lane's 32-column k-group byte
  constexpr int kSubStride = 16 * S::WM;
  // the weight-scale block of this lane's output columns (ACT: lanes 0-31
  // hold gate rows, lanes 32-63 up rows)
  const float* sw_mine =
      sw_panel + (ACT ? (kq >= 2 ? 1 : 0) : (wn * S::WAVE_N) / 128) * S::PG;
  // the weight scale of step kb (NP = 2: the second n-tile's blocks follow
  // the first's in the panel)
  auto sw_of = [&](int kb) {
    return sw_mine[(NP == 2 && kb >= G ? S::NBLK * S::PG : 0) + kabs(kb)];
  };

  // the rest of a k-step: activation rows, their scales, MX weight scales
  // (kb: the block's step index, kabs(kb) the k-step it loads; the MX
  // schemes never rotate and k0 is a multiple of 4, so there kb & 3 is the
  // absolute k-step's position in its group of 4)
  auto issue_as = [&](int kb) {
    const uint32_t st = smem_base + (kb % S::STAGES) * STAGE;
    const int ka = kabs(kb);
#pragma unroll
    for (int i = 0; i < AI; ++i)
      if (i < a_loads)
        dma16(rs_a, st + i * S::THREADS * 16 + wave_slot, a_off[i] + (uint32_t)ka * AROW);
    if (loads_sc) {
      const uint32_t soff = UE8M0 ? (uint32_t)(ka & ~3) : (uint32_t)ka * 4;
      dma4(rs_s, st + SC_OFF + wave_sc, sc_off + soff);
    }
    if (loads_wsc && (kb & 3) == 0)
      dma16(rs_w, smem_base + S::STAGES * STAGE + ((kb >> 2) & 1) * WSC_SLOT + wave_slot,
            wsc_off + (uint32_t)ka * 4);
  };
  auto issue = [&](int kb) {
    issue_as(kb);
    issue_b(kb);
  };
  // loads of k-step s that the prologue issues after every weight copy
  auto as_loads = [&](int s) {
    return a_loads + (loads_sc ? 1 : 0) + (loads_wsc && (s & 3) == 0 ? 1 : 0);
  };

  v4f acc[S::TN][S::TM];
#pragma unroll
  for (int i = 0; i < S::TN; ++i)
#pragma unroll
    for (int j = 0; j < S::TM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // One k-step over the first LIVE activation sub-tiles (the ones holding
  // rows of the expert; the rest cost no LDS reads and no MFMAs): one MFMA
  // per 16x16 sub-tile (K = 128 = one scale block), in activation-major
  // order t = j*TN + i; each partial is promoted into the fp32 accumulator
  // two MFMAs after issue, once it has left the matrix pipe.
  auto compute = [&](int kb, auto live_c) {
    constexpr int LIVE = decltype(live_c)::value;
    if constexpr (A16 && LIVE > 0) {
      // bf16 activations x fp8 weights converted to bf16 (exact): four
      // 16x16x32 bf16 MFMAs per sub-tile per 128-deep block, chained in a
      // partial, then acc += partial * sw
      const uint8_t* sb = smem + (kb % S::STAGES) * STAGE;
      const float sw = sw_of(kb);
      v8bf wb[S::TN][4];
#pragma unroll
      for (int i = 0; i < S::TN; ++i) {
        const v4i lo = *reinterpret_cast<const v4i*>(sb + w_frag0 + i * 4 * WROW);
        const v4i hi = *reinterpret_cast<const v4i*>(sb + w_frag1 + i * 4 * WROW);
        const int words[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          v4i packed;
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            const int w = words[2 * m + h2];
            const v2f f01 = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
            const v2f f23 = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
            // e4m3 values are exact in bf16: keep the upper halves
            packed[2 * h2] = (int)__builtin_amdgcn_perm(__float_as_uint(f01.y),
                                                        __float_as_uint(f01.x), 0x07060302u);
            packed[2 * h2 + 1] = (int)__builtin_amdgcn_perm(__float_as_uint(f23.y),
                                                            __float_as_uint(f23.x), 0x07060302u);
          }
          wb[i][m] = __builtin_bit_cast(v8bf, packed);
        }
      }
#pragma unroll
      for (int j = 0; j < LIVE; ++j) {
        v8bf ab[4];
#pragma unroll
        for (int m = 0; m < 4; ++m)
          ab[m] = __builtin_bit_cast(
              v8bf, *reinterpret_cast<const v4i*>(sb + (a16_frag ^ (m << 4)) +
                                                  j * kSubStride * AROW));
        v4f part[S::TN];
#pragma unroll
        for (int i = 0; i < S::TN; ++i) part[i] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
          for (int i = 0; i < S::TN; ++i)
            part[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wb[i][m], ab[m], part[i], 0, 0, 0);
#pragma unroll
        for (int i = 0; i < S::TN; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] = fmaf(part[i][r], sw, acc[i][j][r]);
      }
    } else if constexpr (MX && LIVE > 0) {
      // both operands carry E8M0 scales per (row, 32 columns): lane l's byte
      // for its row and k-group l >> 4 goes to the MFMA, which accumulates
      // straight into acc (byte 127 = 1.0)
      const uint8_t* sb = smem + (kb % S::STAGES) * STAGE;
      v8i wf[S::TN];
      int sw[S::TN];
#pragma unroll
      for (int i = 0; i < S::TN; ++i) {
        const v4i lo = *reinterpret_cast<const v4i*>(sb + w_frag0 + i * 4 * WROW);
        if constexpr (W4) {
          // an e2m1 operand is 4 registers; the upper four are not read
          wf[i] = v8i{lo.x, lo.y, lo.z, lo.w, 0, 0, 0, 0};
        } else {
          const v4i hi = *reinterpret_cast<const v4i*>(sb + w_frag1 + i * 4 * WROW);
          wf[i] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
        sw[i] = (int)(*reinterpret_cast<const uint32_t*>(
                          smem + wsc_frag[i] + ((kb >> 2) & 1) * WSC_SLOT + (kb & 3) * 4) >>
                      scale_shift);
      }
#pragma unroll
      for (int j = 0; j < LIVE; ++j) {
        const v4i lo = *reinterpret_cast<const v4i*>(sb + a_frag0 + j * kSubStride * kRowBytes);
        const v4i hi = *reinterpret_cast<const v4i*>(sb + a_frag1 + j * kSubStride * kRowBytes);
        const v8i af = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        const int sa =
            (int)(*reinterpret_cast<const uint32_t*>(sb + sc_frag + j * kSubStride * 4) >>
                  scale_shift);
#pragma unroll
        for (int i = 0; i < S::TN; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              wf[i], af, acc[i][j], W4 ? 4 : 0, 0, 0, sw[i], 0, sa);
      }
    } else if constexpr (LIVE > 0) {
      const uint8_t* sb = smem + (kb % S::STAGES) * STAGE;
      v8i wf[S::TN], af[LIVE];
      float fs[LIVE];
#pragma unroll
      for (int i = 0; i < S::TN; ++i) {
        const v4i lo = *reinterpret_cast<const v4i*>(sb + w_frag0 + i * 4 * kRowBytes);
        const v4i hi = *reinterpret_cast<const v4i*>(sb + w_frag1 + i * 4 * kRowBytes);
        wf[i] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
      const float sw = sw_of(kb);
      // activation fragment j (and its scale) is read when sub-tile j-1's
      // MFMAs start, so at most two are live
      auto load_a = [&](int j, v8i& f, float& fs) {
        const v4i lo = *reinterpret_cast<const v4i*>(sb + a_frag0 + j * kSubStride * kRowBytes);
        const v4i hi = *reinterpret_cast<const v4i*>(sb + a_frag1 + j * kSubStride * kRowBytes);
        f = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        const uint32_t word = *reinterpret_cast<const uint32_t*>(sb + sc_frag + j * kSubStride * 4);
        const float sa = UE8M0 ? __uint_as_float(((word >> ((kabs(kb) & 3) * 8)) & 0xFFu) << 23)
                               : __uint_as_float(word);
        fs = sa * sw;
      };
      load_a(0, af[0], fs[0]);
      constexpr int NT = S::TN * LIVE;
      v4f part[3];
#pragma unroll
      for (int t = 0; t < NT + 2; ++t) {
        if (t < NT) {
          if (t % S::TN == 0 && t / S::TN + 1 < LIVE)
            load_a(t / S::TN + 1, af[t / S::TN + 1], fs[t / S::TN + 1]);
          const v4f z = {0.f, 0.f, 0.f, 0.f};
          // Constant zero scale operands make the compiler emit the unscaled
          // v_mfma_f32_16x16x128_f8f6f4 (scale 1.0; the scales are applied in
          // the promotion).  A register holding E8M0 127 would mean the same
          // but selects the scaled encoding, measured ~2% slower here; a
          // scaled instruction with zero operands would mean 2^-254, which
          // every parity test would catch.
          part[t % 3] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              wf[t % S::TN], af[t / S::TN], z, 0, 0, 0, 0, 0, 0);
        }
        if (t >= 2) {
          const int u = t - 2, i = u % S::TN, j = u / S::TN;
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] = fmaf(part[u % 3][r], fs[j], acc[i][j][r]);
        }
        // keep the rolling order: without this fence the scheduler sinks
        // every promotion to the end of the k-step, which keeps all
        // partials live at once
        if constexpr (S::TM * S::TN > 16) __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // plain GEMM epilogue: this lane's rows of acc as bf16, columns nf + [0, 4TN)
  auto store_rows = [&]([[maybe_unused]] int nf) {
    if constexpr (!ACT) {
#pragma unroll
      for (int j = 0; j < S::TM; ++j) {
        const int ml = ml0 + kSubStride * j;
        if (ml >= rows_here) continue;
        const int64_t row = out_row_of(ml);
        if (row < 0) continue;
        uint16_t* dst = p.out + row * (int64_t)p.Nout + nf;
        uint32_t packed[2 * S::TN];
#pragma unroll
        for (int i = 0; i < S::TN; ++i) {
          packed[2 * i] = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
          packed[2 * i + 1] = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
        }
#pragma unroll
        for (int v = 0; v < S::TN / 2; ++v) {
          // written once, read once by the reduce: non-temporal (measured
          // w2 -0.6 % DSv3-shaped, -2.2 % Qwen3-shaped)
          const v4i o = {(int)packed[4 * v], (int)packed[4 * v + 1], (int)packed[4 * v + 2],
                         (int)packed[4 * v + 3]};
          __builtin_nontemporal_store(o, reinterpret_cast<v4i*>(dst) + v);
        }
      }
    }
  };

  auto main_loop = [&](auto live_c) {
    // prologue: STAGES-1 k-steps in flight (their weight copies went first)
#pragma unroll
    for (int s = 0; s < S::STAGES - 1; ++s)
      if (s < GG) issue_as(s);
    for (int kb = 0; kb < GG; ++kb) {
      // k-step kb has landed for every wave, and every wave's reads of
      // k-step kb-1 (whose slot the next issue reuses) have completed
      // (NP = 2: the first tile's epilogue stores, issued after later
      // copies, only make these waits longer, never shorter: the copies
      // land in issue order)
      const int after = min(kb + S::STAGES - 2, GG - 1) - kb;
      if (kb < S::STAGES - 2) {
        // loads issued after k-step kb's last one: the activation parts of
        // the later prologue k-steps and the whole k-steps issued since
        int n = 0;
        for (int s2 = kb + 1; s2 <= kb + after; ++s2)
          n += as_loads(s2) + (s2 < S::STAGES - 1 ? 0 : BI);
        wait_n_then_barrier<3 * LMAX>(n);
      } else if constexpr (MX) {
        // later stages in flight, plus the panel loads among them
        int n = after * loads_per_stage;
        if (loads_wsc)
          for (int s2 = kb + 1; s2 <= kb + after; ++s2) n += (s2 & 3) == 0 ? 1 : 0;
        wait_n_then_barrier<3 * LMAX>(n);
      } else {
        stage_landed<LMAX>(loads_per_stage, after);
      }
      if (kb + S::STAGES - 1 < GG) issue(kb + S::STAGES - 1);
      compute(kb, live_c);
      if constexpr (NP == 2) {
        if (kb == G - 1) {
          // the first n-tile is complete: store it, start the second
          store_rows(n0 + wn * S::WAVE_N + kq * (4 * S::TN));
#pragma unroll
          for (int i = 0; i < S::TN; ++i)
#pragma unroll
            for (int j = 0; j < S::TM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
        }
      }
    }
  };
  // live sub-tiles of this wave (wave-uniform)
  const int live = __builtin_amdgcn_readfirstlane(
      max(0, min(S::TM, (rows_here - wm * 16 + kSubStride - 1) / kSubStride)));
  with_constant<S::TM>(live, main_loop);

  if constexpr (ACT) {
    // ---- fused activation epilogue ----------------------------------------
    // Lane (kq, rho) holds, for activation sub-tile j, wave rows
    // q = 16*kq + 4*i + r: gate columns j0 + 32*wn + q of h for kq < 2, the up
    // columns j0 + 32*wn + q - 32 for kq >= 2, so lanes l and l ^ 32 hold the
    // two halves of the same 32 columns.  After one exchange each lane owns 8
    // consecutive columns: col_off + [0, 8) inside the group.  The values are
    // rounded to bf16 first (the precision of the gate_up buffer of the
    // unfused path), then combined and quantized exactly as the standalone
    // activation kernel does.
    const bool gate_lane = kq < 2;
    const int col_off = 32 * wn + (gate_lane ? 16 * kq : 16 * (kq - 2) + 8);
    float h[S::TM][8];
    float amax[S::TM];
    auto activate = [&](auto f) {
#pragma unroll
      for (int j = 0; j < S::TM; ++j) {
        amax[j] = 0.0f;
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            // swapping the upper half-wave of lo with the lower half-wave of
            // hi leaves, in every lane, its gate value in the first result
            // and its up value in the second (gate lanes keep lo and take the
            // partner's lo; up lanes take the partner's hi and keep hi)
            const uint32_t pk = pack_bf16x2(acc[ii][j][r], acc[ii + 2][j][r]);
            const uint32_t lo = pk << 16;
            const uint32_t hi = pk & 0xFFFF0000u;
            const auto gu = __builtin_amdgcn_permlane32_swap(lo, hi, false, false);
            const float v = f(__uint_as_float(gu[0]), __uint_as_float(gu[1]));
            h[j][4 * ii + r] = v;
            amax[j] = fmaxf(amax[j], fabsf(v));
          }
        }
        // the 4 lanes of this row in the wave: rho, rho + 16, rho + 32, rho + 48
        // (each swap leaves the lane's own value and its partner's)
        const auto m16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(amax[j]),
                                                          __float_as_uint(amax[j]), false, false);
        amax[j] = fmaxf(__uint_as_float(m16[0]), __uint_as_float(m16[1]));
        const auto m32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(amax[j]),
                                                          __float_as_uint(amax[j]), false, false);
        amax[j] = fmaxf(__uint_as_float(m32[0]), __uint_as_float(m32[1]));
      }
    };
    // SiLU gets its own unrolled copy (no per-element branch); the other
    // gated activations (and SiLU with a clamp limit) share one that
    // switches on the kind
    if (p.activation == kActSilu && !(p.act_limit > 0.0f))
      activate([](float g, float u) { return apply_act(kActSilu, g, u); });
    else
      activate([&](float g, float u) { return apply_act(p.activation, g, u, p.act_limit); });
    if constexpr (A16) {
      // unquantized w2 input: h rounded once to bf16, 16 bytes per lane
#pragma unroll
      for (int j = 0; j < S::TM; ++j) {
        const int ml = ml0 + kSubStride * j;
        if (ml >= rows_here) continue;
        const int64_t row = out_row_of(ml);
        if (row < 0) continue;
        *reinterpret_cast<uint4*>(p.act_q + (row * Nh + j0 + col_off) * 2) =
            make_uint4(pack_bf16x2(h[j][0], h[j][1]), pack_bf16x2(h[j][2], h[j][3]),
                       pack_bf16x2(h[j][4], h[j][5]), pack_bf16x2(h[j][6], h[j][7]));
      }
      return;
    }
    // 128-column groups: maximum across the WN = 4 waves sharing the rows,
    // through LDS.  MX 32-column groups: one wave's columns, already reduced.
    float* red = reinterpret_cast<float*>(smem);   // [WN][BM]
    if constexpr (!MX) {
      __syncthreads();                             // every wave is done with the ring
      if (kq == 0) {
#pragma unroll
        for (int j = 0; j < S::TM; ++j) red[wn * S::BM + ml0 + kSubStride * j] = amax[j];
      }
      __syncthreads();
    }
    const int GN = Nh / (MX ? 32 : kGroup);
    const int g_out = MX ? 4 * nt + wn : nt;       // this lane's scale group
#pragma unroll
    for (int j = 0; j < S::TM; ++j) {
      const int ml = ml0 + kSubStride * j;
      if (ml >= rows_here) continue;
      const float a = MX ? amax[j]
                         : fmaxf(fmaxf(red[ml], red[S::BM + ml]),
                                 fmaxf(red[2 * S::BM + ml], red[3 * S::BM + ml]));
      const GroupScale gs = group_scale<UE8M0 || MX>(a);
      uint2 q;
      q.x = f32x4_to_e4m3x4(h[j][0] * gs.recip, h[j][1] * gs.recip, h[j][2] * gs.recip,
                            h[j][3] * gs.recip);
      q.y = f32x4_to_e4m3x4(h[j][4] * gs.recip, h[j][5] * gs.recip, h[j][6] * gs.recip,
                            h[j][7] * gs.recip);
      const int64_t row = out_row_of(ml);
      if (row < 0) continue;
      *reinterpret_cast<uint2*>(p.act_q + row * Nh + j0 + col_off) = q;
      if (kq == 0 && (MX || wn == 0)) {
        if (UE8M0 || MX) {
          uint8_t* sf = p.act_sf + row * p.act_sf_row;
          sf[g_out] = (uint8_t)gs.stored;
          // the row's trailing pad bytes are zero (128-column groups only;
          // 32-column rows have none)
          if (!MX && g_out == GN - 1)
            for (int pad = GN; pad < p.act_sf_row; ++pad) sf[pad] = 0;
        } else {
          reinterpret_cast<uint32_t*>(p.act_sf)[row * p.act_sf_row + g_out] = gs.stored;
        }
      }
    }
  } else {
    // ---- epilogue: lane owns output row m, columns n_first .. n_first+4*TN-1
    const int n_first = n0 + (NP - 1) * S::BN + wn * S::WAVE_N + kq * (4 * S::TN);
    if (nsplit > 1) {
      // split-K: this split's fp32 partial, then a ticket; the block with
      // the last ticket adds the partials in split order (its own from
      // registers: the same values it stored) and rounds once to bf16.
      // Every thread fences its partial stores (device scope: the other
      // splits may run on other XCDs) before the ticket is drawn, and the
      // summing block fences before it reads.
      const int64_t pstride = p.part_rows * (int64_t)p.Nout;
#pragma unroll
      for (int j = 0; j < S::TM; ++j) {
        const int ml = ml0 + kSubStride * j;
        if (ml >= rows_here) continue;
        const int64_t row = out_row_of(ml);
        if (row < 0) continue;
        v4f* dst = reinterpret_cast<v4f*>(p.part + split * pstride + row * p.Nout + n_first);
#pragma unroll
        for (int i = 0; i < S::TN; ++i) dst[i] = acc[i][j];
      }
      // each wave's stores complete, then one device-scope release and the
      // ticket (one L2 write-back per block rather than one per wave)
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __syncthreads();
      int* ticket = reinterpret_cast<int*>(smem);
      const int64_t item = (int64_t)tile * NT + nt;
      if (tid == 0)
        *ticket = __hip_atomic_fetch_add(p.counters + item, 1, __ATOMIC_ACQ_REL,
                                         __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
      if (*ticket != nsplit - 1) return;
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
#pragma unroll
      for (int j = 0; j < S::TM; ++j) {
        const int ml = ml0 + kSubStride * j;
        if (ml >= rows_here) continue;
        const int64_t row = out_row_of(ml);
        if (row < 0) continue;
        v4f sum[S::TN];
#pragma unroll
        for (int s2 = 0; s2 < kMaxSplit; ++s2) {
          if (s2 < nsplit) {
            v4f v[S::TN];
            if (s2 == split) {
#pragma unroll
              for (int i = 0; i < S::TN; ++i) v[i] = acc[i][j];
            } else {
              const v4f* src =
                  reinterpret_cast<const v4f*>(p.part + s2 * pstride + row * p.Nout + n_first);
#pragma unroll
              for (int i = 0; i < S::TN; ++i) v[i] = src[i];
            }
#pragma unroll
            for (int i = 0; i < S::TN; ++i) sum[i] = s2 == 0 ? v[i] : sum[i] + v[i];
          }
        }
#pragma unroll
        for (int i = 0; i < S::TN; ++i) acc[i][j] = sum[i];
      }
      if (tid == 0)
        __hip_atomic_store(p.counters + item, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    store_rows(n_first);
  }
}

// 160-row tiles: the block scheme with fp8 activations only
template <int SC>
constexpr bool kTile160 = SC == kQuantUe8m0 || SC == kQuantF32;
static_assert(Shape<160, 256, 8, 3>::PG >= kTile160MaxGroups &&
                  Shape<160, 128, 8, 3>::PG >= kTile160MaxGroups,
              "160-row tiles: reduction length limit");

template <class S, int SC, bool ACT, int NP = 1>
hipError_t launch_shape(const GemmArgs& pin, int max_tiles, hipStream_t stream) {
  // Item order inside a group: consecutive blocks on an XCD start about a
  // block time / 32 apart and an operand's k-slice stays in L2 for only a few
  // microseconds, so only a few neighbours in dispatch order share data.
  // For the tall tiles (experts of hundreds of rows, groups of a few m-tiles)
  // n-tile pairs walked m-tile-major let neighbours share the activation tile
  // as well as the weight tile: Qwen3-shaped w13 -1.5 % and 9 % fewer HBM /
  // MALL bytes.  At 128-row tiles (groups of up to 8 m-tiles) wider walks
  // measured within noise and moved 5 % more bytes, so those keep the
  // n-tile-major walk.  MOE_SN overrides.
  GemmArgs p = pin;
  {
    static const char* env = getenv("MOE_SN");
    p.sn = env != nullptr ? atoi(env) : (S::BM >= 192 ? 2 : 1);
  }
  // k-step rotation: weight rows of a multiple of 4 KB (the MX schemes keep
  // the plain order: their scale panel arrives in groups of 4 k-steps).
  // MOE_KROT = 0 | 1 overrides (read at every launch).
  constexpr bool mx = SC == kQuantMxfp8 || SC == kSchemeMxfp8W4;
  {
    const char* env = getenv("MOE_KROT");
    const bool want = env != nullptr ? env[0] == '1' : p.Kd % 4096 == 0;
    p.krot = (!mx && want && p.rot_period > 0 && p.rot_period % 256 == 0) ? 1 : 0;
  }
  // the block scheme's weight-scale panel holds S::PG k-steps
  if (!mx && p.Kd / kGroup > S::PG) return hipErrorInvalidValue;
  // every XCD's slice: whole items' splits, ceil(items / 8) * splits blocks
  // (the schedule's slicing; rounding items * splits up to 8 instead would
  // leave splits of the last items without a block)
  const int64_t blocks =
      ((int64_t)max_tiles * (p.Nout / (S::BN * NP)) + 7) / 8 * 8 * (ACT ? 1 : max(p.ksplit, 1));
  const dim3 grid((unsigned)blocks);
  if constexpr (SC == kQuantBf16) {
    // bf16 activation tiles take twice the LDS: only shapes whose ring fits
    constexpr bool fits =
        S::STAGES * (S::BM * 2 * kRowBytes + S::BN * kRowBytes) + S::NBLK * kMaxGroups * 4 <=
        160 * 1024;
    if constexpr (fits)
      grouped_gemm_kernel<S, SC, ACT><<<grid, S::THREADS, 0, stream>>>(p);
    else
      return hipErrorInvalidValue;
  } else {
    grouped_gemm_kernel<S, SC, ACT, NP><<<grid, S::THREADS, 0, stream>>>(p);
  }
  return hipGetLastError();
}

// bf16 activations take twice the activation-tile LDS: two-slot rings and
// tiles of at most 128 rows
template <bool ACT>
hipError_t launch_a16(const GemmArgs& p, int tile_m, int max_tiles, hipStream_t stream) {
  constexpr int q = kQuantBf16;
  if (ACT || p.Nout % 256 == 0) {
    switch (tile_m) {
      case 16: return launch_shape<Shape<16, 256, 4, 2>, q, ACT>(p, max_tiles, stream);
      case 32: return launch_shape<Shape<32, 256, 4, 2>, q, ACT>(p, max_tiles, stream);
      case 64: return launch_shape<Shape<64, 256, 8, 2>, q, ACT>(p, max_tiles, stream);
      case 128: return launch_shape<Shape<128, 256, 8, 2>, q, ACT>(p, max_tiles, stream);
      default: return hipErrorInvalidValue;
    }
  }
  if constexpr (!ACT) {
    switch (tile_m) {
      case 16: return launch_shape<Shape<16, 128, 4, 2>, q, false>(p, max_tiles, stream);
      case 32: return launch_shape<Shape<32, 128, 4, 2>, q, false>(p, max_tiles, stream);
      case 64: return launch_shape<Shape<64, 128, 4, 2>, q, false>(p, max_tiles, stream);
      case 128: return launch_shape<Shape<128, 128, 4, 2>, q, false>(p, max_tiles, stream);
      default: return hipErrorInvalidValue;
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace

// One scale scheme's kernels.  This file is compiled once per scheme
// (MOE_GEMM_SCHEME = the scheme's kQuant* / kScheme* value), so the schemes'
// instantiations build in parallel; launch_grouped_gemm (kernels.h) picks
// the scheme at run time.
template <int SC>
hipError_t launch_grouped_gemm_sc(const GemmArgs& p, int tile_m, int max_tiles, bool act,
                                  hipStream_t stream) {
  if (max_tiles <= 0) return hipSuccess;
  if constexpr (SC == kQuantBf16) {
    if (act && p.Nout % 256 != 0) return hipErrorInvalidValue;
    return act ? launch_a16<true>(p, tile_m, max_tiles, stream)
               : launch_a16<false>(p, tile_m, max_tiles, stream);
  } else {
    if (act) {
      // 256 weight rows = 128 gate + 128 up rows per block, any tile height
      if (p.Nout % 256 != 0) return hipErrorInvalidValue;
      switch (tile_m) {
        case 16: return launch_shape<Shape<16, 256, 4, 3>, SC, true>(p, max_tiles, stream);
        case 32: return launch_shape<Shape<32, 256, 4, 3>, SC, true>(p, max_tiles, stream);
        case 64: return launch_shape<Shape<64, 256, 8, 3>, SC, true>(p, max_tiles, stream);
        case 128: return launch_shape<Shape<128, 256, 8, 3>, SC, true>(p, max_tiles, stream);
        case 160:
          if constexpr (kTile160<SC>)
            return launch_shape<Shape<160, 256, 8, 3>, SC, true>(p, max_tiles, stream);
          return hipErrorInvalidValue;
        case 192: return launch_shape<Shape<192, 256, 8, 2>, SC, true>(p, max_tiles, stream);
        case 256: return launch_shape<Shape<256, 256, 8, 2>, SC, true>(p, max_tiles, stream);
        default: return hipErrorInvalidValue;
      }
    }
    switch (tile_m) {
      case 16: return launch_shape<Shape<16, 128, 4, 4>, SC, false>(p, max_tiles, stream);
      case 32: return launch_shape<Shape<32, 128, 4, 3>, SC, false>(p, max_tiles, stream);
      case 64: return launch_shape<Shape<64, 128, 4, 3>, SC, false>(p, max_tiles, stream);
      case 128: {
        // 256-column tiles (8 waves) halve the activation re-reads; 128-column
        // tiles run two blocks per CU, which measured faster for the MX
        // schemes (whose MFMA consumes its scales directly: less per-k-step
        // work to hide the block prologue behind) -- unless the experts above
        // 128 rows run in their own 256-row tile list beside this one: then
        // 256 columns won for MX too (DSv3-shaped prefill w2, both lists
        // concurrent: MXFP8 1.14 -> 1.00 ms, MXFP4 0.81 -> 0.76 ms).
        // MOE_GEMM_WIDE=0 / 1 forces one or the other.
        static const char* env = getenv("MOE_GEMM_WIDE");
        constexpr bool mx = SC == kQuantMxfp8 || SC == kSchemeMxfp8W4;
        const bool wide = env != nullptr ? env[0] != '0' : (!mx || p.wide == 1);
        if constexpr (SC == kQuantUe8m0 || SC == kQuantF32) {
          // two n-tiles per block where the caller asks for it (no split)
          if (p.pair == 1 && p.Nout % 512 == 0 && p.ksplit <= 1)
            return launch_shape<Shape<128, 256, 8, 3>, SC, false, 2>(p, max_tiles, stream);
        }
        if (wide && p.Nout % 256 == 0)
          return launch_shape<Shape<128, 256, 8, 3>, SC, false>(p, max_tiles, stream);
        return launch_shape<Shape<128, 128, 4, 2>, SC, false>(p, max_tiles, stream);
      }
      // Experts of about 100-160 rows (few experts, a split w2): one tile
      // each, with the 3-slot ring that a 192-row tile cannot fit (block
      // scheme only: the MX weight-scale panel does not fit beside it)
      case 160:
        if constexpr (kTile160<SC>) {
          if (p.Nout % 256 == 0)
            return launch_shape<Shape<160, 256, 8, 3>, SC, false>(p, max_tiles, stream);
          return launch_shape<Shape<160, 128, 8, 3>, SC, false>(p, max_tiles, stream);
        }
        return hipErrorInvalidValue;
      // Experts with hundreds of rows: 1.5x / 2x fewer weight re-reads than
      // 128-row tiles, at the price of a two-slot ring (LDS) and of 128
      // accumulator VGPRs per lane at 256 rows.
      case 192:
        if (p.Nout % 256 == 0)
          return launch_shape<Shape<192, 256, 8, 2>, SC, false>(p, max_tiles, stream);
        return launch_shape<Shape<192, 128, 8, 2>, SC, false>(p, max_tiles, stream);
      case 256:
        if (p.Nout % 256 == 0)
          return launch_shape<Shape<256, 256, 8, 2>, SC, false>(p, max_tiles, stream);
        return launch_shape<Shape<256, 128, 8, 2>, SC, false>(p, max_tiles, stream);
      default: return hipErrorInvalidValue;
    }
  }
}

#ifndef MOE_GEMM_SCHEME
#error "compile this file once per scale scheme with -DMOE_GEMM_SCHEME=<scheme>"
#endif
template hipError_t launch_grouped_gemm_sc<MOE_GEMM_SCHEME>(const GemmArgs&, int, int, bool,
                                                            hipStream_t);

}  // namespace moe
