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
//  * Work unit = (expert, 128-column weight tile, BM-row activation tile).
//    The tile list comes from the routing step, heaviest experts first;
//    grid.x runs over weight tiles, so the tiles of one expert that share a
//    weight tile land on the same XCD (grid.x is a multiple of 8 for every
//    supported width) and re-read it from that XCD's L2.
//  * Rows beyond an expert's count are never loaded (zero-filled in LDS) or
//    stored; the garbage rows of a batched-masked slab never reach an output.
//  * LDS: A tile [BM][128] and B tile [128][128] fp8, double buffered, 16-byte
//    chunks XOR-swizzled per row so the MFMA fragment reads spread across
//    banks.  Global loads for k-step kb+1 are in flight while kb computes.
#include "device_common.h"
#include "kernels.h"

namespace moe {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kBN = 128;       // weight rows (output columns) per tile
constexpr int kRowBytes = 128; // one k-step of a row: 128 fp8 values

template <int BM>
struct Shape {
  static constexpr int WM = BM >= 64 ? 2 : 1;        // waves along activation rows
  static constexpr int WN = 4 / WM;                  // waves along weight rows
  static constexpr int WAVE_N = kBN / WN;            // 64 or 32
  static constexpr int WAVE_M = BM / WM;             // 64, 32, 32, 16
  static constexpr int TN = WAVE_N / 16;             // 16-row MFMA sub-tiles along N
  static constexpr int TM = WAVE_M / 16;             // sub-tiles along M
  static constexpr int LOG_4TN = TN == 4 ? 4 : (TN == 2 ? 3 : 2);
  static constexpr int A_CHUNKS = BM * 8;            // 16-byte chunks per k-step
  static constexpr int A_ITERS = A_CHUNKS >= 256 ? A_CHUNKS / 256 : 1;
  static constexpr int B_ITERS = kBN * 8 / 256;
  static constexpr int TILE_BYTES = (BM + kBN) * kRowBytes;
};

// 16-byte chunk c of row r lives at chunk position c ^ key(r).
__device__ __forceinline__ int key_a(int r) { return r & 7; }
template <int LOG_4TN>
__device__ __forceinline__ int key_b(int r) { return (r & 3) | (((r >> LOG_4TN) & 1) << 2); }

template <int BM, bool UE8M0>
__global__ __launch_bounds__(256, 2) void grouped_gemm_kernel(const GemmArgs p) {
  using S = Shape<BM>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2][S::TILE_BYTES];

  const int tile = blockIdx.y;
  if (tile >= p.tile_list[0]) return;
  const int e = p.tile_list[1 + 2 * tile];
  const int m0 = p.tile_list[2 + 2 * tile];
  const int n0 = blockIdx.x * kBN;
  int cnt = p.counts[e];
  if (p.offsets == nullptr) cnt = min(cnt, p.max_tokens);
  const int rows_here = min(BM, cnt - m0);
  const int64_t base = p.offsets != nullptr ? (int64_t)p.offsets[e] : (int64_t)e * p.max_tokens;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wn = wave % S::WN;
  const int wm = wave / S::WN;
  const int G = p.Kd / kGroup;

  auto a_row_of = [&](int m) -> int64_t {
    const int64_t r = base + m0 + m;
    return p.row_src != nullptr ? (int64_t)p.row_src[r] : r;
  };

  // ---- global -> register -> LDS copy plan -----------------------------
  const uint8_t* a_src[S::A_ITERS];
  int a_lds[S::A_ITERS];
  bool a_on[S::A_ITERS];
#pragma unroll
  for (int i = 0; i < S::A_ITERS; ++i) {
    const int chunk = tid + i * 256;
    const int r = chunk >> 3, c = chunk & 7;
    a_on[i] = chunk < S::A_CHUNKS;
    const bool live = a_on[i] && r < rows_here;
    a_src[i] = live ? p.a + a_row_of(r) * p.Kd + c * 16 : nullptr;
    a_lds[i] = r * kRowBytes + ((c ^ key_a(r)) << 4);
  }
  const uint8_t* b_src[S::B_ITERS];
  int b_lds[S::B_ITERS];
  const uint8_t* w_e = p.w + ((int64_t)e * p.Nout + n0) * p.Kd;
#pragma unroll
  for (int i = 0; i < S::B_ITERS; ++i) {
    const int chunk = tid + i * 256;
    const int r = chunk >> 3, c = chunk & 7;
    b_src[i] = w_e + (int64_t)r * p.Kd + c * 16;
    b_lds[i] = BM * kRowBytes + r * kRowBytes + ((c ^ key_b<S::LOG_4TN>(r)) << 4);
  }
  const float* sw_row = p.w_sf + ((int64_t)e * (p.Nout / kGroup) + n0 / kGroup) * G;

  // ---- per-lane MFMA fragment addresses --------------------------------
  const int rho = lane & 15;
  const int kq = lane >> 4;
  int wf_off[S::TN];
#pragma unroll
  for (int i = 0; i < S::TN; ++i) {
    const int nl = wn * S::WAVE_N + (rho >> 2) * (4 * S::TN) + i * 4 + (rho & 3);
    wf_off[i] = BM * kRowBytes + nl * kRowBytes;
  }
  const int kb_sw = key_b<S::LOG_4TN>(wn * S::WAVE_N + (rho >> 2) * (4 * S::TN) + (rho & 3));
  int af_off[S::TM];
  int af_key[S::TM];
  // activation scale source per sub-tile column (this lane's output row)
  const uint8_t* sa_u8[S::TM];
  const float* sa_f32[S::TM];
  bool m_live[S::TM];
#pragma unroll
  for (int j = 0; j < S::TM; ++j) {
    const int ml = wm * S::WAVE_M + j * 16 + rho;
    af_off[j] = ml * kRowBytes;
    af_key[j] = key_a(ml);
    m_live[j] = ml < rows_here;
    const int64_t ar = m_live[j] ? a_row_of(ml) : 0;
    sa_u8[j] = (const uint8_t*)p.a_sf + ar * p.a_sf_stride;
    sa_f32[j] = (const float*)p.a_sf + ar * p.a_sf_stride;
  }

  uint4 a_reg[S::A_ITERS];
  uint4 b_reg[S::B_ITERS];
  float sa_next[S::TM];
  float sw_next;

  auto load_global = [&](int kb) {
#pragma unroll
    for (int i = 0; i < S::A_ITERS; ++i)
      a_reg[i] = a_src[i] != nullptr
                     ? *reinterpret_cast<const uint4*>(a_src[i] + kb * kRowBytes)
                     : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < S::B_ITERS; ++i)
      b_reg[i] = *reinterpret_cast<const uint4*>(b_src[i] + kb * kRowBytes);
#pragma unroll
    for (int j = 0; j < S::TM; ++j) {
      float s = 0.0f;
      if (m_live[j]) s = UE8M0 ? __uint_as_float((uint32_t)sa_u8[j][kb] << 23) : sa_f32[j][kb];
      sa_next[j] = s;
    }
    sw_next = sw_row[kb];
  };
  auto store_lds = [&](int buf) {
#pragma unroll
    for (int i = 0; i < S::A_ITERS; ++i)
      if (a_on[i]) *reinterpret_cast<uint4*>(&smem[buf][a_lds[i]]) = a_reg[i];
#pragma unroll
    for (int i = 0; i < S::B_ITERS; ++i)
      *reinterpret_cast<uint4*>(&smem[buf][b_lds[i]]) = b_reg[i];
  };

  v4f acc[S::TN][S::TM];
#pragma unroll
  for (int i = 0; i < S::TN; ++i)
#pragma unroll
    for (int j = 0; j < S::TM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  load_global(0);
  store_lds(0);
  float sa_cur[S::TM];
  float sw_cur;
#pragma unroll
  for (int j = 0; j < S::TM; ++j) sa_cur[j] = sa_next[j];
  sw_cur = sw_next;
  __syncthreads();

  for (int kb = 0; kb < G; ++kb) {
    const int buf = kb & 1;
    if (kb + 1 < G) load_global(kb + 1);

    const uint8_t* sb = smem[buf];
    v8i wf[S::TN];
    v8i af[S::TM];
    const int c0 = 2 * kq, c1 = 2 * kq + 1;
#pragma unroll
    for (int i = 0; i < S::TN; ++i) {
      const uint4 lo = *reinterpret_cast<const uint4*>(sb + wf_off[i] + ((c0 ^ kb_sw) << 4));
      const uint4 hi = *reinterpret_cast<const uint4*>(sb + wf_off[i] + ((c1 ^ kb_sw) << 4));
      wf[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z,
                  (int)hi.w};
    }
#pragma unroll
    for (int j = 0; j < S::TM; ++j) {
      const uint4 lo = *reinterpret_cast<const uint4*>(sb + af_off[j] + ((c0 ^ af_key[j]) << 4));
      const uint4 hi = *reinterpret_cast<const uint4*>(sb + af_off[j] + ((c1 ^ af_key[j]) << 4));
      af[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z,
                  (int)hi.w};
    }
    float f[S::TM];
#pragma unroll
    for (int j = 0; j < S::TM; ++j) f[j] = sa_cur[j] * sw_cur;
#pragma unroll
    for (int i = 0; i < S::TN; ++i) {
#pragma unroll
      for (int j = 0; j < S::TM; ++j) {
        const v4f z = {0.f, 0.f, 0.f, 0.f};
        const v4f part =
            __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf[i], af[j], z, 0, 0, 0, 0, 0, 0);
        acc[i][j][0] = fmaf(part[0], f[j], acc[i][j][0]);
        acc[i][j][1] = fmaf(part[1], f[j], acc[i][j][1]);
        acc[i][j][2] = fmaf(part[2], f[j], acc[i][j][2]);
        acc[i][j][3] = fmaf(part[3], f[j], acc[i][j][3]);
      }
    }
    if (kb + 1 < G) {
      store_lds(buf ^ 1);
#pragma unroll
      for (int j = 0; j < S::TM; ++j) sa_cur[j] = sa_next[j];
      sw_cur = sw_next;
    }
    __syncthreads();
  }

  // ---- epilogue: lane owns output row m, columns n_first .. n_first+4*TN-1
  const int n_first = n0 + wn * S::WAVE_N + kq * (4 * S::TN);
#pragma unroll
  for (int j = 0; j < S::TM; ++j) {
    if (!m_live[j]) continue;
    const int ml = wm * S::WAVE_M + j * 16 + rho;
    uint16_t* dst = p.out + (base + m0 + ml) * (int64_t)p.Nout + n_first;
    uint32_t packed[2 * S::TN];
#pragma unroll
    for (int i = 0; i < S::TN; ++i) {
      packed[2 * i] = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
      packed[2 * i + 1] = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
    }
#pragma unroll
    for (int v = 0; v < S::TN / 2; ++v)
      reinterpret_cast<uint4*>(dst)[v] =
          make_uint4(packed[4 * v], packed[4 * v + 1], packed[4 * v + 2], packed[4 * v + 3]);
    if (S::TN == 1) reinterpret_cast<uint2*>(dst)[0] = make_uint2(packed[0], packed[1]);
  }
}

template <int BM>
hipError_t launch_bm(const GemmArgs& p, int max_tiles, int quant, hipStream_t stream) {
  const dim3 grid(p.Nout / kBN, max_tiles);
  if (quant == kQuantUe8m0)
    grouped_gemm_kernel<BM, true><<<grid, 256, 0, stream>>>(p);
  else
    grouped_gemm_kernel<BM, false><<<grid, 256, 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_grouped_gemm(const GemmArgs& p, int tile_m, int max_tiles, int quant,
                               hipStream_t stream) {
  if (max_tiles <= 0) return hipSuccess;
  switch (tile_m) {
    case 16: return launch_bm<16>(p, max_tiles, quant, stream);
    case 32: return launch_bm<32>(p, max_tiles, quant, stream);
    case 64: return launch_bm<64>(p, max_tiles, quant, stream);
    case 128: return launch_bm<128>(p, max_tiles, quant, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
