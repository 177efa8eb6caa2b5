// bf16 GEMMs of the MoE branch on the gfx950 core (gemm_core.h): the dense
// projections, the shared-expert SwiGLU, and the routed experts' grouped
// SwiGLU and down-projection over device-built tile lists (rows gathered
// from the pools or read from an expert-ordered buffer, outputs scattered
// back or written in order).  fp32 accumulation; bf16 outputs.
//
// Tile shapes: 256 x 256 with 8 wavefronts (64 x 128 each) for the dense
// contractions, whose M (tokens) and N are large; 192 x 256 with 8
// wavefronts (96 x 64 each) for the routed experts, whose ~341 rows per
// expert fit two 192-row tiles with little padding, and the 256 x 256 tile
// for them too when experts hold thousands of rows each.  In an expert's
// last tile each wavefront computes only the 16-row blocks of its band that
// hold rows.  The experts' weight tiles stream from HBM once each, so they
// get a third LDS stage.
//
// Workgroups are dealt round-robin to the 8 XCDs, each with its own L2, so
// every kernel maps its linear block index to a tile such that one XCD gets
// a contiguous range of tiles: a group of M panels x all N tiles for the
// dense GEMMs, an eighth of the expert-major tile list for the routed
// experts.  Tiles that share an operand panel then run at the same time on
// the same L2.
#include "common.h"
#include "gemm_core.h"
#include "kernels.h"

namespace moe {
namespace {

using core::Acc;
using core::acc_col;
using core::acc_row;
using core::load_col;
using core::load_row;
using core::mainloop;
using core::RowSrc;
using core::uniform_ptr;
using core::with_row_blocks;

using DenseTile = core::Tile<256, 256, 4, 2, 64, 2>;
// a third B stage, all 160 KB of LDS: the shared SwiGLU GEMM and single-segment dense GEMMs
using DenseTile3B = core::Tile<256, 256, 4, 2, 64, 2, 3>;
using ExpertTile = core::Tile<192, 256, 2, 4, 64, 2, 3>;
// experts with thousands of rows each: the dense GEMMs' 256-row tile (more
// MFMA work per staged operand byte; an expert's padding is then a few per cent)
using ExpertTileTall = core::Tile<256, 256, 4, 2, 64, 2, 3>;
static_assert(ExpertTileTall::BN == ExpertTile::BN, "both expert tiles share the N tiling");
// fp32 output (the router logits): 4 wavefronts of 64 x 48; E = 384 columns
// are four N tiles, so the Marin-shaped router GEMM is 512 tiles, two per CU
using RouterTile = core::Tile<128, 96, 2, 2, 64, 2>;

constexpr int kGroupM = 4;  // M panels per group of the dense tile order (4: measured best of 2, 4, 6, 8, 16)
constexpr int kStagePad = 16;

template <class TL>
constexpr int lds_bytes() {
  return TL::MAIN_LDS > TL::BM * (TL::BN * 2 + kStagePad) ? TL::MAIN_LDS : TL::BM * (TL::BN * 2 + kStagePad);
}

// Linear block index -> index in a sequence in which each XCD owns a
// contiguous range (grids are padded to a multiple of 8 blocks).
__device__ __forceinline__ int xcd_order(int bid, int nblocks) { return (bid & 7) * (nblocks >> 3) + (bid >> 3); }

// Dense tile order: groups of kGroupM M panels, N tiles, M fastest.
__device__ __forceinline__ void dense_tile(int t, int tiles_m, int tiles_n, int& mt, int& nt) {
  const int per_group = kGroupM * tiles_n;
  const int g = t / per_group;
  const int first = g * kGroupM;
  const int gsz = min(tiles_m - first, kGroupM);
  const int r = t - g * per_group;
  mt = first + r % gsz;
  nt = r / gsz;
}

// Stage the accumulator tile as bf16 rows of `ld` bytes.
template <class TL>
__device__ __forceinline__ void stage_bf16(const Acc<TL>& acc, char* lds, int ld) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / TL::WGN, wn = wave % TL::WGN;
#pragma unroll
  for (int mi = 0; mi < TL::MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < TL::NI; ++ni)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = acc_row<TL>(wm, mi, lane, r), col = acc_col<TL>(wn, ni, lane);
        *reinterpret_cast<uint16_t*>(lds + row * ld + col * 2) = f32_to_bf16(acc.v[mi][ni][r]);
      }
}

// Stage silu(gate) * up as bf16: in every wavefront's column range, 16-wide
// blocks alternate gate (even) and up (odd) for the same 16 features, so
// the tile holds BN / 2 features.
template <class TL>
__device__ __forceinline__ void stage_swiglu_bf16(const Acc<TL>& acc, char* lds, int ld) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / TL::WGN, wn = wave % TL::WGN;
#pragma unroll
  for (int mi = 0; mi < TL::MI; ++mi)
#pragma unroll
    for (int q = 0; q < TL::NI / 2; ++q)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = acc_row<TL>(wm, mi, lane, r);
        const int col = wn * (TL::WN / 2) + q * 16 + (lane & 15);
        const float h = silu(acc.v[mi][2 * q][r]) * acc.v[mi][2 * q + 1][r];
        *reinterpret_cast<uint16_t*>(lds + row * ld + col * 2) = f32_to_bf16(h);
      }
}

// B-tile row r of a SwiGLU tile -> (half, feature offset inside the tile):
// half 0 = gate weight row, 1 = up weight row.
template <class TL>
__device__ __forceinline__ int swiglu_feature(int r, int& half) {
  const int wn = r / TL::WN, rr = r - wn * TL::WN;
  half = (rr >> 4) & 1;
  return wn * (TL::WN / 2) + (rr >> 5) * 16 + (rr & 15);
}

// Write staged rows out in 16-byte chunks: row r of the tile goes to
// row_ptr(r) (already at the tile's first column).  kStream: nontemporal
// stores, for outputs the next kernel streams once (no reuse from cache).
template <class TL, bool kStream = false, class RowPtr>
__device__ __forceinline__ void copy_rows(const char* lds, int ld, int chunks_per_row, int valid_rows,
                                          int valid_chunks, RowPtr row_ptr) {
  const int total = TL::BM * chunks_per_row;
  for (int q = threadIdx.x; q < total; q += TL::THREADS) {
    const int r = q / chunks_per_row;
    const int c = q - r * chunks_per_row;
    if (r < valid_rows && c < valid_chunks) {
      if constexpr (kStream)
        st16_stream(row_ptr(r) + c * 16, ld16(lds + r * ld + c * 16));
      else
        st16(row_ptr(r) + c * 16, ld16(lds + r * ld + c * 16));
    }
  }
}

// ------------------------------------------------------------------ dense
// The plain schedule: with the segment loop and the full-width epilogue the
// mid-tile barrier schedule does not fit this kernel's registers.
__global__ __launch_bounds__(DenseTile::THREADS) void dense_bf16_kernel(GemmDense g, int tiles_m, int tiles_n) {
  using TL = DenseTile;
  __shared__ __attribute__((aligned(1024))) char lds[lds_bytes<TL>()];
  const int t = xcd_order(blockIdx.x, gridDim.x);
  if (t >= tiles_m * tiles_n) return;
  int mt, nt;
  dense_tile(t, tiles_m, tiles_n, mt, nt);
  const int m0 = mt * TL::BM, n0 = nt * TL::BN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  Acc<TL> acc;
  acc.zero();
  for (int s = 0; s < g.nseg; ++s) {
    const GemmSeg& sg = g.seg[s];
    RowSrc<TL::A_INS> a_src;
    RowSrc<TL::B_INS> b_src;
    const char* A = uniform_ptr(static_cast<const char*>(sg.A));
    const char* B = uniform_ptr(static_cast<const char*>(sg.B));
#pragma unroll
    for (int i = 0; i < TL::A_INS; ++i) {
      const int m = min(m0 + load_row<TL>(i, wave, lane), g.M - 1);
      a_src.base[i] = A;
      a_src.off[i] = (uint32_t)(m * sg.lda * 2) + load_col<TL>(lane);
    }
#pragma unroll
    for (int i = 0; i < TL::B_INS; ++i) {
      const int n = min(n0 + load_row<TL>(i, wave, lane), g.N - 1);
      b_src.base[i] = B;
      b_src.off[i] = (uint32_t)(n * sg.ldb * 2) + load_col<TL>(lane);
    }
    mainloop<TL, false>(a_src, b_src, sg.K / TL::BK, lds, acc);
  }
  constexpr int ld = TL::BN * 2 + kStagePad;
  stage_bf16<TL>(acc, lds, ld);
  __syncthreads();
  constexpr int cpr = TL::BN * 2 / 16;
  char* C = static_cast<char*>(g.C);
  copy_rows<TL>(lds, ld, cpr, min(TL::BM, g.M - m0), min(cpr, (g.N - n0) * 2 / 16),
                [&](int r) { return C + ((int64_t)(m0 + r) * g.ldc + n0) * 2; });
}

// K ranges whose A parts are consecutive columns of one row-major buffer
// and whose B parts are separate arrays of one row pitch (the output
// projection over [y_lat | shared hidden rows]): A is one operand, B's K
// tile j comes from the range holding it.
struct SegK {
  static constexpr bool kLinear = false;
  const char* p[kMaxSegs];
  int first[kMaxSegs];  // first K tile of each range
  int n;
  __device__ __forceinline__ const char* operator()(const char*, int j, int64_t kstep) const {
    const char* q = p[0];
    int f = 0;
#pragma unroll
    for (int s = 1; s < kMaxSegs; ++s)
      if (s < n && j >= first[s]) {
        q = p[s];
        f = first[s];
      }
    return q + (int64_t)(j - f) * kstep;
  }
};

// One K range (the latent projection), or K ranges joined as SegK
// describes (Seg = true: ktiles K tiles over all of them; the one-range
// kernel reads its K from the segment): the mid-tile barrier schedule with
// a third B stage.
template <bool Seg>
__device__ __forceinline__ void dense1_body(const GemmDense& g, const SegK& bk, int ktiles, int tiles_m,
                                            int tiles_n) {
  using TL = DenseTile3B;
  __shared__ __attribute__((aligned(1024))) char lds[lds_bytes<TL>()];
  const int t = xcd_order(blockIdx.x, gridDim.x);
  if (t >= tiles_m * tiles_n) return;
  int mt, nt;
  dense_tile(t, tiles_m, tiles_n, mt, nt);
  const int m0 = mt * TL::BM, n0 = nt * TL::BN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const GemmSeg& sg = g.seg[0];
  RowSrc<TL::A_INS> a_src;
  RowSrc<TL::B_INS> b_src;
  const char* A = uniform_ptr(static_cast<const char*>(sg.A));
  const char* B = uniform_ptr(static_cast<const char*>(sg.B));
#pragma unroll
  for (int i = 0; i < TL::A_INS; ++i) {
    const int m = min(m0 + load_row<TL>(i, wave, lane), g.M - 1);
    a_src.base[i] = A;
    a_src.off[i] = (uint32_t)(m * sg.lda * 2) + load_col<TL>(lane);
  }
#pragma unroll
  for (int i = 0; i < TL::B_INS; ++i) {
    const int n = min(n0 + load_row<TL>(i, wave, lane), g.N - 1);
    b_src.base[i] = B;
    b_src.off[i] = (uint32_t)(n * sg.ldb * 2) + load_col<TL>(lane);
  }
  Acc<TL> acc;
  acc.zero();
  if constexpr (Seg)
    mainloop<TL, true, false, false, SegK>(a_src, b_src, ktiles, lds, acc, TL::RB, TL::RB, bk);
  else
    mainloop<TL>(a_src, b_src, sg.K / TL::BK, lds, acc);
  constexpr int ld = TL::BN * 2 + kStagePad;
  stage_bf16<TL>(acc, lds, ld);
  __syncthreads();
  constexpr int cpr = TL::BN * 2 / 16;
  char* C = static_cast<char*>(g.C);
  copy_rows<TL>(lds, ld, cpr, min(TL::BM, g.M - m0), min(cpr, (g.N - n0) * 2 / 16),
                [&](int r) { return C + ((int64_t)(m0 + r) * g.ldc + n0) * 2; });
}

__global__ __launch_bounds__(DenseTile3B::THREADS) void dense1_bf16_kernel(GemmDense g, int tiles_m, int tiles_n) {
  dense1_body<false>(g, SegK{}, 0, tiles_m, tiles_n);
}

__global__ __launch_bounds__(DenseTile3B::THREADS) void densecat_bf16_kernel(GemmDense g, SegK bk, int ktiles,
                                                                           int tiles_m, int tiles_n) {
  dense1_body<true>(g, bk, ktiles, tiles_m, tiles_n);
}

// bf16 operands, fp32 output, one K range (the router logits).
__global__ __launch_bounds__(RouterTile::THREADS) void dense_f32out_kernel(GemmDense g, int tiles_m, int tiles_n) {
  using TL = RouterTile;
  constexpr int ld = TL::BN * 4 + kStagePad;
  constexpr int kLds = TL::MAIN_LDS > TL::BM * ld ? TL::MAIN_LDS : TL::BM * ld;
  __shared__ __attribute__((aligned(1024))) char lds[kLds];
  const int t = xcd_order(blockIdx.x, gridDim.x);
  if (t >= tiles_m * tiles_n) return;
  int mt, nt;
  dense_tile(t, tiles_m, tiles_n, mt, nt);
  const int m0 = mt * TL::BM, n0 = nt * TL::BN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const GemmSeg& sg = g.seg[0];
  RowSrc<TL::A_INS> a_src;
  RowSrc<TL::B_INS> b_src;
  const char* A = uniform_ptr(static_cast<const char*>(sg.A));
  const char* B = uniform_ptr(static_cast<const char*>(sg.B));
#pragma unroll
  for (int i = 0; i < TL::A_INS; ++i) {
    const int m = min(m0 + load_row<TL>(i, wave, lane), g.M - 1);
    a_src.base[i] = A;
    a_src.off[i] = (uint32_t)(m * sg.lda * 2) + load_col<TL>(lane);
  }
#pragma unroll
  for (int i = 0; i < TL::B_INS; ++i) {
    const int n = min(n0 + load_row<TL>(i, wave, lane), g.N - 1);
    b_src.base[i] = B;
    b_src.off[i] = (uint32_t)(n * sg.ldb * 2) + load_col<TL>(lane);
  }
  Acc<TL> acc;
  acc.zero();
  mainloop<TL>(a_src, b_src, sg.K / TL::BK, lds, acc);
  const int wm = wave / TL::WGN, wn = wave % TL::WGN;
#pragma unroll
  for (int mi = 0; mi < TL::MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < TL::NI; ++ni)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = acc_row<TL>(wm, mi, lane, r), col = acc_col<TL>(wn, ni, lane);
        *reinterpret_cast<float*>(lds + row * ld + col * 4) = acc.v[mi][ni][r];
      }
  __syncthreads();
  constexpr int cpr = TL::BN * 4 / 16;
  char* C = static_cast<char*>(g.C);
  copy_rows<TL>(lds, ld, cpr, min(TL::BM, g.M - m0), min(cpr, (g.N - n0) * 4 / 16),
                [&](int r) { return C + ((int64_t)(m0 + r) * g.ldc + n0) * 4; });
}

// ------------------------------------------------------------------ SwiGLU
struct SwigluBf16 {
  // A: row m at A + m * lda_bytes
  const char* A;
  int64_t lda_bytes;
  // weights [G][F][K]
  const char* Wg;
  const char* Wu;
  int G, F, K, M;
  int tiles_m, tiles_n;  // per group
  // output
  char* C;
  int64_t ldc_bytes;
};

template <class TL>
__global__ __launch_bounds__(TL::THREADS) void swiglu_bf16_kernel(SwigluBf16 p) {
  __shared__ __attribute__((aligned(1024))) char lds[lds_bytes<TL>()];
  const int t = xcd_order(blockIdx.x, gridDim.x);
  const int per_g = p.tiles_m * p.tiles_n;
  const int g = t / per_g;
  if (g >= p.G) return;
  int mt, nt;
  dense_tile(t - g * per_g, p.tiles_m, p.tiles_n, mt, nt);
  const int rows = p.M;
  const int m0 = mt * TL::BM;
  const int f0 = nt * (TL::BN / 2);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  RowSrc<TL::A_INS> a_src;
  RowSrc<TL::B_INS> b_src;
  const char* A = uniform_ptr(p.A);
#pragma unroll
  for (int i = 0; i < TL::A_INS; ++i) {
    const int m = min(m0 + load_row<TL>(i, wave, lane), rows - 1);
    a_src.base[i] = A;
    a_src.off[i] = (uint32_t)(m * p.lda_bytes) + load_col<TL>(lane);
  }
#pragma unroll
  for (int i = 0; i < TL::B_INS; ++i) {
    int half;  // uniform per instruction: its 8 rows lie in one 16-row block
    const int f = min(f0 + swiglu_feature<TL>(load_row<TL>(i, wave, lane), half), p.F - 1);
    b_src.base[i] = uniform_ptr((half ? p.Wu : p.Wg) + (int64_t)g * p.F * p.K * 2);
    b_src.off[i] = (uint32_t)(f * p.K * 2) + load_col<TL>(lane);
  }
  Acc<TL> acc;
  acc.zero();
  mainloop<TL>(a_src, b_src, p.K / TL::BK, lds, acc);
  constexpr int ld = TL::BN + kStagePad;  // BN / 2 features of bf16
  stage_swiglu_bf16<TL>(acc, lds, ld);
  __syncthreads();
  constexpr int cpr = TL::BN / 16;
  char* C = p.C;
  copy_rows<TL>(lds, ld, cpr, min(TL::BM, rows - m0), min(cpr, (p.F - f0) * 2 / 16), [&](int r) {
    return C + (int64_t)(m0 + r) * p.ldc_bytes + ((int64_t)g * p.F + f0) * 2;
  });
}

// ------------------------------------------------------------------ ragged
// Dropless grouped GEMMs: list entry t = (expert e, n tile, m tile); expert
// e's rows are rows [offsets[e], offsets[e+1]) of A and of C.  XCD x runs an
// eighth of the list, contiguous, so an expert's tiles share one L2.
// kMode: 0 down-projection, 1 SwiGLU (gate and up rows interleaved, h out),
// 2 the backward's recompute of the gate/up pre-activations with the SwiGLU
// backward in the epilogue (da, db, h out).
template <class TL, int kMode>
__global__ __launch_bounds__(TL::THREADS) void ragged_gemm_kernel(RaggedGemm p) {
  constexpr bool kSwiglu = kMode >= 1;
  __shared__ __attribute__((aligned(1024))) char lds[lds_bytes<TL>()];
  // the list's length is known only on the device: deal ceil(n / 8)
  // consecutive entries to each XCD (the grid covers the longest list)
  const int n = *p.ntiles;
  const int per_xcd = (n + 7) >> 3;
  const int local = blockIdx.x >> 3;
  const int t = (blockIdx.x & 7) * per_xcd + local;
  if (local >= per_xcd || t >= n) return;
  const int e = p.list[3 * t], nt = p.list[3 * t + 1], mt = p.list[3 * t + 2];
  const int row0 = p.offsets[e];
  const int rows = p.offsets[e + 1] - row0;
  const int m0 = mt * TL::BM;
  if (m0 >= rows) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  RowSrc<TL::A_INS> a_src;
  RowSrc<TL::B_INS> b_src;
  // A: gathered pool rows (offsets from the pools' base) or the expert's
  // contiguous range
  const char* A = uniform_ptr(p.a_index ? p.A : p.A + (int64_t)row0 * p.a_row_bytes);
#pragma unroll
  for (int i = 0; i < TL::A_INS; ++i) {
    const int m = min(m0 + load_row<TL>(i, wave, lane), rows - 1);
    a_src.base[i] = A;
    if (p.a_index) {
      const int fi = p.a_index[row0 + m];
      const int blk = fi / p.a_block_rows;
      const int slot = fi - blk * p.a_block_rows;
      a_src.off[i] = (uint32_t)(blk * p.a_block_bytes + slot * p.a_row_bytes) + load_col<TL>(lane);
    } else {
      a_src.off[i] = (uint32_t)(m * p.a_row_bytes) + load_col<TL>(lane);
    }
  }
  const int c0 = kSwiglu ? nt * (TL::BN / 2) : nt * TL::BN;
#pragma unroll
  for (int i = 0; i < TL::B_INS; ++i) {
    const int r = load_row<TL>(i, wave, lane);
    if (kSwiglu) {
      int half;  // uniform per instruction: its 8 rows lie in one 16-row block
      const int f = min(c0 + swiglu_feature<TL>(r, half), p.F - 1);
      b_src.base[i] = uniform_ptr((half ? p.W1 : p.W0) + (int64_t)e * p.F * p.K * 2);
      b_src.off[i] = (uint32_t)(f * p.K * 2) + load_col<TL>(lane);
    } else {
      const int n = min(c0 + r, p.N - 1);
      b_src.base[i] = uniform_ptr(p.W0 + (int64_t)e * p.N * p.K * 2);
      b_src.off[i] = (uint32_t)(n * p.K * 2) + load_col<TL>(lane);
    }
  }
  // the backward's dh tile: its loads go out before the K loop (into
  // registers, landing in LDS after it), so their latency is not paid after
  // the tile's last MFMA; zeros outside the expert's rows and features
  constexpr int kDhChunks = kMode == 2 ? TL::BM * (TL::BN / 2) * 2 / 16 / TL::THREADS : 1;
  uint4 dh_reg[kDhChunks];
  if constexpr (kMode == 2) {
    constexpr int cpr = (TL::BN / 2) * 2 / 16;
    const int vr = min(TL::BM, rows - m0), vc = min(cpr, (p.F - c0) * 2 / 16);
    const char* DH = p.dH + (int64_t)(row0 + m0) * p.dh_row_bytes + (int64_t)c0 * 2;
#pragma unroll
    for (int i = 0; i < kDhChunks; ++i) {
      const int q = threadIdx.x + i * TL::THREADS;
      const int r = q / cpr, c = q - r * cpr;
      // clamped address, result selected: no branch between the loads
      const uint4 v = ld16(DH + (int64_t)min(r, vr - 1) * p.dh_row_bytes + min(c, vc - 1) * 16);
      dh_reg[i] = ((r < vr) & (c < vc)) ? v : make_uint4(0, 0, 0, 0);
    }
  }
  // the output row of each 16-byte chunk this thread stores (modes 0, 1),
  // read at the tile's start with every load in flight together, so the
  // store loop holds no load (a load there makes each store wait for the
  // previous one: stores count in the same vector memory counter)
  constexpr int kOutCpr = (kSwiglu ? TL::BN / 2 : TL::BN) * 2 / 16;
  constexpr int kOutIters = kMode == 2 ? 1 : TL::BM * kOutCpr / TL::THREADS;
  static_assert(kMode == 2 || TL::BM * kOutCpr % TL::THREADS == 0, "whole chunks per thread");
  int32_t out_row[kOutIters];
  if constexpr (kMode != 2) {
    const int vr = min(TL::BM, rows - m0);
    if (p.c_index) {
#pragma unroll
      for (int i = 0; i < kOutIters; ++i) {
        const int r = (int)(threadIdx.x + i * TL::THREADS) / kOutCpr;
        out_row[i] = p.c_index[row0 + m0 + max(min(r, vr - 1), 0)];
      }
    } else {
#pragma unroll
      for (int i = 0; i < kOutIters; ++i) out_row[i] = row0 + m0 + (int)(threadIdx.x + i * TL::THREADS) / kOutCpr;
    }
  }
  // this wavefront's band of the tile's rows: its MFMAs (and fragment
  // reads) cover only the 16-row blocks that hold some of the expert's
  // rows (every row the tile stores), so an expert's last tile spends no
  // matrix-core work on whole blocks of padding; loads, barriers and LDS
  // stages are the same in every variant
  const int band = min(TL::BM, rows - m0) - (wave / TL::WGN) * TL::WM;
  const int mie = __builtin_amdgcn_readfirstlane((min(max(band, 1), TL::WM) + 15) >> 4);
  if constexpr (kMode == 2) {
    with_row_blocks<TL>(mie, [&](auto view) {
    using TV = decltype(view);
    Acc<TV> acc;
    acc.zero();
    mainloop<TV>(a_src, b_src, p.K / TL::BK, lds, acc);
    static_assert(((TL::BM * ((TL::BN / 2) * 2 + kStagePad) + 1023) & ~1023) + TL::BM * ((TL::BN / 2) * 2 + kStagePad) <=
                      lds_bytes<TL>(),
                  "output staging and the dh tile fit the kernel's LDS");
    // SwiGLU backward at (row, feature) from the fp32 a (gate) and b (up)
    // of this tile and dh (bf16, rows of p.dH): da = dh b silu'(a),
    // db = dh silu(a), h = silu(a) b.  da is staged first; db and h wait
    // packed in the gate accumulator.  Rows past the expert's rows are not
    // read or written.
    const int wm = wave / TL::WGN, wn = wave % TL::WGN;
    constexpr int ld = (TL::BN / 2) * 2 + kStagePad;
    constexpr int cpr = (TL::BN / 2) * 2 / 16;
    const int vr = min(TL::BM, rows - m0), vc = min(cpr, (p.F - c0) * 2 / 16);
    // the tile's dh rows (loaded before the K loop) staged through LDS,
    // after the staging area of the outputs
    static_assert(TL::BM * cpr == kDhChunks * TL::THREADS, "the dh tile is whole 16-byte chunks per thread");
    char* ldh = lds + ((TL::BM * ld + 1023) & ~1023);
#pragma unroll
    for (int i = 0; i < kDhChunks; ++i) {
      const int q = threadIdx.x + i * TL::THREADS;
      const int r = q / cpr, c = q - r * cpr;
      st16(ldh + r * ld + c * 16, dh_reg[i]);
    }
    __syncthreads();
#pragma unroll
    for (int mi = 0; mi < TV::MI; ++mi)
#pragma unroll
      for (int q = 0; q < TL::NI / 2; ++q)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = acc_row<TV>(wm, mi, lane, r);
          const int col = wn * (TL::WN / 2) + q * 16 + (lane & 15);
          float da = 0.0f, db = 0.0f, h = 0.0f;
          if (m0 + row < rows && c0 + col < p.F) {
            const float a = acc.v[mi][2 * q][r], b = acc.v[mi][2 * q + 1][r];
            const float dh = bf16_to_f32(*reinterpret_cast<const uint16_t*>(ldh + row * ld + col * 2));
            const float sg = sigmoid(a);
            const float sa = a * sg;
            da = dh * b * sg * (1.0f + a * (1.0f - sg));
            db = dh * sa;
            h = sa * b;
          }
          *reinterpret_cast<uint16_t*>(lds + row * ld + col * 2) = f32_to_bf16(da);
          acc.v[mi][2 * q][r] = __uint_as_float(bf16_pair(db, h));
        }
    __syncthreads();
    char* DA = p.C + (int64_t)(row0 + m0) * p.c_row_bytes + (int64_t)c0 * 2;
    copy_rows<TL>(lds, ld, cpr, vr, vc, [&](int r) { return DA + (int64_t)r * p.c_row_bytes; });
#pragma unroll
    for (int pass = 1; pass <= 2; ++pass) {
      __syncthreads();
#pragma unroll
      for (int mi = 0; mi < TV::MI; ++mi)
#pragma unroll
        for (int q = 0; q < TL::NI / 2; ++q)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = acc_row<TV>(wm, mi, lane, r);
            const int col = wn * (TL::WN / 2) + q * 16 + (lane & 15);
            *reinterpret_cast<uint16_t*>(lds + row * ld + col * 2) =
                static_cast<uint16_t>(__float_as_uint(acc.v[mi][2 * q][r]) >> (pass == 1 ? 0 : 16));
          }
      __syncthreads();
      char* dst = pass == 1 ? DA + (int64_t)p.F * 2 : p.H + (int64_t)(row0 + m0) * p.h_row_bytes + (int64_t)c0 * 2;
      const int64_t rb = pass == 1 ? p.c_row_bytes : p.h_row_bytes;
      copy_rows<TL>(lds, ld, cpr, vr, vc, [&](int r) { return dst + (int64_t)r * rb; });
    }
    });
    return;
  }
  const int cols = kSwiglu ? p.F : p.N;
  const int tile_cols = kSwiglu ? TL::BN / 2 : TL::BN;
  const int ld = tile_cols * 2 + kStagePad;
  with_row_blocks<TL>(mie, [&](auto view) {
    using TV = decltype(view);
    Acc<TV> acc;
    acc.zero();
    mainloop<TV>(a_src, b_src, p.K / TL::BK, lds, acc);
    if (kSwiglu)
      stage_swiglu_bf16<TV>(acc, lds, ld);
    else
      stage_bf16<TV>(acc, lds, ld);
  });
  __syncthreads();
  const int vr = min(TL::BM, rows - m0), vc = min(kOutCpr, (cols - c0) * 2 / 16);
  // the row indices have long landed; one wait here, else the compiler
  // waits for them inside the loop by counts that also cover the stores
  wait_vm_all();
#pragma unroll
  for (int i = 0; i < kOutIters; ++i) {
    const int q = threadIdx.x + i * TL::THREADS;
    const int r = q / kOutCpr, c = q - r * kOutCpr;
    if (r < vr && c < vc) {
      const uint4 v = ld16(lds + r * ld + c * 16);
      char* dst = p.C + (int64_t)out_row[i] * p.c_row_bytes + (int64_t)c0 * 2 + c * 16;
      if constexpr (kSwiglu)
        st16(dst, v);
      else
        st16_stream(dst, v);  // the down-projection's rows are read once, by the combine
    }
  }
}

inline int cdiv(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }
inline int pad8(int64_t n) { return (int)((n + 7) / 8 * 8); }

}  // namespace

int ragged_tile_rows(bool tall) { return tall ? ExpertTileTall::BM : ExpertTile::BM; }
int ragged_gate_up_cols() { return ExpertTile::BN / 2; }
int ragged_down_cols() { return ExpertTile::BN; }

hipError_t launch_ragged_gate_up_bf16(const RaggedGemm& g, int64_t max_entries, bool tall, hipStream_t s) {
  if (max_entries <= 0) return hipSuccess;
  if (tall)
    ragged_gemm_kernel<ExpertTileTall, 1><<<pad8(max_entries), ExpertTileTall::THREADS, 0, s>>>(g);
  else
    ragged_gemm_kernel<ExpertTile, 1><<<pad8(max_entries), ExpertTile::THREADS, 0, s>>>(g);
  return hipGetLastError();
}

hipError_t launch_ragged_down_bf16(const RaggedGemm& g, int64_t max_entries, bool tall, hipStream_t s) {
  if (max_entries <= 0) return hipSuccess;
  if (tall)
    ragged_gemm_kernel<ExpertTileTall, 0><<<pad8(max_entries), ExpertTileTall::THREADS, 0, s>>>(g);
  else
    ragged_gemm_kernel<ExpertTile, 0><<<pad8(max_entries), ExpertTile::THREADS, 0, s>>>(g);
  return hipGetLastError();
}

hipError_t launch_ragged_swiglu_bwd_bf16(const RaggedGemm& g, int64_t max_entries, hipStream_t s) {
  if (max_entries <= 0) return hipSuccess;
  ragged_gemm_kernel<ExpertTile, 2><<<pad8(max_entries), ExpertTile::THREADS, 0, s>>>(g);
  return hipGetLastError();
}

// K ranges that can run as one: A parts consecutive columns of one buffer
// with one row pitch, B parts of one row pitch, whole K tiles in each.
bool joinable_segments(const GemmDense& g, SegK& bk, int& ktiles) {
  if (g.nseg < 2 || g.nseg > kMaxSegs) return false;
  const char* a0 = static_cast<const char*>(g.seg[0].A);
  int64_t k = 0;
  for (int s = 0; s < g.nseg; ++s) {
    const GemmSeg& q = g.seg[s];
    if (q.lda != g.seg[0].lda || q.ldb != g.seg[0].ldb || q.K <= 0 || q.K % DenseTile3B::BK) return false;
    if (static_cast<const char*>(q.A) != a0 + k * 2) return false;
    bk.p[s] = static_cast<const char*>(q.B);
    bk.first[s] = (int)(k / DenseTile3B::BK);
    k += q.K;
  }
  if (k > g.seg[0].lda) return false;
  for (int s = g.nseg; s < kMaxSegs; ++s) {
    bk.p[s] = bk.p[0];
    bk.first[s] = (int)(k / DenseTile3B::BK);
  }
  bk.n = g.nseg;
  ktiles = (int)(k / DenseTile3B::BK);
  return true;
}

hipError_t launch_gemm_dense_bf16(const GemmDense& g, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  const int tm = cdiv(g.M, DenseTile::BM), tn = cdiv(g.N, DenseTile::BN);
  SegK bk{};
  int ktiles = 0;
  if (g.nseg == 1)
    dense1_bf16_kernel<<<pad8((int64_t)tm * tn), DenseTile3B::THREADS, 0, s>>>(g, tm, tn);
  else if (joinable_segments(g, bk, ktiles))
    densecat_bf16_kernel<<<pad8((int64_t)tm * tn), DenseTile3B::THREADS, 0, s>>>(g, bk, ktiles, tm, tn);
  else
    dense_bf16_kernel<<<pad8((int64_t)tm * tn), DenseTile::THREADS, 0, s>>>(g, tm, tn);
  return hipGetLastError();
}

bool dense_f32out_supported(const GemmDense& g) {
  // whole 16-byte chunks of fp32 output rows, one K range of whole K tiles,
  // 16-byte aligned operand rows
  return g.nseg == 1 && g.N % 4 == 0 && g.seg[0].K % RouterTile::BK == 0 && g.seg[0].lda % 8 == 0 &&
         g.seg[0].ldb % 8 == 0 && g.ldc % 4 == 0;
}

hipError_t launch_dense_f32out_bf16(const GemmDense& g, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  const int tm = cdiv(g.M, RouterTile::BM), tn = cdiv(g.N, RouterTile::BN);
  dense_f32out_kernel<<<pad8((int64_t)tm * tn), RouterTile::THREADS, 0, s>>>(g, tm, tn);
  return hipGetLastError();
}

hipError_t launch_swiglu_dense_bf16(const void* A, int64_t lda, const void* Wg, const void* Wu, int G, int F,
                                    int K, int M, void* C, int64_t ldc, hipStream_t s) {
  using TL = DenseTile3B;
  if (M <= 0 || G <= 0) return hipSuccess;
  SwigluBf16 p{};
  p.A = static_cast<const char*>(A);
  p.lda_bytes = lda * 2;
  p.Wg = static_cast<const char*>(Wg);
  p.Wu = static_cast<const char*>(Wu);
  p.G = G;
  p.F = F;
  p.K = K;
  p.M = M;
  p.tiles_m = cdiv(M, TL::BM);
  p.tiles_n = cdiv(F, TL::BN / 2);
  p.C = static_cast<char*>(C);
  p.ldc_bytes = ldc * 2;
  swiglu_bf16_kernel<TL><<<pad8((int64_t)G * p.tiles_m * p.tiles_n), TL::THREADS, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace moe
