// bf16 GEMMs of the MoE branch on the gfx950 core (gemm_core.h): the dense
// projections, the shared-expert SwiGLU, and the routed experts' gathered
// SwiGLU and scattered down-projection.  fp32 accumulation; bf16 outputs.
//
// Tile shapes: 256 x 256 with 8 wavefronts (64 x 128 each) for the dense
// contractions, whose M (tokens) and N are large; 192 x 256 with 8
// wavefronts (96 x 64 each) for the routed experts, whose ~341 rows per
// expert fit two 192-row tiles with little padding.  The experts' weight
// tiles stream from HBM once each, so they get a third LDS stage.
//
// Workgroups are dealt round-robin to the 8 XCDs, each with its own L2, so
// every kernel maps its linear block index to a tile such that one XCD gets
// a contiguous range of tiles: a group of M panels x all N tiles for the
// dense GEMMs, whole experts (all M and N tiles of expert e on XCD e % 8)
// for the routed experts.  Tiles that share an operand panel then run at the
// same time on the same L2.
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

using DenseTile = core::Tile<256, 256, 4, 2, 64, 2>;
using ExpertTile = core::Tile<192, 256, 2, 4, 64, 2, 3>;

constexpr int kGroupM = 8;  // M panels per group of the dense tile order
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
// row_ptr(r) (already at the tile's first column).
template <class TL, class RowPtr>
__device__ __forceinline__ void copy_rows(const char* lds, int ld, int chunks_per_row, int valid_rows,
                                          int valid_chunks, RowPtr row_ptr) {
  const int total = TL::BM * chunks_per_row;
  for (int q = threadIdx.x; q < total; q += TL::THREADS) {
    const int r = q / chunks_per_row;
    const int c = q - r * chunks_per_row;
    if (r < valid_rows && c < valid_chunks) st16(row_ptr(r) + c * 16, ld16(lds + r * ld + c * 16));
  }
}

// ------------------------------------------------------------------ dense
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
    const char* a_src[TL::A_INS];
    const char* b_src[TL::B_INS];
#pragma unroll
    for (int i = 0; i < TL::A_INS; ++i) {
      const int m = min(m0 + load_row<TL>(i, wave, lane), g.M - 1);
      a_src[i] = static_cast<const char*>(sg.A) + (int64_t)m * sg.lda * 2 + load_col<TL>(lane);
    }
#pragma unroll
    for (int i = 0; i < TL::B_INS; ++i) {
      const int n = min(n0 + load_row<TL>(i, wave, lane), g.N - 1);
      b_src[i] = static_cast<const char*>(sg.B) + (int64_t)n * sg.ldb * 2 + load_col<TL>(lane);
    }
    mainloop<TL>(a_src, b_src, sg.K / TL::BK, lds, acc);
  }
  constexpr int ld = TL::BN * 2 + kStagePad;
  stage_bf16<TL>(acc, lds, ld);
  __syncthreads();
  constexpr int cpr = TL::BN * 2 / 16;
  char* C = static_cast<char*>(g.C);
  copy_rows<TL>(lds, ld, cpr, min(TL::BM, g.M - m0), min(cpr, (g.N - n0) * 2 / 16),
                [&](int r) { return C + ((int64_t)(m0 + r) * g.ldc + n0) * 2; });
}

// ------------------------------------------------------------------ SwiGLU
struct SwigluBf16 {
  // dense A (shared experts): row m at A + m * lda_bytes
  const char* A;
  int64_t lda_bytes;
  // gathered A (routed experts): flat pool row erow[g][m]
  const char* pools;
  int64_t block_bytes, row_bytes;
  int cap_send;
  const int32_t* erow;
  const int32_t* rows_total;
  int max_rows;
  // weights [G][F][K]
  const char* Wg;
  const char* Wu;
  int G, F, K, M;
  int tiles_m, tiles_n;  // per group
  // output
  char* C;
  int64_t ldc_bytes;
};

template <class TL, bool kGather>
__global__ __launch_bounds__(TL::THREADS) void swiglu_bf16_kernel(SwigluBf16 p) {
  __shared__ __attribute__((aligned(1024))) char lds[lds_bytes<TL>()];
  const int t = xcd_order(blockIdx.x, gridDim.x);
  int g, mt, nt;
  if (kGather) {
    // expert g on XCD g % 8; per XCD: experts in order, then N tile, M fastest
    const int per_g = p.tiles_m * p.tiles_n;
    const int per_xcd = gridDim.x >> 3;
    const int xcd = t / per_xcd, local = t - xcd * per_xcd;
    g = (local / per_g) * 8 + xcd;
    if (g >= p.G) return;
    const int r = local - (local / per_g) * per_g;
    nt = r / p.tiles_m;
    mt = r - nt * p.tiles_m;
  } else {
    const int per_g = p.tiles_m * p.tiles_n;
    g = t / per_g;
    if (g >= p.G) return;
    dense_tile(t - g * per_g, p.tiles_m, p.tiles_n, mt, nt);
  }
  const int rows = kGather ? p.rows_total[g] : p.M;
  const int m0 = mt * TL::BM;
  if (m0 >= rows) return;
  const int f0 = nt * (TL::BN / 2);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const char* a_src[TL::A_INS];
  const char* b_src[TL::B_INS];
#pragma unroll
  for (int i = 0; i < TL::A_INS; ++i) {
    const int m = min(m0 + load_row<TL>(i, wave, lane), rows - 1);
    if (kGather) {
      const int fi = p.erow[(int64_t)g * p.max_rows + m];
      const int blk = fi / p.cap_send;
      const int slot = fi - blk * p.cap_send;
      a_src[i] = p.pools + blk * p.block_bytes + slot * p.row_bytes + load_col<TL>(lane);
    } else {
      a_src[i] = p.A + m * p.lda_bytes + load_col<TL>(lane);
    }
  }
#pragma unroll
  for (int i = 0; i < TL::B_INS; ++i) {
    int half;
    const int f = min(f0 + swiglu_feature<TL>(load_row<TL>(i, wave, lane), half), p.F - 1);
    const char* W = half ? p.Wu : p.Wg;
    b_src[i] = W + ((int64_t)g * p.F + f) * p.K * 2 + load_col<TL>(lane);
  }
  Acc<TL> acc;
  acc.zero();
  mainloop<TL>(a_src, b_src, p.K / TL::BK, lds, acc);
  constexpr int ld = TL::BN + kStagePad;  // BN / 2 features of bf16
  stage_swiglu_bf16<TL>(acc, lds, ld);
  __syncthreads();
  constexpr int cpr = TL::BN / 16;
  const int valid_chunks = min(cpr, (p.F - f0) * 2 / 16);
  char* C = p.C;
  if (kGather) {
    copy_rows<TL>(lds, ld, cpr, min(TL::BM, rows - m0), valid_chunks, [&](int r) {
      return C + (((int64_t)g * p.max_rows + m0 + r) * p.F + f0) * 2;
    });
  } else {
    copy_rows<TL>(lds, ld, cpr, min(TL::BM, rows - m0), valid_chunks, [&](int r) {
      return C + (int64_t)(m0 + r) * p.ldc_bytes + ((int64_t)g * p.F + f0) * 2;
    });
  }
}

// ------------------------------------------------------------------ expert down
__global__ __launch_bounds__(ExpertTile::THREADS) void expert_down_bf16_kernel(ExpertDown p, int tiles_m,
                                                                               int tiles_n) {
  using TL = ExpertTile;
  __shared__ __attribute__((aligned(1024))) char lds[lds_bytes<TL>()];
  const int t = xcd_order(blockIdx.x, gridDim.x);
  const int per_e = tiles_m * tiles_n;
  const int per_xcd = gridDim.x >> 3;
  const int xcd = t / per_xcd, local = t - xcd * per_xcd;
  const int e = (local / per_e) * 8 + xcd;
  if (e >= p.E) return;
  const int r0 = local - (local / per_e) * per_e;
  const int nt = r0 / tiles_m, mt = r0 - nt * tiles_m;
  const int rows = p.rows_total[e];
  const int m0 = mt * TL::BM, n0 = nt * TL::BN;
  if (m0 >= rows) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const char* H = static_cast<const char*>(p.H);
  const char* Wd = static_cast<const char*>(p.Wd);
  const char* a_src[TL::A_INS];
  const char* b_src[TL::B_INS];
#pragma unroll
  for (int i = 0; i < TL::A_INS; ++i) {
    const int m = min(m0 + load_row<TL>(i, wave, lane), rows - 1);
    a_src[i] = H + ((int64_t)e * p.max_rows + m) * p.F * 2 + load_col<TL>(lane);
  }
#pragma unroll
  for (int i = 0; i < TL::B_INS; ++i) {
    const int n = min(n0 + load_row<TL>(i, wave, lane), p.L - 1);
    b_src[i] = Wd + ((int64_t)e * p.L + n) * p.F * 2 + load_col<TL>(lane);
  }
  Acc<TL> acc;
  acc.zero();
  mainloop<TL>(a_src, b_src, p.F / TL::BK, lds, acc);
  constexpr int ld = TL::BN * 2 + kStagePad;
  stage_bf16<TL>(acc, lds, ld);
  __syncthreads();
  constexpr int cpr = TL::BN * 2 / 16;
  char* out = static_cast<char*>(p.out);
  const int32_t* er = p.erow + (int64_t)e * p.max_rows + m0;
  copy_rows<TL>(lds, ld, cpr, min(TL::BM, rows - m0), min(cpr, (p.L - n0) * 2 / 16),
                [&](int r) { return out + ((int64_t)er[r] * p.L + n0) * 2; });
}

// ------------------------------------------------------------------ ragged
// Dropless grouped GEMMs: list entry t = (expert e, n tile, m tile); expert
// e's rows are rows [offsets[e], offsets[e+1]) of A and of C.  XCD x runs an
// eighth of the list, contiguous, so an expert's tiles share one L2.
template <class TL, bool kSwiglu>
__global__ __launch_bounds__(TL::THREADS) void ragged_gemm_kernel(RaggedGemm p) {
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
  const char* a_src[TL::A_INS];
  const char* b_src[TL::B_INS];
#pragma unroll
  for (int i = 0; i < TL::A_INS; ++i) {
    const int m = min(m0 + load_row<TL>(i, wave, lane), rows - 1);
    a_src[i] = p.A + (int64_t)(row0 + m) * p.a_row_bytes + load_col<TL>(lane);
  }
  const int c0 = kSwiglu ? nt * (TL::BN / 2) : nt * TL::BN;
#pragma unroll
  for (int i = 0; i < TL::B_INS; ++i) {
    const int r = load_row<TL>(i, wave, lane);
    if (kSwiglu) {
      int half;
      const int f = min(c0 + swiglu_feature<TL>(r, half), p.F - 1);
      b_src[i] = (half ? p.W1 : p.W0) + ((int64_t)e * p.F + f) * p.K * 2 + load_col<TL>(lane);
    } else {
      const int n = min(c0 + r, p.N - 1);
      b_src[i] = p.W0 + ((int64_t)e * p.N + n) * p.K * 2 + load_col<TL>(lane);
    }
  }
  Acc<TL> acc;
  acc.zero();
  mainloop<TL>(a_src, b_src, p.K / TL::BK, lds, acc);
  const int cols = kSwiglu ? p.F : p.N;
  const int tile_cols = kSwiglu ? TL::BN / 2 : TL::BN;
  const int ld = tile_cols * 2 + kStagePad;
  if (kSwiglu)
    stage_swiglu_bf16<TL>(acc, lds, ld);
  else
    stage_bf16<TL>(acc, lds, ld);
  __syncthreads();
  const int cpr = tile_cols * 2 / 16;
  copy_rows<TL>(lds, ld, cpr, min(TL::BM, rows - m0), min(cpr, (cols - c0) * 2 / 16), [&](int r) {
    return p.C + (int64_t)(row0 + m0 + r) * p.c_row_bytes + (int64_t)c0 * 2;
  });
}

inline int cdiv(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }
inline int pad8(int64_t n) { return (int)((n + 7) / 8 * 8); }

}  // namespace

int ragged_tile_rows() { return ExpertTile::BM; }
int ragged_gate_up_cols() { return ExpertTile::BN / 2; }
int ragged_down_cols() { return ExpertTile::BN; }

hipError_t launch_ragged_gate_up_bf16(const RaggedGemm& g, int64_t max_entries, hipStream_t s) {
  if (max_entries <= 0) return hipSuccess;
  ragged_gemm_kernel<ExpertTile, true><<<pad8(max_entries), ExpertTile::THREADS, 0, s>>>(g);
  return hipGetLastError();
}

hipError_t launch_ragged_down_bf16(const RaggedGemm& g, int64_t max_entries, hipStream_t s) {
  if (max_entries <= 0) return hipSuccess;
  ragged_gemm_kernel<ExpertTile, false><<<pad8(max_entries), ExpertTile::THREADS, 0, s>>>(g);
  return hipGetLastError();
}

hipError_t launch_gemm_dense_bf16(const GemmDense& g, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  const int tm = cdiv(g.M, DenseTile::BM), tn = cdiv(g.N, DenseTile::BN);
  dense_bf16_kernel<<<pad8((int64_t)tm * tn), DenseTile::THREADS, 0, s>>>(g, tm, tn);
  return hipGetLastError();
}

hipError_t launch_swiglu_dense_bf16(const void* A, int64_t lda, const void* Wg, const void* Wu, int G, int F,
                                    int K, int M, void* C, int64_t ldc, hipStream_t s) {
  using TL = DenseTile;
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
  swiglu_bf16_kernel<TL, false><<<pad8((int64_t)G * p.tiles_m * p.tiles_n), TL::THREADS, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_expert_gate_up_bf16(const ExpertGateUp& a, hipStream_t s) {
  using TL = ExpertTile;
  if (a.E <= 0 || a.max_rows <= 0) return hipSuccess;
  SwigluBf16 p{};
  p.pools = a.pools;
  p.block_bytes = a.block_bytes;
  p.row_bytes = a.row_bytes;
  p.cap_send = a.cap_send;
  p.erow = a.erow;
  p.rows_total = a.rows_total;
  p.max_rows = a.max_rows;
  p.Wg = static_cast<const char*>(a.Wg);
  p.Wu = static_cast<const char*>(a.Wu);
  p.G = a.E;
  p.F = a.F;
  p.K = a.L;
  p.tiles_m = cdiv(a.max_rows, TL::BM);
  p.tiles_n = cdiv(a.F, TL::BN / 2);
  p.C = static_cast<char*>(a.H);
  const int64_t blocks = 8 * (int64_t)cdiv(a.E, 8) * p.tiles_m * p.tiles_n;
  swiglu_bf16_kernel<TL, true><<<(unsigned)blocks, TL::THREADS, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_expert_down_bf16(const ExpertDown& a, hipStream_t s) {
  using TL = ExpertTile;
  if (a.E <= 0 || a.max_rows <= 0) return hipSuccess;
  const int tm = cdiv(a.max_rows, TL::BM), tn = cdiv(a.L, TL::BN);
  const int64_t blocks = 8 * (int64_t)cdiv(a.E, 8) * tm * tn;
  expert_down_bf16_kernel<<<(unsigned)blocks, TL::THREADS, 0, s>>>(a, tm, tn);
  return hipGetLastError();
}

}  // namespace moe
