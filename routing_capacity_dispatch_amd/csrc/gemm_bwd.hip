// Grouped GEMMs of the routed experts' backward, bf16 with fp32
// accumulation, over the padded expert-major row order (expert e's rows at
// [offsets[e], offsets[e] + counts[e]), zero rows up to offsets[e+1]).
//
//   dgrad, dh:  dh[r, :] = do[r, :] W_d[e]       (W_d [L][F] read K-major),
//               bf16 out; the SwiGLU backward da = dh b silu'(a),
//               db = dh silu(a), h = silu(a) b then runs in the epilogue of
//               the forward gate/up GEMM recomputing a and b (gemm_bf16.hip)
//   dgrad, du:  du[r, :] = da[r, :] W_g[e] + db[r, :] W_u[e]  (two K
//               segments, W_g / W_u [F][L] read K-major); rows scattered to
//               the pool slots they came from
//   wgrad:      dW[e] = X^T Y over the expert's padded rows, X and Y both
//               read K-major: dW_d = do^T h, dW_g = da^T u, dW_u = db^T u,
//               written in the weights' [out][in] layout
//
// dgrad tiles are 192 rows x 256 columns (8 wavefronts, 96 x 64 each, a
// third LDS stage for the streaming weights) over device-built tile lists
// like the forward's; wgrad tiles are 256 x 256 (8 wavefronts, 64 x 128
// each), an expert's tiles dealt to one XCD.  dgrad runs the forward core's
// split-barrier schedule with a K-major B operand; wgrad, with two K-major
// operands, the plain two-stage one (gemm_core.h).
#include "common.h"
#include "gemm_core.h"
#include "kernels.h"

namespace moe {
namespace {

using core::Acc;
using core::acc_col;
using core::acc_row;
using core::kload_col;
using core::kload_row;
using core::load_col;
using core::load_row;
using core::mainloop;
using core::RowSrc;
using core::uniform_ptr;

using DgradTile = core::Tile<192, 256, 2, 4, 64, 2, 3>;  // the weights stream: a third B stage
using WgradTile = core::Tile<256, 256, 4, 2, 64, 2, 2>;
constexpr int kStagePad = 16;

template <class TL>
constexpr int lds_bytes() {
  return TL::MAIN_LDS > TL::BM * (TL::BN * 2 + kStagePad) ? TL::MAIN_LDS : TL::BM * (TL::BN * 2 + kStagePad);
}

__device__ __forceinline__ int xcd_order(int bid, int nblocks) { return (bid & 7) * (nblocks >> 3) + (bid >> 3); }

template <class TL, class RowPtr>
__device__ __forceinline__ void copy_rows(const char* lds, int ld, int chunks_per_row, int valid_rows,
                                          RowPtr row_ptr) {
  const int total = TL::BM * chunks_per_row;
  for (int q = threadIdx.x; q < total; q += TL::THREADS) {
    const int r = q / chunks_per_row;
    const int c = q - r * chunks_per_row;
    if (r < valid_rows) st16(row_ptr(r) + c * 16, ld16(lds + r * ld + c * 16));
  }
}

// Stage 16 bits of every accumulator (lo: its bf16 value; hi > 0: the
// half of a packed 32-bit pair) as tile rows of `ld` bytes.
template <class TL>
__device__ __forceinline__ void stage(const Acc<TL>& acc, char* lds, int ld, int packed_half) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / TL::WGN, wn = wave % TL::WGN;
#pragma unroll
  for (int mi = 0; mi < TL::MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < TL::NI; ++ni)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = acc_row<TL>(wm, mi, lane, r), col = acc_col<TL>(wn, ni, lane);
        const float v = acc.v[mi][ni][r];
        const uint16_t h = packed_half == 0 ? f32_to_bf16(v)
                                            : static_cast<uint16_t>(__float_as_uint(v) >> (packed_half == 1 ? 0 : 16));
        *reinterpret_cast<uint16_t*>(lds + row * ld + col * 2) = h;
      }
}

// ------------------------------------------------------------------ dgrad
template <int kMode>  // 0: dh, rows in order; 1: du (two segments, rows scattered)
__global__ __launch_bounds__(DgradTile::THREADS) void dgrad_kernel(BwdDgrad p) {
  using TL = DgradTile;
  __shared__ __attribute__((aligned(1024))) char lds[lds_bytes<TL>()];
  const int n = *p.ntiles;
  const int per_xcd = (n + 7) >> 3;
  const int local = blockIdx.x >> 3;
  const int t = (blockIdx.x & 7) * per_xcd + local;
  if (local >= per_xcd || t >= n) return;
  const int e = p.list[3 * t], nt = p.list[3 * t + 1], mt = p.list[3 * t + 2];
  const int row0 = p.offsets[e];
  const int rows_pad = p.offsets[e + 1] - row0;
  const int rows = min(p.counts[e], rows_pad);
  const int m0 = mt * TL::BM, n0 = nt * TL::BN;
  if (m0 >= rows_pad) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  Acc<TL> acc;
  acc.zero();
  const char* A = uniform_ptr(p.A + (int64_t)row0 * p.a_row_bytes);
  for (int seg = 0; seg < (kMode == 1 ? 2 : 1); ++seg) {
    RowSrc<TL::A_INS> a_src;
    RowSrc<TL::B_INS> b_src;
#pragma unroll
    for (int i = 0; i < TL::A_INS; ++i) {
      const int m = min(m0 + load_row<TL>(i, wave, lane), rows_pad - 1);
      a_src.base[i] = A;
      a_src.off[i] = (uint32_t)(m * p.a_row_bytes + seg * p.a_seg_bytes) + load_col<TL>(lane);
    }
    const char* W = uniform_ptr((seg ? p.W1 : p.W0) + (int64_t)e * p.K * p.N * 2 + (int64_t)n0 * 2);
#pragma unroll
    for (int i = 0; i < TL::B_INS; ++i) {
      const int kr = kload_row<TL, TL::BN>(i, wave, lane);
      b_src.base[i] = W;
      b_src.off[i] = (uint32_t)(kr * p.N * 2) + kload_col<TL::BN>(kr, lane);
    }
    mainloop<TL, true, false, true>(a_src, b_src, p.K / TL::BK, lds, acc, TL::RB, (int64_t)64 * p.N * 2);
  }
  constexpr int ld = TL::BN * 2 + kStagePad;
  constexpr int cpr = TL::BN * 2 / 16;
  if constexpr (kMode == 0) {
    // dh rows, padding rows included (their do rows are zero)
    stage<TL>(acc, lds, ld, 0);
    __syncthreads();
    char* C = p.C + (int64_t)(row0 + m0) * p.c_row_bytes + (int64_t)n0 * 2;
    copy_rows<TL>(lds, ld, cpr, min(TL::BM, rows_pad - m0), [&](int r) { return C + (int64_t)r * p.c_row_bytes; });
  } else {
    stage<TL>(acc, lds, ld, 0);
    __syncthreads();
    const int32_t* ci = p.c_index + row0 + m0;
    copy_rows<TL>(lds, ld, cpr, min(TL::BM, rows - m0),
                  [&](int r) { return p.C + (int64_t)ci[r] * p.c_row_bytes + (int64_t)n0 * 2; });
  }
}

// ------------------------------------------------------------------ wgrad
__global__ __launch_bounds__(WgradTile::THREADS) void wgrad_kernel(BwdWgrad p) {
  using TL = WgradTile;
  __shared__ __attribute__((aligned(1024))) char lds[lds_bytes<TL>()];
  const int per_e = p.tiles_m * p.tiles_n;
  const int t = xcd_order(blockIdx.x, gridDim.x);
  const int e = t / per_e;
  if (e >= p.E) return;
  const int r = t - e * per_e;
  const int mt = r % p.tiles_m, nt = r / p.tiles_m;
  const int m0 = mt * TL::BM, n0 = nt * TL::BN;
  const int row0 = p.offsets[e];
  const int ktiles = (p.offsets[e + 1] - row0) / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  RowSrc<TL::A_INS> a_src;
  RowSrc<TL::B_INS> b_src;
  const char* A = uniform_ptr(p.X + (int64_t)row0 * p.x_row_bytes + p.x_col_bytes + (int64_t)m0 * 2);
  const char* B = uniform_ptr(p.Y + (int64_t)row0 * p.y_row_bytes + p.y_col_bytes + (int64_t)n0 * 2);
#pragma unroll
  for (int i = 0; i < TL::A_INS; ++i) {
    const int kr = kload_row<TL, TL::BM>(i, wave, lane);
    a_src.base[i] = A;
    a_src.off[i] = (uint32_t)(kr * p.x_row_bytes) + kload_col<TL::BM>(kr, lane);
  }
#pragma unroll
  for (int i = 0; i < TL::B_INS; ++i) {
    const int kr = kload_row<TL, TL::BN>(i, wave, lane);
    b_src.base[i] = B;
    b_src.off[i] = (uint32_t)(kr * p.y_row_bytes) + kload_col<TL::BN>(kr, lane);
  }
  Acc<TL> acc;
  acc.zero();
  mainloop<TL, false, true, true>(a_src, b_src, ktiles, lds, acc, 64 * p.x_row_bytes, 64 * p.y_row_bytes);
  constexpr int ld = TL::BN * 2 + kStagePad;
  stage<TL>(acc, lds, ld, 0);
  __syncthreads();
  char* C = p.C + ((int64_t)e * p.M + m0) * p.N * 2 + (int64_t)n0 * 2;
  copy_rows<TL>(lds, ld, TL::BN * 2 / 16, TL::BM, [&](int rr) { return C + (int64_t)rr * p.N * 2; });
}

inline int pad8(int64_t n) { return (int)((n + 7) / 8 * 8); }

}  // namespace

int bwd_dgrad_rows() { return DgradTile::BM; }
int bwd_dgrad_cols() { return DgradTile::BN; }
int bwd_wgrad_tile() { return WgradTile::BM; }

hipError_t launch_bwd_dh(const BwdDgrad& p, int64_t max_entries, hipStream_t s) {
  if (max_entries <= 0) return hipSuccess;
  dgrad_kernel<0><<<pad8(max_entries), DgradTile::THREADS, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_bwd_du(const BwdDgrad& p, int64_t max_entries, hipStream_t s) {
  if (max_entries <= 0) return hipSuccess;
  dgrad_kernel<1><<<pad8(max_entries), DgradTile::THREADS, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_bwd_wgrad(const BwdWgrad& p, hipStream_t s) {
  if (p.E <= 0) return hipSuccess;
  wgrad_kernel<<<pad8((int64_t)p.E * p.tiles_m * p.tiles_n), WgradTile::THREADS, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace moe
