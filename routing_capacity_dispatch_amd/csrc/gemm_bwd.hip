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
// like the forward's, on the forward core's split-barrier schedule with a
// K-major B operand (gemm_core.h).  wgrad tiles are 256 x 256 (8
// wavefronts, 64 x 128 each), an expert's tiles dealt to one XCD, in a
// persistent kernel of its own with both operands K-major (below).
#include "common.h"
#include "gemm_core.h"
#include "kernels.h"

namespace moe {
namespace {

using core::Acc;
using core::Frags;
using core::acc_col;
using core::acc_row;
using core::kload_col;
using core::kload_row;
using core::load_col;
using core::load_row;
using core::mainloop;
using core::RowSrc;
using core::uniform_ptr;
using core::with_row_blocks;

using DgradTile = core::Tile<192, 256, 2, 4, 64, 2, 3>;  // the weights stream: a third B stage
using WgradTile = core::Tile<256, 256, 4, 2, 32, 4>;
constexpr int kStagePad = 16;

template <class TL>
constexpr int lds_bytes() {
  return TL::MAIN_LDS > TL::BM * (TL::BN * 2 + kStagePad) ? TL::MAIN_LDS : TL::BM * (TL::BN * 2 + kStagePad);
}

// kStream: nontemporal stores (outputs no later tile of the kernel reads)
template <class TL, bool kStream = false, class RowPtr>
__device__ __forceinline__ void copy_rows(const char* lds, int ld, int chunks_per_row, int valid_rows,
                                          RowPtr row_ptr) {
  const int total = TL::BM * chunks_per_row;
  for (int q = threadIdx.x; q < total; q += TL::THREADS) {
    const int r = q / chunks_per_row;
    const int c = q - r * chunks_per_row;
    if (r < valid_rows) {
      if constexpr (kStream)
        st16_stream(row_ptr(r) + c * 16, ld16(lds + r * ld + c * 16));
      else
        st16(row_ptr(r) + c * 16, ld16(lds + r * ld + c * 16));
    }
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
  // this wavefront's band of the tile's rows: MFMAs only for the 16-row
  // blocks that hold a row the tile stores (dh: every padded row, whose
  // zeros later contractions read; du: the expert's rows)
  const int band = min(TL::BM, (kMode == 0 ? rows_pad : rows) - m0) - (wave / TL::WGN) * TL::WM;
  const int mie = __builtin_amdgcn_readfirstlane((min(max(band, 1), TL::WM) + 15) >> 4);
  with_row_blocks<TL>(mie, [&](auto view) {
  using TV = decltype(view);
  Acc<TV> acc;
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
    mainloop<TV, true, false, true>(a_src, b_src, p.K / TL::BK, lds, acc, TL::RB, (int64_t)64 * p.N * 2);
  }
  constexpr int ld = TL::BN * 2 + kStagePad;
  constexpr int cpr = TL::BN * 2 / 16;
  if constexpr (kMode == 0) {
    // dh rows, padding rows included (their do rows are zero)
    stage<TV>(acc, lds, ld, 0);
    __syncthreads();
    char* C = p.C + (int64_t)(row0 + m0) * p.c_row_bytes + (int64_t)n0 * 2;
    copy_rows<TL>(lds, ld, cpr, min(TL::BM, rows_pad - m0), [&](int r) { return C + (int64_t)r * p.c_row_bytes; });
  } else {
    // the pool slot of each row this thread stores, read before the staging
    // with every load in flight together (a load in the store loop makes each
    // store wait for the previous one: stores count in the same counter); not
    // before the K loop, which is at the register limit
    constexpr int kOutIters = TL::BM * cpr / TL::THREADS;
    static_assert(TL::BM * cpr % TL::THREADS == 0, "whole chunks per thread");
    const int vr = min(TL::BM, rows - m0);  // may be <= 0: a tile of padding rows stores nothing
    int32_t out_row[kOutIters];
#pragma unroll
    for (int i = 0; i < kOutIters; ++i) {
      const int r = (int)(threadIdx.x + i * TL::THREADS) / cpr;
      out_row[i] = p.c_index[row0 + m0 + max(min(r, vr - 1), 0)];
    }
    stage<TV>(acc, lds, ld, 0);
    __syncthreads();
    // one wait for the indices, else the compiler waits for them inside the
    // loop by counts that also cover the stores
    wait_vm_all();
#pragma unroll
    for (int i = 0; i < kOutIters; ++i) {
      const int q = threadIdx.x + i * TL::THREADS;
      const int r = q / cpr, c = q - r * cpr;
      if (r < vr)
        st16(p.C + (int64_t)out_row[i] * p.c_row_bytes + (int64_t)n0 * 2 + c * 16, ld16(lds + r * ld + c * 16));
    }
  }
  });
}

// ------------------------------------------------------------------ wgrad
// Persistent: a workgroup walks every nx-th tile of its XCD's contiguous
// share of the expert-major tile list (nx workgroups per XCD; an expert's
// tiles output-row tile fastest, so the window of tiles running on one XCD
// shares the expert's X columns) through one K pipeline that runs across
// tile boundaries, so the loads of the next tile's first K tiles are in
// flight while the current tile finishes and writes its output.  K tiles of
// 32 in four stages, on a mid-tile barrier schedule split along N (below).
//
// The operands are swapped (the MFMA's M side is Y, the output's columns),
// so each lane holds 4 consecutive output columns of a row; the output goes
// out through a per-wavefront LDS area beside the stages, 16 rows at a
// time, as whole 128-byte row segments with nontemporal stores (no later
// tile of the kernel reads them).
constexpr int kEpiPitch = 144;                      // bytes per staged output row (128 + 16)
constexpr int kEpiWave = 16 * kEpiPitch;            // one wavefront's staging area
// Store instructions per wavefront per tile.  The waits below count them
// among the operations issued after an awaited K tile, which is exact
// because each one writes in-range memory with every lane active: stores
// complete in issue order with the loads around them, but a buffer store
// whose lanes the hardware drops (out of range) need not.
constexpr int kEpiStores = WgradTile::WM * WgradTile::WN * 2 / 1024;

// Wait until the loads of a K tile have landed when `after` K tiles were
// issued after it and, if `stores`, at least one tile's output stores too
// (memory operations of a wavefront complete in issue order), then
// synchronise the workgroup.  The wavefront's LDS reads are complete first,
// so a stage that every wavefront has read may be refilled after the
// barrier.
__device__ __forceinline__ void wgrad_wait(int after, bool stores) {
  constexpr int P = WgradTile::A_INS + WgradTile::B_INS;
  static_assert(WgradTile::NS == 4, "after is 0 .. 3");
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  if (stores) {
    if (after >= 3)
      core::wait_loads<3 * P + kEpiStores>();
    else if (after == 2)
      core::wait_loads<2 * P + kEpiStores>();
    else if (after == 1)
      core::wait_loads<P + kEpiStores>();
    else
      core::wait_loads<kEpiStores>();
  } else {
    if (after >= 3)
      core::wait_loads<3 * P>();
    else if (after == 2)
      core::wait_loads<2 * P>();
    else if (after == 1)
      core::wait_loads<P>();
    else
      core::wait_loads<0>();
  }
}

// Fragments of one K tile split by N: all of A with the first half of B
// (the first phase's MFMAs), and the second half of B.
struct WgradHalf {
  uint4 a[WgradTile::MI];
  uint4 b[WgradTile::NI / 2];
};

template <int kFirst>
__device__ __forceinline__ void wgrad_read_b(const char* sb, uint4* b, int wn, int lane) {
  using TL = WgradTile;
#pragma unroll
  for (int j = 0; j < TL::NI / 2; ++j) b[j] = core::kfrag<TL::BN>(sb, wn * TL::WN + (kFirst + j) * 16, 0, lane);
}

__device__ __forceinline__ void wgrad_read_first(const char* sa, const char* sb, WgradHalf& h, int wm, int wn,
                                                 int lane) {
  using TL = WgradTile;
#pragma unroll
  for (int i = 0; i < TL::MI; ++i) h.a[i] = core::kfrag<TL::BM>(sa, wm * TL::WM + i * 16, 0, lane);
  wgrad_read_b<0>(sb, h.b, wn, lane);
}

template <int kFirst>
__device__ __forceinline__ void wgrad_mfma(const uint4* a, const uint4* b, Acc<WgradTile>& acc) {
  using TL = WgradTile;
#pragma unroll
  for (int i = 0; i < TL::MI; ++i)
#pragma unroll
    for (int j = 0; j < TL::NI / 2; ++j)
      acc.v[i][kFirst + j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          __builtin_bit_cast(bf16x8_t, a[i]), __builtin_bit_cast(bf16x8_t, b[j]), acc.v[i][kFirst + j], 0, 0, 0);
}

// nr LDS reads spread among nm MFMAs
template <int nm, int nr>
__device__ __forceinline__ void wgrad_interleave() {
#pragma unroll
  for (int i = 0; i < nr; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, nm / nr, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, nm - (nm / nr) * nr, 0);
}

// offsets, counts: p.offsets and p.counts as separate restrict arguments, so
// that the compiler reads them with scalar loads (no store of the kernel can
// alias them) instead of vector loads whose waits would drain the loads in
// flight
__global__ __launch_bounds__(WgradTile::THREADS) void wgrad_kernel(BwdWgrad p,
                                                                   const int32_t* __restrict__ offsets,
                                                                   const int32_t* __restrict__ counts) {
  using TL = WgradTile;
  constexpr int NS = TL::NS;
  constexpr int NM = TL::MI * TL::NI / 2;  // MFMAs per phase
  __shared__ __attribute__((aligned(1024))) char lds[TL::MAIN_LDS + TL::NW * kEpiWave];
  const int per_e = p.tiles_m * p.tiles_n;
  const int total = p.E * per_e;
  const int per_xcd = (total + 7) >> 3;
  const int nx = gridDim.x >> 3;
  const int xcd = blockIdx.x & 7;
  const int t0 = xcd * per_xcd + (blockIdx.x >> 3);
  const int t_end = min(total, (xcd + 1) * per_xcd);
  if (t0 >= t_end) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / TL::WGN, wn = wave % TL::WGN;
  char* lds_a = lds;
  char* lds_b = lds + TL::B_BASE;
  // per-lane offsets, the same in every tile: A = Y (K-major, BM wide),
  // B = X (K-major, BN wide)
  uint32_t a_off[TL::A_INS], b_off[TL::B_INS];
#pragma unroll
  for (int i = 0; i < TL::A_INS; ++i) {
    const int kr = kload_row<TL, TL::BM>(i, wave, lane);
    a_off[i] = (uint32_t)(kr * p.y_row_bytes) + kload_col<TL::BM>(kr, lane);
  }
#pragma unroll
  for (int i = 0; i < TL::B_INS; ++i) {
    const int kr = kload_row<TL, TL::BN>(i, wave, lane);
    b_off[i] = (uint32_t)(kr * p.x_row_bytes) + kload_col<TL::BN>(kr, lane);
  }
  const int64_t a_kstep = (int64_t)TL::BK * p.y_row_bytes, b_kstep = (int64_t)TL::BK * p.x_row_bytes;
  // tile t: expert, output origin (m0 rows, n0 columns), K tiles (over the
  // expert's rows: a last K tile of the 64-row padding that holds no row is
  // skipped), and the wave-uniform bases of its Y and X columns
  auto info = [&](int t, int& e, int& m0, int& n0, const char*& ya, const char*& xb) {
    e = t / per_e;
    const int r = t - e * per_e;
    m0 = (r % p.tiles_m) * TL::BN;
    n0 = (r / p.tiles_m) * TL::BM;
    const int row0 = offsets[e];
    ya = uniform_ptr(p.Y + (int64_t)row0 * p.y_row_bytes + p.y_col_bytes + (int64_t)n0 * 2);
    xb = uniform_ptr(p.X + (int64_t)row0 * p.x_row_bytes + p.x_col_bytes + (int64_t)m0 * 2);
    const int rows = max(min(counts[e], offsets[e + 1] - row0), 0);
    return (rows + TL::BK - 1) / TL::BK;
  };
  // the load cursor: tile lt, K tile lk of its lkt
  int lt = t0, lk = 0, lkt = 0;
  const char* la = nullptr;
  const char* lb = nullptr;
  auto seek = [&]() {  // from lt on, the first tile with K tiles
    for (; lt < t_end; lt += nx) {
      int e, m0, n0;
      lkt = info(lt, e, m0, n0, la, lb);
      if (lkt > 0) break;
    }
  };
  auto issue_next = [&](int stage) {
    const int64_t ka = lk * a_kstep, kb = lk * b_kstep;
#pragma unroll
    for (int i = 0; i < TL::A_INS; ++i)
      core::lds_load16(la + ka, a_off[i], lds_a + stage * TL::A_BYTES + (i * TL::NW + wave) * 1024);
#pragma unroll
    for (int i = 0; i < TL::B_INS; ++i)
      core::lds_load16(lb + kb, b_off[i], lds_b + stage * TL::B_BYTES + (i * TL::NW + wave) * 1024);
    if (++lk == lkt) {
      lk = 0;
      lt += nx;
      seek();
    }
  };
  // K tile s of this workgroup's sequence sits in stage s % NS; the loads
  // of K tiles s + 1 .. s + NS are in flight while tile s is consumed:
  //   phase 1: MFMAs of (s, A with B's first half) | reads of B's second half
  //   phase 2: wait for tile s + 1, barrier (every read of tile s done)
  //   phase 3: loads of tile s + NS into stage s % NS;
  //            MFMAs of (s, B's second half) | reads of (s + 1, first half)
  seek();
  int issued = 0;  // K tiles issued so far
  for (int j = 0; j < NS && lt < t_end; ++j) {
    issue_next(j);
    ++issued;
  }
  int s = 0;                // K tiles consumed so far
  int last_epi = -4 * NS;   // the K tile after which the last output stores went out
  char* ew = lds + TL::MAIN_LDS + wave * kEpiWave;
  WgradHalf h0, h1;
  uint4 b2[TL::NI / 2];
  if (issued > 0) {
    wgrad_wait(issued - 1, false);
    wgrad_read_first(lds_a, lds_b, h0, wm, wn, lane);
  }
  Acc<TL> acc;
  acc.zero();
  // one K tile: the MFMAs on cur, the next tile's first half read into nxt
  auto step = [&](WgradHalf& cur, WgradHalf& nxt) __attribute__((always_inline)) {
    const int st = s % NS;
    // phase 1
    wgrad_read_b<TL::NI / 2>(lds_b + st * TL::B_BYTES, b2, wn, lane);
    wgrad_mfma<0>(cur.a, cur.b, acc);
    wgrad_interleave<NM, TL::NI>();
    // phase 2: K tile s + 1 was issued before the loop or in iteration
    // s + 1 - NS, ahead of that iteration's output stores
    if (s + 1 < issued) wgrad_wait(issued - 1 - (s + 1), last_epi >= s + 1 - NS);
    // phase 3 (the reads of a tile past the last one read a stale stage and
    // go unused)
    if (lt < t_end) {
      issue_next(st);
      ++issued;
    }
    const int st1 = (s + 1) % NS;
    wgrad_read_first(lds_a + st1 * TL::A_BYTES, lds_b + st1 * TL::B_BYTES, nxt, wm, wn, lane);
    wgrad_mfma<TL::NI / 2>(cur.a, b2, acc);
    wgrad_interleave<NM, TL::MI * 2 + TL::NI>();
    ++s;
  };
  for (int t = t0; t < t_end; t += nx) {
    int e, m0, n0;
    const char* ya;
    const char* xb;
    const int kt = info(t, e, m0, n0, ya, xb);
    int k = 0;
    for (; k + 1 < kt; k += 2) {
      step(h0, h1);
      step(h1, h0);
    }
    if (k < kt) {  // an odd count: the next K tile's first half went into h1
      step(h0, h1);
      h0 = h1;
    }
    // output rows m0 + wn WN + ni 16 + (0..15), columns n0 + wm WM + (0..63):
    // lane l holds row (l & 15) of block ni, columns mi 16 + 4 (l >> 4) + (0..3)
    char* C = p.C + ((int64_t)e * p.M + m0 + wn * TL::WN) * p.N * 2 + (int64_t)(n0 + wm * TL::WM) * 2;
#pragma unroll
    for (int ni = 0; ni < TL::NI; ++ni) {
#pragma unroll
      for (int mi = 0; mi < TL::MI; ++mi) {
        const f32x4_t v = acc.v[mi][ni];
        const uint2 w = make_uint2(bf16_pair(v[0], v[1]), bf16_pair(v[2], v[3]));
        *reinterpret_cast<uint2*>(ew + (lane & 15) * kEpiPitch + mi * 32 + (lane >> 4) * 8) = w;
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int q = lane + 64 * h, row = q >> 3, c = q & 7;
        st16_stream(C + (int64_t)(ni * 16 + row) * p.N * 2 + c * 16, ld16(ew + row * kEpiPitch + c * 16));
      }
    }
    acc.zero();
    last_epi = s - 1;
  }
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
  const int64_t tiles = (int64_t)p.E * p.tiles_m * p.tiles_n;
  if (tiles <= 0) return hipSuccess;
  // one persistent workgroup per CU (its LDS admits no second), a whole
  // number per XCD
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int64_t grid = std::min<int64_t>(pad8(tiles), std::max(8, cus / 8 * 8));
  wgrad_kernel<<<(int)grid, WgradTile::THREADS, 0, s>>>(p, p.offsets, p.counts);
  return hipGetLastError();
}

}  // namespace moe
