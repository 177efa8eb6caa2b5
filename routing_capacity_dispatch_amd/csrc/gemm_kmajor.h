// K-major operands for the gfx950 bf16 GEMM core (gemm_core.h).
//
// The forward contractions read both operands along their contiguous
// dimension.  The backward of the routed experts contracts weights along
// their output dimension (dgrad: dh = do W_d, du = da W_g + db W_u) and
// activations along their row dimension (wgrad: dW = do^T h, da^T u): such
// an operand is stored K-major, rows along K with the M (or N) index
// contiguous.  A K tile of it is staged in LDS as it lies in memory, 64
// k-rows of X bf16, and turned into MFMA fragments on the way out of LDS by
// ds_read_b64_tr_b16, which transposes 16-bit elements across the lanes of
// each group of 16.
//
// Lane layout of ds_read_b64_tr_b16 (checked on the device): within each
// group of 16 lanes, lane i receives, as its 4 results j = 0..3, element
// (i & 3) of the 4 consecutive elements addressed by lane 4 j + (i >> 2) of
// its group.  So if lane 4 j + q of group g addresses k-row 8 g + 4 h + j at
// column x0 + 4 q, lane i gets column x0 + i of k-rows 8 g + 4 h + 0..3:
// two such reads (h = 0, 1) give the 8 consecutive k of one MFMA operand
// row of v_mfma_f32_16x16x32_bf16, the same registers a row-major read
// yields.
//
// LDS layout of a K-major tile: k-row k at k * 2X bytes, its 16-byte chunks
// XOR-swizzled by kswz(k), so that the 16 k-rows one read touches land on
// distinct chunk positions (2 LDS cycles per read at 256 bytes a cycle).
#pragma once

#include "gemm_core.h"

namespace moe {
namespace core {

typedef short i16x4_t __attribute__((ext_vector_type(4)));

template <int X>
struct KMajor {
  static_assert(X == 128 || X == 256, "K-major tiles are 128 or 256 wide");
  static constexpr int RB = 2 * X;        // bytes per k-row
  static constexpr int CPR = RB / 16;     // 16-byte chunks per k-row
  static constexpr int RPI = 1024 / RB;   // k-rows per load instruction
  // the chunk XOR of k-row k: distinct over k & 3 and bits 3.. of k for the
  // 16 k-rows 8 g + 4 h + j (g < 4, j < 4) of one transposed read
  __device__ __forceinline__ static int swz(int k) {
    return X == 256 ? (((k & 3) | (((k >> 3) & 3) << 2)) << 1) : (((k & 3) | (((k >> 3) & 1) << 2)) << 1);
  }
};

// K-row that lane `lane` of wavefront `wave` loads with instruction i, and
// the byte offset of the logical chunk it fetches (its LDS slot is 16 lane).
template <class TL, int X>
__device__ __forceinline__ int kload_row(int i, int wave, int lane) {
  return (i * TL::NW + wave) * KMajor<X>::RPI + lane / KMajor<X>::CPR;
}
template <int X>
__device__ __forceinline__ int kload_col(int krow, int lane) {
  return ((lane % KMajor<X>::CPR) ^ KMajor<X>::swz(krow)) << 4;
}

// One MFMA operand (16 columns from xb, K sub-step ks of 32) of a K-major
// tile at st: the registers a row-major fragment read would give.
template <int X>
__device__ __forceinline__ uint4 kfrag(const char* st, int xb, int ks, int lane) {
  const int g = (lane >> 4) & 3, j = (lane >> 2) & 3, q = lane & 3;
  const int sw = KMajor<X>::swz(8 * g + j);  // the same for both halves and every ks
  const int c = ((xb >> 3) + (q >> 1)) ^ sw;
  const char* p = st + (ks * 32 + 8 * g + j) * KMajor<X>::RB + (c << 4) + (q & 1) * 8;
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MOE_LDS i16x4_t*)p);
  const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MOE_LDS i16x4_t*)(p + 4 * KMajor<X>::RB));
  const uint2 l = __builtin_bit_cast(uint2, lo), h = __builtin_bit_cast(uint2, hi);
  return make_uint4(l.x, l.y, h.x, h.y);
}

// Fragments of K sub-step ks: A and B each row-major (the Tile layout) or
// K-major (X = BM for A, BN for B).
template <class TL, bool AK, bool BK>
__device__ __forceinline__ void read_frags_t(const char* sa, const char* sb, int ks, Frags<TL>& f, int wm, int wn,
                                             int lane) {
  if constexpr (AK) {
#pragma unroll
    for (int mi = 0; mi < TL::MI; ++mi) f.a[mi] = kfrag<TL::BM>(sa, wm * TL::WM + mi * 16, ks, lane);
  } else {
    const char* a = sa + (wm * TL::WM + (lane & 15)) * TL::RB;
    const int off = ((ks * 4 + (lane >> 4)) ^ TL::swz(lane & 15)) << 4;
#pragma unroll
    for (int mi = 0; mi < TL::MI; ++mi) f.a[mi] = ld16(a + mi * 16 * TL::RB + off);
  }
  if constexpr (BK) {
#pragma unroll
    for (int ni = 0; ni < TL::NI; ++ni) f.b[ni] = kfrag<TL::BN>(sb, wn * TL::WN + ni * 16, ks, lane);
  } else {
    const char* b = sb + (wn * TL::WN + (lane & 15)) * TL::RB;
    const int off = ((ks * 4 + (lane >> 4)) ^ TL::swz(lane & 15)) << 4;
#pragma unroll
    for (int ni = 0; ni < TL::NI; ++ni) f.b[ni] = ld16(b + ni * 16 * TL::RB + off);
  }
}

// Accumulate K range [0, ktiles * 64) with operands in either layout: two
// LDS stages, the loads of tile kt + 1 issued after the barrier that frees
// its stage, then tile kt's MFMAs with the second half's fragment reads
// interleaved.  A row source advances by a_kstep / b_kstep bytes per K tile
// (128 for a row-major operand; 64 k-rows for a K-major one).  Ends with a
// barrier so the caller may reuse the LDS.  (Spreading the loads among the
// MFMAs, as the forward's core does, measured slower here.)
template <class TL, bool AK, bool BK>
__device__ __forceinline__ void mainloop_t(const RowSrc<TL::A_INS>& a_src, const RowSrc<TL::B_INS>& b_src,
                                           int ktiles, char* lds, Acc<TL>& acc, int64_t a_kstep,
                                           int64_t b_kstep) {
  static_assert(TL::NS == 2 && TL::NSB == 2 && TL::KS == 2, "two stages of 64-wide K tiles");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / TL::WGN, wn = wave % TL::WGN;
  char* lds_a = lds;
  char* lds_b = lds + TL::B_BASE;
  if (ktiles > 0) {
    issue_rows<TL>(a_src, 0, lds_a, wave);
    issue_rows<TL>(b_src, 0, lds_b, wave);
  }
  for (int kt = 0; kt < ktiles; ++kt) {
    wait_loads<0>();
    const int st = kt & 1;
    if (kt + 1 < ktiles) {
      issue_rows<TL>(a_src, (kt + 1) * a_kstep, lds_a + (st ^ 1) * TL::A_BYTES, wave);
      issue_rows<TL>(b_src, (kt + 1) * b_kstep, lds_b + (st ^ 1) * TL::B_BYTES, wave);
    }
    const char* sa = lds_a + st * TL::A_BYTES;
    const char* sb = lds_b + st * TL::B_BYTES;
    Frags<TL> f0, f1;
    read_frags_t<TL, AK, BK>(sa, sb, 0, f0, wm, wn, lane);
    read_frags_t<TL, AK, BK>(sa, sb, 1, f1, wm, wn, lane);
    mfma_frags<TL>(f0, acc);
    mfma_frags<TL>(f1, acc);
    // LDS read instructions per sub-step: a K-major fragment takes two
    constexpr int NR = (AK ? 2 : 1) * TL::MI + (BK ? 2 : 1) * TL::NI;
    constexpr int NM = TL::MI * TL::NI;
    __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, NM / NR, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, NM - (NM / NR) * NR, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();
}

}  // namespace core
}  // namespace moe
