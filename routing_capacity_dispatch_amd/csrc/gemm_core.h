// bf16 MFMA GEMM core for gfx950: C = A * B^T, A [M][K] and B [N][K] both
// contiguous along K (weights are stored [out, in]).
//
// Tile BM x BN per workgroup of WGM x WGN wavefronts, each wavefront owning a
// (BM/WGM) x (BN/WGN) sub-tile as 16x16 blocks of v_mfma_f32_16x16x32_bf16.
// Eight wavefronts (two per SIMD) keep the matrix cores busy while the other
// wavefront of the SIMD waits on LDS.  K advances in tiles of 64 bf16 (128
// bytes per tile row).  Operand tiles go straight from global memory into
// LDS with global_load_lds_dwordx4 (no VGPR round trip): one instruction
// moves 8 tile rows (1 KiB), lane l writing the 16 bytes at LDS offset 16 l.
// Rows keep an XOR swizzle of their 16-byte chunks (physical chunk = logical
// chunk ^ (row & 7)), so lane l of an instruction loads logical chunk
// (l & 7) ^ (l >> 3) of row l >> 3, and the fragment reads (16 rows, one
// chunk each) hit 8 distinct chunk positions.  NS LDS stages: the loads of
// the next NS-1 tiles are in flight while one tile feeds the MFMAs (B may
// take one stage more than A).
//
// Row sources are per-lane offsets from per-instruction wave-uniform bases,
// so the same mainloop serves dense operands, rows gathered through an index
// list and interleaved gate/up weight rows.
#pragma once

#include "common.h"

namespace moe {
namespace core {

#define MOE_LDS __attribute__((address_space(3)))

// BK_: bf16 of K per tile (32 or 64: tile rows of 64 or 128 bytes);
// NS_: LDS stages of A (NS - 1 tiles in flight while one feeds the MFMAs);
// NSB_: LDS stages of B, either NS or NS + 1 (B, the weights, then loads one
// tile further ahead: it is the operand that streams from HBM).
template <int BM_, int BN_, int WGM_, int WGN_, int BK_ = 64, int NS_ = 2, int NSB_ = NS_>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, WGM = WGM_, WGN = WGN_, BK = BK_, NS = NS_, NSB = NSB_;
  static constexpr int RB = BK * 2;                    // bytes per tile row
  static constexpr int CPR = RB / 16;                  // 16-byte chunks per row
  static constexpr int RPI = 1024 / RB;                // rows per load instruction
  static constexpr int KS = BK / 32;                   // MFMA K sub-steps per tile
  static constexpr int NW = WGM * WGN;                 // wavefronts
  static constexpr int THREADS = 64 * NW;
  static constexpr int WM = BM / WGM, WN = BN / WGN;   // wavefront sub-tile
  static constexpr int MI = WM / 16, NI = WN / 16;     // 16x16 blocks per wavefront
  static constexpr int A_INS = BM / (RPI * NW);        // load instructions per wavefront per K tile
  static constexpr int B_INS = BN / (RPI * NW);
  static constexpr int A_BYTES = BM * RB;
  static constexpr int B_BYTES = BN * RB;
  static constexpr int B_BASE = NS * A_BYTES;  // B stages follow the A stages
  static constexpr int MAIN_LDS = NS * A_BYTES + NSB * B_BYTES;
  static_assert(BK == 32 || BK == 64, "K tile of 32 or 64");
  static_assert(NS >= 2 && NS <= 5, "2 to 5 stages");
  static_assert(NSB == NS || (NS == 2 && (NSB == 3 || (NSB == 4 && BK == 32))),
                "B stages: NS, or 3 with 2 A stages (4 with K tiles of 32)");
  static_assert(BM % (RPI * NW) == 0 && BN % (RPI * NW) == 0, "tile rows come in whole loads per wavefront");
  static_assert(WM % 16 == 0 && WN % 16 == 0, "wavefront sub-tiles are whole 16x16 blocks");
  // chunk swizzle of row r: XOR applied to the 16-byte chunk index, chosen so
  // that 8 consecutive rows read at one logical chunk hit 8 distinct 16-byte
  // positions of a 128-byte bank line
  __device__ __forceinline__ static int swz(int r) { return RB == 128 ? (r & 7) : ((r >> 1) & 3); }
};

// Tile row that lane `lane` of wavefront `wave` loads with instruction i.
template <class TL>
__device__ __forceinline__ int load_row(int i, int wave, int lane) {
  return (i * TL::NW + wave) * TL::RPI + lane / TL::CPR;
}
// Byte offset inside that row: the logical chunk whose physical position is
// this lane's slot (instruction base rows are multiples of RPI, so the row's
// swizzle depends on the lane only).
template <class TL>
__device__ __forceinline__ int load_col(int lane) {
  return ((lane % TL::CPR) ^ TL::swz(lane / TL::CPR)) << 4;
}

// A wave-uniform pointer, held in scalar registers.
__device__ __forceinline__ const char* uniform_ptr(const char* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<const char*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Row sources of one operand tile: load instruction i of a wavefront reads
// from base[i] (wave-uniform, scalar registers) + off[i] (per lane, 32-bit),
// so an operand buffer addressed from one base must stay below 4 GiB.
template <int N>
struct RowSrc {
  const char* base[N];
  uint32_t off[N];
};

// One 16-byte-per-lane global -> LDS load: lane l's 16 bytes land at
// lds_wave_base + 16 l.  Written as inline assembly so the compiler does not
// make every later LDS read wait for it; the mainloop waits explicitly
// (s_waitcnt vmcnt(n) + barrier) before reading a stage.
__device__ __forceinline__ void lds_load16(const char* sbase, uint32_t voff, char* lds_wave_base) {
  const uint32_t l = __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((MOE_LDS char*)lds_wave_base)));
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(l), "v"(voff), "s"(sbase)
               : "memory", "m0");
}

template <class TL>
struct Acc {
  f32x4_t v[TL::MI][TL::NI];
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < TL::MI; ++i)
#pragma unroll
      for (int j = 0; j < TL::NI; ++j) v[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
};

// Address of K tile j of a row source: tiles follow one another at `kstep`
// bytes from the source's base (every operand but the split output
// projection's weights, whose K ranges sit in separate arrays).
struct LinearK {
  static constexpr bool kLinear = true;
  __device__ __forceinline__ const char* operator()(const char* base, int j, int64_t kstep) const {
    return base + j * kstep;
  }
};

// Issue the loads of one K tile of A or B into one stage: row sources
// advanced by `koff` bytes (wave-uniform).
template <class TL, int N>
__device__ __forceinline__ void issue_rows(const RowSrc<N>& src, int64_t koff, char* stage, int wave) {
#pragma unroll
  for (int i = 0; i < N; ++i) lds_load16(src.base[i] + koff, src.off[i], stage + (i * TL::NW + wave) * 1024);
}

// MFMAs of one staged K tile: fragments of K sub-step 0 are read first; the
// reads of sub-step 1 (64-wide K tiles) are interleaved with the MFMAs of
// sub-step 0.
template <class TL>
__device__ __forceinline__ void compute_tile(const char* sa, const char* sb, Acc<TL>& acc, int wm, int wn,
                                             int lane) {
  const char* a = sa + (wm * TL::WM + (lane & 15)) * TL::RB;
  const char* b = sb + (wn * TL::WN + (lane & 15)) * TL::RB;
  const int sw = TL::swz(lane & 15);
  uint4 fa[TL::KS][TL::MI], fb[TL::KS][TL::NI];
#pragma unroll
  for (int ks = 0; ks < TL::KS; ++ks) {
    const int off = ((ks * 4 + (lane >> 4)) ^ sw) << 4;
#pragma unroll
    for (int mi = 0; mi < TL::MI; ++mi) fa[ks][mi] = ld16(a + mi * 16 * TL::RB + off);
#pragma unroll
    for (int ni = 0; ni < TL::NI; ++ni) fb[ks][ni] = ld16(b + ni * 16 * TL::RB + off);
  }
#pragma unroll
  for (int ks = 0; ks < TL::KS; ++ks)
#pragma unroll
    for (int mi = 0; mi < TL::MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < TL::NI; ++ni)
        acc.v[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8_t, fa[ks][mi]), __builtin_bit_cast(bf16x8_t, fb[ks][ni]), acc.v[mi][ni], 0, 0,
            0);
  constexpr int NR = TL::MI + TL::NI;
  constexpr int NM = TL::MI * TL::NI;
  __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
  if (TL::KS == 2) {
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, NM / NR, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  }
  __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);
}

// Fragments of one 32-wide K sub-step of a staged tile.
template <class TL>
struct Frags {
  uint4 a[TL::MI];
  uint4 b[TL::NI];
};

// ---- K-major operands --------------------------------------------------
// The backward of the routed experts contracts weights along their output
// dimension (dgrad) and activations along their rows (wgrad): such an
// operand is stored K-major, rows along K with the M (or N) index
// contiguous.  Its K tile is staged in LDS as it lies in memory, 64 k-rows
// of X bf16, and turned into MFMA fragments on the way out of LDS by
// ds_read_b64_tr_b16, which transposes 16-bit elements across the lanes of
// each group of 16.
//
// Lane layout of ds_read_b64_tr_b16 (read off the device with an in-bounds
// probe): within each group of 16 lanes, lane i receives, as its 4 results
// j = 0..3, element (i & 3) of the 4 consecutive elements addressed by lane
// 4 j + (i >> 2) of its group.  So if lane 4 j + q of group g addresses k-row
// 8 g + 4 h + j at column x0 + 4 q, lane i gets column x0 + i of k-rows
// 8 g + 4 h + 0..3: two such reads (h = 0, 1) give the 8 consecutive k of
// one v_mfma_f32_16x16x32_bf16 operand row, the registers a row-major
// fragment read yields.
//
// LDS layout of a K-major tile: k-row k at k * 2X bytes, its 16-byte chunks
// XOR-swizzled by swz(k), so that the 16 k-rows one read touches land on
// distinct chunk positions (2 LDS cycles per read at 256 bytes a cycle; the
// profiled SQ_LDS_BANK_CONFLICT is 0).
typedef short i16x4_t __attribute__((ext_vector_type(4)));

template <int X>
struct KMajor {
  static_assert(X == 128 || X == 256, "K-major tiles are 128 or 256 wide");
  static constexpr int RB = 2 * X;        // bytes per k-row
  static constexpr int CPR = RB / 16;     // 16-byte chunks per k-row
  static constexpr int RPI = 1024 / RB;   // k-rows per load instruction
  // distinct over k & 3 and bits 3.. of k for the 16 k-rows 8 g + 4 h + j
  // (g < 4, j < 4) of one transposed read
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
// tile at st.
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

// Fragment r of sub-step ks (r < MI: A block r; else B block r - MI), each
// operand row-major (the Tile layout) or K-major (AK / BK; X = BM or BN).
template <class TL, bool AK, bool BK>
__device__ __forceinline__ uint4 frag(const char* sa, const char* sb, int ks, int r, int wm, int wn, int lane) {
  const int off = ((ks * 4 + (lane >> 4)) ^ TL::swz(lane & 15)) << 4;
  if (r < TL::MI) {
    if constexpr (AK) return kfrag<TL::BM>(sa, wm * TL::WM + r * 16, ks, lane);
    return ld16(sa + (wm * TL::WM + (lane & 15)) * TL::RB + r * 16 * TL::RB + off);
  }
  const int n = r - TL::MI;
  if constexpr (BK) return kfrag<TL::BN>(sb, wn * TL::WN + n * 16, ks, lane);
  return ld16(sb + (wn * TL::WN + (lane & 15)) * TL::RB + n * 16 * TL::RB + off);
}

// LDS read instructions of one sub-step's fragments (a K-major one takes two).
template <class TL, bool AK, bool BK>
constexpr int frag_reads() {
  return (AK ? 2 : 1) * TL::MI + (BK ? 2 : 1) * TL::NI;
}

template <class TL, bool AK = false, bool BK = false>
__device__ __forceinline__ void read_frags(const char* sa, const char* sb, int ks, Frags<TL>& f, int wm, int wn,
                                           int lane) {
  if constexpr (!AK && !BK) {
    const char* a = sa + (wm * TL::WM + (lane & 15)) * TL::RB;
    const char* b = sb + (wn * TL::WN + (lane & 15)) * TL::RB;
    const int off = ((ks * 4 + (lane >> 4)) ^ TL::swz(lane & 15)) << 4;
#pragma unroll
    for (int mi = 0; mi < TL::MI; ++mi) f.a[mi] = ld16(a + mi * 16 * TL::RB + off);
#pragma unroll
    for (int ni = 0; ni < TL::NI; ++ni) f.b[ni] = ld16(b + ni * 16 * TL::RB + off);
  } else {
#pragma unroll
    for (int mi = 0; mi < TL::MI; ++mi) f.a[mi] = frag<TL, AK, BK>(sa, sb, ks, mi, wm, wn, lane);
#pragma unroll
    for (int ni = 0; ni < TL::NI; ++ni) f.b[ni] = frag<TL, AK, BK>(sa, sb, ks, TL::MI + ni, wm, wn, lane);
  }
}

template <class TL>
__device__ __forceinline__ void mfma_frags(const Frags<TL>& f, Acc<TL>& acc) {
#pragma unroll
  for (int mi = 0; mi < TL::MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < TL::NI; ++ni)
      acc.v[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          __builtin_bit_cast(bf16x8_t, f.a[mi]), __builtin_bit_cast(bf16x8_t, f.b[ni]), acc.v[mi][ni], 0, 0, 0);
}

// MFMAs on `cur` with the reads of `nxt` (sub-step ks of the staged tile at
// sa, sb) interleaved among them.
template <class TL, bool AK = false, bool BK = false>
__device__ __forceinline__ void mfma_and_read(const Frags<TL>& cur, Acc<TL>& acc, const char* sa, const char* sb,
                                              int ks, Frags<TL>& nxt, int wm, int wn, int lane) {
  read_frags<TL, AK, BK>(sa, sb, ks, nxt, wm, wn, lane);
  mfma_frags<TL>(cur, acc);
  constexpr int NR = frag_reads<TL, AK, BK>();
  constexpr int NM = TL::MI * TL::NI;
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, NM / NR, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, NM - (NM / NR) * NR, 0);
}

// MFMAs on `cur` and the reads of `nxt` (sub-step ks of the staged tile at
// sa, sb), with P load instructions issue(0) .. issue(P-1) spread among them:
// the loads of a workgroup then reach the memory pipeline over the whole
// phase instead of in one burst that holds up the MFMAs queued behind it.
// Each load sits between two fragment reads in program order (the inline
// assembly is a memory barrier to the compiler), and the reads are
// interleaved with the MFMAs.
template <class TL, int P, bool AK = false, bool BK = false, class F>
__device__ __forceinline__ void mfma_read_issue(const Frags<TL>& cur, Acc<TL>& acc, const char* sa, const char* sb,
                                                int ks, Frags<TL>& nxt, int wm, int wn, int lane, F&& issue) {
  constexpr int NF = TL::MI + TL::NI, NR = frag_reads<TL, AK, BK>(), NM = TL::MI * TL::NI;
  const char* a = sa + (wm * TL::WM + (lane & 15)) * TL::RB;
  const char* b = sb + (wn * TL::WN + (lane & 15)) * TL::RB;
  const int off = ((ks * 4 + (lane >> 4)) ^ TL::swz(lane & 15)) << 4;
#pragma unroll
  for (int r = 0; r < NF; ++r) {
    if constexpr (!AK && !BK) {
      if (r < TL::MI)
        nxt.a[r] = ld16(a + r * 16 * TL::RB + off);
      else
        nxt.b[r - TL::MI] = ld16(b + (r - TL::MI) * 16 * TL::RB + off);
    } else {
      const uint4 v = frag<TL, AK, BK>(sa, sb, ks, r, wm, wn, lane);
      if (r < TL::MI)
        nxt.a[r] = v;
      else
        nxt.b[r - TL::MI] = v;
    }
    // loads s with floor(s * NF / P) == r follow fragment r
#pragma unroll
    for (int s = 0; s < P; ++s)
      if (s * NF / P == r) issue(s);
  }
  mfma_frags<TL>(cur, acc);
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, NM / NR, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, NM - (NM / NR) * NR, 0);
}

// Wavefront priority (s_setprio), pinned between the instructions around it.
template <int prio>
__device__ __forceinline__ void set_prio() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(prio);
  __builtin_amdgcn_sched_barrier(0);
}

// Wait until at most n load instructions of this wavefront are in flight,
// then synchronise the workgroup.
template <int n>
__device__ __forceinline__ void wait_loads() {
  __builtin_amdgcn_sched_barrier(0);
  if (n == 0)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(n) : "memory");
  __syncthreads();
  __builtin_amdgcn_sched_barrier(0);
}

// Accumulate K range [0, ktiles * BK) into acc.  With NS stages of A and B,
// tiles kt+1 .. kt+NS-1 are in flight while tile kt is consumed; with 2 A
// stages and NSB B stages, A(kt+1) and B(kt+1) .. B(kt+NSB-1) are.  Loads return in
// issue order, so waiting until at most n load instructions of a wavefront
// are outstanding means all but its last n have landed.  Ends with a barrier
// so the caller may reuse the LDS.
//
// a_kstep / b_kstep: bytes between consecutive K tiles of one row source (the
// tile row width for row-major operands; a whole packed tile for operands
// stored tile by tile).
// kSplit selects the mid-tile barrier schedule (64-wide K tiles, 2 A
// stages); it holds two fragment sets live, so kernels short of registers
// take the plain schedule.
// bp maps (B base, K tile index, b_kstep) to the tile's address; only the
// split schedule takes a policy other than LinearK.
template <class TL, bool kSplit = true, bool AK = false, bool BK = false, class BP = LinearK>
__device__ __forceinline__ void mainloop(const RowSrc<TL::A_INS>& a_src, const RowSrc<TL::B_INS>& b_src,
                                         int ktiles, char* lds,
                                         Acc<TL>& acc, int64_t a_kstep = TL::RB, int64_t b_kstep = TL::RB,
                                         BP bp = BP()) {
  static_assert(BP::kLinear || (kSplit && TL::KS == 2 && TL::NS == 2), "B tile policy needs the split schedule");
  constexpr int P = TL::A_INS + TL::B_INS;  // load instructions per tile per wavefront
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / TL::WGN, wn = wave % TL::WGN;
  char* lds_a = lds;
  char* lds_b = lds + TL::B_BASE;
  if (ktiles <= 0) return;
  if constexpr (kSplit && TL::KS == 2 && TL::NS == 2) {
    // One barrier per K tile, in the middle of it: the second half's MFMAs
    // (fragments already in registers) cover the reads of the next tile's
    // first half, so no wavefront waits on LDS after the barrier.
    //   phase 1: MFMAs of (kt, first half)  | reads of (kt, second half)
    //   phase 2: wait for tile kt+1, barrier (every read of tile kt done)
    //   phase 3: loads of A(kt+2) and B(kt+NSB) into tile kt's stages;
    //            MFMAs of (kt, second half) | reads of (kt+1, first half)
    // Issue order: A0 B0 A1 B1 [B2] | A2 B(NSB) | A3 B(NSB+1) | ...
    constexpr int PB = TL::B_INS;
    constexpr int DB = TL::NSB - 1;  // B tiles issued ahead
    // B tile j into a stage (LinearK: the row sources advanced j K steps)
    auto issue_b = [&](int j, char* stage) {
#pragma unroll
      for (int i = 0; i < TL::B_INS; ++i)
        lds_load16(bp(b_src.base[i], j, b_kstep), b_src.off[i], stage + (i * TL::NW + wave) * 1024);
    };
    if constexpr (BP::kLinear) {
      issue_rows<TL>(a_src, 0, lds_a, wave);
      issue_rows<TL>(b_src, 0, lds_b, wave);
      if (ktiles > 1) {
        issue_rows<TL>(a_src, a_kstep, lds_a + TL::A_BYTES, wave);
        issue_rows<TL>(b_src, b_kstep, lds_b + TL::B_BYTES, wave);
      }
      if (DB == 2 && ktiles > 2) issue_rows<TL>(b_src, 2 * b_kstep, lds_b + 2 * TL::B_BYTES, wave);
    } else {
      issue_rows<TL>(a_src, 0, lds_a, wave);
      issue_b(0, lds_b);
      if (ktiles > 1) {
        issue_rows<TL>(a_src, a_kstep, lds_a + TL::A_BYTES, wave);
        issue_b(1, lds_b + TL::B_BYTES);
      }
      if (DB == 2 && ktiles > 2) issue_b(2, lds_b + 2 * TL::B_BYTES);
    }
    if (DB == 2 && ktiles > 2)
      wait_loads<P + PB>();
    else if (ktiles > 1)
      wait_loads<P>();
    else
      wait_loads<0>();
    Frags<TL> f0, f1;
    read_frags<TL, AK, BK>(lds_a, lds_b, 0, f0, wm, wn, lane);
    int sb = 0;  // B stage of tile kt
    int kt = 0;
    // every load of the iteration is in range: A(kt+2), B(kt+NSB), issued
    // among the second half's MFMAs.  Each loop body is straight-line, so
    // the accumulators stay in place across iterations.
    for (; kt + TL::NSB < ktiles; ++kt) {
      int sb1 = sb + 1;
      if (sb1 == TL::NSB) sb1 = 0;
      mfma_and_read<TL, AK, BK>(f0, acc, lds_a + (kt & 1) * TL::A_BYTES, lds_b + sb * TL::B_BYTES, 1, f1, wm, wn, lane);
      // landed: A(kt+1), B(kt+1); may still fly: B(kt+2) when B runs 2 ahead
      if (DB == 2)
        wait_loads<PB>();
      else
        wait_loads<0>();
      // phase 3 runs at raised wave priority: the SIMD then prefers the
      // wavefront that has passed the barrier and holds MFMA work over one
      // still waiting for its loads (measured: 1-2 % on the dense split-
      // schedule GEMMs, neutral on the grouped expert GEMMs)
      set_prio<1>();
      // tile kt's stages are free: they take A(kt+2) and B(kt+NSB)
      const int64_t ka = (kt + 2) * a_kstep, kb = (kt + TL::NSB) * b_kstep;
      const int jb = kt + TL::NSB;
      char* da = lds_a + (kt & 1) * TL::A_BYTES + wave * 1024;
      char* db = lds_b + sb * TL::B_BYTES + wave * 1024;
      mfma_read_issue<TL, TL::A_INS + TL::B_INS, AK, BK>(
          f1, acc, lds_a + ((kt + 1) & 1) * TL::A_BYTES, lds_b + sb1 * TL::B_BYTES, 0, f0, wm, wn, lane, [&](int s) {
            if (s < TL::A_INS)
              lds_load16(a_src.base[s] + ka, a_src.off[s], da + s * TL::NW * 1024);
            else
              lds_load16(BP::kLinear ? b_src.base[s - TL::A_INS] + kb : bp(b_src.base[s - TL::A_INS], jb, b_kstep),
                         b_src.off[s - TL::A_INS],
                         db + (s - TL::A_INS) * TL::NW * 1024);
          });
      set_prio<0>();
      sb = sb1;
    }
    // the last NSB - 1 iterations: loads only while in range
    for (; kt + 1 < ktiles; ++kt) {
      int sb1 = sb + 1;
      if (sb1 == TL::NSB) sb1 = 0;
      mfma_and_read<TL, AK, BK>(f0, acc, lds_a + (kt & 1) * TL::A_BYTES, lds_b + sb * TL::B_BYTES, 1, f1, wm, wn, lane);
      if (DB == 2 && kt + 2 < ktiles)
        wait_loads<PB>();
      else
        wait_loads<0>();
      if (kt + 2 < ktiles) issue_rows<TL>(a_src, (kt + 2) * a_kstep, lds_a + (kt & 1) * TL::A_BYTES, wave);
      if (kt + TL::NSB < ktiles) {
        if constexpr (BP::kLinear)
          issue_rows<TL>(b_src, (kt + TL::NSB) * b_kstep, lds_b + sb * TL::B_BYTES, wave);
        else
          issue_b(kt + TL::NSB, lds_b + sb * TL::B_BYTES);
      }
      mfma_and_read<TL, AK, BK>(f1, acc, lds_a + ((kt + 1) & 1) * TL::A_BYTES, lds_b + sb1 * TL::B_BYTES, 0, f0, wm, wn,
                        lane);
      sb = sb1;
    }
    // the last tile: its second half read after the first half's MFMAs,
    // into the same registers (one fragment set live: with two, the
    // accumulators of kernels at the register limit spill here)
    const int kl = ktiles - 1;
    mfma_frags<TL>(f0, acc);
    read_frags<TL, AK, BK>(lds_a + (kl & 1) * TL::A_BYTES, lds_b + sb * TL::B_BYTES, 1, f0, wm, wn, lane);
    mfma_frags<TL>(f0, acc);
  } else if constexpr ((AK || BK) && TL::NSB == TL::NS && TL::NS == 2 && TL::KS == 2) {
    // K-major operands on the plain schedule: the loads of tile kt + 1
    // after the barrier that frees its stage, then tile kt's MFMAs with the
    // second half's fragment reads interleaved (fewer live registers than
    // the split schedule, whose two fragment sets would spill here)
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
      read_frags<TL, AK, BK>(sa, sb, 0, f0, wm, wn, lane);
      read_frags<TL, AK, BK>(sa, sb, 1, f1, wm, wn, lane);
      mfma_frags<TL>(f0, acc);
      mfma_frags<TL>(f1, acc);
      constexpr int NR = frag_reads<TL, AK, BK>();
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
  } else if constexpr (TL::NSB == TL::NS) {
    static_assert(!AK && !BK, "K-major operands: split schedule, or the plain one with 2 stages");
#pragma unroll
    for (int s = 0; s < TL::NS - 1; ++s)
      if (s < ktiles) {
        issue_rows<TL>(a_src, s * a_kstep, lds_a + s * TL::A_BYTES, wave);
        issue_rows<TL>(b_src, s * b_kstep, lds_b + s * TL::B_BYTES, wave);
      }
    int stage = 0;
    auto wait_tile = [&](int kt) {
      // tiles issued after tile kt: min(NS - 2, ktiles - 1 - kt)
      const int after = min(TL::NS - 2, ktiles - 1 - kt);
      if (TL::NS >= 5 && after >= 3)
        wait_loads<3 * P>();
      else if (TL::NS >= 4 && after >= 2)
        wait_loads<2 * P>();
      else if (TL::NS >= 3 && after >= 1)
        wait_loads<P>();
      else
        wait_loads<0>();
    };
    int kt = 0;
    if constexpr (TL::KS == 2) {
      // tile kt + NS - 1 exists: its loads go in among tile kt's MFMAs
      for (; kt + TL::NS - 1 < ktiles; ++kt) {
        wait_tile(kt);
        const int nxt = kt + TL::NS - 1;
        int ns = stage + TL::NS - 1;
        if (ns >= TL::NS) ns -= TL::NS;
        const int64_t ka = nxt * a_kstep, kb = nxt * b_kstep;
        char* da = lds_a + ns * TL::A_BYTES + wave * 1024;
        char* db = lds_b + ns * TL::B_BYTES + wave * 1024;
        const char* sa = lds_a + stage * TL::A_BYTES;
        const char* sb = lds_b + stage * TL::B_BYTES;
        Frags<TL> f0, f1;
        read_frags<TL>(sa, sb, 0, f0, wm, wn, lane);
        __builtin_amdgcn_sched_group_barrier(0x100, TL::MI + TL::NI, 0);
        mfma_read_issue<TL, P>(f0, acc, sa, sb, 1, f1, wm, wn, lane, [&](int s) {
          if (s < TL::A_INS)
            lds_load16(a_src.base[s] + ka, a_src.off[s], da + s * TL::NW * 1024);
          else
            lds_load16(b_src.base[s - TL::A_INS] + kb, b_src.off[s - TL::A_INS], db + (s - TL::A_INS) * TL::NW * 1024);
        });
        mfma_frags<TL>(f1, acc);
        __builtin_amdgcn_sched_group_barrier(0x008, TL::MI * TL::NI, 0);
        if (++stage == TL::NS) stage = 0;
      }
    }
    for (; kt < ktiles; ++kt) {
      wait_tile(kt);
      const int nxt = kt + TL::NS - 1;
      if (nxt < ktiles) {
        int ns = stage + TL::NS - 1;
        if (ns >= TL::NS) ns -= TL::NS;
        issue_rows<TL>(a_src, nxt * a_kstep, lds_a + ns * TL::A_BYTES, wave);
        issue_rows<TL>(b_src, nxt * b_kstep, lds_b + ns * TL::B_BYTES, wave);
      }
      compute_tile<TL>(lds_a + stage * TL::A_BYTES, lds_b + stage * TL::B_BYTES, acc, wm, wn, lane);
      if (++stage == TL::NS) stage = 0;
    }
  } else {
    static_assert(!AK && !BK, "K-major operands: split schedule, or the plain one with 2 stages");
    // 2 A stages (A one tile ahead), NSB B stages (B DB = NSB - 1 tiles
    // ahead).  Issue order: B0 A0 B1 .. B(DB-1) | A1 B(DB) | A2 B(DB+1) | ...
    // At the top of iteration kt >= 1 the last loads issued are A(kt) then
    // B(kt-1+DB), and B(kt) came before A(kt): both have landed once at most
    // the B loads after A(kt) are pending.
    constexpr int PB = TL::B_INS;
    constexpr int DB = TL::NSB - 1;
    issue_rows<TL>(b_src, 0, lds_b, wave);
    issue_rows<TL>(a_src, 0, lds_a, wave);
#pragma unroll
    for (int j = 1; j < DB; ++j)
      if (j < ktiles) issue_rows<TL>(b_src, j * b_kstep, lds_b + j * TL::B_BYTES, wave);
    int sb = 0;  // B stage of tile kt
    for (int kt = 0; kt < ktiles; ++kt) {
      if (kt == 0) {
        const int pend = min(DB - 1, ktiles - 1);  // B(1) .. B(DB-1) after A(0)
        if (DB >= 3 && pend >= 2)
          wait_loads<2 * PB>();
        else if (pend >= 1)
          wait_loads<PB>();
        else
          wait_loads<0>();
      } else if (kt - 1 + DB < ktiles) {
        wait_loads<PB>();
      } else {
        wait_loads<0>();
      }
      if (kt + 1 < ktiles)
        issue_rows<TL>(a_src, (kt + 1) * a_kstep, lds_a + ((kt + 1) & 1) * TL::A_BYTES, wave);
      if (kt + DB < ktiles) {
        int s2 = sb + DB;  // (kt + DB) % NSB
        if (s2 >= TL::NSB) s2 -= TL::NSB;
        issue_rows<TL>(b_src, (kt + DB) * b_kstep, lds_b + s2 * TL::B_BYTES, wave);
      }
      compute_tile<TL>(lds_a + (kt & 1) * TL::A_BYTES, lds_b + sb * TL::B_BYTES, acc, wm, wn, lane);
      if (++sb == TL::NSB) sb = 0;
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();
}

// A wavefront's view of tile TL that computes only its first MIe 16-row
// blocks (every other constant, the loads and the LDS layout unchanged).
template <class TL, int MIe>
struct RowBlocks : TL {
  static_assert(MIe >= 1 && MIe <= TL::MI, "1 .. MI row blocks");
  static constexpr int MI = MIe;
};

// f(RowBlocks<TL, m>{}) with m = clamp(mie, 1, TL::MI): one compile-time
// variant per row-block count, chosen once per tile (mie wave-uniform).
template <class TL, int M = TL::MI, class F>
__device__ __forceinline__ void with_row_blocks(int mie, F&& f) {
  if constexpr (M == 1)
    f(RowBlocks<TL, 1>{});
  else if (mie >= M)
    f(RowBlocks<TL, M>{});
  else
    with_row_blocks<TL, M - 1>(mie, f);
}

// Tile coordinates of register r of block (mi, ni) for this lane.
template <class TL>
__device__ __forceinline__ int acc_row(int wm, int mi, int lane, int r) {
  return wm * TL::WM + mi * 16 + (lane >> 4) * 4 + r;
}
template <class TL>
__device__ __forceinline__ int acc_col(int wn, int ni, int lane) {
  return wn * TL::WN + ni * 16 + (lane & 15);
}

}  // namespace core
}  // namespace moe
