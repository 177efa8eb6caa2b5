// MFMA GEMMs of the MoE branch for gfx950: the fp32 paths and the router
// GEMM (bf16 in, fp32 logits out).  bf16 -> bf16 contractions go to the
// gfx950 core in gemm_bf16.hip.
//
// Every contraction here is C = A * B^T with both operands contiguous along
// K (weights are stored [out, in]).  One workgroup of 4 wavefronts computes a
// 128x128 output tile; each wavefront owns a 64x64 quadrant as 4x4 MFMA
// 16x16 blocks.  K advances in tiles of 128 bytes per row (64 bf16 or
// 32 fp32): global -> registers -> LDS (double-buffered, XOR-swizzled 16-byte
// chunks), then LDS -> registers -> MFMA.  bf16 uses
// v_mfma_f32_16x16x32_bf16 (8 bf16 of K per lane), fp32 uses four
// v_mfma_f32_16x16x4_f32 per 16-byte chunk.  Within a 16-byte chunk the two
// operands use the same K order, so the K permutation inside an MFMA is
// immaterial.  The epilogue stages the tile through LDS and writes whole
// 16-byte chunks of output rows, which lets the same code gather input rows
// and scatter output rows through index lists.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int BM = 128;
constexpr int BN = 128;
constexpr int BKB = 128;                // bytes of K per tile row
constexpr int NTHR = 256;
constexpr int TILE_B = BM * BKB;        // 16 KiB per operand tile
constexpr int LDS_MAIN = 4 * TILE_B;    // A, B x 2 buffers
constexpr int STAGE_PAD = 16;
constexpr int LDS_BYTES = BM * (BN * 4 + STAGE_PAD);  // >= LDS_MAIN, fp32 staging

static_assert(LDS_BYTES >= LDS_MAIN, "staging must cover the main loop");

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * BKB + ((chunk ^ (row & 7)) << 4);
}

template <typename T>
struct Mma;

template <>
struct Mma<bf16_t> {
  __device__ __forceinline__ static void run(const uint4& a, const uint4& b, f32x4_t& c) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
};

template <>
struct Mma<float> {
  __device__ __forceinline__ static void run(const uint4& a, const uint4& b, f32x4_t& c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
  }
};

// Accumulate one K range.  a_src[i] / b_src[i] point at the 16-byte chunk
// this thread loads for tile rows (tid/8 + 32 i), at the first K tile.
// Ends with a barrier, so the caller may reuse the LDS afterwards.
template <typename T>
__device__ __forceinline__ void mainloop(const char* const (&a_src)[4], const char* const (&b_src)[4],
                                         int ktiles, char* lds, f32x4_t (&acc)[4][4]) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lrow = tid >> 3, lchunk = tid & 7;
  char* sA = lds;
  char* sB = lds + 2 * TILE_B;
  uint4 ra[4], rb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ra[i] = ld16(a_src[i]);
    rb[i] = ld16(b_src[i]);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    st16(sA + swz(lrow + 32 * i, lchunk), ra[i]);
    st16(sB + swz(lrow + 32 * i, lchunk), rb[i]);
  }
  __syncthreads();
  for (int kt = 0; kt < ktiles; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < ktiles;
    if (more) {
      const int off = (kt + 1) * BKB;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ra[i] = ld16(a_src[i] + off);
        rb[i] = ld16(b_src[i] + off);
      }
    }
    const char* a = sA + cur * TILE_B;
    const char* b = sB + cur * TILE_B;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int ch = ks * 4 + (lane >> 4);
      uint4 fa[4], fb[4];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) fa[mi] = ld16(a + swz(wm * 64 + mi * 16 + (lane & 15), ch));
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) fb[ni] = ld16(b + swz(wn * 64 + ni * 16 + (lane & 15), ch));
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) Mma<T>::run(fa[mi], fb[ni], acc[mi][ni]);
    }
    if (more) {
      char* na = sA + (cur ^ 1) * TILE_B;
      char* nb = sB + (cur ^ 1) * TILE_B;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        st16(na + swz(lrow + 32 * i, lchunk), ra[i]);
        st16(nb + swz(lrow + 32 * i, lchunk), rb[i]);
      }
    }
    __syncthreads();
  }
}

__device__ __forceinline__ void zero_acc(f32x4_t (&acc)[4][4]) {
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = f32x4_t{0.f, 0.f, 0.f, 0.f};
}

__device__ __forceinline__ void put(char* p, float v, float) { *reinterpret_cast<float*>(p) = v; }
__device__ __forceinline__ void put(char* p, float v, bf16_t) {
  *reinterpret_cast<uint16_t*>(p) = f32_to_bf16(v);
}

// Stage the full 128x128 accumulator tile into LDS rows of ld bytes.
template <typename OutT>
__device__ __forceinline__ void stage_full(const f32x4_t (&acc)[4][4], char* lds, int ld) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = wm * 64 + mi * 16 + (lane >> 4) * 4 + r;
        const int col = wn * 64 + ni * 16 + (lane & 15);
        put(lds + row * ld + col * (int)sizeof(OutT), acc[mi][ni][r], OutT{});
      }
}

// Stage silu(gate) * up as a 128x64 tile: accumulator columns ni and ni+2 of
// every wavefront hold the gate and up projections of the same 16 features.
template <typename OutT>
__device__ __forceinline__ void stage_swiglu(const f32x4_t (&acc)[4][4], char* lds, int ld) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = wm * 64 + mi * 16 + (lane >> 4) * 4 + r;
        const int col = wn * 32 + ni * 16 + (lane & 15);
        const float h = silu(acc[mi][ni][r]) * acc[mi][ni + 2][r];
        put(lds + row * ld + col * (int)sizeof(OutT), h, OutT{});
      }
}

// Copy staged rows out in 16-byte chunks; row_ptr(r) gives the destination
// of tile row r (already offset to the tile's first column).
template <class RowPtr>
__device__ __forceinline__ void copy_out(const char* lds, int ld, int chunks_per_row,
                                         int valid_rows, int valid_chunks, RowPtr row_ptr) {
  const int total = BM * chunks_per_row;
  for (int q = threadIdx.x; q < total; q += NTHR) {
    const int r = q / chunks_per_row;
    const int c = q - r * chunks_per_row;
    if (r < valid_rows && c < valid_chunks) st16(row_ptr(r) + c * 16, ld16(lds + r * ld + c * 16));
  }
}

// ------------------------------------------------------------------ dense
template <typename T, typename OutT>
__global__ __launch_bounds__(NTHR) void gemm_dense_kernel(GemmDense g) {
  __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES];
  const int n0 = blockIdx.x * BN;
  const int m0 = blockIdx.y * BM;
  const int lrow = threadIdx.x >> 3, lchunk = threadIdx.x & 7;
  f32x4_t acc[4][4];
  zero_acc(acc);
  for (int s = 0; s < g.nseg; ++s) {
    const GemmSeg& sg = g.seg[s];
    const char* a_src[4];
    const char* b_src[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = min(m0 + lrow + 32 * i, g.M - 1);
      const int n = min(n0 + lrow + 32 * i, g.N - 1);
      a_src[i] = static_cast<const char*>(sg.A) + ((int64_t)m * sg.lda) * (int64_t)sizeof(T) + lchunk * 16;
      b_src[i] = static_cast<const char*>(sg.B) + ((int64_t)n * sg.ldb) * (int64_t)sizeof(T) + lchunk * 16;
    }
    mainloop<T>(a_src, b_src, sg.K * (int)sizeof(T) / BKB, lds, acc);
  }
  constexpr int ld = BN * (int)sizeof(OutT) + STAGE_PAD;
  stage_full<OutT>(acc, lds, ld);
  __syncthreads();
  constexpr int cpr = BN * (int)sizeof(OutT) / 16;
  const int valid_chunks = min(cpr, (g.N - n0) * (int)sizeof(OutT) / 16);
  char* C = static_cast<char*>(g.C);
  copy_out(lds, ld, cpr, min(BM, g.M - m0), valid_chunks, [&](int r) {
    return C + ((int64_t)(m0 + r) * g.ldc + n0) * (int64_t)sizeof(OutT);
  });
}

// ------------------------------------------------------------------ SwiGLU
// B tile row r of feature tile f0: gate (half 0) or up (half 1) weight row of
// feature f0 + (r / 64) * 32 + r % 32, half = (r / 32) % 2.
struct SwigluArgs {
  // dense A (shared experts)
  const char* A;
  int64_t lda_bytes;
  // gathered A (routed experts)
  const char* pools;
  int64_t block_bytes, row_bytes;
  int cap_send;
  const int32_t* erow;
  const int32_t* rows_total;
  int max_rows;
  // weights [G][F][K]
  const char* Wg;
  const char* Wu;
  int F, K, M;
  // output
  char* C;
  int64_t ldc_bytes;
};

template <typename T, bool kGather>
__global__ __launch_bounds__(NTHR) void swiglu_kernel(SwigluArgs p) {
  __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES];
  const int f0 = blockIdx.x * 64;
  const int m0 = blockIdx.y * BM;
  const int g = blockIdx.z;
  int rows;
  if (kGather) {
    rows = p.rows_total[g];
    if (m0 >= rows) return;
  } else {
    rows = p.M;
  }
  const int lrow = threadIdx.x >> 3, lchunk = threadIdx.x & 7;
  const char* a_src[4];
  const char* b_src[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = min(m0 + lrow + 32 * i, rows - 1);
    if (kGather) {
      const int fi = p.erow[(int64_t)g * p.max_rows + m];
      const int blk = fi / p.cap_send;
      const int slot = fi - blk * p.cap_send;
      a_src[i] = p.pools + blk * p.block_bytes + slot * p.row_bytes + lchunk * 16;
    } else {
      a_src[i] = p.A + m * p.lda_bytes + lchunk * 16;
    }
    const int f = f0 + (i >> 1) * 32 + lrow;
    const char* W = (i & 1) ? p.Wu : p.Wg;
    b_src[i] = W + ((int64_t)g * p.F + f) * p.K * (int64_t)sizeof(T) + lchunk * 16;
  }
  f32x4_t acc[4][4];
  zero_acc(acc);
  mainloop<T>(a_src, b_src, p.K * (int)sizeof(T) / BKB, lds, acc);
  constexpr int ld = 64 * (int)sizeof(T) + STAGE_PAD;
  stage_swiglu<T>(acc, lds, ld);
  __syncthreads();
  constexpr int cpr = 64 * (int)sizeof(T) / 16;
  char* C = p.C;
  if (kGather) {
    // H[g][m][f]
    copy_out(lds, ld, cpr, min(BM, rows - m0), cpr, [&](int r) {
      return C + (((int64_t)g * p.max_rows + m0 + r) * p.F + f0) * (int64_t)sizeof(T);
    });
  } else {
    // C[m][g*F + f]
    copy_out(lds, ld, cpr, min(BM, rows - m0), cpr, [&](int r) {
      return C + (int64_t)(m0 + r) * p.ldc_bytes + ((int64_t)g * p.F + f0) * (int64_t)sizeof(T);
    });
  }
}

// ------------------------------------------------------------------ expert down
template <typename T>
__global__ __launch_bounds__(NTHR) void expert_down_kernel(ExpertDown p) {
  __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES];
  const int n0 = blockIdx.x * BN;
  const int m0 = blockIdx.y * BM;
  const int e = blockIdx.z;
  const int rows = p.rows_total[e];
  if (m0 >= rows) return;
  const int lrow = threadIdx.x >> 3, lchunk = threadIdx.x & 7;
  const char* H = static_cast<const char*>(p.H);
  const char* Wd = static_cast<const char*>(p.Wd);
  const char* a_src[4];
  const char* b_src[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = min(m0 + lrow + 32 * i, rows - 1);
    const int n = min(n0 + lrow + 32 * i, p.L - 1);
    a_src[i] = H + (((int64_t)e * p.max_rows + m) * p.F) * (int64_t)sizeof(T) + lchunk * 16;
    b_src[i] = Wd + (((int64_t)e * p.L + n) * p.F) * (int64_t)sizeof(T) + lchunk * 16;
  }
  f32x4_t acc[4][4];
  zero_acc(acc);
  mainloop<T>(a_src, b_src, p.F * (int)sizeof(T) / BKB, lds, acc);
  constexpr int ld = BN * (int)sizeof(T) + STAGE_PAD;
  stage_full<T>(acc, lds, ld);
  __syncthreads();
  constexpr int cpr = BN * (int)sizeof(T) / 16;
  const int valid_chunks = min(cpr, (p.L - n0) * (int)sizeof(T) / 16);
  char* out = static_cast<char*>(p.out);
  const int32_t* er = p.erow + (int64_t)e * p.max_rows + m0;
  copy_out(lds, ld, cpr, min(BM, rows - m0), valid_chunks, [&](int r) {
    return out + ((int64_t)er[r] * p.L + n0) * (int64_t)sizeof(T);
  });
}

inline int cdiv(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

}  // namespace

hipError_t launch_gemm_dense(int in_dt, int out_dt, const GemmDense& g, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  if (in_dt == DT_BF16 && out_dt == DT_BF16) return launch_gemm_dense_bf16(g, s);
  if (in_dt == DT_BF16 && out_dt == DT_F32 && dense_f32out_supported(g)) return launch_dense_f32out_bf16(g, s);
  const dim3 grid(cdiv(g.N, BN), cdiv(g.M, BM));
  if (in_dt == DT_BF16 && out_dt == DT_F32)
    gemm_dense_kernel<bf16_t, float><<<grid, NTHR, 0, s>>>(g);
  else if (in_dt == DT_F32 && out_dt == DT_F32)
    gemm_dense_kernel<float, float><<<grid, NTHR, 0, s>>>(g);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_swiglu_dense(int dt, const void* A, int64_t lda, const void* Wg,
                               const void* Wu, int G, int F, int K, int M, void* C,
                               int64_t ldc, hipStream_t s) {
  if (M <= 0 || G <= 0) return hipSuccess;
  if (dt == DT_BF16) return launch_swiglu_dense_bf16(A, lda, Wg, Wu, G, F, K, M, C, ldc, s);
  const int eb = 4;
  SwigluArgs p{};
  p.A = static_cast<const char*>(A);
  p.lda_bytes = lda * eb;
  p.Wg = static_cast<const char*>(Wg);
  p.Wu = static_cast<const char*>(Wu);
  p.F = F;
  p.K = K;
  p.M = M;
  p.C = static_cast<char*>(C);
  p.ldc_bytes = ldc * eb;
  const dim3 grid(F / 64, cdiv(M, BM), G);
  swiglu_kernel<float, false><<<grid, NTHR, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_expert_gate_up(int dt, const ExpertGateUp& a, hipStream_t s) {
  if (a.E <= 0 || a.max_rows <= 0) return hipSuccess;
  if (dt != DT_F32) return hipErrorInvalidValue;  // bf16 experts use the grouped kernels
  SwigluArgs p{};
  p.pools = a.pools;
  p.block_bytes = a.block_bytes;
  p.row_bytes = a.row_bytes;
  p.cap_send = a.cap_send;
  p.erow = a.erow;
  p.rows_total = a.rows_total;
  p.max_rows = a.max_rows;
  p.Wg = static_cast<const char*>(a.Wg);
  p.Wu = static_cast<const char*>(a.Wu);
  p.F = a.F;
  p.K = a.L;
  p.C = static_cast<char*>(a.H);
  const dim3 grid(a.F / 64, cdiv(a.max_rows, BM), a.E);
  swiglu_kernel<float, true><<<grid, NTHR, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_expert_down(int dt, const ExpertDown& a, hipStream_t s) {
  if (a.E <= 0 || a.max_rows <= 0) return hipSuccess;
  if (dt != DT_F32) return hipErrorInvalidValue;  // bf16 experts use the grouped kernels
  const dim3 grid(cdiv(a.L, BN), cdiv(a.max_rows, BM), a.E);
  expert_down_kernel<float><<<grid, NTHR, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace moe
