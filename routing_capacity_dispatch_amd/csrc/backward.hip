// Backward of the routed path, the parts that move rows and indices: the
// transpose of combine (gate gradients and the gate-scaled row gradients
// sent back to the pool slots the forward read), the softmax backward over
// the k selected logits, and the padded expert-major layout the grouped
// dgrad / wgrad GEMMs work in (each expert's rows contiguous, rounded up to
// a whole 64-row K tile with zero rows so that wgrad contracts over them).
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

// counts[e] = rows expert e kept over all waves; offsets = exclusive scan of
// counts rounded up to 64 (offsets[E] = the padded total).
__global__ __launch_bounds__(1024) void bwd_offsets_kernel(const int32_t* __restrict__ expert_count, int E, int W,
                                                           int cap_recv, int32_t* __restrict__ counts,
                                                           int32_t* __restrict__ offsets) {
  __shared__ int part[16];
  __shared__ int total;
  const int e = threadIdx.x;
  int c = 0;
  if (e < E)
    for (int w = 0; w < W; ++w) c += min(max(expert_count[(int64_t)w * E + e], 0), cap_recv);
  const int ex = block_excl_scan_1024((c + 63) & ~63, part, &total);
  if (e < E) {
    counts[e] = c;
    offsets[e] = ex;
  }
  if (e == 0) offsets[E] = total;
}

// Flat pool-row index ((w * P + p) * C_send + slot) of padded row i of the
// expert-major order (waves in order, receiver slots in order); -1 for the
// padding rows after an expert's rows.  Counts and slots are clamped to the
// block, so malformed lists cannot send the GEMMs outside the pools.
__global__ __launch_bounds__(64) void bwd_gidx_kernel(const int32_t* __restrict__ bank_rows,
                                                      const int32_t* __restrict__ expert_count,
                                                      const int32_t* __restrict__ offsets, int E, int P, int W,
                                                      int cap_send, int cap_recv, int32_t* __restrict__ gidx) {
  const int e = blockIdx.x, lane = threadIdx.x;
  const int p = e / (E / P);
  int off = offsets[e];
  for (int w = 0; w < W; ++w) {
    const int c = min(max(expert_count[(int64_t)w * E + e], 0), cap_recv);
    const int32_t* br = bank_rows + ((int64_t)w * E + e) * cap_recv;
    const int base = (w * P + p) * cap_send;
    for (int r = lane; r < c; r += 64) gidx[off + r] = base + min(max(br[r], 0), cap_send - 1);
    off += c;
  }
  for (int r = off + lane; r < offsets[e + 1]; r += 64) gidx[r] = -1;
}

// The dropless variant's layout: expert e's rows are [off[e], off[e+1]) of
// the expert-ordered buffer; counts and the padded offsets as above.
__global__ __launch_bounds__(1024) void bwd_offsets_ragged_kernel(const int32_t* __restrict__ off, int E, int64_t n,
                                                                  int32_t* __restrict__ counts,
                                                                  int32_t* __restrict__ offsets) {
  __shared__ int part[16];
  __shared__ int total;
  const int e = threadIdx.x;
  int c = 0;
  if (e < E) {
    const int64_t a = min(max((int64_t)off[e], (int64_t)0), n), b = min(max((int64_t)off[e + 1], a), n);
    c = (int)(b - a);
  }
  const int ex = block_excl_scan_1024((c + 63) & ~63, part, &total);
  if (e < E) {
    counts[e] = c;
    offsets[e] = ex;
  }
  if (e == 0) offsets[E] = total;
}

// Padded row i of expert e -> row off[e] + r of the expert-ordered buffer, or
// -1 for padding.
__global__ __launch_bounds__(64) void bwd_gidx_ragged_kernel(const int32_t* __restrict__ off,
                                                             const int32_t* __restrict__ counts,
                                                             const int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ gidx) {
  const int e = blockIdx.x, lane = threadIdx.x;
  const int c = counts[e], first = off[e], o = offsets[e];
  for (int r = lane; r < c; r += 64) gidx[o + r] = first + r;
  for (int r = o + c + lane; r < offsets[e + 1]; r += 64) gidx[r] = -1;
}

// dst row i = the pool row gidx[i] (block = i / block_rows at block_bytes
// apart, rows row_bytes apart inside a block), or zeros where gidx[i] < 0.
// One wavefront per row (the grid covers the bound on the row count), six
// 16-byte chunks per lane in flight.
__global__ __launch_bounds__(256) void gather_rows_kernel(const char* __restrict__ src, int block_rows,
                                                          int64_t block_bytes, int64_t row_bytes,
                                                          const int32_t* __restrict__ gidx,
                                                          const int32_t* __restrict__ nrows, char* __restrict__ dst) {
  constexpr int CPL = 6;
  const int lane = threadIdx.x & 63;
  const int cpr = (int)(row_bytes / 16);
  // one row per wavefront (the grid covers the bound on the row count), so
  // no row's loads wait behind an earlier row's stores
  const int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (i >= *nrows) return;
  const int fi = gidx[i];
  char* drow = dst + i * row_bytes;
  if (fi < 0) {  // a padding row: zeros
    for (int c = lane; c < cpr; c += 64) st16(drow + (int64_t)c * 16, make_uint4(0, 0, 0, 0));
    return;
  }
  const int blk = fi / block_rows;
  const char* srow = src + blk * block_bytes + (int64_t)(fi - blk * block_rows) * row_bytes;
  for (int c0 = 0; c0 < cpr; c0 += 64 * CPL) {
    uint4 v[CPL];
    // chunk indices clamped (not stored past the row's end): no branch
    // between the loads
#pragma unroll
    for (int u = 0; u < CPL; ++u) v[u] = ld16(srow + (int64_t)min(c0 + u * 64 + lane, cpr - 1) * 16);
#pragma unroll
    for (int u = 0; u < CPL; ++u) {
      const int c = c0 + u * 64 + lane;
      if (c < cpr) st16(drow + (int64_t)c * 16, v[u]);
    }
  }
}

// Transpose of combine, one wavefront per token t: for each receiver-kept
// assignment j (dropless: each assignment with a row, row_of >= 0),
// d_gates[t, j] = <dy[t], o[t, j]> (fp32, lane partial sums in chunk order,
// then a butterfly over the wavefront) and the row g[t, j] * dy[t] goes to
// the pool slot the forward read o[t, j] from.  A dropped assignment gets
// d_gates = 0 and no row.  Lanes j < k load the token's assignments at once;
// the o rows are then read two at a time, and the g dy rows stored after the
// last of them.  dy and o are read once, so their loads carry the
// nontemporal hint.
template <int kMaxChunks, bool kRowOf>
__global__ __launch_bounds__(256) void combine_bwd_kernel(CombineBwdArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  const int k = a.k, epp = a.E / a.P;
  const int64_t w = t / a.Tw;
  const int chunks = (int)(a.row_bytes / 16);
  // No branch separates the loads of a step (a branch between loads makes
  // the compiler wait for every earlier load before the next): every lane
  // loads an assignment (lanes past k re-read the last one), chunk indices
  // past the row's end are clamped (their products are not used), and a
  // dropped assignment reads one of the token's kept rows (its dot product
  // is not used and it stores nothing).
  const int64_t q = t * k + min(lane, k - 1);
  int64_t row;
  if constexpr (kRowOf) {  // dropless: the assignment's row in expert order
    row = a.row_of[q];
  } else {
    const int rs = a.recv_slot[q], e = a.topk[q], ps = a.pool_slot[q];
    // (& rather than &&: no short-circuit branch to sink a load into)
    row = ((rs >= 0) & (e >= 0) & (e < a.E) & (ps >= 0) & (ps < a.cap_send)) ? (w * a.P + e / epp) * a.cap_send + ps
                                                                              : -1;
  }
  const float gq = a.gates[q];
  if (lane >= k) row = -1;
  const float g = row >= 0 ? gq : 0.0f;
  // dy[t] in registers: chunk c = i * 64 + lane
  float dy[kMaxChunks][8];
#pragma unroll
  for (int i = 0; i < kMaxChunks; ++i)
    unpack(ld16_stream(static_cast<const char*>(a.dy) + t * a.row_bytes + (int64_t)min(i * 64 + lane, chunks - 1) * 16),
           dy[i], bf16_t{});
  float dg = 0.0f;  // lane j < k ends with d_gates[t, j]
  const uint64_t kept = ballot64(row >= 0);
  if (kept) {
    const int64_t r_l = row >= 0 ? row : shfl64(row, __builtin_ctzll(kept));
    for (int j = 0; j < k; j += 2) {
      const int j1 = j + 1 < k ? j + 1 : j;
      const bool k0 = readlane64(row, j) >= 0;
      const bool k1 = j + 1 < k && readlane64(row, j1) >= 0;
      const int64_t rb0 = readlane64(r_l, j) * a.row_bytes, rb1 = readlane64(r_l, j1) * a.row_bytes;
      const char* o0 = static_cast<const char*>(a.expert_out) + rb0;
      const char* o1 = static_cast<const char*>(a.expert_out) + rb1;
      uint4 v0[kMaxChunks], v1[kMaxChunks];
#pragma unroll
      for (int i = 0; i < kMaxChunks; ++i) {
        const uint32_t c = (uint32_t)min(i * 64 + lane, chunks - 1) * 16u;
        v0[i] = ld16_stream(o0 + c);
        v1[i] = ld16_stream(o1 + c);
      }
      float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
      for (int i = 0; i < kMaxChunks; ++i) {
        const int c = i * 64 + lane;
        if (c >= chunks) continue;
        float f[8];
        unpack(v0[i], f, bf16_t{});
#pragma unroll
        for (int x = 0; x < 8; ++x) s0 = fmaf(dy[i][x], f[x], s0);
        unpack(v1[i], f, bf16_t{});
#pragma unroll
        for (int x = 0; x < 8; ++x) s1 = fmaf(dy[i][x], f[x], s1);
      }
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) {
        s0 += __shfl_xor(s0, m);
        s1 += __shfl_xor(s1, m);
      }
      if (lane == j) dg = k0 ? s0 : 0.0f;
      if (lane == j + 1) dg = k1 ? s1 : 0.0f;
    }
    // the rows g_j dy go out after every load of the token, so no load waits
    // behind a store (stores count in the same vector memory counter)
    for (int j = 0; j < k; ++j) {
      if (readlane64(row, j) < 0) continue;
      const float gj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(g), j));
      char* d = static_cast<char*>(a.d_expert_out) + readlane64(r_l, j) * a.row_bytes;
#pragma unroll
      for (int i = 0; i < kMaxChunks; ++i) {
        const int c = i * 64 + lane;
        if (c >= chunks) continue;
        float out[8];
#pragma unroll
        for (int x = 0; x < 8; ++x) out[x] = gj * dy[i][x];
        st16(d + (int64_t)c * 16, pack(out, bf16_t{}));
      }
    }
  }
  if (lane < k) a.d_gates[t * k + lane] = dg;
}

// Softmax backward over the k selected raw logits, one wavefront per token:
// d_logits[t, e_j] = g_j (dg_j - sum_i g_i dg_i); every other logit of the
// token gets 0 (the selection is piecewise constant, the bias only selects).
__global__ __launch_bounds__(256) void route_bwd_kernel(const int32_t* __restrict__ topk,
                                                        const float* __restrict__ gates,
                                                        const float* __restrict__ d_gates, int64_t T, int k, int E,
                                                        float* __restrict__ d_logits) {
  __shared__ int sel[4][64];
  __shared__ float val[4][64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t t = (int64_t)blockIdx.x * 4 + wv;
  if (t >= T) return;
  float g = 0.0f, dg = 0.0f;
  int e = -1;
  if (lane < k) {
    g = gates[t * k + lane];
    dg = d_gates[t * k + lane];
    e = topk[t * k + lane];
  }
  float s = g * dg;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) s += __shfl_xor(s, m);
  sel[wv][lane] = e;
  val[wv][lane] = g * (dg - s);
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  for (int x = lane; x < E; x += 64) {
    float v = 0.0f;
    for (int j = 0; j < k; ++j)
      if (sel[wv][j] == x) v = val[wv][j];
    d_logits[t * E + x] = v;
  }
}

}  // namespace

hipError_t launch_bwd_layout(const int32_t* bank_rows, const int32_t* expert_count, int E, int P, int W,
                             int64_t cap_send, int64_t cap_recv, int32_t* counts, int32_t* offsets, int32_t* gidx,
                             hipStream_t s) {
  bwd_offsets_kernel<<<1, 1024, 0, s>>>(expert_count, E, W, (int)cap_recv, counts, offsets);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  bwd_gidx_kernel<<<E, 64, 0, s>>>(bank_rows, expert_count, offsets, E, P, W, (int)cap_send, (int)cap_recv, gidx);
  return hipGetLastError();
}

hipError_t launch_bwd_layout_ragged(const int32_t* expert_offsets, int E, int64_t n, int32_t* counts,
                                    int32_t* offsets, int32_t* gidx, hipStream_t s) {
  bwd_offsets_ragged_kernel<<<1, 1024, 0, s>>>(expert_offsets, E, n, counts, offsets);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  bwd_gidx_ragged_kernel<<<E, 64, 0, s>>>(expert_offsets, counts, offsets, gidx);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const void* src, int block_rows, int64_t block_bytes, int64_t row_bytes,
                              const int32_t* gidx, const int32_t* nrows, int64_t max_rows, void* dst,
                              hipStream_t s) {
  if (max_rows <= 0) return hipSuccess;
  const int64_t want = (max_rows + 3) / 4;  // four rows per block, one per wavefront
  if (want > 0x7fffffff) return hipErrorInvalidValue;
  const unsigned blocks = (unsigned)want;
  gather_rows_kernel<<<blocks, 256, 0, s>>>(static_cast<const char*>(src), block_rows, block_bytes, row_bytes,
                                            gidx, nrows, static_cast<char*>(dst));
  return hipGetLastError();
}

hipError_t launch_combine_bwd(const CombineBwdArgs& a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  const unsigned blocks = (unsigned)((a.T + 3) / 4);
  const int64_t chunks = a.row_bytes / 16;
  const bool ro = a.row_of != nullptr;
  if (chunks <= 64 * 2)
    ro ? combine_bwd_kernel<2, true><<<blocks, 256, 0, s>>>(a) : combine_bwd_kernel<2, false><<<blocks, 256, 0, s>>>(a);
  else if (chunks <= 64 * 6)
    ro ? combine_bwd_kernel<6, true><<<blocks, 256, 0, s>>>(a) : combine_bwd_kernel<6, false><<<blocks, 256, 0, s>>>(a);
  else if (chunks <= 64 * 16)
    ro ? combine_bwd_kernel<16, true><<<blocks, 256, 0, s>>>(a) : combine_bwd_kernel<16, false><<<blocks, 256, 0, s>>>(a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_route_bwd(const int32_t* topk, const float* gates, const float* d_gates, int64_t T, int k, int E,
                            float* d_logits, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  route_bwd_kernel<<<(unsigned)((T + 3) / 4), 256, 0, s>>>(topk, gates, d_gates, T, k, E, d_logits);
  return hipGetLastError();
}

}  // namespace moe
