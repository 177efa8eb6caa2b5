// Dropless ragged dispatch: every assignment is kept.  The T*k assignments
// are ordered by expert, stably in (token, j) order, and each one's z row is
// copied to its position in that order, so expert e's rows are the
// contiguous range [offsets[e], offsets[e+1]) of one buffer.  On one device
// this permutation is what a ragged all-to-all would deliver.
//
// Stable counting sort in three passes over fixed chunks of the assignment
// list: per-chunk expert histograms, a scan over chunks and experts, then
// per-chunk ranks from wavefront match masks.  No atomics touch a result
// that depends on order, so the output is bitwise reproducible.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kSortWaves = 16;
constexpr int kSortThreads = kSortWaves * 64;
constexpr int kTileListBlocks = 32;  // workgroups writing the tile lists
constexpr int kMBand = 8;            // M tiles per band of the expert GEMMs' tile order

__device__ __forceinline__ int key_bits_of(int n) {
  int b = 0;
  while ((1 << b) < n) ++b;
  return b;
}

// Pass 1: hist[blk][e] = assignments of chunk blk that name expert e.
__global__ __launch_bounds__(kSortThreads) void ragged_hist_kernel(const int32_t* __restrict__ topk, int64_t n,
                                                                    int E, int chunk, int32_t* __restrict__ hist) {
  extern __shared__ int32_t h[];  // [E]
  for (int e = threadIdx.x; e < E; e += kSortThreads) h[e] = 0;
  __syncthreads();
  const int64_t lo = (int64_t)blockIdx.x * chunk;
  const int64_t hi = min(n, lo + chunk);
  for (int64_t i = lo + threadIdx.x; i < hi; i += kSortThreads) {
    const int e = topk[i];
    if (e >= 0 && e < E) atomicAdd(&h[e], 1);  // a count: order-free
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kSortThreads) hist[(int64_t)blockIdx.x * E + e] = h[e];
}

// Pass 2 (one workgroup): base[blk][e] = offsets[e] + assignments of expert e
// in chunks before blk; offsets = exclusive scan of the expert totals.
__global__ __launch_bounds__(1024) void ragged_scan_kernel(const int32_t* __restrict__ hist, int nblk, int E,
                                                            int32_t* __restrict__ base,
                                                            int32_t* __restrict__ offsets,
                                                            int64_t* __restrict__ counts, int64_t n) {
  __shared__ int32_t tot[1024];
  __shared__ int32_t part[16];
  const int e = threadIdx.x;
  int run = 0;
  if (e < E) {
    // eight loads in flight at a time
    int b = 0;
    for (; b + 8 <= nblk; b += 8) {
      int x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) x[u] = hist[(int64_t)(b + u) * E + e];
#pragma unroll
      for (int u = 0; u < 8; ++u) run += x[u];
    }
    for (; b < nblk; ++b) run += hist[(int64_t)b * E + e];
  }
  tot[e] = e < E ? run : 0;
  __syncthreads();
  // exclusive scan of tot[0..1023]: per wavefront, then across wavefronts
  const int lane = e & 63, w = e >> 6;
  int v = tot[e];
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(v, d);
    if (lane >= d) v += o;
  }
  if (lane == 63) part[w] = v;
  __syncthreads();
  if (e == 0) {
    int s = 0;
    for (int i = 0; i < 16; ++i) {
      const int t = part[i];
      part[i] = s;
      s += t;
    }
  }
  __syncthreads();
  const int incl = v + part[w];
  const int excl = incl - tot[e];
  if (e < E) {
    offsets[e] = excl;
    int r = excl;
    int b = 0;
    for (; b + 8 <= nblk; b += 8) {
      int x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) x[u] = hist[(int64_t)(b + u) * E + e];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        base[(int64_t)(b + u) * E + e] = r;
        r += x[u];
      }
    }
    for (; b < nblk; ++b) {
      base[(int64_t)b * E + e] = r;
      r += hist[(int64_t)b * E + e];
    }
  }
  if (e == E - 1) {
    offsets[E] = incl;
    if (counts) {
      counts[0] = incl;      // kept: every valid assignment
      counts[1] = n - incl;  // ids outside [0, E) take no row
      counts[2] = 0;
    }
  }
}

// Pass 3: row_of[i] = base[blk][e] + rank of i among chunk blk's
// assignments to e (wavefront ranges in order, lanes in order).
__global__ __launch_bounds__(kSortThreads) void ragged_rank_kernel(const int32_t* __restrict__ topk, int64_t n,
                                                                    int E, int chunk,
                                                                    const int32_t* __restrict__ base,
                                                                    int32_t* __restrict__ row_of) {
  extern __shared__ int32_t hw[];  // [kSortWaves][E]
  const int lane = threadIdx.x & 63, v = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < kSortWaves * E; i += kSortThreads) hw[i] = 0;
  __syncthreads();
  const int64_t lo = (int64_t)blockIdx.x * chunk;
  const int cn = (int)(min(n, lo + chunk) - lo);
  const int per = ((cn + kSortThreads - 1) / kSortThreads) * 64;
  const int wlo = min(cn, v * per), whi = min(cn, wlo + per);
  const int ebits = key_bits_of(E);
  const uint64_t lt = lanemask_lt();
  // per-wavefront histograms
  for (int it = wlo; it < whi; it += 64) {
    const int i = it + lane;
    const int e_in = i < whi ? topk[lo + i] : -1;
    const bool valid = e_in >= 0 && e_in < E;
    const uint64_t me = match_key((uint32_t)(valid ? e_in : 0), ebits, ballot64(valid));
    if (valid && (me & lt) == 0) hw[v * E + e_in] += __popcll(me);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kSortThreads) {
    int run = base[(int64_t)blockIdx.x * E + e];
    for (int u = 0; u < kSortWaves; ++u) {
      const int c = hw[u * E + e];
      hw[u * E + e] = run;
      run += c;
    }
  }
  __syncthreads();
  for (int it = wlo; it < whi; it += 64) {
    const int i = it + lane;
    const int e_in = i < whi ? topk[lo + i] : -1;
    const bool valid = e_in >= 0 && e_in < E;
    const uint64_t me = match_key((uint32_t)(valid ? e_in : 0), ebits, ballot64(valid));
    int r = -1;
    if (valid) r = hw[v * E + e_in] + __popcll(me & lt);
    if (valid && (me & lt) == 0) hw[v * E + e_in] = r + __popcll(me);
    if (i < whi) row_of[lo + i] = r;
  }
}

// One wavefront per token: its lanes load the token's k rows at once, then
// the z row is read once and written to each of them.
__global__ __launch_bounds__(256) void ragged_scatter_kernel(const char* __restrict__ z,
                                                              const int32_t* __restrict__ row_of, int64_t T,
                                                              int k, int64_t row_bytes, char* __restrict__ xs) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  char* dst = nullptr;
  if (lane < k) {
    const int row = row_of[t * k + lane];
    if (row >= 0) dst = xs + (int64_t)row * row_bytes;
  }
  scatter_row(z + t * row_bytes, dst, k, row_bytes);
}

// Tile lists of the grouped expert GEMMs: expert e gets ceil(rows_e / bm) M
// tiles; list0 (list1) holds (e, N tile, M tile) for tiles_n0 (tiles_n1) N
// tiles per M tile.  Order: experts in turn; an expert's M tiles in bands of
// kMBand; within a band the N tiles in turn, each with the band's M tiles
// (M fastest, so the M tiles sharing a weight tile are neighbours, and a
// band's rows stay in cache while every N tile reads them).  An expert with
// at most kMBand M tiles is one band: (N tile, then M tile).  Every block
// scans the experts' M-tile counts in LDS, then the grid writes the entries
// (12 bytes each) with consecutive threads on consecutive entries: entry q of
// a list with tn N tiles belongs to the expert whose M-tile range holds
// q / tn.
__global__ __launch_bounds__(1024) void ragged_tiles_kernel(const int32_t* __restrict__ offsets, int E, int bm,
                                                             int tiles_n0, int tiles_n1,
                                                             int32_t* __restrict__ list0,
                                                             int32_t* __restrict__ list1,
                                                             int32_t* __restrict__ ntiles) {
  __shared__ int32_t first[1025];  // M tiles before expert e; first[E] = all
  __shared__ int32_t part[16];
  __shared__ int32_t total;
  const int e = threadIdx.x;
  const int cnt = e < E ? offsets[e + 1] - offsets[e] : 0;
  const int m = (cnt + bm - 1) / bm;
  const int ex = block_excl_scan_1024(m, part, &total);
  if (e < E) first[e] = ex;
  if (e == 0) first[E] = total;
  __syncthreads();
  const int64_t n0 = (int64_t)total * tiles_n0, n1 = (int64_t)total * tiles_n1;
  if (blockIdx.x == 0 && e == 0) {
    ntiles[0] = (int32_t)n0;
    ntiles[1] = (int32_t)n1;
  }
  for (int64_t q = (int64_t)blockIdx.x * 1024 + e; q < n0 + n1; q += (int64_t)gridDim.x * 1024) {
    const bool one = q >= n0;
    const int64_t qq = one ? q - n0 : q;
    const int tn = one ? tiles_n1 : tiles_n0;
    const int v = (int)(qq / tn);
    // largest x < E with first[x] <= v: the expert whose M-tile range
    // [first[x], first[x + 1]) holds v (experts without rows share their
    // first with the next expert and are skipped)
    int lo = 0, hi = E - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (first[mid] <= v)
        lo = mid;
      else
        hi = mid - 1;
    }
    const int me = first[lo + 1] - first[lo];
    const int rem = (int)(qq - (int64_t)first[lo] * tn);
    const int band = rem / (kMBand * tn);                 // full bands come first
    const int bs = min(kMBand, me - band * kMBand);       // M tiles in this band
    const int within = rem - band * kMBand * tn;
    const int nt = within / bs;
    int32_t* d = (one ? list1 : list0) + 3 * qq;
    d[0] = lo;
    d[1] = nt;
    d[2] = band * kMBand + (within - nt * bs);
  }
}

// y_lat[t] = sum over j with a row of gates[t][j] * out[row_of[t][j]], fp32
// accumulation in j order, one wavefront per token.  gates == NULL: weight 1
// (the transpose of the dropless dispatch).
template <typename T>
__global__ __launch_bounds__(256) void ragged_combine_kernel(const char* __restrict__ out,
                                                              const int32_t* __restrict__ row_of,
                                                              const float* __restrict__ gates, int64_t Tn, int k,
                                                              int64_t row_bytes, char* __restrict__ y,
                                                              int64_t y_pitch) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= Tn) return;
  // (every lane loads: lanes past k re-read the last assignment)
  const int64_t q = t * k + min(lane, k - 1);
  const int64_t r = row_of[q];
  const float gq = gates ? gates[q] : 1.0f;
  const int64_t row = lane < k ? r : -1;
  const float g = lane < k && r >= 0 ? gq : 0.0f;
  combine_rows<T>(out, row, g, k, row_bytes, y + t * y_pitch);
}

}  // namespace

int ragged_sort_blocks(int64_t n) { return n <= 0 ? 0 : (int)((n + kRaggedChunk - 1) / kRaggedChunk); }

hipError_t launch_ragged_sort(const int32_t* topk, int64_t n, int E, int32_t* hist, int32_t* base,
                              int32_t* offsets, int32_t* row_of, int64_t* counts, hipStream_t s) {
  const int nblk = ragged_sort_blocks(n);
  if (nblk > 0) {
    ragged_hist_kernel<<<nblk, kSortThreads, sizeof(int32_t) * E, s>>>(topk, n, E, kRaggedChunk, hist);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  ragged_scan_kernel<<<1, 1024, 0, s>>>(hist, nblk, E, base, offsets, counts, n);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nblk == 0) return e;
  const size_t lds = sizeof(int32_t) * (size_t)kSortWaves * E;
  if (lds >= 64 * 1024) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(ragged_rank_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  ragged_rank_kernel<<<nblk, kSortThreads, lds, s>>>(topk, n, E, kRaggedChunk, base, row_of);
  return hipGetLastError();
}

hipError_t launch_ragged_scatter(const void* z, const int32_t* row_of, int64_t T, int k, int64_t row_bytes,
                                 void* xs, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  ragged_scatter_kernel<<<(unsigned)((T + 3) / 4), 256, 0, s>>>(static_cast<const char*>(z), row_of, T, k,
                                                                  row_bytes, static_cast<char*>(xs));
  return hipGetLastError();
}

hipError_t launch_ragged_tiles(const int32_t* offsets, int E, int bm, int tiles_n0, int tiles_n1,
                               int32_t* list0, int32_t* list1, int32_t* ntiles, hipStream_t s) {
  ragged_tiles_kernel<<<kTileListBlocks, 1024, 0, s>>>(offsets, E, bm, tiles_n0, tiles_n1, list0, list1, ntiles);
  return hipGetLastError();
}

hipError_t launch_ragged_combine(int dt, const void* out, const int32_t* row_of, const float* gates, int64_t T,
                                 int k, int64_t row_bytes, void* y, hipStream_t s, int64_t y_pitch) {
  if (T <= 0) return hipSuccess;
  if (y_pitch == 0) y_pitch = row_bytes;
  const unsigned blocks = (unsigned)((T + 3) / 4);
  const char* o = static_cast<const char*>(out);
  char* yy = static_cast<char*>(y);
  if (dt == DT_BF16)
    ragged_combine_kernel<bf16_t><<<blocks, 256, 0, s>>>(o, row_of, gates, T, k, row_bytes, yy, y_pitch);
  else
    ragged_combine_kernel<float><<<blocks, 256, 0, s>>>(o, row_of, gates, T, k, row_bytes, yy, y_pitch);
  return hipGetLastError();
}

}  // namespace moe
