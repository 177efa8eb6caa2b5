// Pooled-wave dispatch: slot assignment, row scatter into the per-destination
// pool blocks, and receiver-side binning from the packed id column.
//
// Slot assignment is a deterministic stable counting pass per wave: one
// workgroup of 16 wavefronts per wave, each wavefront owning a contiguous
// range of the wave's (token, j) assignments.  Pass 1 builds per-wavefront
// histograms over experts and pools from wavefront match masks (ballots on
// the key bits), the workgroup scans them across wavefronts, and pass 2
// walks the ranges again to turn match-mask ranks plus the scanned bases
// into pool and receiver slots.  No atomics touch the result.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kAssignWaves = 16;
constexpr int kAssignThreads = kAssignWaves * 64;

__device__ __forceinline__ int key_bits(int n) {  // bits to hold 0..n-1
  int b = 0;
  while ((1 << b) < n) ++b;
  return b;
}

__global__ __launch_bounds__(kAssignThreads) void assign_kernel(DispatchArgs a) {
  extern __shared__ int32_t sh[];
  const int E = a.E, P = a.P, k = a.k;
  int32_t* hist_e = sh;                              // [16][E]
  int32_t* hist_p = hist_e + kAssignWaves * E;       // [16][P]
  int32_t* demand_p = hist_p + kAssignWaves * P;     // [P]
  __shared__ int64_t red[kAssignWaves][2];

  const int w = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, v = tid >> 6;
  const int64_t t0 = (int64_t)w * a.Tw;
  const int64_t t1 = min(a.T, t0 + a.Tw);
  const int n = t1 > t0 ? (int)((t1 - t0) * k) : 0;
  const int64_t base = t0 * k;
  const int epp = E / P;
  const int ebits = key_bits(E), pbits = key_bits(P);
  const int cap_send = (int)a.cap_send, cap_recv = (int)a.cap_recv;

  for (int i = tid; i < kAssignWaves * (E + P); i += kAssignThreads) sh[i] = 0;
  __syncthreads();

  // contiguous range of this wavefront, a multiple of 64 assignments
  const int per = ((n + kAssignWaves * 64 - 1) / (kAssignWaves * 64)) * 64;
  const int lo = min(n, v * per), hi = min(n, lo + per);
  const uint64_t lt = lanemask_lt();

  // pass 1: per-wavefront histograms (expert ids outside [0, E) take no
  // slot and count as sender drops)
  for (int it = lo; it < hi; it += 64) {
    const int i = it + lane;
    const int e_in = i < hi ? a.topk[base + i] : 0;
    const bool valid = i < hi && e_in >= 0 && e_in < E;
    const int e = valid ? e_in : 0;
    const int p = e / epp;
    const uint64_t act = ballot64(valid);
    const uint64_t me = match_key((uint32_t)e, ebits, act);
    const uint64_t mp = match_key((uint32_t)p, pbits, act);
    if (valid && (me & lt) == 0) hist_e[v * E + e] += __popcll(me);
    if (valid && (mp & lt) == 0) hist_p[v * P + p] += __popcll(mp);
  }
  __syncthreads();

  // exclusive scan across wavefronts; totals are the wave's demand
  for (int e = tid; e < E; e += kAssignThreads) {
    int run = 0;
    for (int u = 0; u < kAssignWaves; ++u) {
      const int c = hist_e[u * E + e];
      hist_e[u * E + e] = run;
      run += c;
    }
  }
  int64_t sd = 0;
  for (int p = tid; p < P; p += kAssignThreads) {
    int run = 0;
    for (int u = 0; u < kAssignWaves; ++u) {
      const int c = hist_p[u * P + p];
      hist_p[u * P + p] = run;
      run += c;
    }
    demand_p[p] = run;
    a.pool_count[w * P + p] = min(run, cap_send);
    sd += max(0, run - cap_send);
  }
  __syncthreads();

  // empty slots of the id column
  for (int64_t q = tid; q < (int64_t)P * cap_send; q += kAssignThreads) {
    const int p = (int)(q / cap_send);
    const int s = (int)(q - (int64_t)p * cap_send);
    if (s >= demand_p[p]) {
      int32_t* ids = reinterpret_cast<int32_t*>(a.pools + ((int64_t)w * P + p) * a.block_bytes + a.ids_offset);
      ids[s] = -1;
    }
  }

  // pass 2: slots
  int64_t kept = 0, rd = 0;
  for (int it = lo; it < hi; it += 64) {
    const int i = it + lane;
    const int e_in = i < hi ? a.topk[base + i] : 0;
    const bool valid = i < hi && e_in >= 0 && e_in < E;
    const int e = valid ? e_in : 0;
    const int p = e / epp;
    if (i < hi && !valid) {
      a.pool_slot[base + i] = -1;
      a.recv_slot[base + i] = -1;
      ++sd;
    }
    const uint64_t act = ballot64(valid);
    const uint64_t me = match_key((uint32_t)e, ebits, act);
    const uint64_t mp = match_key((uint32_t)p, pbits, act);
    int rank_e = 0, rank_p = 0;
    if (valid) {
      rank_e = hist_e[v * E + e] + __popcll(me & lt);
      rank_p = hist_p[v * P + p] + __popcll(mp & lt);
    }
    if (valid && (me & lt) == 0) hist_e[v * E + e] = rank_e + __popcll(me);
    if (valid && (mp & lt) == 0) hist_p[v * P + p] = rank_p + __popcll(mp);
    if (valid) {
      int ps = -1, rs = -1;
      if (rank_p < cap_send) {
        ps = rank_p;
        int32_t* ids = reinterpret_cast<int32_t*>(a.pools + ((int64_t)w * P + p) * a.block_bytes + a.ids_offset);
        ids[ps] = e;
        // every earlier assignment to e shares pool p and was sent, so the
        // expert rank is the receiver's binning order
        if (rank_e < cap_recv) {
          rs = rank_e;
          ++kept;
        } else {
          ++rd;
        }
      }
      a.pool_slot[base + i] = ps;
      a.recv_slot[base + i] = rs;
    }
  }
  // workgroup reduction of the wave's counters
  for (int m = 32; m >= 1; m >>= 1) {
    kept += __shfl_xor(kept, m);
    rd += __shfl_xor(rd, m);
  }
  // sender drops were summed per pool by the threads that scanned them
  __shared__ int64_t red_sd[kAssignWaves];
  for (int m = 32; m >= 1; m >>= 1) sd += __shfl_xor(sd, m);
  if (lane == 0) {
    red[v][0] = kept;
    red[v][1] = rd;
    red_sd[v] = sd;
  }
  __syncthreads();
  if (tid == 0) {
    int64_t K = 0, R = 0, S = 0;
    for (int u = 0; u < kAssignWaves; ++u) {
      K += red[u][0];
      R += red[u][1];
      S += red_sd[u];
    }
    a.wave_counts[w * 3 + 0] = K;
    a.wave_counts[w * 3 + 1] = S;
    a.wave_counts[w * 3 + 2] = R;
  }
}

__global__ void finalize_counts_kernel(const int64_t* wave_counts, int W, int64_t* counts) {
  if (threadIdx.x < 3) {
    int64_t s = 0;
    for (int w = 0; w < W; ++w) s += wave_counts[w * 3 + threadIdx.x];
    counts[threadIdx.x] = s;
  }
}

// One wavefront per token: its lanes load the token's k pool slots at once,
// then the z row is read once and written to every slot the token took.
__global__ __launch_bounds__(256) void scatter_kernel(DispatchArgs a, const char* __restrict__ z) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  const int k = a.k, epp = a.E / a.P;
  const int64_t w = t / a.Tw;
  char* dst = nullptr;
  if (lane < k) {
    const int ps = a.pool_slot[t * k + lane];
    if (ps >= 0) {
      const int p = a.topk[t * k + lane] / epp;
      dst = a.pools + (w * a.P + p) * a.block_bytes + (int64_t)ps * a.row_bytes;
    }
  }
  scatter_row(z + t * a.row_bytes, dst, k, a.row_bytes);
}

// Receiver side: one wavefront per (wave, pool) block reads only the id
// column, in slot order, and bins slots to its E/P local experts, keeping the
// first C_recv of each.
__global__ __launch_bounds__(64) void recv_bin_kernel(DispatchArgs a, int32_t* __restrict__ bank_rows,
                                                      int32_t* __restrict__ expert_count) {
  extern __shared__ int32_t cnt[];  // [E/P]
  const int lane = threadIdx.x;
  const int P = a.P, E = a.E;
  const int w = blockIdx.x / P, p = blockIdx.x - (blockIdx.x / P) * P;
  const int epp = E / P;
  const int lbits = key_bits(epp);
  const int cap_send = (int)a.cap_send, cap_recv = (int)a.cap_recv;
  for (int i = lane; i < epp; i += 64) cnt[i] = 0;
  __syncthreads();
  const int32_t* ids = reinterpret_cast<const int32_t*>(a.pools + ((int64_t)w * P + p) * a.block_bytes + a.ids_offset);
  const uint64_t lt = lanemask_lt();
  for (int it = 0; it < cap_send; it += 64) {
    const int s = it + lane;
    const int id = s < cap_send ? ids[s] : -1;
    const int le = id - p * epp;
    const bool valid = id >= 0 && le >= 0 && le < epp;
    const uint64_t act = ballot64(valid);
    const uint64_t m = match_key((uint32_t)(valid ? le : 0), lbits, act);
    int r = 0;
    if (valid) r = cnt[le] + __popcll(m & lt);
    if (valid && (m & lt) == 0) cnt[le] = r + __popcll(m);
    if (valid && r < cap_recv) bank_rows[((int64_t)w * E + id) * cap_recv + r] = s;
  }
  __syncthreads();
  for (int i = lane; i < epp; i += 64) expert_count[(int64_t)w * E + p * epp + i] = min(cnt[i], cap_recv);
}

// Per expert, the rows of all waves as one list of flat pool-row indices.
__global__ __launch_bounds__(64) void expert_rows_kernel(const int32_t* __restrict__ bank_rows,
                                                         const int32_t* __restrict__ expert_count,
                                                         int E, int P, int W, int cap_send, int cap_recv,
                                                         int32_t* __restrict__ erow,
                                                         int32_t* __restrict__ rows_total, int max_rows) {
  const int e = blockIdx.x, lane = threadIdx.x;
  const int p = e / (E / P);
  int off = 0;
  for (int w = 0; w < W; ++w) {
    // counts and slots are clamped to the block, so malformed lists cannot
    // send the GEMMs outside the pools
    const int c = min(max(expert_count[(int64_t)w * E + e], 0), cap_recv);
    const int32_t* br = bank_rows + ((int64_t)w * E + e) * cap_recv;
    const int base = (w * P + p) * cap_send;
    for (int r = lane; r < c; r += 64)
      erow[(int64_t)e * max_rows + off + r] = base + min(max(br[r], 0), cap_send - 1);
    off += c;
  }
  if (lane == 0) rows_total[e] = off;
}

// Kept rows per expert over all waves, and their exclusive scan: expert e's
// rows are [offsets[e], offsets[e+1]) of the expert-major row order.
__global__ __launch_bounds__(1024) void expert_offsets_kernel(const int32_t* __restrict__ expert_count, int E,
                                                               int W, int cap_recv,
                                                               int32_t* __restrict__ offsets) {
  __shared__ int part[16];
  __shared__ int total;
  const int e = threadIdx.x;
  int c = 0;
  if (e < E)
    for (int w = 0; w < W; ++w) c += min(max(expert_count[(int64_t)w * E + e], 0), cap_recv);
  const int ex = block_excl_scan_1024(c, part, &total);
  if (e < E) offsets[e] = ex;
  if (e == 0) offsets[E] = total;
}

// Flat pool-row index ((w * P + p) * C_send + slot) of every kept row, in
// expert-major order (waves in order, receiver slots in order).  Counts and
// slots are clamped to the block, so malformed lists cannot send the GEMMs
// outside the pools.
__global__ __launch_bounds__(64) void expert_gidx_kernel(const int32_t* __restrict__ bank_rows,
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
}

__global__ void zero_i64_kernel(int64_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

}  // namespace

hipError_t launch_assign(const DispatchArgs& a, hipStream_t s) {
  const size_t lds = sizeof(int32_t) * ((size_t)kAssignWaves * (a.E + a.P) + a.P);
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(assign_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  assign_kernel<<<a.W, kAssignThreads, lds, s>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !a.counts) return e;
  finalize_counts_kernel<<<1, 64, 0, s>>>(a.wave_counts, a.W, a.counts);
  return hipGetLastError();
}

hipError_t launch_scatter_rows(const DispatchArgs& a, const void* z, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  scatter_kernel<<<(unsigned)((a.T + 3) / 4), 256, 0, s>>>(a, static_cast<const char*>(z));
  return hipGetLastError();
}

hipError_t launch_recv_bin(const DispatchArgs& a, int32_t* bank_rows, int32_t* expert_count,
                           hipStream_t s) {
  const size_t lds = sizeof(int32_t) * (a.E / a.P);
  recv_bin_kernel<<<a.W * a.P, 64, lds, s>>>(a, bank_rows, expert_count);
  return hipGetLastError();
}

hipError_t launch_expert_rows(const int32_t* bank_rows, const int32_t* expert_count, int E, int P,
                              int W, int64_t cap_send, int64_t cap_recv, int32_t* erow,
                              int32_t* rows_total, int max_rows, hipStream_t s) {
  expert_rows_kernel<<<E, 64, 0, s>>>(bank_rows, expert_count, E, P, W, (int)cap_send,
                                      (int)cap_recv, erow, rows_total, max_rows);
  return hipGetLastError();
}

hipError_t launch_expert_gidx(const int32_t* bank_rows, const int32_t* expert_count, int E, int P, int W,
                              int64_t cap_send, int64_t cap_recv, int32_t* offsets, int32_t* gidx,
                              hipStream_t s) {
  expert_offsets_kernel<<<1, 1024, 0, s>>>(expert_count, E, W, (int)cap_recv, offsets);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  expert_gidx_kernel<<<E, 64, 0, s>>>(bank_rows, expert_count, offsets, E, P, W, (int)cap_send, (int)cap_recv,
                                      gidx);
  return hipGetLastError();
}

hipError_t launch_zero_i64(int64_t* p, int n, hipStream_t s) {
  zero_i64_kernel<<<(n + 63) / 64, 64, 0, s>>>(p, n);
  return hipGetLastError();
}

}  // namespace moe
