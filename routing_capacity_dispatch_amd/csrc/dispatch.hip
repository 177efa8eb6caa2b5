// Pooled-wave dispatch: slot assignment, row scatter into the per-destination
// pool blocks, and receiver-side binning from the packed id column.
//
// Slot assignment is a deterministic stable counting scan per wave over
// chunks of 1024 (token, j) assignments, one workgroup per (chunk, wave):
// pass 1 counts each chunk's assignments per expert and per pool; pass 2
// takes a key's base from the counts of the wave's earlier chunks and ranks
// the chunk's own assignments with wavefront match masks (ballots on the key
// bits) and a scan across its wavefronts.  Integer counts make every slot
// independent of the order in which atomics land.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kAssignWaves = 16;
constexpr int kAssignThreads = kAssignWaves * 64;
constexpr int kChunk = kAssignThreads;  // assignments per block of the slot scan
constexpr int kRecvBatch = 16;          // id-column loads in flight per lane in receiver binning
constexpr int kGidxChunk = 2048;        // row-list entries per workgroup of the expert-major row list

inline int64_t ceil_div_i64(int64_t a, int64_t b) { return (a + b - 1) / b; }

__device__ __forceinline__ int key_bits(int n) {  // bits to hold 0..n-1
  int b = 0;
  while ((1 << b) < n) ++b;
  return b;
}

// Chunk c of wave w: assignments [c * kChunk, (c + 1) * kChunk) of the wave's
// (token, j) order.
struct ChunkRange {
  int w, c, n, lo, hi;
  int64_t base;  // flat index of the wave's first assignment
};

__device__ __forceinline__ ChunkRange chunk_range(const DispatchArgs& a) {
  ChunkRange r;
  r.w = blockIdx.y;
  r.c = blockIdx.x;
  const int64_t t0 = (int64_t)r.w * a.Tw;
  const int64_t t1 = min(a.T, t0 + a.Tw);
  r.n = t1 > t0 ? (int)((t1 - t0) * a.k) : 0;
  r.base = t0 * a.k;
  r.lo = min(r.n, r.c * kChunk);
  r.hi = min(r.n, r.lo + kChunk);
  return r;
}

// Pass 1: per chunk, the number of assignments to each expert and to each
// pool (integer LDS atomics, so the counts do not depend on their order).
// Also clears the per-wave counters and marks every id slot empty; pass 2
// then writes the occupied ones.
__global__ __launch_bounds__(kAssignThreads) void assign_count_kernel(DispatchArgs a) {
  extern __shared__ int32_t hist[];  // [E + P]
  const ChunkRange r = chunk_range(a);
  const int E = a.E, P = a.P, epp = E / P, cap_send = (int)a.cap_send;
  const int tid = threadIdx.x;
  if (r.c == 0 && r.w == 0)
    for (int j = tid; j < 3 * a.W; j += kAssignThreads) a.wave_counts[j] = 0;
  {
    // id column of every pool block of this wave: -1 = empty
    const int64_t nslots = (int64_t)P * cap_send;
    for (int64_t q = (int64_t)r.c * kAssignThreads + tid; q < nslots; q += (int64_t)gridDim.x * kAssignThreads) {
      const int pp = (int)(q / cap_send);
      const int ss = (int)(q - (int64_t)pp * cap_send);
      reinterpret_cast<int32_t*>(a.pools + ((int64_t)r.w * P + pp) * a.block_bytes + a.ids_offset)[ss] = -1;
    }
  }
  if (r.lo >= r.hi) return;
  for (int j = tid; j < E + P; j += kAssignThreads) hist[j] = 0;
  __syncthreads();
  const int i = r.lo + tid;
  if (i < r.hi) {
    const int e = a.topk[r.base + i];
    if (e >= 0 && e < E) {
      atomicAdd(&hist[e], 1);
      atomicAdd(&hist[E + e / epp], 1);
    }
  }
  __syncthreads();
  int32_t* out = a.chunk_counts + ((int64_t)r.w * a.n_chunks + r.c) * (E + P);
  for (int j = tid; j < E + P; j += kAssignThreads) out[j] = hist[j];
}

// Pass 2: per chunk, the expert and pool ranks of its assignments.  A key's
// base is its count over the wave's earlier chunks; inside the chunk each
// wavefront's share comes from match masks (ballots on the key bits) and an
// exclusive scan across the chunk's wavefronts.  The wave's last chunk also
// writes the pool occupancy.  Kept / sender-dropped / receiver-dropped
// counts are integer atomics into the per-wave counters.
__global__ __launch_bounds__(kAssignThreads) void assign_slots_kernel(DispatchArgs a) {
  extern __shared__ int32_t sh[];
  const int E = a.E, P = a.P, K = E + P;
  int32_t* wh = sh;                          // [16][E + P]: per-wavefront counts, then their bases
  __shared__ int64_t red[kAssignWaves][3];
  const ChunkRange r = chunk_range(a);
  const int tid = threadIdx.x, lane = tid & 63, v = tid >> 6;
  const int epp = E / P;
  const int ebits = key_bits(E), pbits = key_bits(P);
  const int cap_send = (int)a.cap_send, cap_recv = (int)a.cap_recv;
  if (r.n == 0) {  // an empty wave: nothing sent
    if (r.c == 0)
      for (int pp = tid; pp < P; pp += kAssignThreads) a.pool_count[r.w * P + pp] = 0;
    return;
  }
  if (r.lo >= r.hi) return;
  const bool last = r.hi == r.n;
  for (int j = tid; j < kAssignWaves * K; j += kAssignThreads) wh[j] = 0;
  __syncthreads();

  const int i = r.lo + v * 64 + lane;
  const int e_in = i < r.hi ? a.topk[r.base + i] : 0;
  const bool valid = i < r.hi && e_in >= 0 && e_in < E;
  const int e = valid ? e_in : 0;
  const int p = e / epp;
  const uint64_t lt = lanemask_lt();
  const uint64_t act = ballot64(valid);
  const uint64_t me = match_key((uint32_t)e, ebits, act);
  const uint64_t mp = match_key((uint32_t)p, pbits, act);
  if (valid && (me & lt) == 0) wh[v * K + e] = __popcll(me);
  if (valid && (mp & lt) == 0) wh[v * K + E + p] = __popcll(mp);
  __syncthreads();

  // per key: the count over earlier chunks, then an exclusive scan over
  // this chunk's wavefronts
  const int32_t* cnt = a.chunk_counts + (int64_t)r.w * a.n_chunks * K;
  for (int j = tid; j < K; j += kAssignThreads) {
    int run = 0;
    {
      // eight loads in flight at a time
      int c = 0;
      for (; c + 8 <= r.c; c += 8) {
        int x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) x[u] = cnt[(int64_t)(c + u) * K + j];
#pragma unroll
        for (int u = 0; u < 8; ++u) run += x[u];
      }
      for (; c < r.c; ++c) run += cnt[(int64_t)c * K + j];
    }
    for (int u = 0; u < kAssignWaves; ++u) {
      const int x = wh[u * K + j];
      wh[u * K + j] = run;
      run += x;
    }
    if (last && j >= E) a.pool_count[r.w * P + (j - E)] = min(run, cap_send);
  }
  __syncthreads();

  int64_t kept = 0, sd = 0, rd = 0;
  if (i < r.hi) {
    int ps = -1, rs = -1;
    if (!valid) {
      ++sd;
    } else {
      const int rank_p = wh[v * K + E + p] + __popcll(mp & lt);
      const int rank_e = wh[v * K + e] + __popcll(me & lt);
      if (rank_p < cap_send) {
        ps = rank_p;
        reinterpret_cast<int32_t*>(a.pools + ((int64_t)r.w * P + p) * a.block_bytes + a.ids_offset)[ps] = e;
        // every earlier assignment to e shares pool p and was sent, so the
        // expert rank is the receiver's binning order
        if (rank_e < cap_recv) {
          rs = rank_e;
          ++kept;
        } else {
          ++rd;
        }
      } else {
        ++sd;
      }
    }
    a.pool_slot[r.base + i] = ps;
    a.recv_slot[r.base + i] = rs;
  }
  for (int m = 32; m >= 1; m >>= 1) {
    kept += __shfl_xor(kept, m);
    sd += __shfl_xor(sd, m);
    rd += __shfl_xor(rd, m);
  }
  if (lane == 0) red[v][0] = kept, red[v][1] = sd, red[v][2] = rd;
  __syncthreads();
  if (tid < 3) {
    int64_t t = 0;
    for (int u = 0; u < kAssignWaves; ++u) t += red[u][tid];
    if (t) atomicAdd(reinterpret_cast<unsigned long long*>(a.wave_counts + r.w * 3 + tid), (unsigned long long)t);
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
  const char* src = z + t * a.row_bytes;
  const int chunks = (int)(a.row_bytes / 16);
  // a row of up to 512 chunks: its loads first (clamped past the row's end,
  // not stored), then the assignments' (every lane loads: lanes past k
  // re-read the last one), so no branch separates any of the loads
  uint4 r[8];
  if (chunks <= 512) {
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = ld16(src + (int64_t)min(i * 64 + lane, chunks - 1) * 16);
  }
  const int64_t q = t * k + min(lane, k - 1);
  const int ps = a.pool_slot[q], e = a.topk[q];
  const int64_t off = (w * a.P + e / epp) * a.block_bytes + (int64_t)ps * a.row_bytes;  // used only if kept
  char* dst = ((lane < k) & (ps >= 0)) ? a.pools + off : nullptr;
  if (chunks > 512) {
    scatter_row(src, dst, k, a.row_bytes);
    return;
  }
  for (int j = 0; j < k; ++j) {
    char* d = reinterpret_cast<char*>(readlane64(reinterpret_cast<int64_t>(dst), j));
    if (!d) continue;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = i * 64 + lane;
      if (c < chunks) st16(d + (int64_t)c * 16, r[i]);
    }
  }
}

// Receiver side: one wavefront per (wave, pool) block reads only the id
// column, in slot order, and bins slots to its E/P local experts, keeping the
// first C_recv of each.  The id column is read kRecvBatch x 64 slots at a
// time (all loads in flight together), then binned 64 slots per step.
__global__ __launch_bounds__(64) void recv_bin_kernel(DispatchArgs a, int32_t* __restrict__ bank_rows,
                                                      int32_t* __restrict__ expert_count) {
  extern __shared__ int32_t cnt[];  // [E/P]
  const int lane = threadIdx.x;
  const int P = a.P, E = a.E;
  const int w = blockIdx.x / P, p = blockIdx.x - (blockIdx.x / P) * P;
  const int epp = E / P;
  const int lbits = key_bits(epp);
  const int cap_send = (int)a.cap_send, cap_recv = (int)a.cap_recv;
  // the step's kept / sender-dropped / receiver-dropped totals from the slot
  // scan's per-wave counters (complete: the scan ran in an earlier launch)
  if (blockIdx.x == 0 && a.counts && lane < 3) {
    int64_t t = 0;
    for (int ww = 0; ww < a.W; ++ww) t += a.wave_counts[ww * 3 + lane];
    a.counts[lane] = t;
  }
  for (int i = lane; i < epp; i += 64) cnt[i] = 0;
  __syncthreads();
  const int32_t* ids = reinterpret_cast<const int32_t*>(a.pools + ((int64_t)w * P + p) * a.block_bytes + a.ids_offset);
  const uint64_t lt = lanemask_lt();
  for (int it0 = 0; it0 < cap_send; it0 += 64 * kRecvBatch) {
    int idv[kRecvBatch];
#pragma unroll
    for (int b = 0; b < kRecvBatch; ++b) {
      const int s = it0 + b * 64 + lane;
      idv[b] = s < cap_send ? ids[s] : -1;
    }
#pragma unroll
    for (int b = 0; b < kRecvBatch; ++b) {
      const int s = it0 + b * 64 + lane;
      const int id = idv[b];
      const int le = id - p * epp;
      const bool valid = id >= 0 && le >= 0 && le < epp;
      const uint64_t act = ballot64(valid);
      if (!act) continue;  // wave-uniform
      const uint64_t m = match_key((uint32_t)(valid ? le : 0), lbits, act);
      int r = 0;
      if (valid) r = cnt[le] + __popcll(m & lt);
      if (valid && (m & lt) == 0) cnt[le] = r + __popcll(m);
      if (valid && r < cap_recv) bank_rows[((int64_t)w * E + id) * cap_recv + r] = s;
    }
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
// expert-major order (waves in order, receiver slots in order).  Workgroup
// (x, e) writes expert e's list entries [x * kGidxChunk, (x + 1) * kGidxChunk),
// so an expert with many rows is spread over many workgroups.  Counts and
// slots are clamped to the block, so malformed lists cannot send the GEMMs
// outside the pools.
__global__ __launch_bounds__(256) void expert_gidx_kernel(const int32_t* __restrict__ bank_rows,
                                                          const int32_t* __restrict__ expert_count,
                                                          const int32_t* __restrict__ offsets, int E, int P, int W,
                                                          int cap_send, int cap_recv, int32_t* __restrict__ gidx) {
  const int e = blockIdx.y;
  const int p = e / (E / P);
  const int lo = blockIdx.x * kGidxChunk, hi = lo + kGidxChunk;
  const int off = offsets[e];
  int pre = 0;  // the expert's rows in earlier waves
  for (int w = 0; w < W && pre < hi; ++w) {
    const int c = min(max(expert_count[(int64_t)w * E + e], 0), cap_recv);
    const int a = max(lo, pre), b = min(hi, pre + c);
    const int32_t* br = bank_rows + ((int64_t)w * E + e) * cap_recv - pre;
    const int base = (w * P + p) * cap_send;
    for (int i = a + (int)threadIdx.x; i < b; i += 256) gidx[off + i] = base + min(max(br[i], 0), cap_send - 1);
    pre += c;
  }
}

__global__ void zero_i64_kernel(int64_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

}  // namespace

int assign_chunks(int64_t Tw, int k) { return (int)std::max<int64_t>(1, (Tw * k + kChunk - 1) / kChunk); }

hipError_t launch_assign(const DispatchArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)a.n_chunks, (unsigned)a.W);
  const size_t lds1 = sizeof(int32_t) * (size_t)(a.E + a.P);
  assign_count_kernel<<<grid, kAssignThreads, lds1, s>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t lds2 = sizeof(int32_t) * (size_t)kAssignWaves * (a.E + a.P);
  if (lds2 > 64 * 1024) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(assign_slots_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds2);
    if (e != hipSuccess) return e;
  }
  assign_slots_kernel<<<grid, kAssignThreads, lds2, s>>>(a);
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
  if ((int64_t)W * cap_recv <= 0 || E <= 0) return hipSuccess;  // no kept rows: the list is empty
  const dim3 grid((unsigned)ceil_div_i64((int64_t)W * cap_recv, kGidxChunk), (unsigned)E);
  expert_gidx_kernel<<<grid, 256, 0, s>>>(bank_rows, expert_count, offsets, E, P, W, (int)cap_send, (int)cap_recv,
                                          gidx);
  return hipGetLastError();
}

hipError_t launch_zero_i64(int64_t* p, int n, hipStream_t s) {
  zero_i64_kernel<<<(n + 63) / 64, 64, 0, s>>>(p, n);
  return hipGetLastError();
}

}  // namespace moe
