// Router balancing-bias update: the next step's zero-mean bias from
// histograms of this step's router logits (ranhao.site notes on Marin 535B,
// section 2.2: top-8 routing by a histogram-based quantile router whose
// bias is zero-mean, computed for the next step and outside the gradient).
//
// Per expert e: the range [lo_e, hi_e] of its logit column, an nb-bin
// equal-width histogram over that range (the bin of v decided in fp32 as
// min(nb - 1, trunc((v - lo_e) * scale_e)), bin 0 for v = lo_e, scale_e =
// fl32(nb / (hi_e - lo_e)) or 0 for a constant column), the quantile Q_e of level 1 - k/E read
// off the histogram by linear interpolation inside the bin holding rank
// (E - k) T / E, and the bias mean(Q) - Q_e.
//
// Four launches over logits [T][E] fp32, read as 128-byte row segments of 32
// experts (one cache line; 16-byte lanes when E is a multiple of 4):
//   range_kernel      per (row chunk, expert group): partial min / max
//   hist_kernel       per (row chunk, expert group): the group's range from
//                     the partials, an LDS histogram with integer LDS
//                     atomics, written out as that chunk's partial counts
//   quantile_kernel   one block per expert: sums the chunk partials bin by
//                     bin, finds the rank's bin with a wavefront scan and a
//                     ballot, and evaluates Q_e in fp64
//   bias_kernel       one block: the mean of Q in a fixed order, the bias
// Integer counts make the histogram independent of the grid and of the
// order of the atomics, so the result is bitwise reproducible.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kGroup = 32;      // experts per block: 128 bytes of a row
constexpr int kThreads = 1024;
constexpr int kUnroll = 4;      // row loads in flight per thread
constexpr int kMaxBins = 1024;
constexpr int kRangeRows = 1024;

struct BiasArgs {
  const float* logits;
  int64_t T;
  int E, k, nb;
  int rows2;             // rows per hist_kernel block
  int c1, c2;            // row chunks of range_kernel and hist_kernel
  float* range_part;     // [c1][E][2]
  uint32_t* hist_part;   // [c2][E][nb]
  float* lohi;           // [E][2]
  double* q;             // [E]
  int32_t* hist_out;     // [E][nb] or null
  float* lohi_out;       // [E][2] or null
  float* bias;           // [E]
};

// V logits per lane: 4 when every row is 16-byte aligned, else 1.
template <int V>
struct RowMap {
  static constexpr int kLanesPerRow = kGroup / V;
  static constexpr int kRowsPerPass = kThreads / kLanesPerRow;
  int q, rr;
  __device__ RowMap() : q(threadIdx.x % kLanesPerRow), rr(threadIdx.x / kLanesPerRow) {}
};

template <int V>
__device__ __forceinline__ void load_row(const float* p, bool ok, float* v) {
  if constexpr (V == 4) {
    float4 x = ok ? *reinterpret_cast<const float4*>(p) : make_float4(0.f, 0.f, 0.f, 0.f);
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
  } else {
    v[0] = ok ? *p : 0.f;
  }
}

template <int V>
__global__ __launch_bounds__(kThreads) void range_kernel(BiasArgs a) {
  using M = RowMap<V>;
  const M m;
  const int e0 = blockIdx.y * kGroup + m.q * V;
  const bool col_ok = e0 < a.E;  // V = 4 needs E % 4 == 0: all V columns or none
  const int64_t t0 = (int64_t)blockIdx.x * kRangeRows;
  const int64_t t1 = min(a.T, t0 + kRangeRows);
  float mn[V], mx[V];
#pragma unroll
  for (int x = 0; x < V; ++x) mn[x] = INFINITY, mx[x] = -INFINITY;
  for (int64_t base = t0 + m.rr; base < t1; base += (int64_t)M::kRowsPerPass * kUnroll) {
    float v[kUnroll][V];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t t = base + (int64_t)u * M::kRowsPerPass;
      load_row<V>(a.logits + t * a.E + e0, col_ok && t < t1, v[u]);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (base + (int64_t)u * M::kRowsPerPass < t1) {
#pragma unroll
        for (int x = 0; x < V; ++x) mn[x] = fminf(mn[x], v[u][x]), mx[x] = fmaxf(mx[x], v[u][x]);
      }
    }
  }
  // lanes with equal q hold the same experts: fold the wavefront's rows
#pragma unroll
  for (int s = M::kLanesPerRow; s < 64; s <<= 1)
#pragma unroll
    for (int x = 0; x < V; ++x) mn[x] = fminf(mn[x], __shfl_xor(mn[x], s)), mx[x] = fmaxf(mx[x], __shfl_xor(mx[x], s));
  __shared__ float smn[kThreads / 64][kGroup], smx[kThreads / 64][kGroup];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane < M::kLanesPerRow) {
#pragma unroll
    for (int x = 0; x < V; ++x) smn[wave][lane * V + x] = mn[x], smx[wave][lane * V + x] = mx[x];
  }
  __syncthreads();
  if (threadIdx.x < kGroup) {
    const int e = blockIdx.y * kGroup + threadIdx.x;
    float lo = INFINITY, hi = -INFINITY;
    for (int w = 0; w < kThreads / 64; ++w) lo = fminf(lo, smn[w][threadIdx.x]), hi = fmaxf(hi, smx[w][threadIdx.x]);
    if (e < a.E) {
      float* p = a.range_part + ((int64_t)blockIdx.x * a.E + e) * 2;
      p[0] = lo;
      p[1] = hi;
    }
  }
}

template <int V, int kBins>  // kBins: the most bins the LDS histogram holds
__global__ __launch_bounds__(kThreads) void hist_kernel(BiasArgs a) {
  using M = RowMap<V>;
  constexpr int kPitch = kBins + 1;  // words per expert row of the LDS histogram
  __shared__ uint32_t h[kGroup * kPitch];
  __shared__ float s_lo[kGroup], s_scale[kGroup];
  __shared__ float s_pmn[kThreads / kGroup][kGroup], s_pmx[kThreads / kGroup][kGroup];
  const int g0 = blockIdx.y * kGroup;
  {
    // thread (c0, el) folds chunks c0, c0 + 32, ... of expert g0 + el
    const int el = threadIdx.x % kGroup, c0 = threadIdx.x / kGroup;
    const int e = g0 + el;
    float lo = INFINITY, hi = -INFINITY;
    if (e < a.E) {
      for (int c = c0; c < a.c1; c += kThreads / kGroup) {
        const float* p = a.range_part + ((int64_t)c * a.E + e) * 2;
        lo = fminf(lo, p[0]);
        hi = fmaxf(hi, p[1]);
      }
    }
    s_pmn[c0][el] = lo;
    s_pmx[c0][el] = hi;
  }
  __syncthreads();
  if (threadIdx.x < kGroup) {
    const int e = g0 + threadIdx.x;
    float lo = 0.f, hi = 0.f;
    if (e < a.E) {
      lo = INFINITY, hi = -INFINITY;
      for (int c = 0; c < kThreads / kGroup; ++c) lo = fminf(lo, s_pmn[c][threadIdx.x]), hi = fmaxf(hi, s_pmx[c][threadIdx.x]);
      if (blockIdx.x == 0) {
        a.lohi[2 * e] = lo, a.lohi[2 * e + 1] = hi;
        if (a.lohi_out) a.lohi_out[2 * e] = lo, a.lohi_out[2 * e + 1] = hi;
      }
    }
    // the exact difference of two fp32 values, one fp64 quotient, then fp32
    const double width = (double)hi - (double)lo;
    s_lo[threadIdx.x] = lo;
    s_scale[threadIdx.x] = width > 0.0 ? (float)((double)a.nb / width) : 0.f;
  }
  for (int i = threadIdx.x; i < kGroup * kPitch; i += kThreads) h[i] = 0;
  __syncthreads();
  const M m;
  const int el0 = m.q * V;
  const bool col_ok = g0 + el0 < a.E;
  float lo[V], sc[V];
#pragma unroll
  for (int x = 0; x < V; ++x) lo[x] = s_lo[el0 + x], sc[x] = s_scale[el0 + x];
  const int64_t t0 = (int64_t)blockIdx.x * a.rows2;
  const int64_t t1 = min(a.T, t0 + a.rows2);
  const int last = a.nb - 1;
  const float fnb = (float)a.nb;
  for (int64_t base = t0 + m.rr; base < t1; base += (int64_t)M::kRowsPerPass * kUnroll) {
    float v[kUnroll][V];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t t = base + (int64_t)u * M::kRowsPerPass;
      load_row<V>(a.logits + t * a.E + g0 + el0, col_ok && t < t1, v[u]);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (col_ok && base + (int64_t)u * M::kRowsPerPass < t1) {
#pragma unroll
        for (int x = 0; x < V; ++x) {
          const float d = v[u][x] - lo[x];  // >= 0: v is inside the column's range
          const float p = d * sc[x];        // inf only when the scale overflowed and d > 0
          const int b = d == 0.f ? 0 : (p >= fnb ? last : (int)p);
          atomicAdd(&h[(el0 + x) * kPitch + b], 1u);
        }
      }
    }
  }
  __syncthreads();
  uint32_t* out = a.hist_part + ((int64_t)blockIdx.x * a.E + g0) * a.nb;
  const int n_e = min(kGroup, a.E - g0);
  for (int i = threadIdx.x; i < n_e * a.nb; i += kThreads) {
    const int el = i / a.nb, b = i - el * a.nb;
    out[i] = h[el * kPitch + b];
  }
}

__device__ __forceinline__ int64_t wave_incl_scan(int64_t v, int lane) {
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) {
    const int64_t o = __shfl_up(v, s);
    if (lane >= s) v += o;
  }
  return v;
}

// Q_e = lo + (j + (r - C_{j-1}) / h_j) * (hi - lo) / nb, each operation
// rounded on its own (no contraction into a fused multiply-add).
__device__ __noinline__ double interp_quantile(float lo, float hi, int nb, int64_t j, int64_t c_prev, int64_t h,
                                               int64_t r_num, int E) {
#pragma clang fp contract(off)
  const double r = (double)r_num / (double)E;
  const double frac = (r - (double)c_prev) / (double)h;
  const double width = ((double)hi - (double)lo) / (double)nb;
  return (double)lo + ((double)j + frac) * width;
}

// Sum of the chunk partials of one bin: independent loads, 8 in flight.
__device__ __forceinline__ int64_t bin_total(const uint32_t* p, int64_t stride, int n) {
  uint32_t s[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  int c = 0;
  for (; c + 8 <= n; c += 8) {
#pragma unroll
    for (int u = 0; u < 8; ++u) s[u] += p[(c + u) * stride];
  }
  for (; c < n; ++c) s[0] += p[c * stride];
  int64_t t = 0;
#pragma unroll
  for (int u = 0; u < 8; ++u) t += s[u];
  return t;
}

// One block per expert: its threads total the chunk partials of every bin
// into LDS, then one wavefront scans the bins for the rank.
__global__ __launch_bounds__(256) void quantile_kernel(BiasArgs a) {
  __shared__ uint32_t cnt_s[kMaxBins];
  const int e = blockIdx.x;
  const int64_t stride = (int64_t)a.E * a.nb;
  for (int b = threadIdx.x; b < a.nb; b += 256) {
    const int64_t c = bin_total(a.hist_part + (int64_t)e * a.nb + b, stride, a.c2);
    cnt_s[b] = (uint32_t)c;
    if (a.hist_out) a.hist_out[(int64_t)e * a.nb + b] = (int32_t)c;
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int64_t r_num = (int64_t)(a.E - a.k) * a.T;  // rank r = r_num / E
    int64_t running = 0;
    int64_t j = -1, c_prev = 0, hj = 0;
    for (int i = 0; i < a.nb && j < 0; i += 64) {
      const int b = i + lane;
      const int64_t cnt = b < a.nb ? (int64_t)cnt_s[b] : 0;
      const int64_t incl = wave_incl_scan(cnt, lane);
      const int64_t cum = running + incl;
      const uint64_t hit = __ballot(b < a.nb && cum * a.E >= r_num);
      if (hit) {
        const int f = __ffsll((unsigned long long)hit) - 1;
        const int64_t cf = __shfl(cum, f), hf = __shfl(cnt, f);
        j = i + f;
        c_prev = cf - hf;
        hj = hf;
      }
      running += __shfl(incl, 63);
    }
    if (lane == 0) a.q[e] = interp_quantile(a.lohi[2 * e], a.lohi[2 * e + 1], a.nb, j, c_prev, hj, r_num, a.E);
  }
}

// One block: the mean of Q in a fixed order, then bias = mean - Q.
__global__ __launch_bounds__(256) void bias_kernel(BiasArgs a) {
  __shared__ double part[256];
  double s = 0.0;
  for (int i = threadIdx.x; i < a.E; i += 256) s += a.q[i];
  part[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  const double mean = part[0] / (double)a.E;
  for (int i = threadIdx.x; i < a.E; i += 256) a.bias[i] = (float)(mean - a.q[i]);
}

struct BiasLayout {
  int64_t c1, c2, rows2;
  int64_t range_off, hist_off, lohi_off, q_off, total;
};

int64_t up256(int64_t x) { return (x + 255) & ~int64_t(255); }

BiasLayout layout(int64_t T, int E, int nb) {
  BiasLayout l;
  l.rows2 = nb * 2 > 1024 ? nb * 2 : 1024;
  l.c1 = (T + kRangeRows - 1) / kRangeRows;
  l.c2 = (T + l.rows2 - 1) / l.rows2;
  l.range_off = 0;
  l.hist_off = up256(l.c1 * E * 2 * 4);
  l.lohi_off = l.hist_off + up256(l.c2 * E * (int64_t)nb * 4);
  l.q_off = l.lohi_off + up256((int64_t)E * 2 * 4);
  l.total = l.q_off + up256((int64_t)E * 8);
  return l;
}

}  // namespace

int bias_max_bins() { return kMaxBins; }

int64_t bias_ws_bytes(int64_t T, int E, int nb) { return layout(T, E, nb).total; }

hipError_t launch_bias_update(const float* logits, int64_t T, int E, int k, int nb, float* bias, int32_t* hist_out,
                              float* lohi_out, void* ws, hipStream_t s, void* const* events) {
  const BiasLayout l = layout(T, E, nb);
  char* w = static_cast<char*>(ws);
  BiasArgs a;
  a.logits = logits;
  a.T = T;
  a.E = E;
  a.k = k;
  a.nb = nb;
  a.rows2 = (int)l.rows2;
  a.c1 = (int)l.c1;
  a.c2 = (int)l.c2;
  a.range_part = reinterpret_cast<float*>(w + l.range_off);
  a.hist_part = reinterpret_cast<uint32_t*>(w + l.hist_off);
  a.lohi = reinterpret_cast<float*>(w + l.lohi_off);
  a.q = reinterpret_cast<double*>(w + l.q_off);
  a.hist_out = hist_out;
  a.lohi_out = lohi_out;
  a.bias = bias;
  // events[i] (when given) is recorded before launch i and events[4] after the last
  int next = 0;
  auto mark = [&]() -> hipError_t {
    return events ? hipEventRecord(static_cast<hipEvent_t>(events[next++]), s) : hipSuccess;
  };
  const unsigned groups = (unsigned)((E + kGroup - 1) / kGroup);
  const bool vec = (E % 4 == 0) && (reinterpret_cast<uintptr_t>(logits) % 16 == 0);
  hipError_t e;
  if ((e = mark()) != hipSuccess) return e;
  if (vec)
    range_kernel<4><<<dim3((unsigned)l.c1, groups), kThreads, 0, s>>>(a);
  else
    range_kernel<1><<<dim3((unsigned)l.c1, groups), kThreads, 0, s>>>(a);
  if ((e = mark()) != hipSuccess) return e;
  const dim3 hgrid((unsigned)l.c2, groups);
  if (nb <= 256) {  // a 33 KB histogram: several blocks per CU
    if (vec)
      hist_kernel<4, 256><<<hgrid, kThreads, 0, s>>>(a);
    else
      hist_kernel<1, 256><<<hgrid, kThreads, 0, s>>>(a);
  } else {
    if (vec)
      hist_kernel<4, kMaxBins><<<hgrid, kThreads, 0, s>>>(a);
    else
      hist_kernel<1, kMaxBins><<<hgrid, kThreads, 0, s>>>(a);
  }
  if ((e = mark()) != hipSuccess) return e;
  quantile_kernel<<<(unsigned)E, 256, 0, s>>>(a);
  if ((e = mark()) != hipSuccess) return e;
  bias_kernel<<<1, 256, 0, s>>>(a);
  if ((e = mark()) != hipSuccess) return e;
  return hipGetLastError();
}

}  // namespace moe
