// Router selection: top-k by fl32(logit + bias) with ties to the lower expert
// index, and gates = softmax over the selected raw logits.
//
// One wavefront per token.  Lane l holds experts l, l+64, ... as 64-bit keys
// (order-preserving fp32 score bits << 32 | ~expert), so a single unsigned
// max picks the highest score and, among equal scores, the lowest index.
// k rounds of a wavefront max select the experts in output order.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

__device__ __forceinline__ uint64_t shfl_xor64(uint64_t v, int m) {
  const uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), m);
  const uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), m);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

__device__ __forceinline__ uint64_t wave_max64(uint64_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const uint64_t o = shfl_xor64(v, m);
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

// Total order on finite fp32 scores as unsigned keys; -0 is mapped to +0.
__device__ __forceinline__ uint32_t score_key(float s) {
  if (s == 0.0f) s = 0.0f;
  const uint32_t u = __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int NPER>  // experts per lane: E <= 64 * NPER
__global__ __launch_bounds__(256) void topk_gates_kernel(const float* __restrict__ logits,
                                                         const float* __restrict__ bias,
                                                         int64_t T, int E, int k,
                                                         int32_t* __restrict__ topk,
                                                         float* __restrict__ gates) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + t * E;
  uint64_t key[NPER];
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const int e = i * 64 + lane;
    key[i] = 0;
    if (e < E) {
      const float s = row[e] + (bias ? bias[e] : 0.0f);
      key[i] = (static_cast<uint64_t>(score_key(s)) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(e));
    }
  }
  int mine = -1;  // lane j < k ends with the j-th selected expert
  for (int j = 0; j < k; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < NPER; ++i) best = key[i] > best ? key[i] : best;
    best = wave_max64(best);
    const int e = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(best));
    if ((e & 63) == lane) {
#pragma unroll
      for (int i = 0; i < NPER; ++i)
        if (i == (e >> 6)) key[i] = 0;
    }
    if (lane == j) mine = e;
  }
  const bool sel = lane < k;
  const float l = sel ? row[mine] : -INFINITY;
  const float m = wave_max(l);
  const float ex = sel ? expf(l - m) : 0.0f;
  const float sum = wave_sum(ex);
  if (sel) {
    topk[t * k + lane] = mine;
    gates[t * k + lane] = ex / sum;
  }
}

}  // namespace

hipError_t launch_topk_gates(const float* logits, const float* bias, int64_t T, int E, int k,
                             int32_t* topk_idx, float* gates, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const int64_t blocks = (T + 3) / 4;
  const dim3 grid((unsigned)blocks);
  const int nper = (E + 63) / 64;
  if (nper <= 1)
    topk_gates_kernel<1><<<grid, 256, 0, s>>>(logits, bias, T, E, k, topk_idx, gates);
  else if (nper <= 2)
    topk_gates_kernel<2><<<grid, 256, 0, s>>>(logits, bias, T, E, k, topk_idx, gates);
  else if (nper <= 4)
    topk_gates_kernel<4><<<grid, 256, 0, s>>>(logits, bias, T, E, k, topk_idx, gates);
  else if (nper <= 6)
    topk_gates_kernel<6><<<grid, 256, 0, s>>>(logits, bias, T, E, k, topk_idx, gates);
  else if (nper <= 8)
    topk_gates_kernel<8><<<grid, 256, 0, s>>>(logits, bias, T, E, k, topk_idx, gates);
  else
    topk_gates_kernel<16><<<grid, 256, 0, s>>>(logits, bias, T, E, k, topk_idx, gates);
  return hipGetLastError();
}

}  // namespace moe
