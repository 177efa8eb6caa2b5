// Router selection: top-k by fl32(logit + bias) with ties to the lower expert
// index, and gates = softmax over the selected raw logits.
//
// One wavefront per token.  Lane l holds experts l, l+64, ... as unsigned
// keys that order the fp32 scores (0 marks an absent or taken expert).  Each
// of k rounds takes the wavefront's largest key (DPP within rows of 16
// lanes, then the four row results read into scalar registers) and, among
// the experts holding it, the lowest index (ballots: the first register
// slot with a match, then its lowest lane), so the experts come out in
// output order with ties to the lower index.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

// DPP controls: lane i of each row of 16 reads lane i^1, i^2 (quad
// permutes), 7-i within its half row, 15-i within its row
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

__device__ __forceinline__ uint32_t dpp_max(uint32_t v, int ctrl_sel) {
  uint32_t o;
  switch (ctrl_sel) {
    case 0: o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppXor1, 0xF, 0xF, false); break;
    case 1: o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppXor2, 0xF, 0xF, false); break;
    case 2: o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppHalfMirror, 0xF, 0xF, false); break;
    default: o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppMirror, 0xF, 0xF, false); break;
  }
  return o > v ? o : v;
}

// Largest value over the wavefront, wave-uniform.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int c = 0; c < 4; ++c) v = dpp_max(v, c);  // every lane: its row's max
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  const uint32_t a = r0 > r1 ? r0 : r1, b = r2 > r3 ? r2 : r3;
  return a > b ? a : b;
}

// Lane i^1, i^2, 7-i (half row), 15-i (row) of v, as a float.
__device__ __forceinline__ float dpp_f(float v, int ctrl_sel) {
  const int b = __float_as_int(v);
  switch (ctrl_sel) {
    case 0: return __int_as_float(__builtin_amdgcn_update_dpp(0, b, kDppXor1, 0xF, 0xF, false));
    case 1: return __int_as_float(__builtin_amdgcn_update_dpp(0, b, kDppXor2, 0xF, 0xF, false));
    case 2: return __int_as_float(__builtin_amdgcn_update_dpp(0, b, kDppHalfMirror, 0xF, 0xF, false));
    default: return __int_as_float(__builtin_amdgcn_update_dpp(0, b, kDppMirror, 0xF, 0xF, false));
  }
}
__device__ __forceinline__ float row_lane(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int c = 0; c < 4; ++c) v = fmaxf(v, dpp_f(v, c));
  return fmaxf(fmaxf(row_lane(v, 0), row_lane(v, 16)), fmaxf(row_lane(v, 32), row_lane(v, 48)));
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int c = 0; c < 4; ++c) v += dpp_f(v, c);
  return (row_lane(v, 0) + row_lane(v, 16)) + (row_lane(v, 32) + row_lane(v, 48));
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
  // every lane loads every slot (past E: the last expert again, unused), so
  // no branch separates the loads and they are all in flight together
  float v[NPER], b[NPER];
#pragma unroll
  for (int i = 0; i < NPER; ++i) v[i] = row[min(i * 64 + lane, E - 1)];
#pragma unroll
  for (int i = 0; i < NPER; ++i) b[i] = 0.0f;
  if (bias) {
#pragma unroll
    for (int i = 0; i < NPER; ++i) b[i] = bias[min(i * 64 + lane, E - 1)];
  }
  uint32_t key[NPER];
#pragma unroll
  for (int i = 0; i < NPER; ++i)
    // at least 1 (only one NaN pattern maps to 0), so with k <= E every
    // round finds a present expert
    key[i] = i * 64 + lane < E ? max(score_key(v[i] + b[i]), 1u) : 0u;
  int mine = -1;  // lane j < k ends with the j-th selected expert
  for (int j = 0; j < k; ++j) {
    uint32_t best = 0;
#pragma unroll
    for (int i = 0; i < NPER; ++i) best = key[i] > best ? key[i] : best;
    best = wave_max_u32(best);
    // lowest expert index holding the key: the first slot i with a match,
    // then its lowest lane
    int e = 0;
#pragma unroll
    for (int i = NPER - 1; i >= 0; --i) {
      const uint64_t hit = ballot64(key[i] == best);
      if (hit) e = i * 64 + __builtin_ctzll(hit);
    }
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
