// Gate-weighted combine: y_lat[t] = sum over receiver-kept j of
// g[t,j] * expert_out[row(t,j)], fp32 accumulation in j order, no
// renormalisation of the gates.  One wavefront per token, 16-byte chunks,
// up to 8 chunks per lane per pass.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  constexpr int EPC = Chunk<T>::kElems;  // elements per 16-byte chunk
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  const int k = a.k, epp = a.E / a.P;
  const int64_t w = t / a.Tw;
  const int chunks = (int)(a.row_bytes / 16);
  char* dst = static_cast<char*>(a.y) + t * a.row_bytes;
  for (int seg = 0; seg < chunks; seg += 64 * 8) {
    float acc[8][EPC];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int q = 0; q < EPC; ++q) acc[i][q] = 0.0f;
    for (int j = 0; j < k; ++j) {
      if (a.recv_slot[t * k + j] < 0) continue;
      const int e = a.topk[t * k + j];
      const int ps = a.pool_slot[t * k + j];
      if (e < 0 || e >= a.E || ps < 0 || ps >= a.cap_send) continue;  // malformed: skipped
      const float g = a.gates[t * k + j];
      const int p = e / epp;
      const int64_t row = (w * a.P + p) * a.cap_send + ps;
      const char* src = a.expert_out + row * a.row_bytes;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int c = seg + i * 64 + lane;
        if (c < chunks) {
          float v[EPC];
          unpack(ld16(src + (int64_t)c * 16), v, T{});
#pragma unroll
          for (int q = 0; q < EPC; ++q) acc[i][q] = fmaf(g, v[q], acc[i][q]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = seg + i * 64 + lane;
      if (c < chunks) st16(dst + (int64_t)c * 16, pack(acc[i], T{}));
    }
  }
}

}  // namespace

hipError_t launch_combine(int dt, const CombineArgs& a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  const unsigned blocks = (unsigned)((a.T + 3) / 4);
  if (dt == DT_BF16)
    combine_kernel<bf16_t><<<blocks, 256, 0, s>>>(a);
  else
    combine_kernel<float><<<blocks, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace moe
