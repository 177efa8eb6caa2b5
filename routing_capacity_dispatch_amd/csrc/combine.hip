// Gate-weighted combine: y_lat[t] = sum over receiver-kept j of
// g[t,j] * expert_out[row(t,j)], fp32 accumulation in j order, no
// renormalisation of the gates.  With gates == NULL every kept row has
// weight 1: the transpose of dispatch (a token's row gradient summed over
// the slots it was sent to).  One wavefront per token: its lanes load the
// token's k assignments at once, then the rows are read two at a time in
// 16-byte chunks.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  const int k = a.k, epp = a.E / a.P;
  const int64_t w = t / a.Tw;
  // lane j < k: the pool row and gate of the token's assignment j, all
  // loaded at once (an assignment whose expert id or pool slot is out of
  // range adds nothing)
  // (every lane loads: lanes past k re-read the last assignment, so no
  // branch separates the loads)
  const int64_t q = t * k + min(lane, k - 1);
  const int rs = a.recv_slot[q], e = a.topk[q], ps = a.pool_slot[q];
  const float gq = a.gates ? a.gates[q] : 1.0f;
  // (& rather than &&: no short-circuit branch to sink a load into)
  const bool ok = (lane < k) & (rs >= 0) & (e >= 0) & (e < a.E) & (ps >= 0) & (ps < a.cap_send);
  const int64_t row = ok ? (w * a.P + e / epp) * a.cap_send + ps : -1;
  const float g = ok ? gq : 0.0f;
  combine_rows<T>(a.expert_out, row, g, k, a.row_bytes,
                  static_cast<char*>(a.y) + t * (a.y_pitch ? a.y_pitch : a.row_bytes));
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
