// Device helpers shared by the gfx950 kernels of the MoE branch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// bf16 storage is a raw 16-bit pattern
struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// fp32 -> bf16, round to nearest even (inputs are finite)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

template <typename T>
struct ElemOps;

template <>
struct ElemOps<float> {
  static constexpr int kBytes = 4;
  __device__ __forceinline__ static float to_f32(float v) { return v; }
};

template <>
struct ElemOps<bf16_t> {
  static constexpr int kBytes = 2;
};

// 16-byte global/LDS accesses
__device__ __forceinline__ uint4 ld16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}
__device__ __forceinline__ void st16(void* p, const uint4& v) {
  *reinterpret_cast<uint4*>(p) = v;
}

// Unpack a 16-byte chunk of T into floats: 4 (f32) or 8 (bf16) values.
__device__ __forceinline__ void unpack(const uint4& v, float* out, float) {
  out[0] = __uint_as_float(v.x);
  out[1] = __uint_as_float(v.y);
  out[2] = __uint_as_float(v.z);
  out[3] = __uint_as_float(v.w);
}
__device__ __forceinline__ void unpack(const uint4& v, float* out, bf16_t) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ uint4 pack(const float* in, float) {
  return make_uint4(__float_as_uint(in[0]), __float_as_uint(in[1]),
                    __float_as_uint(in[2]), __float_as_uint(in[3]));
}
__device__ __forceinline__ uint4 pack(const float* in, bf16_t) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = static_cast<uint32_t>(f32_to_bf16(in[2 * i])) |
           (static_cast<uint32_t>(f32_to_bf16(in[2 * i + 1])) << 16);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

template <typename T>
struct Chunk {
  static constexpr int kElems = 16 / (int)sizeof(T);
};

__device__ __forceinline__ float silu(float a) { return a / (1.0f + __expf(-a)); }

__device__ __forceinline__ uint64_t ballot64(bool p) {
  return __ballot(p);
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = threadIdx.x & 63;
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Mask of the lanes of the wavefront whose `bits`-bit key equals this lane's,
// restricted to `active`.
__device__ __forceinline__ uint64_t match_key(uint32_t key, int bits, uint64_t active) {
  uint64_t m = active;
  for (int b = 0; b < bits; ++b) {
    const bool set = (key >> b) & 1u;
    const uint64_t bal = ballot64(set);
    m &= set ? bal : ~bal;
  }
  return m;
}

// Exclusive scan of one int per thread over a workgroup of 1024 threads
// (16 wavefronts).  part: 16 ints of LDS.  *total (LDS) receives the sum.
__device__ __forceinline__ int block_excl_scan_1024(int v, int* part, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(x, d);
    if (lane >= d) x += o;
  }
  if (lane == 63) part[w] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    int s = 0;
    for (int i = 0; i < 16; ++i) {
      const int t = part[i];
      part[i] = s;
      s += t;
    }
    *total = s;
  }
  __syncthreads();
  return x + part[w] - v;
}

}  // namespace moe
