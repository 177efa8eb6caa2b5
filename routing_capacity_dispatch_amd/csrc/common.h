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

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 (lo in the low half), round to nearest even: one
// v_cvt_pk_bf16_f32.  On every finite input it equals adding 0x7FFF plus
// the lowest kept bit to the fp32 bit pattern and keeping the high half
// (checked over all finite fp32 patterns on the device).
__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// fp32 -> bf16, round to nearest even (inputs are finite)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return static_cast<uint16_t>(bf16_pair(f, 0.0f)); }

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

// Streaming load for data read once per step (nontemporal hint: the lines
// are not kept in the caches for reuse)
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16_stream(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Wait for every vector memory operation of the wavefront (vmcnt(0); the
// other counters left alone), as an instruction the compiler's own wait
// placement takes into account, unlike a wait written in inline assembly
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Streaming store of data the next kernel reads once (nontemporal hint)
__device__ __forceinline__ void st16_stream(void* p, const uint4& v) {
  __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4_t*>(p));
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
    w[i] = bf16_pair(in[2 * i], in[2 * i + 1]);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

template <typename T>
struct Chunk {
  static constexpr int kElems = 16 / (int)sizeof(T);
};

// 1 / (1 + e^-a) with the hardware reciprocal (about 1 ulp): every SwiGLU
// output is rounded to bf16 or checked at fp32 tolerance, and a correctly
// rounded division costs ten more instructions per output in the GEMM
// epilogues.  a -> -inf: e^-a = inf, reciprocal 0.
__device__ __forceinline__ float sigmoid(float a) { return __builtin_amdgcn_rcpf(1.0f + __expf(-a)); }
__device__ __forceinline__ float silu(float a) { return a * sigmoid(a); }

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

// Lane `l`'s 64-bit value (l wave-uniform), read into scalar registers.
__device__ __forceinline__ int64_t readlane64(int64_t v, int l) {
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint64_t>(v)), l);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint64_t>(v) >> 32), l);
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Lane `src`'s 64-bit value, broadcast to the wavefront.
__device__ __forceinline__ int64_t shfl64(int64_t v, int src) {
  const uint32_t lo = __shfl(static_cast<uint32_t>(v), src);
  const uint32_t hi = __shfl(static_cast<uint32_t>(static_cast<uint64_t>(v) >> 32), src);
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

// One wavefront: dst = sum over j < k of g_j * rows[r_j], where lane j holds
// (r_j, g_j) in (row, g) and r_j < 0 adds nothing; fp32 accumulation in j
// order, stored as T.  Rows are row_bytes (a multiple of 16) apart from
// base.  Two rows' loads are in flight per step.  Each row is read once, so
// the reads carry the nontemporal hint.
// Every load is unconditional (a branch between loads makes the compiler
// wait for all earlier loads before the next): a dropped assignment reads
// one of the token's kept rows with weight 0 (adding +-0 leaves every sum
// unchanged, and kept rows are finite), and chunk indices past the row's end
// are clamped and not stored.  A token with no kept row gets zeros.
template <typename T>
__device__ __forceinline__ void combine_rows(const char* __restrict__ base, int64_t row, float g, int k,
                                             int64_t row_bytes, char* __restrict__ dst) {
  constexpr int EPC = Chunk<T>::kElems;
  constexpr int CPL = 6;  // 16-byte chunks per lane per pass: a 3072-wide bf16 row in one pass
  const int lane = threadIdx.x & 63;
  const int chunks = (int)(row_bytes / 16);
  const uint64_t kept = ballot64(lane < k && row >= 0);
  if (kept == 0) {
    for (int c = lane; c < chunks; c += 64) st16(dst + (int64_t)c * 16, make_uint4(0, 0, 0, 0));
    return;
  }
  const int64_t stand_in = shfl64(row, __builtin_ctzll(kept));
  const int64_t r_l = (lane < k && row >= 0) ? row : stand_in;
  const float g_l = (lane < k && row >= 0) ? g : 0.0f;
  for (int seg = 0; seg < chunks; seg += 64 * CPL) {
    float acc[CPL][EPC];
#pragma unroll
    for (int i = 0; i < CPL; ++i)
#pragma unroll
      for (int q = 0; q < EPC; ++q) acc[i][q] = 0.0f;
    for (int j = 0; j < k; j += 2) {
      // the two rows' addresses and gates are wave-uniform: scalar registers
      const int j1 = j + 1 < k ? j + 1 : j;
      const char* p0 = base + readlane64(r_l, j) * row_bytes;
      const char* p1 = base + readlane64(r_l, j1) * row_bytes;
      const float g0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(g_l), j));
      const float g1 = j + 1 < k ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(g_l), j1)) : 0.0f;
      uint4 v0[CPL], v1[CPL];
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const uint32_t c = (uint32_t)min(seg + i * 64 + lane, chunks - 1) * 16u;
        v0[i] = ld16_stream(p0 + c);
        v1[i] = ld16_stream(p1 + c);
      }
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        float f[EPC];
        unpack(v0[i], f, T{});
#pragma unroll
        for (int q = 0; q < EPC; ++q) acc[i][q] = fmaf(g0, f[q], acc[i][q]);
        unpack(v1[i], f, T{});
#pragma unroll
        for (int q = 0; q < EPC; ++q) acc[i][q] = fmaf(g1, f[q], acc[i][q]);
      }
    }
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = seg + i * 64 + lane;
      if (c < chunks) st16(dst + (int64_t)c * 16, pack(acc[i], T{}));
    }
  }
}

// One wavefront: copy the row at src to each destination named by lanes
// 0..k-1 (dst_j = nullptr: none).  16-byte chunks.
__device__ __forceinline__ void scatter_row(const char* __restrict__ src, char* dst, int k, int64_t row_bytes) {
  const int lane = threadIdx.x & 63;
  const int chunks = (int)(row_bytes / 16);
  for (int seg = 0; seg < chunks; seg += 64 * 8) {
    uint4 r[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)  // clamped past the row's end (not stored): no branch between the loads
      r[i] = ld16(src + (int64_t)min(seg + i * 64 + lane, chunks - 1) * 16);
    for (int j = 0; j < k; ++j) {
      char* d = reinterpret_cast<char*>(shfl64(reinterpret_cast<int64_t>(dst), j));
      if (!d) continue;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int c = seg + i * 64 + lane;
        if (c < chunks) st16(d + (int64_t)c * 16, r[i]);
      }
    }
  }
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
