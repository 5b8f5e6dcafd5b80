// Classifier-free guidance combine (gfx950).
//
// edge-dit.cpp "Parallel execution", CFG parallelism section: after the
// all-gather of the two branch predictions, the guided prediction is
// p_uncond + g * (p_cond - p_uncond).  Evaluated per element as one fused
// multiply-add fmaf(g, p_cond - p_uncond, p_uncond) in fp32.
//
// HBM-bound elementwise pass: 16-byte non-temporal vector loads of both
// inputs and one 16-byte non-temporal store per thread.  `out` may alias an
// input exactly (each element is read before it is written by the same
// thread), so no restrict qualifiers.
#include "dit_internal.h"

namespace dit {
namespace {

constexpr int kThreads = 256;
constexpr int kVecPerThread = 1;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void cfg_f32_kernel(const float* u, const float* c, float* out,
                                                           int64_t n, float g) {
  const int64_t nvec = n >> 2;
  const int64_t base = (int64_t)blockIdx.x * (kThreads * kVecPerThread) + threadIdx.x;
  f32x4 uu[kVecPerThread], cc[kVecPerThread];
#pragma unroll
  for (int i = 0; i < kVecPerThread; ++i) {
    const int64_t v = base + (int64_t)i * kThreads;
    if (v < nvec) {
      uu[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(u) + v);
      cc[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(c) + v);
    }
  }
#pragma unroll
  for (int i = 0; i < kVecPerThread; ++i) {
    const int64_t v = base + (int64_t)i * kThreads;
    if (v < nvec) {
      f32x4 r;
#pragma unroll
      for (int e = 0; e < 4; ++e) r[e] = __builtin_fmaf(g, cc[i][e] - uu[i][e], uu[i][e]);
      __builtin_nontemporal_store(r, reinterpret_cast<f32x4*>(out) + v);
    }
  }
  // scalar tail (n % 4 elements), taken by the first threads of block 0
  if (blockIdx.x == 0 && threadIdx.x < (n & 3)) {
    const int64_t e = nvec * 4 + threadIdx.x;
    out[e] = __builtin_fmaf(g, c[e] - u[e], u[e]);
  }
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16 round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t x = __float_as_uint(f);
  if ((x & 0x7fffffffu) > 0x7f800000u) return (x >> 16) | 0x40u;
  return (x + 0x7fffu + ((x >> 16) & 1u)) >> 16;
}

__global__ __launch_bounds__(kThreads) void cfg_bf16_kernel(const uint16_t* u, const uint16_t* c,
                                                            uint16_t* out, int64_t n, float g) {
  const int64_t nvec = n >> 3;  // 8 bf16 per 16-byte vector
  const int64_t base = (int64_t)blockIdx.x * (kThreads * kVecPerThread) + threadIdx.x;
  u32x4 uu[kVecPerThread], cc[kVecPerThread];
#pragma unroll
  for (int i = 0; i < kVecPerThread; ++i) {
    const int64_t v = base + (int64_t)i * kThreads;
    if (v < nvec) {
      uu[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(u) + v);
      cc[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(c) + v);
    }
  }
#pragma unroll
  for (int i = 0; i < kVecPerThread; ++i) {
    const int64_t v = base + (int64_t)i * kThreads;
    if (v < nvec) {
      u32x4 r;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float u0 = bf16_to_f32(uu[i][w] & 0xffffu), u1 = bf16_to_f32(uu[i][w] >> 16);
        const float c0 = bf16_to_f32(cc[i][w] & 0xffffu), c1 = bf16_to_f32(cc[i][w] >> 16);
        const uint32_t r0 = f32_to_bf16_rne(__builtin_fmaf(g, c0 - u0, u0));
        const uint32_t r1 = f32_to_bf16_rne(__builtin_fmaf(g, c1 - u1, u1));
        r[w] = r0 | (r1 << 16);
      }
      __builtin_nontemporal_store(r, reinterpret_cast<u32x4*>(out) + v);
    }
  }
  if (blockIdx.x == 0 && threadIdx.x < (n & 7)) {
    const int64_t e = nvec * 8 + threadIdx.x;
    const float uf = bf16_to_f32(u[e]), cf = bf16_to_f32(c[e]);
    out[e] = (uint16_t)f32_to_bf16_rne(__builtin_fmaf(g, cf - uf, uf));
  }
}

int64_t blocks_for(int64_t nvec) {
  const int64_t per = kThreads * kVecPerThread;
  const int64_t b = (nvec + per - 1) / per;
  return b > 0 ? b : 1;
}

}  // namespace

hipError_t launch_cfg_combine_f32(const float* u, const float* c, float* out, int64_t n, float g,
                                  hipStream_t stream) {
  cfg_f32_kernel<<<(unsigned)blocks_for(n >> 2), kThreads, 0, stream>>>(u, c, out, n, g);
  return hipGetLastError();
}

hipError_t launch_cfg_combine_bf16(const uint16_t* u, const uint16_t* c, uint16_t* out, int64_t n,
                                   float g, hipStream_t stream) {
  cfg_bf16_kernel<<<(unsigned)blocks_for(n >> 3), kThreads, 0, stream>>>(u, c, out, n, g);
  return hipGetLastError();
}

}  // namespace dit
