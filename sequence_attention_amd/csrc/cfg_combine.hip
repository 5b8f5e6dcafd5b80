// Classifier-free guidance combine (gfx950).
//
// edge-dit.cpp "Parallel execution", CFG parallelism section: after the
// all-gather of the two branch predictions, the guided prediction is
// p_uncond + g * (p_cond - p_uncond).  Evaluated per element as one fused
// multiply-add fmaf(g, p_cond - p_uncond, p_uncond) in fp32.
//
// HBM-bound elementwise pass: 16-byte vector loads of both inputs, one
// 16-byte store, several vectors per thread in flight.  `out` may alias an
// input exactly (each element is read before it is written by the same
// thread), so no restrict qualifiers.
#include "dit_internal.h"

namespace dit {
namespace {

constexpr int kThreads = 256;
constexpr int kVecPerThread = 4;

__global__ __launch_bounds__(kThreads) void cfg_f32_kernel(const float* u, const float* c, float* out,
                                                           int64_t n, float g) {
  const int64_t nvec = n >> 2;
  const int64_t base = (int64_t)blockIdx.x * (kThreads * kVecPerThread) + threadIdx.x;
  float4 uu[kVecPerThread], cc[kVecPerThread];
#pragma unroll
  for (int i = 0; i < kVecPerThread; ++i) {
    const int64_t v = base + (int64_t)i * kThreads;
    if (v < nvec) {
      uu[i] = reinterpret_cast<const float4*>(u)[v];
      cc[i] = reinterpret_cast<const float4*>(c)[v];
    }
  }
#pragma unroll
  for (int i = 0; i < kVecPerThread; ++i) {
    const int64_t v = base + (int64_t)i * kThreads;
    if (v < nvec) {
      float4 r;
      r.x = __builtin_fmaf(g, cc[i].x - uu[i].x, uu[i].x);
      r.y = __builtin_fmaf(g, cc[i].y - uu[i].y, uu[i].y);
      r.z = __builtin_fmaf(g, cc[i].z - uu[i].z, uu[i].z);
      r.w = __builtin_fmaf(g, cc[i].w - uu[i].w, uu[i].w);
      reinterpret_cast<float4*>(out)[v] = r;
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
  uint4 uu[kVecPerThread], cc[kVecPerThread];
#pragma unroll
  for (int i = 0; i < kVecPerThread; ++i) {
    const int64_t v = base + (int64_t)i * kThreads;
    if (v < nvec) {
      uu[i] = reinterpret_cast<const uint4*>(u)[v];
      cc[i] = reinterpret_cast<const uint4*>(c)[v];
    }
  }
#pragma unroll
  for (int i = 0; i < kVecPerThread; ++i) {
    const int64_t v = base + (int64_t)i * kThreads;
    if (v < nvec) {
      const uint32_t* pu = &uu[i].x;
      const uint32_t* pc = &cc[i].x;
      uint4 r;
      uint32_t* pr = &r.x;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float u0 = bf16_to_f32(pu[w] & 0xffffu), u1 = bf16_to_f32(pu[w] >> 16);
        const float c0 = bf16_to_f32(pc[w] & 0xffffu), c1 = bf16_to_f32(pc[w] >> 16);
        const uint32_t r0 = f32_to_bf16_rne(__builtin_fmaf(g, c0 - u0, u0));
        const uint32_t r1 = f32_to_bf16_rne(__builtin_fmaf(g, c1 - u1, u1));
        pr[w] = r0 | (r1 << 16);
      }
      reinterpret_cast<uint4*>(out)[v] = r;
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
