// Shader-clock probe: a measurement aid for reporting the clock a timed run
// sustained (no page defines it).  Each workgroup reads the shader cycle
// counter (s_memtime) and the constant 100 MHz real-time counter
// (s_memrealtime) around a loop of work, and thread 0 writes the two
// deltas; the host divides one by the other.  The loop is either a chain of
// dependent FMAs (a light load: the clock the device idles up to) or
// back-to-back bf16 MFMAs on every wave (the matrix-core load attention
// puts on the chip, under which the power limit sets the clock).
#include "dit_internal.h"

namespace dit {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <bool kMfma>
__global__ __launch_bounds__(256) void clock_probe_kernel(int64_t* out, int32_t spin) {
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  float live;
  if constexpr (kMfma) {
    // four independent accumulators keep the matrix pipe of each SIMD full;
    // the operands are pseudo-random bf16 values of either sign in [1, 2)
    // with all mantissa bits in play (operands with empty mantissas, such as
    // small multiples of 1/8, draw visibly less power and let the clock
    // stay higher than attention's score and value data do)
    bf16x8 a, b;
    uint32_t h = threadIdx.x * 0x9E3779B9u + blockIdx.x * 0x85EBCA6Bu + 1u;
    for (int e = 0; e < 8; ++e) {
      h ^= h << 13;
      h ^= h >> 17;
      h ^= h << 5;
      a[e] = __builtin_bit_cast(__bf16, (uint16_t)((h & 0x807Fu) | 0x3F80u));
      b[e] = __builtin_bit_cast(__bf16, (uint16_t)(((h >> 16) & 0x807Fu) | 0x3F80u));
    }
    f32x16 acc[4];
    for (int j = 0; j < 4; ++j)
      for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;
    for (int i = 0; i < spin; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
    }
    live = acc[0][0] + acc[1][1] + acc[2][2] + acc[3][3];
  } else {
    float x = (float)threadIdx.x * 1e-3f, y = 1.0f;
    for (int i = 0; i < spin; ++i) {
      x = __builtin_fmaf(x, 0.999f, y);
      y = __builtin_fmaf(y, 0.999f, x);
    }
    live = x + y;
  }
  const uint64_t c1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    out[2 * blockIdx.x] = (int64_t)(c1 - c0);
    out[2 * blockIdx.x + 1] = (int64_t)(r1 - r0);
  }
  if (live == 12345.678f) out[0] = -1;  // keeps the loop's results live
}

}  // namespace

hipError_t launch_clock_probe(int64_t* out, int32_t workgroups, int32_t spin, bool mfma,
                              hipStream_t stream) {
  if (mfma) clock_probe_kernel<true><<<workgroups, 256, 0, stream>>>(out, spin);
  else clock_probe_kernel<false><<<workgroups, 256, 0, stream>>>(out, spin);
  return hipGetLastError();
}

}  // namespace dit
