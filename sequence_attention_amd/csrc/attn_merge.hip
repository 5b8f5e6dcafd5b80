// Online-softmax merge of partial attention results (gfx950).
//
// SGLang "Parallelism Overview": ring attention keeps Q in place while K/V
// rotate; every hop yields a partial (O, LSE) over a disjoint key set, and
// the partials -- also replicated-prefix and tail-padded parts -- are
// combined with the online-softmax rule, which is why a ring-capable kernel
// must expose its LSE ("Constraints").  For one row, with m = max(La, Lp)
// and w = exp(L - m):
//   L = m + ln(wa + wp),  O = (wa Oa + wp Op) / (wa + wp).
// A side with L = -inf holds no keys and is selected away (never
// multiplied), so NaN or stale data in an empty accumulator cannot leak.
//
// HBM-bound: per row the kernel reads two O rows and two LSE values and
// writes one of each.  One thread owns 8 consecutive elements of a row
// (16 bytes of bf16 / 32 bytes of fp32); the D/8 threads of a row read the
// same two LSE values (one cache line serves many rows), and the row's
// first thread writes the merged LSE.  O moves with non-temporal loads and
// stores (touched once).
#include "dit_internal.h"

namespace dit {
namespace {

constexpr int kThreads = 256;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t x = __float_as_uint(f);
  if ((x & 0x7fffffffu) > 0x7f800000u) return (x >> 16) | 0x40u;
  return (x + 0x7fffu + ((x >> 16) & 1u)) >> 16;
}

template <bool kF32>
__global__ __launch_bounds__(kThreads) void merge_kernel(void* __restrict__ o_acc, float* __restrict__ lse_acc,
                                                         const void* __restrict__ o_part,
                                                         const float* __restrict__ lse_part, int32_t Sq,
                                                         int32_t H, uint32_t chunks_per_row,
                                                         FastDiv div_chunks, FastDiv div_h, FastDiv div_sq,
                                                         uint32_t total_chunks) {
  const uint32_t idx = blockIdx.x * kThreads + threadIdx.x;
  if (idx >= total_chunks) return;
  const uint32_t row = fdiv(idx, div_chunks);          // row of [B, Sq, H]
  const uint32_t chunk = idx - row * chunks_per_row;
  const uint32_t bi = fdiv(row, div_h);                 // b * Sq + i
  const uint32_t h = row - bi * H;
  const uint32_t b = fdiv(bi, div_sq);
  const uint32_t i = bi - b * Sq;
  const size_t lse_idx = ((size_t)b * H + h) * Sq + i;  // LSE is [B, H, Sq]

  const float la = lse_acc[lse_idx];
  const float lp = lse_part[lse_idx];
  const float m = fmaxf(la, lp);
  const bool empty = (m == -INFINITY);
  const bool use_a = (la != -INFINITY);
  const bool use_p = (lp != -INFINITY);
  const float wa = use_a ? __expf(la - m) : 0.0f;
  const float wp = use_p ? __expf(lp - m) : 0.0f;
  const float wsum = wa + wp;
  const float inv = empty ? 0.0f : 1.0f / wsum;
  const float ca = wa * inv, cp = wp * inv;

  float xa[8], xp[8], r[8];
  if constexpr (kF32) {
    const f32x4* pa = reinterpret_cast<const f32x4*>(o_acc) + (size_t)idx * 2;
    const f32x4* pp = reinterpret_cast<const f32x4*>(o_part) + (size_t)idx * 2;
    const f32x4 a0 = __builtin_nontemporal_load(pa), a1 = __builtin_nontemporal_load(pa + 1);
    const f32x4 p0 = __builtin_nontemporal_load(pp), p1 = __builtin_nontemporal_load(pp + 1);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      xa[e] = a0[e]; xa[4 + e] = a1[e];
      xp[e] = p0[e]; xp[4 + e] = p1[e];
    }
  } else {
    const u32x4 a = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(o_acc) + idx);
    const u32x4 p = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(o_part) + idx);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      xa[2 * w] = bf16_lo(a[w]); xa[2 * w + 1] = bf16_hi(a[w]);
      xp[2 * w] = bf16_lo(p[w]); xp[2 * w + 1] = bf16_hi(p[w]);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float ta = use_a ? ca * xa[e] : 0.0f;
    const float tp = use_p ? cp * xp[e] : 0.0f;
    r[e] = ta + tp;
  }
  if constexpr (kF32) {
    f32x4* pa = reinterpret_cast<f32x4*>(o_acc) + (size_t)idx * 2;
    __builtin_nontemporal_store(f32x4{r[0], r[1], r[2], r[3]}, pa);
    __builtin_nontemporal_store(f32x4{r[4], r[5], r[6], r[7]}, pa + 1);
  } else {
    u32x4 out;
#pragma unroll
    for (int w = 0; w < 4; ++w) out[w] = f32_to_bf16_rne(r[2 * w]) | (f32_to_bf16_rne(r[2 * w + 1]) << 16);
    __builtin_nontemporal_store(out, reinterpret_cast<u32x4*>(o_acc) + idx);
  }
  if (chunk == 0) lse_acc[lse_idx] = empty ? -INFINITY : m + __logf(wsum);
}

}  // namespace

hipError_t launch_attn_merge(void* o_acc, float* lse_acc, const void* o_part, const float* lse_part,
                             int32_t B, int32_t Sq, int32_t H, int32_t D, bool o_f32,
                             hipStream_t stream) {
  const uint32_t chunks_per_row = (uint32_t)D / 8;
  const uint64_t total = (uint64_t)B * Sq * H * chunks_per_row;  // < 2^31: checked by the ABI layer
  if (total == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((total + kThreads - 1) / kThreads);
  const FastDiv dc = make_fastdiv(chunks_per_row), dh = make_fastdiv((uint32_t)H),
                dsq = make_fastdiv((uint32_t)Sq);
  if (o_f32)
    merge_kernel<true><<<blocks, kThreads, 0, stream>>>(o_acc, lse_acc, o_part, lse_part, Sq, H,
                                                        chunks_per_row, dc, dh, dsq, (uint32_t)total);
  else
    merge_kernel<false><<<blocks, kThreads, 0, stream>>>(o_acc, lse_acc, o_part, lse_part, Sq, H,
                                                         chunks_per_row, dc, dh, dsq, (uint32_t)total);
  return hipGetLastError();
}

}  // namespace dit
