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
// writes one of each.  A workgroup takes max(32, 2048 / D) consecutive query
// rows of one (batch, head): the LSE of those rows is one contiguous run of
// the [B, H, Sq] arrays (at least 128 bytes), read and written whole by one
// workgroup, while each O
// row (D contiguous elements) is read by D/8 threads of 8 elements (16
// bytes of bf16 / 32 bytes of fp32).  The threads of a row sit in one wave,
// which reads the row's two LSE values before its first thread writes the
// merged one (program order).  O moves with non-temporal loads and stores
// (touched once).
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

template <int D>
constexpr int rows_per_wg() {  // query rows per workgroup
  return (kThreads / (D / 8)) > 32 ? kThreads / (D / 8) : 32;
}

template <bool kF32, int D>
__global__ __launch_bounds__(kThreads) void merge_kernel(void* __restrict__ o_acc, float* __restrict__ lse_acc,
                                                         const void* __restrict__ o_part,
                                                         const float* __restrict__ lse_part, int32_t Sq,
                                                         int32_t H, int32_t row_blocks) {
  constexpr int kChunks = D / 8;                       // 8-element chunks per row
  constexpr int kRows = rows_per_wg<D>();
  constexpr int kPer = kRows * kChunks / kThreads;     // chunks per thread (1 to 8)
  constexpr int kRowsPerPass = kThreads / kChunks;
  const int bh = blockIdx.x / row_blocks;              // b * H + h
  const int i0 = (blockIdx.x - bh * row_blocks) * kRows;
  const int h = bh % H;
  const int b = bh / H;
  const int c = threadIdx.x % kChunks;
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int i = i0 + (int)threadIdx.x / kChunks + u * kRowsPerPass;
    if (i >= Sq) break;
    const size_t lse_idx = (size_t)bh * Sq + i;        // LSE is [B, H, Sq]
    const size_t chunk = (((size_t)b * Sq + i) * H + h) * kChunks + c;  // O is [B, Sq, H, D]

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
      const f32x4* pa = reinterpret_cast<const f32x4*>(o_acc) + chunk * 2;
      const f32x4* pp = reinterpret_cast<const f32x4*>(o_part) + chunk * 2;
      const f32x4 a0 = __builtin_nontemporal_load(pa), a1 = __builtin_nontemporal_load(pa + 1);
      const f32x4 p0 = __builtin_nontemporal_load(pp), p1 = __builtin_nontemporal_load(pp + 1);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        xa[e] = a0[e]; xa[4 + e] = a1[e];
        xp[e] = p0[e]; xp[4 + e] = p1[e];
      }
    } else {
      const u32x4 a = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(o_acc) + chunk);
      const u32x4 p = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(o_part) + chunk);
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
      f32x4* pa = reinterpret_cast<f32x4*>(o_acc) + chunk * 2;
      __builtin_nontemporal_store(f32x4{r[0], r[1], r[2], r[3]}, pa);
      __builtin_nontemporal_store(f32x4{r[4], r[5], r[6], r[7]}, pa + 1);
    } else {
      u32x4 out;
#pragma unroll
      for (int w = 0; w < 4; ++w) out[w] = f32_to_bf16_rne(r[2 * w]) | (f32_to_bf16_rne(r[2 * w + 1]) << 16);
      __builtin_nontemporal_store(out, reinterpret_cast<u32x4*>(o_acc) + chunk);
    }
    if (c == 0) lse_acc[lse_idx] = empty ? -INFINITY : m + __logf(wsum);
  }
}

template <int D>
hipError_t launch_d(void* o_acc, float* lse_acc, const void* o_part, const float* lse_part, int32_t B,
                    int32_t Sq, int32_t H, bool o_f32, hipStream_t stream) {
  constexpr int kRows = rows_per_wg<D>();
  const int32_t row_blocks = (Sq + kRows - 1) / kRows;
  const uint64_t blocks = (uint64_t)B * H * row_blocks;  // < 2^31: rows * D / 8 < 2^31 (ABI layer)
  if (blocks == 0) return hipSuccess;
  if (o_f32)
    merge_kernel<true, D><<<(unsigned)blocks, kThreads, 0, stream>>>(o_acc, lse_acc, o_part, lse_part, Sq, H,
                                                                    row_blocks);
  else
    merge_kernel<false, D><<<(unsigned)blocks, kThreads, 0, stream>>>(o_acc, lse_acc, o_part, lse_part, Sq, H,
                                                                     row_blocks);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_merge(void* o_acc, float* lse_acc, const void* o_part, const float* lse_part,
                             int32_t B, int32_t Sq, int32_t H, int32_t D, bool o_f32,
                             hipStream_t stream) {
  // D = 8 * 2^k <= 512 (checked by the ABI layer)
  switch (D) {
    case 8: return launch_d<8>(o_acc, lse_acc, o_part, lse_part, B, Sq, H, o_f32, stream);
    case 16: return launch_d<16>(o_acc, lse_acc, o_part, lse_part, B, Sq, H, o_f32, stream);
    case 32: return launch_d<32>(o_acc, lse_acc, o_part, lse_part, B, Sq, H, o_f32, stream);
    case 64: return launch_d<64>(o_acc, lse_acc, o_part, lse_part, B, Sq, H, o_f32, stream);
    case 128: return launch_d<128>(o_acc, lse_acc, o_part, lse_part, B, Sq, H, o_f32, stream);
    case 256: return launch_d<256>(o_acc, lse_acc, o_part, lse_part, B, Sq, H, o_f32, stream);
    default: return launch_d<512>(o_acc, lse_acc, o_part, lse_part, B, Sq, H, o_f32, stream);
  }
}

}  // namespace dit
