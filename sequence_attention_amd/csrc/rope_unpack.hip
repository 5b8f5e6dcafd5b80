// Fused receive preparation: sequence-to-head unpack with rotary position
// embedding on the Q and K planes (gfx950).
//
// edge-dit.cpp "Parallel execution", Ulysses section: the receive path
// decodes the rank-major receive buffer, extracts the Q/K/V planes, builds
// the head-sharded attention layout and applies RoPE to Q and K in one pass,
// instead of separate unpack, reshape, permute, materialisation and RoPE
// operators.  The rotation (RoFormer convention, pairs of adjacent head
// dims): for position t and pair i of a head,
//   y[2i]   = x[2i] cos(t, i) - x[2i+1] sin(t, i)
//   y[2i+1] = x[2i] sin(t, i) + x[2i+1] cos(t, i)
// with the caller's fp32 tables cos/sin of shape [S, D/2] (any angle
// schedule: one-axis, or the per-axis schedules of image/video tokens, is
// a table).  Computed in fp32, rounded to the plane dtype (round to nearest
// even); plane 2 (V), when present, is copied bit for bit.
//
// HBM-bound: one 16-byte vector of the output per thread (8 bf16/f16 or 4
// fp32 elements = 4 or 2 pairs), read from its one source vector in the
// receive buffer; the matching 16 or 8 bytes of cos and sin come from the
// tables, which are small ([S, D/2] fp32 each) and stay in L2 across heads
// and planes.  Non-temporal loads and stores for the streamed data.
#include "dit_internal.h"

namespace dit {
namespace {

constexpr int kThreads = 256;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

struct RopeGeom {
  const char* recv;
  char* out[3];
  const float* cos;
  const float* sin;
  uint32_t total_vecs;   // n_planes * B * S * run_vecs
  uint32_t run_vecs;     // vectors per sequence row of one plane: H_loc * D / per-vector
  uint32_t head_vecs;    // vectors per head: D / per-vector
  FastDiv div_run, div_s, div_b, div_sloc, div_head;
  int32_t B, S, S_loc, n_planes, half_d;  // half_d = D / 2: row length of the tables
};

__device__ __forceinline__ float lo16_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi16_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t x = __float_as_uint(f);
  if ((x & 0x7fffffffu) > 0x7f800000u) return (x >> 16) | 0x40u;
  return (x + 0x7fffu + ((x >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ void rotate(float x0, float x1, float c, float s, float& y0, float& y1) {
  y0 = __builtin_fmaf(x0, c, -(x1 * s));
  y1 = __builtin_fmaf(x0, s, x1 * c);
}

// ELEM: 0 = bf16, 1 = f16, 2 = f32
template <int ELEM>
__global__ __launch_bounds__(kThreads) void rope_unpack_kernel(RopeGeom g) {
  const uint32_t v = blockIdx.x * kThreads + threadIdx.x;
  if (v >= g.total_vecs) return;
  // output plane pl, row (b, t), vector `off` of the row
  const uint32_t row = fdiv(v, g.div_run);
  const uint32_t off = v - row * g.run_vecs;
  const uint32_t t0 = fdiv(row, g.div_s);
  const uint32_t t = row - t0 * g.S;
  const uint32_t pl = fdiv(t0, g.div_b);
  const uint32_t b = t0 - pl * g.B;
  const uint32_t p = fdiv(t, g.div_sloc);
  const uint32_t s = t - p * g.S_loc;
  // source: recv[p, pl, b, s, :, :] (a run of H_loc * D elements)
  const size_t src_row = (((size_t)p * g.n_planes + pl) * g.B + b) * g.S_loc + s;
  const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(g.recv) + src_row * g.run_vecs + off);
  u32x4* dst = reinterpret_cast<u32x4*>(g.out[pl]) + ((size_t)b * g.S + t) * g.run_vecs + off;
  if (pl >= 2) {  // V: plain copy
    __builtin_nontemporal_store(x, dst);
    return;
  }
  const uint32_t head = fdiv(off, g.div_head);
  const uint32_t dv = off - head * g.head_vecs;       // vector index inside the head
  constexpr int kPairs = ELEM == 2 ? 2 : 4;           // pairs per 16-byte vector
  const size_t tab = (size_t)t * g.half_d + (size_t)dv * kPairs;
  u32x4 y;
  if constexpr (ELEM == 2) {
    const f32x2 c = *reinterpret_cast<const f32x2*>(g.cos + tab);
    const f32x2 sn = *reinterpret_cast<const f32x2*>(g.sin + tab);
    const f32x4 xf = __builtin_bit_cast(f32x4, x);
    float r0, r1, r2, r3;
    rotate(xf[0], xf[1], c[0], sn[0], r0, r1);
    rotate(xf[2], xf[3], c[1], sn[1], r2, r3);
    y = __builtin_bit_cast(u32x4, f32x4{r0, r1, r2, r3});
  } else {
    const f32x4 c = *reinterpret_cast<const f32x4*>(g.cos + tab);
    const f32x4 sn = *reinterpret_cast<const f32x4*>(g.sin + tab);
#pragma unroll
    for (int w = 0; w < 4; ++w) {  // word w holds pair w: elements (2w, 2w + 1)
      float x0, x1, y0, y1;
      if constexpr (ELEM == 0) {
        x0 = lo16_bf16(x[w]);
        x1 = hi16_bf16(x[w]);
      } else {
        x0 = (float)__builtin_bit_cast(_Float16, (uint16_t)(x[w] & 0xffffu));
        x1 = (float)__builtin_bit_cast(_Float16, (uint16_t)(x[w] >> 16));
      }
      rotate(x0, x1, c[w], sn[w], y0, y1);
      if constexpr (ELEM == 0) {
        y[w] = f32_to_bf16_rne(y0) | (f32_to_bf16_rne(y1) << 16);
      } else {
        y[w] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)y0) |
               ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)y1) << 16);
      }
    }
  }
  __builtin_nontemporal_store(y, dst);
}

}  // namespace

hipError_t launch_rope_unpack(const RopeUnpackArgs& a, hipStream_t stream) {
  const int per_vec = 16 / a.elem_bytes;
  RopeGeom g;
  g.recv = static_cast<const char*>(a.recv);
  for (int i = 0; i < 3; ++i) g.out[i] = static_cast<char*>(a.out[i]);
  g.cos = a.cos;
  g.sin = a.sin;
  g.head_vecs = (uint32_t)(a.D / per_vec);
  g.run_vecs = g.head_vecs * (uint32_t)a.H_loc;
  const uint64_t total = (uint64_t)a.n_planes * a.B * a.S * g.run_vecs;
  if (total == 0) return hipSuccess;
  g.total_vecs = (uint32_t)total;  // < 2^31: checked by the ABI layer
  g.div_run = make_fastdiv(g.run_vecs);
  g.div_s = make_fastdiv((uint32_t)a.S);
  g.div_b = make_fastdiv((uint32_t)a.B);
  g.div_sloc = make_fastdiv((uint32_t)a.S_loc);
  g.div_head = make_fastdiv(g.head_vecs);
  g.B = a.B; g.S = a.S; g.S_loc = a.S_loc; g.n_planes = a.n_planes; g.half_d = a.D / 2;
  const unsigned blocks = (unsigned)((total + kThreads - 1) / kThreads);
  switch (a.elem_bytes) {
    case 4: rope_unpack_kernel<2><<<blocks, kThreads, 0, stream>>>(g); break;
    default:
      if (a.is_f16) rope_unpack_kernel<1><<<blocks, kThreads, 0, stream>>>(g);
      else rope_unpack_kernel<0><<<blocks, kThreads, 0, stream>>>(g);
      break;
  }
  return hipGetLastError();
}

}  // namespace dit
