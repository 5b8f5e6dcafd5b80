// FP8 Ulysses pack / unpack (gfx950).
//
// cache-dit "Context Parallelism", Async FP8 Ulysses Attention: Q, V and the
// attention output O cross the all-to-alls as FP8 while K stays 16-bit (the
// softmax of Q K^T is the precision-sensitive part).  Format and scaling are
// not given there; this library encodes OCP E4M3 ("FN", largest finite 448)
// with one power-of-two scale per 32 consecutive elements of a head vector
// (the block size and E8M0 scale byte of the OCP Microscaling formats):
//   k = smallest integer with amax <= 448 * 2^k, clamped to [-117, 126],
//   code = E4M3 round-to-nearest-even of x * 2^-k (exact product),
//   scale byte = k + 127,  decoded value = value(code) * 2^k (exact in bf16).
// The maps around the codes are the padded Ulysses maps (pad rows and pad
// heads encode as zeros, are never read on the pack side and are dropped or
// zeroed on the unpack side exactly as in the 16-bit maps).
//
// Chunk of one peer (bytes), E = B * S_loc * H_loc * D:
//   sequence to head: Q codes [0, E), V codes [E, 2E), K bf16 [2E, 4E),
//                     Q scales [4E, 4E + E/32), V scales [4E + E/32, 4E + E/16)
//   head to sequence: O codes [0, E), O scales [E, E + E/32)
// padded with zero bytes to a multiple of 256 (the per-peer stride).
//
// HBM-bound.  A thread owns 8 consecutive elements (16 bytes of bf16 in, 8
// bytes of codes out); the 4 threads of a 32-element block are adjacent
// lanes and take the block maximum with two quad swaps (DPP).  The
// conversions use gfx950's packed FP8 instructions (round to nearest even;
// |x * 2^-k| <= 448 by the choice of k, so they never saturate).  Grid: x
// over the 8-element groups of one plane's chunk (or output plane), y over
// (peer, plane) or plane, so the section a workgroup writes is uniform.
#include "dit_internal.h"

namespace dit {
namespace {

constexpr int kThreads = 256;
constexpr int kKMin = -117, kKMax = 126;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float pow2f(int e) {  // 2^e for e in [-126, 127]
  return __uint_as_float((uint32_t)(e + 127) << 23);
}

// Block exponent of a non-negative maximum: amax = 1.f * 2^(ef - 127) fits
// 448 * 2^k = 1.75 * 2^(k + 8) iff k >= ef - 135 when 1.f <= 1.75, else
// k >= ef - 134.  Zero and fp32 subnormals take the lower clamp.
__device__ __forceinline__ int block_exp(float amax) {
  const uint32_t b = __float_as_uint(amax);
  const int ef = (int)(b >> 23);
  if (ef == 0) return kKMin;
  const int k = ((b & 0x7fffffu) <= 0x600000u) ? ef - 135 : ef - 134;
  return min(max(k, kKMin), kKMax);
}

__device__ __forceinline__ float quad_max(float v) {
  int x = __float_as_int(v);
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(x, x, 0xB1, 0xF, 0xF, false)));  // quad_perm 1,0,3,2
  x = __float_as_int(v);
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(x, x, 0x4E, 0xF, 0xF, false)));  // quad_perm 2,3,0,1
  return v;
}

__device__ __forceinline__ void bf16x8_to_f32(const u32x4& w, float* x) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// Encode the thread's 8 values of a 32-element block whose 4 threads are a
// lane quad; returns the codes and the block's scale byte.
__device__ __forceinline__ u32x2 encode8(const u32x4& w, uint32_t* scale_byte) {
  float x[8];
  bf16x8_to_f32(w, x);
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
  amax = quad_max(amax);
  const int k = block_exp(amax);
  const float inv = pow2f(-k);
  u32x2 c;
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(x[0] * inv, x[1] * inv, 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(x[2] * inv, x[3] * inv, lo, true);
  int hi = __builtin_amdgcn_cvt_pk_fp8_f32(x[4] * inv, x[5] * inv, 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(x[6] * inv, x[7] * inv, hi, true);
  c[0] = (uint32_t)lo;
  c[1] = (uint32_t)hi;
  *scale_byte = (uint32_t)(k + 127);
  return c;
}

// Decode 8 codes with scale byte sb to 8 bf16 (exact: the products are bf16 values).
__device__ __forceinline__ u32x4 decode8(const u32x2& c, uint32_t sb) {
  const float s = pow2f((int)sb - 127);
  u32x4 out;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const v2f a = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[i], false);
    const v2f b = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[i], true);
    out[2 * i] = (__float_as_uint(a[0] * s) >> 16) | (__float_as_uint(a[1] * s) & 0xffff0000u);
    out[2 * i + 1] = (__float_as_uint(b[0] * s) >> 16) | (__float_as_uint(b[1] * s) & 0xffff0000u);
  }
  return out;
}

struct Fp8Geom {
  const uint16_t* planes_in[3];
  uint16_t* planes_out[3];
  const uint8_t* buf_in;
  uint8_t* buf_out;
  uint64_t stride;        // bytes per peer chunk
  uint64_t E;             // elements per plane per chunk
  uint32_t used;          // bytes of a chunk before its zero tail
  uint32_t groups;        // 8-element groups in x
  FastDiv div_g, div_hloc, div_rows;  // by D/8, H_loc, S_loc (pack) or S (unpack s2h)
  FastDiv div_sloc;
  int32_t B, S, H, D, S_loc, H_loc, rank;
};

// Section offsets in a sequence-to-head chunk for plane pl (0 = Q, 1 = K, 2 = V).
__device__ __forceinline__ uint64_t code_sec(const Fp8Geom& g, int pl) { return pl == 0 ? 0 : g.E; }
__device__ __forceinline__ uint64_t scale_sec(const Fp8Geom& g, int pl) {
  return 4 * g.E + (pl == 0 ? 0 : g.E / 32);
}

// Pack, sequence to head.  grid.y = p * 3 + pl; x over [B][S_loc][H_loc][D/8].
__global__ __launch_bounds__(kThreads) void pack_s2h_fp8(const Fp8Geom g) {
  const uint32_t v = blockIdx.x * kThreads + threadIdx.x;
  const int p = (int)blockIdx.y / 3, pl = (int)blockIdx.y - 3 * ((int)blockIdx.y / 3);
  uint8_t* chunk = g.buf_out + (uint64_t)p * g.stride;
  if (pl == 0 && v < g.stride - g.used) chunk[g.used + v] = 0;  // zero tail
  if (v >= g.groups) return;
  const uint32_t row = fdiv(v, g.div_g);  // ((b * S_loc + s) * H_loc + h')
  const uint32_t grp = v - row * (uint32_t)(g.D / 8);
  const uint32_t bs = fdiv(row, g.div_hloc);
  const uint32_t hh = row - bs * (uint32_t)g.H_loc;
  const uint32_t b = fdiv(bs, g.div_rows);
  const uint32_t s = bs - b * (uint32_t)g.S_loc;
  const int head = p * g.H_loc + (int)hh;
  u32x4 w = u32x4(0);
  if (g.rank * g.S_loc + (int)s < g.S && head < g.H) {
    const uint64_t src = (((uint64_t)b * g.S_loc + s) * g.H + head) * g.D + grp * 8;
    w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(g.planes_in[pl] + src));
  }
  if (pl == 1) {  // K stays bf16
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(chunk + 2 * g.E) + v);
    return;
  }
  uint32_t sb;
  const u32x2 c = encode8(w, &sb);
  __builtin_nontemporal_store(c, reinterpret_cast<u32x2*>(chunk + code_sec(g, pl)) + v);
  if ((v & 3) == 0) chunk[scale_sec(g, pl) + v / 4] = (uint8_t)sb;
}

// Unpack, sequence to head.  grid.y = pl; x over the output plane [B][S][H_loc][D/8].
__global__ __launch_bounds__(kThreads) void unpack_s2h_fp8(const Fp8Geom g) {
  const uint32_t v = blockIdx.x * kThreads + threadIdx.x;
  if (v >= g.groups) return;
  const int pl = (int)blockIdx.y;
  const uint32_t row = fdiv(v, g.div_g);  // ((b * S + t) * H_loc + h')
  const uint32_t grp = v - row * (uint32_t)(g.D / 8);
  const uint32_t bt = fdiv(row, g.div_hloc);
  const uint32_t hh = row - bt * (uint32_t)g.H_loc;
  const uint32_t b = fdiv(bt, g.div_rows);
  const uint32_t t = bt - b * (uint32_t)g.S;
  const uint32_t p = fdiv(t, g.div_sloc);
  const uint32_t s = t - p * (uint32_t)g.S_loc;
  const uint8_t* chunk = g.buf_in + (uint64_t)p * g.stride;
  const uint64_t e = (((uint64_t)b * g.S_loc + s) * g.H_loc + hh) * g.D + grp * 8;  // element in section
  u32x4 out;
  if (pl == 1) {
    out = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(chunk + 2 * g.E + 2 * e));
  } else {
    const u32x2 c = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(chunk + code_sec(g, pl) + e));
    out = decode8(c, chunk[scale_sec(g, pl) + e / 32]);
  }
  __builtin_nontemporal_store(out, reinterpret_cast<u32x4*>(g.planes_out[pl]) + v);
}

// Pack, head to sequence (plane O).  grid.y = p; x over [B][S_loc][H_loc][D/8].
__global__ __launch_bounds__(kThreads) void pack_h2s_fp8(const Fp8Geom g) {
  const uint32_t v = blockIdx.x * kThreads + threadIdx.x;
  const int p = (int)blockIdx.y;
  uint8_t* chunk = g.buf_out + (uint64_t)p * g.stride;
  if (v < g.stride - g.used) chunk[g.used + v] = 0;  // zero tail
  if (v >= g.groups) return;
  const uint32_t row = fdiv(v, g.div_g);
  const uint32_t grp = v - row * (uint32_t)(g.D / 8);
  const uint32_t bs = fdiv(row, g.div_hloc);
  const uint32_t hh = row - bs * (uint32_t)g.H_loc;
  const uint32_t b = fdiv(bs, g.div_rows);
  const uint32_t s = bs - b * (uint32_t)g.S_loc;
  const int t = p * g.S_loc + (int)s;
  u32x4 w = u32x4(0);
  if (t < g.S && g.rank * g.H_loc + (int)hh < g.H) {
    const uint64_t src = (((uint64_t)b * g.S + t) * g.H_loc + hh) * g.D + grp * 8;
    w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(g.planes_in[0] + src));
  }
  uint32_t sb;
  const u32x2 c = encode8(w, &sb);
  __builtin_nontemporal_store(c, reinterpret_cast<u32x2*>(chunk) + v);
  if ((v & 3) == 0) chunk[g.E + v / 4] = (uint8_t)sb;
}

// Unpack, head to sequence.  grid.y = source p; x over [B][S_loc][H_loc][D/8].
__global__ __launch_bounds__(kThreads) void unpack_h2s_fp8(const Fp8Geom g) {
  const uint32_t v = blockIdx.x * kThreads + threadIdx.x;
  if (v >= g.groups) return;
  const int p = (int)blockIdx.y;
  const uint32_t row = fdiv(v, g.div_g);
  const uint32_t grp = v - row * (uint32_t)(g.D / 8);
  const uint32_t bs = fdiv(row, g.div_hloc);
  const uint32_t hh = row - bs * (uint32_t)g.H_loc;
  const uint32_t b = fdiv(bs, g.div_rows);
  const uint32_t s = bs - b * (uint32_t)g.S_loc;
  const int head = p * g.H_loc + (int)hh;
  if (head >= g.H) return;  // pad head: dropped
  const uint8_t* chunk = g.buf_in + (uint64_t)p * g.stride;
  u32x4 out = u32x4(0);
  if (g.rank * g.S_loc + (int)s < g.S) {
    const u32x2 c = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(chunk) + v);
    out = decode8(c, chunk[g.E + v / 4]);
  }
  const uint64_t dst = (((uint64_t)b * g.S_loc + s) * g.H + head) * g.D + grp * 8;
  __builtin_nontemporal_store(out, reinterpret_cast<u32x4*>(g.planes_out[0] + dst));
}

}  // namespace

hipError_t launch_fp8_permute(PermuteKind kind, const Fp8PermuteArgs& a, hipStream_t stream) {
  Fp8Geom g;
  for (int i = 0; i < 3; ++i) {
    g.planes_in[i] = static_cast<const uint16_t*>(a.planes[i]);
    g.planes_out[i] = static_cast<uint16_t*>(const_cast<void*>(a.planes[i]));
  }
  g.buf_in = static_cast<const uint8_t*>(a.buf);
  g.buf_out = static_cast<uint8_t*>(const_cast<void*>(a.buf));
  g.stride = (uint64_t)a.stride;
  g.E = (uint64_t)a.B * a.S_loc * a.H_loc * a.D;
  g.used = (uint32_t)a.used;
  g.B = a.B; g.S = a.S; g.H = a.H; g.D = a.D; g.S_loc = a.S_loc; g.H_loc = a.H_loc; g.rank = a.rank;
  g.div_g = make_fastdiv((uint32_t)(a.D / 8));
  g.div_hloc = make_fastdiv((uint32_t)a.H_loc);
  const bool unpack_s2h = (kind == UNPACK_SEQ_TO_HEAD);
  g.div_rows = make_fastdiv((uint32_t)(unpack_s2h ? a.S : a.S_loc));
  g.div_sloc = make_fastdiv((uint32_t)a.S_loc);
  const uint64_t rows = (uint64_t)a.B * (unpack_s2h ? a.S : a.S_loc) * a.H_loc;
  g.groups = (uint32_t)(rows * (a.D / 8));  // < 2^31: checked by the ABI layer
  // pack kernels also zero each chunk's tail with their first threads
  const uint64_t tail = g.stride - g.used;
  uint64_t xthreads = g.groups;
  if ((kind == PACK_SEQ_TO_HEAD || kind == PACK_HEAD_TO_SEQ) && tail > xthreads) xthreads = tail;
  const unsigned gx = (unsigned)((xthreads + kThreads - 1) / kThreads);
  if (gx == 0) return hipSuccess;
  switch (kind) {
    case PACK_SEQ_TO_HEAD: pack_s2h_fp8<<<dim3(gx, 3 * a.U), kThreads, 0, stream>>>(g); break;
    case UNPACK_SEQ_TO_HEAD: unpack_s2h_fp8<<<dim3(gx, 3), kThreads, 0, stream>>>(g); break;
    case PACK_HEAD_TO_SEQ: pack_h2s_fp8<<<dim3(gx, a.U), kThreads, 0, stream>>>(g); break;
    default: unpack_h2s_fp8<<<dim3(gx, a.U), kThreads, 0, stream>>>(g); break;
  }
  return hipGetLastError();
}

}  // namespace dit
