// Ulysses pack / unpack permutations around the all-to-alls (gfx950).
//
// edge-dit.cpp "Parallel execution" describes fused layout operators on
// either side of the two Ulysses all-to-alls: the packed QKV operator
// (planes concatenated, split by destination head group, flattened
// peer-major), the receive preparation (rank-major buffer decoded into the
// head-sharded attention layout), and the packed head-to-sequence operator
// with its receive-side unpack.  SGLang "Parallelism Overview" ("The
// Ulysses transport") keeps the three Q/K/V exchanges in one
// destination-major buffer.  All four maps are pure permutations with zero
// fill of pad rows and pad heads.
//
// HBM-bound copy.  Every map moves contiguous runs of H_loc*D elements (one
// row of one head group), so each thread moves 16-byte vectors (or the
// widest width the run length and pointers allow) and a wave covers
// consecutive vectors of one or two runs: both sides are read and written in
// long coalesced segments.  The index of a vector is decomposed with
// multiply-high division by the run-time sizes.  Both sides use
// non-temporal loads and stores (every byte is touched exactly once); one
// vector per thread measured fastest for this streaming pattern on MI355X.
#include "dit_internal.h"

namespace dit {
namespace {

constexpr int kThreads = 256;
constexpr int kVecPerThread = 1;  // measured fastest for streaming on MI355X (with non-temporal access)

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct PermuteGeom {
  const char* in[3];
  char* out[3];
  uint32_t total_vecs;      // vectors in the iteration space
  uint32_t run_vecs;        // vectors per run (H_loc * D * elem / vec)
  FastDiv div_run;          // by run_vecs
  FastDiv div_a, div_b, div_c;  // row decomposition, see each kind
  int32_t B, S, H, D, U, n_planes, S_loc, H_loc, rank;
  uint32_t head_vecs;       // vectors per head (D * elem / vec)
};

template <typename V>
__device__ __forceinline__ V zero_vec() {
  return V(0);
}

template <typename V>
__device__ __forceinline__ void store_nt(V* p, const V& v) {
  __builtin_nontemporal_store(v, p);
}

template <typename V>
__device__ __forceinline__ V load_nt(const V* p) {
  return __builtin_nontemporal_load(p);
}

// PACK_SEQ_TO_HEAD: iterate over the send buffer [U, n, B, S_loc, H_loc, D].
//   run row = ((p * n + pl) * B + b) * S_loc + s;  div_a = S_loc, div_b = B, div_c = n.
// Each map returns the value of iteration index v and sets *dst to where it
// goes (nullptr: nothing to write).  Loads of several indices are issued
// before any store so that a thread keeps several vectors in flight.
template <typename V>
__device__ __forceinline__ V pack_s2h(const PermuteGeom& g, uint32_t v, V** dst) {
  const uint32_t row = fdiv(v, g.div_run);
  const uint32_t off = v - row * g.run_vecs;
  const uint32_t t0 = fdiv(row, g.div_a);
  const uint32_t s = row - t0 * g.S_loc;
  const uint32_t t1 = fdiv(t0, g.div_b);
  const uint32_t b = t0 - t1 * g.B;
  const uint32_t p = fdiv(t1, g.div_c);
  const uint32_t pl = t1 - p * g.n_planes;
  V val = zero_vec<V>();
  const int valid_heads = g.H - (int)p * g.H_loc;  // may be <= 0 past H
  if ((int)(g.rank * g.S_loc + s) < g.S && (int)off < valid_heads * (int)g.head_vecs) {
    // in_pl[b, s, p*H_loc + h', d]: run starts at ((b*S_loc + s)*H + p*H_loc)*D
    const size_t src_vec = ((size_t)(b * g.S_loc + s) * g.H + (size_t)p * g.H_loc) * g.head_vecs + off;
    val = load_nt(reinterpret_cast<const V*>(g.in[pl]) + src_vec);
  }
  *dst = reinterpret_cast<V*>(g.out[0]) + v;
  return val;
}

// UNPACK_SEQ_TO_HEAD: iterate over the output planes [n][B, S, H_loc, D].
//   run row = (pl * B + b) * S + t;  div_a = S, div_b = B, div_c = S_loc.
template <typename V>
__device__ __forceinline__ V unpack_s2h(const PermuteGeom& g, uint32_t v, V** dst) {
  const uint32_t row = fdiv(v, g.div_run);
  const uint32_t off = v - row * g.run_vecs;
  const uint32_t t0 = fdiv(row, g.div_a);
  const uint32_t t = row - t0 * g.S;
  const uint32_t pl = fdiv(t0, g.div_b);
  const uint32_t b = t0 - pl * g.B;
  const uint32_t p = fdiv(t, g.div_c);
  const uint32_t s = t - p * g.S_loc;
  // recv[p, pl, b, s, :, :]
  const size_t src_row = (((size_t)p * g.n_planes + pl) * g.B + b) * g.S_loc + s;
  const V val = load_nt(reinterpret_cast<const V*>(g.in[0]) + src_row * g.run_vecs + off);
  const size_t dst_row = (size_t)b * g.S + t;
  *dst = reinterpret_cast<V*>(g.out[pl]) + dst_row * g.run_vecs + off;
  return val;
}

// PACK_HEAD_TO_SEQ: iterate over the send buffer [U, n, B, S_loc, H_loc, D].
//   run row = ((p * n + pl) * B + b) * S_loc + s;  div_a = S_loc, div_b = B, div_c = n.
template <typename V>
__device__ __forceinline__ V pack_h2s(const PermuteGeom& g, uint32_t v, V** dst) {
  const uint32_t row = fdiv(v, g.div_run);
  const uint32_t off = v - row * g.run_vecs;
  const uint32_t t0 = fdiv(row, g.div_a);
  const uint32_t s = row - t0 * g.S_loc;
  const uint32_t t1 = fdiv(t0, g.div_b);
  const uint32_t b = t0 - t1 * g.B;
  const uint32_t p = fdiv(t1, g.div_c);
  const uint32_t pl = t1 - p * g.n_planes;
  V val = zero_vec<V>();
  const int valid_heads = g.H - g.rank * g.H_loc;
  const uint32_t t = p * g.S_loc + s;
  if ((int)t < g.S && (int)off < valid_heads * (int)g.head_vecs) {
    // in_pl[b, t, :, :] of [B, S, H_loc, D]
    const size_t src_vec = ((size_t)b * g.S + t) * g.run_vecs + off;
    val = load_nt(reinterpret_cast<const V*>(g.in[pl]) + src_vec);
  }
  *dst = reinterpret_cast<V*>(g.out[0]) + v;
  return val;
}

// UNPACK_HEAD_TO_SEQ: iterate over the receive buffer [U, n, B, S_loc, H_loc, D]
// (each real output element has exactly one source; pad heads are dropped,
// pad rows are written as zeros).
//   run row = ((p * n + pl) * B + b) * S_loc + s;  div_a = S_loc, div_b = B, div_c = n.
template <typename V>
__device__ __forceinline__ V unpack_h2s(const PermuteGeom& g, uint32_t v, V** dst) {
  const uint32_t row = fdiv(v, g.div_run);
  const uint32_t off = v - row * g.run_vecs;
  const uint32_t t0 = fdiv(row, g.div_a);
  const uint32_t s = row - t0 * g.S_loc;
  const uint32_t t1 = fdiv(t0, g.div_b);
  const uint32_t b = t0 - t1 * g.B;
  const uint32_t p = fdiv(t1, g.div_c);
  const uint32_t pl = t1 - p * g.n_planes;
  const int valid_heads = g.H - (int)p * g.H_loc;
  V val = zero_vec<V>();
  *dst = nullptr;
  if ((int)off >= valid_heads * (int)g.head_vecs) return val;  // pad head: dropped
  if ((int)(g.rank * g.S_loc + s) < g.S) val = load_nt(reinterpret_cast<const V*>(g.in[0]) + v);
  // out_pl[b, s, p*H_loc + h', d] of [B, S_loc, H, D]
  const size_t dst_vec = ((size_t)(b * g.S_loc + s) * g.H + (size_t)p * g.H_loc) * g.head_vecs + off;
  *dst = reinterpret_cast<V*>(g.out[pl]) + dst_vec;
  return val;
}

template <int KIND, typename V>
__global__ __launch_bounds__(kThreads) void permute_kernel(PermuteGeom g) {
  const uint32_t base = blockIdx.x * (kThreads * kVecPerThread) + threadIdx.x;
  V val[kVecPerThread];
  V* dst[kVecPerThread];
#pragma unroll
  for (int i = 0; i < kVecPerThread; ++i) {
    const uint32_t v = base + i * kThreads;
    dst[i] = nullptr;
    if (v < g.total_vecs) {
      if constexpr (KIND == PACK_SEQ_TO_HEAD) val[i] = pack_s2h<V>(g, v, &dst[i]);
      else if constexpr (KIND == UNPACK_SEQ_TO_HEAD) val[i] = unpack_s2h<V>(g, v, &dst[i]);
      else if constexpr (KIND == PACK_HEAD_TO_SEQ) val[i] = pack_h2s<V>(g, v, &dst[i]);
      else val[i] = unpack_h2s<V>(g, v, &dst[i]);
    }
  }
#pragma unroll
  for (int i = 0; i < kVecPerThread; ++i)
    if (dst[i] != nullptr) store_nt(dst[i], val[i]);
}

template <int KIND>
hipError_t launch_kind(const PermuteGeom& g, int vec_bytes, hipStream_t stream) {
  const uint32_t per_block = kThreads * kVecPerThread;
  const uint32_t blocks = (g.total_vecs + per_block - 1) / per_block;
  if (blocks == 0) return hipSuccess;
  switch (vec_bytes) {
    case 16: permute_kernel<KIND, u32x4><<<blocks, kThreads, 0, stream>>>(g); break;
    case 8: permute_kernel<KIND, u32x2><<<blocks, kThreads, 0, stream>>>(g); break;
    case 4: permute_kernel<KIND, uint32_t><<<blocks, kThreads, 0, stream>>>(g); break;
    default: permute_kernel<KIND, uint16_t><<<blocks, kThreads, 0, stream>>>(g); break;
  }
  return hipGetLastError();
}

// The packs with a conversion on the way in (edge-dit.cpp "Parallel
// execution": the packed QKV operator's optional F32-to-F16 conversion, and
// F16 / BF16 output produced directly on the head-to-sequence path).  The
// planes are float32, the send buffer 16-bit: each thread reads E floats
// through the same index maps as the plain packs (a "vector" is E elements
// on both sides) and stores the E rounded values at out[0] + v.  The packed
// hardware conversions round to nearest, ties to even, keep subnormals
// (the kernel runs with f32 and f16 denormals preserved), send overflow to
// infinity and NaN to a quiet NaN.
template <int KIND, int E, bool kBf16>
__global__ __launch_bounds__(kThreads) void pack_convert_kernel(PermuteGeom g) {
  typedef float SV __attribute__((ext_vector_type(E)));
  typedef __bf16 BV __attribute__((ext_vector_type(E)));
  typedef _Float16 HV __attribute__((ext_vector_type(E)));
  const uint32_t v = blockIdx.x * kThreads + threadIdx.x;
  if (v >= g.total_vecs) return;
  SV* unused;
  SV x;
  if constexpr (KIND == PACK_SEQ_TO_HEAD) x = pack_s2h<SV>(g, v, &unused);
  else x = pack_h2s<SV>(g, v, &unused);
  if constexpr (kBf16) {
    store_nt(reinterpret_cast<BV*>(g.out[0]) + v, __builtin_convertvector(x, BV));
  } else {
    store_nt(reinterpret_cast<HV*>(g.out[0]) + v, __builtin_convertvector(x, HV));
  }
}

template <int KIND, bool kBf16>
hipError_t launch_convert_kind(const PermuteGeom& g, int E, hipStream_t stream) {
  const uint32_t blocks = (g.total_vecs + kThreads - 1) / kThreads;
  if (blocks == 0) return hipSuccess;
  switch (E) {
    case 8: pack_convert_kernel<KIND, 8, kBf16><<<blocks, kThreads, 0, stream>>>(g); break;
    case 4: pack_convert_kernel<KIND, 4, kBf16><<<blocks, kThreads, 0, stream>>>(g); break;
    case 2: pack_convert_kernel<KIND, 2, kBf16><<<blocks, kThreads, 0, stream>>>(g); break;
    default: pack_convert_kernel<KIND, 1, kBf16><<<blocks, kThreads, 0, stream>>>(g); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_permute(PermuteKind kind, const PermuteArgs& a, hipStream_t stream) {
  // Widest vector that divides a head's bytes and keeps every pointer aligned.
  const uint32_t head_bytes = (uint32_t)a.D * a.elem_bytes;
  uint32_t align_bits = 0;
  for (int i = 0; i < 3; ++i) {
    align_bits |= (uint32_t)(uintptr_t)a.in[i];
    align_bits |= (uint32_t)(uintptr_t)a.out[i];
  }
  int vec = 16;
  while (vec > a.elem_bytes && ((head_bytes % vec) != 0 || (align_bits % vec) != 0)) vec >>= 1;

  PermuteGeom g;
  for (int i = 0; i < 3; ++i) {
    g.in[i] = static_cast<const char*>(a.in[i]);
    g.out[i] = static_cast<char*>(a.out[i]);
  }
  g.B = a.B; g.S = a.S; g.H = a.H; g.D = a.D; g.U = a.U; g.n_planes = a.n_planes;
  g.S_loc = a.S_loc; g.H_loc = a.H_loc; g.rank = a.rank;
  g.head_vecs = head_bytes / vec;
  g.run_vecs = g.head_vecs * a.H_loc;
  if (g.run_vecs == 0) return hipSuccess;
  g.div_run = make_fastdiv(g.run_vecs);
  uint64_t rows;
  switch (kind) {
    case UNPACK_SEQ_TO_HEAD:
      rows = (uint64_t)a.n_planes * a.B * a.S;
      g.div_a = make_fastdiv(a.S > 0 ? a.S : 1);
      g.div_b = make_fastdiv(a.B > 0 ? a.B : 1);
      g.div_c = make_fastdiv(a.S_loc > 0 ? a.S_loc : 1);
      break;
    default:  // the three kinds that walk [U, n, B, S_loc, H_loc, D]
      rows = (uint64_t)a.U * a.n_planes * a.B * a.S_loc;
      g.div_a = make_fastdiv(a.S_loc > 0 ? a.S_loc : 1);
      g.div_b = make_fastdiv(a.B > 0 ? a.B : 1);
      g.div_c = make_fastdiv(a.n_planes);
      break;
  }
  g.total_vecs = (uint32_t)(rows * g.run_vecs);  // < 2^31: checked by the ABI layer
  switch (kind) {
    case PACK_SEQ_TO_HEAD: return launch_kind<PACK_SEQ_TO_HEAD>(g, vec, stream);
    case UNPACK_SEQ_TO_HEAD: return launch_kind<UNPACK_SEQ_TO_HEAD>(g, vec, stream);
    case PACK_HEAD_TO_SEQ: return launch_kind<PACK_HEAD_TO_SEQ>(g, vec, stream);
    default: return launch_kind<UNPACK_HEAD_TO_SEQ>(g, vec, stream);
  }
}

hipError_t launch_pack_convert(PermuteKind kind, const PermuteArgs& a, bool to_bf16,
                               hipStream_t stream) {
  // E elements per thread: the most that divides a head and keeps every
  // float32 load (4E bytes) and 16-bit store (2E bytes) aligned.
  uint32_t in_bits = 0, out_bits = (uint32_t)(uintptr_t)a.out[0];
  for (int i = 0; i < a.n_planes; ++i) in_bits |= (uint32_t)(uintptr_t)a.in[i];
  int E = 8;
  while (E > 1 && (a.D % E != 0 || in_bits % (4 * E) != 0 || out_bits % (2 * E) != 0)) E >>= 1;

  PermuteGeom g;
  for (int i = 0; i < 3; ++i) {
    g.in[i] = static_cast<const char*>(a.in[i]);
    g.out[i] = static_cast<char*>(a.out[i]);
  }
  g.B = a.B; g.S = a.S; g.H = a.H; g.D = a.D; g.U = a.U; g.n_planes = a.n_planes;
  g.S_loc = a.S_loc; g.H_loc = a.H_loc; g.rank = a.rank;
  g.head_vecs = a.D / E;
  g.run_vecs = g.head_vecs * a.H_loc;
  if (g.run_vecs == 0) return hipSuccess;
  g.div_run = make_fastdiv(g.run_vecs);
  g.div_a = make_fastdiv(a.S_loc > 0 ? a.S_loc : 1);
  g.div_b = make_fastdiv(a.B > 0 ? a.B : 1);
  g.div_c = make_fastdiv(a.n_planes);
  const uint64_t rows = (uint64_t)a.U * a.n_planes * a.B * a.S_loc;
  g.total_vecs = (uint32_t)(rows * g.run_vecs);  // < 2^31: checked by the ABI layer
  if (kind == PACK_SEQ_TO_HEAD)
    return to_bf16 ? launch_convert_kind<PACK_SEQ_TO_HEAD, true>(g, E, stream)
                   : launch_convert_kind<PACK_SEQ_TO_HEAD, false>(g, E, stream);
  return to_bf16 ? launch_convert_kind<PACK_HEAD_TO_SEQ, true>(g, E, stream)
                 : launch_convert_kind<PACK_HEAD_TO_SEQ, false>(g, E, stream);
}

}  // namespace dit
