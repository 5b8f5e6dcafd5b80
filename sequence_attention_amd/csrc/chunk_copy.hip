// Per-peer chunk copies between head/sequence planes and an exchange buffer
// whose chunks have different sizes (gfx950).
//
// cache-dit "Context Parallelism" (Ulysses Anything Attention): a sequence
// of any length is split across the Ulysses ranks without padding, each rank
// learning the others' lengths from a scalar gather; the no-pad variant of
// Any Head Num splits the heads unevenly the same way.  The all-to-all then
// exchanges chunks of per-peer sizes, so the send and receive buffers are the
// back-to-back concatenation of one chunk per peer.  diffusers "Distributed
// inference" (Ring Anything Attention) pads each rank's K/V to the longest
// rank, gathers the padded buffers and cuts them back to the real lengths.
//
// All of these are one operation: for every peer p, a 2-D block of `rows`
// rows of `run` contiguous elements moves between a chunk of the buffer
// ([n, B, chunk_rows, run] at a per-peer offset) and a window of the planes
// (row stride plane_row, starting plane_off elements into each batch's
// block).  Toward the buffer, rows in [rows, chunk_rows) are written as zeros
// (Ring Anything's pad rows); from the buffer they are skipped.
//
// HBM-bound copy.  Grid (x: vectors of the largest per-(plane, batch) block,
// y: peer, z: plane x batch), so the peer descriptor is uniform across a
// workgroup and comes from the kernel arguments through scalar loads; a
// thread moves one vector of up to 16 bytes, consecutive lanes take
// consecutive vectors of a row, and both sides use non-temporal accesses
// (every byte is touched once).  Workgroups past a small peer's block exit at
// once.
#include "dit_internal.h"

namespace dit {
namespace {

constexpr int kThreads = 256;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct PeerGeom {
  uint32_t rows, chunk_rows, run;  // in vectors for `run`
  FastDiv div_run;
  uint32_t plane_off;              // vectors
  uint32_t chunk_off;              // vectors
};

struct ChunkGeom {
  char* planes[3];
  char* chunk;
  uint32_t B;
  uint32_t plane_b_rows, plane_row;  // plane_row in vectors
  PeerGeom peer[kMaxPeers];
};

template <typename V, bool kToChunk>
__global__ __launch_bounds__(kThreads) void chunk_copy_kernel(const ChunkGeom g) {
  const PeerGeom& pg = g.peer[blockIdx.y];
  const uint32_t n = pg.chunk_rows * pg.run;
  const uint32_t v = blockIdx.x * kThreads + threadIdx.x;
  if (v >= n) return;
  const uint32_t plb = blockIdx.z;  // pl * B + b
  const uint32_t pl = plb / g.B;
  const uint32_t b = plb - pl * g.B;
  const uint32_t s = fdiv(v, pg.div_run);
  const uint32_t off = v - s * pg.run;
  V* chunk = reinterpret_cast<V*>(g.chunk) + pg.chunk_off + ((size_t)plb * pg.chunk_rows + s) * pg.run + off;
  if (s < pg.rows) {
    V* plane = reinterpret_cast<V*>(g.planes[pl]) + ((size_t)b * g.plane_b_rows + s) * g.plane_row +
               pg.plane_off + off;
    if constexpr (kToChunk)
      __builtin_nontemporal_store(__builtin_nontemporal_load(plane), chunk);
    else
      __builtin_nontemporal_store(__builtin_nontemporal_load(chunk), plane);
  } else if constexpr (kToChunk) {
    __builtin_nontemporal_store(V(0), chunk);
  }
}

template <typename V>
hipError_t launch_v(const ChunkGeom& g, bool to_chunk, dim3 grid, hipStream_t stream) {
  if (to_chunk)
    chunk_copy_kernel<V, true><<<grid, kThreads, 0, stream>>>(g);
  else
    chunk_copy_kernel<V, false><<<grid, kThreads, 0, stream>>>(g);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_copy(const ChunkCopyArgs& a, hipStream_t stream) {
  // Widest vector dividing every run, offset and row stride (all multiples
  // of D elements) and keeping every pointer aligned.
  const uint32_t unit_bytes = (uint32_t)a.D * a.elem_bytes;
  uintptr_t align_bits = (uintptr_t)a.chunk;
  for (int i = 0; i < a.n_planes; ++i) align_bits |= (uintptr_t)a.planes[i];
  int vec = 16;
  while (vec > a.elem_bytes && ((unit_bytes % vec) != 0 || (align_bits % vec) != 0)) vec >>= 1;
  const uint32_t per_elem = (uint32_t)(vec / a.elem_bytes);  // elements per vector

  ChunkGeom g;
  for (int i = 0; i < 3; ++i) g.planes[i] = static_cast<char*>(i < a.n_planes ? a.planes[i] : nullptr);
  g.chunk = static_cast<char*>(a.chunk);
  g.B = (uint32_t)a.B;
  g.plane_b_rows = (uint32_t)a.plane_b_rows;
  g.plane_row = (uint32_t)(a.plane_row / per_elem);
  uint64_t max_block = 0;
  for (int p = 0; p < a.n_peers; ++p) {
    const ChunkPeer& c = a.peer[p];
    PeerGeom& q = g.peer[p];
    q.run = (uint32_t)(c.run / per_elem);
    q.rows = (uint32_t)c.rows;
    q.chunk_rows = (uint32_t)c.chunk_rows;
    if (q.run == 0 || q.chunk_rows == 0) {  // empty chunk: no workgroup does anything
      q.run = 1;
      q.rows = q.chunk_rows = 0;
    }
    q.div_run = make_fastdiv(q.run);
    q.plane_off = (uint32_t)(c.plane_off / per_elem);
    q.chunk_off = (uint32_t)(c.chunk_off / per_elem);
    const uint64_t blk = (uint64_t)q.chunk_rows * q.run;
    if (blk > max_block) max_block = blk;
  }
  const uint64_t gx = (max_block + kThreads - 1) / kThreads;
  const uint32_t gz = (uint32_t)(a.n_planes * a.B);
  if (gx == 0 || gz == 0 || a.n_peers == 0) return hipSuccess;
  const dim3 grid((unsigned)gx, (unsigned)a.n_peers, gz);
  switch (vec) {
    case 16: return launch_v<u32x4>(g, a.to_chunk, grid, stream);
    case 8: return launch_v<u32x2>(g, a.to_chunk, grid, stream);
    case 4: return launch_v<uint32_t>(g, a.to_chunk, grid, stream);
    default: return launch_v<uint16_t>(g, a.to_chunk, grid, stream);
  }
}

}  // namespace dit
