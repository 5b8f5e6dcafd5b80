// Fills around attention stored straight into the head-to-sequence send
// buffer (edge-dit.cpp "Parallel execution", packed head-to-sequence
// operator: the output partitioned by destination sequence shard into a
// peer-major buffer).  Attention writes the real query rows; the pad rows
// of the padded sequence have no query and are zeroed here, and an empty
// key set (O = 0, LSE = -inf everywhere) is a plain fill.
#include "dit_internal.h"

namespace dit {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// One 16-byte vector per thread over the pad rows [t0, t1) of every batch.
__global__ __launch_bounds__(256) void send_rows_zero_kernel(u32x4* send, uint32_t total,
                                                             FastDiv div_row, FastDiv div_rows,
                                                             uint32_t row_vecs, uint32_t n_rows,
                                                             int32_t t0, int32_t S_loc, int32_t B) {
  const uint32_t i = blockIdx.x * 256u + threadIdx.x;
  if (i >= total) return;
  const uint32_t r = fdiv(i, div_row);          // (b, t) pair index
  const uint32_t e = i - r * row_vecs;
  const uint32_t b = fdiv(r, div_rows);
  const uint32_t t = (uint32_t)t0 + (r - b * n_rows);
  const uint32_t peer = t / (uint32_t)S_loc;
  const uint32_t s = t - peer * (uint32_t)S_loc;
  const size_t row = ((size_t)peer * B + b) * S_loc + s;
  __builtin_nontemporal_store(u32x4{0u, 0u, 0u, 0u}, send + row * row_vecs + e);
}

__global__ __launch_bounds__(256) void fill_words_kernel(uint32_t* p, uint64_t n, uint32_t value) {
  const uint64_t i = (uint64_t)blockIdx.x * 256u + threadIdx.x;
  if (i < n) p[i] = value;
}

}  // namespace

hipError_t launch_send_rows_zero(void* send, int32_t B, int32_t S_loc, int32_t t0, int32_t t1,
                                 int64_t row_elems, hipStream_t stream) {
  if (B <= 0 || t1 <= t0 || row_elems <= 0) return hipSuccess;
  const uint32_t row_vecs = (uint32_t)(row_elems * 2 / 16);
  const uint32_t n_rows = (uint32_t)(t1 - t0);
  const uint64_t total = (uint64_t)B * n_rows * row_vecs;
  const uint32_t blocks = (uint32_t)((total + 255) / 256);
  send_rows_zero_kernel<<<blocks, 256, 0, stream>>>(static_cast<u32x4*>(send), (uint32_t)total,
                                                     make_fastdiv(row_vecs), make_fastdiv(n_rows),
                                                     row_vecs, n_rows, t0, S_loc, B);
  return hipGetLastError();
}

hipError_t launch_fill_words(void* p, uint64_t n, uint32_t value, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const uint64_t blocks = (n + 255) / 256;
  fill_words_kernel<<<(unsigned)blocks, 256, 0, stream>>>(static_cast<uint32_t*>(p), n, value);
  return hipGetLastError();
}

}  // namespace dit
