// Attention over an empty key set (Skv == 0): O = 0 and LSE = -inf, the
// identity element of the online-softmax merge, so an empty ring hop merges
// away exactly.  Written with a fill kernel rather than a memset so that the
// call stays safe inside a captured HIP graph.
#include "dit_internal.h"

namespace dit {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void fill_kernel(uint32_t* __restrict__ o, uint64_t o_words,
                                                        float* __restrict__ lse, uint64_t n_lse) {
  const uint64_t stride = (uint64_t)gridDim.x * kThreads;
  for (uint64_t i = (uint64_t)blockIdx.x * kThreads + threadIdx.x; i < o_words; i += stride) o[i] = 0u;
  if (lse != nullptr)
    for (uint64_t i = (uint64_t)blockIdx.x * kThreads + threadIdx.x; i < n_lse; i += stride)
      lse[i] = -INFINITY;
}

}  // namespace

hipError_t launch_attn_empty(const AttnArgs& a, bool in_f32, hipStream_t stream) {
  const uint64_t elems = (uint64_t)a.B * a.Sq * a.H * a.D;
  const uint64_t o_bytes = elems * ((in_f32 || a.o_f32) ? 4 : 2);
  const uint64_t words = o_bytes / 4;  // D is even, so whole 32-bit words
  const uint64_t n_lse = (uint64_t)a.B * a.H * a.Sq;
  const uint64_t work = words > n_lse ? words : n_lse;
  uint64_t blocks = (work + kThreads - 1) / kThreads;
  if (blocks > 4096) blocks = 4096;
  if (blocks == 0) return hipSuccess;
  fill_kernel<<<(unsigned)blocks, kThreads, 0, stream>>>(static_cast<uint32_t*>(a.o), words, a.lse, n_lse);
  return hipGetLastError();
}

}  // namespace dit
