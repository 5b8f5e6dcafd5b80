// fp32 attention with per-row LSE: the full-precision path (gfx950).
//
// Same operation as the bf16 MFMA kernel (edge-dit.cpp "Parallel
// execution", Ulysses section: exact softmax attention of the rank's heads;
// SGLang "Parallelism Overview", Constraints: LSE exposed for the ring
// merge), computed in fp32 throughout for callers whose tensors are fp32.
// This is the accuracy path, not the throughput path: two lanes own one
// query row (each holds half of q and of the O accumulator in registers and
// the two halves of a dot product meet with one lane swap), a workgroup of
// 64 rows shares K and V tiles of 32 keys staged in LDS (lanes read the same
// key, so LDS reads are broadcasts), and the online softmax rescales once
// per tile.
#include "dit_internal.h"

namespace dit {
namespace {

constexpr int kRows = 64;   // query rows per workgroup
constexpr int kKeys = 32;   // keys per LDS tile
constexpr int kThreads = 2 * kRows;  // two lanes per row, each owning D/2 columns

template <int D, bool kMerge>
__global__ __launch_bounds__(kThreads) void attn_f32_kernel(const float* __restrict__ q,
                                                            const float* __restrict__ k,
                                                            const float* __restrict__ v,
                                                            float* __restrict__ o,
                                                            float* __restrict__ lse,
                                                            const int32_t* __restrict__ kv_len,
                                                            int32_t Sq, int32_t Skv, int32_t H,
                                                            float scale) {
  constexpr int DH = D / 2;
  __shared__ float ks[kKeys][D];
  __shared__ float vs[kKeys][D];
  const int b = blockIdx.z, h = blockIdx.y;
  const int half = threadIdx.x & 1;
  const int i = blockIdx.x * kRows + (threadIdx.x >> 1);
  const bool row_ok = i < Sq;
  const size_t row_stride = (size_t)H * D;  // elements between consecutive sequence rows
  // keys of this batch that take part (tail-padded keys are excluded)
  const int skv = kv_len != nullptr ? min(max(kv_len[b], 0), Skv) : Skv;
  if (skv == 0) {  // the merge identity, or an untouched accumulator
    if (!kMerge && row_ok) {
      float* op = o + ((size_t)b * Sq + i) * row_stride + (size_t)h * D + half * (D / 2);
      for (int d = 0; d < D / 2; ++d) op[d] = 0.0f;
      if (lse && half == 0) lse[((size_t)b * H + h) * Sq + i] = -INFINITY;
    }
    return;
  }

  float qr[DH], acc[DH];
  const float* qp = q + ((size_t)b * Sq + (row_ok ? i : 0)) * row_stride + (size_t)h * D + half * DH;
#pragma unroll
  for (int d = 0; d < DH; ++d) {
    qr[d] = row_ok ? qp[d] : 0.0f;
    acc[d] = 0.0f;
  }
  float m = -INFINITY, l = 0.0f;

  for (int j0 = 0; j0 < skv; j0 += kKeys) {
    __syncthreads();
    for (int e = threadIdx.x; e < kKeys * D; e += kThreads) {
      const int jj = e / D, d = e % D;
      const int j = j0 + jj;
      const size_t off = ((size_t)b * Skv + (j < skv ? j : 0)) * row_stride + (size_t)h * D + d;
      ks[jj][d] = j < skv ? k[off] : 0.0f;
      vs[jj][d] = j < skv ? v[off] : 0.0f;
    }
    __syncthreads();
    const int nk = min(kKeys, skv - j0);
    float s[kKeys];
    float mt = -INFINITY;
#pragma unroll
    for (int jj = 0; jj < kKeys; ++jj) {
      float part = 0.0f;
#pragma unroll
      for (int d = 0; d < DH; ++d) part = __builtin_fmaf(qr[d], ks[jj][half * DH + d], part);
      const float dot = (part + __shfl_xor(part, 1)) * scale;
      s[jj] = jj < nk ? dot : -INFINITY;
      mt = fmaxf(mt, s[jj]);
    }
    const float mn = fmaxf(m, mt);
    const float alpha = expf(m - mn);  // m = -inf on the first tile: alpha = 0
    l *= alpha;
#pragma unroll
    for (int d = 0; d < DH; ++d) acc[d] *= alpha;
#pragma unroll
    for (int jj = 0; jj < kKeys; ++jj) {
      const float p = expf(s[jj] - mn);  // masked keys: exp(-inf) = 0
      l += p;
#pragma unroll
      for (int d = 0; d < DH; ++d) acc[d] = __builtin_fmaf(p, vs[jj][half * DH + d], acc[d]);
    }
    m = mn;
  }
  if (!row_ok) return;
  float* op = o + ((size_t)b * Sq + i) * row_stride + (size_t)h * D + half * DH;
  const size_t lse_idx = ((size_t)b * H + h) * Sq + i;
  const float l_c = m + logf(l);
  float cc = 1.0f / l, ca = 0.0f, l_new = l_c;
  if constexpr (kMerge) {
    // merge into the partial result already in (o, lse): online-softmax
    // rule, an accumulator with LSE = -inf is replaced; both lanes of the
    // row read the old LSE before lane 0 writes it (same wave)
    const float l_a = lse[lse_idx];
    if (l_a != -INFINITY) {
      const float mm = fmaxf(l_a, l_c);
      const float wa = expf(l_a - mm), wc = expf(l_c - mm);
      const float den = wa + wc;
      ca = wa / den;
      cc = wc / (den * l);
      l_new = mm + logf(den);
    }
  }
  // an empty accumulator (ca = 0) is never read: it may hold anything
  const bool use_prev = kMerge && ca != 0.0f;
#pragma unroll
  for (int d = 0; d < DH; ++d) {
    float r = acc[d] * cc;
    if (use_prev) r = __builtin_fmaf(ca, op[d], r);
    op[d] = r;
  }
  if (lse && half == 0) lse[lse_idx] = l_new;
}

template <int D>
hipError_t launch_d(const AttnArgs& a, hipStream_t stream) {
  dim3 grid((a.Sq + kRows - 1) / kRows, a.H, a.B);
  if (a.merge)
    attn_f32_kernel<D, true><<<grid, kThreads, 0, stream>>>(
        static_cast<const float*>(a.q), static_cast<const float*>(a.k), static_cast<const float*>(a.v),
        static_cast<float*>(a.o), a.lse, a.kv_len, a.Sq, a.Skv, a.H, a.scale);
  else
    attn_f32_kernel<D, false><<<grid, kThreads, 0, stream>>>(
        static_cast<const float*>(a.q), static_cast<const float*>(a.k), static_cast<const float*>(a.v),
        static_cast<float*>(a.o), a.lse, a.kv_len, a.Sq, a.Skv, a.H, a.scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd_f32(const AttnArgs& a, hipStream_t stream) {
  return a.D == 64 ? launch_d<64>(a, stream) : launch_d<128>(a, stream);
}

}  // namespace dit
