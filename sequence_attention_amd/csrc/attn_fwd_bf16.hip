// bf16 flash attention with per-row LSE on CDNA4 matrix cores (gfx950).
//
// Operation (edge-dit.cpp "Parallel execution", Ulysses section): after the
// sequence-to-head exchange a rank evaluates exact, non-causal
// O = softmax(scale * Q K^T) V over the full sequence for its heads.  SGLang
// "Parallelism Overview" (Constraints) requires a ring-capable kernel to
// also return the per-row softmax LSE, which the online-softmax merge of the
// ring hops consumes; LSE = ln sum_j exp(scale * q . k_j).
//
// Design (MI355X-first, not a translation of any CUDA kernel):
//  * A workgroup of 4 waves owns 128 query rows of one (b, h); each wave owns
//    32 rows and keeps its Q slice in registers for the whole key loop.
//  * Keys are consumed in blocks of 64, staged in LDS: K row-major (padded
//    rows, conflict-free 16-byte operand reads) and V transposed to [d][key]
//    so that the PV product can take V as the A operand.
//  * Both products use v_mfma_f32_32x32x16_bf16 in a transposed orientation:
//    S^T = K Q^T and O^T = V^T P^T.  The S^T accumulator gives each lane one
//    query and 16 keys, so the row max needs one swap with the partner lane
//    (l ^ 32), the row sum stays lane-local until the end, the rescale of
//    O^T by exp(m_old - m_new) is a per-lane scalar, and the accumulator
//    registers, rounded to bf16, are directly the B operand of the PV MFMA.
//    The key order inside each 16-key step implied by that reuse is absorbed
//    by storing V^T with the matching permutation (bits 2 and 3 of the key
//    index swapped inside each group of 16).
//  * Softmax runs in fp32 with exp2 and scale*log2(e) folded into one FMA;
//    tail keys past Skv are masked to -inf, tail query rows are never stored.
//  * Work tiles are renumbered so that consecutive query tiles of one head
//    land on the same XCD (workgroups are dealt round-robin over the 8
//    XCDs): the head's K/V stream is then served from that XCD's L2.
#include "dit_internal.h"

namespace dit {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kBM = 32 * kWaves;  // query rows per workgroup
constexpr int kBN = 64;           // keys per block
constexpr int kNumXcd = 8;
constexpr float kLog2e = 1.4426950408889634f;

struct Params {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  void* o;
  float* lse;
  int32_t Sq, Skv, H;
  int32_t n_qtiles;
  uint32_t n_tiles;
  float scale;
};

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& u) {
  return __builtin_bit_cast(bf16x8, u);
}

// Position of key kl (0..63) inside a V^T row: bits 2 and 3 swapped.
__device__ __forceinline__ int vt_pos(int kl) {
  return (kl & ~12) | ((kl & 4) << 1) | ((kl & 8) >> 1);
}

__device__ __forceinline__ uint32_t tile_of_block(uint32_t bid, uint32_t n) {
  const uint32_t xcd = bid % kNumXcd, local = bid / kNumXcd;
  const uint32_t q = n / kNumXcd, r = n % kNumXcd;
  return xcd < r ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
}

template <int D, bool kOutF32>
__global__ __launch_bounds__(kThreads, 2) void attn_bf16_kernel(Params p) {
  constexpr int KS = D + 8;       // K row stride in LDS (bf16 elements)
  constexpr int VS = kBN + 8;     // V^T row stride in LDS
  constexpr int KSTEPS = D / 16;  // MFMA k-steps over the head dim
  constexpr int DT = D / 32;      // 32-row tiles of O^T
  constexpr int KCHUNKS = kBN * D / 8 / kThreads;  // 16-byte K loads per thread
  constexpr int VUNITS = (kBN / 4) * (D / 8);       // 4-key x 8-dim V units
  static_assert(KCHUNKS >= 1 && VUNITS <= kThreads, "tile shape");

  __shared__ __attribute__((aligned(16))) uint16_t ks[kBN * KS];
  __shared__ __attribute__((aligned(16))) uint16_t vt[D * VS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int g = lane >> 5;

  const uint32_t tile = tile_of_block(blockIdx.x, p.n_tiles);
  const int qt = tile % p.n_qtiles;
  const int bh = tile / p.n_qtiles;
  const int h = bh % p.H;
  const int b = bh / p.H;
  const size_t rs = (size_t)p.H * D;  // elements between sequence rows
  const uint16_t* kbase = p.k + (size_t)b * p.Skv * rs + (size_t)h * D;
  const uint16_t* vbase = p.v + (size_t)b * p.Skv * rs + (size_t)h * D;

  // ---- Q slice of this wave in registers: B operand of S^T = K Q^T -------
  const int q_row = qt * kBM + wave * 32 + l32;
  const bool q_ok = q_row < p.Sq;
  bf16x8 qf[KSTEPS];
  {
    const uint16_t* qp = p.q + ((size_t)b * p.Sq + (q_ok ? q_row : 0)) * rs + (size_t)h * D + 8 * g;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      uint4 u = q_ok ? *reinterpret_cast<const uint4*>(qp + kk * 16) : make_uint4(0, 0, 0, 0);
      qf[kk] = as_bf16x8(u);
    }
  }

  // ---- global -> register prefetch of one K/V block ------------------------
  uint4 kreg[KCHUNKS];
  uint4 vreg[4];
  const bool v_active = tid < VUNITS;
  const int v_kg = tid % (kBN / 4);  // key group of 4 (lanes -> consecutive groups)
  const int v_dc = tid / (kBN / 4);  // 8-wide column chunk
  auto load_block = [&](int j0) {
#pragma unroll
    for (int i = 0; i < KCHUNKS; ++i) {
      const int c = tid + i * kThreads;
      const int row = c / (D / 8), col = c % (D / 8);
      const int j = j0 + row;
      kreg[i] = j < p.Skv ? *reinterpret_cast<const uint4*>(kbase + (size_t)j * rs + col * 8)
                          : make_uint4(0, 0, 0, 0);
    }
    if (v_active) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = j0 + 4 * v_kg + r;
        vreg[r] = j < p.Skv ? *reinterpret_cast<const uint4*>(vbase + (size_t)j * rs + v_dc * 8)
                            : make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto store_block = [&]() {
#pragma unroll
    for (int i = 0; i < KCHUNKS; ++i) {
      const int c = tid + i * kThreads;
      const int row = c / (D / 8), col = c % (D / 8);
      *reinterpret_cast<uint4*>(&ks[row * KS + col * 8]) = kreg[i];
    }
    if (v_active) {
      // 4 keys x 8 dims -> 8 rows of V^T, 4 consecutive (permuted) key slots each
      const uint32_t* w0 = &vreg[0].x;
      const uint32_t* w1 = &vreg[1].x;
      const uint32_t* w2 = &vreg[2].x;
      const uint32_t* w3 = &vreg[3].x;
      const int pos = vt_pos(4 * v_kg);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // dims 2e (low halves) and 2e+1 (high halves)
        uint2 lo, hi;
        lo.x = __builtin_amdgcn_perm(w1[e], w0[e], 0x05040100u);
        lo.y = __builtin_amdgcn_perm(w3[e], w2[e], 0x05040100u);
        hi.x = __builtin_amdgcn_perm(w1[e], w0[e], 0x07060302u);
        hi.y = __builtin_amdgcn_perm(w3[e], w2[e], 0x07060302u);
        const int d = v_dc * 8 + 2 * e;
        *reinterpret_cast<uint2*>(&vt[d * VS + pos]) = lo;
        *reinterpret_cast<uint2*>(&vt[(d + 1) * VS + pos]) = hi;
      }
    }
  };

  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.0f;
  float m = -INFINITY;  // running max of raw scores q . k (unscaled)
  float lsum = 0.0f;    // this lane's share of the row sum
  const float c = p.scale * kLog2e;

  const int nblocks = (p.Skv + kBN - 1) / kBN;
  load_block(0);
  for (int kb = 0; kb < nblocks; ++kb) {
    const int j0 = kb * kBN;
    __syncthreads();  // previous block's LDS reads are done
    store_block();
    __syncthreads();
    if (kb + 1 < nblocks) load_block(j0 + kBN);

    // S^T = K Q^T: two 32-key tiles
    f32x16 s[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[t][r] = 0.0f;
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) {
        const uint4 a = *reinterpret_cast<const uint4*>(&ks[(32 * t + l32) * KS + kk * 16 + 8 * g]);
        s[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), qf[kk], s[t], 0, 0, 0);
      }
    }
    // lane holds S^T[key = 32t + 8(r/4) + 4g + r%4][query l32]
    if (j0 + kBN > p.Skv) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j0 + 32 * t + 8 * (r >> 2) + 4 * g + (r & 3);
          if (key >= p.Skv) s[t][r] = -INFINITY;
        }
    }
    float mx = s[0][0];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[t][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m, mx);
    const float alpha = __builtin_amdgcn_exp2f((m - m_new) * c);
    const float mc = m_new * c;
    m = m_new;

    bf16x8 pb[2][2];
    float bsum = 0.0f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][r], c, -mc));
        bsum += pr;
        pb[t][r >> 3][r & 7] = (__bf16)pr;
      }
    lsum = __builtin_fmaf(lsum, alpha, bsum);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;

    // O^T += V^T P^T: 4 key steps of 16
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int jh = 0; jh < 2; ++jh) {
        const int kofs = (2 * t + jh) * 16 + 8 * g;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const uint4 a = *reinterpret_cast<const uint4*>(&vt[(dt * 32 + l32) * VS + kofs]);
          oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), pb[t][jh], oacc[dt], 0, 0, 0);
        }
      }
  }

  // ---- epilogue: normalise, store O (lane: one query, 16 dims per tile) ---
  const float ltot = lsum + __shfl_xor(lsum, 32);
  if (!q_ok) return;
  const float inv = 1.0f / ltot;
  const size_t orow = ((size_t)b * p.Sq + q_row) * rs + (size_t)h * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int d = dt * 32 + 8 * u + 4 * g;
      const float o0 = oacc[dt][4 * u + 0] * inv, o1 = oacc[dt][4 * u + 1] * inv;
      const float o2 = oacc[dt][4 * u + 2] * inv, o3 = oacc[dt][4 * u + 3] * inv;
      if constexpr (kOutF32) {
        *reinterpret_cast<float4*>(static_cast<float*>(p.o) + orow + d) = make_float4(o0, o1, o2, o3);
      } else {
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        bf16x4 w;
        w[0] = (__bf16)o0; w[1] = (__bf16)o1; w[2] = (__bf16)o2; w[3] = (__bf16)o3;
        *reinterpret_cast<bf16x4*>(static_cast<uint16_t*>(p.o) + orow + d) = w;
      }
    }
  if (p.lse != nullptr && g == 0)
    p.lse[((size_t)b * p.H + h) * p.Sq + q_row] = m * p.scale + __logf(ltot);
}

template <int D, bool kOutF32>
hipError_t launch_t(const AttnArgs& a, hipStream_t stream) {
  Params p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.o = a.o;
  p.lse = a.lse;
  p.Sq = a.Sq;
  p.Skv = a.Skv;
  p.H = a.H;
  p.n_qtiles = (a.Sq + kBM - 1) / kBM;
  p.n_tiles = (uint32_t)p.n_qtiles * a.H * a.B;
  p.scale = a.scale;
  attn_bf16_kernel<D, kOutF32><<<p.n_tiles, kThreads, 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd_bf16(const AttnArgs& a, hipStream_t stream) {
  if (a.D == 64) return a.o_f32 ? launch_t<64, true>(a, stream) : launch_t<64, false>(a, stream);
  return a.o_f32 ? launch_t<128, true>(a, stream) : launch_t<128, false>(a, stream);
}

}  // namespace dit
