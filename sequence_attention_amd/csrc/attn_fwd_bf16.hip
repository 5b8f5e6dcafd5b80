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
//  * Keys are consumed in blocks of 64.  K and V blocks go from HBM/L2
//    straight into LDS with global_load_lds_dwordx4 (no VGPR staging, no
//    VALU), double-buffered so that the next block streams in while the
//    current one is multiplied; one barrier per block.  Rows are stored with
//    an XOR swizzle of their 16-byte chunks, chosen so that both operand
//    reads below are bank-conflict free.
//  * Both products use v_mfma_f32_32x32x16_bf16 in a transposed orientation:
//    S^T = K Q^T and O^T = V^T P^T.  The S^T accumulator gives each lane one
//    query and 16 keys, so the row max needs one swap with the partner lane
//    (l ^ 32), the row sum stays lane-local until the end, the rescale of
//    O^T is a per-lane scalar, and the accumulator registers, rounded to
//    bf16, are directly the B operand of the PV MFMA.  The A operand V^T is
//    read from row-major V with ds_read_b64_tr_b16 (gfx950 LDS transpose
//    read: a 16-lane group gets a 4-key x 16-dim block with one dim per
//    lane), in the key order the accumulator reuse implies.
//  * Softmax runs in fp32 with exp2 and scale*log2(e) folded into one FMA.
//    The running max is only raised when a block's max exceeds it by more
//    than 2^8 in the exp2 domain (a wave-uniform branch), so the O rescale
//    is rare; P then stays <= 256, exact enough in bf16 and far from fp32
//    limits.  Tail keys past Skv are clamped on load and masked to -inf;
//    tail query rows are never stored.
//  * Work tiles are renumbered so that consecutive query tiles of one head
//    land on the same XCD (workgroups are dealt round-robin over the 8
//    XCDs): the head's K/V stream is then served from that XCD's L2.
#include <type_traits>

#include "dit_internal.h"

namespace dit {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void gbl_void;

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kBM = 32 * kWaves;  // query rows per workgroup
constexpr int kBN = 64;           // keys per block
constexpr int kNumXcd = 8;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleLog2 = 8.0f;  // lazy-rescale threshold (exp2 domain)

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

__device__ __forceinline__ uint32_t tile_of_block(uint32_t bid, uint32_t n) {
  const uint32_t xcd = bid % kNumXcd, local = bid / kNumXcd;
  const uint32_t q = n / kNumXcd, r = n % kNumXcd;
  return xcd < r ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
}

// XOR swizzle of the 16-byte chunk index inside an LDS row of K or V.
// D = 128 (16 chunks, 256-byte rows): a bit permutation of r mod 16, so the
//   32 rows of an A-operand read (same logical chunk) hit 16 distinct chunk
//   positions per half wave, and the 4 rows of a transpose read land their
//   two chunks on 8 distinct positions.
// D = 64 (8 chunks, 128-byte rows, two rows per bank line): the same two
//   properties with the row parity taking one bank half.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) return ((r & 3) << 1) | ((r >> 2) & 1) | (r & 8);
  else return (((r >> 1) & 3) << 1) | ((r >> 3) & 1);
}

template <int D, bool kOutF32>
__global__ __launch_bounds__(kThreads, 2) void attn_bf16_kernel(Params p) {
  constexpr int ROWB = D * 2;                 // bytes of one K/V row
  constexpr int BLKB = kBN * ROWB;            // bytes of one K or V block
  constexpr int NINSTR = BLKB / 1024;         // 1 KB direct loads per tensor per block
  constexpr int INSTR_W = NINSTR / kWaves;    // ... per wave
  constexpr int KSTEPS = D / 16;              // MFMA k-steps over the head dim
  constexpr int DT = D / 32;                  // 32-row tiles of O^T
  static_assert(NINSTR % kWaves == 0, "direct-load split");

  // Two stages of K and V as four distinct LDS objects: the compiler can then
  // prove that a direct load into one stage does not alias reads of the
  // other and does not wait for the load before those reads.
  __shared__ __attribute__((aligned(1024))) char k_st0[BLKB];
  __shared__ __attribute__((aligned(1024))) char v_st0[BLKB];
  __shared__ __attribute__((aligned(1024))) char k_st1[BLKB];
  __shared__ __attribute__((aligned(1024))) char v_st1[BLKB];

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
      const uint4 u = q_ok ? *reinterpret_cast<const uint4*>(qp + kk * 16) : make_uint4(0, 0, 0, 0);
      qf[kk] = __builtin_bit_cast(bf16x8, u);
    }
  }

  // ---- direct global -> LDS loads of one K and one V block ----------------
  // lane i of load instruction j fills LDS bytes j*1024 + 16*i of the block:
  // row = that offset / ROWB, physical chunk pc, logical chunk pc ^ swz(row).
  int ld_row[INSTR_W], ld_col[INSTR_W];
#pragma unroll
  for (int u = 0; u < INSTR_W; ++u) {
    const int off = (wave * INSTR_W + u) * 1024 + lane * 16;
    ld_row[u] = off / ROWB;
    ld_col[u] = (((off % ROWB) / 16) ^ swz<D>(ld_row[u])) * 8;  // element column
  }
  const int last_key = p.Skv - 1;
  auto issue_block = [&](int j0, char* kdst, char* vdst) {
#pragma unroll
    for (int u = 0; u < INSTR_W; ++u) {
      const int j = min(j0 + ld_row[u], last_key);  // tail rows: any valid row, masked later
      const size_t go = (size_t)j * rs + ld_col[u];
      const int dst = (wave * INSTR_W + u) * 1024;
      __builtin_amdgcn_global_load_lds((gbl_void*)(kbase + go), (lds_void*)(kdst + dst), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((gbl_void*)(vbase + go), (lds_void*)(vdst + dst), 16, 0, 0);
    }
  };

  // ---- per-lane LDS read offsets ------------------------------------------
  // K operand (ds_read_b128): row 32t + l32, logical chunk 2kk + g.
  const int k_sw = swz<D>(l32);
  // V^T operand (ds_read_b64_tr_b16): in a 16-lane group, lane i16 addresses
  // key row (base + i16/4) and dims 4*(i16%4)..+3 of the group's 16 dims.
  const int i16 = lane & 15;
  const int g16 = (lane >> 4) & 1;     // which 16 dims of the 32-dim tile
  const int v_rsub = i16 >> 2;         // key row inside the 4-row group
  const int v_piece = i16 & 3;         // 4-dim piece inside the 16 dims

  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.0f;
  float m_used = -INFINITY;  // running reference max of raw scores q . k
  float lsum = 0.0f;         // this lane's share of the row sum
  const float c = p.scale * kLog2e;

  const int nblocks = (p.Skv + kBN - 1) / kBN;
  // one key block from stage ST; the next block is streamed into stage ST^1
  auto block = [&](auto stage, int kb) {
    constexpr bool ST = decltype(stage)::value;
    const int j0 = kb * kBN;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's loads of block kb landed
    __syncthreads();                     // ... and everyone's; stage ST^1 is free again
    if (kb + 1 < nblocks) {
      if constexpr (ST) issue_block(j0 + kBN, k_st0, v_st0);
      else issue_block(j0 + kBN, k_st1, v_st1);
    }
    const char* ks = ST ? k_st1 : k_st0;
    const char* vs = ST ? v_st1 : v_st0;

    // S^T = K Q^T: two 32-key tiles
    f32x16 s[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[t][r] = 0.0f;
      const char* krow = ks + (32 * t + l32) * ROWB;
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) {
        const uint4 a = *reinterpret_cast<const uint4*>(krow + (((2 * kk + g) ^ k_sw) << 4));
        s[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), qf[kk], s[t], 0, 0, 0);
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
    const bool raise = (mx - m_used) * c > kRescaleLog2;
    if (__any(raise)) {
      const float m_new = raise ? mx : m_used;
      const float alpha = __builtin_amdgcn_exp2f((m_used - m_new) * c);
      lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
      m_used = m_new;
    }
    const float mc = m_used * c;

    // LSE needs the row sum of the unrounded P: a bf16-rounded sum would be
    // off by up to 2^-9 relative (about 2e-3 in LSE) on near one-hot rows.
    bf16x8 pb[2][2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][r], c, -mc));
        lsum += pr;
        pb[t][r >> 3][r & 7] = (__bf16)pr;
      }

    // O^T += V^T P^T: 4 key steps of 16 keys
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int jh = 0; jh < 2; ++jh) {
        const int kbase16 = (2 * t + jh) * 16;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          i16x4 half[2];
#pragma unroll
          for (int rd = 0; rd < 2; ++rd) {
            const int row = kbase16 + 8 * rd + 4 * g + v_rsub;
            const int d = dt * 32 + 16 * g16 + 4 * v_piece;
            const int off = row * ROWB + ((((d >> 3) ^ swz<D>(row))) << 4) + ((d & 4) << 1);
            half[rd] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(vs + off));
          }
          const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7));
          oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[t][jh], oacc[dt], 0, 0, 0);
        }
      }
  };
  issue_block(0, k_st0, v_st0);
  for (int kb = 0; kb < nblocks; kb += 2) {
    block(std::integral_constant<bool, false>{}, kb);
    if (kb + 1 < nblocks) block(std::integral_constant<bool, true>{}, kb + 1);
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
    p.lse[((size_t)b * p.H + h) * p.Sq + q_row] = m_used * p.scale + __logf(ltot);
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
