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
//  * A workgroup of 8 waves (2 per SIMD) owns 256 query rows of one (b, h);
//    each wave owns 32 rows and keeps its Q slice in registers for the whole
//    key loop.  All 8 waves share each K/V block, so L2 traffic is one K/V
//    pass per 256 query rows.
//  * Keys are consumed in blocks of 64.  K and V blocks go from L2 straight
//    into LDS with buffer_load_dwordx4 ... lds (no VGPR staging; the
//    per-block address is a scalar buffer base, so no VALU either) through a
//    4-stage ring: after the barrier of block kb, block kb + 2 is issued
//    into the stage of block kb - 2, so two blocks are in flight while one
//    is multiplied (measured slightly faster than three ahead); one barrier
//    per block.  The address range of each block's buffer descriptor ends
//    at the last valid key (and is empty for a block past the workgroup's
//    range), so tail rows and the look-ahead past the end are out-of-range
//    loads that touch no memory: the block loop issues and waits the same
//    way every time, without branches.  Rows are stored with an XOR swizzle
//    of their 16-byte chunks, chosen so that both operand reads below are
//    bank-conflict free.
//  * Both products use v_mfma_f32_32x32x16_bf16 in a transposed orientation:
//    S^T = K Q^T and O^T = V^T P^T.  The S^T accumulator gives each lane one
//    query and 16 keys, so the row max needs one swap with the partner lane
//    (l ^ 32, v_permlane32_swap: a VALU op, no LDS round trip), the row sum
//    stays lane-local until the end, the rescale of
//    O^T is a per-lane scalar, and the accumulator registers, rounded to
//    bf16, are directly the B operand of the PV MFMA.  The A operand V^T is
//    read from row-major V with ds_read_b64_tr_b16 (gfx950 LDS transpose
//    read: a 16-lane group gets a 4-key x 16-dim block with one dim per
//    lane), in the key order the accumulator reuse implies.
//  * Softmax runs in fp32 with exp2 and scale*log2(e) folded into one FMA.
//    The weights are taken against a running reference score that is
//    raised only when some weight of a block would exceed 2^32 (a
//    wave-uniform test on the lanes' block sums, which also catches the
//    first block): no per-block row max is computed, and the O rescale is
//    rare.  Weights up to 2^32 keep fp32 sums and accumulators far from
//    overflow, and bf16 keeps 8 significant bits at any magnitude.  The PV product
//    uses P rounded to bf16, so O is normalised by the sum of those rounded
//    weights (a consistent weighted average of V rows): with the lazy
//    rescale the dominant weight of a near one-hot row is not exactly 1, and
//    normalising by the unrounded sum would leave its rounding error
//    (2^-9 |v|) in O.  LSE takes the sum of the unrounded weights.  Tail
//    keys past Skv read as zeros (out of the descriptor range) and are
//    masked to -inf; tail query rows are never stored.
//  * Inside a block the operand reads are pinned against the MFMAs with
//    scheduling-group barriers: four K reads in flight, then one per QK
//    MFMA; eight V reads in flight, then two per PV MFMA.
//  * Layouts: Q, K, V as [B, S, H, D] tensors, or (kIn 1, 2) as the three
//    planes of the Ulysses sequence-to-head receive buffer (edge-dit.cpp
//    "Parallel execution": the received, peer-major buffer is decoded by
//    the attention's own addressing instead of an unpack pass; with a chunk
//    length that is a multiple of 64 no key block straddles two peers and
//    the per-lane peer select is compiled out); O to [B, Sq, H, D] or
//    straight into the head-to-sequence send buffer.
//  * Work tiles are renumbered so that consecutive query tiles of one head
//    land on the same XCD (workgroups are dealt round-robin over the 8
//    XCDs): the head's K/V stream is then served from that XCD's L2.
#include <algorithm>
#include <atomic>
#include <mutex>
#include <type_traits>

#include "dit_internal.h"

namespace dit {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kBM = 32 * kWaves;  // query rows per workgroup
constexpr int kBN = 64;           // keys per block
constexpr int kNumXcd = 8;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kMaxWeight = 4294967296.0f;  // 2^32: largest block weight sum per lane against the reference
constexpr int kBufferWord3 = 0x00020000;  // raw buffer descriptor flags (gfx9 family)
constexpr uint64_t kMaxSplit = 8;        // key chunks per tile in the split round
constexpr int kScopeAgent = 16;           // buffer cache policy: sc1, device-scope coherent

struct Params {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  void* o;
  float* lse;
  float* part;    // partial-result slots, one per workgroup of the split round
  int32_t* cnt;   // arrival counters of the split tiles: zero on entry, left zero
  const int32_t* kv_len;  // valid keys per batch ([B], device), or null: all Skv
  int32_t Sq, Skv, H;
  int32_t n_qtiles;
  int32_t nblocks;   // key blocks per tile
  uint32_t n_whole;  // tiles taken whole, one per workgroup
  uint32_t split;    // pieces per tile of the split round (>= 2 when used)
  uint32_t split_wgs;  // workgroups of the split round: split x (tiles - n_whole)
  float scale;
  // Where O goes: send_rows == 0: [B, Sq, H, D].  Otherwise the peer-major
  // head-to-sequence send buffer [U, 1, B, send_rows, H, D]: query row t is
  // row t % send_rows of peer t / send_rows's chunk, and heads at or past
  // o_heads (pad heads) are stored as zeros.
  int32_t send_rows;
  int32_t send_batches;
  int32_t o_heads;
  // kRecv: Q, K and V are planes of the sequence-to-head receive buffer
  // [U, 3, B, in_rows, H, D] (q, k, v point at planes 0, 1, 2 of peer 0's
  // chunk; in_peer elements between peers): global row t is row t % in_rows
  // of peer t / in_rows.
  int32_t in_rows;
  int32_t in_last_peer;  // U - 1
  FastDiv in_div;        // division by in_rows
  int64_t in_peer;
};

// Element offset of the first dim of query row q_row of batch b in O
// (row stride rs = H * D elements).
__device__ __forceinline__ size_t o_row_offset(const Params& p, int b, int q_row, size_t rs) {
  if (p.send_rows == 0) return ((size_t)b * p.Sq + q_row) * rs;
  const int peer = q_row / p.send_rows;
  const int s = q_row - peer * p.send_rows;
  return (((size_t)peer * p.send_batches + b) * p.send_rows + s) * rs;
}

// Workgroups are dealt round-robin over the XCDs; renumber them so that each
// XCD owns one contiguous range of logical indices (a bijection on [0, n)).
__device__ __forceinline__ uint32_t logical_wg(uint32_t bid, uint32_t n) {
  const uint32_t xcd = bid % kNumXcd, local = bid / kNumXcd;
  const uint32_t q = n / kNumXcd, r = n % kNumXcd;
  return xcd < r ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
}

// XOR swizzle of the 16-byte chunk index inside an LDS row of K or V.
// gfx950's LDS serves 64 banks x 4 bytes per cycle: 16 lanes of a 16-byte
// read (the K operand) or 32 lanes of an 8-byte read (the V^T transpose
// read) per cycle.  The swizzle depends on r mod 16 only and keeps both
// conflict-free, also under a 32-bank reading (8 / 16 lanes per cycle):
//   K: any 16 aligned rows, same logical chunk, land on distinct banks;
//   V^T: 4 aligned rows x 4 consecutive logical chunks (D = 128; two rows
//   share a 256-byte bank line at D = 64) land on distinct banks.
// With r = (r3 r2 r1 r0): D = 128: (r1^r3, r0, r1, r2); D = 64: (r1, r0^r3, r2).
// (The counter SQ_LDS_BANK_CONFLICT reads 0 for both head sizes.)
template <int D>
__device__ __forceinline__ int swz(int r) {
  const int r0 = r & 1, r1 = (r >> 1) & 1, r2 = (r >> 2) & 1, r3 = (r >> 3) & 1;
  if constexpr (D == 128) return ((r1 ^ r3) << 3) | (r0 << 2) | (r1 << 1) | r2;
  else return (r1 << 2) | ((r0 ^ r3) << 1) | r2;
}

// s_waitcnt with vmcnt(n), other counters untouched (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 16, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

// Floats of one partial-result slot: per lane the D/2 accumulator registers
// of O^T, then the running max, the lane's share of the row sum and of the
// rounded-weight sum, and one unused float (16 bytes per lane).
template <int D>
constexpr size_t slot_floats() {
  return (size_t)kWaves * 64 * (D / 2 + 4);
}

// kIn: 0 Q, K, V as [B, S, H, D] tensors; 1 planes of the receive buffer;
// 2 the same when the chunk length is a multiple of the key block (no
// block then straddles two peers, and the per-lane peer select is dropped).
template <int D, bool kOutF32, bool kMerge, int kIn>
__global__ __launch_bounds__(kThreads, 2) void attn_bf16_kernel(Params p) {
  constexpr bool kRecv = kIn != 0;
  constexpr int ROWB = D * 2;                 // bytes of one K/V row
  constexpr int BLKB = kBN * ROWB;            // bytes of one K or V block
  constexpr int NINSTR = BLKB / 1024;         // 1 KB direct loads per tensor per block
  constexpr int INSTR_W = NINSTR / kWaves;    // ... per wave
  constexpr int LPB = 2 * INSTR_W;            // load instructions per block per wave (K + V)
  constexpr int KSTEPS = D / 16;              // MFMA k-steps over the head dim
  constexpr int DT = D / 32;                  // 32-row tiles of O^T
  constexpr size_t SLOT = slot_floats<D>();
  constexpr size_t ML_OFF = (size_t)kWaves * 64 * (D / 2);
  static_assert(NINSTR % kWaves == 0 && INSTR_W >= 1, "direct-load split");
  static_assert(2 * LPB < 16, "vmcnt budget");

  // The ring's stages are distinct LDS objects: the compiler can then prove
  // that a direct load into one stage does not alias reads of another and
  // does not wait for the load before those reads.
  __shared__ __attribute__((aligned(1024))) char k_s0[BLKB];
  __shared__ __attribute__((aligned(1024))) char v_s0[BLKB];
  __shared__ __attribute__((aligned(1024))) char k_s1[BLKB];
  __shared__ __attribute__((aligned(1024))) char v_s1[BLKB];
  __shared__ __attribute__((aligned(1024))) char k_s2[BLKB];
  __shared__ __attribute__((aligned(1024))) char v_s2[BLKB];
  __shared__ __attribute__((aligned(1024))) char k_s3[BLKB];
  __shared__ __attribute__((aligned(1024))) char v_s3[BLKB];
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int g = lane >> 5;
  const size_t rs = (size_t)p.H * D;  // elements between sequence rows
  const int nblocks = p.nblocks;
  const float c = p.scale * kLog2e;

  // ---- direct L2 -> LDS load geometry ----------------------------------------
  // lane i of load instruction j fills LDS bytes j*1024 + 16*i of the block:
  // row = that offset / ROWB, physical chunk pc, logical chunk pc ^ swz(row).
  // The block's base address is a scalar buffer descriptor, so the per-lane
  // byte offset is loop-invariant; rows past the last key are out of the
  // descriptor's range (read as zeros, their scores masked).
  uint32_t ld_off[INSTR_W];
  int ld_row[INSTR_W];
#pragma unroll
  for (int u = 0; u < INSTR_W; ++u) {
    const int off = (wave * INSTR_W + u) * 1024 + lane * 16;
    const int row = off / ROWB;
    const int col = (((off % ROWB) / 16) ^ swz<D>(row)) * 8;  // element column
    ld_off[u] = (uint32_t)(((size_t)row * rs + col) * 2);
    ld_row[u] = row;
  }

  // ---- per-lane LDS read offsets ------------------------------------------
  // K operand (ds_read_b128): row 32t + l32, logical chunk 2kk + g.
  const int k_sw = swz<D>(l32);
  // V^T operand (ds_read_b64_tr_b16): in a 16-lane group, lane i16 addresses
  // key row (base + i16/4) and dims 4*(i16%4)..+3 of the group's 16 dims.
  const int i16 = lane & 15;
  const int g16 = (lane >> 4) & 1;     // which 16 dims of the 32-dim tile
  const int v_rsub = i16 >> 2;         // key row inside the 4-row group
  const int v_piece = i16 & 3;         // 4-dim piece inside the 16 dims

  // The workgroup's segment: key blocks [kb0, kb1) of one tile.  The first
  // n_whole workgroups take one tile each; the rest take key chunk
  // (j % split) of tile n_whole + j / split.  Workgroups are dealt
  // round-robin over the XCDs in index order; both ranges are renumbered so
  // that each XCD gets contiguous tiles (one head's K/V then streams through
  // that XCD's L2) and an even share of both kinds (n_whole is a multiple of
  // the XCD count whenever chunks follow).
  {
    const bool whole = blockIdx.x < p.n_whole;
    const uint32_t j = whole ? logical_wg(blockIdx.x, p.n_whole) : logical_wg(blockIdx.x - p.n_whole, p.split_wgs);
    const uint32_t piece = whole ? 0 : j % p.split;
    const uint32_t tile = whole ? j : p.n_whole + j / p.split;
    const int kb0 = whole ? 0 : (int)((uint64_t)piece * nblocks / p.split);

    const int qt = tile % p.n_qtiles;
    const int bh = tile / p.n_qtiles;
    const int h = bh % p.H;
    const int b = bh / p.H;
    // keys of this batch that take part: with per-batch lengths (tail-padded
    // text) the keys past kv_len[b] are excluded, i.e. their scores are -inf
    const int skv = p.kv_len != nullptr ? min(max(p.kv_len[b], 0), p.Skv) : p.Skv;
    const int kb1 = min(whole ? nblocks : (int)((uint64_t)(piece + 1) * nblocks / p.split),
                        (skv + kBN - 1) / kBN);
    const size_t kv_batch = kRecv ? (size_t)p.in_rows : (size_t)p.Skv;  // rows between batches
    const uint16_t* kbase = p.k + (size_t)b * kv_batch * rs + (size_t)h * D;
    const uint16_t* vbase = p.v + (size_t)b * kv_batch * rs + (size_t)h * D;

    // ---- Q slice of this wave in registers: B operand of S^T = K Q^T -----
    const int q_row = qt * kBM + wave * 32 + l32;
    const bool q_ok = q_row < p.Sq;
    bf16x8 qf[KSTEPS];
    {
      const int qr = q_ok ? q_row : 0;
      const uint16_t* qp;
      if constexpr (kRecv) {
        const uint32_t peer = fdiv((uint32_t)qr, p.in_div);
        const int sr = qr - (int)peer * p.in_rows;
        qp = p.q + (size_t)peer * p.in_peer + ((size_t)b * p.in_rows + sr) * rs + (size_t)h * D + 8 * g;
      } else {
        qp = p.q + ((size_t)b * p.Sq + qr) * rs + (size_t)h * D + 8 * g;
      }
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) {
        const uint4 u = q_ok ? *reinterpret_cast<const uint4*>(qp + kk * 16) : make_uint4(0, 0, 0, 0);
        qf[kk] = __builtin_bit_cast(bf16x8, u);
      }
    }

    // kRecv: peer, local row and element offset of the next block to issue
    // (blocks are issued in increasing order, one at a time)
    uint32_t nx_p = 0, nx_s = 0;
    size_t nx_blk = 0;
    if constexpr (kRecv) {
      const uint32_t j = (uint32_t)kb0 * kBN;
      nx_p = fdiv(j, p.in_div);
      nx_s = j - nx_p * (uint32_t)p.in_rows;
      nx_blk = (size_t)nx_p * p.in_peer + (size_t)nx_s * rs;
    }
    auto issue = [&](int kb, char* kdst, char* vdst) __attribute__((always_inline)) {
      const int j0 = kb * kBN;
      size_t blk = (size_t)j0 * rs;  // element offset of the block's first row
      uint32_t nrec;                 // bytes from the block start that may be read
      uint32_t lim = kBN, jump = 0;  // kRecv: rows >= lim lie in the next peer's chunk
      if constexpr (kRecv) {
        // block rows before lim are rows s0.. of peer p0; the rest (in_rows
        // >= kBN, so at most one boundary) continue at row 0 of peer p0 + 1,
        // `jump` bytes further on; past the last peer's chunk nothing is read
        const uint32_t p0 = nx_p, s0 = nx_s;
        blk = nx_blk;
        lim = (uint32_t)p.in_rows - s0;
        nx_s = s0 + kBN;
        nx_blk += (size_t)kBN * rs;
        if (nx_s >= (uint32_t)p.in_rows) {
          nx_s -= (uint32_t)p.in_rows;
          nx_p += 1;
          nx_blk += (size_t)p.in_peer - (size_t)p.in_rows * rs;
        }
        jump = (uint32_t)((p.in_peer - (int64_t)p.in_rows * (int64_t)rs) * 2);
        const uint32_t last = (uint32_t)min((uint64_t)lim * (uint64_t)(rs * 2), (uint64_t)0x7fffffff);
        nrec = kb < kb1 ? ((int)p0 == p.in_last_peer ? last : 0x7fffffffu) : 0u;
      } else {
        // bytes of this batch's keys from the block start, none for a block
        // past kb1: loads beyond them are out of range, access no memory and
        // fill their LDS bytes with zeros (finite; those scores are masked)
        // (a scalar select, not a branch: the QK products and the weights
        // stay in one scheduling region)
        const uint32_t rows = kb < kb1 ? (uint32_t)max(skv - j0, 0) : 0u;
        nrec = (uint32_t)min((uint64_t)rows * (uint64_t)(rs * 2), (uint64_t)0x7fffffff);
      }
      const uint16_t* kb_ptr = kbase + blk;
      const uint16_t* vb_ptr = vbase + blk;
      const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc((void*)kb_ptr, (short)0, (int)nrec, kBufferWord3);
      const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc((void*)vb_ptr, (short)0, (int)nrec, kBufferWord3);
#pragma unroll
      for (int u = 0; u < INSTR_W; ++u) {
        uint32_t off = ld_off[u];
        if constexpr (kIn == 1) off += (uint32_t)ld_row[u] >= lim ? jump : 0u;
        const int dst = (wave * INSTR_W + u) * 1024;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void*)(kdst + dst), 16, off, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void*)(vdst + dst), 16, off, 0, 0, 0);
      }
    };

    f32x16 oacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.0f;
    float m_used = -INFINITY;  // running reference max of raw scores q . k
    float lsum = 0.0f;         // this lane's share of the row sum (for LSE)
    float lsum_r = 0.0f;       // ... of the bf16-rounded weights (normalises O)

    // one key block from stage ST; block kb + 2 is streamed into stage
    // ST + 2 (block kb - 2's); kMask: the block reaches past skv
    auto block = [&](auto stage, int kb, auto masked) __attribute__((always_inline)) {
      constexpr int ST = decltype(stage)::value;
      constexpr bool kMask = decltype(masked)::value;
      const int j0 = kb * kBN;
      // this wave's loads of block kb have landed once only those of block
      // kb + 1 are outstanding (always issued, past kb1 empty)
      wait_vmcnt<LPB>();
      // Workgroup barrier without __syncthreads()'s release fence, which
      // would wait for every outstanding load (vmcnt(0)) and drain the ring.
      // LDS reads of the stage being recycled completed before their MFMAs
      // issued; the empty asm statements keep the compiler from moving
      // memory accesses across the barrier.
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();  // everyone's loads of block kb landed; stage ST + 2 is free
      asm volatile("" ::: "memory");
      const char* ks = ST == 0 ? k_s0 : ST == 1 ? k_s1 : ST == 2 ? k_s2 : k_s3;
      const char* vs = ST == 0 ? v_s0 : ST == 1 ? v_s1 : ST == 2 ? v_s2 : v_s3;
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
      // Schedule: four K-operand reads in flight ahead of the MFMAs, then
      // one read per MFMA (measured 2 % faster than the default order, which
      // keeps one or two reads ahead).
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // DS reads
#pragma unroll
      for (int i = 0; i < 2 * KSTEPS - 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      // Stream block kb + 2 into the free stage.  Issued here, after the QK
      // products rather than right after the barrier, so that the eight
      // waves' loads do not all queue at once in front of their first LDS
      // reads (measured 2-3 % faster).
      if constexpr (ST == 0) issue(kb + 2, k_s2, v_s2);
      else if constexpr (ST == 1) issue(kb + 2, k_s3, v_s3);
      else if constexpr (ST == 2) issue(kb + 2, k_s0, v_s0);
      else issue(kb + 2, k_s1, v_s1);
      // lane holds S^T[key = 32t + 8(r/4) + 4g + r%4][query l32]
      if constexpr (kMask) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = j0 + 32 * t + 8 * (r >> 2) + 4 * g + (r & 3);
            if (key >= skv) s[t][r] = -INFINITY;
          }
      }
      // Weights against the running reference m_used, and this block's sums
      // of the unrounded (bs, for LSE) and bf16-rounded (br, for O) weights.
      bf16x8 pb[2][2];
      float bs, br;
      auto weights = [&]() __attribute__((always_inline)) {
        const float mc = m_used * c;
        bs = 0.0f;
        br = 0.0f;
        const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int r = 0; r < 16; r += 2) {
            const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][r], c, -mc));
            const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][r + 1], c, -mc));
            bs += p0;
            bs += p1;
            const bf16x2 pr = {(__bf16)p0, (__bf16)p1};
            pb[t][r >> 3][r & 7] = pr[0];
            pb[t][r >> 3][(r & 7) + 1] = pr[1];
            br = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, br, false);
          }
      };
      weights();
      // The reference only has to keep every weight at most 2^32 (fp32 sums
      // and the O accumulators stay far from overflow; bf16 keeps 8 bits
      // of any magnitude), so no row max is taken in the common case.  A
      // lane sum above 2^32 (or NaN: the first block, with m_used = -inf,
      // gives inf or NaN) raises the reference to the block's row max,
      // rescales what was accumulated and recomputes the weights.
      if (__builtin_expect(__any(!(bs <= kMaxWeight)), 0)) {
        float mx = s[0][0];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[t][r]);
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        // a processed block always holds a valid key, so mx is finite
        const float m_new = fmaxf(m_used, mx);
        const float alpha = m_used == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((m_used - m_new) * c);
        lsum *= alpha;
        lsum_r *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
        m_used = m_new;
        weights();
      }
      lsum += bs;
      lsum_r += br;

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
      // Schedule: eight V-operand reads (four MFMA operands) in flight, then
      // two reads per MFMA (measured 5-6 % faster than the default order,
      // which issues the reads in bursts).
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
      for (int i = 0; i < 4 * DT - 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    };
    if (kb1 <= kb0) {
      // no key of this batch takes part (only with per-batch lengths, which
      // never split tiles): the merge identity O = 0, LSE = -inf, or an
      // accumulator left as it is
      if constexpr (!kMerge) {
        if (q_row < p.Sq) {
          const size_t orow = o_row_offset(p, b, q_row, rs) + (size_t)h * D;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const int d = dt * 32 + 8 * u + 4 * g;
              if constexpr (kOutF32)
                *reinterpret_cast<float4*>(static_cast<float*>(p.o) + orow + d) = make_float4(0.f, 0.f, 0.f, 0.f);
              else
                *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.o) + orow + d) = make_uint2(0u, 0u);
            }
          if (p.lse != nullptr && g == 0) p.lse[((size_t)b * p.H + h) * p.Sq + q_row] = -INFINITY;
        }
      }
      return;
    }
    issue(kb0, k_s0, v_s0);
    issue(kb0 + 1, k_s1, v_s1);
    // Blocks wholly inside the key range need no mask; the partial last
    // block (present when kb1 reaches past skv rounded down) is peeled off.
    // Stage of block x: (x - kb0) mod 4.
    {
      using Full = std::false_type;
      using Part = std::true_type;
      const int kbf = min(kb1, skv / kBN);
      for (int kb = kb0; kb < kbf; kb += 4) {
        block(std::integral_constant<int, 0>{}, kb, Full{});
        if (kb + 1 < kbf) block(std::integral_constant<int, 1>{}, kb + 1, Full{});
        if (kb + 2 < kbf) block(std::integral_constant<int, 2>{}, kb + 2, Full{});
        if (kb + 3 < kbf) block(std::integral_constant<int, 3>{}, kb + 3, Full{});
      }
      if (kbf < kb1) {
        switch ((kbf - kb0) & 3) {
          case 0: block(std::integral_constant<int, 0>{}, kbf, Part{}); break;
          case 1: block(std::integral_constant<int, 1>{}, kbf, Part{}); break;
          case 2: block(std::integral_constant<int, 2>{}, kbf, Part{}); break;
          default: block(std::integral_constant<int, 3>{}, kbf, Part{}); break;
        }
      }
    }
    // the look-ahead loads past kb1 complete before this workgroup's LDS
    // can be handed to another
    wait_vmcnt<0>();

    // ---- normalise and store O and LSE (lane: one query, 16 dims per tile) --
    // Normalise and store O and LSE.  With kMerge, (O, LSE) already hold a
    // partial result over other keys (a previous ring hop) and this chunk is
    // merged into them by the online-softmax rule: with L_c = this chunk's
    // LSE, m = max(L_a, L_c) and w_x = exp(L_x - m),
    //   O = (w_a O_a + w_c O_c) / (w_a + w_c),  LSE = m + ln(w_a + w_c);
    // an accumulator with L_a = -inf holds no keys and is replaced.  The two
    // lanes of a row read the old LSE before the first of them writes it
    // (same wave, program order).
    auto store_out = [&](const f32x16 (&acc)[DT], float m_ref, float l_lane, float lr_lane)
                         __attribute__((always_inline)) {
      typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
      const float ltot = l_lane + __shfl_xor(l_lane, 32);
      const float lrtot = lr_lane + __shfl_xor(lr_lane, 32);
      if (!q_ok) return;
      const size_t orow = o_row_offset(p, b, q_row, rs) + (size_t)h * D;
      const bool pad_head = h >= p.o_heads;
      const size_t lse_idx = ((size_t)b * p.H + h) * p.Sq + q_row;
      const float l_c = m_ref * p.scale + __logf(ltot);
      float cc = 1.0f / lrtot, ca = 0.0f, l_new = l_c;
      if constexpr (kMerge) {
        const float l_a = p.lse[lse_idx];
        if (l_a != -INFINITY) {
          const float m = fmaxf(l_a, l_c);
          const float wa = __expf(l_a - m), wc = __expf(l_c - m);
          const float den = wa + wc;
          ca = wa / den;
          cc = wc / (den * lrtot);
          l_new = m + __logf(den);
        }
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int d = dt * 32 + 8 * u + 4 * g;
          float o[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = acc[dt][4 * u + e] * cc;
          if constexpr (kMerge) {
            if (ca != 0.0f) {
              float prev[4];
              if constexpr (kOutF32) {
                const float4 x = *reinterpret_cast<const float4*>(static_cast<const float*>(p.o) + orow + d);
                prev[0] = x.x; prev[1] = x.y; prev[2] = x.z; prev[3] = x.w;
              } else {
                const bf16x4 x = *reinterpret_cast<const bf16x4*>(static_cast<const uint16_t*>(p.o) + orow + d);
#pragma unroll
                for (int e = 0; e < 4; ++e) prev[e] = (float)x[e];
              }
#pragma unroll
              for (int e = 0; e < 4; ++e) o[e] = __builtin_fmaf(ca, prev[e], o[e]);
            }
          }
          if (pad_head) {
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = 0.0f;
          }
          if constexpr (kOutF32) {
            *reinterpret_cast<float4*>(static_cast<float*>(p.o) + orow + d) = make_float4(o[0], o[1], o[2], o[3]);
          } else {
            bf16x4 w;
            w[0] = (__bf16)o[0]; w[1] = (__bf16)o[1]; w[2] = (__bf16)o[2]; w[3] = (__bf16)o[3];
            *reinterpret_cast<bf16x4*>(static_cast<uint16_t*>(p.o) + orow + d) = w;
          }
        }
      if (p.lse != nullptr && g == 0) p.lse[lse_idx] = l_new;
    };

    if (whole) {
      store_out(oacc, m_used, lsum, lsum_r);
    } else {
      // ---- split tile: publish this piece, the last piece to arrive merges --
      // The tile's pieces are the workgroups first .. first + split - 1 of
      // the split round, in key order; each owns the slot of its index.
      const uint32_t first = j - piece;
      auto slot_of = [&](uint32_t w) __attribute__((always_inline)) {
        return __builtin_amdgcn_make_buffer_rsrc(p.part + (size_t)w * SLOT, (short)0,
                                                 (int)(SLOT * sizeof(float)), kBufferWord3);
      };
      // byte offsets inside a slot: lane-contiguous 16-byte pieces of O^T,
      // then (running max, row-sum share) per lane
      auto o_off = [&](int dt, int u) __attribute__((always_inline)) {
        return (int)((((dt * 4 + u) * kWaves + wave) * 64 + lane) * 16);
      };
      const int ml_off = (int)(ML_OFF * sizeof(float)) + (wave * 64 + lane) * 16;
      {
        const __amdgpu_buffer_rsrc_t sl = slot_of(j);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const f32x4 v4 = {oacc[dt][4 * u], oacc[dt][4 * u + 1], oacc[dt][4 * u + 2], oacc[dt][4 * u + 3]};
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v4), sl, o_off(dt, u), 0, kScopeAgent);
          }
        const u32x4 ml = {__float_as_uint(m_used), __float_as_uint(lsum), __float_as_uint(lsum_r), 0u};
        __builtin_amdgcn_raw_buffer_store_b128(ml, sl, ml_off, 0, kScopeAgent);
      }
      // Slot traffic uses device-scope coherent accesses (they bypass the
      // XCD-private L2 state), so completion of this wave's stores is all the
      // release the counter increment needs; no cache-wide writeback or
      // invalidate that would also evict the other workgroups' K/V lines.
      wait_vmcnt<0>();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      int32_t* counter = p.cnt + (tile - p.n_whole);
      if (tid == 0) s_last = atomicAdd(counter, 1) == (int)p.split - 1;
      __syncthreads();
      if (s_last) {
        // merge all pieces in key order, this one re-read from its slot too,
        // so the result does not depend on which piece arrived last
        float M = -INFINITY;
        for (uint32_t w = first; w < first + p.split; ++w) {
          const u32x4 ml = __builtin_amdgcn_raw_buffer_load_b128(slot_of(w), ml_off, 0, kScopeAgent);
          M = fmaxf(M, __uint_as_float(ml[0]));
        }
        f32x16 acc[DT];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[dt][r] = 0.0f;
        float l = 0.0f, lr = 0.0f;
        for (uint32_t w = first; w < first + p.split; ++w) {
          const __amdgpu_buffer_rsrc_t sl = slot_of(w);
          const u32x4 ml = __builtin_amdgcn_raw_buffer_load_b128(sl, ml_off, 0, kScopeAgent);
          const float alpha = __builtin_amdgcn_exp2f((__uint_as_float(ml[0]) - M) * c);
          l += alpha * __uint_as_float(ml[1]);
          lr += alpha * __uint_as_float(ml[2]);
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const f32x4 v4 = __builtin_bit_cast(
                  f32x4, __builtin_amdgcn_raw_buffer_load_b128(sl, o_off(dt, u), 0, kScopeAgent));
#pragma unroll
              for (int e = 0; e < 4; ++e) acc[dt][4 * u + e] += alpha * v4[e];
            }
        }
        store_out(acc, M, l, lr);
        if (tid == 0) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

// How a call is laid out over the workgroups: one workgroup per tile, in
// rounds of `slots` resident workgroups (CUs x occupancy).  When the last
// round would leave many of them idle, its tiles are instead cut into
// `split` key chunks, one workgroup each, merged by the online-softmax rule;
// that needs `ws_bytes` of workspace: a fixed region of arrival counters
// (kAttnCounterBytes), then one partial-result slot per chunk.
struct Plan {
  uint64_t n_tiles = 0, last = 0, split = 1;
  size_t cnt_bytes = 0, ws_bytes = 0;
};

template <int D, bool kOutF32, bool kMerge>
hipError_t occupancy_of(int dev, int* occ) {
  static std::atomic<int> cached[kMaxDevices];  // per instantiation, zero-initialised
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    const hipError_t e =
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, attn_bf16_kernel<D, kOutF32, kMerge, 0>, kThreads, 0);
    if (e != hipSuccess) return e;
    if (n < 1) n = 1;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  *occ = n;
  return hipSuccess;
}

template <int D, bool kOutF32, bool kMerge>
hipError_t plan_t(const AttnArgs& a, Plan* pl) {
  *pl = Plan();
  const uint64_t n_qtiles = (a.Sq + kBM - 1) / kBM;
  const uint64_t nblocks = (a.Skv + kBN - 1) / kBN;
  pl->n_tiles = n_qtiles * a.H * a.B;
  if (pl->n_tiles == 0 || nblocks == 0 || a.kv_len != nullptr) return hipSuccess;  // masks: whole tiles
  int dev = 0, occ = 0, cus = 0;
  hipError_t e;
  if ((e = current_device(&dev)) != hipSuccess) return e;
  if ((e = occupancy_of<D, kOutF32, kMerge>(dev, &occ)) != hipSuccess) return e;
  if ((e = device_cu_count(&cus)) != hipSuccess) return e;
  const uint64_t slots = (uint64_t)cus * occ;
  pl->last = pl->n_tiles % slots;  // tiles of the last, partial round
  if (pl->last == 0) return hipSuccess;
  const uint64_t split = std::min<uint64_t>({kMaxSplit, slots / pl->last, nblocks});
  if (split < 2) return hipSuccess;
  pl->split = split;
  // The counter region has one fixed size for every call (split tiles are
  // fewer than `slots`), so a workspace reused by calls of different shapes
  // or kernels never finds an earlier call's slot data where its counters
  // must be zero.
  if (pl->last * sizeof(int32_t) > kAttnCounterBytes) return hipErrorInvalidConfiguration;
  pl->cnt_bytes = kAttnCounterBytes;
  pl->ws_bytes = pl->cnt_bytes + pl->last * split * slot_floats<D>() * sizeof(float);
  return hipSuccess;
}

template <int D, bool kOutF32, bool kMerge>
hipError_t launch_t(const AttnArgs& a, hipStream_t stream) {
  Plan pl;
  hipError_t e = plan_t<D, kOutF32, kMerge>(a, &pl);
  if (e != hipSuccess) return e;
  Params p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.o = a.o;
  p.lse = a.lse;
  p.kv_len = a.kv_len;
  p.Sq = a.Sq;
  p.Skv = a.Skv;
  p.H = a.H;
  p.n_qtiles = (a.Sq + kBM - 1) / kBM;
  p.nblocks = (a.Skv + kBN - 1) / kBN;
  p.scale = a.scale;
  p.send_rows = a.send_rows;
  p.send_batches = a.B;
  p.o_heads = a.send_rows > 0 ? a.o_heads : a.H;
  p.in_rows = a.in_rows;
  p.in_last_peer = a.in_peers - 1;
  p.in_div = make_fastdiv(a.in_rows > 0 ? (uint32_t)a.in_rows : 1u);
  p.in_peer = a.in_peer;
  if (pl.n_tiles == 0 || p.nblocks == 0) return hipSuccess;
  // without (enough) workspace every tile is taken whole
  const bool split = pl.split > 1 && a.workspace != nullptr && a.workspace_bytes >= pl.ws_bytes;
  p.n_whole = (uint32_t)(split ? pl.n_tiles - pl.last : pl.n_tiles);
  p.split = split ? (uint32_t)pl.split : 1u;
  p.split_wgs = split ? (uint32_t)(pl.last * pl.split) : 0u;
  p.cnt = split ? static_cast<int32_t*>(a.workspace) : nullptr;
  p.part = split ? reinterpret_cast<float*>(static_cast<char*>(a.workspace) + pl.cnt_bytes) : nullptr;
  const uint64_t grid = (uint64_t)p.n_whole + p.split_wgs;
  if constexpr (!kOutF32 && !kMerge) {
    if (a.in_rows > 0) {  // Q, K, V from the receive buffer (bf16 O only)
      if (a.in_rows % kBN == 0)
        attn_bf16_kernel<D, false, false, 2><<<(unsigned)grid, kThreads, 0, stream>>>(p);
      else
        attn_bf16_kernel<D, false, false, 1><<<(unsigned)grid, kThreads, 0, stream>>>(p);
      return hipGetLastError();
    }
  }
  if (a.in_rows > 0) return hipErrorInvalidValue;
  attn_bf16_kernel<D, kOutF32, kMerge, 0><<<(unsigned)grid, kThreads, 0, stream>>>(p);
  return hipGetLastError();
}

template <int D, bool kOutF32>
hipError_t workspace_t(const AttnArgs& a, size_t* bytes) {
  Plan pl;
  const hipError_t e = a.merge ? plan_t<D, kOutF32, true>(a, &pl) : plan_t<D, kOutF32, false>(a, &pl);
  *bytes = pl.ws_bytes;
  return e;
}

// ---- scratch of the no-allocation entry point ----------------------------------
// A file-scope device array stands in for the caller's workspace: the
// counter region plus 256 partial-result slots at D = 128 (the most a
// 256-CU device's split round uses) fit in kAttnScratchBytes = 36 MiB.  Each
// device that runs the library holds its own copy until the process ends.
// Host code never passes the array's name to a kernel (on the host it is
// only a stand-in): it uses the address hipGetSymbolAddress returns for the
// current device.
__device__ __align__(256) char scratch[kAttnScratchBytes];
static_assert(kAttnScratchBytes >= kAttnCounterBytes + 256 * slot_floats<128>() * sizeof(float),
              "scratch holds a 256-CU device's split round");

__global__ void zero_words(uint32_t* p, uint32_t n) {
  const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

struct ScratchState {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
ScratchState g_scratch[kMaxDevices];

}  // namespace

hipError_t attn_scratch(hipStream_t stream, void** ptr, size_t* bytes) {
  int dev = 0;
  hipError_t e = current_device(&dev);
  if (e != hipSuccess) return e;
  ScratchState& st = g_scratch[dev];
  std::call_once(st.once, [&] {
    void* p = nullptr;
    st.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (st.err != hipSuccess) return;
    // The counters must start at zero (every call leaves them zero): clear
    // the largest counter region a call can use once, on the first caller's
    // stream, with a kernel (not a memset node, so a caller may capture
    // later calls in a graph).
    constexpr uint32_t kWords = kAttnCounterBytes / 4;
    zero_words<<<kWords / 256, 256, 0, stream>>>(static_cast<uint32_t*>(p), kWords);
    st.err = hipGetLastError();
    if (st.err == hipSuccess) st.ptr = p;
  });
  if (st.err != hipSuccess) return st.err;
  *ptr = st.ptr;
  *bytes = kAttnScratchBytes;
  return hipSuccess;
}


hipError_t attn_bf16_workspace_bytes(const AttnArgs& a, size_t* bytes) {
  *bytes = 0;
  if (a.D == 64) return a.o_f32 ? workspace_t<64, true>(a, bytes) : workspace_t<64, false>(a, bytes);
  return a.o_f32 ? workspace_t<128, true>(a, bytes) : workspace_t<128, false>(a, bytes);
}

hipError_t launch_attn_fwd_bf16(const AttnArgs& a, hipStream_t stream) {
  if (a.merge) {
    if (a.D == 64) return a.o_f32 ? launch_t<64, true, true>(a, stream) : launch_t<64, false, true>(a, stream);
    return a.o_f32 ? launch_t<128, true, true>(a, stream) : launch_t<128, false, true>(a, stream);
  }
  if (a.D == 64) return a.o_f32 ? launch_t<64, true, false>(a, stream) : launch_t<64, false, false>(a, stream);
  return a.o_f32 ? launch_t<128, true, false>(a, stream) : launch_t<128, false, false>(a, stream);
}

}  // namespace dit
