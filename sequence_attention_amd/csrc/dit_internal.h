// Internal launch interface between the C-ABI layer (dit_abi.cpp) and the
// gfx950 kernels.  Every launcher assumes its arguments were validated by
// the ABI layer (sizes, alignment, dtype) and only enqueues work on
// `stream`; it returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dit {

// Division by a run-time constant n / d for 0 <= n < 2^31, 1 <= d < 2^31
// (round-up multiplier method, Granlund and Montgomery 1994):
//   s = ceil(log2 d), m = floor(2^32 (2^s - d) / d) + 1,
//   n / d = (mulhi(n, m) + n) >> s.
struct FastDiv {
  uint32_t d, m, s;
};

inline FastDiv make_fastdiv(uint32_t d) {
  FastDiv f;
  f.d = d;
  uint32_t s = 0;
  while ((1ull << s) < d) ++s;
  f.s = s;
  f.m = (uint32_t)((((1ull << s) - d) << 32) / d + 1);
  return f;
}

__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv& f) {
  return (__umulhi(n, f.m) + n) >> f.s;
}

// ---- device resources ---------------------------------------------------------
constexpr int kMaxDevices = 64;

// The current device's index, checked against kMaxDevices.
hipError_t current_device(int* dev);

// Compute units of the current device (queried once per device).
hipError_t device_cu_count(int* cus);

// ---- Ulysses permutes -------------------------------------------------------
enum PermuteKind : int {
  PACK_SEQ_TO_HEAD = 0,
  UNPACK_SEQ_TO_HEAD = 1,
  PACK_HEAD_TO_SEQ = 2,
  UNPACK_HEAD_TO_SEQ = 3,
};

struct PermuteArgs {
  const void* in[3];   // PACK: planes; UNPACK: in[0] = receive buffer
  void* out[3];        // PACK: out[0] = send buffer; UNPACK: planes
  int32_t B, S, H, D, U, n_planes, S_loc, H_loc, rank;
  int32_t elem_bytes;
};

hipError_t launch_permute(PermuteKind kind, const PermuteArgs& a, hipStream_t stream);
// The two pack kinds over float32 planes into a 16-bit send buffer (bf16 or
// f16, round to nearest even); elem_bytes is ignored.
hipError_t launch_pack_convert(PermuteKind kind, const PermuteArgs& a, bool to_bf16,
                               hipStream_t stream);

// Per-peer chunk copies between planes and a buffer of back-to-back chunks
// of per-peer sizes (padding-free Ulysses maps, Ring Anything pad / trim).
// For peer p and every plane pl, batch b, row s < chunk_rows, element e < run:
//   buffer  [chunk_off + ((pl*B + b)*chunk_rows + s)*run + e]
//   plane_pl[(b*plane_b_rows + s)*plane_row + plane_off + e]
// are copied for s < rows (direction set by to_chunk); toward the buffer,
// rows s >= rows are written as zeros.  Sizes and offsets are in elements;
// run, plane_off, plane_row and chunk_off are multiples of D.
constexpr int kMaxPeers = 64;

struct ChunkPeer {
  int64_t rows, chunk_rows, run, plane_off, chunk_off;
};

struct ChunkCopyArgs {
  void* planes[3];
  void* chunk;
  bool to_chunk;
  int32_t n_planes, B, D, elem_bytes, n_peers;
  int64_t plane_b_rows, plane_row;
  ChunkPeer peer[kMaxPeers];
};

hipError_t launch_chunk_copy(const ChunkCopyArgs& a, hipStream_t stream);

// FP8 Ulysses maps (bf16 planes <-> block-scaled E4M3 chunks, K kept bf16).
// planes: PACK inputs / UNPACK outputs (sequence to head: Q, K, V; head to
// sequence: O); buf: the send (PACK) or receive (UNPACK) buffer of U chunks
// of `stride` bytes, the first `used` bytes of each holding the sections.
// D is a multiple of 32, all pointers 16-byte aligned.
struct Fp8PermuteArgs {
  const void* planes[3];
  const void* buf;
  int64_t stride, used;
  int32_t B, S, H, D, U, S_loc, H_loc, rank;
};

hipError_t launch_fp8_permute(PermuteKind kind, const Fp8PermuteArgs& a, hipStream_t stream);

// Sequence-to-head unpack with RoPE on planes 0 and 1 (Q, K); plane 2 copied.
struct RopeUnpackArgs {
  const void* recv;    // [U, n_planes, B, S_loc, H_loc, D]
  void* out[3];        // n_planes x [B, S, H_loc, D]
  const float* cos;    // [S, D/2]
  const float* sin;    // [S, D/2]
  int32_t B, S, D, U, n_planes, S_loc, H_loc;
  int32_t elem_bytes;  // 2 (bf16 / f16) or 4 (f32); D * elem_bytes a multiple of 16
  bool is_f16;
};

hipError_t launch_rope_unpack(const RopeUnpackArgs& a, hipStream_t stream);

// ---- CFG combine ------------------------------------------------------------
hipError_t launch_cfg_combine_f32(const float* u, const float* c, float* out, int64_t n, float g,
                                  hipStream_t stream);
hipError_t launch_cfg_combine_bf16(const uint16_t* u, const uint16_t* c, uint16_t* out, int64_t n,
                                   float g, hipStream_t stream);

// ---- merge -------------------------------------------------------------------
hipError_t launch_attn_merge(void* o_acc, float* lse_acc, const void* o_part, const float* lse_part,
                             int32_t B, int32_t Sq, int32_t H, int32_t D, bool o_f32,
                             hipStream_t stream);

// ---- attention ---------------------------------------------------------------
struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;  // may be null
  int32_t B, Sq, Skv, H, D;
  float scale;
  bool o_f32;  // bf16 input only: write O as fp32
  bool merge = false;  // o / lse hold a partial result to merge this call into
  const int32_t* kv_len = nullptr;  // [B] valid keys per batch (device), or null
  // Caller-owned device memory for the split last round of the bf16 path
  // (arrival counters, all zero on entry and left zero, then partial-result
  // slots), or null: tiles are then never split.
  void* workspace = nullptr;
  size_t workspace_bytes = 0;
  // bf16 path only: send_rows > 0 stores O in the head-to-sequence send
  // buffer [U, 1, B, send_rows, H, D] (query row t -> peer t / send_rows,
  // row t % send_rows), heads at or past o_heads as zeros.
  int32_t send_rows = 0;
  int32_t o_heads = 0;
  // bf16 path, bf16 O only: in_rows > 0 reads Q, K and V from the
  // sequence-to-head receive buffer [in_peers, 3, B, in_rows, H, D] (q, k,
  // v at planes 0, 1, 2 of the first peer's chunk, in_peer elements between
  // peers); in_rows >= 64.
  int32_t in_rows = 0;
  int32_t in_peers = 0;
  int64_t in_peer = 0;
};

// Zero rows [t0, t1) (t1 <= U * S_loc) of every batch of a bf16 send buffer
// [U, 1, B, S_loc, row_elems] (row t -> peer t / S_loc, row t % S_loc);
// row_elems * 2 bytes must be a multiple of 16.
hipError_t launch_send_rows_zero(void* send, int32_t B, int32_t S_loc, int32_t t0, int32_t t1,
                                 int64_t row_elems, hipStream_t stream);
// Write `value` into n 32-bit words.
hipError_t launch_fill_words(void* p, uint64_t n, uint32_t value, hipStream_t stream);

// Bytes of workspace the bf16 path uses for this call on the current device
// (0: no tile is split).  Host-only queries of the device.
hipError_t attn_bf16_workspace_bytes(const AttnArgs& a, size_t* bytes);
// Workspace layout of the split last round: a fixed region of arrival
// counters (room for 16384 split tiles; one size for every call, so calls of
// different shapes may share a workspace), then partial-result slots.
constexpr size_t kAttnCounterBytes = size_t(64) << 10;
// Size of the static scratch of the no-allocation entry point.
constexpr size_t kAttnScratchBytes = size_t(36) << 20;
// The current device's static scratch (address and size) for callers that
// cannot allocate; its counter region is zeroed on the first call per device
// (on `stream`).  Every call on a device shares it.
hipError_t attn_scratch(hipStream_t stream, void** ptr, size_t* bytes);
hipError_t launch_attn_fwd_bf16(const AttnArgs& a, hipStream_t stream);
hipError_t launch_attn_fwd_f32(const AttnArgs& a, hipStream_t stream);
// Skv == 0: O = 0, LSE = -inf.
hipError_t launch_attn_empty(const AttnArgs& a, bool in_f32, hipStream_t stream);

// ---- measurement aid ------------------------------------------------------------
// out: [workgroups][2] int64 (shader cycles, 100 MHz real-time ticks).
hipError_t launch_clock_probe(int64_t* out, int32_t workgroups, int32_t spin, bool mfma,
                              hipStream_t stream);

}  // namespace dit
