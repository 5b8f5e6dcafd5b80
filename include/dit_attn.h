/*
 * dit_attn.h -- C ABI of the per-GPU hot path of sequence-parallel DiT
 * attention on AMD Instinct MI355X (gfx950).
 *
 * One rank's share of a Ulysses x ring split is computed by these kinds of
 * call:
 *   dit_ulysses_pack / dit_ulysses_unpack  layout transforms around the
 *                                          Ulysses all-to-alls
 *   dit_ulysses_pack_convert               the pack from float32 planes into a
 *                                          bf16 / f16 send buffer
 *   dit_ulysses_unpack_rope                the receive-side unpack fused with
 *                                          RoPE on Q and K
 *   dit_ulysses_pack_uneven / _unpack_uneven  the same transforms for
 *                                          per-rank sequence and head counts
 *                                          (no padding)
 *   dit_ring_anything_pad / _trim          equal-size K/V gather of uneven
 *                                          sequence shards
 *   dit_ulysses_pack_fp8 / _unpack_fp8     the Ulysses maps with Q, V and O
 *                                          exchanged as FP8 (K kept bf16)
 *   dit_attn_fwd_send                      attention that stores O straight into
 *                                          the head-to-sequence send buffer
 *   dit_attn_fwd_a2a                       ... that also reads Q, K and V
 *                                          straight from the sequence-to-head
 *                                          receive buffer
 *   dit_attn_fwd, dit_attn_fwd_ws          attention with per-row LSE (_ws:
 *                                          with a caller workspace that lets
 *                                          the kernel split the last round)
 *   dit_attn_workspace_size                that workspace's size
 *   dit_attn_fwd_noalloc                   ... with a static scratch instead
 *                                          (callers that cannot allocate)
 *   dit_attn_fwd_kvlen                     ... over a per-batch key prefix
 *   dit_attn_merge                         online-softmax merge of partial
 *                                          results (ring hops)
 *   dit_attn_fwd_merge                     one ring hop: attention of a K/V
 *                                          chunk merged into the accumulator
 *   dit_cfg_combine                        classifier-free guidance combine
 *
 * Shapes follow SGLang Diffusion "Parallelism Overview" ("What happens to
 * the shapes"): sequence-sharded [B, S/(U*R), H/T, D] outside attention,
 * head-sharded [B, S/R, H/(T*U), D] inside it.  In this header S denotes the
 * sequence of one Ulysses group (S/R globally) and H the heads entering the
 * Ulysses split (H/T globally).
 *
 * Conventions shared by every entry point:
 *   - Tensor pointers are DEVICE pointers to contiguous row-major tensors,
 *     owned by the caller; the library never allocates, frees or retains
 *     device memory (a workspace, where an entry point takes one, is the
 *     caller's too).  Thread-safe; the only state kept between calls is
 *     the per-thread error text and per-device facts (compute-unit count,
 *     kernel occupancy) queried once per device.
 *   - Every call is asynchronous on `stream` (a hipStream_t passed as void*,
 *     NULL = the default stream) and never synchronizes.
 *   - All validation happens before any launch; on an error nothing is
 *     written and the call returns a non-zero status whose detail
 *     dit_last_error() gives.  DIT_ERR_UNSUPPORTED means "valid request that
 *     this library does not serve": the caller should fall back to generic
 *     operators (edge-dit.cpp "Parallel execution": unsupported shapes or
 *     dtypes take the generic operator path).
 *   - Tensor pointers of attention, merge and CFG calls must be 16-byte
 *     aligned (LSE: 4-byte); permute pointers need only element alignment
 *     (DIT_ERR_UNSUPPORTED otherwise).
 */
#ifndef DIT_ATTN_H
#define DIT_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DIT_ABI_VERSION 2

typedef enum {
  DIT_OK = 0,
  DIT_ERR_INVALID_ARGUMENT = 1, /* null pointer, negative size, bad enum, rank out of range */
  DIT_ERR_UNSUPPORTED = 2,      /* valid but not served: head dim, dtype, alignment */
  DIT_ERR_HIP = 3               /* a kernel launch failed */
} dit_status_t;

typedef enum { DIT_BF16 = 0, DIT_F16 = 1, DIT_F32 = 2 } dit_dtype_t;

typedef enum {
  DIT_SEQ_TO_HEAD = 0, /* sequence-sharded -> head-sharded (before attention) */
  DIT_HEAD_TO_SEQ = 1  /* head-sharded -> sequence-sharded (after attention) */
} dit_a2a_dir_t;

/*
 * Layout of one Ulysses redistribution.  Mirrors the sequence-split and
 * all-to-all layout state of edge-dit.cpp "Parallel execution" (original /
 * padded / local sequence length; global / local heads; batch; head dim;
 * elements per peer).  Fill it with dit_a2a_layout_init(); the derived
 * fields are read-only for callers.
 *
 * Padding (explicit here, never hidden global state):
 *   S_pad = ceil(S / lcm(U, seq_align)) * lcm(U, seq_align), S_loc = S_pad/U.
 *     seq_align = 1 pads to a multiple of U (edge-dit: S divisible by the
 *     SP degree or padded); seq_align = 64 gives xLLM's lcm(SP, 64) rule
 *     ("DiT Architecture and Capability Matrix", MiniMax-H3 boundaries).
 *     Pad rows are the global tail (rows >= S, on the last ranks).
 *   H_pad = ceil(H / U) * U, H_loc = H_pad / U (cache-dit "Context
 *     Parallelism", Any Head Num).  Pad heads are global indices >= H.
 * Pad rows and pad heads are always written as zeros; they are never read.
 */
typedef struct {
  int32_t B, S, H, D, U;  /* real sizes of the Ulysses group */
  int32_t seq_align;      /* >= 1 */
  int32_t n_planes;       /* 1 (one tensor) or 3 (packed Q, K, V) */
  dit_dtype_t dtype;      /* element type; permutes are bit copies */
  int32_t S_pad, S_loc, H_pad, H_loc; /* derived */
  int64_t elems_per_peer;             /* derived: n_planes*B*S_loc*H_loc*D */
} dit_a2a_layout;

/* DIT_ABI_VERSION of the loaded library. */
int dit_abi_version(void);

/* Static text for a status code (never NULL). */
const char* dit_status_string(dit_status_t status);

/* Detail of the calling thread's last failed call ("" if none).  The
 * pointer stays valid until the thread's next library call. */
const char* dit_last_error(void);

/*
 * Fill *out from the real sizes.  B, S, H, D >= 0 (S or B may be 0: an empty
 * exchange); U >= 1; seq_align >= 1; n_planes in {1, 3}; dtype any of the
 * enum.  Errors: DIT_ERR_INVALID_ARGUMENT (out NULL, a negative size, bad
 * U / seq_align / n_planes / dtype, or sizes whose element count overflows
 * int64).  Host-only; touches no device.
 */
dit_status_t dit_a2a_layout_init(int32_t B, int32_t S, int32_t H, int32_t D, int32_t U,
                                 int32_t seq_align, int32_t n_planes, dit_dtype_t dtype,
                                 dit_a2a_layout* out);

/*
 * Pack the send buffer of Ulysses rank `rank` (edge-dit.cpp "Parallel
 * execution": packed QKV operator for sequence-to-head, packed
 * head-to-sequence operator for the inverse; SGLang "The Ulysses
 * transport": one destination-major buffer for all planes).
 *
 * send_buf: [U (destination peer), n_planes, B, S_loc, H_loc, D]; the
 *   chunk for peer p starts at element p * elems_per_peer.
 * DIT_SEQ_TO_HEAD: in_planes[pl] is the rank's sequence shard
 *   [B, S_loc, H, D];
 *   send[p,pl,b,s,h',d] = in_pl[b, s, p*H_loc + h', d]
 *   if rank*S_loc + s < S and p*H_loc + h' < H, else 0.
 *   Rows of in_pl whose global index is >= S are never read.
 * DIT_HEAD_TO_SEQ: in_planes[pl] is the rank's head shard [B, S, H_loc, D];
 *   send[p,pl,b,s,h',d] = in_pl[b, p*S_loc + s, h', d]
 *   if p*S_loc + s < S and rank*H_loc + h' < H, else 0.
 *   Heads of in_pl whose global index is >= H are never read.
 *
 * in_planes is a HOST array of n_planes device pointers.  No aliasing
 * between inputs and send_buf.  Errors: INVALID_ARGUMENT (null layout,
 * in_planes or pointer of a non-empty tensor, bad direction, rank outside
 * [0, U), layout fields inconsistent with dit_a2a_layout_init, overlapping
 * tensors); UNSUPPORTED (pointer not element-aligned, exchange of 2^31 or
 * more elements); HIP.
 */
dit_status_t dit_ulysses_pack(const dit_a2a_layout* layout, dit_a2a_dir_t dir, int32_t rank,
                              const void* const* in_planes, void* send_buf, void* stream);

/*
 * dit_ulysses_pack with float32 planes and a 16-bit send buffer: every
 * element is rounded to layout->dtype (DIT_BF16 or DIT_F16) on its way into
 * the buffer (edge-dit.cpp "Parallel execution": the packed QKV operator's
 * optional F32-to-F16 conversion; F16 / BF16 output produced directly on the
 * head-to-sequence path).  The maps, pads and buffer layout are those of
 * dit_ulysses_pack for the same layout and direction; only the element type
 * of in_planes differs (float32, 4-byte aligned).
 *
 * Rounding: IEEE 754 round to nearest, ties to even; magnitudes at or past
 * the overflow midpoint become infinity; subnormal results are kept; NaN
 * becomes a quiet NaN (sign and payload unspecified).  Pad elements are +0.
 *
 * Errors: as dit_ulysses_pack, plus UNSUPPORTED when layout->dtype is not
 * DIT_BF16 or DIT_F16.  Uses no memory beyond its arguments.
 */
dit_status_t dit_ulysses_pack_convert(const dit_a2a_layout* layout, dit_a2a_dir_t dir,
                                      int32_t rank, const void* const* in_planes, void* send_buf,
                                      void* stream);

/*
 * Unpack the receive buffer of Ulysses rank `rank` after the all-to-all
 * (edge-dit.cpp receive preparation without RoPE; receive-side unpack of the
 * head-to-sequence path).  recv_buf: [U (source peer), n_planes, B, S_loc,
 * H_loc, D]: the chunk that source peer p addressed to this rank.
 *
 * DIT_SEQ_TO_HEAD: out_planes[pl] is [B, S, H_loc, D] (the S real rows:
 *   pad rows are dropped, so attention sees exactly the real keys);
 *   out_pl[b,t,h',d] = recv[t / S_loc, pl, b, t % S_loc, h', d].
 *   Pad heads of this rank arrive as zeros and stay zero.
 * DIT_HEAD_TO_SEQ: out_planes[pl] is [B, S_loc, H, D] (the H real heads);
 *   out_pl[b,s,h,d] = recv[h / H_loc, pl, b, s, h % H_loc, d] for
 *   rank*S_loc + s < S, and 0 on this rank's pad rows.
 *
 * out_planes is a HOST array of n_planes device pointers.  Errors as for
 * dit_ulysses_pack.
 */
dit_status_t dit_ulysses_unpack(const dit_a2a_layout* layout, dit_a2a_dir_t dir, int32_t rank,
                                const void* recv_buf, void* const* out_planes, void* stream);

/*
 * Fused receive preparation: the sequence-to-head unpack of the packed
 * Q, K, V receive buffer with rotary position embedding applied to Q and K
 * in the same pass (edge-dit.cpp "Parallel execution", Ulysses section:
 * receive-buffer decoding, plane extraction, head-sharded layout and RoPE
 * on Q and K in one operator).
 *
 * layout: as dit_ulysses_unpack with n_planes = 3 (planes Q, K, V).
 * recv_buf: [U (source peer), 3, B, S_loc, H_loc, D]; out_planes: host
 *   array of 3 device pointers, each [B, S, H_loc, D] (pad rows dropped).
 * rope_cos, rope_sin: [S, D/2] fp32 tables indexed by the global sequence
 *   position t and the pair index i; pair i of each Q and K head vector is
 *   rotated (RoFormer convention, adjacent dims):
 *     y[2i]   = x[2i] cos[t][i] - x[2i+1] sin[t][i]
 *     y[2i+1] = x[2i] sin[t][i] + x[2i+1] cos[t][i]
 *   evaluated in fp32 and rounded to the layout dtype (nearest even).  Any
 *   angle schedule (one axis, or per-axis schedules of image and video
 *   tokens) is expressed by the tables.  V is copied bit for bit; with
 *   cos = 1 and sin = 0 the call equals dit_ulysses_unpack bit for bit.
 * dtype: bf16, f16 or f32 with D * element size a multiple of 16 bytes;
 *   all pointers 16-byte aligned.  Outputs must not overlap the inputs.
 * Errors: INVALID_ARGUMENT (layout, rank, n_planes != 3, NULL pointers,
 * overlap); UNSUPPORTED (head size, alignment, size limits); HIP.
 */
dit_status_t dit_ulysses_unpack_rope(const dit_a2a_layout* layout, int32_t rank, const void* recv_buf,
                                     void* const* out_planes, const float* rope_cos,
                                     const float* rope_sin, void* stream);

/*
 * FP8 exchange (cache-dit "Context Parallelism", Async FP8 Ulysses
 * Attention: Q, V and O cross the all-to-alls as FP8, K stays 16-bit because
 * the softmax of Q K^T is sensitive to its precision).  The pages give no
 * format or scaling; this library's encoding is:
 *   - OCP E4M3 ("FN": bias 7, largest finite 448, no infinities);
 *   - one power-of-two scale per block of 32 consecutive elements of a head
 *     vector (the OCP Microscaling block size, E8M0 scale byte): k is the
 *     smallest integer with max|x| <= 448 * 2^k over the block, clamped to
 *     [-117, 126]; scale byte = k + 127;
 *   - code = round-to-nearest-even E4M3 of x * 2^-k (sign kept, also of
 *     zero); decoding gives value(code) * 2^k, which bf16 holds exactly.
 *   Per element |decoded - x| <= max(2^-4 |x|, 2^(k-10)).
 * The maps around the codes are those of dit_ulysses_pack / _unpack for the
 * same layout (pad rows and heads encode as zeros; pad rows are dropped at
 * the sequence-to-head unpack; pad heads are dropped and this rank's pad
 * rows zeroed at the head-to-sequence unpack).
 *
 * Layout requirements: dtype bf16, D a multiple of 32; DIT_SEQ_TO_HEAD takes
 * n_planes = 3 (planes Q, K, V, in that order), DIT_HEAD_TO_SEQ n_planes = 1
 * (plane O).  Plane pointers and the buffer are 16-byte aligned.
 *
 * Buffers hold U chunks of dit_a2a_fp8_bytes_per_peer() bytes (chunk p for
 * / from peer p).  With E = B * S_loc * H_loc * D, a chunk is, in bytes:
 *   DIT_SEQ_TO_HEAD: Q codes [0, E), V codes [E, 2E), K bf16 [2E, 4E),
 *                    Q scale bytes [4E, 4E + E/32), V scale bytes
 *                    [4E + E/32, 4E + E/16);
 *   DIT_HEAD_TO_SEQ: O codes [0, E), O scale bytes [E, E + E/32);
 * codes and K in the element order [B, S_loc, H_loc, D] of the 16-bit
 * chunk, scale byte i covering elements [32 i, 32 i + 32); zero bytes pad
 * the chunk to a multiple of 256.  Sequence to head moves 4E + E/16 bytes
 * per peer instead of 6E; head to sequence E + E/32 instead of 2E.
 *
 * Errors: INVALID_ARGUMENT (as dit_ulysses_pack, plus a wrong n_planes for
 * the direction); UNSUPPORTED (dtype, D, alignment, size limits); HIP.
 */
dit_status_t dit_a2a_fp8_bytes_per_peer(const dit_a2a_layout* layout, dit_a2a_dir_t dir,
                                        int64_t* bytes);
dit_status_t dit_ulysses_pack_fp8(const dit_a2a_layout* layout, dit_a2a_dir_t dir, int32_t rank,
                                  const void* const* in_planes, void* send_buf, void* stream);
dit_status_t dit_ulysses_unpack_fp8(const dit_a2a_layout* layout, dit_a2a_dir_t dir, int32_t rank,
                                    const void* recv_buf, void* const* out_planes, void* stream);

/* Largest Ulysses (or ring) degree of the per-rank count layouts. */
#define DIT_MAX_RANKS 64

/*
 * Layout of a padding-free Ulysses redistribution (cache-dit "Context
 * Parallelism": Ulysses Anything Attention, any sequence length with zero
 * padding after a scalar gather of every rank's length; the no-pad variant
 * of Any Head Num).  Rank r holds the contiguous sequence rows
 * [seq_offsets[r], seq_offsets[r] + seq_counts[r]) outside attention and the
 * contiguous heads [head_offsets[r], head_offsets[r] + head_counts[r])
 * inside it.  A count may be 0 (that rank then holds no rows / no heads).
 * Unlike the padded layout nothing is zero-filled and nothing is dropped:
 * every exchanged element is real.  Fill it with dit_a2a_uneven_init(); the
 * derived fields (offsets, S_max) are read-only for callers.
 *
 * Exchange buffers are back-to-back chunks, one per peer in peer order (the
 * split sizes of an all-to-all-v); each chunk is [n_planes, B, rows, heads,
 * D].  dit_a2a_uneven_sizes() gives the element counts.
 */
typedef struct {
  int32_t B, S, H, D, U;  /* S = sum of seq_counts, H = sum of head_counts */
  int32_t n_planes;       /* 1 to 3 (3: packed Q, K, V; 2: K, V) */
  dit_dtype_t dtype;
  int32_t S_max;          /* derived: largest seq count */
  int32_t seq_counts[DIT_MAX_RANKS];
  int32_t head_counts[DIT_MAX_RANKS];
  int32_t seq_offsets[DIT_MAX_RANKS + 1];  /* derived prefix sums */
  int32_t head_offsets[DIT_MAX_RANKS + 1]; /* derived prefix sums */
} dit_a2a_uneven_layout;

/*
 * Fill *out.  seq_counts / head_counts: HOST arrays of U non-negative counts
 * summing to S / H, or NULL for the balanced split (count_r = floor(S/U),
 * plus one on the first S mod U ranks; likewise for H).  B, S, H, D >= 0;
 * 1 <= U <= DIT_MAX_RANKS; 1 <= n_planes <= 3.  Errors:
 * DIT_ERR_INVALID_ARGUMENT (out NULL, negative size or count, counts not
 * summing to S / H, bad U / n_planes / dtype, element counts overflowing
 * int64).  Host-only.
 */
dit_status_t dit_a2a_uneven_init(int32_t B, int32_t S, int32_t H, int32_t D, int32_t U,
                                 int32_t n_planes, dit_dtype_t dtype, const int32_t* seq_counts,
                                 const int32_t* head_counts, dit_a2a_uneven_layout* out);

/*
 * Per-peer element counts of rank `rank`'s exchange in direction `dir`:
 * send_counts[p] (chunk this rank sends to p) and recv_counts[p] (chunk it
 * receives from p), HOST arrays of U entries (either may be NULL); chunk p
 * of a buffer starts at the sum of the counts before it.
 *   DIT_SEQ_TO_HEAD: send n*B*S_rank*H_p*D, receive n*B*S_p*H_rank*D.
 *   DIT_HEAD_TO_SEQ: send n*B*S_p*H_rank*D, receive n*B*S_rank*H_p*D.
 * Errors: INVALID_ARGUMENT (layout inconsistent with dit_a2a_uneven_init,
 * bad direction or rank).  Host-only.
 */
dit_status_t dit_a2a_uneven_sizes(const dit_a2a_uneven_layout* layout, dit_a2a_dir_t dir,
                                  int32_t rank, int64_t* send_counts, int64_t* recv_counts);

/*
 * Pack rank `rank`'s send buffer for a padding-free exchange.  With
 * so / ho the seq / head offsets:
 * DIT_SEQ_TO_HEAD: in_planes[pl] is the rank's shard [B, S_rank, H, D];
 *   chunk p is [n, B, S_rank, H_p, D] = in_pl[:, :, ho[p] : ho[p] + H_p].
 * DIT_HEAD_TO_SEQ: in_planes[pl] is the rank's head shard [B, S, H_rank, D];
 *   chunk p is [n, B, S_p, H_rank, D] = in_pl[:, so[p] : so[p] + S_p].
 * A bit copy; in_planes is a HOST array of n_planes device pointers; no
 * aliasing between inputs and send_buf.  Errors: INVALID_ARGUMENT (layout,
 * direction, rank, NULL pointer of a non-empty tensor, overlap);
 * UNSUPPORTED (pointer not element-aligned, 2^31 or more elements on either
 * side, B * n_planes above 65535); HIP.
 */
dit_status_t dit_ulysses_pack_uneven(const dit_a2a_uneven_layout* layout, dit_a2a_dir_t dir,
                                     int32_t rank, const void* const* in_planes, void* send_buf,
                                     void* stream);

/*
 * Unpack rank `rank`'s receive buffer (chunk p came from peer p):
 * DIT_SEQ_TO_HEAD: out_planes[pl] is [B, S, H_rank, D]; rows
 *   [so[p], so[p] + S_p) come from chunk p ([n, B, S_p, H_rank, D]).
 * DIT_HEAD_TO_SEQ: out_planes[pl] is [B, S_rank, H, D]; heads
 *   [ho[p], ho[p] + H_p) come from chunk p ([n, B, S_rank, H_p, D]).
 * Every output element is written.  Errors as dit_ulysses_pack_uneven.
 */
dit_status_t dit_ulysses_unpack_uneven(const dit_a2a_uneven_layout* layout, dit_a2a_dir_t dir,
                                       int32_t rank, const void* recv_buf, void* const* out_planes,
                                       void* stream);

/*
 * Ring Anything (diffusers "Distributed inference", Ring Anything
 * Attention): an all-gather needs equal sizes, so each ring rank pads its
 * K/V shard to the longest rank's length, the padded shards are gathered,
 * and the gathered buffer is cut back to the real lengths before attention.
 * The layout's seq_counts are the ring ranks' lengths (head_counts unused:
 * every rank keeps all H heads).
 *
 * dit_ring_anything_pad: in_planes[pl] is rank `rank`'s shard
 *   [B, S_rank, H, D]; send_buf is [n, B, S_max, H, D] with rows >= S_rank
 *   set to zero.
 * dit_ring_anything_trim: gathered is [U, n, B, S_max, H, D] (rank-major);
 *   out_planes[pl] is [B, S, H, D] with rows [so[p], so[p] + S_p) taken from
 *   rank p's first S_p rows.  Pad rows are never read.
 * Errors as dit_ulysses_pack_uneven.
 */
dit_status_t dit_ring_anything_pad(const dit_a2a_uneven_layout* layout, int32_t rank,
                                   const void* const* in_planes, void* send_buf, void* stream);
dit_status_t dit_ring_anything_trim(const dit_a2a_uneven_layout* layout, const void* gathered,
                                    void* const* out_planes, void* stream);

/*
 * Non-causal attention with per-row log-sum-exp (edge-dit.cpp "Parallel
 * execution", Ulysses section: exact softmax(Q K^T / sqrt(D)) V over the
 * full sequence of the rank's heads; SGLang "Parallelism Overview",
 * Constraints: a ring-capable kernel must expose its softmax LSE).
 *
 *   s_ij   = scale * q_i . k_j
 *   O_i    = sum_j softmax_j(s_i) v_j
 *   LSE_i  = ln sum_j exp(s_ij)          (natural log, scale included)
 *
 * q: [B, Sq, H, D], k and v: [B, Skv, H, D] in in_dtype (DIT_BF16: bf16
 *   MFMA with fp32 accumulation and fp32 softmax; DIT_F32: fp32 throughout).
 * o: [B, Sq, H, D] in o_dtype (= in_dtype, or DIT_F32 for a bf16 input whose
 *   output feeds an fp32 ring accumulator).
 * lse: [B, H, Sq] fp32, or NULL when not needed.
 * scale > 0 and finite (1/sqrt(D) for standard attention).
 * D in {64, 128}.
 * Sq == 0 or B == 0 or H == 0: no-op.  Skv == 0: O = 0 and LSE = -inf (the
 *   identity of dit_attn_merge).
 * No aliasing between inputs and outputs.  Deterministic: a repeated call
 *   on the same device returns bitwise identical O and LSE.
 * Uses no memory beyond its arguments: every query tile is taken whole
 *   (dit_attn_fwd_ws may be faster on shapes whose tiles do not fill the
 *   last round of the device).
 * Errors: INVALID_ARGUMENT (null pointer of a non-empty tensor, negative
 * size, bad scale or dtype); UNSUPPORTED (D, dtype pair, alignment); HIP.
 */
dit_status_t dit_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                          int32_t B, int32_t Sq, int32_t Skv, int32_t H, int32_t D, float scale,
                          dit_dtype_t in_dtype, dit_dtype_t o_dtype, void* stream);

/*
 * Bytes of workspace that dit_attn_fwd_ws (merge = 0) or dit_attn_fwd_merge
 * (merge = 1) use for a call of these sizes on the CURRENT device (the
 * device's compute-unit count decides how the work is cut).  0 means the
 * call never splits a tile (fp32 path, empty calls, shapes that fill the
 * device's rounds exactly).  Arguments as dit_attn_fwd.  For a bf16 call on a
 * 256-CU device the size is at most 65536 + 256 x 139264 bytes (about
 * 35.7 MB at D = 128).  Layout: 65536 bytes of arrival counters (the same
 * for every call), then the partial-result slots.  Host-only apart from device attribute queries.
 * Errors: INVALID_ARGUMENT (bytes NULL, negative size, bad dtype or merge),
 * UNSUPPORTED (as dit_attn_fwd), HIP (no device).
 */
dit_status_t dit_attn_workspace_size(int32_t B, int32_t Sq, int32_t Skv, int32_t H, int32_t D,
                                     dit_dtype_t in_dtype, dit_dtype_t o_dtype, int32_t merge,
                                     int64_t* bytes);

/*
 * dit_attn_fwd with a caller-owned workspace.  When the query tiles do not
 * fill the device's last round of resident workgroups, the bf16 path cuts
 * that round's tiles into key chunks, one workgroup each; every chunk writes
 * its unnormalised partial result to a workspace slot and the last chunk of
 * a tile to arrive merges them (online-softmax rule, fixed key order, so
 * the result stays deterministic).  Same results as dit_attn_fwd within the
 * attention tolerance (not bitwise: the split changes the summation order).
 *
 * workspace: device memory of workspace_bytes bytes, 256-byte aligned,
 *   whose first 65536 bytes (the arrival counters) are ZERO the first time
 *   it is used (e.g. zero-filled once after allocation); every call leaves
 *   them zero again, so one workspace serves calls of any shape.  NULL with workspace_bytes = 0: no split (= dit_attn_fwd).
 *   workspace_bytes must be at least dit_attn_workspace_size() for the call.
 *   Calls that may run at the same time (different streams) need different
 *   workspaces; calls on one stream may share one.
 * Errors: as dit_attn_fwd; INVALID_ARGUMENT also for a workspace smaller
 * than needed, NULL with a nonzero size, or overlapping a tensor;
 * UNSUPPORTED for a misaligned workspace.
 */
dit_status_t dit_attn_fwd_ws(const void* q, const void* k, const void* v, void* o, float* lse,
                             int32_t B, int32_t Sq, int32_t Skv, int32_t H, int32_t D, float scale,
                             dit_dtype_t in_dtype, dit_dtype_t o_dtype, void* workspace,
                             int64_t workspace_bytes, void* stream);

/*
 * Attention of Ulysses rank `rank` with O stored straight into the
 * head-to-sequence send buffer (edge-dit.cpp "Parallel execution": the
 * packed head-to-sequence operator partitions the attention output by
 * destination sequence shard into a peer-major send buffer; here attention
 * writes that buffer itself, so the separate pack and its read and write of
 * O disappear).  The result equals, bit for bit,
 *   dit_attn_fwd_ws(q, k, v, o, lse, B, S, Skv, H_loc, D, scale, BF16, BF16,
 *                   workspace, workspace_bytes)
 *   followed by dit_ulysses_pack(layout, DIT_HEAD_TO_SEQ, rank, {o}, send_buf):
 *   send[p,0,b,s,h',d] = O[b, p*S_loc + s, h', d] for p*S_loc + s < S and
 *   rank*H_loc + h' < H, else 0 (pad rows and pad heads are written as 0).
 *
 * layout: from dit_a2a_layout_init with n_planes = 1 and dtype DIT_BF16;
 *   B, S, H_loc and D of the call come from it.
 * q: [B, S, H_loc, D] bf16 (the head-sharded queries of this rank);
 * k, v: [B, Skv, H_loc, D] bf16; lse: [B, H_loc, S] fp32 or NULL;
 * send_buf: [U, 1, B, S_loc, H_loc, D] bf16, every element written.
 * workspace, workspace_bytes: as dit_attn_fwd_ws (sized by
 *   dit_attn_workspace_size(B, S, Skv, H_loc, D, BF16, BF16, 0, ...)).
 * Skv = 0 writes a zero buffer and LSE = -inf.  Uses no memory beyond its
 * arguments.
 * Errors: INVALID_ARGUMENT (as dit_ulysses_pack for the layout and rank,
 *   n_planes != 1, and as dit_attn_fwd_ws for the tensors, with the whole
 *   send buffer as the output); UNSUPPORTED (layout dtype not bf16, and as
 *   dit_attn_fwd); HIP.
 */
dit_status_t dit_attn_fwd_send(const void* q, const void* k, const void* v, void* send_buf,
                               float* lse, const dit_a2a_layout* layout, int32_t rank, int32_t Skv,
                               float scale, void* workspace, int64_t workspace_bytes, void* stream);

/*
 * Attention of Ulysses rank `rank` between the two all-to-alls: Q, K and V
 * are read straight from the packed sequence-to-head receive buffer and O
 * is stored straight into the head-to-sequence send buffer (edge-dit.cpp
 * "Parallel execution", Ulysses section: receive-buffer decoding and plane
 * extraction into the head-sharded layout before attention, and the packed
 * head-to-sequence operator after it; here the attention kernel addresses
 * both buffers itself, so neither the unpack nor the pack moves Q, K, V or
 * O through HBM).  The result equals, bit for bit,
 *   dit_ulysses_unpack(layout, DIT_SEQ_TO_HEAD, rank, recv_buf, {q, k, v})
 *   followed by dit_attn_fwd_send(q, k, v, send_buf, lse, layout1, rank, S,
 *   scale, workspace, workspace_bytes), with layout1 the same group with
 *   n_planes = 1.
 * Query and key row t of the sequence (t < S) are row t % S_loc of source
 * peer t / S_loc's chunk of the receive buffer: Q, K, V[b, t, h', :] =
 * recv[t / S_loc, plane 0 / 1 / 2, b, t % S_loc, h', :].  Pad rows (t >= S)
 * are not attended to.
 *
 * layout: from dit_a2a_layout_init with n_planes = 3 and dtype DIT_BF16,
 *   S_loc >= 64; B, S, H_loc and D of the call come from it.
 * recv_buf: [U, 3, B, S_loc, H_loc, D] bf16 as received (16-byte aligned);
 * send_buf: [U, 1, B, S_loc, H_loc, D] bf16, every element written
 *   (pad rows and pad heads as 0); lse: [B, H_loc, S] fp32 or NULL.
 * workspace, workspace_bytes: as dit_attn_fwd_ws (sized by
 *   dit_attn_workspace_size(B, S, S, H_loc, D, BF16, BF16, 0, ...)).
 * Uses no memory beyond its arguments.
 * Errors: INVALID_ARGUMENT (as dit_ulysses_unpack for the layout and rank,
 *   n_planes != 3, outputs or workspace overlapping the receive buffer, and
 *   as dit_attn_fwd_ws for the other arguments); UNSUPPORTED (dtype not
 *   bf16, S_loc < 64, alignment, size limits); HIP.
 */
dit_status_t dit_attn_fwd_a2a(const void* recv_buf, void* send_buf, float* lse,
                              const dit_a2a_layout* layout, int32_t rank, float scale, void* workspace,
                              int64_t workspace_bytes, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * dit_attn_fwd_ws with the workspace taken from a static scratch array in
 * the library instead of an argument.  Arguments and results as
 * dit_attn_fwd_ws; no call allocates.
 *
 * The scratch is one 36 MiB (37748736-byte) array per device, held from the
 * first call on that device until the process ends; its counter region is
 * zeroed by the first call on the device (on that call's stream) and left
 * zero by every call.  Every call on a device shares it, so calls that may
 * overlap on one device (different streams, or threads without ordering)
 * RACE: serialize them.  A call whose split plan needs more than the scratch
 * holds is refused (DIT_ERR_UNSUPPORTED) before anything runs; on a 256-CU
 * device no call does (at most 65536 + 256 x 139264 bytes).
 * Errors: as dit_attn_fwd; UNSUPPORTED also for a plan beyond the scratch.
 */
dit_status_t dit_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                  int32_t B, int32_t Sq, int32_t Skv, int32_t H, int32_t D, float scale,
                                  dit_dtype_t in_dtype, dit_dtype_t o_dtype, void* stream);

/*
 * Attention over a per-batch prefix of the keys: keys j >= kv_len[b] of
 * batch b are excluded (their scores count as -inf), e.g. the tail padding
 * of a fixed-length text segment (SGLang "Parallelism Overview": the
 * masked / tail-padded text path of joint text+image attention; xLLM
 * "DiT Architecture and Capability Matrix": a replacement kernel must keep
 * the padding exclusion).  With merge = 1 the result is merged into
 * (o, lse) as dit_attn_fwd_merge does, which is how a replicated text
 * segment attended once is combined with the ring result.
 *
 * kv_len: [B] int32 DEVICE array, 4-byte aligned; values are clamped to
 *   [0, Skv].  A batch with no valid key yields O = 0, LSE = -inf (merge = 0)
 *   or leaves the accumulator unchanged (merge = 1).
 * Other arguments as dit_attn_fwd (merge = 0) or dit_attn_fwd_merge
 *   (merge = 1: o / lse are the accumulator, lse required).
 * Tiles are never split into key chunks on this path (no workspace).
 * Errors: as dit_attn_fwd; INVALID_ARGUMENT also for a NULL kv_len or
 * merge outside {0, 1}.
 */
dit_status_t dit_attn_fwd_kvlen(const void* q, const void* k, const void* v, const int32_t* kv_len,
                                void* o, float* lse, int32_t B, int32_t Sq, int32_t Skv, int32_t H,
                                int32_t D, float scale, dit_dtype_t in_dtype, dit_dtype_t o_dtype,
                                int32_t merge, void* stream);

/*
 * In-place online-softmax merge of a partial result into an accumulator
 * (SGLang "Parallelism Overview": the ring per-hop merge, also used for
 * replicated and tail-padded parts, combines partial results with the
 * kernel's LSE).  Per row (b, i, h), with m = max(L_acc, L_part) and
 * w_x = exp(L_x - m):
 *   L_acc <- m + ln(w_acc + w_part)
 *   O_acc <- (w_acc O_acc + w_part O_part) / (w_acc + w_part)
 * A side whose LSE is -inf is empty and is dropped (selected away, never
 * multiplied, so its O may hold anything); both empty -> (0, -inf).
 * Math in fp32.
 *
 * o_acc, o_part: [B, Sq, H, D] in o_dtype (DIT_BF16 or DIT_F32), D one of
 * 8, 16, 32, ..., 512; lse_acc, lse_part: [B, H, Sq] fp32.  o_acc / lse_acc
 * are read and written in place; they must not overlap the part tensors.
 * Errors: INVALID_ARGUMENT (negative sizes, NULL pointers, overlap),
 * UNSUPPORTED (dtype, head size, alignment, 2^31 or more 8-element chunks),
 * HIP.
 */
dit_status_t dit_attn_merge(void* o_acc, float* lse_acc, const void* o_part,
                            const float* lse_part, int32_t B, int32_t Sq, int32_t H, int32_t D,
                            dit_dtype_t o_dtype, void* stream);

/*
 * One ring hop in one call: attention of q over this K/V chunk merged into
 * the running accumulator (SGLang "Parallelism Overview": the ring keeps Q
 * in place while K/V chunks rotate, and each hop's partial result is folded
 * into the running one with the online-softmax rule through its LSE).  The
 * result equals dit_attn_fwd into a temporary followed by dit_attn_merge,
 * up to rounding (the chunk's O is not rounded to acc_dtype before the
 * merge), without the temporary's HBM round trip.
 *
 * q, k, v, scale, in_dtype: as dit_attn_fwd.
 * o_acc: [B, Sq, H, D] in acc_dtype (in_dtype, or DIT_F32 for bf16 input);
 * lse_acc: [B, H, Sq] fp32, required.  Both are read and written in place.
 *   A row whose lse_acc is -inf holds no keys yet: the call overwrites it
 *   with this chunk's result (so an accumulator set to the identity
 *   O = 0, LSE = -inf starts the hop loop).
 * Skv == 0: the chunk is empty, the accumulator is left unchanged.
 * No aliasing between q/k/v and the accumulator.  Deterministic.
 * workspace, workspace_bytes: as dit_attn_fwd_ws (size from
 *   dit_attn_workspace_size with merge = 1); NULL and 0 for none.
 * Errors: as dit_attn_fwd_ws; INVALID_ARGUMENT also when lse_acc is NULL.
 */
dit_status_t dit_attn_fwd_merge(const void* q, const void* k, const void* v, void* o_acc,
                                float* lse_acc, int32_t B, int32_t Sq, int32_t Skv, int32_t H,
                                int32_t D, float scale, dit_dtype_t in_dtype, dit_dtype_t acc_dtype,
                                void* workspace, int64_t workspace_bytes, void* stream);

/*
 * Classifier-free guidance combine (edge-dit.cpp "Parallel execution", CFG
 * parallelism section): out = p_uncond + g * (p_cond - p_uncond), evaluated
 * per element as fmaf(g, p_cond - p_uncond, p_uncond) in fp32.
 * p_uncond, p_cond, out: n elements of dtype (DIT_F32, or DIT_BF16 with fp32
 * math and round-to-nearest-even output).  out may alias either input
 * exactly (in-place); partial overlap is not allowed.  n == 0: no-op.
 * Errors: INVALID_ARGUMENT (null pointer for n > 0, n < 0, g not finite),
 * UNSUPPORTED (dtype, alignment), HIP.
 */
dit_status_t dit_cfg_combine(const void* p_uncond, const void* p_cond, void* out, int64_t n,
                             float g, dit_dtype_t dtype, void* stream);

/*
 * Measurement aid (not a step of the method): reports the shader clock.
 * Launches `workgroups` workgroups of 256 threads; each runs `spin`
 * iterations of a loop and writes, at out[2*i] and out[2*i+1], the shader
 * cycles (s_memtime) and the ticks of the 100 MHz real-time counter
 * (s_memrealtime) that elapsed in workgroup i.  The clock in GHz is
 * cycles / ticks / 10.  mfma = 0: the loop is two dependent FMAs (a light
 * load); mfma = 1: four independent bf16 32x32x16 MFMAs per wave (the
 * matrix-core load of attention, under which the power limit sets the
 * clock).  out: device memory of 2 * workgroups int64, 8-byte aligned.
 * Errors: INVALID_ARGUMENT (workgroups outside [1, 65536], spin < 0, mfma
 * not 0 or 1, out NULL); UNSUPPORTED (alignment); HIP.
 */
dit_status_t dit_clock_probe(int64_t* out, int32_t workgroups, int32_t spin, int32_t mfma,
                             void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DIT_ATTN_H */
