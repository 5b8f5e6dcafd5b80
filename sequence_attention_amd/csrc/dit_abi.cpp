// C ABI of libdit_attn: argument validation, layout derivation and kernel
// dispatch.  Every check runs on the host before any HIP call, so a failed
// call writes nothing and touches no device (the CPU test suite drives every
// error path on a machine without a GPU).  The library keeps no state apart
// from the calling thread's last error text and per-device facts (compute
// unit count, kernel occupancy) cached on first use.
#include <algorithm>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "../../include/dit_attn.h"
#include "dit_internal.h"

namespace {

thread_local char g_last_error[512] = "";

void clear_error() { g_last_error[0] = '\0'; }

dit_status_t fail(dit_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

dit_status_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return DIT_OK;
  return fail(DIT_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool dtype_ok(int dt) { return dt == DIT_BF16 || dt == DIT_F16 || dt == DIT_F32; }
int dtype_bytes(dit_dtype_t dt) { return dt == DIT_F32 ? 4 : 2; }
bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// a*b*... with overflow detection against int64
bool mul_ok(int64_t& acc, int64_t x) {
  if (x != 0 && acc > INT64_MAX / x) return false;
  acc *= x;
  return true;
}

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t pa = (uintptr_t)a, pb = (uintptr_t)b;
  return na > 0 && nb > 0 && pa < pb + nb && pb < pa + na;
}

int64_t gcd64(int64_t a, int64_t b) {
  while (b) {
    const int64_t t = a % b;
    a = b;
    b = t;
  }
  return a;
}

dit_status_t derive_layout(int32_t B, int32_t S, int32_t H, int32_t D, int32_t U, int32_t seq_align,
                           int32_t n_planes, dit_dtype_t dtype, dit_a2a_layout* L) {
  if (B < 0 || S < 0 || H < 0 || D < 0)
    return fail(DIT_ERR_INVALID_ARGUMENT, "negative size (B=%d S=%d H=%d D=%d)", B, S, H, D);
  if (U < 1) return fail(DIT_ERR_INVALID_ARGUMENT, "Ulysses degree U=%d must be >= 1", U);
  if (seq_align < 1) return fail(DIT_ERR_INVALID_ARGUMENT, "seq_align=%d must be >= 1", seq_align);
  if (n_planes != 1 && n_planes != 3)
    return fail(DIT_ERR_INVALID_ARGUMENT, "n_planes=%d must be 1 or 3", n_planes);
  if (!dtype_ok(dtype)) return fail(DIT_ERR_INVALID_ARGUMENT, "unknown dtype %d", (int)dtype);
  const int64_t align = (int64_t)U / gcd64(U, seq_align) * seq_align;  // lcm(U, seq_align)
  const int64_t S_pad = (S + align - 1) / align * align;
  const int64_t S_loc = S_pad / U;
  const int64_t H_pad = ((int64_t)H + U - 1) / U * U;
  const int64_t H_loc = H_pad / U;
  if (S_pad > INT32_MAX || H_pad > INT32_MAX)
    return fail(DIT_ERR_INVALID_ARGUMENT, "padded sizes overflow int32 (S_pad=%lld H_pad=%lld)",
                (long long)S_pad, (long long)H_pad);
  int64_t epp = n_planes;
  if (!mul_ok(epp, B) || !mul_ok(epp, S_loc) || !mul_ok(epp, H_loc) || !mul_ok(epp, D) ||
      epp > INT64_MAX / U / 4)
    return fail(DIT_ERR_INVALID_ARGUMENT, "element count overflows int64");
  L->B = B; L->S = S; L->H = H; L->D = D; L->U = U;
  L->seq_align = seq_align;
  L->n_planes = n_planes;
  L->dtype = dtype;
  L->S_pad = (int32_t)S_pad;
  L->S_loc = (int32_t)S_loc;
  L->H_pad = (int32_t)H_pad;
  L->H_loc = (int32_t)H_loc;
  L->elems_per_peer = epp;
  return DIT_OK;
}

dit_status_t check_permute(const dit_a2a_layout* L, int dir, int32_t rank) {
  if (L == nullptr) return fail(DIT_ERR_INVALID_ARGUMENT, "layout is NULL");
  dit_a2a_layout ref;
  const dit_status_t st =
      derive_layout(L->B, L->S, L->H, L->D, L->U, L->seq_align, L->n_planes, L->dtype, &ref);
  if (st != DIT_OK) return st;
  if (ref.S_pad != L->S_pad || ref.S_loc != L->S_loc || ref.H_pad != L->H_pad ||
      ref.H_loc != L->H_loc || ref.elems_per_peer != L->elems_per_peer)
    return fail(DIT_ERR_INVALID_ARGUMENT,
                "layout derived fields do not match its sizes (use dit_a2a_layout_init)");
  if (dir != DIT_SEQ_TO_HEAD && dir != DIT_HEAD_TO_SEQ)
    return fail(DIT_ERR_INVALID_ARGUMENT, "unknown direction %d", dir);
  if (rank < 0 || rank >= L->U)
    return fail(DIT_ERR_INVALID_ARGUMENT, "rank %d outside [0, U=%d)", rank, L->U);
  // iteration space of the kernels is indexed with 32-bit unsigned math
  if (L->elems_per_peer * L->U >= (int64_t)1 << 31 ||
      (int64_t)L->n_planes * L->B * L->S * L->H_loc * L->D >= (int64_t)1 << 31)
    return fail(DIT_ERR_UNSUPPORTED, "exchange of %lld elements exceeds 2^31",
                (long long)(L->elems_per_peer * L->U));
  return DIT_OK;
}

dit_status_t run_permute(const dit_a2a_layout* L, int dir, int32_t rank, bool pack,
                         const void* const* in_planes, const void* in_buf, void* const* out_planes,
                         void* out_buf, void* stream) {
  dit_status_t st = check_permute(L, dir, rank);
  if (st != DIT_OK) return st;
  const int eb = dtype_bytes(L->dtype);
  const int64_t buf_elems = L->elems_per_peer * L->U;
  // plane tensor size on the non-buffer side
  const int64_t plane_elems =
      dir == DIT_SEQ_TO_HEAD
          ? (pack ? (int64_t)L->B * L->S_loc * L->H * L->D : (int64_t)L->B * L->S * L->H_loc * L->D)
          : (pack ? (int64_t)L->B * L->S * L->H_loc * L->D : (int64_t)L->B * L->S_loc * L->H * L->D);
  if (buf_elems == 0 && plane_elems == 0) {
    clear_error();
    return DIT_OK;
  }
  const char* side = pack ? "in_planes" : "out_planes";
  if ((pack ? (const void*)in_planes : (const void*)out_planes) == nullptr)
    return fail(DIT_ERR_INVALID_ARGUMENT, "%s array is NULL", side);
  const void* planes[3] = {nullptr, nullptr, nullptr};
  for (int i = 0; i < L->n_planes; ++i) {
    planes[i] = pack ? in_planes[i] : out_planes[i];
    if (plane_elems > 0 && planes[i] == nullptr)
      return fail(DIT_ERR_INVALID_ARGUMENT, "%s[%d] is NULL", side, i);
    if (!aligned(planes[i], eb))
      return fail(DIT_ERR_UNSUPPORTED, "%s[%d] not aligned to its element size", side, i);
  }
  const void* buf = pack ? (const void*)out_buf : in_buf;
  if (buf_elems > 0 && buf == nullptr)
    return fail(DIT_ERR_INVALID_ARGUMENT, "%s is NULL", pack ? "send_buf" : "recv_buf");
  if (!aligned(buf, eb)) return fail(DIT_ERR_UNSUPPORTED, "exchange buffer not element-aligned");
  for (int i = 0; i < L->n_planes; ++i)
    if (overlap(planes[i], (size_t)plane_elems * eb, buf, (size_t)buf_elems * eb))
      return fail(DIT_ERR_INVALID_ARGUMENT, "plane %d overlaps the exchange buffer", i);
  if (!pack)
    for (int i = 0; i < L->n_planes; ++i)
      for (int j = i + 1; j < L->n_planes; ++j)
        if (overlap(planes[i], (size_t)plane_elems * eb, planes[j], (size_t)plane_elems * eb))
          return fail(DIT_ERR_INVALID_ARGUMENT, "output planes %d and %d overlap", i, j);

  dit::PermuteArgs a;
  for (int i = 0; i < 3; ++i) {
    a.in[i] = nullptr;
    a.out[i] = nullptr;
  }
  if (pack) {
    for (int i = 0; i < L->n_planes; ++i) a.in[i] = planes[i];
    a.out[0] = out_buf;
  } else {
    a.in[0] = in_buf;
    for (int i = 0; i < L->n_planes; ++i) a.out[i] = const_cast<void*>(planes[i]);
  }
  a.B = L->B; a.S = L->S; a.H = L->H; a.D = L->D; a.U = L->U; a.n_planes = L->n_planes;
  a.S_loc = L->S_loc; a.H_loc = L->H_loc; a.rank = rank;
  a.elem_bytes = eb;
  const dit::PermuteKind kind =
      dir == DIT_SEQ_TO_HEAD ? (pack ? dit::PACK_SEQ_TO_HEAD : dit::UNPACK_SEQ_TO_HEAD)
                             : (pack ? dit::PACK_HEAD_TO_SEQ : dit::UNPACK_HEAD_TO_SEQ);
  st = hip_status(dit::launch_permute(kind, a, (hipStream_t)stream), "permute launch");
  if (st == DIT_OK) clear_error();
  return st;
}

}  // namespace

extern "C" {

int dit_abi_version(void) { return DIT_ABI_VERSION; }

const char* dit_status_string(dit_status_t status) {
  switch (status) {
    case DIT_OK: return "DIT_OK";
    case DIT_ERR_INVALID_ARGUMENT: return "DIT_ERR_INVALID_ARGUMENT";
    case DIT_ERR_UNSUPPORTED: return "DIT_ERR_UNSUPPORTED";
    case DIT_ERR_HIP: return "DIT_ERR_HIP";
  }
  return "DIT_ERR_UNKNOWN_STATUS";
}

const char* dit_last_error(void) { return g_last_error; }

dit_status_t dit_a2a_layout_init(int32_t B, int32_t S, int32_t H, int32_t D, int32_t U,
                                 int32_t seq_align, int32_t n_planes, dit_dtype_t dtype,
                                 dit_a2a_layout* out) {
  if (out == nullptr) return fail(DIT_ERR_INVALID_ARGUMENT, "out is NULL");
  dit_a2a_layout L;
  const dit_status_t st = derive_layout(B, S, H, D, U, seq_align, n_planes, dtype, &L);
  if (st != DIT_OK) return st;
  *out = L;
  clear_error();
  return DIT_OK;
}

dit_status_t dit_ulysses_pack(const dit_a2a_layout* layout, dit_a2a_dir_t dir, int32_t rank,
                              const void* const* in_planes, void* send_buf, void* stream) {
  return run_permute(layout, (int)dir, rank, true, in_planes, nullptr, nullptr, send_buf, stream);
}

dit_status_t dit_ulysses_unpack(const dit_a2a_layout* layout, dit_a2a_dir_t dir, int32_t rank,
                                const void* recv_buf, void* const* out_planes, void* stream) {
  return run_permute(layout, (int)dir, rank, false, nullptr, recv_buf, out_planes, nullptr, stream);
}

dit_status_t dit_ulysses_pack_convert(const dit_a2a_layout* L, dit_a2a_dir_t dir, int32_t rank,
                                      const void* const* in_planes, void* send_buf, void* stream) {
  dit_status_t st = check_permute(L, (int)dir, rank);
  if (st != DIT_OK) return st;
  if (L->dtype != DIT_BF16 && L->dtype != DIT_F16)
    return fail(DIT_ERR_UNSUPPORTED, "the converting pack writes a bf16 or f16 send buffer "
                                     "(layout dtype %d)", (int)L->dtype);
  const int64_t buf_elems = L->elems_per_peer * L->U;
  const int64_t plane_elems = dir == DIT_SEQ_TO_HEAD ? (int64_t)L->B * L->S_loc * L->H * L->D
                                                     : (int64_t)L->B * L->S * L->H_loc * L->D;
  if (buf_elems == 0 && plane_elems == 0) {
    clear_error();
    return DIT_OK;
  }
  if (in_planes == nullptr) return fail(DIT_ERR_INVALID_ARGUMENT, "in_planes array is NULL");
  if (send_buf == nullptr) return fail(DIT_ERR_INVALID_ARGUMENT, "send_buf is NULL");
  if (!aligned(send_buf, 2)) return fail(DIT_ERR_UNSUPPORTED, "send_buf not 2-byte aligned");
  for (int i = 0; i < L->n_planes; ++i) {
    if (in_planes[i] == nullptr) return fail(DIT_ERR_INVALID_ARGUMENT, "in_planes[%d] is NULL", i);
    if (!aligned(in_planes[i], 4))
      return fail(DIT_ERR_UNSUPPORTED, "in_planes[%d] not 4-byte aligned", i);
    if (overlap(in_planes[i], (size_t)plane_elems * 4, send_buf, (size_t)buf_elems * 2))
      return fail(DIT_ERR_INVALID_ARGUMENT, "plane %d overlaps the send buffer", i);
  }
  dit::PermuteArgs a;
  for (int i = 0; i < 3; ++i) {
    a.in[i] = i < L->n_planes ? in_planes[i] : nullptr;
    a.out[i] = nullptr;
  }
  a.out[0] = send_buf;
  a.B = L->B; a.S = L->S; a.H = L->H; a.D = L->D; a.U = L->U; a.n_planes = L->n_planes;
  a.S_loc = L->S_loc; a.H_loc = L->H_loc; a.rank = rank;
  a.elem_bytes = 4;
  const dit::PermuteKind kind = dir == DIT_SEQ_TO_HEAD ? dit::PACK_SEQ_TO_HEAD : dit::PACK_HEAD_TO_SEQ;
  st = hip_status(dit::launch_pack_convert(kind, a, L->dtype == DIT_BF16, (hipStream_t)stream),
                  "converting pack launch");
  if (st == DIT_OK) clear_error();
  return st;
}

dit_status_t dit_ulysses_unpack_rope(const dit_a2a_layout* L, int32_t rank, const void* recv_buf,
                                     void* const* out_planes, const float* rope_cos,
                                     const float* rope_sin, void* stream) {
  dit_status_t st = check_permute(L, DIT_SEQ_TO_HEAD, rank);
  if (st != DIT_OK) return st;
  if (L->n_planes != 3)
    return fail(DIT_ERR_INVALID_ARGUMENT, "RoPE receive preparation takes the packed Q, K, V buffer "
                                          "(n_planes = 3, got %d)", L->n_planes);
  const int eb = dtype_bytes(L->dtype);
  if (L->D % 2 != 0 || (L->D * eb) % 16 != 0)
    return fail(DIT_ERR_UNSUPPORTED, "head of %d x %d bytes is not a whole number of 16-byte vectors",
                L->D, eb);
  const int64_t buf_elems = L->elems_per_peer * L->U;
  const int64_t plane_elems = (int64_t)L->B * L->S * L->H_loc * L->D;
  if (buf_elems == 0 && plane_elems == 0) {
    clear_error();
    return DIT_OK;
  }
  if (out_planes == nullptr) return fail(DIT_ERR_INVALID_ARGUMENT, "out_planes array is NULL");
  if (recv_buf == nullptr) return fail(DIT_ERR_INVALID_ARGUMENT, "recv_buf is NULL");
  if (rope_cos == nullptr || rope_sin == nullptr)
    return fail(DIT_ERR_INVALID_ARGUMENT, "RoPE tables are NULL");
  const size_t table_bytes = (size_t)L->S * (L->D / 2) * sizeof(float);
  if (!aligned(recv_buf, 16) || !aligned(rope_cos, 16) || !aligned(rope_sin, 16))
    return fail(DIT_ERR_UNSUPPORTED, "recv_buf and the RoPE tables must be 16-byte aligned");
  for (int i = 0; i < 3; ++i) {
    if (out_planes[i] == nullptr) return fail(DIT_ERR_INVALID_ARGUMENT, "out_planes[%d] is NULL", i);
    if (!aligned(out_planes[i], 16))
      return fail(DIT_ERR_UNSUPPORTED, "out_planes[%d] must be 16-byte aligned", i);
    const size_t pb = (size_t)plane_elems * eb;
    if (overlap(out_planes[i], pb, recv_buf, (size_t)buf_elems * eb) ||
        overlap(out_planes[i], pb, rope_cos, table_bytes) || overlap(out_planes[i], pb, rope_sin, table_bytes))
      return fail(DIT_ERR_INVALID_ARGUMENT, "out_planes[%d] overlaps an input", i);
    for (int j = i + 1; j < 3; ++j)
      if (overlap(out_planes[i], pb, out_planes[j], pb))
        return fail(DIT_ERR_INVALID_ARGUMENT, "output planes %d and %d overlap", i, j);
  }
  dit::RopeUnpackArgs a;
  a.recv = recv_buf;
  for (int i = 0; i < 3; ++i) a.out[i] = out_planes[i];
  a.cos = rope_cos;
  a.sin = rope_sin;
  a.B = L->B; a.S = L->S; a.D = L->D; a.U = L->U; a.n_planes = 3; a.S_loc = L->S_loc; a.H_loc = L->H_loc;
  a.elem_bytes = eb;
  a.is_f16 = (L->dtype == DIT_F16);
  st = hip_status(dit::launch_rope_unpack(a, (hipStream_t)stream), "RoPE unpack launch");
  if (st == DIT_OK) clear_error();
  return st;
}

namespace {

// ---- padding-free (uneven) layouts ---------------------------------------------

void balanced_split(int32_t total, int32_t U, int32_t* counts) {
  for (int r = 0; r < U; ++r) counts[r] = total / U + (r < total % U ? 1 : 0);
}

dit_status_t derive_uneven(int32_t B, int32_t S, int32_t H, int32_t D, int32_t U, int32_t n_planes,
                           dit_dtype_t dtype, const int32_t* seq_counts, const int32_t* head_counts,
                           dit_a2a_uneven_layout* L) {
  if (B < 0 || S < 0 || H < 0 || D < 0)
    return fail(DIT_ERR_INVALID_ARGUMENT, "negative size (B=%d S=%d H=%d D=%d)", B, S, H, D);
  if (U < 1 || U > DIT_MAX_RANKS)
    return fail(DIT_ERR_INVALID_ARGUMENT, "degree U=%d outside [1, %d]", U, DIT_MAX_RANKS);
  if (n_planes < 1 || n_planes > 3)
    return fail(DIT_ERR_INVALID_ARGUMENT, "n_planes=%d outside [1, 3]", n_planes);
  if (!dtype_ok(dtype)) return fail(DIT_ERR_INVALID_ARGUMENT, "unknown dtype %d", (int)dtype);
  memset(L, 0, sizeof(*L));
  L->B = B; L->S = S; L->H = H; L->D = D; L->U = U; L->n_planes = n_planes; L->dtype = dtype;
  if (seq_counts) memcpy(L->seq_counts, seq_counts, sizeof(int32_t) * U);
  else balanced_split(S, U, L->seq_counts);
  if (head_counts) memcpy(L->head_counts, head_counts, sizeof(int32_t) * U);
  else balanced_split(H, U, L->head_counts);
  int64_t so = 0, ho = 0;
  for (int r = 0; r < U; ++r) {
    if (L->seq_counts[r] < 0 || L->head_counts[r] < 0)
      return fail(DIT_ERR_INVALID_ARGUMENT, "negative count for rank %d", r);
    L->seq_offsets[r] = (int32_t)so;
    L->head_offsets[r] = (int32_t)ho;
    so += L->seq_counts[r];
    ho += L->head_counts[r];
    if (so > S || ho > H) break;
    if (L->seq_counts[r] > L->S_max) L->S_max = L->seq_counts[r];
  }
  if (so != S || ho != H)
    return fail(DIT_ERR_INVALID_ARGUMENT, "counts sum to S=%lld H=%lld, expected S=%d H=%d",
                (long long)so, (long long)ho, S, H);
  L->seq_offsets[U] = S;
  L->head_offsets[U] = H;
  int64_t e = n_planes;
  if (!mul_ok(e, B) || !mul_ok(e, S) || !mul_ok(e, H) || !mul_ok(e, D) ||
      !mul_ok(e, U))  // covers the padded Ring Anything gather U*n*B*S_max*H*D as well
    return fail(DIT_ERR_INVALID_ARGUMENT, "element count overflows int64");
  return DIT_OK;
}

dit_status_t check_uneven(const dit_a2a_uneven_layout* L) {
  if (L == nullptr) return fail(DIT_ERR_INVALID_ARGUMENT, "layout is NULL");
  if (L->U < 1 || L->U > DIT_MAX_RANKS)
    return fail(DIT_ERR_INVALID_ARGUMENT, "degree U=%d outside [1, %d]", L->U, DIT_MAX_RANKS);
  dit_a2a_uneven_layout ref;
  const dit_status_t st = derive_uneven(L->B, L->S, L->H, L->D, L->U, L->n_planes, L->dtype,
                                        L->seq_counts, L->head_counts, &ref);
  if (st != DIT_OK) return st;
  if (ref.S_max != L->S_max ||
      memcmp(ref.seq_offsets, L->seq_offsets, sizeof(int32_t) * (L->U + 1)) != 0 ||
      memcmp(ref.head_offsets, L->head_offsets, sizeof(int32_t) * (L->U + 1)) != 0)
    return fail(DIT_ERR_INVALID_ARGUMENT,
                "layout derived fields do not match its counts (use dit_a2a_uneven_init)");
  return DIT_OK;
}

// The chunk geometry of one padding-free map (see launch_chunk_copy), with
// the element counts of both sides for validation.
struct UnevenPlan {
  dit::ChunkCopyArgs a;
  int64_t plane_elems;  // one plane
  int64_t buf_elems;    // the whole buffer
};

void plan_uneven(const dit_a2a_uneven_layout* L, int dir, int32_t r, bool pack, UnevenPlan* P) {
  dit::ChunkCopyArgs& a = P->a;
  memset(&a, 0, sizeof(a));
  const int64_t n = L->n_planes, B = L->B, D = L->D;
  a.to_chunk = pack;
  a.n_planes = L->n_planes; a.B = L->B; a.D = L->D; a.elem_bytes = dtype_bytes(L->dtype);
  a.n_peers = L->U;
  // head-slice maps move head windows of rank r's own rows; row-block maps
  // move row windows of rank r's own heads.
  const bool head_slice = (dir == DIT_SEQ_TO_HEAD) == pack;
  int64_t off = 0;
  if (head_slice) {
    const int64_t R = L->seq_counts[r];
    a.plane_b_rows = R;
    a.plane_row = (int64_t)L->H * D;
    for (int p = 0; p < L->U; ++p) {
      const int64_t Hp = L->head_counts[p];
      a.peer[p] = {R, R, Hp * D, (int64_t)L->head_offsets[p] * D, off};
      off += n * B * R * Hp * D;
    }
    P->plane_elems = B * R * L->H * D;
  } else {
    const int64_t Hr = L->head_counts[r];
    a.plane_b_rows = L->S;
    a.plane_row = Hr * D;
    for (int p = 0; p < L->U; ++p) {
      const int64_t Sp = L->seq_counts[p];
      a.peer[p] = {Sp, Sp, Hr * D, (int64_t)L->seq_offsets[p] * Hr * D, off};
      off += n * B * Sp * Hr * D;
    }
    P->plane_elems = B * (int64_t)L->S * Hr * D;
  }
  P->buf_elems = off;
}

void plan_ring_anything(const dit_a2a_uneven_layout* L, int32_t r, bool pad, UnevenPlan* P) {
  dit::ChunkCopyArgs& a = P->a;
  memset(&a, 0, sizeof(a));
  const int64_t n = L->n_planes, B = L->B, HD = (int64_t)L->H * L->D, Smax = L->S_max;
  a.to_chunk = pad;
  a.n_planes = L->n_planes; a.B = L->B; a.D = L->D; a.elem_bytes = dtype_bytes(L->dtype);
  a.plane_row = HD;
  if (pad) {
    a.n_peers = 1;
    a.plane_b_rows = L->seq_counts[r];
    a.peer[0] = {L->seq_counts[r], Smax, HD, 0, 0};
    P->plane_elems = B * L->seq_counts[r] * HD;
    P->buf_elems = n * B * Smax * HD;
  } else {
    a.n_peers = L->U;
    a.plane_b_rows = L->S;
    for (int p = 0; p < L->U; ++p)
      a.peer[p] = {L->seq_counts[p], Smax, HD, (int64_t)L->seq_offsets[p] * HD, p * n * B * Smax * HD};
    P->plane_elems = B * (int64_t)L->S * HD;
    P->buf_elems = L->U * n * B * Smax * HD;
  }
}

dit_status_t run_uneven(const dit_a2a_uneven_layout* L, UnevenPlan& P, const void* const* planes_in,
                        const void* buf_in, void* const* planes_out, void* buf_out, void* stream) {
  const bool pack = P.a.to_chunk;
  const int eb = dtype_bytes(L->dtype);
  if (P.buf_elems == 0 && P.plane_elems == 0) {
    clear_error();
    return DIT_OK;
  }
  if (P.buf_elems >= ((int64_t)1 << 31) || P.plane_elems >= ((int64_t)1 << 31))
    return fail(DIT_ERR_UNSUPPORTED, "2^31 or more elements on one side of the copy");
  if ((int64_t)L->n_planes * L->B > 65535)
    return fail(DIT_ERR_UNSUPPORTED, "B * n_planes = %lld exceeds 65535",
                (long long)L->n_planes * L->B);
  const char* side = pack ? "in_planes" : "out_planes";
  const void* const* planes = pack ? planes_in : (const void* const*)planes_out;
  if (planes == nullptr) return fail(DIT_ERR_INVALID_ARGUMENT, "%s array is NULL", side);
  for (int i = 0; i < L->n_planes; ++i) {
    if (P.plane_elems > 0 && planes[i] == nullptr)
      return fail(DIT_ERR_INVALID_ARGUMENT, "%s[%d] is NULL", side, i);
    if (!aligned(planes[i], eb))
      return fail(DIT_ERR_UNSUPPORTED, "%s[%d] not aligned to its element size", side, i);
  }
  const void* buf = pack ? (const void*)buf_out : buf_in;
  if (P.buf_elems > 0 && buf == nullptr)
    return fail(DIT_ERR_INVALID_ARGUMENT, "exchange buffer is NULL");
  if (!aligned(buf, eb)) return fail(DIT_ERR_UNSUPPORTED, "exchange buffer not element-aligned");
  const size_t pb = (size_t)P.plane_elems * eb;
  for (int i = 0; i < L->n_planes; ++i) {
    if (overlap(planes[i], pb, buf, (size_t)P.buf_elems * eb))
      return fail(DIT_ERR_INVALID_ARGUMENT, "plane %d overlaps the exchange buffer", i);
    if (!pack)
      for (int j = i + 1; j < L->n_planes; ++j)
        if (overlap(planes[i], pb, planes[j], pb))
          return fail(DIT_ERR_INVALID_ARGUMENT, "output planes %d and %d overlap", i, j);
  }
  for (int i = 0; i < L->n_planes; ++i) P.a.planes[i] = const_cast<void*>(planes[i]);
  P.a.chunk = const_cast<void*>(buf);
  const dit_status_t st =
      hip_status(dit::launch_chunk_copy(P.a, (hipStream_t)stream), "chunk copy launch");
  if (st == DIT_OK) clear_error();
  return st;
}

dit_status_t check_dir_rank(const dit_a2a_uneven_layout* L, int dir, int32_t rank) {
  if (dir != DIT_SEQ_TO_HEAD && dir != DIT_HEAD_TO_SEQ)
    return fail(DIT_ERR_INVALID_ARGUMENT, "unknown direction %d", dir);
  if (rank < 0 || rank >= L->U)
    return fail(DIT_ERR_INVALID_ARGUMENT, "rank %d outside [0, U=%d)", rank, L->U);
  return DIT_OK;
}

}  // namespace

dit_status_t dit_a2a_uneven_init(int32_t B, int32_t S, int32_t H, int32_t D, int32_t U,
                                 int32_t n_planes, dit_dtype_t dtype, const int32_t* seq_counts,
                                 const int32_t* head_counts, dit_a2a_uneven_layout* out) {
  if (out == nullptr) return fail(DIT_ERR_INVALID_ARGUMENT, "out is NULL");
  dit_a2a_uneven_layout L;
  const dit_status_t st = derive_uneven(B, S, H, D, U, n_planes, dtype, seq_counts, head_counts, &L);
  if (st != DIT_OK) return st;
  *out = L;
  clear_error();
  return DIT_OK;
}

dit_status_t dit_a2a_uneven_sizes(const dit_a2a_uneven_layout* L, dit_a2a_dir_t dir, int32_t rank,
                                  int64_t* send_counts, int64_t* recv_counts) {
  dit_status_t st = check_uneven(L);
  if (st == DIT_OK) st = check_dir_rank(L, (int)dir, rank);
  if (st != DIT_OK) return st;
  const int64_t base = (int64_t)L->n_planes * L->B * L->D;
  for (int p = 0; p < L->U; ++p) {
    const int64_t mine_s = L->seq_counts[rank], mine_h = L->head_counts[rank];
    const int64_t peer_s = L->seq_counts[p], peer_h = L->head_counts[p];
    const int64_t out_e = dir == DIT_SEQ_TO_HEAD ? base * mine_s * peer_h : base * peer_s * mine_h;
    const int64_t in_e = dir == DIT_SEQ_TO_HEAD ? base * peer_s * mine_h : base * mine_s * peer_h;
    if (send_counts) send_counts[p] = out_e;
    if (recv_counts) recv_counts[p] = in_e;
  }
  clear_error();
  return DIT_OK;
}

dit_status_t dit_ulysses_pack_uneven(const dit_a2a_uneven_layout* L, dit_a2a_dir_t dir, int32_t rank,
                                     const void* const* in_planes, void* send_buf, void* stream) {
  dit_status_t st = check_uneven(L);
  if (st == DIT_OK) st = check_dir_rank(L, (int)dir, rank);
  if (st != DIT_OK) return st;
  UnevenPlan P;
  plan_uneven(L, (int)dir, rank, true, &P);
  return run_uneven(L, P, in_planes, nullptr, nullptr, send_buf, stream);
}

dit_status_t dit_ulysses_unpack_uneven(const dit_a2a_uneven_layout* L, dit_a2a_dir_t dir, int32_t rank,
                                       const void* recv_buf, void* const* out_planes, void* stream) {
  dit_status_t st = check_uneven(L);
  if (st == DIT_OK) st = check_dir_rank(L, (int)dir, rank);
  if (st != DIT_OK) return st;
  UnevenPlan P;
  plan_uneven(L, (int)dir, rank, false, &P);
  return run_uneven(L, P, nullptr, recv_buf, out_planes, nullptr, stream);
}

dit_status_t dit_ring_anything_pad(const dit_a2a_uneven_layout* L, int32_t rank,
                                   const void* const* in_planes, void* send_buf, void* stream) {
  dit_status_t st = check_uneven(L);
  if (st == DIT_OK) st = check_dir_rank(L, DIT_SEQ_TO_HEAD, rank);
  if (st != DIT_OK) return st;
  UnevenPlan P;
  plan_ring_anything(L, rank, true, &P);
  return run_uneven(L, P, in_planes, nullptr, nullptr, send_buf, stream);
}

dit_status_t dit_ring_anything_trim(const dit_a2a_uneven_layout* L, const void* gathered,
                                    void* const* out_planes, void* stream) {
  const dit_status_t st = check_uneven(L);
  if (st != DIT_OK) return st;
  UnevenPlan P;
  plan_ring_anything(L, 0, false, &P);
  return run_uneven(L, P, nullptr, gathered, out_planes, nullptr, stream);
}

namespace {

// ---- FP8 exchange --------------------------------------------------------------

// Bytes of one peer's FP8 chunk: `used` holds the sections, `stride` rounds
// it up to a multiple of 256.
void fp8_chunk_bytes(const dit_a2a_layout* L, int dir, int64_t* used, int64_t* stride) {
  const int64_t E = (int64_t)L->B * L->S_loc * L->H_loc * L->D;
  *used = dir == DIT_SEQ_TO_HEAD ? 4 * E + E / 16 : E + E / 32;
  *stride = (*used + 255) / 256 * 256;
}

dit_status_t check_fp8(const dit_a2a_layout* L, int dir, int32_t rank) {
  dit_status_t st = check_permute(L, dir, rank);
  if (st != DIT_OK) return st;
  if (L->dtype != DIT_BF16) return fail(DIT_ERR_UNSUPPORTED, "the FP8 exchange takes bf16 planes");
  if (L->D % 32 != 0)
    return fail(DIT_ERR_UNSUPPORTED, "head dim %d is not a multiple of the 32-element scale block", L->D);
  const int want = dir == DIT_SEQ_TO_HEAD ? 3 : 1;
  if (L->n_planes != want)
    return fail(DIT_ERR_INVALID_ARGUMENT, "the FP8 %s exchange takes n_planes = %d (got %d)",
                dir == DIT_SEQ_TO_HEAD ? "sequence-to-head (Q, K, V)" : "head-to-sequence (O)", want,
                L->n_planes);
  int64_t used, stride;
  fp8_chunk_bytes(L, dir, &used, &stride);
  if (stride * L->U >= ((int64_t)1 << 40))
    return fail(DIT_ERR_UNSUPPORTED, "FP8 exchange buffer too large");
  return DIT_OK;
}

dit_status_t run_fp8(const dit_a2a_layout* L, int dir, int32_t rank, bool pack, const void* const* planes,
                     const void* buf, void* stream) {
  dit_status_t st = check_fp8(L, dir, rank);
  if (st != DIT_OK) return st;
  int64_t used, stride;
  fp8_chunk_bytes(L, dir, &used, &stride);
  const int64_t buf_bytes = stride * L->U;
  const int64_t plane_elems =
      dir == DIT_SEQ_TO_HEAD
          ? (pack ? (int64_t)L->B * L->S_loc * L->H * L->D : (int64_t)L->B * L->S * L->H_loc * L->D)
          : (pack ? (int64_t)L->B * L->S * L->H_loc * L->D : (int64_t)L->B * L->S_loc * L->H * L->D);
  if (buf_bytes == 0 && plane_elems == 0) {
    clear_error();
    return DIT_OK;
  }
  const char* side = pack ? "in_planes" : "out_planes";
  if (planes == nullptr) return fail(DIT_ERR_INVALID_ARGUMENT, "%s array is NULL", side);
  for (int i = 0; i < L->n_planes; ++i) {
    if (plane_elems > 0 && planes[i] == nullptr)
      return fail(DIT_ERR_INVALID_ARGUMENT, "%s[%d] is NULL", side, i);
    if (!aligned(planes[i], 16)) return fail(DIT_ERR_UNSUPPORTED, "%s[%d] must be 16-byte aligned", side, i);
  }
  if (buf_bytes > 0 && buf == nullptr)
    return fail(DIT_ERR_INVALID_ARGUMENT, "%s is NULL", pack ? "send_buf" : "recv_buf");
  if (!aligned(buf, 16)) return fail(DIT_ERR_UNSUPPORTED, "the FP8 exchange buffer must be 16-byte aligned");
  const size_t pb = (size_t)plane_elems * 2;
  for (int i = 0; i < L->n_planes; ++i) {
    if (overlap(planes[i], pb, buf, (size_t)buf_bytes))
      return fail(DIT_ERR_INVALID_ARGUMENT, "plane %d overlaps the exchange buffer", i);
    if (!pack)
      for (int j = i + 1; j < L->n_planes; ++j)
        if (overlap(planes[i], pb, planes[j], pb))
          return fail(DIT_ERR_INVALID_ARGUMENT, "output planes %d and %d overlap", i, j);
  }
  dit::Fp8PermuteArgs a;
  for (int i = 0; i < 3; ++i) a.planes[i] = i < L->n_planes ? planes[i] : nullptr;
  a.buf = buf;
  a.stride = stride;
  a.used = used;
  a.B = L->B; a.S = L->S; a.H = L->H; a.D = L->D; a.U = L->U; a.S_loc = L->S_loc; a.H_loc = L->H_loc;
  a.rank = rank;
  const dit::PermuteKind kind =
      dir == DIT_SEQ_TO_HEAD ? (pack ? dit::PACK_SEQ_TO_HEAD : dit::UNPACK_SEQ_TO_HEAD)
                             : (pack ? dit::PACK_HEAD_TO_SEQ : dit::UNPACK_HEAD_TO_SEQ);
  st = hip_status(dit::launch_fp8_permute(kind, a, (hipStream_t)stream), "FP8 permute launch");
  if (st == DIT_OK) clear_error();
  return st;
}

}  // namespace

dit_status_t dit_a2a_fp8_bytes_per_peer(const dit_a2a_layout* L, dit_a2a_dir_t dir, int64_t* bytes) {
  if (bytes == nullptr) return fail(DIT_ERR_INVALID_ARGUMENT, "bytes is NULL");
  const dit_status_t st = check_fp8(L, (int)dir, 0);
  if (st != DIT_OK) return st;
  int64_t used, stride;
  fp8_chunk_bytes(L, (int)dir, &used, &stride);
  *bytes = stride;
  clear_error();
  return DIT_OK;
}

dit_status_t dit_ulysses_pack_fp8(const dit_a2a_layout* L, dit_a2a_dir_t dir, int32_t rank,
                                  const void* const* in_planes, void* send_buf, void* stream) {
  return run_fp8(L, (int)dir, rank, true, in_planes, send_buf, stream);
}

dit_status_t dit_ulysses_unpack_fp8(const dit_a2a_layout* L, dit_a2a_dir_t dir, int32_t rank,
                                    const void* recv_buf, void* const* out_planes, void* stream) {
  return run_fp8(L, (int)dir, rank, false, (const void* const*)out_planes, recv_buf, stream);
}

}  // extern "C"

namespace {

// Checks shared by every attention call and the workspace size query.
dit_status_t check_attn_shape(int32_t B, int32_t Sq, int32_t Skv, int32_t H, int32_t D,
                              dit_dtype_t in_dtype, dit_dtype_t o_dtype) {
  if (B < 0 || Sq < 0 || Skv < 0 || H < 0 || D < 0)
    return fail(DIT_ERR_INVALID_ARGUMENT, "negative size (B=%d Sq=%d Skv=%d H=%d D=%d)", B, Sq, Skv,
                H, D);
  if (!dtype_ok(in_dtype) || !dtype_ok(o_dtype))
    return fail(DIT_ERR_INVALID_ARGUMENT, "unknown dtype (in=%d o=%d)", (int)in_dtype, (int)o_dtype);
  if (in_dtype == DIT_F16) return fail(DIT_ERR_UNSUPPORTED, "fp16 attention is not served");
  if (in_dtype == DIT_BF16 && o_dtype != DIT_BF16 && o_dtype != DIT_F32)
    return fail(DIT_ERR_UNSUPPORTED, "bf16 attention writes bf16 or fp32 output");
  if (in_dtype == DIT_F32 && o_dtype != DIT_F32)
    return fail(DIT_ERR_UNSUPPORTED, "fp32 attention writes fp32 output");
  if (D != 64 && D != 128) return fail(DIT_ERR_UNSUPPORTED, "head dim %d not in {64, 128}", D);
  // tile counts are 32-bit; the fp32 path puts H and B on grid y / z
  if ((int64_t)B * H * ((Sq + 127) / 128) >= (int64_t)1 << 31)
    return fail(DIT_ERR_UNSUPPORTED, "too many query tiles");
  // the bf16 kernel addresses a 64-row K/V block with 32-bit byte offsets
  if ((int64_t)H * D * 2 * 64 >= ((int64_t)1 << 30))
    return fail(DIT_ERR_UNSUPPORTED, "row stride H*D=%lld too large", (long long)H * D);
  if (in_dtype == DIT_F32 && (H > 65535 || B > 65535))
    return fail(DIT_ERR_UNSUPPORTED, "fp32 path limits B and H to 65535");
  return DIT_OK;
}

dit::AttnArgs attn_args(int32_t B, int32_t Sq, int32_t Skv, int32_t H, int32_t D, float scale,
                        dit_dtype_t o_dtype, bool merge) {
  dit::AttnArgs a;
  a.q = a.k = a.v = nullptr;
  a.o = nullptr;
  a.lse = nullptr;
  a.B = B; a.Sq = Sq; a.Skv = Skv; a.H = H; a.D = D;
  a.scale = scale;
  a.o_f32 = (o_dtype == DIT_F32);
  a.merge = merge;
  return a;
}

// Workspace bytes of a validated call (0 when no tile is ever split: fp32
// path, empty calls, per-batch key lengths).
dit_status_t attn_workspace_need(const dit::AttnArgs& a, dit_dtype_t in_dtype, bool has_kv_len,
                                 size_t* need) {
  *need = 0;
  if (in_dtype != DIT_BF16 || has_kv_len || (int64_t)a.B * a.Sq * a.H == 0 || a.Skv == 0) return DIT_OK;
  return hip_status(dit::attn_bf16_workspace_bytes(a, need), "workspace size query");
}

// dit_attn_fwd, _ws, _kvlen and _merge: one validation path; `merge` makes
// (o, lse) an accumulator that this call merges into.
dit_status_t attn_call(const void* q, const void* k, const void* v, void* o, float* lse, int32_t B,
                       int32_t Sq, int32_t Skv, int32_t H, int32_t D, float scale, dit_dtype_t in_dtype,
                       dit_dtype_t o_dtype, void* stream, bool merge, const int32_t* kv_len = nullptr,
                       bool has_kv_len = false, void* workspace = nullptr, int64_t workspace_bytes = 0,
                       bool static_scratch = false, const dit_a2a_layout* send = nullptr,
                       int32_t send_rank = 0, const dit_a2a_layout* recv = nullptr) {
  dit_status_t st = check_attn_shape(B, Sq, Skv, H, D, in_dtype, o_dtype);
  if (st != DIT_OK) return st;
  if (!(scale > 0.0f) || !isfinite(scale))
    return fail(DIT_ERR_INVALID_ARGUMENT, "scale must be finite and > 0");
  if (workspace_bytes < 0) return fail(DIT_ERR_INVALID_ARGUMENT, "workspace_bytes < 0");
  if (workspace == nullptr && workspace_bytes != 0)
    return fail(DIT_ERR_INVALID_ARGUMENT, "workspace is NULL but workspace_bytes is not 0");
  if (workspace != nullptr && !aligned(workspace, 256))
    return fail(DIT_ERR_UNSUPPORTED, "workspace must be 256-byte aligned");
  if ((int64_t)B * Sq * H == 0) {
    clear_error();
    return DIT_OK;
  }
  if (q == nullptr || o == nullptr) return fail(DIT_ERR_INVALID_ARGUMENT, "q or o is NULL");
  if (merge && lse == nullptr) return fail(DIT_ERR_INVALID_ARGUMENT, "the merge needs the accumulator's LSE");
  if (has_kv_len && kv_len == nullptr) return fail(DIT_ERR_INVALID_ARGUMENT, "kv_len is NULL");
  if (has_kv_len && !aligned(kv_len, 4)) return fail(DIT_ERR_UNSUPPORTED, "kv_len not 4-byte aligned");
  if (Skv > 0 && (k == nullptr || v == nullptr))
    return fail(DIT_ERR_INVALID_ARGUMENT, "k or v is NULL");
  if (!aligned(q, 16) || !aligned(o, 16) || (Skv > 0 && (!aligned(k, 16) || !aligned(v, 16))))
    return fail(DIT_ERR_UNSUPPORTED, "q/k/v/o must be 16-byte aligned");
  if (lse != nullptr && !aligned(lse, 4)) return fail(DIT_ERR_UNSUPPORTED, "lse not 4-byte aligned");
  const int eb = dtype_bytes(in_dtype);
  // with a receive buffer, q is its start and the three planes lie inside it
  const size_t q_bytes = recv != nullptr ? (size_t)recv->U * recv->elems_per_peer * eb : (size_t)B * Sq * H * D * eb;
  const size_t kv_bytes = recv != nullptr ? 0 : (size_t)B * Skv * H * D * eb;
  // O is [B, Sq, H, D], or the whole send buffer [U, 1, B, S_loc, H, D]
  const size_t o_bytes = send != nullptr ? (size_t)send->U * send->elems_per_peer * 2
                                         : (size_t)B * Sq * H * D * dtype_bytes(o_dtype);
  const size_t lse_bytes = (size_t)B * H * Sq * 4;
  if (overlap(o, o_bytes, q, q_bytes) || overlap(o, o_bytes, k, kv_bytes) ||
      overlap(o, o_bytes, v, kv_bytes) ||
      (lse != nullptr && (overlap(lse, lse_bytes, o, o_bytes) || overlap(lse, lse_bytes, q, q_bytes) ||
                          overlap(lse, lse_bytes, k, kv_bytes) || overlap(lse, lse_bytes, v, kv_bytes))))
    return fail(DIT_ERR_INVALID_ARGUMENT, "outputs overlap inputs");
  if (workspace != nullptr) {
    const size_t wb = (size_t)workspace_bytes;
    if (overlap(workspace, wb, o, o_bytes) || overlap(workspace, wb, q, q_bytes) ||
        overlap(workspace, wb, k, kv_bytes) || overlap(workspace, wb, v, kv_bytes) ||
        (lse != nullptr && overlap(workspace, wb, lse, (size_t)B * H * Sq * 4)))
      return fail(DIT_ERR_INVALID_ARGUMENT, "workspace overlaps a tensor");
  }

  if (merge && Skv == 0) {  // an empty chunk is the merge identity
    clear_error();
    return DIT_OK;
  }
  if (send != nullptr && Skv == 0) {  // O = 0 everywhere, pads included; LSE = -inf
    hipError_t e = dit::launch_fill_words(o, o_bytes / 4, 0u, (hipStream_t)stream);
    if (e == hipSuccess && lse != nullptr)
      e = dit::launch_fill_words(lse, (uint64_t)B * H * Sq, 0xFF800000u, (hipStream_t)stream);
    st = hip_status(e, "empty attention fill");
    if (st == DIT_OK) clear_error();
    return st;
  }
  dit::AttnArgs a = attn_args(B, Sq, Skv, H, D, scale, o_dtype, merge);
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  a.kv_len = has_kv_len ? kv_len : nullptr;
  if (send != nullptr) {
    a.send_rows = send->S_loc;
    a.o_heads = std::max(0, std::min(send->H_loc, send->H - send_rank * send->H_loc));
  }
  if (recv != nullptr) {
    a.in_rows = recv->S_loc;
    a.in_peers = recv->U;
    a.in_peer = recv->elems_per_peer;
  }
  if (workspace != nullptr) {
    size_t need = 0;
    if ((st = attn_workspace_need(a, in_dtype, has_kv_len, &need)) != DIT_OK) return st;
    if ((size_t)workspace_bytes < need)
      return fail(DIT_ERR_INVALID_ARGUMENT,
                  "workspace of %lld bytes; this call needs %llu (dit_attn_workspace_size)",
                  (long long)workspace_bytes, (unsigned long long)need);
    a.workspace = workspace;
    a.workspace_bytes = (size_t)workspace_bytes;
  } else if (static_scratch) {
    size_t need = 0;
    if ((st = attn_workspace_need(a, in_dtype, has_kv_len, &need)) != DIT_OK) return st;
    if (need > dit::kAttnScratchBytes)
      return fail(DIT_ERR_UNSUPPORTED, "this call needs %llu bytes of scratch; the static scratch holds %llu",
                  (unsigned long long)need, (unsigned long long)dit::kAttnScratchBytes);
    if (need > 0) {
      void* ptr = nullptr;
      size_t cap = 0;
      if ((st = hip_status(dit::attn_scratch((hipStream_t)stream, &ptr, &cap), "static scratch")) != DIT_OK)
        return st;
      a.workspace = ptr;
      a.workspace_bytes = cap;
    }
  }
  hipError_t e;
  if (Skv == 0) e = dit::launch_attn_empty(a, in_dtype == DIT_F32, (hipStream_t)stream);
  else if (in_dtype == DIT_BF16) e = dit::launch_attn_fwd_bf16(a, (hipStream_t)stream);
  else e = dit::launch_attn_fwd_f32(a, (hipStream_t)stream);
  // pad rows of the padded sequence have no query: zero them in the buffer
  if (e == hipSuccess && send != nullptr && (int64_t)send->U * send->S_loc > Sq)
    e = dit::launch_send_rows_zero(o, B, send->S_loc, Sq, send->U * send->S_loc, (int64_t)H * D,
                                   (hipStream_t)stream);
  st = hip_status(e, "attention launch");
  if (st == DIT_OK) clear_error();
  return st;
}

}  // namespace

extern "C" {

dit_status_t dit_attn_workspace_size(int32_t B, int32_t Sq, int32_t Skv, int32_t H, int32_t D,
                                     dit_dtype_t in_dtype, dit_dtype_t o_dtype, int32_t merge,
                                     int64_t* bytes) {
  if (bytes == nullptr) return fail(DIT_ERR_INVALID_ARGUMENT, "bytes is NULL");
  if (merge != 0 && merge != 1) return fail(DIT_ERR_INVALID_ARGUMENT, "merge must be 0 or 1");
  dit_status_t st = check_attn_shape(B, Sq, Skv, H, D, in_dtype, o_dtype);
  if (st != DIT_OK) return st;
  size_t need = 0;
  st = attn_workspace_need(attn_args(B, Sq, Skv, H, D, 1.0f, o_dtype, merge == 1), in_dtype, false, &need);
  if (st != DIT_OK) return st;
  *bytes = (int64_t)need;
  clear_error();
  return DIT_OK;
}

dit_status_t dit_attn_fwd_ws(const void* q, const void* k, const void* v, void* o, float* lse,
                             int32_t B, int32_t Sq, int32_t Skv, int32_t H, int32_t D, float scale,
                             dit_dtype_t in_dtype, dit_dtype_t o_dtype, void* workspace,
                             int64_t workspace_bytes, void* stream) {
  return attn_call(q, k, v, o, lse, B, Sq, Skv, H, D, scale, in_dtype, o_dtype, stream, false, nullptr,
                   false, workspace, workspace_bytes);
}

dit_status_t dit_attn_fwd_send(const void* q, const void* k, const void* v, void* send_buf, float* lse,
                               const dit_a2a_layout* layout, int32_t rank, int32_t Skv, float scale,
                               void* workspace, int64_t workspace_bytes, void* stream) {
  dit_status_t st = check_permute(layout, DIT_HEAD_TO_SEQ, rank);
  if (st != DIT_OK) return st;
  if (layout->n_planes != 1)
    return fail(DIT_ERR_INVALID_ARGUMENT, "the send buffer holds one plane (O); layout has n_planes = %d",
                layout->n_planes);
  if (layout->dtype != DIT_BF16)
    return fail(DIT_ERR_UNSUPPORTED, "attention into the send buffer is served for bf16 only");
  return attn_call(q, k, v, send_buf, lse, layout->B, layout->S, Skv, layout->H_loc, layout->D, scale,
                   DIT_BF16, DIT_BF16, stream, false, nullptr, false, workspace, workspace_bytes, false,
                   layout, rank);
}

dit_status_t dit_attn_fwd_a2a(const void* recv_buf, void* send_buf, float* lse,
                              const dit_a2a_layout* layout, int32_t rank, float scale, void* workspace,
                              int64_t workspace_bytes, void* stream) {
  dit_status_t st = check_permute(layout, DIT_SEQ_TO_HEAD, rank);
  if (st != DIT_OK) return st;
  if (layout->n_planes != 3)
    return fail(DIT_ERR_INVALID_ARGUMENT, "the receive buffer holds three planes (Q, K, V); layout has n_planes = %d",
                layout->n_planes);
  if (layout->dtype != DIT_BF16)
    return fail(DIT_ERR_UNSUPPORTED, "attention from the receive buffer is served for bf16 only");
  if (layout->S_loc < 64)
    return fail(DIT_ERR_UNSUPPORTED, "attention from the receive buffer needs S_loc >= 64 (S_loc = %d)",
                layout->S_loc);
  if ((int64_t)layout->B * layout->S * layout->H_loc == 0) {
    clear_error();
    return DIT_OK;
  }
  if (recv_buf == nullptr) return fail(DIT_ERR_INVALID_ARGUMENT, "recv_buf is NULL");
  // O goes to the head-to-sequence send buffer: the same group with one plane
  dit_a2a_layout out = *layout;
  out.n_planes = 1;
  out.elems_per_peer = layout->elems_per_peer / 3;
  const int64_t plane = out.elems_per_peer;  // B * S_loc * H_loc * D
  const uint16_t* q = static_cast<const uint16_t*>(recv_buf);
  return attn_call(q, q + plane, q + 2 * plane, send_buf, lse, layout->B, layout->S, layout->S, layout->H_loc,
                   layout->D, scale, DIT_BF16, DIT_BF16, stream, false, nullptr, false, workspace,
                   workspace_bytes, false, &out, rank, layout);
}

dit_status_t dit_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                  int32_t B, int32_t Sq, int32_t Skv, int32_t H, int32_t D, float scale,
                                  dit_dtype_t in_dtype, dit_dtype_t o_dtype, void* stream) {
  return attn_call(q, k, v, o, lse, B, Sq, Skv, H, D, scale, in_dtype, o_dtype, stream, false, nullptr,
                   false, nullptr, 0, true);
}

dit_status_t dit_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                          int32_t B, int32_t Sq, int32_t Skv, int32_t H, int32_t D, float scale,
                          dit_dtype_t in_dtype, dit_dtype_t o_dtype, void* stream) {
  return attn_call(q, k, v, o, lse, B, Sq, Skv, H, D, scale, in_dtype, o_dtype, stream, false);
}

dit_status_t dit_attn_fwd_kvlen(const void* q, const void* k, const void* v, const int32_t* kv_len,
                                void* o, float* lse, int32_t B, int32_t Sq, int32_t Skv, int32_t H,
                                int32_t D, float scale, dit_dtype_t in_dtype, dit_dtype_t o_dtype,
                                int32_t merge, void* stream) {
  if (merge != 0 && merge != 1) return fail(DIT_ERR_INVALID_ARGUMENT, "merge must be 0 or 1");
  return attn_call(q, k, v, o, lse, B, Sq, Skv, H, D, scale, in_dtype, o_dtype, stream, merge == 1,
                   kv_len, true);
}

dit_status_t dit_attn_fwd_merge(const void* q, const void* k, const void* v, void* o_acc,
                                float* lse_acc, int32_t B, int32_t Sq, int32_t Skv, int32_t H,
                                int32_t D, float scale, dit_dtype_t in_dtype, dit_dtype_t acc_dtype,
                                void* workspace, int64_t workspace_bytes, void* stream) {
  return attn_call(q, k, v, o_acc, lse_acc, B, Sq, Skv, H, D, scale, in_dtype, acc_dtype, stream, true,
                   nullptr, false, workspace, workspace_bytes);
}

dit_status_t dit_attn_merge(void* o_acc, float* lse_acc, const void* o_part, const float* lse_part,
                            int32_t B, int32_t Sq, int32_t H, int32_t D, dit_dtype_t o_dtype,
                            void* stream) {
  if (B < 0 || Sq < 0 || H < 0 || D < 0)
    return fail(DIT_ERR_INVALID_ARGUMENT, "negative size (B=%d Sq=%d H=%d D=%d)", B, Sq, H, D);
  if (!dtype_ok(o_dtype)) return fail(DIT_ERR_INVALID_ARGUMENT, "unknown dtype %d", (int)o_dtype);
  if (o_dtype == DIT_F16) return fail(DIT_ERR_UNSUPPORTED, "fp16 merge is not served");
  // one row's D/8 lanes must sit in one wavefront (the row's LSE is updated
  // in place after all of them read it)
  if (D < 8 || D % 8 != 0 || D / 8 > 64 || ((D / 8) & (D / 8 - 1)) != 0)
    return fail(DIT_ERR_UNSUPPORTED, "head dim %d: merge needs D = 8 * 2^k <= 512", D);
  const int64_t rows = (int64_t)B * Sq * H;
  if (rows == 0) {
    clear_error();
    return DIT_OK;
  }
  if (o_acc == nullptr || lse_acc == nullptr || o_part == nullptr || lse_part == nullptr)
    return fail(DIT_ERR_INVALID_ARGUMENT, "NULL tensor pointer");
  if (!aligned(o_acc, 16) || !aligned(o_part, 16) || !aligned(lse_acc, 4) || !aligned(lse_part, 4))
    return fail(DIT_ERR_UNSUPPORTED, "O must be 16-byte and LSE 4-byte aligned");
  const size_t o_bytes = (size_t)rows * D * dtype_bytes(o_dtype);
  const size_t l_bytes = (size_t)rows * 4;
  if (overlap(o_acc, o_bytes, o_part, o_bytes) || overlap(lse_acc, l_bytes, lse_part, l_bytes) ||
      overlap(o_acc, o_bytes, lse_acc, l_bytes) || overlap(o_acc, o_bytes, lse_part, l_bytes) ||
      overlap(lse_acc, l_bytes, o_part, o_bytes))
    return fail(DIT_ERR_INVALID_ARGUMENT, "accumulator overlaps the partial result");
  if (rows * (D / 8) >= (int64_t)1 << 31) return fail(DIT_ERR_UNSUPPORTED, "merge too large");
  const dit_status_t st =
      hip_status(dit::launch_attn_merge(o_acc, lse_acc, o_part, lse_part, B, Sq, H, D,
                                        o_dtype == DIT_F32, (hipStream_t)stream),
                 "merge launch");
  if (st == DIT_OK) clear_error();
  return st;
}

dit_status_t dit_cfg_combine(const void* p_uncond, const void* p_cond, void* out, int64_t n, float g,
                             dit_dtype_t dtype, void* stream) {
  if (n < 0) return fail(DIT_ERR_INVALID_ARGUMENT, "n=%lld < 0", (long long)n);
  if (!isfinite(g)) return fail(DIT_ERR_INVALID_ARGUMENT, "guidance scale is not finite");
  if (!dtype_ok(dtype)) return fail(DIT_ERR_INVALID_ARGUMENT, "unknown dtype %d", (int)dtype);
  if (dtype == DIT_F16) return fail(DIT_ERR_UNSUPPORTED, "fp16 CFG combine is not served");
  if (n == 0) {
    clear_error();
    return DIT_OK;
  }
  if (p_uncond == nullptr || p_cond == nullptr || out == nullptr)
    return fail(DIT_ERR_INVALID_ARGUMENT, "NULL tensor pointer");
  if (!aligned(p_uncond, 16) || !aligned(p_cond, 16) || !aligned(out, 16))
    return fail(DIT_ERR_UNSUPPORTED, "tensors must be 16-byte aligned");
  const size_t bytes = (size_t)n * dtype_bytes(dtype);
  if ((out != p_uncond && overlap(out, bytes, p_uncond, bytes)) ||
      (out != p_cond && overlap(out, bytes, p_cond, bytes)))
    return fail(DIT_ERR_INVALID_ARGUMENT, "out partially overlaps an input");
  if (n / 4096 >= ((int64_t)1 << 31)) return fail(DIT_ERR_UNSUPPORTED, "n too large");
  hipError_t e;
  if (dtype == DIT_F32)
    e = dit::launch_cfg_combine_f32(static_cast<const float*>(p_uncond),
                                    static_cast<const float*>(p_cond), static_cast<float*>(out), n, g,
                                    (hipStream_t)stream);
  else
    e = dit::launch_cfg_combine_bf16(static_cast<const uint16_t*>(p_uncond),
                                     static_cast<const uint16_t*>(p_cond), static_cast<uint16_t*>(out),
                                     n, g, (hipStream_t)stream);
  const dit_status_t st = hip_status(e, "CFG launch");
  if (st == DIT_OK) clear_error();
  return st;
}

dit_status_t dit_clock_probe(int64_t* out, int32_t workgroups, int32_t spin, int32_t mfma, void* stream) {
  if (workgroups < 1 || workgroups > 65536)
    return fail(DIT_ERR_INVALID_ARGUMENT, "workgroups=%d outside [1, 65536]", workgroups);
  if (spin < 0) return fail(DIT_ERR_INVALID_ARGUMENT, "spin=%d < 0", spin);
  if (mfma != 0 && mfma != 1) return fail(DIT_ERR_INVALID_ARGUMENT, "mfma=%d must be 0 or 1", mfma);
  if (out == nullptr) return fail(DIT_ERR_INVALID_ARGUMENT, "out is NULL");
  if (!aligned(out, 8)) return fail(DIT_ERR_UNSUPPORTED, "out not 8-byte aligned");
  const dit_status_t st = hip_status(dit::launch_clock_probe(out, workgroups, spin, mfma != 0, (hipStream_t)stream),
                                     "clock probe launch");
  if (st == DIT_OK) clear_error();
  return st;
}

}  // extern "C"
