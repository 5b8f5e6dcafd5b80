// C ABI of libdit_attn: argument validation, layout derivation and kernel
// dispatch.  Every check runs on the host before any HIP call, so a failed
// call writes nothing and touches no device (the CPU test suite drives every
// error path on a machine without a GPU).  The library keeps no state apart
// from the calling thread's last error text.
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

// dit_attn_fwd and dit_attn_fwd_merge: one validation path; `merge` makes
// (o, lse) an accumulator that this call merges into.
dit_status_t attn_call(const void* q, const void* k, const void* v, void* o, float* lse, int32_t B,
                       int32_t Sq, int32_t Skv, int32_t H, int32_t D, float scale, dit_dtype_t in_dtype,
                       dit_dtype_t o_dtype, void* stream, bool merge, const int32_t* kv_len = nullptr,
                       bool has_kv_len = false) {
  if (B < 0 || Sq < 0 || Skv < 0 || H < 0 || D < 0)
    return fail(DIT_ERR_INVALID_ARGUMENT, "negative size (B=%d Sq=%d Skv=%d H=%d D=%d)", B, Sq, Skv,
                H, D);
  if (!dtype_ok(in_dtype) || !dtype_ok(o_dtype))
    return fail(DIT_ERR_INVALID_ARGUMENT, "unknown dtype (in=%d o=%d)", (int)in_dtype, (int)o_dtype);
  if (!(scale > 0.0f) || !isfinite(scale))
    return fail(DIT_ERR_INVALID_ARGUMENT, "scale must be finite and > 0");
  if (in_dtype == DIT_F16) return fail(DIT_ERR_UNSUPPORTED, "fp16 attention is not served");
  if (in_dtype == DIT_BF16 && o_dtype != DIT_BF16 && o_dtype != DIT_F32)
    return fail(DIT_ERR_UNSUPPORTED, "bf16 attention writes bf16 or fp32 output");
  if (in_dtype == DIT_F32 && o_dtype != DIT_F32)
    return fail(DIT_ERR_UNSUPPORTED, "fp32 attention writes fp32 output");
  if (D != 64 && D != 128) return fail(DIT_ERR_UNSUPPORTED, "head dim %d not in {64, 128}", D);
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
  const size_t q_bytes = (size_t)B * Sq * H * D * eb;
  const size_t kv_bytes = (size_t)B * Skv * H * D * eb;
  const size_t o_bytes = (size_t)B * Sq * H * D * dtype_bytes(o_dtype);
  if (overlap(o, o_bytes, q, q_bytes) || overlap(o, o_bytes, k, kv_bytes) ||
      overlap(o, o_bytes, v, kv_bytes) ||
      (lse != nullptr && overlap(lse, (size_t)B * H * Sq * 4, o, o_bytes)))
    return fail(DIT_ERR_INVALID_ARGUMENT, "outputs overlap inputs");
  // tile counts are 32-bit; the fp32 path puts H and B on grid y / z
  if ((int64_t)B * H * ((Sq + 127) / 128) >= (int64_t)1 << 31)
    return fail(DIT_ERR_UNSUPPORTED, "too many query tiles");
  // the bf16 kernel addresses a 64-row K/V block with 32-bit byte offsets
  if ((int64_t)H * D * 2 * 64 >= ((int64_t)1 << 30))
    return fail(DIT_ERR_UNSUPPORTED, "row stride H*D=%lld too large", (long long)H * D);
  if (in_dtype == DIT_F32 && (H > 65535 || B > 65535))
    return fail(DIT_ERR_UNSUPPORTED, "fp32 path limits B and H to 65535");

  if (merge && Skv == 0) {  // an empty chunk is the merge identity
    clear_error();
    return DIT_OK;
  }
  dit::AttnArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  a.merge = merge;
  a.kv_len = has_kv_len ? kv_len : nullptr;
  a.B = B; a.Sq = Sq; a.Skv = Skv; a.H = H; a.D = D;
  a.scale = scale;
  a.o_f32 = (o_dtype == DIT_F32);
  hipError_t e;
  if (Skv == 0) e = dit::launch_attn_empty(a, in_dtype == DIT_F32, (hipStream_t)stream);
  else if (in_dtype == DIT_BF16) e = dit::launch_attn_fwd_bf16(a, (hipStream_t)stream);
  else e = dit::launch_attn_fwd_f32(a, (hipStream_t)stream);
  const dit_status_t st = hip_status(e, "attention launch");
  if (st == DIT_OK) clear_error();
  return st;
}

}  // namespace

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
                                void* stream) {
  return attn_call(q, k, v, o_acc, lse_acc, B, Sq, Skv, H, D, scale, in_dtype, acc_dtype, stream, true);
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
  if (D % 8 != 0 || D / 8 > 64 || ((D / 8) & (D / 8 - 1)) != 0)
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

}  // extern "C"
