"""Plain float64 definitions of every step on the hot path.

TEST INFRASTRUCTURE ONLY (see the package docstring): not imported by the
product package, and it imports nothing from it.

Each function is the definition written out with numpy; a matrix product is
the only library primitive used as a step.  Where the pages leave a step
open, the reading taken is stated in the function's docstring.

Tensor conventions (all row-major numpy arrays):
  Q          [B, Sq,  H, D]
  K, V       [B, Skv, H, D]
  O          [B, Sq,  H, D]
  LSE        [B, H, Sq]      natural log of sum_j exp(scale * q . k_j)
  send/recv  [U, n_planes, B, S_loc, H_loc, D]   peer-major exchange buffer
"""

from __future__ import annotations

import math

import numpy as np

F64 = np.float64
NEG_INF = -np.inf


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=F64)


# ---------------------------------------------------------------------------
# Attention with per-row log-sum-exp
# ---------------------------------------------------------------------------

def attention(q, k, v, scale: float, rows=None, row_group: int = 1024):
    """Exact non-causal attention and its per-row LSE.

    Follows edge-dit.cpp "Parallel execution", Ulysses section: after the
    sequence-to-head redistribution each rank evaluates the full softmax
    attention O = softmax(Q K^T / sqrt(D)) V for its heads, with no mask and
    no approximation.  The LSE output is what SGLang's "Parallelism
    Overview", "Constraints" section requires of a ring-capable kernel.

    For every (b, h, i):
        s_j   = scale * sum_d q[b,i,h,d] * k[b,j,h,d]
        m     = max_j s_j
        l     = sum_j exp(s_j - m)
        O     = (sum_j exp(s_j - m) * v[b,j,h,:]) / l
        LSE   = m + ln(l)
    Skv == 0: O = 0 and LSE = -inf (the identity of ``merge``).

    ``scale`` is the caller's value (a float32 in the library) promoted to
    float64.  ``rows`` optionally restricts the query rows evaluated (row
    outputs are independent, so a sample is exact for its rows); the returned
    arrays then hold only those rows, in the order given.  ``row_group`` only
    bounds memory: rows are evaluated group by group, each row's arithmetic
    unchanged.
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    if rows is not None:
        q = q[:, np.asarray(rows, dtype=np.int64)]
    B, Sq, H, D = q.shape
    Skv = k.shape[1]
    assert k.shape == (B, Skv, H, D) and v.shape == (B, Skv, H, D)
    scale = float(scale)
    o = np.zeros((B, Sq, H, D), dtype=F64)
    lse = np.full((B, H, Sq), NEG_INF, dtype=F64)
    if Skv == 0 or Sq == 0:
        return o, lse
    for b in range(B):
        for h in range(H):
            kh = k[b, :, h, :]
            vh = v[b, :, h, :]
            for r0 in range(0, Sq, row_group):
                r1 = min(Sq, r0 + row_group)
                s = scale * (q[b, r0:r1, h, :] @ kh.T)          # [rows, Skv]
                m = s.max(axis=1, keepdims=True)
                e = np.exp(s - m)
                l = e.sum(axis=1, keepdims=True)
                o[b, r0:r1, h, :] = (e @ vh) / l
                lse[b, h, r0:r1] = (m + np.log(l))[:, 0]
    return o, lse


# ---------------------------------------------------------------------------
# Online-softmax merge of partial results (ring hops)
# ---------------------------------------------------------------------------

def attention_kv_len(q, k, v, scale: float, kv_len, rows=None):
    """Attention of batch b over its first kv_len[b] keys only.

    SGLang "Parallelism Overview": the masked / tail-padded text path of
    joint text+image attention; xLLM "DiT Architecture and Capability
    Matrix": a replacement kernel preserves the padding exclusion.  Keys
    past the valid length do not take part (their scores count as -inf);
    a batch with no valid key gives the merge identity (O = 0, LSE = -inf).
    kv_len values are clamped to [0, Skv].
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Sq, H, D = q.shape
    Skv = k.shape[1]
    nr = Sq if rows is None else len(rows)
    o = np.zeros((B, nr, H, D))
    lse = np.full((B, H, nr), NEG_INF)
    for b in range(B):
        n = int(min(max(int(kv_len[b]), 0), Skv))
        if n == 0:
            continue
        ob, lb = attention(q[b:b + 1], k[b:b + 1, :n], v[b:b + 1, :n], scale, rows=rows)
        o[b], lse[b] = ob[0], lb[0]
    return o, lse


def merge(o_a, lse_a, o_c, lse_c):
    """Combine two partial attention results over disjoint key sets.

    SGLang "Parallelism Overview": the ring per-hop merge and the merge of
    replicated / tail-padded parts use the online-softmax rule with the
    kernel's LSE ("What happens to the shapes", "Constraints").

    With m = max(L_a, L_c) and w_x = exp(L_x - m):
        L = m + ln(w_a + w_c)
        O = (w_a O_a + w_c O_c) / (w_a + w_c)
    A part whose LSE is -inf holds no keys: its term is dropped (selected
    away, never multiplied), so whatever its O holds cannot leak.  If both
    are -inf the result is (0, -inf).
    """
    o_a = _f64(o_a)
    o_c = _f64(o_c)
    la = np.transpose(_f64(lse_a), (0, 2, 1))[..., None]   # [B,Sq,H,1]
    lc = np.transpose(_f64(lse_c), (0, 2, 1))[..., None]
    m = np.maximum(la, lc)
    empty = m == NEG_INF
    m_safe = np.where(empty, 0.0, m)
    with np.errstate(invalid="ignore", over="ignore"):
        wa = np.where(la == NEG_INF, 0.0, np.exp(la - m_safe))
        wc = np.where(lc == NEG_INF, 0.0, np.exp(lc - m_safe))
    wsum = wa + wc
    # select before multiplying: a dropped part contributes exactly 0
    num = wa * np.where(wa > 0, o_a, 0.0) + wc * np.where(wc > 0, o_c, 0.0)
    o = np.where(empty, 0.0, num / np.where(empty, 1.0, wsum))
    with np.errstate(divide="ignore"):
        lse = np.where(empty, NEG_INF, m_safe + np.log(np.where(empty, 1.0, wsum)))
    return o, np.transpose(lse[..., 0], (0, 2, 1)).copy()


def ring_hop_order(R: int, rank: int = 0):
    """Order in which ring rank ``rank`` sees the R key/value chunks.

    Reading (the pages say K/V rotate between neighbours but not which way):
    a rank first attends its own chunk, then the chunk of its previous
    neighbour, and so on -- chunk (rank - k) mod R at hop k.
    """
    return [(rank - t) % R for t in range(R)]


def ring_attention(q, k, v, scale: float, bounds, order=None):
    """Ring attention of one rank, with its hops run one after another.

    ``bounds`` = [b_0 = 0, b_1, ..., b_R = Skv]: chunk c holds keys
    [b_c, b_{c+1}) (chunks may be empty or uneven).  The result is the left
    fold of ``merge`` over the chunk results in ``order`` (default 0..R-1),
    as SGLang "Parallelism Overview" describes ring attention: Q stays put,
    each K/V hop yields a partial (O, LSE) that is merged into the running
    result.
    """
    R = len(bounds) - 1
    if order is None:
        order = list(range(R))
    k = _f64(k)
    v = _f64(v)
    acc = None
    for c in order:
        part = attention(q, k[:, bounds[c]:bounds[c + 1]], v[:, bounds[c]:bounds[c + 1]], scale)
        acc = part if acc is None else merge(acc[0], acc[1], part[0], part[1])
    return acc


# ---------------------------------------------------------------------------
# Ulysses all-to-all layout and the pack / unpack permutations
# ---------------------------------------------------------------------------

def a2a_layout(B, S, H, D, U, seq_align=1, n_planes=1):
    """Derived sizes of one Ulysses redistribution.

    edge-dit.cpp "Parallel execution": the sequence split records original,
    padded and local lengths; the all-to-all layout records global and local
    heads and sequence lengths, batch, head dim and elements per peer.

    Readings:
      * sequence padding (edge-dit: divisible or padded; xLLM "MiniMax-H3
        boundaries": padded to a multiple of lcm(SP, 64)):
        S_pad = ceil(S / lcm(U, seq_align)) * lcm(U, seq_align), S_loc = S_pad / U;
      * head padding (cache-dit "Any Head Num"): H_pad = ceil(H / U) * U,
        H_loc = H_pad / U; pad heads are the global indices >= H.
    """
    align = U * seq_align // math.gcd(U, seq_align)
    S_pad = -(-S // align) * align
    S_loc = S_pad // U
    H_pad = -(-H // U) * U
    H_loc = H_pad // U
    return dict(B=B, S=S, H=H, D=D, U=U, seq_align=seq_align, n_planes=n_planes,
                S_pad=S_pad, S_loc=S_loc, H_pad=H_pad, H_loc=H_loc,
                elems_per_peer=n_planes * B * S_loc * H_loc * D)


def _gather(src: np.ndarray, idx: np.ndarray, valid: np.ndarray) -> np.ndarray:
    flat = src.reshape(-1)
    out = np.zeros(idx.shape, dtype=src.dtype)
    out[valid] = flat[idx[valid]]
    return out


def pack_seq_to_head(in_planes, L, rank):
    """Sequence-to-head send buffer of Ulysses rank ``rank``.

    edge-dit.cpp packed QKV operator: the planes are concatenated, split by
    destination head group and flattened peer-major.  Reading of the order:
    send[p, pl, b, s, h', d] = in_pl[b, s, p*H_loc + h', d] when the global
    row rank*S_loc + s < S and the global head p*H_loc + h' < H, else 0.
    in_planes: n_planes arrays [B, S_loc, H, D] (rows past S never read).
    Written as a gather: the source flat index of every output element.
    """
    U, B, S, H, D = L["U"], L["B"], L["S"], L["H"], L["D"]
    S_loc, H_loc, n = L["S_loc"], L["H_loc"], L["n_planes"]
    assert len(in_planes) == n
    p, pl, b, s, hh, d = np.ix_(np.arange(U), np.arange(n), np.arange(B),
                                np.arange(S_loc), np.arange(H_loc), np.arange(D))
    head = p * H_loc + hh
    valid = (rank * S_loc + s < S) & (head < H)
    src_idx = (((pl * B + b) * S_loc + s) * H + head) * D + d
    shape = (U, n, B, S_loc, H_loc, D)
    valid = np.broadcast_to(valid, shape)
    src_idx = np.broadcast_to(src_idx, shape)
    stacked = np.stack([np.asarray(x).reshape(B, S_loc, H, D) for x in in_planes])
    return _gather(stacked, np.where(valid, src_idx, 0), valid)


def unpack_seq_to_head(recv, L, rank):
    """Head-sharded full-sequence planes from a sequence-to-head receive buffer.

    edge-dit.cpp receive preparation (without RoPE): the rank-major receive
    buffer is decoded into one [B, S, H_loc, D] tensor per plane:
    out_pl[b, t, h', d] = recv[t // S_loc, pl, b, t mod S_loc, h', d] for the
    S real rows t < S.  Pad rows are dropped here, so attention sees exactly
    the real keys (xLLM: padding exclusion).  ``rank`` does not enter the map.
    """
    U, B, S, D = L["U"], L["B"], L["S"], L["D"]
    S_loc, H_loc, n = L["S_loc"], L["H_loc"], L["n_planes"]
    pl, b, t, hh, d = np.ix_(np.arange(n), np.arange(B), np.arange(S),
                             np.arange(H_loc), np.arange(D))
    src_idx = (((((t // S_loc) * n + pl) * B + b) * S_loc + t % S_loc) * H_loc + hh) * D + d
    shape = (n, B, S, H_loc, D)
    src_idx = np.broadcast_to(src_idx, shape)
    out = _gather(np.asarray(recv), src_idx, np.ones(shape, dtype=bool))
    return [out[i] for i in range(n)]


def rope(x, cos, sin):
    """Rotary position embedding of a [B, S, H, D] tensor.

    edge-dit.cpp "Parallel execution" (receive preparation) applies RoPE to
    Q and K; the pages do not fix its convention.  Reading: the RoFormer
    rotation of adjacent head-dim pairs (2i, 2i+1) by the angle of sequence
    position t and pair i, given as tables cos, sin of shape [S, D/2]:
      y[.., t, .., 2i]   = x[.., 2i] cos[t, i] - x[.., 2i+1] sin[t, i]
      y[.., t, .., 2i+1] = x[.., 2i] sin[t, i] + x[.., 2i+1] cos[t, i]
    """
    x = _f64(x)
    c = _f64(cos)[None, :, None, :]
    s = _f64(sin)[None, :, None, :]
    x0, x1 = x[..., 0::2], x[..., 1::2]
    y = np.empty_like(x)
    y[..., 0::2] = x0 * c - x1 * s
    y[..., 1::2] = x0 * s + x1 * c
    return y


def unpack_seq_to_head_rope(recv, L, rank, cos, sin):
    """The fused receive preparation: the sequence-to-head unpack of the
    packed Q, K, V buffer (n_planes = 3) followed by RoPE on planes 0 (Q)
    and 1 (K) at their global sequence positions; V unchanged."""
    assert L["n_planes"] == 3
    q, k, v = unpack_seq_to_head(recv, L, rank)
    return [rope(q, cos, sin), rope(k, cos, sin), _f64(v)]


def pack_head_to_seq(in_planes, L, rank):
    """Head-to-sequence send buffer of Ulysses rank ``rank``.

    edge-dit.cpp packed head-to-sequence operator: the head-sharded output
    is split by destination sequence shard and flattened peer-major:
    send[p, pl, b, s, h', d] = in_pl[b, p*S_loc + s, h', d] when
    p*S_loc + s < S and rank*H_loc + h' < H, else 0.
    in_planes: n_planes arrays [B, S, H_loc, D].
    """
    U, B, S, H, D = L["U"], L["B"], L["S"], L["H"], L["D"]
    S_loc, H_loc, n = L["S_loc"], L["H_loc"], L["n_planes"]
    assert len(in_planes) == n
    p, pl, b, s, hh, d = np.ix_(np.arange(U), np.arange(n), np.arange(B),
                                np.arange(S_loc), np.arange(H_loc), np.arange(D))
    row = p * S_loc + s
    valid = (row < S) & (rank * H_loc + hh < H)
    src_idx = (((pl * B + b) * S + row) * H_loc + hh) * D + d
    shape = (U, n, B, S_loc, H_loc, D)
    valid = np.broadcast_to(valid, shape)
    src_idx = np.broadcast_to(src_idx, shape)
    stacked = np.stack([np.asarray(x).reshape(B, S, H_loc, D) for x in in_planes])
    return _gather(stacked, np.where(valid, src_idx, 0), valid)


def unpack_head_to_seq(recv, L, rank):
    """Sequence-sharded planes from a head-to-sequence receive buffer.

    edge-dit.cpp receive-side unpack of the head-to-sequence path:
    out_pl[b, s, h, d] = recv[h // H_loc, pl, b, s, h mod H_loc, d] for the
    H real heads (pad heads dropped); local rows whose global index
    rank*S_loc + s >= S are pad rows and are written as 0.
    Output: n_planes arrays [B, S_loc, H, D].
    """
    U, B, S, H, D = L["U"], L["B"], L["S"], L["H"], L["D"]
    S_loc, H_loc, n = L["S_loc"], L["H_loc"], L["n_planes"]
    pl, b, s, h, d = np.ix_(np.arange(n), np.arange(B), np.arange(S_loc),
                            np.arange(H), np.arange(D))
    src_idx = (((((h // H_loc) * n + pl) * B + b) * S_loc + s) * H_loc + h % H_loc) * D + d
    valid = rank * S_loc + s < S
    shape = (n, B, S_loc, H, D)
    valid = np.broadcast_to(valid, shape)
    src_idx = np.broadcast_to(src_idx, shape)
    out = _gather(np.asarray(recv), np.where(valid, src_idx, 0), valid)
    return [out[i] for i in range(n)]


# -- padding-free (uneven) splits ------------------------------------------------
#
# cache-dit "Context Parallelism" (Ulysses Anything Attention): arbitrary
# sequence lengths without padding, each rank's length gathered from the
# others; arbitrary head counts without padding (the no-pad variant).
# Reading: rank r holds the contiguous rows [so[r], so[r] + S_r) of the
# sequence and, inside attention, the contiguous heads [ho[r], ho[r] + H_r),
# with so / ho the prefix sums of the per-rank counts.  The exchange buffer
# is the concatenation, in peer order, of one chunk per peer (an all-to-all
# with per-peer split sizes); each chunk is [n_planes, B, rows, heads, D].


def _prefix(counts):
    return np.concatenate([[0], np.cumsum(np.asarray(counts, dtype=np.int64))])


def pack_seq_to_head_uneven(in_planes, seq_counts, head_counts, rank):
    """Send buffer (1-D) of rank ``rank``: chunk p = in_pl[:, :, ho[p]:ho[p]+H_p]
    for every plane; in_planes: n arrays [B, S_rank, H, D]."""
    ho = _prefix(head_counts)
    x = np.stack([np.asarray(t) for t in in_planes])          # [n, B, S_r, H, D]
    assert x.shape[2] == seq_counts[rank] and x.shape[3] == ho[-1]
    chunks = [x[:, :, :, ho[p]:ho[p + 1]].reshape(-1) for p in range(len(head_counts))]
    return np.concatenate(chunks) if chunks else np.zeros(0, x.dtype)


def unpack_seq_to_head_uneven(recv, B, D, n_planes, seq_counts, head_counts, rank):
    """Planes [B, S, H_rank, D] from the receive buffer: the chunk from source
    p holds rows [so[p], so[p] + S_p) of this rank's heads."""
    H_r = head_counts[rank]
    parts, off = [], 0
    for p, S_p in enumerate(seq_counts):
        size = n_planes * B * S_p * H_r * D
        parts.append(np.asarray(recv)[off:off + size].reshape(n_planes, B, S_p, H_r, D))
        off += size
    assert off == np.asarray(recv).size
    x = np.concatenate(parts, axis=2)                          # [n, B, S, H_r, D]
    return [x[i] for i in range(n_planes)]


def pack_head_to_seq_uneven(in_planes, seq_counts, head_counts, rank):
    """Send buffer (1-D) of rank ``rank``: chunk p = rows [so[p], so[p] + S_p)
    of every plane; in_planes: n arrays [B, S, H_rank, D]."""
    so = _prefix(seq_counts)
    x = np.stack([np.asarray(t) for t in in_planes])          # [n, B, S, H_r, D]
    assert x.shape[2] == so[-1] and x.shape[3] == head_counts[rank]
    chunks = [x[:, :, so[p]:so[p + 1]].reshape(-1) for p in range(len(seq_counts))]
    return np.concatenate(chunks) if chunks else np.zeros(0, x.dtype)


def unpack_head_to_seq_uneven(recv, B, D, n_planes, seq_counts, head_counts, rank):
    """Planes [B, S_rank, H, D] from the receive buffer: the chunk from source
    p holds heads [ho[p], ho[p] + H_p) of this rank's rows."""
    S_r = seq_counts[rank]
    parts, off = [], 0
    for p, H_p in enumerate(head_counts):
        size = n_planes * B * S_r * H_p * D
        parts.append(np.asarray(recv)[off:off + size].reshape(n_planes, B, S_r, H_p, D))
        off += size
    assert off == np.asarray(recv).size
    x = np.concatenate(parts, axis=3)                          # [n, B, S_r, H, D]
    return [x[i] for i in range(n_planes)]


def uneven_chunk_sizes(B, D, n_planes, seq_counts, head_counts, rank, seq_to_head=True):
    """Elements rank ``rank`` sends to / receives from each peer."""
    U = len(seq_counts)
    if seq_to_head:
        send = [n_planes * B * seq_counts[rank] * head_counts[p] * D for p in range(U)]
        recv = [n_planes * B * seq_counts[p] * head_counts[rank] * D for p in range(U)]
    else:
        send = [n_planes * B * seq_counts[p] * head_counts[rank] * D for p in range(U)]
        recv = [n_planes * B * seq_counts[rank] * head_counts[p] * D for p in range(U)]
    return send, recv


def all_to_all_uneven(sends, send_sizes):
    """The exchange with per-peer split sizes (a test helper):
    recv_r = concat over p of the part of send_p addressed to r."""
    U = len(sends)
    out = []
    for r in range(U):
        parts = []
        for p in range(U):
            off = int(sum(send_sizes[p][:r]))
            parts.append(np.asarray(sends[p])[off:off + send_sizes[p][r]])
        out.append(np.concatenate(parts))
    return out


# -- Ring Anything: equal-size gather of uneven shards ----------------------------
#
# diffusers "Distributed inference" (Ring Anything Attention): each rank pads
# its local K/V rows up to the largest rank's length, the padded buffers are
# all-gathered, and the result is cut back to every rank's real length before
# attention.  Reading: pad rows are zeros and sit after a rank's real rows
# (per batch); the gathered buffer is rank-major [U, n, B, S_max, H, D].


def ring_anything_pad(in_planes, S_max):
    """[n, B, S_max, H, D] from n planes [B, S_r, H, D]; rows >= S_r are zero."""
    x = np.stack([np.asarray(t) for t in in_planes])
    n, B, S_r, H, D = x.shape
    assert S_r <= S_max
    out = np.zeros((n, B, S_max, H, D), dtype=x.dtype)
    out[:, :, :S_r] = x
    return out


def ring_anything_trim(gathered, seq_counts):
    """n planes [B, S, H, D] (S = sum of the counts) from the gathered buffer
    [U, n, B, S_max, H, D]: rank p's first S_p rows, in rank order."""
    g = np.asarray(gathered)
    assert g.shape[0] == len(seq_counts) and max(seq_counts, default=0) <= g.shape[3]
    x = np.concatenate([g[p, :, :, :seq_counts[p]] for p in range(len(seq_counts))], axis=2)
    return [x[i] for i in range(x.shape[0])]


# -- FP8 Ulysses ------------------------------------------------------------------
#
# cache-dit "Context Parallelism" (Async FP8 Ulysses Attention): the
# all-to-alls of Q, V and O move FP8 data, while K stays in 16-bit because
# the softmax of Q K^T is sensitive to its precision.  The pages fix neither
# the FP8 format nor the scaling.  Readings taken:
#   * format: OCP 8-bit floating point E4M3 ("FN": bias 7, no infinities,
#     largest finite 448, code 0x7F / 0xFF is NaN, subnormals m/8 * 2^-6);
#   * scaling: one power-of-two scale per block of 32 consecutive elements
#     of a head vector (the block size and E8M0 scale byte of the OCP
#     Microscaling (MX) format), with the exponent chosen so that the block's
#     largest magnitude fits: k = the smallest integer with
#     amax <= 448 * 2^k, clamped to [-117, 126]; the scale byte is k + 127;
#   * encoding: y = x * 2^-k (exact), code = y rounded to the nearest E4M3
#     value, ties to the even code (mantissa LSB 0), sign kept (also of
#     zero); decoding: value(code) * 2^k (exact in bf16 for k >= -117).


E4M3_MAX = 448.0
FP8_BLOCK = 32
K_MIN, K_MAX = -117, 126


def e4m3_value(code):
    """Value of E4M3 codes (uint8 array) in float64; NaN for 0x7F / 0xFF."""
    c = np.asarray(code).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


_E4M3_POS = e4m3_value(np.arange(0x7F))   # the 127 finite non-negative values, increasing


def e4m3_encode(y):
    """Codes of float64 values |y| <= 448: round to nearest, ties to even."""
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    assert np.all(a <= E4M3_MAX), "values beyond the largest finite E4M3 magnitude"
    hi = np.clip(np.searchsorted(_E4M3_POS, a, side="left"), 0, 0x7E)   # first value >= a
    lo = np.clip(hi - 1, 0, 0x7E)
    d_hi = _E4M3_POS[hi] - a
    d_lo = a - _E4M3_POS[lo]
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & (lo % 2 == 0))
    code = np.where(pick_lo, lo, hi).astype(np.int64)
    code = np.where(np.signbit(y), code | 0x80, code)
    return code.astype(np.uint8)


def fp8_scale_exp(amax):
    """Smallest integer k with amax <= 448 * 2^k, clamped to [K_MIN, K_MAX]."""
    amax = np.asarray(amax, dtype=np.float64)
    m, e = np.frexp(amax)                      # amax = m * 2^e, m in [0.5, 1)
    # 448 * 2^(e-9) = 0.875 * 2^e: fits when m <= 0.875, else one more
    k = np.where(m <= 0.875, e - 9, e - 8)
    k = np.where(amax == 0, K_MIN, k)
    return np.clip(k, K_MIN, K_MAX).astype(np.int64)


def quantize_fp8_blocks(x):
    """(codes uint8 [..., D], scale bytes uint8 [..., D/32]) of float64 x [..., D]."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    assert D % FP8_BLOCK == 0
    blocks = x.reshape(x.shape[:-1] + (D // FP8_BLOCK, FP8_BLOCK))
    k = fp8_scale_exp(np.max(np.abs(blocks), axis=-1))
    y = blocks * np.exp2(-k.astype(np.float64))[..., None]
    codes = e4m3_encode(y).reshape(x.shape)
    return codes, (k + 127).astype(np.uint8)


def dequantize_fp8_blocks(codes, scale_bytes):
    """float64 values of block-scaled E4M3 codes [..., D]."""
    codes = np.asarray(codes)
    D = codes.shape[-1]
    k = np.asarray(scale_bytes).astype(np.int64) - 127
    v = e4m3_value(codes).reshape(codes.shape[:-1] + (D // FP8_BLOCK, FP8_BLOCK))
    return (v * np.exp2(k.astype(np.float64))[..., None]).reshape(codes.shape)


def bf16_bits_to_f64(bits):
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits_exact(x):
    """bf16 bit patterns of values that bf16 represents exactly (asserted)."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    assert np.array_equal(f.astype(np.float64), np.asarray(x, dtype=np.float64), equal_nan=True)
    u = f.view(np.uint32)
    assert not np.any(u & 0xFFFF), "not a bf16 value"
    return (u >> 16).astype(np.uint16).view(np.int16)


def fp8_chunk_sections(L, seq_to_head):
    """Byte offsets of the sections of one peer's chunk and the chunk stride.

    Sequence to head (planes Q, K, V): Q codes, V codes, K (bf16), Q scale
    bytes, V scale bytes.  Head to sequence (plane O): O codes, O scale
    bytes.  E = B * S_loc * H_loc * D elements per plane; the stride rounds
    the chunk up to a multiple of 256 bytes, the tail bytes being zero.
    """
    E = L["B"] * L["S_loc"] * L["H_loc"] * L["D"]
    if seq_to_head:
        sec = dict(q=0, v=E, k=2 * E, q_scale=4 * E, v_scale=4 * E + E // 32)
        used = 4 * E + E // 16
    else:
        sec = dict(o=0, o_scale=E)
        used = E + E // 32
    stride = -(-used // 256) * 256
    return sec, used, stride


def pack_seq_to_head_fp8(q_bits, k_bits, v_bits, L, rank):
    """FP8 sequence-to-head send buffer (uint8 [U, stride]) of rank ``rank``:
    the padded pack of each plane (pad rows / heads zero), Q and V encoded
    by block, K kept as bf16 bit patterns.  Inputs: bf16 bits [B, S_loc, H, D]."""
    assert L["D"] % FP8_BLOCK == 0
    L1 = dict(L, n_planes=1)
    sec, used, stride = fp8_chunk_sections(L, True)
    U, E = L["U"], L["B"] * L["S_loc"] * L["H_loc"] * L["D"]
    out = np.zeros((U, stride), dtype=np.uint8)
    planes = {}
    for name, t in (("q", q_bits), ("k", k_bits), ("v", v_bits)):
        planes[name] = pack_seq_to_head([t], L1, rank).reshape(U, E)      # bf16 bits
    for p in range(U):
        for name in ("q", "v"):
            codes, sbytes = quantize_fp8_blocks(bf16_bits_to_f64(planes[name][p]).reshape(-1, L["D"]))
            out[p, sec[name]:sec[name] + E] = codes.reshape(-1)
            out[p, sec[name + "_scale"]:sec[name + "_scale"] + E // 32] = sbytes.reshape(-1)
        out[p, sec["k"]:sec["k"] + 2 * E] = planes["k"][p].astype(np.int16).view(np.uint8)
    return out


def unpack_seq_to_head_fp8(recv, L, rank):
    """[Q, K, V] bf16 bits [B, S, H_loc, D] from an FP8 sequence-to-head
    receive buffer (uint8 [U, stride], chunk p from source p): Q and V
    decoded, K copied; pad rows dropped as in the 16-bit map."""
    sec, used, stride = fp8_chunk_sections(L, True)
    U, E, D = L["U"], L["B"] * L["S_loc"] * L["H_loc"] * L["D"], L["D"]
    recv = np.asarray(recv, dtype=np.uint8).reshape(U, stride)
    L1 = dict(L, n_planes=1)
    res = {}
    for name in ("q", "v"):
        chunks = []
        for p in range(U):
            codes = recv[p, sec[name]:sec[name] + E].reshape(-1, D)
            sb = recv[p, sec[name + "_scale"]:sec[name + "_scale"] + E // 32].reshape(-1, D // 32)
            chunks.append(f64_to_bf16_bits_exact(dequantize_fp8_blocks(codes, sb)).reshape(-1))
        res[name] = unpack_seq_to_head(np.stack(chunks).reshape(-1), L1, rank)[0]
    kk = np.ascontiguousarray(recv[:, sec["k"]:sec["k"] + 2 * E]).view(np.int16).reshape(-1)
    res["k"] = unpack_seq_to_head(kk, L1, rank)[0]
    return [res["q"], res["k"], res["v"]]


def pack_head_to_seq_fp8(o_bits, L, rank):
    """FP8 head-to-sequence send buffer (uint8 [U, stride]) of the attention
    output O (bf16 bits [B, S, H_loc, D]): the padded pack, encoded by block."""
    sec, used, stride = fp8_chunk_sections(L, False)
    U, E, D = L["U"], L["B"] * L["S_loc"] * L["H_loc"] * L["D"], L["D"]
    packed = pack_head_to_seq([o_bits], dict(L, n_planes=1), rank).reshape(U, E)
    out = np.zeros((U, stride), dtype=np.uint8)
    for p in range(U):
        codes, sb = quantize_fp8_blocks(bf16_bits_to_f64(packed[p]).reshape(-1, D))
        out[p, :E] = codes.reshape(-1)
        out[p, sec["o_scale"]:sec["o_scale"] + E // 32] = sb.reshape(-1)
    return out


def unpack_head_to_seq_fp8(recv, L, rank):
    """O bf16 bits [B, S_loc, H, D] from an FP8 head-to-sequence receive
    buffer: decoded, pad heads dropped, this rank's pad rows zero."""
    sec, used, stride = fp8_chunk_sections(L, False)
    U, E, D = L["U"], L["B"] * L["S_loc"] * L["H_loc"] * L["D"], L["D"]
    recv = np.asarray(recv, dtype=np.uint8).reshape(U, stride)
    chunks = []
    for p in range(U):
        codes = recv[p, :E].reshape(-1, D)
        sb = recv[p, sec["o_scale"]:sec["o_scale"] + E // 32].reshape(-1, D // 32)
        chunks.append(f64_to_bf16_bits_exact(dequantize_fp8_blocks(codes, sb)).reshape(-1))
    return unpack_head_to_seq(np.stack(chunks).reshape(-1), dict(L, n_planes=1), rank)[0]


def all_to_all(sends):
    """The exchange itself (a test helper; the library never performs it).

    recv_r[p] = send_p[r]: the chunk rank p addressed to rank r.  SGLang
    "The Ulysses transport": an all-to-all only permutes data.
    """
    U = len(sends)
    return [np.stack([sends[p][r] for p in range(U)]) for r in range(U)]


# ---------------------------------------------------------------------------
# Classifier-free guidance combine
# ---------------------------------------------------------------------------

def cfg_combine(u, c, g: float):
    """edge-dit.cpp "Parallel execution", CFG section: the guided prediction
    is p_uncond + g * (p_cond - p_uncond); evaluated here in float64."""
    u = _f64(u)
    c = _f64(c)
    return u + float(g) * (c - u)


def fmaf(a, b, c):
    """Correctly rounded float32 fused multiply-add of float32 arrays.

    a*b is exact in float64 (24 + 24 significant bits).  The float64 sum is
    formed with rounding to odd -- round to nearest, then, when the TwoSum
    error (Knuth) is non-zero and the last significand bit is even, step one
    ulp toward the error -- and the result rounded once more to float32.
    Boldo and Melquiond (IEEE Trans. Computers, 2008) prove that this double
    rounding equals a single rounding of the exact a*b + c when the
    intermediate format has at least 2p + 2 bits (53 >= 2*24 + 2).
    """
    a = np.asarray(a, dtype=np.float32).astype(F64)
    b = np.asarray(b, dtype=np.float32).astype(F64)
    c = np.asarray(c, dtype=np.float32).astype(F64)
    p = a * b
    s = p + c
    bb = s - p
    err = (p - (s - bb)) + (c - bb)
    even = (s.view(np.int64) & 1) == 0
    fix = (err != 0) & even & np.isfinite(s)
    toward = np.where(err > 0, np.inf, -np.inf)
    s = np.where(fix, np.nextafter(s, toward), s)
    return s.astype(np.float32)


def cfg_combine_f32(u, c, g: float):
    """The float32 evaluation the library performs: d = fl32(c - u), then one
    fused multiply-add g*d + u, rounded once (the same formula as
    ``cfg_combine``, at float32)."""
    u = np.asarray(u, dtype=np.float32)
    c = np.asarray(c, dtype=np.float32)
    d = (c - u).astype(np.float32)
    return fmaf(np.float32(g), d, u)


# ---------------------------------------------------------------------------
# Packing with a conversion to a 16-bit exchange type
# ---------------------------------------------------------------------------
#
# edge-dit.cpp "Parallel execution": the packed QKV operator may convert F32
# input to F16 on the way into the send buffer, and the head-to-sequence
# path may produce F16 or BF16 output directly.  Readings: the conversion is
# IEEE 754 rounding to nearest with ties to even, overflow going to
# infinity, subnormal results kept (no flush to zero), NaN staying NaN (its
# sign and payload unspecified); BF16 is served as well as F16; pad
# positions of the send buffer are +0.
#
# The formats, from their definitions (sign, biased exponent, fraction):
#   F16  -- 1 + 5 + 10 bits, bias 15:  codes 0x7C00 inf, 0x7C01.. NaN
#   BF16 -- 1 + 8 +  7 bits, bias 127: codes 0x7F80 inf, 0x7F81.. NaN

HALF_FORMATS = {"f16": (5, 10), "bf16": (8, 7)}   # exponent bits, fraction bits


def half_value(code, fmt):
    """float64 value of 16-bit codes of format ``fmt`` ("f16" or "bf16")."""
    e_bits, f_bits = HALF_FORMATS[fmt]
    c = np.asarray(code).astype(np.int64) & 0xFFFF
    bias = (1 << (e_bits - 1)) - 1
    e_all = (1 << e_bits) - 1
    sign = np.where(c >> 15, -1.0, 1.0)
    e = (c >> f_bits) & e_all
    f = (c & ((1 << f_bits) - 1)).astype(np.float64)
    mag = np.where(e == 0, f * 2.0 ** (1 - bias - f_bits),
                   (1.0 + f * 2.0 ** -f_bits) * 2.0 ** (e.astype(np.float64) - bias))
    mag = np.where(e == e_all, np.where(f == 0, np.inf, np.nan), mag)
    return sign * mag


def _half_ladder(fmt):
    """Values of the non-negative codes 0 .. inf, increasing with the code;
    the infinity code stands at the value the next binade would start at, so
    that overflow follows the same nearest / ties-to-even rule."""
    e_bits, f_bits = HALF_FORMATS[fmt]
    inf_code = ((1 << e_bits) - 1) << f_bits
    v = half_value(np.arange(inf_code + 1), fmt)
    bias = (1 << (e_bits - 1)) - 1
    v[inf_code] = 2.0 ** (bias + 1)
    return v, inf_code


def round_to_half(x, fmt):
    """uint16 codes of float64 values in format ``fmt``: the nearest code,
    ties to the code whose last fraction bit is 0; magnitudes at or past the
    midpoint between the largest finite value and 2^(emax+1) give infinity;
    NaN gives the quiet NaN with only the top fraction bit set."""
    ladder, inf_code = _half_ladder(fmt)
    _, f_bits = HALF_FORMATS[fmt]
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    nan = np.isnan(a)
    a = np.where(nan, 0.0, a)
    hi = np.clip(np.searchsorted(ladder, a, side="left"), 0, inf_code)   # first value >= a
    lo = np.clip(hi - 1, 0, inf_code)
    d_hi = ladder[hi] - a
    d_lo = a - ladder[lo]
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & (lo % 2 == 0))
    code = np.where(pick_lo, lo, hi)
    code = np.where(np.isinf(a), inf_code, code)
    code = np.where(np.signbit(x), code | 0x8000, code)
    code = np.where(nan, inf_code | (1 << (f_bits - 1)), code)
    return code.astype(np.uint16)


def half_is_nan(code, fmt):
    e_bits, f_bits = HALF_FORMATS[fmt]
    c = np.asarray(code).astype(np.int64) & 0x7FFF
    return c > (((1 << e_bits) - 1) << f_bits)


def pack_seq_to_head_convert(in_planes, L, rank, fmt):
    """The sequence-to-head send buffer of ``pack_seq_to_head`` over float32
    planes, each element rounded to ``fmt`` (uint16 codes; pad elements +0)."""
    return round_to_half(pack_seq_to_head(in_planes, L, rank), fmt)


def pack_head_to_seq_convert(in_planes, L, rank, fmt):
    """The head-to-sequence send buffer of ``pack_head_to_seq`` over float32
    planes, each element rounded to ``fmt`` (uint16 codes; pad elements +0)."""
    return round_to_half(pack_head_to_seq(in_planes, L, rank), fmt)
