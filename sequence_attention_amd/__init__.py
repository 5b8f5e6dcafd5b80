"""Per-GPU hot path of sequence-parallel DiT attention on MI355X (gfx950).

Thin Python binding over libdit_attn.so.  Every function has the name of the
C entry point it wraps (include/dit_attn.h) and only marshals arguments:
torch supplies device memory and the current HIP stream, all computation
runs in the library's HIP kernels.  There is no CPU or PyTorch fallback: if
the library is missing, or a tensor is not on the GPU, the call raises.

    o, lse = dit_attn_fwd(q, k, v)                      # [B,S,H,D] bf16 / fp32
                                                        # (via dit_attn_fwd_ws)
    dit_attn_merge(o_acc, lse_acc, o_part, lse_part)    # in place
    L = dit_a2a_layout_init(B, S, H, D, U, n_planes=3)
    send = dit_ulysses_pack(L, DIT_SEQ_TO_HEAD, rank, [q, k, v])
    q, k, v = dit_ulysses_unpack(L, DIT_SEQ_TO_HEAD, rank, recv)
    out = dit_cfg_combine(p_uncond, p_cond, g)
"""

from __future__ import annotations

import ctypes
import math

from ._lib import (  # noqa: F401
    DIT_BF16, DIT_F16, DIT_F32, DIT_HEAD_TO_SEQ, DIT_OK, DIT_SEQ_TO_HEAD,
    DIT_ERR_HIP, DIT_ERR_INVALID_ARGUMENT, DIT_ERR_UNSUPPORTED,
    DitA2ALayout, DitA2AUnevenLayout, DitError, EXPORTS, LIB_PATH, check, lib,
)

__all__ = [
    "dit_abi_version", "dit_a2a_layout_init", "dit_ulysses_pack", "dit_ulysses_pack_convert",
    "dit_ulysses_unpack",
    "dit_ulysses_unpack_rope",
    "dit_a2a_uneven_init", "dit_a2a_uneven_sizes", "dit_ulysses_pack_uneven",
    "dit_ulysses_unpack_uneven", "dit_ring_anything_pad", "dit_ring_anything_trim",
    "DitA2AUnevenLayout",
    "dit_a2a_fp8_bytes_per_peer", "dit_ulysses_pack_fp8", "dit_ulysses_unpack_fp8",
    "dit_attn_fwd", "dit_attn_fwd_ws", "dit_attn_fwd_send", "dit_attn_fwd_a2a", "dit_attn_fwd_noalloc", "dit_attn_workspace_size", "dit_attn_fwd_kvlen", "dit_attn_merge",
    "dit_attn_fwd_merge", "dit_cfg_combine", "dit_clock_probe", "DitA2ALayout", "DitError",
    "DIT_BF16", "DIT_F16", "DIT_F32", "DIT_SEQ_TO_HEAD", "DIT_HEAD_TO_SEQ",
]


def _torch():
    import torch
    return torch


def _dtype_code(dt) -> int:
    torch = _torch()
    if dt == torch.bfloat16:
        return DIT_BF16
    if dt == torch.float16:
        return DIT_F16
    if dt == torch.float32:
        return DIT_F32
    raise TypeError(f"unsupported tensor dtype {dt}")


def _torch_dtype(code: int):
    torch = _torch()
    return {DIT_BF16: torch.bfloat16, DIT_F16: torch.float16, DIT_F32: torch.float32}[code]


def _dev(t, name: str):
    """Device pointer of a contiguous GPU tensor."""
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _expect(t, name: str, numel: int, dtype, device=None):
    """The library cannot see buffer sizes: check a caller-supplied tensor's
    dtype, element count and device against what the call will touch."""
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if t.numel() != numel:
        raise ValueError(f"{name}: {t.numel()} elements, expected {numel}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device} (one device per call)")


def _expect_all(ts, name: str, numel: int, dtype, device=None):
    for i, t in enumerate(ts):
        _expect(t, f"{name}[{i}]", numel, dtype, device)


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(_torch().cuda.current_stream().cuda_stream)
    if hasattr(stream, "cuda_stream"):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def dit_abi_version() -> int:
    return lib().dit_abi_version()


def dit_a2a_layout_init(B, S, H, D, U, seq_align=1, n_planes=1, dtype=DIT_BF16) -> DitA2ALayout:
    """Derived sizes of one Ulysses redistribution (host only)."""
    if not isinstance(dtype, int):
        dtype = _dtype_code(dtype)
    L = DitA2ALayout()
    check(lib().dit_a2a_layout_init(B, S, H, D, U, seq_align, n_planes, dtype, ctypes.byref(L)),
          "dit_a2a_layout_init")
    return L


def _send_shape(L):
    return (L.U, L.n_planes, L.B, L.S_loc, L.H_loc, L.D)


def _plane_numel(L, direction, pack):
    """Elements of one plane on the non-buffer side of a padded map."""
    seq_shard = L.B * L.S_loc * L.H * L.D       # [B, S_loc, H, D]
    head_shard = L.B * L.S * L.H_loc * L.D      # [B, S, H_loc, D]
    if direction == DIT_SEQ_TO_HEAD:
        return seq_shard if pack else head_shard
    return head_shard if pack else seq_shard


def dit_ulysses_pack(layout: DitA2ALayout, direction: int, rank: int, planes, send=None,
                     stream=None):
    """Pack rank `rank`'s planes into a peer-major send buffer
    [U, n_planes, B, S_loc, H_loc, D] (allocated if `send` is None)."""
    torch = _torch()
    planes = list(planes)
    if len(planes) != layout.n_planes:
        raise ValueError(f"expected {layout.n_planes} planes, got {len(planes)}")
    dt, dev = _torch_dtype(layout.dtype), planes[0].device
    _expect_all(planes, "planes", _plane_numel(layout, direction, True), dt, dev)
    if send is None:
        send = torch.empty(_send_shape(layout), dtype=dt, device=dev)
    _expect(send, "send", layout.U * layout.elems_per_peer, dt, dev)
    arr = (ctypes.c_void_p * 3)(*[_dev(p, f"planes[{i}]") for i, p in enumerate(planes)])
    check(lib().dit_ulysses_pack(ctypes.byref(layout), direction, rank, arr, _dev(send, "send"),
                                 _stream(stream)), "dit_ulysses_pack")
    return send


def dit_ulysses_pack_convert(layout: DitA2ALayout, direction: int, rank: int, planes, send=None,
                             stream=None):
    """Pack float32 planes into a send buffer of the layout's 16-bit dtype
    (bf16 or f16), rounding each element to nearest, ties to even; the maps
    are those of dit_ulysses_pack."""
    torch = _torch()
    planes = list(planes)
    if len(planes) != layout.n_planes:
        raise ValueError(f"expected {layout.n_planes} planes, got {len(planes)}")
    if layout.dtype not in (DIT_BF16, DIT_F16):
        raise ValueError("the converting pack writes a bf16 or f16 send buffer")
    dt, dev = _torch_dtype(layout.dtype), planes[0].device
    _expect_all(planes, "planes", _plane_numel(layout, direction, True), torch.float32, dev)
    if send is None:
        send = torch.empty(_send_shape(layout), dtype=dt, device=dev)
    _expect(send, "send", layout.U * layout.elems_per_peer, dt, dev)
    arr = (ctypes.c_void_p * 3)(*[_dev(p, f"planes[{i}]") for i, p in enumerate(planes)])
    check(lib().dit_ulysses_pack_convert(ctypes.byref(layout), direction, rank, arr,
                                         _dev(send, "send"), _stream(stream)),
          "dit_ulysses_pack_convert")
    return send


def dit_ulysses_unpack(layout: DitA2ALayout, direction: int, rank: int, recv, out=None,
                       stream=None):
    """Unpack a receive buffer into n_planes tensors: [B, S, H_loc, D] for
    DIT_SEQ_TO_HEAD, [B, S_loc, H, D] for DIT_HEAD_TO_SEQ."""
    torch = _torch()
    dt = _torch_dtype(layout.dtype)
    _expect(recv, "recv", layout.U * layout.elems_per_peer, dt)
    if out is None:
        shape = ((layout.B, layout.S, layout.H_loc, layout.D) if direction == DIT_SEQ_TO_HEAD
                 else (layout.B, layout.S_loc, layout.H, layout.D))
        out = [torch.empty(shape, dtype=dt, device=recv.device) for _ in range(layout.n_planes)]
    out = list(out)
    if len(out) != layout.n_planes:
        raise ValueError(f"expected {layout.n_planes} output planes, got {len(out)}")
    _expect_all(out, "out", _plane_numel(layout, direction, False), dt, recv.device)
    arr = (ctypes.c_void_p * 3)(*[_dev(p, f"out[{i}]") for i, p in enumerate(out)])
    check(lib().dit_ulysses_unpack(ctypes.byref(layout), direction, rank, _dev(recv, "recv"), arr,
                                   _stream(stream)), "dit_ulysses_unpack")
    return out


def dit_ulysses_unpack_rope(layout: DitA2ALayout, rank: int, recv, rope_cos, rope_sin, out=None,
                            stream=None):
    """Sequence-to-head unpack of the packed Q, K, V receive buffer with RoPE
    applied to Q and K (tables [S, D/2] fp32); returns [q, k, v], each
    [B, S, H_loc, D]."""
    torch = _torch()
    dt = _torch_dtype(layout.dtype)
    _expect(recv, "recv", layout.U * layout.elems_per_peer, dt)
    for name, t in (("rope_cos", rope_cos), ("rope_sin", rope_sin)):
        _expect(t, name, layout.S * (layout.D // 2), torch.float32, recv.device)
    if out is None:
        shape = (layout.B, layout.S, layout.H_loc, layout.D)
        out = [torch.empty(shape, dtype=dt, device=recv.device) for _ in range(3)]
    out = list(out)
    if len(out) != 3:
        raise ValueError("expected 3 output planes (q, k, v)")
    _expect_all(out, "out", layout.B * layout.S * layout.H_loc * layout.D, dt, recv.device)
    arr = (ctypes.c_void_p * 3)(*[_dev(p, f"out[{i}]") for i, p in enumerate(out)])
    check(lib().dit_ulysses_unpack_rope(ctypes.byref(layout), rank, _dev(recv, "recv"), arr,
                                        _dev(rope_cos, "rope_cos"), _dev(rope_sin, "rope_sin"),
                                        _stream(stream)), "dit_ulysses_unpack_rope")
    return out


def dit_a2a_uneven_init(B, S, H, D, U, n_planes=1, dtype=DIT_BF16, seq_counts=None,
                        head_counts=None) -> DitA2AUnevenLayout:
    """Padding-free layout from per-rank counts (None: the balanced split)."""
    if not isinstance(dtype, int):
        dtype = _dtype_code(dtype)

    def arr(c):
        if c is None:
            return None
        c = list(c)
        if len(c) != U:
            raise ValueError(f"expected {U} counts, got {len(c)}")
        return (ctypes.c_int32 * U)(*c)

    L = DitA2AUnevenLayout()
    check(lib().dit_a2a_uneven_init(B, S, H, D, U, n_planes, dtype, arr(seq_counts), arr(head_counts),
                                    ctypes.byref(L)), "dit_a2a_uneven_init")
    return L


def dit_a2a_uneven_sizes(layout: DitA2AUnevenLayout, direction: int, rank: int):
    """(send_counts, recv_counts): elements exchanged with each peer."""
    U = layout.U
    send = (ctypes.c_int64 * U)()
    recv = (ctypes.c_int64 * U)()
    check(lib().dit_a2a_uneven_sizes(ctypes.byref(layout), direction, rank, send, recv),
          "dit_a2a_uneven_sizes")
    return list(send), list(recv)


def _uneven_plane_numel(L, direction, rank, pack):
    """Elements of one plane of a padding-free map: head windows of the
    rank's rows ([B, S_rank, H, D]) or row windows of its heads
    ([B, S, H_rank, D])."""
    if (direction == DIT_SEQ_TO_HEAD) == pack:
        return L.B * L.seq_counts[rank] * L.H * L.D
    return L.B * L.S * L.head_counts[rank] * L.D


def _plane_ptrs(planes, name):
    return (ctypes.c_void_p * 3)(*[_dev(p, f"{name}[{i}]") for i, p in enumerate(planes)])


def dit_ulysses_pack_uneven(layout: DitA2AUnevenLayout, direction: int, rank: int, planes, send=None,
                            stream=None):
    """Pack rank `rank`'s planes into back-to-back per-peer chunks (1-D send
    buffer, allocated if `send` is None)."""
    torch = _torch()
    planes = list(planes)
    if len(planes) != layout.n_planes:
        raise ValueError(f"expected {layout.n_planes} planes, got {len(planes)}")
    dt, dev = _torch_dtype(layout.dtype), planes[0].device
    _expect_all(planes, "planes", _uneven_plane_numel(layout, direction, rank, True), dt, dev)
    n = sum(dit_a2a_uneven_sizes(layout, direction, rank)[0])
    if send is None:
        send = torch.empty(n, dtype=dt, device=dev)
    _expect(send, "send", n, dt, dev)
    check(lib().dit_ulysses_pack_uneven(ctypes.byref(layout), direction, rank, _plane_ptrs(planes, "planes"),
                                        _dev(send, "send"), _stream(stream)), "dit_ulysses_pack_uneven")
    return send


def dit_ulysses_unpack_uneven(layout: DitA2AUnevenLayout, direction: int, rank: int, recv, out=None,
                              stream=None):
    """Unpack a receive buffer of per-peer chunks into n_planes tensors:
    [B, S, H_rank, D] for DIT_SEQ_TO_HEAD, [B, S_rank, H, D] for DIT_HEAD_TO_SEQ."""
    torch = _torch()
    dt = _torch_dtype(layout.dtype)
    _expect(recv, "recv", sum(dit_a2a_uneven_sizes(layout, direction, rank)[1]), dt)
    if out is None:
        shape = ((layout.B, layout.S, layout.head_counts[rank], layout.D) if direction == DIT_SEQ_TO_HEAD
                 else (layout.B, layout.seq_counts[rank], layout.H, layout.D))
        out = [torch.empty(shape, dtype=dt, device=recv.device) for _ in range(layout.n_planes)]
    out = list(out)
    if len(out) != layout.n_planes:
        raise ValueError(f"expected {layout.n_planes} output planes, got {len(out)}")
    _expect_all(out, "out", _uneven_plane_numel(layout, direction, rank, False), dt, recv.device)
    check(lib().dit_ulysses_unpack_uneven(ctypes.byref(layout), direction, rank, _dev(recv, "recv"),
                                          _plane_ptrs(out, "out"), _stream(stream)),
          "dit_ulysses_unpack_uneven")
    return out


def dit_ring_anything_pad(layout: DitA2AUnevenLayout, rank: int, planes, send=None, stream=None):
    """Rank `rank`'s shards [B, S_rank, H, D] padded into [n, B, S_max, H, D]."""
    torch = _torch()
    planes = list(planes)
    if len(planes) != layout.n_planes:
        raise ValueError(f"expected {layout.n_planes} planes, got {len(planes)}")
    if not 0 <= rank < layout.U:
        raise ValueError(f"rank {rank} outside [0, {layout.U})")
    dt, dev = _torch_dtype(layout.dtype), planes[0].device
    _expect_all(planes, "planes", layout.B * layout.seq_counts[rank] * layout.H * layout.D, dt, dev)
    shape = (layout.n_planes, layout.B, layout.S_max, layout.H, layout.D)
    if send is None:
        send = torch.empty(shape, dtype=dt, device=dev)
    _expect(send, "send", math.prod(shape), dt, dev)
    check(lib().dit_ring_anything_pad(ctypes.byref(layout), rank, _plane_ptrs(planes, "planes"),
                                      _dev(send, "send"), _stream(stream)), "dit_ring_anything_pad")
    return send


def dit_ring_anything_trim(layout: DitA2AUnevenLayout, gathered, out=None, stream=None):
    """The gathered [U, n, B, S_max, H, D] buffer cut to n planes [B, S, H, D]."""
    torch = _torch()
    dt = _torch_dtype(layout.dtype)
    _expect(gathered, "gathered",
            layout.U * layout.n_planes * layout.B * layout.S_max * layout.H * layout.D, dt)
    if out is None:
        out = [torch.empty((layout.B, layout.S, layout.H, layout.D), dtype=dt, device=gathered.device)
               for _ in range(layout.n_planes)]
    out = list(out)
    if len(out) != layout.n_planes:
        raise ValueError(f"expected {layout.n_planes} output planes, got {len(out)}")
    _expect_all(out, "out", layout.B * layout.S * layout.H * layout.D, dt, gathered.device)
    check(lib().dit_ring_anything_trim(ctypes.byref(layout), _dev(gathered, "gathered"),
                                       _plane_ptrs(out, "out"), _stream(stream)), "dit_ring_anything_trim")
    return out


def dit_a2a_fp8_bytes_per_peer(layout: DitA2ALayout, direction: int) -> int:
    """Bytes of one peer's chunk of the FP8 exchange buffer."""
    n = ctypes.c_int64()
    check(lib().dit_a2a_fp8_bytes_per_peer(ctypes.byref(layout), direction, ctypes.byref(n)),
          "dit_a2a_fp8_bytes_per_peer")
    return n.value


def dit_ulysses_pack_fp8(layout: DitA2ALayout, direction: int, rank: int, planes, send=None, stream=None):
    """FP8 send buffer (uint8 [U, bytes_per_peer]) from bf16 planes: [q, k, v]
    shards for DIT_SEQ_TO_HEAD, [o] for DIT_HEAD_TO_SEQ."""
    torch = _torch()
    planes = list(planes)
    if len(planes) != layout.n_planes:
        raise ValueError(f"expected {layout.n_planes} planes, got {len(planes)}")
    dev = planes[0].device
    _expect_all(planes, "planes", _plane_numel(layout, direction, True), torch.bfloat16, dev)
    nbytes = layout.U * dit_a2a_fp8_bytes_per_peer(layout, direction)
    if send is None:
        send = torch.empty((layout.U, nbytes // layout.U), dtype=torch.uint8, device=dev)
    _expect(send, "send", nbytes, torch.uint8, dev)
    check(lib().dit_ulysses_pack_fp8(ctypes.byref(layout), direction, rank, _plane_ptrs(planes, "planes"),
                                     _dev(send, "send"), _stream(stream)), "dit_ulysses_pack_fp8")
    return send


def dit_ulysses_unpack_fp8(layout: DitA2ALayout, direction: int, rank: int, recv, out=None, stream=None):
    """bf16 planes from an FP8 receive buffer: [q, k, v] of [B, S, H_loc, D]
    for DIT_SEQ_TO_HEAD, [o] of [B, S_loc, H, D] for DIT_HEAD_TO_SEQ."""
    torch = _torch()
    _expect(recv, "recv", layout.U * dit_a2a_fp8_bytes_per_peer(layout, direction), torch.uint8)
    if out is None:
        shape = ((layout.B, layout.S, layout.H_loc, layout.D) if direction == DIT_SEQ_TO_HEAD
                 else (layout.B, layout.S_loc, layout.H, layout.D))
        out = [torch.empty(shape, dtype=torch.bfloat16, device=recv.device) for _ in range(layout.n_planes)]
    out = list(out)
    if len(out) != layout.n_planes:
        raise ValueError(f"expected {layout.n_planes} output planes, got {len(out)}")
    _expect_all(out, "out", _plane_numel(layout, direction, False), torch.bfloat16, recv.device)
    check(lib().dit_ulysses_unpack_fp8(ctypes.byref(layout), direction, rank, _dev(recv, "recv"),
                                       _plane_ptrs(out, "out"), _stream(stream)), "dit_ulysses_unpack_fp8")
    return out


def _check_qkv(q, k, v):
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k and v must be [B, S, H, D]")
    B, Sq, H, D = q.shape
    Skv = k.shape[1]
    if tuple(k.shape) != (B, Skv, H, D) or tuple(v.shape) != (B, Skv, H, D):
        raise ValueError(f"k {tuple(k.shape)} / v {tuple(v.shape)} do not match q {tuple(q.shape)}")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k and v must share one dtype")
    if k.device != q.device or v.device != q.device:
        raise ValueError("q, k and v must be on one device")
    return B, Sq, Skv, H, D


def _check_out(o, lse, B, Sq, H, D, device, lse_required):
    if o.dtype not in (_torch().bfloat16, _torch().float32):
        raise ValueError(f"o: dtype {o.dtype}, expected bfloat16 or float32")
    _expect(o, "o", B * Sq * H * D, o.dtype, device)
    if lse is not None:
        _expect(lse, "lse", B * H * Sq, _torch().float32, device)
    elif lse_required:
        raise ValueError("lse is required")


# Workspace of the bf16 attention's split last round, one per (device,
# stream): caller-owned memory in the C ABI's terms, here owned by this
# binding and zero-filled once (the kernels leave its counters zero).  A
# workspace that has to grow is replaced; the old one is kept alive, since
# launches already queued may still use it.
_WORKSPACES = {}
_RETIRED = []


def dit_attn_workspace_size(B, Sq, Skv, H, D, in_dtype=DIT_BF16, o_dtype=None, merge=False) -> int:
    """Bytes of workspace dit_attn_fwd_ws / dit_attn_fwd_merge use for these
    sizes on the current device (0: no tile is split)."""
    if not isinstance(in_dtype, int):
        in_dtype = _dtype_code(in_dtype)
    if o_dtype is None:
        o_dtype = in_dtype
    elif not isinstance(o_dtype, int):
        o_dtype = _dtype_code(o_dtype)
    n = ctypes.c_int64()
    check(lib().dit_attn_workspace_size(B, Sq, Skv, H, D, in_dtype, o_dtype, 1 if merge else 0,
                                        ctypes.byref(n)), "dit_attn_workspace_size")
    return n.value


def _workspace(nbytes, device, stream):
    if nbytes == 0:
        return None
    torch = _torch()
    key = (device.index, stream.value)
    ws = _WORKSPACES.get(key)
    if ws is None or ws.numel() < nbytes:
        if ws is not None:
            _RETIRED.append(ws)
        ws = torch.zeros(nbytes, dtype=torch.uint8, device=device)
        # the zero fill runs on torch's current stream; order it before a
        # launch on any other stream
        if stream.value != torch.cuda.current_stream(device).cuda_stream:
            torch.cuda.current_stream(device).synchronize()
        _WORKSPACES[key] = ws
    return ws


def dit_attn_fwd(q, k, v, o=None, lse=None, scale=None, o_dtype=None, want_lse=True,
                 stream=None, workspace=True):
    """Attention over [B, S, H, D] tensors; returns (O, LSE) with LSE
    [B, H, Sq] fp32 (None if want_lse is False and no buffer was given).

    workspace=True calls dit_attn_fwd_ws with this binding's workspace for
    the stream (the kernel may then split the last round of tiles);
    workspace=False calls dit_attn_fwd, which uses no memory beyond its
    arguments; a uint8 GPU tensor is passed through as the workspace."""
    torch = _torch()
    B, Sq, Skv, H, D = _check_qkv(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    in_code = _dtype_code(q.dtype)
    if o is None:
        o = torch.empty((B, Sq, H, D), dtype=o_dtype or q.dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    _check_out(o, lse, B, Sq, H, D, q.device, False)
    lse_ptr = _dev(lse, "lse") if lse is not None else ctypes.c_void_p(0)
    st = _stream(stream)
    args = [_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "o"), lse_ptr,
            B, Sq, Skv, H, D, float(scale), in_code, _dtype_code(o.dtype)]
    if workspace is False:
        check(lib().dit_attn_fwd(*args, st), "dit_attn_fwd")
        return o, lse
    if workspace is True:
        workspace = _workspace(dit_attn_workspace_size(B, Sq, Skv, H, D, in_code, _dtype_code(o.dtype)),
                               q.device, st)
    ws_ptr, ws_bytes = (ctypes.c_void_p(0), 0) if workspace is None else (_dev(workspace, "workspace"),
                                                                         workspace.numel())
    check(lib().dit_attn_fwd_ws(*args, ws_ptr, ws_bytes, st), "dit_attn_fwd_ws")
    return o, lse


def dit_attn_fwd_ws(q, k, v, workspace, o=None, lse=None, scale=None, o_dtype=None, stream=None):
    """dit_attn_fwd with an explicit workspace (uint8 GPU tensor, zero-filled
    before its first use, at least dit_attn_workspace_size() bytes)."""
    if workspace is not None and workspace.dtype != _torch().uint8:
        raise ValueError("workspace must be a uint8 tensor")
    return dit_attn_fwd(q, k, v, o=o, lse=lse, scale=scale, o_dtype=o_dtype, stream=stream,
                        workspace=workspace)


def dit_attn_fwd_send(q, k, v, layout: DitA2ALayout, rank: int, send=None, lse=None, scale=None,
                      want_lse=True, stream=None, workspace=True):
    """Attention of Ulysses rank `rank` with O stored straight into the
    head-to-sequence send buffer [U, 1, B, S_loc, H_loc, D] (bf16): equal,
    bit for bit, to dit_attn_fwd_ws followed by dit_ulysses_pack(layout,
    DIT_HEAD_TO_SEQ, rank, [O]).  q is [B, S, H_loc, D], k / v are
    [B, Skv, H_loc, D] (bf16); layout has n_planes = 1 and dtype bf16.
    Returns (send, LSE [B, H_loc, S] or None)."""
    torch = _torch()
    B, Sq, Skv, H, D = _check_qkv(q, k, v)
    if layout.n_planes != 1 or layout.dtype != DIT_BF16:
        raise ValueError("the send layout must have n_planes = 1 and dtype bf16")
    if (B, Sq, H, D) != (layout.B, layout.S, layout.H_loc, layout.D):
        raise ValueError(f"q {tuple(q.shape)} does not match the layout "
                         f"[B={layout.B}, S={layout.S}, H_loc={layout.H_loc}, D={layout.D}]")
    if q.dtype != torch.bfloat16:
        raise ValueError(f"q: dtype {q.dtype}, expected bfloat16")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if send is None:
        send = torch.empty(_send_shape(layout), dtype=torch.bfloat16, device=q.device)
    _expect(send, "send", layout.U * layout.elems_per_peer, torch.bfloat16, q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _expect(lse, "lse", B * H * Sq, torch.float32, q.device)
    st = _stream(stream)
    if workspace is True:
        workspace = _workspace(dit_attn_workspace_size(B, Sq, Skv, H, D, DIT_BF16, DIT_BF16),
                               q.device, st)
    elif workspace is False:
        workspace = None
    elif workspace.dtype != torch.uint8:
        raise ValueError("workspace must be a uint8 tensor")
    ws_ptr, ws_bytes = (ctypes.c_void_p(0), 0) if workspace is None else (_dev(workspace, "workspace"),
                                                                         workspace.numel())
    lse_ptr = _dev(lse, "lse") if lse is not None else ctypes.c_void_p(0)
    check(lib().dit_attn_fwd_send(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(send, "send"), lse_ptr,
                                  ctypes.byref(layout), rank, Skv, float(scale), ws_ptr, ws_bytes, st),
          "dit_attn_fwd_send")
    return send, lse


def dit_attn_fwd_a2a(recv, layout: DitA2ALayout, rank: int, send=None, lse=None, scale=None,
                     want_lse=True, stream=None, workspace=True):
    """Attention of Ulysses rank `rank` read straight from the packed
    sequence-to-head receive buffer recv [U, 3, B, S_loc, H_loc, D] (planes
    Q, K, V; bf16) and stored straight into the head-to-sequence send buffer
    [U, 1, B, S_loc, H_loc, D]: equal, bit for bit, to dit_ulysses_unpack
    (SEQ_TO_HEAD) followed by dit_attn_fwd_send.  layout has n_planes = 3,
    dtype bf16 and S_loc >= 64.  Returns (send, LSE [B, H_loc, S] or None)."""
    torch = _torch()
    if layout.n_planes != 3 or layout.dtype != DIT_BF16:
        raise ValueError("the receive layout must have n_planes = 3 and dtype bf16")
    _expect(recv, "recv", layout.U * layout.elems_per_peer, torch.bfloat16)
    dev = recv.device
    B, S, H, D = layout.B, layout.S, layout.H_loc, layout.D
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    one = layout.U * (layout.elems_per_peer // 3)
    if send is None:
        send = torch.empty((layout.U, 1, B, layout.S_loc, H, D), dtype=torch.bfloat16, device=dev)
    _expect(send, "send", one, torch.bfloat16, dev)
    if lse is None and want_lse:
        lse = torch.empty((B, H, S), dtype=torch.float32, device=dev)
    if lse is not None:
        _expect(lse, "lse", B * H * S, torch.float32, dev)
    st = _stream(stream)
    if workspace is True:
        workspace = _workspace(dit_attn_workspace_size(B, S, S, H, D, DIT_BF16, DIT_BF16), dev, st)
    elif workspace is False:
        workspace = None
    elif workspace.dtype != torch.uint8:
        raise ValueError("workspace must be a uint8 tensor")
    ws_ptr, ws_bytes = (ctypes.c_void_p(0), 0) if workspace is None else (_dev(workspace, "workspace"),
                                                                         workspace.numel())
    lse_ptr = _dev(lse, "lse") if lse is not None else ctypes.c_void_p(0)
    check(lib().dit_attn_fwd_a2a(_dev(recv, "recv"), _dev(send, "send"), lse_ptr, ctypes.byref(layout), rank,
                                 float(scale), ws_ptr, ws_bytes, st), "dit_attn_fwd_a2a")
    return send, lse


def dit_attn_fwd_noalloc(q, k, v, o, lse, scale=None, stream=None):
    """dit_attn_fwd with the library's static scratch as workspace: o and
    lse are caller buffers, nothing is allocated.  Calls that may overlap on
    one device race on the shared scratch."""
    B, Sq, Skv, H, D = _check_qkv(q, k, v)
    _check_out(o, lse, B, Sq, H, D, q.device, False)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    lse_ptr = _dev(lse, "lse") if lse is not None else ctypes.c_void_p(0)
    check(lib().dit_attn_fwd_noalloc(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "o"), lse_ptr,
                                     B, Sq, Skv, H, D, float(scale), _dtype_code(q.dtype),
                                     _dtype_code(o.dtype), _stream(stream)), "dit_attn_fwd_noalloc")
    return o, lse


def dit_attn_fwd_kvlen(q, k, v, kv_len, o=None, lse=None, scale=None, o_dtype=None, merge=False,
                       stream=None):
    """Attention where batch b attends only to its first kv_len[b] keys
    (kv_len: int32 GPU tensor [B]).  merge=True folds the result into the
    accumulator (o, lse) instead of writing it."""
    torch = _torch()
    B, Sq, Skv, H, D = _check_qkv(q, k, v)
    _expect(kv_len, "kv_len", B, torch.int32, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if merge and (o is None or lse is None):
        raise ValueError("merge=True needs the accumulator (o, lse)")
    if o is None:
        o = torch.empty((B, Sq, H, D), dtype=o_dtype or q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    _check_out(o, lse, B, Sq, H, D, q.device, True)
    check(lib().dit_attn_fwd_kvlen(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(kv_len, "kv_len"),
                                   _dev(o, "o"), _dev(lse, "lse"), B, Sq, Skv, H, D, float(scale),
                                   _dtype_code(q.dtype), _dtype_code(o.dtype), 1 if merge else 0,
                                   _stream(stream)), "dit_attn_fwd_kvlen")
    return o, lse


def dit_attn_merge(o_acc, lse_acc, o_part, lse_part, stream=None):
    """In-place merge of (o_part, lse_part) into (o_acc, lse_acc)."""
    torch = _torch()
    if o_acc.dim() != 4:
        raise ValueError("o_acc must be [B, Sq, H, D]")
    B, Sq, H, D = o_acc.shape
    if tuple(o_part.shape) != (B, Sq, H, D) or o_part.dtype != o_acc.dtype:
        raise ValueError("o_part must match o_acc in shape and dtype")
    for name, t in (("lse_acc", lse_acc), ("lse_part", lse_part)):
        if tuple(t.shape) != (B, H, Sq):
            raise ValueError(f"{name} must be [B, H, Sq] = {(B, H, Sq)}")
        _expect(t, name, B * H * Sq, torch.float32, o_acc.device)
    _expect(o_part, "o_part", B * Sq * H * D, o_acc.dtype, o_acc.device)
    check(lib().dit_attn_merge(_dev(o_acc, "o_acc"), _dev(lse_acc, "lse_acc"), _dev(o_part, "o_part"),
                               _dev(lse_part, "lse_part"), B, Sq, H, D, _dtype_code(o_acc.dtype),
                               _stream(stream)), "dit_attn_merge")
    return o_acc, lse_acc


def dit_attn_fwd_merge(q, k, v, o_acc, lse_acc, scale=None, stream=None, workspace=True):
    """One ring hop: attention of q over the chunk (k, v) merged in place
    into the accumulator (o_acc [B, Sq, H, D], lse_acc [B, H, Sq] fp32).
    workspace: as dit_attn_fwd (True: this binding's, False / None: none)."""
    B, Sq, Skv, H, D = _check_qkv(q, k, v)
    if tuple(o_acc.shape) != (B, Sq, H, D) or tuple(lse_acc.shape) != (B, H, Sq):
        raise ValueError("accumulator must be o [B, Sq, H, D] and lse [B, H, Sq]")
    _check_out(o_acc, lse_acc, B, Sq, H, D, q.device, True)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    st = _stream(stream)
    in_code, acc_code = _dtype_code(q.dtype), _dtype_code(o_acc.dtype)
    if workspace is True:
        workspace = _workspace(dit_attn_workspace_size(B, Sq, Skv, H, D, in_code, acc_code, merge=True),
                               q.device, st)
    elif workspace is False:
        workspace = None
    ws_ptr, ws_bytes = (ctypes.c_void_p(0), 0) if workspace is None else (_dev(workspace, "workspace"),
                                                                         workspace.numel())
    check(lib().dit_attn_fwd_merge(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o_acc, "o_acc"),
                                   _dev(lse_acc, "lse_acc"), B, Sq, Skv, H, D, float(scale),
                                   in_code, acc_code, ws_ptr, ws_bytes, st), "dit_attn_fwd_merge")
    return o_acc, lse_acc


def dit_cfg_combine(p_uncond, p_cond, g: float, out=None, stream=None):
    """out = p_uncond + g * (p_cond - p_uncond) elementwise (out may be an input)."""
    torch = _torch()
    if p_cond.shape != p_uncond.shape or p_cond.dtype != p_uncond.dtype:
        raise ValueError("p_cond must match p_uncond in shape and dtype")
    if p_cond.device != p_uncond.device:
        raise ValueError("p_cond and p_uncond must be on one device")
    if out is None:
        out = torch.empty_like(p_uncond)
    elif out.shape != p_uncond.shape or out.dtype != p_uncond.dtype:
        raise ValueError("out must match p_uncond in shape and dtype")
    _expect(out, "out", p_uncond.numel(), p_uncond.dtype, p_uncond.device)
    check(lib().dit_cfg_combine(_dev(p_uncond, "p_uncond"), _dev(p_cond, "p_cond"), _dev(out, "out"),
                                p_uncond.numel(), float(g), _dtype_code(p_uncond.dtype),
                                _stream(stream)), "dit_cfg_combine")
    return out


def dit_clock_probe(workgroups=256, spin=20000, mfma=False, stream=None):
    """Shader clock in GHz seen by `workgroups` probe workgroups (median,
    min, max) under a light FMA load or (mfma=True) a bf16 MFMA load;
    synchronizes the stream to read the result."""
    torch = _torch()
    out = torch.empty(2 * workgroups, dtype=torch.int64, device="cuda")
    check(lib().dit_clock_probe(_dev(out, "out"), workgroups, spin, int(bool(mfma)), _stream(stream)),
          "dit_clock_probe")
    s = out.view(-1, 2).double().cpu()
    ghz = (s[:, 0] / s[:, 1] / 10.0).sort().values
    return {"median": float(ghz[len(ghz) // 2]), "min": float(ghz[0]), "max": float(ghz[-1])}
