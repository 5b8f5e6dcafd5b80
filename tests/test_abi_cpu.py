"""C-ABI checks that need no GPU: the library loads, exports every entry
point the header declares, derives Ulysses layouts like the oracle, and
rejects every invalid call with its status code before any HIP call (fake,
never dereferenced device addresses stand in for tensors)."""

import ctypes
import math
import os
import re

import pytest

import oracle
import sequence_attention_amd as sa
from sequence_attention_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dit_attn.h")

INV = sa.DIT_ERR_INVALID_ARGUMENT
UNS = sa.DIT_ERR_UNSUPPORTED
P = ctypes.c_void_p
A = 0x7f0000000000          # fake, 256-byte aligned device address
NULL = P(0)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from sequence_attention_amd import build
        build.build()
    return _lib.lib()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dit_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert set(names) == set(_lib.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_header_is_plain_c():
    text = open(HEADER).read()
    assert "#include <stdint.h>" in text
    code = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    assert re.findall(r"#include\s*[<\"]([^>\"]+)", code) == ["stdint.h"]
    assert "hipStream_t" not in code
    assert "torch" not in text.lower()


def test_version_and_status_strings(lib):
    assert lib.dit_abi_version() == 2
    for code, name in [(0, "DIT_OK"), (1, "DIT_ERR_INVALID_ARGUMENT"), (2, "DIT_ERR_UNSUPPORTED"),
                       (3, "DIT_ERR_HIP")]:
        assert lib.dit_status_string(code).decode() == name
    assert lib.dit_status_string(42)


@pytest.mark.parametrize("args", [
    (1, 256, 4, 64, 2, 1, 3), (1, 4608, 24, 128, 2, 1, 3), (2, 7145, 24, 128, 4, 1, 3),
    (2, 7145, 24, 128, 5, 1, 3), (2, 7145, 24, 128, 4, 64, 1), (1, 75600, 40, 128, 8, 1, 1),
    (3, 10, 7, 8, 3, 4, 1), (1, 0, 4, 8, 2, 1, 1), (0, 5, 3, 8, 4, 1, 3), (1, 3, 4, 2, 4, 1, 1),
])
def test_layout_matches_oracle(lib, args):
    L = sa.dit_a2a_layout_init(*args)
    want = oracle.a2a_layout(*args)
    for key in ("S_pad", "S_loc", "H_pad", "H_loc", "elems_per_peer"):
        assert getattr(L, key) == want[key], key


def _layout(lib, *args):
    L = _lib.DitA2ALayout()
    assert lib.dit_a2a_layout_init(*args, ctypes.byref(L)) == 0
    return L


@pytest.mark.parametrize("args,code", [
    ((-1, 8, 4, 8, 2, 1, 1, 0), INV),
    ((1, -8, 4, 8, 2, 1, 1, 0), INV),
    ((1, 8, 4, -8, 2, 1, 1, 0), INV),
    ((1, 8, 4, 8, 0, 1, 1, 0), INV),
    ((1, 8, 4, 8, 2, 0, 1, 0), INV),
    ((1, 8, 4, 8, 2, 1, 2, 0), INV),
    ((1, 8, 4, 8, 2, 1, 1, 9), INV),
    ((2**30, 2**30, 4, 2**30, 1, 1, 3, 0), INV),
])
def test_layout_init_rejects(lib, args, code):
    L = _lib.DitA2ALayout()
    assert lib.dit_a2a_layout_init(*args, ctypes.byref(L)) == code
    assert lib.dit_last_error().decode() != ""


def test_layout_init_null_out(lib):
    assert lib.dit_a2a_layout_init(1, 8, 4, 8, 2, 1, 1, 0, None) == INV


def _planes(*ptrs):
    return (P * 3)(*[P(p) for p in ptrs])


def test_pack_unpack_rejects(lib):
    L = _layout(lib, 1, 8, 4, 8, 2, 1, 3, 0)
    ok3 = _planes(A, A + 4096, A + 8192)
    send = P(A + 65536)
    pack, unpack = lib.dit_ulysses_pack, lib.dit_ulysses_unpack
    assert pack(None, 0, 0, ok3, send, NULL) == INV
    assert pack(ctypes.byref(L), 2, 0, ok3, send, NULL) == INV           # direction
    assert pack(ctypes.byref(L), 0, -1, ok3, send, NULL) == INV          # rank
    assert pack(ctypes.byref(L), 0, 2, ok3, send, NULL) == INV           # rank == U
    assert pack(ctypes.byref(L), 0, 0, None, send, NULL) == INV          # plane array
    assert pack(ctypes.byref(L), 0, 0, _planes(A, 0, A + 8192), send, NULL) == INV
    assert pack(ctypes.byref(L), 0, 0, ok3, NULL, NULL) == INV           # send buffer
    assert pack(ctypes.byref(L), 0, 0, _planes(A + 1, A + 4096, A + 8192), send, NULL) == UNS
    assert pack(ctypes.byref(L), 0, 0, ok3, P(A + 4096), NULL) == INV    # overlap
    assert "overlap" in lib.dit_last_error().decode()
    assert unpack(ctypes.byref(L), 0, 0, NULL, ok3, NULL) == INV         # recv NULL
    assert unpack(ctypes.byref(L), 1, 0, send, _planes(A, A, A + 8192), NULL) == INV  # outputs overlap
    assert unpack(ctypes.byref(L), 0, 0, send, None, NULL) == INV
    bad = _lib.DitA2ALayout.from_buffer_copy(L)
    bad.S_loc += 1                                                        # tampered derived field
    assert pack(ctypes.byref(bad), 0, 0, ok3, send, NULL) == INV
    assert "derived" in lib.dit_last_error().decode()
    huge = _layout(lib, 1, 2**21, 1024, 128, 2, 1, 3, 0)                  # >= 2^31 elements
    assert pack(ctypes.byref(huge), 0, 0, ok3, send, NULL) == UNS


def test_unpack_rope_rejects(lib):
    # B=1, S=8, H=4, D=16 bf16, U=2: planes of 1*8*2*16 elements = 512 B
    L3 = _layout(lib, 1, 8, 4, 16, 2, 1, 3, 0)
    L1 = _layout(lib, 1, 8, 4, 16, 2, 1, 1, 0)
    ok3 = _planes(A, A + 4096, A + 8192)
    recv, cs, sn = P(A + 65536), P(A + 131072), P(A + 196608)
    f = lib.dit_ulysses_unpack_rope
    assert f(None, 0, recv, ok3, cs, sn, NULL) == INV
    assert f(ctypes.byref(L1), 0, recv, ok3, cs, sn, NULL) == INV        # n_planes must be 3
    assert f(ctypes.byref(L3), 2, recv, ok3, cs, sn, NULL) == INV        # rank
    assert f(ctypes.byref(L3), 0, NULL, ok3, cs, sn, NULL) == INV        # recv
    assert f(ctypes.byref(L3), 0, recv, None, cs, sn, NULL) == INV       # plane array
    assert f(ctypes.byref(L3), 0, recv, ok3, NULL, sn, NULL) == INV      # tables
    assert f(ctypes.byref(L3), 0, recv, ok3, cs, NULL, NULL) == INV
    assert f(ctypes.byref(L3), 0, recv, _planes(A, 0, A + 8192), cs, sn, NULL) == INV
    assert f(ctypes.byref(L3), 0, recv, _planes(A + 2, A + 4096, A + 8192), cs, sn, NULL) == UNS
    assert f(ctypes.byref(L3), 0, recv, ok3, P(A + 131072 + 4), sn, NULL) == UNS
    assert f(ctypes.byref(L3), 0, recv, _planes(A, A + 256, A + 8192), cs, sn, NULL) == INV  # overlap
    assert f(ctypes.byref(L3), 0, P(A + 4096), ok3, cs, sn, NULL) == INV  # plane overlaps recv
    assert f(ctypes.byref(L3), 0, recv, ok3, P(A + 8192), sn, NULL) == INV  # plane overlaps a table
    L_small_d = _layout(lib, 1, 8, 4, 4, 2, 1, 3, 0)                      # 8-byte heads
    assert f(ctypes.byref(L_small_d), 0, recv, ok3, cs, sn, NULL) == UNS
    empty = _layout(lib, 0, 8, 4, 16, 2, 1, 3, 0)
    assert f(ctypes.byref(empty), 0, NULL, _planes(0, 0, 0), NULL, NULL, NULL) == 0


def test_pack_convert_rejects(lib):
    # B=1, S=8, H=4, D=8, U=2, 3 planes: f32 planes of 1*4*4*8*4 = 512 B,
    # a bf16 send buffer of 2*3*1*4*2*8*2 = 768 B
    L = _layout(lib, 1, 8, 4, 8, 2, 1, 3, 0)
    ok3 = _planes(A, A + 4096, A + 8192)
    send = P(A + 65536)
    f = lib.dit_ulysses_pack_convert
    assert f(None, 0, 0, ok3, send, NULL) == INV
    assert f(ctypes.byref(L), 2, 0, ok3, send, NULL) == INV              # direction
    assert f(ctypes.byref(L), 0, 2, ok3, send, NULL) == INV              # rank == U
    assert f(ctypes.byref(L), 0, 0, None, send, NULL) == INV             # plane array
    assert f(ctypes.byref(L), 0, 0, _planes(A, 0, A + 8192), send, NULL) == INV
    assert f(ctypes.byref(L), 0, 0, ok3, NULL, NULL) == INV              # send buffer
    assert f(ctypes.byref(L), 0, 0, _planes(A + 2, A + 4096, A + 8192), send, NULL) == UNS
    assert f(ctypes.byref(L), 0, 0, ok3, P(A + 65537), NULL) == UNS      # odd send address
    assert f(ctypes.byref(L), 0, 0, ok3, P(A + 4096 + 256), NULL) == INV  # overlaps plane 1
    assert "overlap" in lib.dit_last_error().decode()
    f32 = _layout(lib, 1, 8, 4, 8, 2, 1, 3, 2)                            # 32-bit send buffer
    assert f(ctypes.byref(f32), 0, 0, ok3, send, NULL) == UNS
    bad = _lib.DitA2ALayout.from_buffer_copy(L)
    bad.H_loc += 1
    assert f(ctypes.byref(bad), 0, 0, ok3, send, NULL) == INV
    huge = _layout(lib, 1, 2**21, 1024, 128, 2, 1, 3, 1)                  # >= 2^31 elements
    assert f(ctypes.byref(huge), 0, 0, ok3, send, NULL) == UNS
    empty = _layout(lib, 0, 8, 4, 8, 2, 1, 3, 1)
    assert f(ctypes.byref(empty), 1, 1, _planes(0, 0, 0), NULL, NULL) == 0


def test_empty_exchange_is_a_no_op(lib):
    L = _layout(lib, 0, 8, 4, 8, 2, 1, 3, 0)
    assert lib.dit_ulysses_pack(ctypes.byref(L), 0, 0, _planes(0, 0, 0), NULL, NULL) == 0
    assert lib.dit_ulysses_unpack(ctypes.byref(L), 1, 1, NULL, _planes(0, 0, 0), NULL) == 0


def _attn(lib, q=A, k=A + 2**24, v=A + 2**25, o=A + 2**26, lse=A + 2**27, B=1, Sq=128, Skv=128,
          H=2, D=64, scale=0.125, din=0, dout=0):
    return lib.dit_attn_fwd(P(q), P(k), P(v), P(o), P(lse), B, Sq, Skv, H, D, scale, din, dout, NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(B=-1), INV), (dict(Sq=-1), INV), (dict(Skv=-5), INV), (dict(H=-1), INV),
    (dict(din=7), INV), (dict(dout=5), INV),
    (dict(scale=0.0), INV), (dict(scale=-1.0), INV), (dict(scale=math.nan), INV),
    (dict(scale=math.inf), INV),
    (dict(din=1, dout=1), UNS),                     # fp16 not served
    (dict(D=96), UNS), (dict(D=256), UNS),
    (dict(din=0, dout=1), UNS), (dict(din=2, dout=0), UNS),
    (dict(q=0), INV), (dict(o=0), INV), (dict(k=0), INV), (dict(v=0), INV),
    (dict(q=A + 8), UNS), (dict(k=A + 2**24 + 2), UNS), (dict(o=A + 2**26 + 4), UNS),
    (dict(lse=A + 2**27 + 2), UNS),
    (dict(o=A + 1024), INV),                        # o overlaps q
    (dict(lse=A + 2**26 + 64), INV),                # lse overlaps o
    # size limits, checked before any pointer
    (dict(B=65536, H=32768), UNS),                  # 2^31 query tiles of 128 rows
    (dict(H=131072), UNS),                          # 64-row K/V block of 2^30 bytes
    (dict(din=2, dout=2, H=65536), UNS),            # fp32 path: H on a grid axis of 65535
    (dict(din=2, dout=2, B=65536), UNS),            # ... and B
])
def test_attn_rejects(lib, kw, code):
    assert _attn(lib, **kw) == code, lib.dit_last_error()
    assert lib.dit_last_error().decode() != ""


def test_attn_empty_is_a_no_op(lib):
    assert _attn(lib, q=0, k=0, v=0, o=0, lse=0, Sq=0) == 0
    assert _attn(lib, q=0, k=0, v=0, o=0, lse=0, B=0) == 0
    assert _attn(lib, q=0, k=0, v=0, o=0, lse=0, H=0) == 0
    assert lib.dit_last_error().decode() == ""


def _attn_merge(lib, q=A, k=A + 2**24, v=A + 2**25, o=A + 2**26, lse=A + 2**27, B=1, Sq=128, Skv=128,
                H=2, D=64, scale=0.125, din=0, dacc=0, ws=0, ws_bytes=0):
    return lib.dit_attn_fwd_merge(P(q), P(k), P(v), P(o), P(lse), B, Sq, Skv, H, D, scale, din, dacc,
                                  P(ws), ws_bytes, NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(B=-1), INV), (dict(din=7), INV), (dict(scale=0.0), INV), (dict(scale=math.nan), INV),
    (dict(din=1, dacc=1), UNS), (dict(D=96), UNS), (dict(din=2, dacc=0), UNS),
    (dict(q=0), INV), (dict(o=0), INV), (dict(k=0), INV),
    (dict(lse=0), INV),                             # the accumulator's LSE is required
    (dict(q=A + 8), UNS), (dict(lse=A + 2**27 + 2), UNS),
    (dict(o=A + 1024), INV),                        # accumulator overlaps q
])
def test_attn_fwd_merge_rejects(lib, kw, code):
    assert _attn_merge(lib, **kw) == code, lib.dit_last_error()
    assert lib.dit_last_error().decode() != ""


def _attn_ws(lib, q=A, k=A + 2**24, v=A + 2**25, o=A + 2**26, lse=A + 2**27, B=1, Sq=128, Skv=128,
             H=2, D=64, scale=0.125, din=0, dout=0, ws=A + 2**29, ws_bytes=1 << 20):
    return lib.dit_attn_fwd_ws(P(q), P(k), P(v), P(o), P(lse), B, Sq, Skv, H, D, scale, din, dout,
                               P(ws), ws_bytes, NULL)


# workspace arguments are checked before any device query or launch
@pytest.mark.parametrize("call", ["ws", "merge"])
@pytest.mark.parametrize("kw,code", [
    (dict(ws=0, ws_bytes=64), INV),                 # NULL workspace with a size
    (dict(ws_bytes=-1), INV),                       # negative size
    (dict(ws=A + 2**29 + 16), UNS),                 # not 256-byte aligned
    (dict(ws=A + 2**26, ws_bytes=1 << 20), INV),    # workspace overlaps o
    (dict(ws=A, ws_bytes=1 << 20), INV),            # workspace overlaps q
    (dict(B=-1), INV), (dict(D=96), UNS), (dict(scale=0.0), INV),
])
def test_attn_workspace_rejects(lib, call, kw, code):
    if call == "ws":
        st = _attn_ws(lib, **kw)
    else:
        kw = {k2: v2 for k2, v2 in kw.items()}
        kw.setdefault("ws", A + 2**29)
        kw.setdefault("ws_bytes", 1 << 20)
        st = _attn_merge(lib, **kw)
    assert st == code, lib.dit_last_error()
    assert lib.dit_last_error().decode() != ""


def test_attn_ws_empty_is_a_no_op(lib):
    assert _attn_ws(lib, q=0, k=0, v=0, o=0, lse=0, Sq=0) == 0
    assert _attn_ws(lib, ws=0, ws_bytes=0, q=0, k=0, v=0, o=0, lse=0, B=0) == 0


def test_attn_fwd_send_rejects(lib):
    # B=1, S=64, H=4, D=64 bf16, U=2: q [1,64,2,64] = 16 KiB, send 16 KiB
    L = _layout(lib, 1, 64, 4, 64, 2, 1, 1, 0)
    f = lib.dit_attn_fwd_send
    q, k, v, send, lse = P(A), P(A + 2**20), P(A + 2**21), P(A + 2**22), P(A + 2**23)

    def call(layout=ctypes.byref(L), rank=0, Skv=64, scale=0.125, send_=send, q_=q, ws=NULL, wsb=0):
        return f(q_, k, v, send_, ctypes.cast(lse, ctypes.POINTER(ctypes.c_float)), layout, rank, Skv,
                 scale, ws, wsb, NULL)

    assert call(layout=None) == INV
    assert call(rank=2) == INV
    assert call(rank=-1) == INV
    assert call(Skv=-1) == INV
    assert call(scale=0.0) == INV
    assert call(q_=NULL) == INV
    assert call(send_=NULL) == INV
    assert call(send_=P(A + 8192)) == INV                                  # send overlaps q
    assert call(send_=P(A + 2**22 + 8)) == UNS                             # misaligned
    assert call(ws=P(A + 2**24 + 64), wsb=4096) == UNS                     # workspace alignment
    assert call(ws=NULL, wsb=64) == INV
    L3 = _layout(lib, 1, 64, 4, 64, 2, 1, 3, 0)
    assert call(layout=ctypes.byref(L3)) == INV                            # n_planes must be 1
    Lh = _layout(lib, 1, 64, 4, 64, 2, 1, 1, 1)
    assert call(layout=ctypes.byref(Lh)) == UNS                            # f16 buffer
    Ld = _layout(lib, 1, 64, 4, 96, 2, 1, 1, 0)
    assert call(layout=ctypes.byref(Ld)) == UNS                            # head dim
    bad = _lib.DitA2ALayout.from_buffer_copy(L)
    bad.S_loc += 1
    assert call(layout=ctypes.byref(bad)) == INV
    empty = _layout(lib, 0, 64, 4, 64, 2, 1, 1, 0)
    assert call(layout=ctypes.byref(empty), q_=NULL, send_=NULL) == 0


def test_attn_fwd_a2a_rejects(lib):
    # B=1, S=256, H=4, D=64 bf16, U=2: S_loc 128; recv [2,3,1,128,2,64] = 192 KiB, send 64 KiB
    L = _layout(lib, 1, 256, 4, 64, 2, 1, 3, 0)
    f = lib.dit_attn_fwd_a2a
    recv, send, lse = P(A), P(A + 2**22), P(A + 2**23)

    def call(layout=ctypes.byref(L), rank=0, scale=0.125, recv_=recv, send_=send, lse_=lse, ws=NULL, wsb=0):
        return f(recv_, send_, ctypes.cast(lse_, ctypes.POINTER(ctypes.c_float)), layout, rank, scale,
                 ws, wsb, NULL)

    assert call(layout=None) == INV
    assert call(rank=2) == INV
    assert call(rank=-1) == INV
    assert call(scale=0.0) == INV
    assert call(scale=float("nan")) == INV
    assert call(recv_=NULL) == INV
    assert call(send_=NULL) == INV
    assert call(send_=P(A + 3 * 2**16 - 1024)) == INV                     # send inside the recv buffer
    assert call(lse_=P(A + 1024)) == INV                                  # lse inside the recv buffer
    assert call(ws=P(A + 2**24 + 64), wsb=4096) == UNS                    # workspace alignment
    assert call(ws=P(A + 256), wsb=4096) == INV                           # workspace inside recv
    assert call(send_=P(A + 2**22 + 8)) == UNS                            # misaligned
    L1 = _layout(lib, 1, 256, 4, 64, 2, 1, 1, 0)
    assert call(layout=ctypes.byref(L1)) == INV                           # n_planes must be 3
    Lh = _layout(lib, 1, 256, 4, 64, 2, 1, 3, 1)
    assert call(layout=ctypes.byref(Lh)) == UNS                           # f16 buffer
    Ls = _layout(lib, 1, 100, 4, 64, 2, 1, 3, 0)
    assert call(layout=ctypes.byref(Ls)) == UNS                           # S_loc 50 < 64
    Ld = _layout(lib, 1, 256, 4, 96, 2, 1, 3, 0)
    assert call(layout=ctypes.byref(Ld)) == UNS                           # head dim
    bad = _lib.DitA2ALayout.from_buffer_copy(L)
    bad.elems_per_peer += 1
    assert call(layout=ctypes.byref(bad)) == INV
    empty = _layout(lib, 0, 256, 4, 64, 2, 1, 3, 0)
    assert call(layout=ctypes.byref(empty), recv_=NULL, send_=NULL) == 0


def _ws_size(lib, B=1, Sq=128, Skv=128, H=2, D=64, din=0, dout=0, merge=0, out=True):
    n = ctypes.c_int64(-5)
    st = lib.dit_attn_workspace_size(B, Sq, Skv, H, D, din, dout, merge, ctypes.byref(n) if out else None)
    return st, n.value


@pytest.mark.parametrize("kw,code", [
    (dict(out=False), INV), (dict(merge=2), INV), (dict(B=-1), INV), (dict(din=9), INV),
    (dict(D=96), UNS), (dict(din=1, dout=1), UNS), (dict(din=2, dout=0), UNS),
])
def test_attn_workspace_size_rejects(lib, kw, code):
    assert _ws_size(lib, **kw)[0] == code, lib.dit_last_error()


def test_attn_workspace_size_without_a_device_query(lib):
    # calls that never split need no workspace and touch no device
    assert _ws_size(lib, din=2, dout=2) == (0, 0)          # fp32 path
    assert _ws_size(lib, Sq=0) == (0, 0)
    assert _ws_size(lib, Skv=0, merge=1) == (0, 0)


def test_attn_fwd_merge_empty_chunk_is_a_no_op(lib):
    # Skv = 0 is the merge identity: nothing is launched, no pointer is used
    assert _attn_merge(lib, k=0, v=0, Skv=0) == 0
    assert _attn_merge(lib, q=0, k=0, v=0, o=0, lse=0, Sq=0) == 0
    assert lib.dit_last_error().decode() == ""


def _attn_kvlen(lib, q=A, k=A + 2**24, v=A + 2**25, kvl=A + 2**28, o=A + 2**26, lse=A + 2**27, B=1,
                Sq=128, Skv=128, H=2, D=64, scale=0.125, din=0, dout=0, merge=0):
    return lib.dit_attn_fwd_kvlen(P(q), P(k), P(v), P(kvl), P(o), P(lse), B, Sq, Skv, H, D, scale, din,
                                  dout, merge, NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(kvl=0), INV), (dict(kvl=A + 2**28 + 2), UNS), (dict(merge=2), INV), (dict(merge=-1), INV),
    (dict(merge=1, lse=0), INV), (dict(B=-1), INV), (dict(D=96), UNS), (dict(o=A + 1024), INV),
])
def test_attn_kvlen_rejects(lib, kw, code):
    assert _attn_kvlen(lib, **kw) == code, lib.dit_last_error()


def test_attn_kvlen_empty_is_a_no_op(lib):
    assert _attn_kvlen(lib, q=0, k=0, v=0, o=0, lse=0, kvl=A, Sq=0) == 0
    assert _attn_kvlen(lib, k=0, v=0, Skv=0, merge=1) == 0   # merging an empty key set


def _merge(lib, oa=A, la=A + 2**24, op=A + 2**25, lp=A + 2**26, B=1, Sq=16, H=2, D=64, dt=0):
    return lib.dit_attn_merge(P(oa), P(la), P(op), P(lp), B, Sq, H, D, dt, NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(B=-1), INV), (dict(D=-8), INV), (dict(dt=9), INV), (dict(dt=1), UNS),
    (dict(D=96), UNS), (dict(D=12), UNS), (dict(D=1024), UNS), (dict(D=0), UNS),
    (dict(oa=0), INV), (dict(lp=0), INV),
    (dict(oa=A + 8), UNS), (dict(la=A + 2**24 + 2), UNS),
    (dict(op=A + 256), INV), (dict(lp=A + 2**24 + 4), INV),
])
def test_merge_rejects(lib, kw, code):
    assert _merge(lib, **kw) == code


def test_merge_empty_is_a_no_op(lib):
    assert _merge(lib, oa=0, la=0, op=0, lp=0, Sq=0) == 0


def _cfg(lib, u=A, c=A + 2**20, out=A + 2**21, n=1000, g=4.0, dt=2):
    return lib.dit_cfg_combine(P(u), P(c), P(out), n, g, dt, NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(n=-1), INV), (dict(g=math.inf), INV), (dict(g=math.nan), INV), (dict(dt=4), INV),
    (dict(dt=1), UNS), (dict(u=0), INV), (dict(out=0), INV),
    (dict(u=A + 4), UNS), (dict(out=A + 16), INV),  # partial overlap with u
])
def test_cfg_rejects(lib, kw, code):
    assert _cfg(lib, **kw) == code


def test_cfg_empty_is_a_no_op(lib):
    assert _cfg(lib, u=0, c=0, out=0, n=0) == 0


def test_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 4, 1, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        sa.dit_attn_fwd(q, q, q, o=q.clone(), lse=torch.zeros(1, 1, 4))


# ---- padding-free (uneven) layouts ---------------------------------------------

def _uneven(lib, B, S, H, D, U, n=1, dt=0, sc=None, hc=None):
    L = _lib.DitA2AUnevenLayout()
    arr = lambda c: None if c is None else (ctypes.c_int32 * U)(*c)
    st = lib.dit_a2a_uneven_init(B, S, H, D, U, n, dt, arr(sc), arr(hc), ctypes.byref(L))
    assert st == 0, lib.dit_last_error()
    return L


@pytest.mark.parametrize("S,H,U,sc,hc", [
    (4481, 24, 4, None, None), (10, 5, 3, None, None), (9, 5, 3, [0, 4, 5], [2, 0, 3]),
    (7, 1, 4, None, None), (0, 0, 2, None, None),
])
def test_uneven_layout_and_sizes_match_oracle(lib, S, H, U, sc, hc):
    B, D, n = 2, 8, 3
    L = _uneven(lib, B, S, H, D, U, n, 0, sc, hc)
    want_s = sc or [S // U + (1 if r < S % U else 0) for r in range(U)]
    want_h = hc or [H // U + (1 if r < H % U else 0) for r in range(U)]
    assert L.counts() == (want_s, want_h)
    so, ho = L.offsets()
    assert so == [sum(want_s[:r]) for r in range(U + 1)] and ho == [sum(want_h[:r]) for r in range(U + 1)]
    assert L.S_max == max(want_s)
    for r in range(U):
        for d, s2h in ((0, True), (1, False)):
            send = (ctypes.c_int64 * U)()
            recv = (ctypes.c_int64 * U)()
            assert lib.dit_a2a_uneven_sizes(ctypes.byref(L), d, r, send, recv) == 0
            ws, wr = oracle.uneven_chunk_sizes(B, D, n, want_s, want_h, r, s2h)
            assert list(send) == ws and list(recv) == wr


@pytest.mark.parametrize("args,code", [
    ((1, 10, 4, 8, 0, 1, 0, None, None), INV),                 # U = 0
    ((1, 10, 4, 8, 65, 1, 0, None, None), INV),                # U > DIT_MAX_RANKS
    ((1, 10, 4, 8, 2, 4, 0, None, None), INV),                 # n_planes
    ((1, 10, 4, 8, 2, 0, 0, None, None), INV),
    ((1, 10, 4, 8, 2, 1, 9, None, None), INV),                 # dtype
    ((-1, 10, 4, 8, 2, 1, 0, None, None), INV),
    ((1, 10, 4, 8, 2, 1, 0, [5, 6], None), INV),               # counts sum to 11, not 10
    ((1, 10, 4, 8, 2, 1, 0, None, [1, 2]), INV),               # heads sum to 3, not 4
    ((1, 10, 4, 8, 2, 1, 0, [12, -2], None), INV),             # negative count
])
def test_uneven_init_rejects(lib, args, code):
    B, S, H, D, U, n, dt, sc, hc = args
    arr = lambda c: None if c is None else (ctypes.c_int32 * len(c))(*c)
    L = _lib.DitA2AUnevenLayout()
    assert lib.dit_a2a_uneven_init(B, S, H, D, U, n, dt, arr(sc), arr(hc), ctypes.byref(L)) == code
    assert lib.dit_a2a_uneven_init(1, 10, 4, 8, 2, 1, 0, None, None, None) == INV


def test_uneven_pack_unpack_rejects(lib):
    L = _uneven(lib, 1, 9, 5, 8, 3, 3, 0, [4, 0, 5], [2, 2, 1])
    ok3 = _planes(A, A + 4096, A + 8192)
    buf = P(A + 65536)
    pk, up = lib.dit_ulysses_pack_uneven, lib.dit_ulysses_unpack_uneven
    assert pk(None, 0, 0, ok3, buf, NULL) == INV
    assert pk(ctypes.byref(L), 2, 0, ok3, buf, NULL) == INV             # direction
    assert pk(ctypes.byref(L), 0, 3, ok3, buf, NULL) == INV             # rank
    assert pk(ctypes.byref(L), 0, 0, None, buf, NULL) == INV
    assert pk(ctypes.byref(L), 0, 0, _planes(A, 0, A + 8192), buf, NULL) == INV
    assert pk(ctypes.byref(L), 0, 0, ok3, NULL, NULL) == INV
    assert pk(ctypes.byref(L), 0, 0, _planes(A + 1, A + 4096, A + 8192), buf, NULL) == UNS
    assert pk(ctypes.byref(L), 0, 0, ok3, P(A + 4096), NULL) == INV     # overlap
    assert up(ctypes.byref(L), 0, 0, NULL, ok3, NULL) == INV
    assert up(ctypes.byref(L), 0, 0, buf, _planes(A, A, A + 8192), NULL) == INV  # outputs overlap
    bad = _lib.DitA2AUnevenLayout.from_buffer_copy(L)
    bad.seq_offsets[1] += 1                                             # tampered derived field
    assert pk(ctypes.byref(bad), 0, 0, ok3, buf, NULL) == INV
    assert "derived" in lib.dit_last_error().decode()
    bad = _lib.DitA2AUnevenLayout.from_buffer_copy(L)
    bad.U = 99
    assert pk(ctypes.byref(bad), 0, 0, ok3, buf, NULL) == INV
    huge = _uneven(lib, 1, 2**21, 1024, 128, 2, 1, 0)                   # >= 2^31 elements
    assert pk(ctypes.byref(huge), 0, 0, ok3, buf, NULL) == UNS
    many = _uneven(lib, 30000, 4, 2, 8, 2, 3, 0)                        # B * n_planes > 65535
    assert pk(ctypes.byref(many), 0, 0, ok3, buf, NULL) == UNS
    # rank 1 holds no rows: its sequence-to-head pack and head-to-sequence unpack are empty
    assert pk(ctypes.byref(L), 0, 1, _planes(0, 0, 0), NULL, NULL) == 0
    assert up(ctypes.byref(L), 1, 1, NULL, _planes(0, 0, 0), NULL) == 0


def test_ring_anything_rejects(lib):
    L = _uneven(lib, 2, 9, 2, 8, 3, 1, 0, [4, 0, 5])
    pad, trim = lib.dit_ring_anything_pad, lib.dit_ring_anything_trim
    one = _planes(A, 0, 0)
    assert pad(None, 0, one, P(A + 65536), NULL) == INV
    assert pad(ctypes.byref(L), 3, one, P(A + 65536), NULL) == INV      # rank
    assert pad(ctypes.byref(L), 0, one, NULL, NULL) == INV
    assert pad(ctypes.byref(L), 0, one, P(A + 64), NULL) == INV         # overlap
    assert trim(ctypes.byref(L), NULL, one, NULL) == INV
    assert trim(ctypes.byref(L), P(A + 65536), None, NULL) == INV
    assert trim(None, P(A + 65536), one, NULL) == INV
    empty = _uneven(lib, 0, 9, 2, 8, 3, 1, 0, [4, 0, 5])
    assert trim(ctypes.byref(empty), NULL, _planes(0, 0, 0), NULL) == 0


# ---- FP8 exchange ----------------------------------------------------------------

@pytest.mark.parametrize("args,dirn", [((1, 4608, 24, 128, 2, 1, 3), 0), ((2, 37, 5, 64, 3, 1, 3), 0),
                                       ((1, 4608, 24, 128, 2, 1, 1), 1), ((1, 10, 4, 32, 4, 1, 1), 1)])
def test_fp8_bytes_per_peer_matches_oracle(lib, args, dirn):
    L = _layout(lib, *args, 0)
    n = ctypes.c_int64()
    assert lib.dit_a2a_fp8_bytes_per_peer(ctypes.byref(L), dirn, ctypes.byref(n)) == 0
    Lo = oracle.a2a_layout(*args)
    assert n.value == oracle.fp8_chunk_sections(Lo, dirn == 0)[2]


def test_fp8_rejects(lib):
    L3 = _layout(lib, 1, 8, 4, 32, 2, 1, 3, 0)
    L1 = _layout(lib, 1, 8, 4, 32, 2, 1, 1, 0)
    ok3 = _planes(A, A + 8192, A + 16384)
    buf = P(A + 65536)
    pk, up = lib.dit_ulysses_pack_fp8, lib.dit_ulysses_unpack_fp8
    n = ctypes.c_int64()
    assert lib.dit_a2a_fp8_bytes_per_peer(ctypes.byref(L3), 0, None) == INV
    assert lib.dit_a2a_fp8_bytes_per_peer(ctypes.byref(L3), 1, ctypes.byref(n)) == INV   # O needs n_planes 1
    assert pk(None, 0, 0, ok3, buf, NULL) == INV
    assert pk(ctypes.byref(L1), 0, 0, ok3, buf, NULL) == INV          # Q, K, V need n_planes 3
    assert pk(ctypes.byref(L3), 1, 0, ok3, buf, NULL) == INV          # O needs n_planes 1
    assert pk(ctypes.byref(L3), 0, 2, ok3, buf, NULL) == INV          # rank
    assert pk(ctypes.byref(L3), 0, 0, None, buf, NULL) == INV
    assert pk(ctypes.byref(L3), 0, 0, _planes(A, 0, A + 16384), buf, NULL) == INV
    assert pk(ctypes.byref(L3), 0, 0, ok3, NULL, NULL) == INV
    assert pk(ctypes.byref(L3), 0, 0, _planes(A + 8, A + 8192, A + 16384), buf, NULL) == UNS
    assert pk(ctypes.byref(L3), 0, 0, ok3, P(A + 65536 + 8), NULL) == UNS
    assert pk(ctypes.byref(L3), 0, 0, ok3, P(A + 8192), NULL) == INV  # overlap
    assert up(ctypes.byref(L1), 1, 0, buf, None, NULL) == INV
    assert up(ctypes.byref(L3), 0, 0, NULL, ok3, NULL) == INV
    assert up(ctypes.byref(L3), 0, 0, buf, _planes(A, A, A + 16384), NULL) == INV   # outputs overlap
    f32 = _layout(lib, 1, 8, 4, 32, 2, 1, 3, 2)
    assert pk(ctypes.byref(f32), 0, 0, ok3, buf, NULL) == UNS         # bf16 only
    d16 = _layout(lib, 1, 8, 4, 16, 2, 1, 3, 0)
    assert pk(ctypes.byref(d16), 0, 0, ok3, buf, NULL) == UNS         # D not a multiple of 32
    empty = _layout(lib, 0, 8, 4, 32, 2, 1, 3, 0)
    assert pk(ctypes.byref(empty), 0, 0, _planes(0, 0, 0), NULL, NULL) == 0


def test_clock_probe_rejects(lib):
    f = lib.dit_clock_probe
    out = ctypes.cast(P(A), ctypes.POINTER(ctypes.c_int64))
    assert f(out, 0, 10, 0, NULL) == INV                     # no workgroups
    assert f(out, 65537, 10, 0, NULL) == INV
    assert f(out, 4, -1, 0, NULL) == INV                     # spin
    assert f(out, 4, 10, 2, NULL) == INV                     # mode
    assert f(None, 4, 10, 0, NULL) == INV
    assert f(ctypes.cast(P(A + 4), ctypes.POINTER(ctypes.c_int64)), 4, 10, 1, NULL) == UNS
