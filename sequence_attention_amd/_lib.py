"""ctypes view of libdit_attn.so (the C ABI declared in include/dit_attn.h).

Only argument marshalling lives here.  The library is loaded on first use;
if it is missing the call raises instead of falling back to anything else.
"""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdit_attn.so")

# dit_status_t
DIT_OK = 0
DIT_ERR_INVALID_ARGUMENT = 1
DIT_ERR_UNSUPPORTED = 2
DIT_ERR_HIP = 3

# dit_dtype_t
DIT_BF16 = 0
DIT_F16 = 1
DIT_F32 = 2

# dit_a2a_dir_t
DIT_SEQ_TO_HEAD = 0
DIT_HEAD_TO_SEQ = 1

EXPORTS = (
    "dit_abi_version",
    "dit_status_string",
    "dit_last_error",
    "dit_a2a_layout_init",
    "dit_ulysses_pack",
    "dit_ulysses_pack_convert",
    "dit_ulysses_unpack",
    "dit_ulysses_unpack_rope",
    "dit_a2a_uneven_init",
    "dit_a2a_uneven_sizes",
    "dit_ulysses_pack_uneven",
    "dit_ulysses_unpack_uneven",
    "dit_ring_anything_pad",
    "dit_ring_anything_trim",
    "dit_a2a_fp8_bytes_per_peer",
    "dit_ulysses_pack_fp8",
    "dit_ulysses_unpack_fp8",
    "dit_attn_fwd",
    "dit_attn_workspace_size",
    "dit_attn_fwd_ws",
    "dit_attn_fwd_send",
    "dit_attn_fwd_a2a",
    "dit_attn_fwd_noalloc",
    "dit_attn_fwd_kvlen",
    "dit_attn_merge",
    "dit_attn_fwd_merge",
    "dit_cfg_combine",
    "dit_clock_probe",
)


class DitA2ALayout(ctypes.Structure):
    """Mirror of dit_a2a_layout."""
    _fields_ = [
        ("B", ctypes.c_int32), ("S", ctypes.c_int32), ("H", ctypes.c_int32),
        ("D", ctypes.c_int32), ("U", ctypes.c_int32),
        ("seq_align", ctypes.c_int32),
        ("n_planes", ctypes.c_int32),
        ("dtype", ctypes.c_int),
        ("S_pad", ctypes.c_int32), ("S_loc", ctypes.c_int32),
        ("H_pad", ctypes.c_int32), ("H_loc", ctypes.c_int32),
        ("elems_per_peer", ctypes.c_int64),
    ]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


DIT_MAX_RANKS = 64


class DitA2AUnevenLayout(ctypes.Structure):
    """Mirror of dit_a2a_uneven_layout."""
    _fields_ = [
        ("B", ctypes.c_int32), ("S", ctypes.c_int32), ("H", ctypes.c_int32),
        ("D", ctypes.c_int32), ("U", ctypes.c_int32),
        ("n_planes", ctypes.c_int32),
        ("dtype", ctypes.c_int),
        ("S_max", ctypes.c_int32),
        ("seq_counts", ctypes.c_int32 * DIT_MAX_RANKS),
        ("head_counts", ctypes.c_int32 * DIT_MAX_RANKS),
        ("seq_offsets", ctypes.c_int32 * (DIT_MAX_RANKS + 1)),
        ("head_offsets", ctypes.c_int32 * (DIT_MAX_RANKS + 1)),
    ]

    def counts(self):
        U = self.U
        return list(self.seq_counts[:U]), list(self.head_counts[:U])

    def offsets(self):
        U = self.U
        return list(self.seq_offsets[:U + 1]), list(self.head_offsets[:U + 1])


class DitError(RuntimeError):
    def __init__(self, status: int, func: str, detail: str):
        self.status = status
        self.func = func
        self.detail = detail
        super().__init__(f"{func} failed: {status_name(status)}: {detail}")


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_LIB = None


def _declare(lib):
    lib.dit_abi_version.restype = ctypes.c_int
    lib.dit_abi_version.argtypes = []
    lib.dit_status_string.restype = ctypes.c_char_p
    lib.dit_status_string.argtypes = [ctypes.c_int]
    lib.dit_last_error.restype = ctypes.c_char_p
    lib.dit_last_error.argtypes = []
    lib.dit_a2a_layout_init.restype = ctypes.c_int
    lib.dit_a2a_layout_init.argtypes = [_I32] * 7 + [ctypes.c_int, ctypes.POINTER(DitA2ALayout)]
    lib.dit_ulysses_pack.restype = ctypes.c_int
    lib.dit_ulysses_pack.argtypes = [ctypes.POINTER(DitA2ALayout), ctypes.c_int, _I32,
                                     ctypes.POINTER(_P), _P, _P]
    lib.dit_ulysses_pack_convert.restype = ctypes.c_int
    lib.dit_ulysses_pack_convert.argtypes = [ctypes.POINTER(DitA2ALayout), ctypes.c_int, _I32,
                                             ctypes.POINTER(_P), _P, _P]
    lib.dit_ulysses_unpack.restype = ctypes.c_int
    lib.dit_ulysses_unpack.argtypes = [ctypes.POINTER(DitA2ALayout), ctypes.c_int, _I32, _P,
                                       ctypes.POINTER(_P), _P]
    lib.dit_ulysses_unpack_rope.restype = ctypes.c_int
    lib.dit_ulysses_unpack_rope.argtypes = [ctypes.POINTER(DitA2ALayout), _I32, _P, ctypes.POINTER(_P),
                                            _P, _P, _P]
    _UL = ctypes.POINTER(DitA2AUnevenLayout)
    _I32P = ctypes.POINTER(_I32)
    _I64P = ctypes.POINTER(ctypes.c_int64)
    lib.dit_a2a_uneven_init.restype = ctypes.c_int
    lib.dit_a2a_uneven_init.argtypes = [_I32] * 6 + [ctypes.c_int, _I32P, _I32P, _UL]
    lib.dit_a2a_uneven_sizes.restype = ctypes.c_int
    lib.dit_a2a_uneven_sizes.argtypes = [_UL, ctypes.c_int, _I32, _I64P, _I64P]
    lib.dit_ulysses_pack_uneven.restype = ctypes.c_int
    lib.dit_ulysses_pack_uneven.argtypes = [_UL, ctypes.c_int, _I32, ctypes.POINTER(_P), _P, _P]
    lib.dit_ulysses_unpack_uneven.restype = ctypes.c_int
    lib.dit_ulysses_unpack_uneven.argtypes = [_UL, ctypes.c_int, _I32, _P, ctypes.POINTER(_P), _P]
    lib.dit_ring_anything_pad.restype = ctypes.c_int
    lib.dit_ring_anything_pad.argtypes = [_UL, _I32, ctypes.POINTER(_P), _P, _P]
    lib.dit_ring_anything_trim.restype = ctypes.c_int
    lib.dit_ring_anything_trim.argtypes = [_UL, _P, ctypes.POINTER(_P), _P]
    lib.dit_a2a_fp8_bytes_per_peer.restype = ctypes.c_int
    lib.dit_a2a_fp8_bytes_per_peer.argtypes = [ctypes.POINTER(DitA2ALayout), ctypes.c_int, _I64P]
    lib.dit_ulysses_pack_fp8.restype = ctypes.c_int
    lib.dit_ulysses_pack_fp8.argtypes = [ctypes.POINTER(DitA2ALayout), ctypes.c_int, _I32,
                                         ctypes.POINTER(_P), _P, _P]
    lib.dit_ulysses_unpack_fp8.restype = ctypes.c_int
    lib.dit_ulysses_unpack_fp8.argtypes = [ctypes.POINTER(DitA2ALayout), ctypes.c_int, _I32, _P,
                                           ctypes.POINTER(_P), _P]
    lib.dit_attn_fwd.restype = ctypes.c_int
    lib.dit_attn_fwd.argtypes = [_P, _P, _P, _P, _P] + [_I32] * 5 + [ctypes.c_float, ctypes.c_int,
                                                                     ctypes.c_int, _P]
    lib.dit_attn_workspace_size.restype = ctypes.c_int
    lib.dit_attn_workspace_size.argtypes = [_I32] * 5 + [ctypes.c_int, ctypes.c_int, _I32, _I64P]
    lib.dit_attn_fwd_ws.restype = ctypes.c_int
    lib.dit_attn_fwd_ws.argtypes = [_P, _P, _P, _P, _P] + [_I32] * 5 + [ctypes.c_float, ctypes.c_int,
                                                                        ctypes.c_int, _P, ctypes.c_int64, _P]
    lib.dit_attn_fwd_send.restype = ctypes.c_int
    lib.dit_attn_fwd_send.argtypes = [_P, _P, _P, _P, _P, ctypes.POINTER(DitA2ALayout), _I32, _I32,
                                      ctypes.c_float, _P, ctypes.c_int64, _P]
    lib.dit_attn_fwd_a2a.restype = ctypes.c_int
    lib.dit_attn_fwd_a2a.argtypes = [_P, _P, _P, ctypes.POINTER(DitA2ALayout), _I32, ctypes.c_float, _P,
                                     ctypes.c_int64, _P]
    lib.dit_attn_fwd_noalloc.restype = ctypes.c_int
    lib.dit_attn_fwd_noalloc.argtypes = [_P, _P, _P, _P, _P] + [_I32] * 5 + [ctypes.c_float, ctypes.c_int,
                                                                            ctypes.c_int, _P]
    lib.dit_attn_fwd_kvlen.restype = ctypes.c_int
    lib.dit_attn_fwd_kvlen.argtypes = [_P, _P, _P, _P, _P, _P] + [_I32] * 5 + [ctypes.c_float, ctypes.c_int,
                                                                               ctypes.c_int, _I32, _P]
    lib.dit_attn_merge.restype = ctypes.c_int
    lib.dit_attn_merge.argtypes = [_P, _P, _P, _P] + [_I32] * 4 + [ctypes.c_int, _P]
    lib.dit_attn_fwd_merge.restype = ctypes.c_int
    lib.dit_attn_fwd_merge.argtypes = [_P, _P, _P, _P, _P] + [_I32] * 5 + [ctypes.c_float, ctypes.c_int,
                                                                           ctypes.c_int, _P, ctypes.c_int64, _P]
    lib.dit_clock_probe.restype = ctypes.c_int
    lib.dit_clock_probe.argtypes = [_P, _I32, _I32, _I32, _P]
    lib.dit_cfg_combine.restype = ctypes.c_int
    lib.dit_cfg_combine.argtypes = [_P, _P, _P, ctypes.c_int64, ctypes.c_float, ctypes.c_int, _P]


def lib():
    """The loaded library; raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m sequence_attention_amd.build` "
                "(or __graft_entry__.build()); there is no fallback path")
        handle = ctypes.CDLL(LIB_PATH)
        _declare(handle)
        _LIB = handle
    return _LIB


def status_name(status: int) -> str:
    return lib().dit_status_string(status).decode()


def check(status: int, func: str):
    if status != DIT_OK:
        raise DitError(status, func, lib().dit_last_error().decode())
