"""The Python binding checks every caller-supplied buffer before calling the
C ABI, which cannot see buffer sizes: a tensor with the wrong element count,
dtype or device would otherwise become an out-of-bounds access on the GPU.
These checks run before the binding asks for a device pointer, so CPU (and
meta) tensors exercise them here without a GPU."""

import pytest
import torch

import sequence_attention_amd as sa

BF = torch.bfloat16


def _t(*shape, dtype=BF, device="cpu"):
    return torch.zeros(shape, dtype=dtype, device=device)


L3 = None


@pytest.fixture(scope="module", autouse=True)
def layouts():
    global L3
    L3 = sa.dit_a2a_layout_init(1, 10, 4, 64, 2, 1, 3)     # S_loc 5, H_loc 2


def test_pack_rejects_a_short_plane():
    planes = [_t(1, 5, 4, 64), _t(1, 4, 4, 64), _t(1, 5, 4, 64)]
    with pytest.raises(ValueError, match=r"planes\[1\]: .* elements"):
        sa.dit_ulysses_pack(L3, sa.DIT_SEQ_TO_HEAD, 0, planes)


def test_pack_rejects_a_send_buffer_of_the_wrong_size_or_dtype():
    planes = [_t(1, 5, 4, 64) for _ in range(3)]
    with pytest.raises(ValueError, match="send: .* elements"):
        sa.dit_ulysses_pack(L3, sa.DIT_SEQ_TO_HEAD, 0, planes, send=_t(2, 3, 1, 5, 2, 63))
    with pytest.raises(ValueError, match="send: dtype"):
        sa.dit_ulysses_pack(L3, sa.DIT_SEQ_TO_HEAD, 0, planes, send=_t(2, 3, 1, 5, 2, 64, dtype=torch.float16))


def test_pack_rejects_planes_on_two_devices():
    planes = [_t(1, 5, 4, 64), _t(1, 5, 4, 64, device="meta"), _t(1, 5, 4, 64)]
    with pytest.raises(ValueError, match="expected cpu"):
        sa.dit_ulysses_pack(L3, sa.DIT_SEQ_TO_HEAD, 0, planes)


def test_pack_convert_checks_plane_dtype_and_send_buffer():
    planes = [_t(1, 5, 4, 64, dtype=torch.float32) for _ in range(3)]
    with pytest.raises(ValueError, match=r"planes\[0\]: dtype"):
        sa.dit_ulysses_pack_convert(L3, sa.DIT_SEQ_TO_HEAD, 0, [_t(1, 5, 4, 64)] * 3)
    with pytest.raises(ValueError, match=r"planes\[2\]: .* elements"):
        sa.dit_ulysses_pack_convert(L3, sa.DIT_SEQ_TO_HEAD, 0,
                                    planes[:2] + [_t(1, 5, 4, 63, dtype=torch.float32)])
    with pytest.raises(ValueError, match="send: dtype"):
        sa.dit_ulysses_pack_convert(L3, sa.DIT_SEQ_TO_HEAD, 0, planes,
                                    send=_t(2, 3, 1, 5, 2, 64, dtype=torch.float16))
    with pytest.raises(ValueError, match="bf16 or f16"):
        sa.dit_ulysses_pack_convert(sa.dit_a2a_layout_init(1, 10, 4, 64, 2, 1, 3, torch.float32),
                                    sa.DIT_SEQ_TO_HEAD, 0, planes)


def test_unpack_checks_receive_buffer_and_outputs():
    with pytest.raises(ValueError, match="recv: .* elements"):
        sa.dit_ulysses_unpack(L3, sa.DIT_SEQ_TO_HEAD, 0, _t(2, 3, 1, 5, 2, 32))
    recv = _t(2, 3, 1, 5, 2, 64)
    with pytest.raises(ValueError, match=r"out\[2\]: .* elements"):
        sa.dit_ulysses_unpack(L3, sa.DIT_SEQ_TO_HEAD, 0, recv,
                              out=[_t(1, 10, 2, 64), _t(1, 10, 2, 64), _t(1, 9, 2, 64)])
    # head-to-sequence outputs are [B, S_loc, H, D]
    with pytest.raises(ValueError, match=r"out\[0\]: .* elements"):
        sa.dit_ulysses_unpack(L3, sa.DIT_HEAD_TO_SEQ, 0, recv, out=[_t(1, 10, 4, 64)] * 3)


def test_unpack_rope_checks_tables():
    recv = _t(2, 3, 1, 5, 2, 64)
    cos = torch.zeros(10, 32)
    with pytest.raises(ValueError, match="rope_sin: .* elements"):
        sa.dit_ulysses_unpack_rope(L3, 0, recv, cos, torch.zeros(10, 31))
    with pytest.raises(ValueError, match="rope_cos: dtype"):
        sa.dit_ulysses_unpack_rope(L3, 0, recv, cos.double(), cos)


def test_uneven_maps_check_sizes():
    L = sa.dit_a2a_uneven_init(1, 10, 4, 64, 2, 1, seq_counts=[7, 3], head_counts=[3, 1])
    with pytest.raises(ValueError, match=r"planes\[0\]: .* elements"):
        sa.dit_ulysses_pack_uneven(L, sa.DIT_SEQ_TO_HEAD, 1, [_t(1, 7, 4, 64)])
    send_n = sum(sa.dit_a2a_uneven_sizes(L, sa.DIT_SEQ_TO_HEAD, 1)[0])
    with pytest.raises(ValueError, match="send: .* elements"):
        sa.dit_ulysses_pack_uneven(L, sa.DIT_SEQ_TO_HEAD, 1, [_t(1, 3, 4, 64)], send=_t(send_n + 1))
    recv_n = sum(sa.dit_a2a_uneven_sizes(L, sa.DIT_SEQ_TO_HEAD, 1)[1])
    with pytest.raises(ValueError, match=r"out\[0\]: .* elements"):
        sa.dit_ulysses_unpack_uneven(L, sa.DIT_SEQ_TO_HEAD, 1, _t(recv_n), out=[_t(1, 10, 3, 64)])
    with pytest.raises(ValueError, match="send: .* elements"):
        sa.dit_ring_anything_pad(L, 1, [_t(1, 3, 4, 64)], send=_t(1, 1, 3, 4, 64))
    with pytest.raises(ValueError, match="gathered: .* elements"):
        sa.dit_ring_anything_trim(L, _t(2, 1, 1, 6, 4, 64))


def test_fp8_maps_check_sizes_and_dtypes():
    L = sa.dit_a2a_layout_init(1, 10, 4, 64, 2, 1, 3)
    with pytest.raises(ValueError, match=r"planes\[0\]: dtype"):
        sa.dit_ulysses_pack_fp8(L, sa.DIT_SEQ_TO_HEAD, 0, [_t(1, 5, 4, 64, dtype=torch.float16)] * 3)
    nb = 2 * sa.dit_a2a_fp8_bytes_per_peer(L, sa.DIT_SEQ_TO_HEAD)
    with pytest.raises(ValueError, match="recv: .* elements"):
        sa.dit_ulysses_unpack_fp8(L, sa.DIT_SEQ_TO_HEAD, 0, _t(nb - 256, dtype=torch.uint8))


def test_attention_checks_outputs():
    q, k, v = _t(1, 8, 2, 64), _t(1, 9, 2, 64), _t(1, 9, 2, 64)
    with pytest.raises(ValueError, match="o: .* elements"):
        sa.dit_attn_fwd(q, k, v, o=_t(1, 7, 2, 64))
    with pytest.raises(ValueError, match="lse: dtype"):
        sa.dit_attn_fwd(q, k, v, lse=torch.zeros(1, 2, 8, dtype=torch.float64))
    with pytest.raises(ValueError, match="lse: .* elements"):
        sa.dit_attn_fwd(q, k, v, lse=torch.zeros(1, 2, 9))
    with pytest.raises(ValueError, match="do not match"):
        sa.dit_attn_fwd(q, _t(1, 9, 3, 64), v)
    with pytest.raises(ValueError, match="one device"):
        sa.dit_attn_fwd(q, k, _t(1, 9, 2, 64, device="meta"))
    with pytest.raises(ValueError, match="kv_len: dtype"):
        sa.dit_attn_fwd_kvlen(q, k, v, torch.zeros(1, dtype=torch.int64))
    with pytest.raises(ValueError, match="kv_len: .* elements"):
        sa.dit_attn_fwd_kvlen(q, k, v, torch.zeros(2, dtype=torch.int32))
    with pytest.raises(ValueError, match="needs the accumulator"):
        sa.dit_attn_fwd_kvlen(q, k, v, torch.zeros(1, dtype=torch.int32), o=_t(1, 8, 2, 64), merge=True)


def test_merge_and_fwd_merge_check_the_accumulator():
    o = _t(1, 8, 2, 64)
    with pytest.raises(ValueError, match="lse_part: dtype"):
        sa.dit_attn_merge(o, torch.zeros(1, 2, 8), _t(1, 8, 2, 64), torch.zeros(1, 2, 8, dtype=torch.float64))
    with pytest.raises(ValueError, match="must be"):
        sa.dit_attn_merge(o, torch.zeros(1, 8, 2), _t(1, 8, 2, 64), torch.zeros(1, 2, 8))
    q, k, v = _t(1, 8, 2, 64), _t(1, 9, 2, 64), _t(1, 9, 2, 64)
    with pytest.raises(ValueError, match="lse: dtype"):
        sa.dit_attn_fwd_merge(q, k, v, o, torch.zeros(1, 2, 8, dtype=torch.float16))


def test_cfg_checks_out():
    u, c = torch.zeros(4, 8), torch.zeros(4, 8)
    with pytest.raises(ValueError, match="out must match"):
        sa.dit_cfg_combine(u, c, 4.0, out=torch.zeros(4, 7))
    with pytest.raises(ValueError, match="one device"):
        sa.dit_cfg_combine(u, torch.zeros(4, 8, device="meta"), 4.0)
