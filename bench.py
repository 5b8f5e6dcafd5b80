#!/usr/bin/env python3
"""Throughput of the per-GPU DiT sequence-parallel attention hot path.

One step = one pass of the whole hot path of one Ulysses rank over one
batch of synthetic input, the FLUX.1-like 1024x1024 shard by default
(B=1, joint sequence 4608 = 4096 image + 512 text tokens, 24 heads of 128,
Ulysses degree 2, ring degree 1):

  A1  QKV sequence-to-head pack   [1,2304,24,128] x3 -> [2,3,1,2304,12,128]
  A3  QKV unpack                  (the send buffer stands in for the received
                                   one: same bytes and shape; the all-to-all
                                   itself is a collective, outside this path)
  B/C attention with LSE          [1,4608,12,128]; ring degree 1, so the hop
                                   loop is one chunk and no merge
  D   O head-to-sequence pack     [1,4608,12,128] -> [2,1,1,2304,12,128]
  E   O unpack                    -> [1,2304,24,128]
  F   CFG combine                 [2,4096,64] fp32 latent prediction, g = 4

`value` is the step's algorithmic attention FLOP (4*B*H*Sq*Skv*D) divided by
the measured step time (K steps bracketed by two HIP events on the launch
stream).  Inputs are resident in HBM before timing; input sets rotate so
that successive steps do not find their data in the 256 MB Infinity Cache.
Before the warm-up steps, untimed steps run for --clock-warmup-s seconds:
the GPU clock needs a few hundred milliseconds of sustained work to leave
its idle level, and a denoising loop runs its attention blocks for seconds.
The JSON line also carries the attention kernel's roofline (its average
launch duration: K back-to-back launches bracketed by events), per-kernel
times, attention at every DiT shard shape, side measurements of the headline
permute (Wan [1,9450,40,128]) and of the ring merge, and the fp64 CPU oracle
timed on this host on the same workload.

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload flux]
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention TFLOP/s and % bf16 MFMA peak per DiT shard shape; permute GB/s"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, AMD published
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E, AMD published
MALL_BYTES = 256 << 20        # Infinity Cache
CFG_SHAPE = (2, 4096, 64)     # FLUX 1024x1024 latent prediction: 64x64 patches x 64 channels

# HBM bytes per launch of the FLUX attention kernel from two rocprofv3 --pmc
# passes (FETCH_SIZE, WRITE_SIZE; profiles/flux_attention_hbm_counters.md),
# each scaled by what the counter reads for a device copy of known size.
# Valid only for the kernel source they were taken on (SHA-256 below); any
# change to that file reports traffic as null until the counters are re-taken.
ATTN_SRC = os.path.join(ROOT, "sequence_attention_amd", "csrc", "attn_fwd_bf16.hip")
ATTN_TRAFFIC = {"src_sha256": "3aa960c5b509104b0a5a0cff5b3c3fc37d05e589d395b040d7faad06f6c9a042",
                "workload": "flux", "fetch_bytes": 52_216_832, "write_bytes": 14_377_024}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="flux", choices=["flux", "qwen_u4", "qwen_u5", "wan"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-side", action="store_true", help="skip the side permute / merge measurements")
    ap.add_argument("--no-configs", action="store_true", help="skip the per-config attention timings")
    ap.add_argument("--clock-warmup-s", type=float, default=0.5,
                    help="seconds of untimed steps before the warm-up steps, to bring the GPU clock up")
    return ap.parse_args()


class Step:
    """Buffers and launches of one rank's hot-path step."""

    def __init__(self, w, torch, sa, workloads, seed):
        dev = "cuda"
        self.w = w
        self.L3 = sa.dit_a2a_layout_init(w.B, w.S, w.H_total, w.D, w.U, 1, 3)
        self.L1 = sa.dit_a2a_layout_init(w.B, w.S, w.H_total, w.D, w.U, 1, 1)
        self.shard = [t.to(dev) for t in workloads.seq_sharded_planes(w, 3, self.L3.S_loc, seed=seed)]
        L3, L1 = self.L3, self.L1
        bf16 = torch.bfloat16
        self.send3 = torch.empty((w.U, 3, w.B, L3.S_loc, L3.H_loc, w.D), dtype=bf16, device=dev)
        self.qkv = [torch.empty((w.B, w.S, L3.H_loc, w.D), dtype=bf16, device=dev) for _ in range(3)]
        self.o = torch.empty((w.B, w.S, L3.H_loc, w.D), dtype=bf16, device=dev)
        self.lse = torch.empty((w.B, L3.H_loc, w.S), dtype=torch.float32, device=dev)
        self.send1 = torch.empty((w.U, 1, w.B, L1.S_loc, L1.H_loc, w.D), dtype=bf16, device=dev)
        self.out = torch.empty((w.B, L1.S_loc, w.H_total, w.D), dtype=bf16, device=dev)
        cfg = workloads.cfg_inputs(CFG_SHAPE, seed=seed)
        self.u = cfg[0].contiguous().to(dev)
        self.c = cfg[1].contiguous().to(dev)
        self.guided = torch.empty_like(self.u)

    def bytes(self):
        n = 0
        for t in self.shard + self.qkv + [self.send3, self.o, self.lse, self.send1, self.out, self.u,
                                          self.c, self.guided]:
            n += t.numel() * t.element_size()
        return n

    def run(self, sa, rank, only=None):
        """Enqueue one step (or only its kernel `only`)."""
        S2H, H2S = sa.DIT_SEQ_TO_HEAD, sa.DIT_HEAD_TO_SEQ
        launches = (
            ("A1_pack_qkv", lambda: sa.dit_ulysses_pack(self.L3, S2H, rank, self.shard, send=self.send3)),
            ("A3_unpack_qkv", lambda: sa.dit_ulysses_unpack(self.L3, S2H, rank, self.send3, out=self.qkv)),
            ("B_attention", lambda: sa.dit_attn_fwd(*self.qkv, o=self.o, lse=self.lse, scale=self.w.scale)),
            ("D_pack_o", lambda: sa.dit_ulysses_pack(self.L1, H2S, rank, [self.o], send=self.send1)),
            ("E_unpack_o", lambda: sa.dit_ulysses_unpack(self.L1, H2S, rank, self.send1, out=[self.out])),
            ("F_cfg", lambda: sa.dit_cfg_combine(self.u, self.c, 4.0, out=self.guided)),
        )
        for name, fn in launches:
            if only is None or only == name:
                fn()


def kernel_bytes(step):
    """Algorithmic HBM bytes per launch: every input element read once and
    every output element written once (pad elements written count)."""
    w, L3, L1 = step.w, step.L3, step.L1
    e = 2
    send3 = w.U * L3.elems_per_peer * e
    send1 = w.U * L1.elems_per_peer * e
    shard3 = 3 * w.B * min(L3.S_loc, w.S) * w.H_total * w.D * e
    qkv = 3 * w.B * w.S * L3.H_loc * w.D * e
    o = w.B * w.S * L3.H_loc * w.D * e
    out = w.B * L1.S_loc * w.H_total * w.D * e
    cfg = 3 * math.prod(CFG_SHAPE[1:]) * 4
    return {
        "A1_pack_qkv": shard3 + send3,
        "A3_unpack_qkv": send3 + qkv,
        "D_pack_o": o + send1,
        "E_unpack_o": send1 + out,
        "F_cfg": cfg,
    }


def side_measurements(torch, sa, workloads, reps=20):
    """Headline permute (Wan [1,9450,40,128]) and ring merge GB/s, each over
    buffer sets rotated beyond the Infinity Cache."""
    res = {}
    w = workloads.WORKLOADS["wan"]
    for n_planes in (1, 3):
        L = sa.dit_a2a_layout_init(w.B, w.S, w.H_total, w.D, w.U, 1, n_planes)
        plane_bytes = w.B * L.S_loc * w.H_total * w.D * 2
        moved = 2 * n_planes * plane_bytes
        sets = max(2, math.ceil(2 * MALL_BYTES / moved) + 1)
        bufs = []
        for i in range(sets):
            shard = [torch.empty((w.B, L.S_loc, w.H_total, w.D), dtype=torch.bfloat16, device="cuda").normal_()
                     for _ in range(n_planes)]
            send = torch.empty((w.U, n_planes, w.B, L.S_loc, L.H_loc, w.D), dtype=torch.bfloat16, device="cuda")
            bufs.append((shard, send))
        for kind in ("pack", "unpack"):
            def go(i):
                shard, send = bufs[i % sets]
                if kind == "pack":
                    sa.dit_ulysses_pack(L, sa.DIT_SEQ_TO_HEAD, 0, shard, send=send)
                else:
                    # head-to-sequence unpack: [U,n,B,S_loc,H_loc,D] -> n x [B,S_loc,H,D]
                    sa.dit_ulysses_unpack(L, sa.DIT_HEAD_TO_SEQ, 0, send, out=shard)
            us = _time_launches(torch, go, reps)
            res[f"wan_{kind}_{n_planes}plane"] = {
                "bytes": moved, "us": round(us, 2), "GB/s": round(moved / us / 1e3, 1),
                "frac_hbm_peak": round(moved / us / 1e3 / PEAK_HBM_GBPS, 4)}
        del bufs
    # fused receive preparation (unpack + RoPE on Q and K) at the FLUX U=2 shape,
    # against the plain unpack of the same buffer
    fw = workloads.WORKLOADS["flux"]
    L = sa.dit_a2a_layout_init(fw.B, fw.S, fw.H_total, fw.D, fw.U, 1, 3)
    recv_bytes = fw.U * L.elems_per_peer * 2
    plane_bytes = 3 * fw.B * fw.S * L.H_loc * fw.D * 2
    cos, sin = workloads.rope_tables(fw.S, fw.D)
    cos, sin = cos.to("cuda"), sin.to("cuda")
    table_bytes = 2 * cos.numel() * 4
    sets = max(2, math.ceil(2 * MALL_BYTES / (recv_bytes + plane_bytes)) + 1)
    bufs = [(torch.empty((fw.U, 3, fw.B, L.S_loc, L.H_loc, fw.D), dtype=torch.bfloat16, device="cuda").normal_(),
             [torch.empty((fw.B, fw.S, L.H_loc, fw.D), dtype=torch.bfloat16, device="cuda") for _ in range(3)])
            for _ in range(sets)]
    us = _time_launches(torch, lambda i: sa.dit_ulysses_unpack_rope(L, 0, bufs[i % sets][0], cos, sin,
                                                                    out=bufs[i % sets][1]), reps)
    moved = recv_bytes + plane_bytes + table_bytes
    res["flux_unpack_rope_qkv"] = {"bytes": moved, "us": round(us, 2), "GB/s": round(moved / us / 1e3, 1),
                                   "frac_hbm_peak": round(moved / us / 1e3 / PEAK_HBM_GBPS, 4)}
    us = _time_launches(torch, lambda i: sa.dit_ulysses_unpack(L, sa.DIT_SEQ_TO_HEAD, 0, bufs[i % sets][0],
                                                               out=bufs[i % sets][1]), reps)
    moved = recv_bytes + plane_bytes
    res["flux_unpack_qkv_plain"] = {"bytes": moved, "us": round(us, 2), "GB/s": round(moved / us / 1e3, 1),
                                    "frac_hbm_peak": round(moved / us / 1e3 / PEAK_HBM_GBPS, 4)}
    del bufs
    # padding-free split of FLUX at 1008x1008 (S = 512 text + 63*63 image = 4481
    # rows over U = 4): packed QKV sequence-to-head pack and unpack of rank 0,
    # against the padded layout of the same sequence; GB/s on the real bytes
    S_u, U_u, H_u, D_u = 4481, 4, 24, 128
    Lu = sa.dit_a2a_uneven_init(1, S_u, H_u, D_u, U_u, 3)
    Lp = sa.dit_a2a_layout_init(1, S_u, H_u, D_u, U_u, 1, 3)
    r_rows, _ = Lu.counts()
    real = {"pack": 2 * 3 * r_rows[0] * H_u * D_u * 2,
            "unpack": 2 * 3 * S_u * (H_u // U_u) * D_u * 2}
    sets = max(2, math.ceil(2 * MALL_BYTES / (2 * real["pack"] + 2 * real["unpack"])) + 1)
    bufs = []
    for i in range(sets):
        shard_u = [torch.empty((1, r_rows[0], H_u, D_u), dtype=torch.bfloat16, device="cuda").normal_()
                   for _ in range(3)]
        shard_p = [torch.empty((1, Lp.S_loc, H_u, D_u), dtype=torch.bfloat16, device="cuda").normal_()
                   for _ in range(3)]
        send_u = sa.dit_ulysses_pack_uneven(Lu, sa.DIT_SEQ_TO_HEAD, 0, shard_u)
        send_p = sa.dit_ulysses_pack(Lp, sa.DIT_SEQ_TO_HEAD, 0, shard_p)
        recv_u = torch.empty(sum(sa.dit_a2a_uneven_sizes(Lu, sa.DIT_SEQ_TO_HEAD, 0)[1]),
                             dtype=torch.bfloat16, device="cuda").normal_()
        out = [torch.empty((1, S_u, H_u // U_u, D_u), dtype=torch.bfloat16, device="cuda") for _ in range(3)]
        bufs.append((shard_u, shard_p, send_u, send_p, recv_u, out))
    legs = {
        "flux1008_uneven_pack_qkv": ("pack", lambda b: sa.dit_ulysses_pack_uneven(
            Lu, sa.DIT_SEQ_TO_HEAD, 0, b[0], send=b[2])),
        "flux1008_padded_pack_qkv": ("pack", lambda b: sa.dit_ulysses_pack(
            Lp, sa.DIT_SEQ_TO_HEAD, 0, b[1], send=b[3])),
        "flux1008_uneven_unpack_qkv": ("unpack", lambda b: sa.dit_ulysses_unpack_uneven(
            Lu, sa.DIT_SEQ_TO_HEAD, 0, b[4], out=b[5])),
        "flux1008_padded_unpack_qkv": ("unpack", lambda b: sa.dit_ulysses_unpack(
            Lp, sa.DIT_SEQ_TO_HEAD, 0, b[3], out=b[5])),
    }
    for name, (kind, fn) in legs.items():
        us = _time_launches(torch, lambda i, fn=fn: fn(bufs[i % sets]), reps)
        res[name] = {"real_bytes": real[kind], "us": round(us, 2), "GB/s": round(real[kind] / us / 1e3, 1),
                     "frac_hbm_peak": round(real[kind] / us / 1e3 / PEAK_HBM_GBPS, 4)}
    del bufs
    # Ring Anything trim of the gathered FLUX 1008x1008 K and V over a ring of 4
    Lr = sa.dit_a2a_uneven_init(1, S_u, H_u, D_u, U_u, 1)
    kv_bytes = S_u * H_u * D_u * 2
    sets = max(2, math.ceil(2 * MALL_BYTES / (4 * kv_bytes)) + 1)
    Lr2 = sa.dit_a2a_uneven_init(1, S_u, H_u, D_u, U_u, 2)
    bufs = [(torch.empty((U_u, 2, 1, Lr.S_max, H_u, D_u), dtype=torch.bfloat16, device="cuda").normal_(),
             [torch.empty((1, S_u, H_u, D_u), dtype=torch.bfloat16, device="cuda") for _ in range(2)])
            for _ in range(sets)]
    us = _time_launches(torch, lambda i: sa.dit_ring_anything_trim(Lr2, bufs[i % sets][0],
                                                                  out=bufs[i % sets][1]), reps)
    res["flux1008_ring_anything_trim_kv"] = {"real_bytes": 4 * kv_bytes, "us": round(us, 2),
                                             "GB/s": round(4 * kv_bytes / us / 1e3, 1),
                                             "frac_hbm_peak": round(4 * kv_bytes / us / 1e3 / PEAK_HBM_GBPS, 4)}
    del bufs
    # FP8 exchange at the FLUX U=2 shape: Q, V (and O) as block-scaled E4M3,
    # K bf16; bytes are the planes read / written plus the FP8 buffer
    L3 = sa.dit_a2a_layout_init(fw.B, fw.S, fw.H_total, fw.D, fw.U, 1, 3)
    L1 = sa.dit_a2a_layout_init(fw.B, fw.S, fw.H_total, fw.D, fw.U, 1, 1)
    st3 = sa.dit_a2a_fp8_bytes_per_peer(L3, sa.DIT_SEQ_TO_HEAD)
    st1 = sa.dit_a2a_fp8_bytes_per_peer(L1, sa.DIT_HEAD_TO_SEQ)
    shard_b = fw.B * L3.S_loc * fw.H_total * fw.D * 2
    head_b = fw.B * fw.S * L3.H_loc * fw.D * 2
    sets = max(2, math.ceil(2 * MALL_BYTES / (3 * shard_b + 3 * head_b + fw.U * (st3 + st1))) + 1)
    bufs = []
    for i in range(sets):
        shard = [torch.empty((fw.B, L3.S_loc, fw.H_total, fw.D), dtype=torch.bfloat16, device="cuda").normal_()
                 for _ in range(3)]
        heads = [torch.empty((fw.B, fw.S, L3.H_loc, fw.D), dtype=torch.bfloat16, device="cuda").normal_()
                 for _ in range(3)]
        s3 = sa.dit_ulysses_pack_fp8(L3, sa.DIT_SEQ_TO_HEAD, 0, shard)
        s1 = sa.dit_ulysses_pack_fp8(L1, sa.DIT_HEAD_TO_SEQ, 0, heads[:1])
        bufs.append((shard, heads, s3, s1))
    legs = {
        "flux_fp8_pack_qkv": (3 * shard_b + fw.U * st3, lambda b: sa.dit_ulysses_pack_fp8(
            L3, sa.DIT_SEQ_TO_HEAD, 0, b[0], send=b[2])),
        "flux_fp8_unpack_qkv": (3 * head_b + fw.U * st3, lambda b: sa.dit_ulysses_unpack_fp8(
            L3, sa.DIT_SEQ_TO_HEAD, 0, b[2], out=b[1])),
        "flux_fp8_pack_o": (head_b + fw.U * st1, lambda b: sa.dit_ulysses_pack_fp8(
            L1, sa.DIT_HEAD_TO_SEQ, 0, b[1][:1], send=b[3])),
        "flux_fp8_unpack_o": (shard_b + fw.U * st1, lambda b: sa.dit_ulysses_unpack_fp8(
            L1, sa.DIT_HEAD_TO_SEQ, 0, b[3], out=b[0][:1])),
    }
    for name, (moved, fn) in legs.items():
        us = _time_launches(torch, lambda i, fn=fn: fn(bufs[i % sets]), reps)
        res[name] = {"bytes": moved, "us": round(us, 2), "GB/s": round(moved / us / 1e3, 1),
                     "frac_hbm_peak": round(moved / us / 1e3 / PEAK_HBM_GBPS, 4)}
    res["flux_fp8_exchange_bytes"] = {"qkv_fp8": fw.U * st3, "qkv_bf16": fw.U * L3.elems_per_peer * 2,
                                      "o_fp8": fw.U * st1, "o_bf16": fw.U * L1.elems_per_peer * 2}
    del bufs
    # hipMemcpy-class device copy of the same bytes, as the achievable-copy reference
    n_bytes = 2 * 96_768_000 // 2
    src = [torch.empty(n_bytes // 2, dtype=torch.bfloat16, device="cuda") for _ in range(6)]
    dst = [torch.empty_like(s) for s in src]
    us = _time_launches(torch, lambda i: dst[i % 6].copy_(src[i % 6]), reps)
    res["device_copy_96.8MB"] = {"bytes": 2 * n_bytes, "us": round(us, 2),
                                 "GB/s": round(2 * n_bytes / us / 1e3, 1)}
    del src, dst
    # ring merge at the ring shard shape [1,4096,24,128]
    rw = workloads.WORKLOADS["ring"]
    rows = rw.B * rw.Sq * rw.H
    mb = (3 * rows * rw.D * 2) + 3 * rows * 4
    sets = max(2, math.ceil(2 * MALL_BYTES / mb) + 1)
    accs = [(torch.randn(rw.B, rw.Sq, rw.H, rw.D, device="cuda").to(torch.bfloat16),
             torch.randn(rw.B, rw.H, rw.Sq, device="cuda"),
             torch.randn(rw.B, rw.Sq, rw.H, rw.D, device="cuda").to(torch.bfloat16),
             torch.randn(rw.B, rw.H, rw.Sq, device="cuda")) for _ in range(sets)]
    us = _time_launches(torch, lambda i: sa.dit_attn_merge(*accs[i % sets]), reps)
    res["ring_merge_bf16"] = {"bytes": mb, "us": round(us, 2), "GB/s": round(mb / us / 1e3, 1),
                              "frac_hbm_peak": round(mb / us / 1e3 / PEAK_HBM_GBPS, 4)}
    return res


def attention_configs(torch, sa, workloads, reps=10):
    """Attention (and its permutes) at every DiT shard shape: TFLOP/s and
    fraction of the bf16 MFMA peak, median of `reps` launches."""
    res = {}

    def dev_randn(shape, seed):
        g = torch.Generator(device="cuda").manual_seed(seed)
        return torch.randn(shape, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)

    def attn_entry(w, us, note=None):
        fl = w.attn_flop()
        d = {"shape_q": [w.B, w.Sq, w.H, w.D], "Skv": w.Skv, "flop": fl, "us": round(us, 2),
             "TFLOP/s": round(fl / us / 1e6, 1), "frac_mfma_peak": round(fl / us / 1e6 / PEAK_BF16_TFLOPS, 4)}
        if note:
            d["note"] = note
        return d

    for name in ("flux", "qwen_u4", "qwen_u5", "wan"):
        w = workloads.WORKLOADS[name]
        q = dev_randn((w.B, w.Sq, w.H, w.D), 1)
        k = dev_randn((w.B, w.Skv, w.H, w.D), 2)
        v = dev_randn((w.B, w.Skv, w.H, w.D), 3)
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.H, w.Sq), dtype=torch.float32, device="cuda")
        n = reps if name != "wan" else max(3, reps // 3)
        us = _time_launches(torch, lambda i: sa.dit_attn_fwd(q, k, v, o=o, lse=lse, scale=w.scale), n)
        note = None
        if name == "qwen_u5":
            note = (f"5 heads incl. the zero pad head; useful TFLOP/s (x24/25) = "
                    f"{w.attn_flop() / us / 1e6 * 24 / 25:.1f}")
        res[f"attn_{name}"] = attn_entry(w, us, note)
        del q, k, v, o, lse

    # ring shard: 4 K/V chunks of 4096 keys, each followed by a merge into the
    # bf16 accumulator, against one unchunked call over all 16384 keys
    rw = workloads.WORKLOADS["ring"]
    q = dev_randn((rw.B, rw.Sq, rw.H, rw.D), 4)
    k = dev_randn((rw.B, rw.Skv, rw.H, rw.D), 5)
    v = dev_randn((rw.B, rw.Skv, rw.H, rw.D), 6)
    chunk = rw.Skv // rw.R
    o_acc = torch.empty_like(q)
    lse_acc = torch.empty((rw.B, rw.H, rw.Sq), dtype=torch.float32, device="cuda")
    o_part = torch.empty_like(q)
    lse_part = torch.empty_like(lse_acc)
    order = [(0 - t) % rw.R for t in range(rw.R)]

    def ring(i):
        for t, c in enumerate(order):
            kc, vc = k[:, c * chunk:(c + 1) * chunk], v[:, c * chunk:(c + 1) * chunk]
            if t == 0:
                sa.dit_attn_fwd(q, kc, vc, o=o_acc, lse=lse_acc, scale=rw.scale)
            else:
                sa.dit_attn_fwd(q, kc, vc, o=o_part, lse=lse_part, scale=rw.scale)
                sa.dit_attn_merge(o_acc, lse_acc, o_part, lse_part)

    us = _time_launches(torch, ring, reps)
    fl = rw.attn_flop()
    res["attn_ring_chunked_e2e"] = {
        "chunks": rw.R, "merges": rw.R - 1, "flop": fl, "us": round(us, 2), "TFLOP/s": round(fl / us / 1e6, 1),
        "frac_mfma_peak": round(fl / us / 1e6 / PEAK_BF16_TFLOPS, 4),
        "note": "4 x attention [1,4096,24,128] x 4096 keys + 3 bf16 merges, hop order 0,3,2,1"}

    def ring_fused(i):
        for t, c in enumerate(order):
            kc, vc = k[:, c * chunk:(c + 1) * chunk], v[:, c * chunk:(c + 1) * chunk]
            if t == 0:
                sa.dit_attn_fwd(q, kc, vc, o=o_acc, lse=lse_acc, scale=rw.scale)
            else:
                sa.dit_attn_fwd_merge(q, kc, vc, o_acc, lse_acc, scale=rw.scale)

    us = _time_launches(torch, ring_fused, reps)
    res["attn_ring_fused_e2e"] = {
        "chunks": rw.R, "flop": fl, "us": round(us, 2), "TFLOP/s": round(fl / us / 1e6, 1),
        "frac_mfma_peak": round(fl / us / 1e6 / PEAK_BF16_TFLOPS, 4),
        "note": "hop 0 with dit_attn_fwd, hops 1-3 with dit_attn_fwd_merge (merge in the epilogue)"}
    # joint text+image ring: the 4 image chunks as above, then a replicated,
    # tail-padded text segment (512 slots, 300 valid) attended once with its
    # valid length and merged into the same accumulator
    k_txt = dev_randn((rw.B, 512, rw.H, rw.D), 7)
    v_txt = dev_randn((rw.B, 512, rw.H, rw.D), 8)
    txt_len = torch.full((rw.B,), 300, dtype=torch.int32, device="cuda")

    def ring_joint(i):
        ring_fused(i)
        sa.dit_attn_fwd_kvlen(q, k_txt, v_txt, txt_len, o=o_acc, lse=lse_acc, scale=rw.scale, merge=True)

    us = _time_launches(torch, ring_joint, reps)
    fl_joint = 4 * rw.B * rw.H * rw.Sq * (rw.Skv + 300) * rw.D
    res["attn_joint_text_image_ring_e2e"] = {
        "flop": fl_joint, "us": round(us, 2), "TFLOP/s": round(fl_joint / us / 1e6, 1),
        "frac_mfma_peak": round(fl_joint / us / 1e6 / PEAK_BF16_TFLOPS, 4),
        "note": "ring of 4 image chunks (fused hops) + 300 valid of 512 text keys merged once; "
                "FLOP counts valid keys only"}
    del k_txt, v_txt
    kc, vc = k[:, :chunk], v[:, :chunk]
    us = _time_launches(torch, lambda i: sa.dit_attn_fwd(q, kc, vc, o=o_part, lse=lse_part, scale=rw.scale),
                        reps)
    res["attn_ring_chunk"] = {"flop": fl // rw.R, "us": round(us, 2), "TFLOP/s": round(fl / rw.R / us / 1e6, 1),
                              "frac_mfma_peak": round(fl / rw.R / us / 1e6 / PEAK_BF16_TFLOPS, 4)}
    us = _time_launches(torch, lambda i: sa.dit_attn_fwd(q, k, v, o=o_acc, lse=lse_acc, scale=rw.scale), reps)
    res["attn_ring_unchunked"] = {"flop": fl, "us": round(us, 2), "TFLOP/s": round(fl / us / 1e6, 1),
                                  "frac_mfma_peak": round(fl / us / 1e6 / PEAK_BF16_TFLOPS, 4)}
    del q, k, v, o_acc, o_part

    # Qwen Ulysses QKV pack / unpack at U=4 (sequence pad) and U=5 (head pad)
    for name in ("qwen_u4", "qwen_u5"):
        w = workloads.WORKLOADS[name]
        L = sa.dit_a2a_layout_init(w.B, w.S, w.H_total, w.D, w.U, 1, 3)
        rank = w.U - 1  # the rank that holds the pad rows / pad head
        shard_elems = w.B * L.S_loc * w.H_total * w.D
        send_elems = w.U * L.elems_per_peer
        out_elems = w.B * w.S * L.H_loc * w.D
        shard = [torch.empty(shard_elems, dtype=torch.bfloat16, device="cuda").view(w.B, L.S_loc, w.H_total, w.D)
                 for _ in range(3)]
        for t in shard:
            t.normal_()
        send = torch.empty((w.U, 3, w.B, L.S_loc, L.H_loc, w.D), dtype=torch.bfloat16, device="cuda")
        outs = [torch.empty((w.B, w.S, L.H_loc, w.D), dtype=torch.bfloat16, device="cuda") for _ in range(3)]
        real_rows = min(L.S_loc, w.S - rank * L.S_loc)
        pack_bytes = 2 * (3 * w.B * real_rows * w.H_total * w.D + send_elems)
        unpack_bytes = 2 * (send_elems + 3 * out_elems)
        us = _time_launches(torch, lambda i: sa.dit_ulysses_pack(L, sa.DIT_SEQ_TO_HEAD, rank, shard, send=send),
                            reps)
        res[f"{name}_pack_qkv"] = {"rank": rank, "bytes": pack_bytes, "us": round(us, 2),
                                   "GB/s": round(pack_bytes / us / 1e3, 1),
                                   "frac_hbm_peak": round(pack_bytes / us / 1e3 / PEAK_HBM_GBPS, 4),
                                   "note": "MALL-warm: one buffer set"}
        us = _time_launches(torch, lambda i: sa.dit_ulysses_unpack(L, sa.DIT_SEQ_TO_HEAD, rank, send, out=outs),
                            reps)
        res[f"{name}_unpack_qkv"] = {"rank": rank, "bytes": unpack_bytes, "us": round(us, 2),
                                     "GB/s": round(unpack_bytes / us / 1e3, 1),
                                     "frac_hbm_peak": round(unpack_bytes / us / 1e3 / PEAK_HBM_GBPS, 4),
                                     "note": "MALL-warm: one buffer set"}
        del shard, send, outs
    return res


def warm_clock(torch, fn, seconds):
    """Keep the GPU busy with `fn` for about `seconds` of wall time.  The
    shader clock ramps up over a few hundred milliseconds of sustained work
    (measured with s_memtime / s_memrealtime: ~1.7 GHz in the first
    milliseconds after idle, ~2.0-2.2 GHz once warm); a DiT denoising loop
    runs its attention blocks back to back for seconds, so timings are taken
    at the warm clock."""
    t_end = time.perf_counter() + seconds
    i = 0
    while time.perf_counter() < t_end:
        for _ in range(8):
            fn(i)
            i += 1
        torch.cuda.synchronize()


def _time_launches(torch, fn, reps, warm_s=0.15):
    warm_clock(torch, fn, warm_s)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for i, (a, b) in enumerate(evs):
        a.record()
        fn(i)
        b.record()
    torch.cuda.synchronize()
    times = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
    return times[len(times) // 2]


def attn_traffic(w):
    """Counter-measured HBM bytes per attention launch, or None when the
    kernel source changed since the counters were taken."""
    import hashlib
    if w.name != ATTN_TRAFFIC["workload"]:
        return None
    with open(ATTN_SRC, "rb") as f:
        if hashlib.sha256(f.read()).hexdigest() != ATTN_TRAFFIC["src_sha256"]:
            return None
    return ATTN_TRAFFIC["fetch_bytes"] + ATTN_TRAFFIC["write_bytes"]


def cpu_baseline(w, attn_flop):
    """The fp64 oracle, as it stands, on this host: one full step of the
    same workload (rank 0), timed per stage."""
    import numpy as np
    import oracle
    from sequence_attention_amd import workloads as wl
    try:
        from threadpoolctl import threadpool_info
        threads = max([i["num_threads"] for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    L3 = oracle.a2a_layout(w.B, w.S, w.H_total, w.D, w.U, 1, 3)
    L1 = oracle.a2a_layout(w.B, w.S, w.H_total, w.D, w.U, 1, 1)
    shard = [t.float().numpy().astype(np.float64) for t in wl.seq_sharded_planes(w, 3, L3["S_loc"])]
    cfg = wl.cfg_inputs(CFG_SHAPE).numpy()
    t0 = time.perf_counter()
    send = oracle.pack_seq_to_head(shard, L3, 0)
    q, k, v = oracle.unpack_seq_to_head(send, L3, 0)
    o, _ = oracle.attention(q, k, v, w.scale)
    send1 = oracle.pack_head_to_seq([o], L1, 0)
    oracle.unpack_head_to_seq(send1, L1, 0)
    oracle.cfg_combine(cfg[0], cfg[1], 4.0)
    sec = time.perf_counter() - t0
    return {"value": round(attn_flop / sec / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", "seconds_per_step": round(sec, 3),
            "sample": f"one full {w.name} step (rank 0: QKV pack/unpack, attention, O pack/unpack, "
                      f"CFG) in float64 numpy on this host"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the hot path is the per-GPU share; collectives are outside it)", file=sys.stderr)
        sys.exit(2)
    import torch
    import sequence_attention_amd as sa
    from sequence_attention_amd import workloads
    sa.lib()  # fail loudly if the HIP library is missing
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    w = workloads.WORKLOADS[args.workload]
    one = Step(w, torch, sa, workloads, seed=0)
    n_sets = max(2, math.ceil(2 * MALL_BYTES / one.bytes()) + 1)
    steps = [one] + [Step(w, torch, sa, workloads, seed=i) for i in range(1, n_sets)]
    names = ["A1_pack_qkv", "A3_unpack_qkv", "B_attention", "D_pack_o", "E_unpack_o", "F_cfg"]
    rank = 0

    warm_clock(torch, lambda i: steps[i % n_sets].run(sa, rank), args.clock_warmup_s)
    for i in range(args.warmup):
        steps[i % n_sets].run(sa, rank)
    torch.cuda.synchronize()

    # timed region: K steps bracketed by two HIP events on the launch stream.
    # No events between kernels: each event record idles the stream for
    # several microseconds, which would stretch the step.
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for i in range(args.steps):
        steps[i % n_sets].run(sa, rank)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = start.elapsed_time(end) / args.steps

    # per-kernel average launch duration: each kernel of the step launched K
    # times back to back over the rotated input sets, the run bracketed by
    # two events on the same stream (region time / K)
    per_kernel = {}
    for n in names:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        warm_clock(torch, lambda i: steps[i % n_sets].run(sa, rank, only=n), 0.1)
        a.record()
        for i in range(args.steps):
            steps[i % n_sets].run(sa, rank, only=n)
        b.record()
        torch.cuda.synchronize()
        per_kernel[n] = a.elapsed_time(b) / args.steps * 1e3
    attn_us = per_kernel["B_attention"]

    attn_flop = w.attn_flop()
    value = attn_flop / (ms_per_step * 1e-3) / 1e12
    achieved = attn_flop / (attn_us * 1e-6) / 1e12
    kb = kernel_bytes(one)
    kernels = {}
    for n in names:
        d = {"us": round(per_kernel[n], 2)}
        if n in kb:
            d["bytes"] = kb[n]
            d["GB/s"] = round(kb[n] / per_kernel[n] / 1e3, 1)
            d["frac_hbm_peak"] = round(kb[n] / per_kernel[n] / 1e3 / PEAK_HBM_GBPS, 4)
        else:
            d["flop"] = attn_flop
            d["TFLOP/s"] = round(achieved, 1)
        kernels[n] = d

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.note}", "B": w.B, "S": w.S, "H_total": w.H_total,
                   "H_rank": w.H, "D": w.D, "ulysses": w.U, "ring": w.R, "rank": rank,
                   "input_sets_rotated": n_sets, "wall_s_timed": round(wall, 3),
                   "clock_warmup_s": args.clock_warmup_s},
        "roofline": {"kernel": "attn_bf16_kernel<128>", "bound": "mfma", "achieved": round(achieved, 1),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": attn_traffic(w),
                     "algorithmic_flop_per_launch": attn_flop, "avg_launch_us": round(attn_us, 2)},
        "kernels": kernels,
    }
    if not args.no_side:
        result["side"] = side_measurements(torch, sa, workloads)
    if not args.no_configs:
        result["configs"] = attention_configs(torch, sa, workloads)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, attn_flop)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
