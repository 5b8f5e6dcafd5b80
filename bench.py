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
the measured step time.  Inputs are resident in HBM before timing; input
sets rotate so that successive steps do not find their data in the 256 MB
Infinity Cache.  The JSON line also carries the attention kernel's roofline
(HIP events on the launch stream), per-kernel times, side measurements of
the headline permute (Wan [1,9450,40,128]) and of the ring merge, and the
fp64 CPU oracle timed on this host on the same workload.

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


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="flux", choices=["flux", "qwen_u4", "qwen_u5", "wan"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-side", action="store_true", help="skip the side permute / merge measurements")
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

    def run(self, sa, rank, ev=None):
        """Enqueue one step; ev: optional dict name -> (start, end) events."""
        S2H, H2S = sa.DIT_SEQ_TO_HEAD, sa.DIT_HEAD_TO_SEQ

        def timed(name, fn):
            if ev is not None:
                ev[name][0].record()
            fn()
            if ev is not None:
                ev[name][1].record()

        timed("A1_pack_qkv", lambda: sa.dit_ulysses_pack(self.L3, S2H, rank, self.shard, send=self.send3))
        timed("A3_unpack_qkv", lambda: sa.dit_ulysses_unpack(self.L3, S2H, rank, self.send3, out=self.qkv))
        timed("B_attention", lambda: sa.dit_attn_fwd(*self.qkv, o=self.o, lse=self.lse, scale=self.w.scale))
        timed("D_pack_o", lambda: sa.dit_ulysses_pack(self.L1, H2S, rank, [self.o], send=self.send1))
        timed("E_unpack_o", lambda: sa.dit_ulysses_unpack(self.L1, H2S, rank, self.send1, out=[self.out]))
        timed("F_cfg", lambda: sa.dit_cfg_combine(self.u, self.c, 4.0, out=self.guided))


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


def _time_launches(torch, fn, reps):
    for i in range(3):
        fn(i)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for i, (a, b) in enumerate(evs):
        a.record()
        fn(i)
        b.record()
    torch.cuda.synchronize()
    times = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
    return times[len(times) // 2]


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

    for i in range(args.warmup):
        steps[i % n_sets].run(sa, rank)
    torch.cuda.synchronize()

    # timed region: K steps, events around every kernel on the launch stream
    ev = [{n: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for n in names}
          for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for i in range(args.steps):
        steps[i % n_sets].run(sa, rank, ev[i])
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = start.elapsed_time(end) / args.steps
    per_kernel = {n: sum(e[n][0].elapsed_time(e[n][1]) for e in ev) / args.steps * 1e3 for n in names}

    attn_flop = w.attn_flop()
    value = attn_flop / (ms_per_step * 1e-3) / 1e12
    attn_us = per_kernel["B_attention"]
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
                   "input_sets_rotated": n_sets, "wall_s_timed": round(wall, 3)},
        "roofline": {"kernel": "attn_bf16_kernel<128>", "bound": "mfma", "achieved": round(achieved, 1),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "algorithmic_flop_per_launch": attn_flop, "avg_launch_us": round(attn_us, 2)},
        "kernels": kernels,
    }
    if not args.no_side:
        result["side"] = side_measurements(torch, sa, workloads)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, attn_flop)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
