#!/usr/bin/env python3
"""Throughput of the per-GPU DiT sequence-parallel attention hot path.

One step = one pass of the whole hot path of one Ulysses rank over one
batch of synthetic input, the FLUX.1-like 1024x1024 shard by default
(B=1, joint sequence 4608 = 4096 image + 512 text tokens, 24 heads of 128,
Ulysses degree 2, ring degree 1):

  A1  QKV sequence-to-head pack   [1,2304,24,128] x3 -> [2,3,1,2304,12,128]
  ABD attention with LSE reading Q, K, V straight from the receive buffer
      [2,3,1,2304,12,128] (the send buffer stands in for the received one:
      same bytes and shape; the all-to-all itself is a collective, outside
      this path) and storing O straight into the head-to-sequence send
      buffer [2,1,1,2304,12,128]; ring degree 1, so the hop loop is one chunk
      and no merge (the unpack A3, attention B and pack D of the method in
      one kernel; the unfused launches are timed beside it)
  E   O unpack                    -> [1,2304,24,128]
  F   CFG combine                 [2,4096,64] fp32 latent prediction, g = 4

`value` is the step's algorithmic attention FLOP (4*B*H*Sq*Skv*D) divided by
the measured step time (K steps bracketed by two HIP events on the launch
stream).  Inputs are resident in HBM before timing; input sets rotate so
that successive steps do not find their data in the 256 MB Infinity Cache.
Before the warm-up steps, untimed steps run for --clock-warmup-s seconds:
the GPU clock needs a few hundred milliseconds of sustained work to leave
its idle level, and a denoising loop runs its attention blocks for seconds.
A shader-clock probe runs right after the timed steps and its reading is
part of the JSON line.

Kernel figures (`kernels`, `side`, the permutes in `configs`) are average
launch durations: N launches of the kernel over rotated buffer sets are
captured in one HIP graph after an eager warm-up, and the graph is replayed
between two events (no host launch gaps, so microsecond kernels are timed
as kernels).  Attention shapes also report the median and minimum of
per-launch events.  The roofline of the dominant kernel (the step's
attention) uses its graph-replay average.  `cpu_baseline` times the fp64
oracle on this host's cores.

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload flux]
       python bench.py --trace-summary prof_results.db   (rocprofv3 kernel trace -> table)
       python bench.py --pmc-summary counter_collection.csv   (rocprofv3 --pmc -> table)
"""

from __future__ import annotations

import argparse
import json
import math
import os
import statistics
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

# HBM bytes per launch of the attention kernel, from two rocprofv3 --pmc
# passes (FETCH_SIZE, WRITE_SIZE), each scaled by what the counter reads for
# a device copy of known size (the factors are in the profile).  Valid only
# for the kernel code they were taken on (SHA-256 below, of the source with
# its // comments and blank lines removed): any change to that code reports
# traffic as null until the counters are taken again.
ATTN_SRC = os.path.join(ROOT, "sequence_attention_amd", "csrc", "attn_fwd_bf16.hip")
ATTN_TRAFFIC = {
    "src_sha256": "66985ac27e3210730afbaec9b7c0c346b43b9c08830a50f1822cef183f8b33d5",
    # shape: (read bytes, write bytes) per launch; flux_a2a is the step's
    # attention from the receive buffer (dit_attn_fwd_a2a)
    "per_shape": {"flux": (52_175_872, 14_377_165), "flux_a2a": (52_184_064, 14_377_677),
                  "qwen_u4": (151_069_082, 55_749_222),
                  "qwen_u5": (133_027_021, 45_325_619), "wan": (2_109_947_699, 98_289_254),
                  "ring_chunk": (111_770_214, 61_230_694), "ring_unchunked": (262_763_315, 61_251_686),
                  "ring_fused_hop": (137_255_117, 65_658_163)},
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="flux", choices=["flux", "qwen_u4", "qwen_u5", "wan"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-baseline", default="full", choices=["full", "step"],
                    help="full: every config the oracle times (minutes of host time); step: the FLUX step only")
    ap.add_argument("--no-side", action="store_true", help="skip the side permute / merge measurements")
    ap.add_argument("--no-configs", action="store_true", help="skip the per-config attention timings")
    ap.add_argument("--clock-warmup-s", type=float, default=0.5,
                    help="seconds of untimed steps before the warm-up steps, to bring the GPU clock up")
    ap.add_argument("--graph-launches", type=int, default=20,
                    help="launches captured per graph for the kernel timings")
    ap.add_argument("--only", metavar="NAMES",
                    help="comma-separated parts to run alone, for profiling one measurement per run: "
                         "'kernels' (the step's per-kernel timings), 'side', or entries of `configs`")
    ap.add_argument("--trace-summary", metavar="DB",
                    help="print the per-kernel table of a rocprofv3 kernel-trace database and exit")
    ap.add_argument("--pmc-summary", metavar="CSV",
                    help="print the per-kernel table of a rocprofv3 --pmc counter CSV and exit")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# timing helpers
# ---------------------------------------------------------------------------

def warm_clock(torch, fn, seconds):
    """Keep the GPU busy with `fn` for about `seconds` of wall time.  The
    shader clock ramps up over a few hundred milliseconds of sustained work
    (~1.7 GHz in the first milliseconds after idle, ~2.0-2.2 GHz once warm,
    as the clock probe shows); a DiT denoising loop runs its attention blocks
    back to back for seconds, so timings are taken at the warm clock."""
    t_end = time.perf_counter() + seconds
    i = 0
    while time.perf_counter() < t_end:
        for _ in range(8):
            fn(i)
            i += 1
        torch.cuda.synchronize()


def time_graph(torch, fn, launches, replays=3, warm_s=0.1):
    """Average launch duration (us) of fn(0) .. fn(launches-1) captured in one
    HIP graph and replayed `replays` times between two events, after
    untimed replays for `warm_s` seconds (the first replays after a capture
    run slow, and they bring the clock to its sustained level)."""
    fn(0)  # one eager call, so the library's per-device facts exist before the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(launches):
            fn(i)
    t_end = time.perf_counter() + warm_s
    g.replay()
    torch.cuda.synchronize()
    while time.perf_counter() < t_end:
        g.replay()
        torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(replays):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / (replays * launches)
    del g
    return us


def time_events(torch, fn, reps, warm_s=0.1):
    """Median and minimum (us) of per-launch events around fn(i)."""
    warm_clock(torch, fn, warm_s)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for i, (a, b) in enumerate(evs):
        a.record()
        fn(i)
        b.record()
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
    return t[len(t) // 2], t[0]


def rot_sets(bytes_per_set):
    """Buffer sets to rotate so that one pass over them exceeds twice the
    Infinity Cache."""
    return max(2, math.ceil(2 * MALL_BYTES / max(1, bytes_per_set)) + 1)


def hbm_entry(nbytes, us, **extra):
    d = dict(extra)
    d.update({"bytes": int(nbytes), "us": round(us, 2), "GB/s": round(nbytes / us / 1e3, 1),
              "frac_hbm_peak": round(nbytes / us / 1e3 / PEAK_HBM_GBPS, 4)})
    return d


def attn_code_sha256(path=None):
    """SHA-256 of the attention kernel source without // comments, trailing
    blanks and empty lines: a comment edit keeps the counters valid, any
    change to the code does not."""
    import hashlib
    with open(path or ATTN_SRC, encoding="utf-8") as f:
        lines = [ln.split("//", 1)[0].rstrip() for ln in f.read().splitlines()]
    return hashlib.sha256("\n".join(ln for ln in lines if ln).encode()).hexdigest()


def attn_traffic(shape_name):
    """Counter-measured HBM bytes per attention launch at this shape, or
    None when the kernel source changed since the counters were taken."""
    per = ATTN_TRAFFIC["per_shape"].get(shape_name)
    if per is None or ATTN_TRAFFIC["src_sha256"] is None:
        return None
    if attn_code_sha256() != ATTN_TRAFFIC["src_sha256"]:
        return None
    return per[0] + per[1]


def attn_roofline(shape_name, flop, avg_us, ev_median=None, ev_min=None, **extra):
    achieved = flop / avg_us / 1e6
    d = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
         "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": attn_traffic(shape_name),
         "flop": int(flop), "avg_launch_us": round(avg_us, 2)}
    if ev_median is not None:
        d["event_median_us"] = round(ev_median, 2)
        d["event_min_us"] = round(ev_min, 2)
    d.update(extra)
    return d


# ---------------------------------------------------------------------------
# the step
# ---------------------------------------------------------------------------

class Step:
    """Buffers and launches of one rank's hot-path step (one input set)."""

    NAMES = ("A1_pack_qkv", "ABD_attention_a2a", "E_unpack_o", "F_cfg")
    # the launches ABD replaces: the unpack A3 and attention into the send
    # buffer BD, which itself replaces attention B and the pack D
    UNFUSED = ("A3_unpack_qkv", "BD_attention_send", "B_attention", "D_pack_o")

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
        ws = sa.dit_attn_workspace_size(w.B, w.S, w.S, L3.H_loc, w.D)
        self.ws = torch.zeros(max(ws, 256), dtype=torch.uint8, device=dev)

    def bytes(self):
        n = 0
        for t in self.shard + self.qkv + [self.send3, self.o, self.lse, self.send1, self.out, self.u,
                                          self.c, self.guided]:
            n += t.numel() * t.element_size()
        return n

    def run(self, sa, rank, only=None):
        """Enqueue one step (or only its launch `only`, which may also name
        one of the unfused pair)."""
        S2H, H2S = sa.DIT_SEQ_TO_HEAD, sa.DIT_HEAD_TO_SEQ
        w = self.w
        launches = {
            "A1_pack_qkv": lambda: sa.dit_ulysses_pack(self.L3, S2H, rank, self.shard, send=self.send3),
            "A3_unpack_qkv": lambda: sa.dit_ulysses_unpack(self.L3, S2H, rank, self.send3, out=self.qkv),
            "ABD_attention_a2a": lambda: sa.dit_attn_fwd_a2a(self.send3, self.L3, rank, send=self.send1,
                                                             lse=self.lse, scale=w.scale, workspace=self.ws),
            "BD_attention_send": lambda: sa.dit_attn_fwd_send(*self.qkv, self.L1, rank, send=self.send1,
                                                              lse=self.lse, scale=w.scale, workspace=self.ws),
            "E_unpack_o": lambda: sa.dit_ulysses_unpack(self.L1, H2S, rank, self.send1, out=[self.out]),
            "F_cfg": lambda: sa.dit_cfg_combine(self.u, self.c, 4.0, out=self.guided),
            "B_attention": lambda: sa.dit_attn_fwd(*self.qkv, o=self.o, lse=self.lse, scale=w.scale,
                                                   workspace=self.ws),
            "D_pack_o": lambda: sa.dit_ulysses_pack(self.L1, H2S, rank, [self.o], send=self.send1),
        }
        if only is not None:
            launches[only]()
            return
        for name in self.NAMES:
            launches[name]()


def kernel_pools(w, torch, sa, step, rank):
    """For each launch of the step, a function of the launch index over its
    own rotated buffer sets (at least twice the Infinity Cache of that
    launch's own traffic), so every kernel figure reads cold data."""
    dev, bf16 = "cuda", torch.bfloat16
    L3, L1 = step.L3, step.L1
    S2H, H2S = sa.DIT_SEQ_TO_HEAD, sa.DIT_HEAD_TO_SEQ
    kb = kernel_bytes(step)
    o_b = w.B * w.S * L3.H_loc * w.D * 2
    kb["BD_attention_send"] = 3 * o_b + kb["D_pack_o"] - o_b
    kb["ABD_attention_a2a"] = w.U * L3.elems_per_peer * 2 + kb["D_pack_o"] - o_b
    kb["B_attention"] = 4 * o_b
    shard = lambda: [torch.empty((w.B, L3.S_loc, w.H_total, w.D), dtype=bf16, device=dev).normal_()
                     for _ in range(3)]
    send3 = lambda: torch.empty((w.U, 3, w.B, L3.S_loc, L3.H_loc, w.D), dtype=bf16, device=dev).normal_()
    heads = lambda n: [torch.empty((w.B, w.S, L3.H_loc, w.D), dtype=bf16, device=dev).normal_() for _ in range(n)]
    send1 = lambda: torch.empty((w.U, 1, w.B, L1.S_loc, L1.H_loc, w.D), dtype=bf16, device=dev).normal_()
    lse = lambda: torch.empty((w.B, L3.H_loc, w.S), dtype=torch.float32, device=dev)
    out = lambda: torch.empty((w.B, L1.S_loc, w.H_total, w.D), dtype=bf16, device=dev)
    cfg = lambda: torch.randn((3,) + CFG_SHAPE[1:], device=dev)
    make = {
        "A1_pack_qkv": (lambda: (shard(), send3()),
                        lambda b: sa.dit_ulysses_pack(L3, S2H, rank, b[0], send=b[1])),
        "A3_unpack_qkv": (lambda: (send3(), heads(3)),
                          lambda b: sa.dit_ulysses_unpack(L3, S2H, rank, b[0], out=b[1])),
        "ABD_attention_a2a": (lambda: (send3(), send1(), lse()),
                              lambda b: sa.dit_attn_fwd_a2a(b[0], L3, rank, send=b[1], lse=b[2], scale=w.scale,
                                                            workspace=step.ws)),
        "BD_attention_send": (lambda: (heads(3), send1(), lse()),
                              lambda b: sa.dit_attn_fwd_send(*b[0], L1, rank, send=b[1], lse=b[2], scale=w.scale,
                                                             workspace=step.ws)),
        "E_unpack_o": (lambda: (send1(), out()),
                       lambda b: sa.dit_ulysses_unpack(L1, H2S, rank, b[0], out=[b[1]])),
        "F_cfg": (cfg, lambda b: sa.dit_cfg_combine(b[0], b[1], 4.0, out=b[2])),
        "B_attention": (lambda: (heads(4), lse()),
                        lambda b: sa.dit_attn_fwd(*b[0][:3], o=b[0][3], lse=b[1], scale=w.scale,
                                                  workspace=step.ws)),
        "D_pack_o": (lambda: (heads(1), send1()),
                     lambda b: sa.dit_ulysses_pack(L1, H2S, rank, b[0], send=b[1])),
    }
    return make, kb


def kernel_timings(w, torch, sa, workloads, step, rank, launches):
    """Average launch duration of each launch of the step (and of the
    unfused pair BD replaces): graph replay, each kernel over buffer sets of
    its own, rotated beyond the Infinity Cache.  Returns the `kernels`
    entries and the attention's average launch duration."""
    make, kb_all = kernel_pools(w, torch, sa, step, rank)
    kb = kernel_bytes(step)
    attn_flop = w.attn_flop()
    kernels, per_kernel = {}, {}
    for n in Step.NAMES + Step.UNFUSED:
        alloc, call = make[n]
        k_sets = rot_sets(kb_all[n])
        bufs = [alloc() for _ in range(k_sets)]
        per_kernel[n] = time_graph(torch, lambda i: call(bufs[i % k_sets]), max(launches, k_sets))
        del bufs
        if n in kb:
            kernels[n] = hbm_entry(kb[n], per_kernel[n], sets=k_sets)
        else:
            kernels[n] = {"us": round(per_kernel[n], 2), "flop": attn_flop,
                          "TFLOP/s": round(attn_flop / per_kernel[n] / 1e6, 1), "sets": k_sets}
    kernels["ABD_attention_a2a"]["note"] = ("attention reading Q, K, V from the receive buffer and storing O "
                                            "into the send buffer (replaces A3 + BD)")
    kernels["BD_attention_send"]["note"] = "attention storing O into the send buffer (replaces B + D)"
    kernels["unfused_A3_plus_BD_us"] = round(per_kernel["A3_unpack_qkv"] + per_kernel["BD_attention_send"], 2)
    kernels["unfused_B_plus_D_us"] = round(per_kernel["B_attention"] + per_kernel["D_pack_o"], 2)
    return kernels, per_kernel["ABD_attention_a2a"]


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
    return {"A1_pack_qkv": shard3 + send3, "A3_unpack_qkv": send3 + qkv, "D_pack_o": o + send1,
            "E_unpack_o": send1 + out, "F_cfg": cfg}


# ---------------------------------------------------------------------------
# attention at every shard shape, and the ring
# ---------------------------------------------------------------------------

def attention_configs(torch, sa, workloads, launches, reps=20, only=None):
    res = {}

    def want(name):
        return only is None or name in only

    def dev_randn(shape, seed):
        g = torch.Generator(device="cuda").manual_seed(seed)
        return torch.randn(shape, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)

    def ws_for(B, Sq, Skv, H, D, merge=False):
        n = sa.dit_attn_workspace_size(B, Sq, Skv, H, D, merge=merge)
        return torch.zeros(max(n, 256), dtype=torch.uint8, device="cuda")

    for name in ("flux", "qwen_u4", "qwen_u5", "wan"):
        if not want(f"attn_{name}"):
            continue
        w = workloads.WORKLOADS[name]
        q = dev_randn((w.B, w.Sq, w.H, w.D), 1)
        k = dev_randn((w.B, w.Skv, w.H, w.D), 2)
        v = dev_randn((w.B, w.Skv, w.H, w.D), 3)
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.H, w.Sq), dtype=torch.float32, device="cuda")
        ws = ws_for(w.B, w.Sq, w.Skv, w.H, w.D)
        fn = lambda i: sa.dit_attn_fwd(q, k, v, o=o, lse=lse, scale=w.scale, workspace=ws)
        big = name == "wan"
        avg = time_graph(torch, fn, 3 if big else launches, replays=1 if big else 3)
        med, mn = time_events(torch, fn, 5 if big else reps)
        extra = {"shape_q": [w.B, w.Sq, w.H, w.D], "Skv": w.Skv}
        if name == "qwen_u5":
            extra["useful_TFLOP/s"] = round(w.attn_flop() / avg / 1e6 * 24 / 25, 1)
            extra["note"] = "5 heads incl. the zero pad head; useful = x24/25"
        res[f"attn_{name}"] = attn_roofline(name, w.attn_flop(), avg, med, mn, **extra)
        del q, k, v, o, lse, ws

    # ring shard: 4 K/V chunks of 4096 keys merged into one accumulator
    ring_names = ("attn_ring_chunked_e2e", "attn_ring_fused_e2e", "attn_joint_text_image_ring_e2e",
                  "attn_ring_chunk", "attn_ring_fused_hop", "attn_ring_unchunked")
    if any(want(n) for n in ring_names):
        ring_configs(torch, sa, workloads, launches, reps, want, dev_randn, ws_for, res)
    qwen_permutes(torch, sa, workloads, launches, want, res)
    return res


def ring_configs(torch, sa, workloads, launches, reps, want, dev_randn, ws_for, res):
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
    ws_c = ws_for(rw.B, rw.Sq, chunk, rw.H, rw.D)
    ws_m = ws_for(rw.B, rw.Sq, chunk, rw.H, rw.D, merge=True)
    ws_u = ws_for(rw.B, rw.Sq, rw.Skv, rw.H, rw.D)
    kc = [k[:, c * chunk:(c + 1) * chunk] for c in range(rw.R)]
    vc = [v[:, c * chunk:(c + 1) * chunk] for c in range(rw.R)]

    def ring(i):
        for t, c in enumerate(order):
            if t == 0:
                sa.dit_attn_fwd(q, kc[c], vc[c], o=o_acc, lse=lse_acc, scale=rw.scale, workspace=ws_c)
            else:
                sa.dit_attn_fwd(q, kc[c], vc[c], o=o_part, lse=lse_part, scale=rw.scale, workspace=ws_c)
                sa.dit_attn_merge(o_acc, lse_acc, o_part, lse_part)

    def ring_fused(i):
        for t, c in enumerate(order):
            if t == 0:
                sa.dit_attn_fwd(q, kc[c], vc[c], o=o_acc, lse=lse_acc, scale=rw.scale, workspace=ws_c)
            else:
                sa.dit_attn_fwd_merge(q, kc[c], vc[c], o_acc, lse_acc, scale=rw.scale, workspace=ws_m)

    fl = rw.attn_flop()
    passes = max(2, launches // 4)
    us = us_f = None
    if want("attn_ring_chunked_e2e"):
        us = time_graph(torch, ring, passes, replays=2)
        res["attn_ring_chunked_e2e"] = attn_roofline(
            "ring_chunked_e2e", fl, us, chunks=rw.R, merges=rw.R - 1,
            note="4 x attention [1,4096,24,128] x 4096 keys + 3 bf16 merges, hop order 0,3,2,1; "
                 "avg_launch_us is one whole pass")
    if want("attn_ring_fused_e2e"):
        us_f = time_graph(torch, ring_fused, passes, replays=2)
        res["attn_ring_fused_e2e"] = attn_roofline(
            "ring_fused_e2e", fl, us_f, chunks=rw.R,
            note="hop 0 with dit_attn_fwd, hops 1-3 with dit_attn_fwd_merge (merge in the epilogue); "
                 "avg_launch_us is one whole pass")
    # joint text+image ring: the fused ring, then 300 valid of 512 replicated
    # text keys attended once and merged into the same accumulator
    k_txt = dev_randn((rw.B, 512, rw.H, rw.D), 7)
    v_txt = dev_randn((rw.B, 512, rw.H, rw.D), 8)
    txt_len = torch.full((rw.B,), 300, dtype=torch.int32, device="cuda")

    def ring_joint(i):
        ring_fused(i)
        sa.dit_attn_fwd_kvlen(q, k_txt, v_txt, txt_len, o=o_acc, lse=lse_acc, scale=rw.scale, merge=True)

    if want("attn_joint_text_image_ring_e2e"):
        us_j = time_graph(torch, ring_joint, passes, replays=2)
        fl_joint = 4 * rw.B * rw.H * rw.Sq * (rw.Skv + 300) * rw.D
        res["attn_joint_text_image_ring_e2e"] = attn_roofline(
            "joint_e2e", fl_joint, us_j,
            note="ring of 4 image chunks (fused hops) + 300 valid of 512 text keys merged once; "
                 "FLOP counts valid keys only")
    del k_txt, v_txt
    if want("attn_ring_chunk"):
        fn = lambda i: sa.dit_attn_fwd(q, kc[i % rw.R], vc[i % rw.R], o=o_part, lse=lse_part, scale=rw.scale,
                                       workspace=ws_c)
        avg = time_graph(torch, fn, launches)
        med, mn = time_events(torch, fn, reps)
        res["attn_ring_chunk"] = attn_roofline("ring_chunk", fl // rw.R, avg, med, mn)
    if want("attn_ring_fused_hop"):
        fn = lambda i: sa.dit_attn_fwd_merge(q, kc[1 + i % 3], vc[1 + i % 3], o_acc, lse_acc, scale=rw.scale,
                                             workspace=ws_m)
        avg = time_graph(torch, fn, launches)
        res["attn_ring_fused_hop"] = attn_roofline("ring_fused_hop", fl // rw.R, avg,
                                                   note="one dit_attn_fwd_merge hop at the chunk shape")
    if want("attn_ring_unchunked"):
        fn = lambda i: sa.dit_attn_fwd(q, k, v, o=o_acc, lse=lse_acc, scale=rw.scale, workspace=ws_u)
        avg = time_graph(torch, fn, max(4, launches // 4))
        med, mn = time_events(torch, fn, max(5, reps // 4))
        res["attn_ring_unchunked"] = attn_roofline("ring_unchunked", fl, avg, med, mn)
        if us is not None and us_f is not None:
            res["ring_chunking_ratio"] = {
                "fused_e2e_over_unchunked": round(us_f / avg, 4),
                "chunked_e2e_over_unchunked": round(us / avg, 4)}
    del q, k, v, o_acc, o_part, kc, vc


def qwen_permutes(torch, sa, workloads, launches, want, res):

    # Qwen Ulysses QKV pack / unpack at U=4 (sequence pad) and U=5 (head pad),
    # on the rank that holds the pad rows / pad head, buffers rotated
    for name in ("qwen_u4", "qwen_u5"):
        if not (want(f"{name}_pack_qkv") or want(f"{name}_unpack_qkv")):
            continue
        w = workloads.WORKLOADS[name]
        L = sa.dit_a2a_layout_init(w.B, w.S, w.H_total, w.D, w.U, 1, 3)
        rank = w.U - 1
        send_elems = w.U * L.elems_per_peer
        out_elems = w.B * w.S * L.H_loc * w.D
        real_rows = min(L.S_loc, w.S - rank * L.S_loc)
        pack_bytes = 2 * (3 * w.B * real_rows * w.H_total * w.D + send_elems)
        unpack_bytes = 2 * (send_elems + 3 * out_elems)
        sets = rot_sets(min(pack_bytes, unpack_bytes))   # each leg touches half of a set
        bufs = []
        for _ in range(sets):
            shard = [torch.empty((w.B, L.S_loc, w.H_total, w.D), dtype=torch.bfloat16, device="cuda").normal_()
                     for _ in range(3)]
            send = torch.empty((w.U, 3, w.B, L.S_loc, L.H_loc, w.D), dtype=torch.bfloat16, device="cuda")
            outs = [torch.empty((w.B, w.S, L.H_loc, w.D), dtype=torch.bfloat16, device="cuda") for _ in range(3)]
            bufs.append((shard, send, outs))
        us = time_graph(torch, lambda i: sa.dit_ulysses_pack(L, sa.DIT_SEQ_TO_HEAD, rank, bufs[i % sets][0],
                                                             send=bufs[i % sets][1]), launches)
        res[f"{name}_pack_qkv"] = hbm_entry(pack_bytes, us, rank=rank, sets=sets)
        us = time_graph(torch, lambda i: sa.dit_ulysses_unpack(L, sa.DIT_SEQ_TO_HEAD, rank, bufs[i % sets][1],
                                                               out=bufs[i % sets][2]), launches)
        res[f"{name}_unpack_qkv"] = hbm_entry(unpack_bytes, us, rank=rank, sets=sets)
        del bufs


# ---------------------------------------------------------------------------
# side measurements: the headline permute, fused receive preparation,
# padding-free maps, FP8, conversion, merge, copy references
# ---------------------------------------------------------------------------

def side_measurements(torch, sa, workloads, launches):
    res = {}
    bf16 = torch.bfloat16
    w = workloads.WORKLOADS["wan"]
    for n_planes in (1, 3):
        L = sa.dit_a2a_layout_init(w.B, w.S, w.H_total, w.D, w.U, 1, n_planes)
        plane_bytes = w.B * L.S_loc * w.H_total * w.D * 2
        moved = 2 * n_planes * plane_bytes
        sets = rot_sets(moved)
        bufs = []
        for _ in range(sets):
            shard = [torch.empty((w.B, L.S_loc, w.H_total, w.D), dtype=bf16, device="cuda").normal_()
                     for _ in range(n_planes)]
            send = torch.empty((w.U, n_planes, w.B, L.S_loc, L.H_loc, w.D), dtype=bf16, device="cuda")
            bufs.append((shard, send))
        us = time_graph(torch, lambda i: sa.dit_ulysses_pack(L, sa.DIT_SEQ_TO_HEAD, 0, bufs[i % sets][0],
                                                             send=bufs[i % sets][1]), launches)
        res[f"wan_pack_{n_planes}plane"] = hbm_entry(moved, us)
        # head-to-sequence unpack: [U,n,B,S_loc,H_loc,D] -> n x [B,S_loc,H,D]
        us = time_graph(torch, lambda i: sa.dit_ulysses_unpack(L, sa.DIT_HEAD_TO_SEQ, 0, bufs[i % sets][1],
                                                               out=bufs[i % sets][0]), launches)
        res[f"wan_unpack_{n_planes}plane"] = hbm_entry(moved, us)
        del bufs

    # fused receive preparation (unpack + RoPE on Q and K) at the FLUX U=2
    # shape, against the plain unpack of the same buffer
    fw = workloads.WORKLOADS["flux"]
    L = sa.dit_a2a_layout_init(fw.B, fw.S, fw.H_total, fw.D, fw.U, 1, 3)
    recv_bytes = fw.U * L.elems_per_peer * 2
    plane_bytes = 3 * fw.B * fw.S * L.H_loc * fw.D * 2
    cos, sin = workloads.rope_tables(fw.S, fw.D)
    cos, sin = cos.to("cuda"), sin.to("cuda")
    table_bytes = 2 * cos.numel() * 4
    sets = rot_sets(recv_bytes + plane_bytes)
    bufs = [(torch.empty((fw.U, 3, fw.B, L.S_loc, L.H_loc, fw.D), dtype=bf16, device="cuda").normal_(),
             [torch.empty((fw.B, fw.S, L.H_loc, fw.D), dtype=bf16, device="cuda") for _ in range(3)])
            for _ in range(sets)]
    us = time_graph(torch, lambda i: sa.dit_ulysses_unpack_rope(L, 0, bufs[i % sets][0], cos, sin,
                                                                out=bufs[i % sets][1]), launches)
    res["flux_unpack_rope_qkv"] = hbm_entry(recv_bytes + plane_bytes + table_bytes, us)
    us = time_graph(torch, lambda i: sa.dit_ulysses_unpack(L, sa.DIT_SEQ_TO_HEAD, 0, bufs[i % sets][0],
                                                           out=bufs[i % sets][1]), launches)
    res["flux_unpack_qkv_plain"] = hbm_entry(recv_bytes + plane_bytes, us)
    del bufs

    # the QKV pack from float32 planes with the conversion to bf16 / f16
    # (round to nearest even) at the FLUX U=2 shape
    for name, code, dt in (("bf16", sa.DIT_BF16, bf16), ("f16", sa.DIT_F16, torch.float16)):
        Lc = sa.dit_a2a_layout_init(fw.B, fw.S, fw.H_total, fw.D, fw.U, 1, 3, code)
        shard_b = 3 * fw.B * Lc.S_loc * fw.H_total * fw.D * 4
        send_b = fw.U * Lc.elems_per_peer * 2
        sets = rot_sets(shard_b + send_b)
        bufs = [([torch.empty((fw.B, Lc.S_loc, fw.H_total, fw.D), device="cuda").normal_() for _ in range(3)],
                 torch.empty((fw.U, 3, fw.B, Lc.S_loc, Lc.H_loc, fw.D), dtype=dt, device="cuda"))
                for _ in range(sets)]
        us = time_graph(torch, lambda i: sa.dit_ulysses_pack_convert(Lc, sa.DIT_SEQ_TO_HEAD, 0, bufs[i % sets][0],
                                                                     send=bufs[i % sets][1]), launches)
        res[f"flux_pack_convert_qkv_f32_to_{name}"] = hbm_entry(shard_b + send_b, us)
        del bufs

    # padding-free split of FLUX at 1008x1008 (S = 512 text + 63*63 image =
    # 4481 rows over U = 4): packed QKV sequence-to-head pack and unpack of
    # rank 0, against the padded layout of the same sequence; GB/s on the
    # real bytes
    S_u, U_u, H_u, D_u = 4481, 4, 24, 128
    Lu = sa.dit_a2a_uneven_init(1, S_u, H_u, D_u, U_u, 3)
    Lp = sa.dit_a2a_layout_init(1, S_u, H_u, D_u, U_u, 1, 3)
    r_rows, _ = Lu.counts()
    real = {"pack": 2 * 3 * r_rows[0] * H_u * D_u * 2, "unpack": 2 * 3 * S_u * (H_u // U_u) * D_u * 2}
    sets = rot_sets(min(real.values()))   # each leg touches its own buffers only
    bufs = []
    for _ in range(sets):
        shard_u = [torch.empty((1, r_rows[0], H_u, D_u), dtype=bf16, device="cuda").normal_() for _ in range(3)]
        shard_p = [torch.empty((1, Lp.S_loc, H_u, D_u), dtype=bf16, device="cuda").normal_() for _ in range(3)]
        send_u = sa.dit_ulysses_pack_uneven(Lu, sa.DIT_SEQ_TO_HEAD, 0, shard_u)
        send_p = sa.dit_ulysses_pack(Lp, sa.DIT_SEQ_TO_HEAD, 0, shard_p)
        recv_u = torch.empty(sum(sa.dit_a2a_uneven_sizes(Lu, sa.DIT_SEQ_TO_HEAD, 0)[1]),
                             dtype=bf16, device="cuda").normal_()
        out = [torch.empty((1, S_u, H_u // U_u, D_u), dtype=bf16, device="cuda") for _ in range(3)]
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
        us = time_graph(torch, lambda i, fn=fn: fn(bufs[i % sets]), launches)
        res[name] = hbm_entry(real[kind], us, note="bytes: the real (unpadded) rows")
    del bufs

    # Ring Anything trim of the gathered FLUX 1008x1008 K and V over a ring of 4
    Lr2 = sa.dit_a2a_uneven_init(1, S_u, H_u, D_u, U_u, 2)
    kv_bytes = S_u * H_u * D_u * 2
    sets = rot_sets(4 * kv_bytes)
    bufs = [(torch.empty((U_u, 2, 1, Lr2.S_max, H_u, D_u), dtype=bf16, device="cuda").normal_(),
             [torch.empty((1, S_u, H_u, D_u), dtype=bf16, device="cuda") for _ in range(2)])
            for _ in range(sets)]
    us = time_graph(torch, lambda i: sa.dit_ring_anything_trim(Lr2, bufs[i % sets][0], out=bufs[i % sets][1]),
                    launches)
    res["flux1008_ring_anything_trim_kv"] = hbm_entry(4 * kv_bytes, us, note="bytes: real rows read + written")
    del bufs

    # FP8 exchange at the FLUX U=2 shape: Q, V (and O) as block-scaled E4M3,
    # K bf16; bytes are the planes read / written plus the FP8 buffer
    L3 = sa.dit_a2a_layout_init(fw.B, fw.S, fw.H_total, fw.D, fw.U, 1, 3)
    L1 = sa.dit_a2a_layout_init(fw.B, fw.S, fw.H_total, fw.D, fw.U, 1, 1)
    st3 = sa.dit_a2a_fp8_bytes_per_peer(L3, sa.DIT_SEQ_TO_HEAD)
    st1 = sa.dit_a2a_fp8_bytes_per_peer(L1, sa.DIT_HEAD_TO_SEQ)
    shard_b = fw.B * L3.S_loc * fw.H_total * fw.D * 2
    head_b = fw.B * fw.S * L3.H_loc * fw.D * 2
    sets = rot_sets(head_b + shard_b + fw.U * st1)   # the smallest leg's own bytes
    bufs = []
    for _ in range(sets):
        shard = [torch.empty((fw.B, L3.S_loc, fw.H_total, fw.D), dtype=bf16, device="cuda").normal_()
                 for _ in range(3)]
        heads = [torch.empty((fw.B, fw.S, L3.H_loc, fw.D), dtype=bf16, device="cuda").normal_()
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
        us = time_graph(torch, lambda i, fn=fn: fn(bufs[i % sets]), launches)
        res[name] = hbm_entry(moved, us)
    res["flux_fp8_exchange_bytes"] = {"qkv_fp8": fw.U * st3, "qkv_bf16": fw.U * L3.elems_per_peer * 2,
                                      "o_fp8": fw.U * st1, "o_bf16": fw.U * L1.elems_per_peer * 2}
    del bufs

    # ring merge at the ring shard shape [1,4096,24,128], bf16 accumulator
    rw = workloads.WORKLOADS["ring"]
    rows = rw.B * rw.Sq * rw.H
    mb = 3 * rows * rw.D * 2 + 3 * rows * 4
    sets = rot_sets(mb)
    accs = [(torch.randn(rw.B, rw.Sq, rw.H, rw.D, device="cuda").to(bf16),
             torch.randn(rw.B, rw.H, rw.Sq, device="cuda"),
             torch.randn(rw.B, rw.Sq, rw.H, rw.D, device="cuda").to(bf16),
             torch.randn(rw.B, rw.H, rw.Sq, device="cuda")) for _ in range(sets)]
    us = time_graph(torch, lambda i: sa.dit_attn_merge(*accs[i % sets]), launches)
    res["ring_merge_bf16"] = hbm_entry(mb, us)
    del accs

    # copy references of the same sizes as the FLUX QKV pack (84.9 MB moved)
    # and the Wan 1-plane permute (193.5 MB moved): torch's device copy
    for label, half in (("84.9MB", 42_467_328), ("193.5MB", 96_768_000)):
        sets = rot_sets(2 * half)
        src = [torch.empty(half // 2, dtype=bf16, device="cuda") for _ in range(sets)]
        dst = [torch.empty_like(s) for s in src]
        us = time_graph(torch, lambda i: dst[i % sets].copy_(src[i % sets]), launches)
        res[f"device_copy_{label}"] = hbm_entry(2 * half, us)
        del src, dst
    return res


# ---------------------------------------------------------------------------
# the fp64 oracle on the host
# ---------------------------------------------------------------------------

def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(w, attn_flop, full=True):
    """The fp64 oracle, as it stands, on this host's cores.

    Full problems: the Tiny and FLUX steps (packs, unpacks, attention, CFG),
    Qwen U=4 / U=5 attention, the ring shard chunked (4 chunks + 3 merges)
    and unchunked.  Wan: 4096 seeded random query rows of each of its 5
    heads against all 75600 keys (rows are independent, so the sample is
    exact for its rows), timed and extrapolated to the full 75600 rows.
    Host GB/s for the FLUX permutes and the CFG combine."""
    import numpy as np
    import oracle
    from sequence_attention_amd import workloads as wl
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        blas = max([i["num_threads"] for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threadpool_limits, blas = None, 1
    affinity = len(os.sched_getaffinity(0))
    cores = max(1, min(affinity, blas))
    limiter = threadpool_limits(cores) if threadpool_limits else None
    try:
        res, flux_sec = _cpu_runs(w, np, oracle, wl, full)
    finally:
        if limiter is not None:
            limiter.restore_original_limits()
    value = attn_flop / flux_sec / 1e12 if flux_sec else None
    return {"value": round(value, 6) if value else None, "unit": "TFLOP/s", "cores": int(cores),
            "kind": "oracle", "cpu_model": cpu_model(), "affinity_cores": affinity, "blas_threads": blas,
            "sample": "one full FLUX step of rank 0 (QKV pack/unpack, attention, O pack/unpack, CFG) in "
                      "float64 numpy, value = its attention FLOP / step seconds"
                      + ("; also the Tiny step, Qwen U=4/U=5 and ring (chunked, unchunked) attention in full, "
                         "Wan sampled and extrapolated (details)" if full else ""),
            "details": res}


def _cpu_runs(w, np, oracle, wl, full):

    def f64(t):
        return t.float().numpy().astype(np.float64)

    def timed(fn):
        t0 = time.perf_counter()
        out = fn()
        return out, time.perf_counter() - t0

    res = {}

    def step(wk, name):
        L3 = oracle.a2a_layout(wk.B, wk.S, wk.H_total, wk.D, wk.U, 1, 3)
        L1 = oracle.a2a_layout(wk.B, wk.S, wk.H_total, wk.D, wk.U, 1, 1)
        shard = [f64(t) for t in wl.seq_sharded_planes(wk, 3, L3["S_loc"])]
        cfg_shape = CFG_SHAPE if name == "flux" else (2, 256, 256)
        cfg = wl.cfg_inputs(cfg_shape).numpy()
        st = {}
        send, st["pack_qkv"] = timed(lambda: oracle.pack_seq_to_head(shard, L3, 0))
        (q, k, v), st["unpack_qkv"] = timed(lambda: oracle.unpack_seq_to_head(send, L3, 0))
        (o, _), st["attention"] = timed(lambda: oracle.attention(q, k, v, wk.scale))
        send1, st["pack_o"] = timed(lambda: oracle.pack_head_to_seq([o], L1, 0))
        _, st["unpack_o"] = timed(lambda: oracle.unpack_head_to_seq(send1, L1, 0))
        _, st["cfg"] = timed(lambda: oracle.cfg_combine(cfg[0], cfg[1], 4.0))
        total = sum(st.values())
        b3 = 2 * (3 * wk.B * L3["S_loc"] * wk.H_total * wk.D + wk.U * L3["elems_per_peer"]) * 2
        b1 = 2 * (wk.B * wk.S * L1["H_loc"] * wk.D + wk.U * L1["elems_per_peer"]) * 2
        cfg_b = 3 * math.prod(cfg_shape[1:]) * 4
        res[f"{name}_step"] = {
            "seconds": round(total, 3), "attention_TFLOP/s": round(wk.attn_flop() / st["attention"] / 1e12, 6),
            "stage_seconds": {k2: round(v2, 4) for k2, v2 in st.items()},
            "host_GB/s": {"pack_qkv": round(b3 / 2 / st["pack_qkv"] / 1e9, 3),
                          "unpack_qkv": round(b3 / 2 / st["unpack_qkv"] / 1e9, 3),
                          "pack_o": round(b1 / 2 / st["pack_o"] / 1e9, 3),
                          "unpack_o": round(b1 / 2 / st["unpack_o"] / 1e9, 3),
                          "cfg": round(cfg_b / st["cfg"] / 1e9, 3)},
            "bytes_note": "GB/s on bf16-sized bytes (elements read + written x 2 B; CFG 12 B per element) "
                          "although the oracle holds float64"}
        return total

    flux_sec = step(w, "flux") if w.name == "flux" else None
    progress("cpu baseline: FLUX step done")
    if not full:
        return res, flux_sec
    step(wl.WORKLOADS["tiny"], "tiny")

    for name in ("qwen_u4", "qwen_u5"):
        wk = wl.WORKLOADS[name]
        q, k, v = (f64(t) for t in wl.attention_inputs(wk))
        _, sec = timed(lambda: oracle.attention(q, k, v, wk.scale))
        res[f"{name}_attention"] = {"seconds": round(sec, 3), "TFLOP/s": round(wk.attn_flop() / sec / 1e12, 6)}
        del q, k, v
        progress(f"cpu baseline: {name} attention done")

    rw = wl.WORKLOADS["ring"]
    q, k, v = (f64(t) for t in wl.attention_inputs(rw))
    chunk = rw.Skv // rw.R
    bounds = [c * chunk for c in range(rw.R + 1)]
    order = [(0 - t) % rw.R for t in range(rw.R)]
    _, sec_c = timed(lambda: oracle.ring_attention(q, k, v, rw.scale, bounds, order))
    progress("cpu baseline: ring chunked done")
    _, sec_u = timed(lambda: oracle.attention(q, k, v, rw.scale))
    progress("cpu baseline: ring unchunked done")
    res["ring_chunked"] = {"seconds": round(sec_c, 3), "TFLOP/s": round(rw.attn_flop() / sec_c / 1e12, 6),
                           "note": "4 chunks + 3 merges, hop order 0,3,2,1"}
    res["ring_unchunked"] = {"seconds": round(sec_u, 3), "TFLOP/s": round(rw.attn_flop() / sec_u / 1e12, 6)}
    del q, k, v

    ww = wl.WORKLOADS["wan"]
    q, k, v = (f64(t) for t in wl.attention_inputs(ww))
    rows = np.sort(np.random.default_rng(0).choice(ww.Sq, size=4096, replace=False))
    _, sec = timed(lambda: oracle.attention(q, k, v, ww.scale, rows=rows))
    full = sec * ww.Sq / len(rows)
    res["wan_attention_sampled"] = {
        "rows_per_head": len(rows), "heads": ww.H, "seconds_sample": round(sec, 3),
        "seconds_full_extrapolated": round(full, 1), "TFLOP/s": round(ww.attn_flop() / full / 1e12, 6),
        "note": "extrapolated: 4096 seeded random query rows per head against all 75600 keys, "
                "time x 75600 / 4096"}
    del q, k, v
    return res, flux_sec


# ---------------------------------------------------------------------------
# profile summaries (for the tables committed with the profiles)
# ---------------------------------------------------------------------------

def kernel_short_name(name):
    """Kernel name without namespaces and parameter list (cut at the first
    '(' outside template brackets); vector types shortened."""
    name = name.replace("void ", "").replace("dit::(anonymous namespace)::", "")
    name = name.replace("unsigned int __vector(4)", "u32x4").replace("unsigned int __vector(2)", "u32x2")
    depth = 0
    for i, ch in enumerate(name):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            return name[:i]
    return name


def trace_summary(db_path):
    """Per (kernel, grid) durations of a rocprofv3 kernel-trace database."""
    import sqlite3
    con = sqlite3.connect(db_path)
    rows = con.execute("select name, grid_x, grid_y, grid_z, start, end from kernels").fetchall()
    groups = {}
    for name, gx, gy, gz, s, e in rows:
        if name.startswith("void at::") or name.startswith("at::") or "rocclr" in name or "__amd" in name:
            continue
        short = kernel_short_name(name)
        grid = f"{gx}" if gy == 1 and gz == 1 else f"{gx}x{gy}x{gz}"
        groups.setdefault((short, grid), []).append((e - s) / 1e3)
    print("| Kernel | Grid (threads) | Calls | Average (us) | Median (us) | Min (us) | Max (us) |")
    print("|:--|--:|--:|--:|--:|--:|--:|")
    for (short, grid), d in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        print(f"| {short} | {grid} | {len(d)} | {sum(d) / len(d):.2f} | {statistics.median(d):.2f} | "
              f"{min(d):.2f} | {max(d):.2f} |")


def pmc_summary(csv_path):
    """Median per dispatch of each counter, per (kernel, grid), of a
    rocprofv3 --pmc CSV."""
    import csv
    groups = {}
    with open(csv_path, newline="") as f:
        for r in csv.DictReader(f):
            name = r.get("Kernel_Name") or r.get("Kernel-Name") or ""
            if name.startswith("void at::") or "rocclr" in name or "__amd" in name:
                if "copyBuffer" not in name:
                    continue
            short = kernel_short_name(name)
            grid = r.get("Grid_Size") or r.get("Grid_Size_X") or "?"
            groups.setdefault((short, grid, r["Counter_Name"]), []).append(float(r["Counter_Value"]))
    print("| Kernel | Grid (threads) | Counter | Dispatches | Median per dispatch |")
    print("|:--|--:|:--|--:|--:|")
    for (short, grid, ctr), v in sorted(groups.items()):
        print(f"| {short} | {grid} | {ctr} | {len(v)} | {statistics.median(v):.1f} |")


# ---------------------------------------------------------------------------

def progress(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.trace_summary:
        trace_summary(args.trace_summary)
        return
    if args.pmc_summary:
        pmc_summary(args.pmc_summary)
        return
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
    if args.only:
        only = set(args.only.split(","))
        out = {}
        if "kernels" in only:
            out["kernels"] = kernel_timings(w, torch, sa, workloads, Step(w, torch, sa, workloads, seed=0), 0,
                                            args.graph_launches)[0]
        if "side" in only:
            out["side"] = side_measurements(torch, sa, workloads, args.graph_launches)
        rest = only - {"kernels", "side"}
        if rest:
            out["configs"] = attention_configs(torch, sa, workloads, args.graph_launches, only=rest)
        print(json.dumps(out), flush=True)
        return
    one = Step(w, torch, sa, workloads, seed=0)
    n_sets = rot_sets(one.bytes())
    steps = [one] + [Step(w, torch, sa, workloads, seed=i) for i in range(1, n_sets)]
    rank = 0

    warm_clock(torch, lambda i: steps[i % n_sets].run(sa, rank), args.clock_warmup_s)
    for i in range(args.warmup):
        steps[i % n_sets].run(sa, rank)
    torch.cuda.synchronize()

    # timed region: K steps bracketed by two HIP events on the launch stream
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
    clock = {"fma": sa.dit_clock_probe(), "mfma": sa.dit_clock_probe(mfma=True, spin=5000),
             "mfma_sustained": sa.dit_clock_probe(mfma=True, spin=80000)}
    progress(f"timed steps done: {ms_per_step:.4f} ms/step")

    # the same K steps replayed from one captured graph
    steps_graph_us = time_graph(torch, lambda i: steps[i % n_sets].run(sa, rank), args.steps, replays=2)

    kernels, attn_us = kernel_timings(w, torch, sa, workloads, one, rank, args.graph_launches)
    progress("per-kernel graph timings done")
    attn_flop = w.attn_flop()
    value = attn_flop / (ms_per_step * 1e-3) / 1e12

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
                   "clock_warmup_s": args.clock_warmup_s, "graph_launches": args.graph_launches},
        "gpu_clock_ghz": {"after_timed_steps": {m: {k: round(v, 3) for k, v in c.items()}
                                                for m, c in clock.items()},
                          "method": "dit_clock_probe right after the region: s_memtime cycles / "
                                    "s_memrealtime (100 MHz) ticks per workgroup, 256 workgroups, "
                                    "median / min / max; fma = light load, mfma = bf16 MFMA load "
                                    "(~0.3 ms), mfma_sustained = the same MFMA load for ~5 ms, "
                                    "long enough for the power limit to set the clock"},
        "ms_per_step_graph": round(steps_graph_us / 1e3, 4),
        "roofline": attn_roofline(w.name + "_a2a", attn_flop, attn_us,
                                  kernel="attn_bf16_kernel<128, false, false, 2> (dit_attn_fwd_a2a, chunk of whole key blocks)"),
        "kernels": kernels,
    }
    result["roofline"].pop("flop", None)
    result["roofline"]["algorithmic_flop_per_launch"] = attn_flop
    if not args.no_side:
        result["side"] = side_measurements(torch, sa, workloads, args.graph_launches)
        progress("side measurements done")
    if not args.no_configs:
        result["configs"] = attention_configs(torch, sa, workloads, args.graph_launches)
        result["gpu_clock_ghz"]["after_configs"] = {
            k: round(v, 3) for k, v in sa.dit_clock_probe(mfma=True, spin=5000).items()}
        progress("attention configs done")
    if not args.no_cpu_baseline:
        progress("cpu baseline (fp64 oracle on the host) ...")
        result["cpu_baseline"] = cpu_baseline(w, attn_flop, full=args.cpu_baseline == "full")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
