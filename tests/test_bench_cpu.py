"""Host logic of bench.py that needs no GPU: the refusal of more than one GPU
and the keying of the counter-measured attention traffic to the kernel code
(a comment edit keeps it, a code edit drops it to null)."""

import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps", "1"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_traffic_hash_ignores_comments_but_not_code(tmp_path):
    with open(bench.ATTN_SRC, encoding="utf-8") as f:
        src = f.read()
    base = bench.attn_code_sha256()
    commented = tmp_path / "a.hip"
    commented.write_text("// a new header line\n\n" + src.replace("\n", "  // trailing note\n", 3) + "\n\n")
    assert bench.attn_code_sha256(str(commented)) == base
    changed = tmp_path / "b.hip"
    i = src.index("kThreads")
    changed.write_text(src[:i] + "kThread" + src[i + len("kThreads"):])
    assert bench.attn_code_sha256(str(changed)) != base


def test_traffic_reported_only_for_known_shapes():
    t = bench.attn_traffic("flux_a2a")
    if bench.attn_code_sha256() == bench.ATTN_TRAFFIC["src_sha256"]:
        rd, wr = bench.ATTN_TRAFFIC["per_shape"]["flux_a2a"]
        assert t == rd + wr
    else:
        assert t is None
    assert bench.attn_traffic("no_such_shape") is None
