"""Host logic of bench.py that needs no GPU: the refusal of more than one GPU,
the keying of the counter-measured attention traffic to the kernel code (a
comment edit keeps it, a code edit drops it to null), and the summaries the
profile tables are made from (kernel names shortened, medians of rocprofv3
counter rows per kernel and grid)."""

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


def test_kernel_short_name_cuts_the_parameter_list_outside_templates():
    full = ("void dit::(anonymous namespace)::attn_bf16_kernel<128, false, false, 2>"
            "(dit::(anonymous namespace)::Params)")
    assert bench.kernel_short_name(full) == "attn_bf16_kernel<128, false, false, 2>"
    vec = "void dit::(anonymous namespace)::permute_kernel<0, unsigned int __vector(4)>(dit::PermuteGeom)"
    assert bench.kernel_short_name(vec) == "permute_kernel<0, u32x4>"
    assert bench.kernel_short_name("plain") == "plain"


def test_pmc_summary_takes_the_median_per_kernel_grid_and_counter(tmp_path, capsys):
    k = "void dit::(anonymous namespace)::merge_kernel<false, 128>(void*, float*, void const*, float const*, int, int, int)"
    rows = [("Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value")]
    rows += [(k, "786432", "FETCH_SIZE", v) for v in ("10", "30", "20")]
    rows += [(k, "786432", "WRITE_SIZE", "5")]
    rows += [("void at::native::some_torch_kernel(int)", "64", "FETCH_SIZE", "999")]     # torch's: dropped
    rows += [("__amd_rocclr_copyBuffer", "131072", "FETCH_SIZE", "7")]                    # the device copy: kept
    csv_path = tmp_path / "c.csv"
    csv_path.write_text("\n".join(",".join(f'"{x}"' for x in r) for r in rows) + "\n")
    bench.pmc_summary(str(csv_path))
    out = capsys.readouterr().out
    assert "| merge_kernel<false, 128> | 786432 | FETCH_SIZE | 3 | 20.0 |" in out
    assert "| merge_kernel<false, 128> | 786432 | WRITE_SIZE | 1 | 5.0 |" in out
    assert "__amd_rocclr_copyBuffer" in out and "some_torch_kernel" not in out
