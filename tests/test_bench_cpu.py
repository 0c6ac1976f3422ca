"""Host-side checks of bench.py (no GPU): the one-GPU contract and the committed HBM-byte
summary it reports as the dominant kernel's traffic."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_summary_matches_the_algorithmic_bytes_and_the_sources():
    import bench
    from nvfp4_block_scaled_gather_amd import build
    fields = {}
    for line in open(bench.TRAFFIC_FILE).read().splitlines():
        if ":" in line and not line.startswith(("#", " ", "|")):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    # 288 experts x 9,437,184 B of w13 weights + 570 NVFP4 activation rows of H = 4096
    # (2048 + 256 bytes) + 570 fp32 output rows of N = 4096
    alg = 288 * 9437184 + 570 * (4096 // 2 + 4096 // 16) + 570 * 4096 * 4
    assert int(fields["algorithmic_bytes_per_launch"]) == alg
    traffic = int(fields["traffic_bytes_per_launch"])
    assert alg <= traffic < 1.05 * alg          # every weight byte read from HBM once
    # the figure is reported only while the summary was taken at the current GEMM sources;
    # after a change to them it is withheld (null) until the counters are taken again
    fresh = fields["kernel_sources_sha256"] == build.kernel_source_hash()
    assert bench.measured_traffic("ragged570") == (traffic if fresh else None)
    assert bench.measured_traffic("ragged2303") is None  # summary is for ragged570 only


def test_kernel_hash_ignores_comments_but_not_code():
    from nvfp4_block_scaled_gather_amd import build
    a = "int f(int x) { return x + 1; }  // one\n/* block\n comment */"
    b = "int f(int x) {\n  return x + 1;  // another comment\n}"
    c = "int f(int x) { return x + 2; }"
    assert build._code_only(a) == build._code_only(b)
    assert build._code_only(a) != build._code_only(c)
