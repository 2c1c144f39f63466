"""Host-side checks of bench.py: the one-GPU refusal and the algorithmic
counts its figures divide by (no GPU needed)."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr and p.stdout == ""


def test_layer_flops_of_the_workloads():
    # attn7b: M = K = N = 4096, r = 64
    assert bench.layer_flops(4096, 4096, 4096, 64) == (141_733_920_768, 146_028_888_064)
    # forward 2MKN + 2MKr + 2MrN and backward 2MNK + 4MNr + 4MKr, term by term on a small case
    M, K, N, r = 3, 5, 7, 2
    fwd, bwd = bench.layer_flops(M, K, N, r)
    assert fwd == 2 * (M * K * N) + 2 * (M * K * r) + 2 * (M * r * N)
    assert bwd == 2 * (M * N * K) + 4 * (M * N * r) + 4 * (M * K * r)
    # the dominant kernels: base product plus the rank-r extension only
    assert bench.kernel_flops("fwd_gemm", 4096, 4096, 4096, 64) == 139_586_437_120
    assert bench.kernel_flops("bwd_dx", M, K, N, r) == 2 * M * N * K + 2 * M * r * K


def test_committed_traffic_figure_is_used_only_for_the_profiled_source():
    # the figure is read only when the summary's source hash matches the kernel source
    got = bench.read_traffic("fwd_gemm")
    text = open(os.path.join(ROOT, "profiles", "fwd_gemm_attn7b_4096_pmc.md"), encoding="utf-8").read()
    same = f"source_sha256_16: {bench.src_hash('gemm_big.hip')}" in text
    assert (got is not None) == same
    if got is not None:
        assert 100e6 < got < 1e9
