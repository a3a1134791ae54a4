"""bench.py's command-line contract that holds without a GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
    assert r.stdout.strip() == ""  # no JSON line


def test_counter_summaries_match_the_decode_kernel_sources():
    """The committed counter summaries carry the sha256 of the sources their kernels were
    built from; bench.py reports traffic only while they match, so a stale summary would
    silently drop it from the bench line."""
    sys.path.insert(0, ROOT)
    import bench
    for srcs, name in ((bench.DECODE_FFN_SOURCES, "ffn_dot_decode_e256_k6_d4096_f2048_T8_counters.txt"),
                       (bench.MXFP4_FFN_SOURCES, "ffn_mx_decode_e256_k6_d4096_f2048_T8_counters.txt")):
        assert bench._counter_traffic(srcs, name) is not None, name


def test_prefill_traffic_summary_matches_the_gemm_sources():
    """The same for the prefill grouped GEMMs (bf16 and MXFP4), per Zipf alpha."""
    sys.path.insert(0, ROOT)
    import bench
    import gen
    for dtype in (None, gen.MXFP4):
        for alpha in (0.2, 1.0):
            t = bench._prefill_traffic(dtype, alpha)
            assert t is not None and t > 1e9, (dtype, alpha)
