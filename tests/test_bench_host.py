"""Host-side checks of bench.py that need no GPU: it refuses more than one GPU before it
touches any device, it rejects an unknown prefix-cache type, and it reads the shader
clock from the sysfs level listing."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args, env=None):
    e = dict(os.environ)
    e.update(env or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120, env=e, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""   # no JSON line


def test_world_size_above_one_is_refused():
    r = _run(env={"WORLD_SIZE": "8", "RANK": "0"})
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_unknown_cache_type_is_rejected():
    r = _run("--kv", "int4")
    assert r.returncode != 0
    assert "invalid choice" in r.stderr


def test_clock_listing_parser():
    sys.path.insert(0, ROOT)
    import bench
    # listings as the sysfs file shows them under load and at idle
    assert bench.current_sclk_mhz("0: 500Mhz\n1: 2152Mhz *\n2: 2400Mhz\n") == 2152
    assert bench.current_sclk_mhz("S: 96Mhz *\n0: 500Mhz\n1: 2400Mhz\n") == 96
    assert bench.current_sclk_mhz("0: 500Mhz\n1: 2400Mhz\n") is None


def test_compulsory_bytes_and_labels():
    """Algorithmic bytes of one denoising launch: bf16 Q, K, V read and O written for the
    image rows, plus the prefix cache read once at its element size."""
    sys.path.insert(0, ROOT)
    import pytest
    qi = pytest.importorskip("block_causal_attention_qi_amd.qi")
    import bench
    from block_causal_attention_qi_amd import synth
    w = synth.WORKLOADS["t2i1024"]
    p = qi.Plan(w.requests, w.n_heads, w.head_dim, w.kv_dtype)
    hd = 24 * 128
    assert bench.compulsory_bytes(p, w) == 4 * 4096 * hd * 2 + 2 * 256 * hd * 2 == 103809024
    w8 = synth.WORKLOADS["wave8"]
    p8 = qi.Plan(w8.requests, w8.n_heads, w8.head_dim, w8.kv_dtype)
    pre = sum(w8.prefix_lens)
    assert bench.compulsory_bytes(p8, w8) == 4 * 8 * 4096 * hd * 2 + 2 * pre * hd + 8 * 24 * 8
    assert round(bench.compulsory_bytes(p8, w8) / 1e6, 1) == 1394.7
    assert bench.kernel_label(128, "fp8") == "attn_pp_kernel<128, fp8 cache>"


def test_host_info_names_cores_and_threads():
    sys.path.insert(0, ROOT)
    import bench
    info = bench.host_info()
    assert info["os_cpu_count"] == os.cpu_count()
    assert set(info["env"]) == {"OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"}
    if "blas" in info:
        assert info["blas"]["threads"] >= 1
