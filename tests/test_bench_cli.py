"""Host-side checks of bench.py's contract (no GPU): the one-GPU guard, the
fwd+bwd work count, and the GEMM source hash that keys the stored HBM counters."""
import importlib.util
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_flops_count():
    b = load_bench()
    # c2: 4 M h o for the two base products, 6 M r (h + o) for the adapter products
    assert b.flops_fwd_bwd(2048, 4096, 4096, 16) == 4.0 * 2048 * 4096 * 4096 + 6.0 * 2048 * 16 * 8192
    assert b.flops_fwd_bwd(0, 4096, 4096, 16) == 0.0


def test_gemm_hash_ignores_comments_only(tmp_path, monkeypatch):
    b = load_bench()
    src = tmp_path / "k.hip"
    src.write_text("int a = 1;  // one\n\nint b = 2;\n")
    monkeypatch.setattr(b, "ROOT", str(tmp_path))
    monkeypatch.setattr(b, "GEMM_SOURCES", ["k.hip"])
    h0 = b.kernel_source_hash()
    src.write_text("// a new comment\nint a = 1;  // changed comment\nint b = 2;   \n\n")
    assert b.kernel_source_hash() == h0
    src.write_text("int a = 1;\nint b = 3;\n")
    assert b.kernel_source_hash() != h0


def test_stored_counters_name_the_current_kernel_hash_format():
    b = load_bench()
    with open(b.TRAFFIC_FILE) as f:
        tr = json.load(f)
    assert len(tr["kernel_source_hash"]) == 16
    for k in ("nf4_gemm_fwd", "nf4_gemm_dx"):
        assert tr["kernels"][k]["bytes_per_launch"] > 0


def test_cpu_passes_rates():
    import numpy as np
    b = load_bench()
    # algorithmic bytes per weight: fp32 read, 4-bit code, 8-bit scale per 64, fp32 step per 16384
    assert abs(b.QUANT_DQ_BYTES_PER_WEIGHT - 4.5159) < 1e-4 and b.ERROR_BYTES_PER_WEIGHT == 4.0
    W = (np.random.default_rng(0).standard_normal((128, 4096), dtype=np.float32) * np.float32(0.02))
    r = b.cpu_passes(W, threads=2, reps=1)
    assert r["quantize_dq_GBps"] > 0 and r["layer_error_GBps"] > 0 and r["threads"] == 2
    assert "524288 weights" in r["sample"] and "2 chunks of 64 rows" in r["sample"]
