"""Host-side checks of the benchmark script (no GPU needed)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    proc = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                          capture_output=True, text=True, timeout=120)
    assert proc.returncode == 2
    assert "one GPU" in proc.stderr


def test_weighted_and_probs_on_input_are_alternatives():
    proc = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--weighted", "--probs-on-input"],
                          capture_output=True, text=True, timeout=120)
    assert proc.returncode == 2
    assert "alternatives" in proc.stderr


def test_cpu_baseline_on_the_tiny_workload():
    sys.path.insert(0, ROOT)
    import bench
    import workload
    case = workload.draw_case(workload.by_name("tiny_e4_h64_f128"))
    rec, sample = bench.cpu_baseline(case, 0.2)
    assert sample["y"].shape == (sample["rows"].size, case.H)
    assert rec["kind"] == "oracle" and rec["unit"] == "TFLOP/s"
    assert rec["value"] > 0 and rec["cores"] >= 1 and rec["seconds"] > 0
    assert "routed rows" in rec["sample"]


def test_algorithmic_bytes_counts_only_experts_with_rows():
    sys.path.insert(0, ROOT)
    import bench
    fwd, dg = bench.algorithmic_bytes(M=10, H=8, F=16, n_live=3)
    assert fwd == 6 * 8 * 16 * 3 + 4 * 10 * 8 + 8 * 10 * 16
    assert dg == 6 * 8 * 16 * 3 + 4 * 10 * 8 + 12 * 10 * 16


def test_kernel_source_hash_ignores_comments_and_layout(tmp_path, monkeypatch):
    """The key of the stored traffic counters changes with the code of the
    kernel and launch sources, not with their comments or layout."""
    sys.path.insert(0, ROOT)
    import shutil

    import bench
    for rel in bench.KERNEL_SOURCES:
        dst = tmp_path / rel
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copy(os.path.join(ROOT, rel), dst)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    base = bench.kernel_source_hash()
    src = tmp_path / bench.KERNEL_SOURCES[0]
    text = src.read_text()
    src.write_text("// a comment\n/* and a\n   block comment */\n" + text.replace("\n", "\n\n", 3))
    assert bench.kernel_source_hash() == base
    assert "wait_vmcnt<28>" in text
    src.write_text(text.replace("wait_vmcnt<28>", "wait_vmcnt<27>", 1))
    assert bench.kernel_source_hash() != base
