"""bench.py's host-side contract, on the CPU: one GPU only, and traffic
figures taken from the committed counter summary only when they were measured
on the kernel sources as they stand.

Nothing here touches a device.
"""
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def load_bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", BENCH)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True,
                       timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert r.stdout == ""
    assert "one GPU" in r.stderr


def test_source_digest_ignores_comments_and_layout():
    b = load_bench()
    code = "int f(int x) {\n    return x + 1;  // add one\n}\n"
    same = "/* header */\nint f(int x)\n{ return x + 1; }\n"
    other = "int f(int x) {\n    return x + 2;\n}\n"
    assert b.code_text(code) == b.code_text(same)
    assert b.code_text(code) != b.code_text(other)


def test_traffic_is_read_only_for_the_current_sources(tmp_path, monkeypatch):
    b = load_bench()
    digest = b.source_digest()
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "counters.txt").write_text(
        f"traffic fold_vec<8,4,F16> 302000000 sources={digest}\n"
        "traffic exchange_k<2,true,F16> 1145930 sources=0000000000000000\n")
    # the digest is of the package's sources; only the summary's location moves
    csrc = os.path.join(ROOT, "message_fp16_all_amd")
    os.symlink(csrc, tmp_path / "message_fp16_all_amd")
    monkeypatch.setattr(b, "ROOT", str(tmp_path))
    assert b.measured_traffic("fold_vec<8,4,F16>") == 302000000.0
    assert b.measured_traffic("exchange_k<2,true,F16>") is None   # taken on other sources
    assert b.measured_traffic("fold_vec<2,1,F16>") is None        # never measured
