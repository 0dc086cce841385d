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


def fake_full(b):
    """A full result set shaped like bench.py's, with long worst-case numbers."""
    x = 123456.789012
    ex = lambda w, t, algo, auto=False: {
        "world": w, "algorithm": algo, "link_mbps": 50000, "tokens": t, "N": 4096 * t,
        "bytes_per_call": (w + 1) * 4096 * t * 2, "graph_us": x, "graph_GBps": x, "graph_frac_link": x,
        "link_GBps_per_dir": x, "link_busiest_dir_frac": x, "eager_us": x, "eager_GBps": x,
        "eager_frac_link": x, "graph_calls": 500, "replays": 1, "gate_ms": x, "host_submit_ms": x,
        "gate_covered_submit": True, "bit_exact": True, "auto": auto}
    fold = lambda G, n: {"G": G, "N": n, "bytes_per_call": (G + 1) * n * 2,
                         **{f"{k}_{u}": x for k in ("warm", "graph", "cold_single", "cold", "cold_graph",
                                                     "cold_workspace", "cold_workspace_graph")
                            for u in ("us", "GBps", "frac_hbm")},
                         "bit_exact": True}
    algos = ("low-latency", "one-shot", "two-shot")
    cfgs = {
        "host_link_probe": {s: {k: {"us": x, "GBps": x} for k in ("h2d", "d2h", "bidir")}
                            for s in ("20KiB", "256KiB", "64MiB")},
        "exchange_2rank_host_slots": [ex(2, t, a, a == "one-shot") for t in (1, 4, 8, 16, 32) for a in algos],
        "exchange_2rank_prefill": [{"N": n, "MiB_per_rank": n * 2 / 2**20, "algorithm": a, "paced": p,
                                    "graph_us": x, "graph_GBps": x, "graph_frac_link": x,
                                    "link_GBps_per_dir": x, "bit_exact": True}
                                   for n in (1 << 19, 1 << 23) for a, p in (("one-shot", True),
                                                                            ("one-shot", False),
                                                                            ("two-shot", True))],
        "exchange_world_host_slots": [ex(w, t, a) for w in (4, 8) for t in (1, 8, 32) for a in algos],
        "exchange_group_launch_host_slots": [dict(ex(w, t, a), launch="group") for w in (2, 4, 8)
                                             for t in (1, 8, 32) for a in algos],
        "exchange_graph_1000_calls_N10240": {"N": 10240, "calls": 1000, "algorithm": "low-latency",
                                             "us_per_call": x, "GBps": x, "frac_link": x,
                                             "host_submit_ms": x, "gate_covered_submit": True,
                                             "bit_exact": True},
        "exchange_graph_1000_calls_N10240_one_shot": {"N": 10240, "calls": 1000, "algorithm": "one-shot",
                                                      "us_per_call": x, "GBps": x, "frac_link": x,
                                                      "host_submit_ms": x, "gate_covered_submit": True,
                                                      "bit_exact": True},
        "fold_graph_node_floor": {"G": 1, "N": 8, "graph_calls": 100, "graph_us": x},
        "fold_G2_N4096_specials": fold(2, 4096),
        "fold_G8_N393216": fold(8, 393216),
        "fold_G8_N16777216": fold(8, 16777216),
        "bf16": {"fold_G8_N16777216_workspace": {"cold_us": x, "cold_GBps": x, "cold_frac_hbm": x,
                                                 "bit_exact": True},
                 "exchange_2rank_256KiB_graph": {"us": x, "GBps": x, "frac_link": x, "bit_exact": True}},
    }
    head = ex(2, 32, "one-shot")
    cpu = {"all": {"us_per_call": x, "GBps": x, "cores": 256, "calls": 123456, "wall_s": 1.5},
           "one": {"us_per_call": x, "GBps": x, "cores": 1, "calls": 1234},
           "gpu_matches_oracle": True}
    return {"args": {"steps": 20, "warmup": 5, "tokens": 32, "quick": False, "only": ""},
            "elapsed_s": 0.34, "link_peak": 55.48, "headline": head, "configs": cfgs, "cpu": cpu,
            "device": {"name": "AMD Instinct MI355X", "cus": 256, "hip": "7.0", "torch": "2.10"},
            "host": {"cpu": "AMD EPYC 9575F 64-Core Processor with a long model name", "cores": 16},
            "traffic": {"exchange": 1146314.0, "fold": 302024701.0}}


def test_last_line_is_compact_and_carries_the_contract():
    import json
    b = load_bench()
    full = fake_full(b)
    line = json.dumps(b.make_line(full, os.path.join(ROOT, "gpurun_out", "bench_full.json")),
                      separators=(",", ":"))
    assert len(line.encode()) <= b.LINE_MAX_BYTES, len(line.encode())
    d = json.loads(line)
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
              "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "roofline_hbm_fold",
              "cpu_baseline", "table_us_frac", "bit_exact"):
        assert k in d, k
    assert d["metric"] == b.METRIC
    assert d["n_gpus"] == 1 and d["steps"] == 20 and d["warmup"] == 5
    assert "workload" in d["config"]
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic", "busiest_dir_frac"):
        assert k in d["roofline"], k
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in d["roofline_hbm_fold"], k
    for k in ("value", "unit", "cores", "kind", "sample"):
        assert k in d["cpu_baseline"], k
    assert d["cpu_baseline"]["kind"] == "oracle"
    # one step is one replay of the fixed-size graph: the per-step time is
    # the elapsed time over the timed steps, the value per call
    calls = 20 * b.CALLS_PER_STEP
    assert abs(d["ms_per_step"] - 0.34 / 20 * 1e3) < 1e-3
    assert abs(d["value"] - 3 * 131072 * 2 / (0.34 / calls) / 1e9) < 1e-2
    for name in ("C1_fold_G2_N4096_graph", "C2_32tok_graph", "C3_fold_G8_N393216_graph",
                 "C4_fold_cold_workspace", "C5_graph1000"):
        assert name in d["table_us_frac"], name


def test_a_failed_comparison_anywhere_clears_bit_exact():
    b = load_bench()
    full = fake_full(b)
    full["configs"]["exchange_world_host_slots"][3]["bit_exact"] = False
    assert b.make_line(full)["bit_exact"] is False


def test_steps_counts_graph_replays():
    b = load_bench()
    import inspect
    src = inspect.getsource(b.main)
    assert "replays=args.steps" in src and "warm_replays=args.warmup" in src
    assert b.CALLS_PER_STEP == 1000
