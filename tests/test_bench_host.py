"""Host logic of the measurement tools, on the CPU: the algorithmic FLOP and
byte counts bench.py divides by, its refusal of more than one GPU, the
source-hash check that retires stale profile records, and the arithmetic of
the rocprofv3 summaries (copy calibration of the traffic counters, per-dispatch
sums, duration records).  No GPU is touched."""

from __future__ import annotations

import csv
import hashlib
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from spherical_block_sparse_amd import CONFIGS  # noqa: E402
from spherical_block_sparse_amd import rocprof_summary as rs  # noqa: E402


def _window_brute(n_tok: int, window: int) -> int:
    """Keys of every clipped centred window [t - floor(W/2), t + ceil(W/2)) ∩ [0, N), one query at a time."""
    total = 0
    for t in range(n_tok):
        total += sum(1 for u in range(n_tok) if t - window // 2 <= u < t + (window + 1) // 2)
    return total


@pytest.mark.parametrize("n_tok,window", [(48, 1), (48, 7), (48, 16), (192, 100), (192, 191), (192, 500)])
def test_window_keys_total_brute_force(n_tok, window):
    assert bench.window_keys_total(n_tok, window) == _window_brute(n_tok, window)


def test_fine_flops_counts_both_branches():
    cfg = CONFIGS["ns32"].with_(nside=8, block=16, topn=4, window=100, batch=1, heads=2)
    per_query_sel = 4 * cfg.head_dim * cfg.topn * cfg.block
    win = _window_brute(cfg.n_tokens, cfg.window)
    expect = cfg.slices * (cfg.n_tokens * per_query_sel + 4 * cfg.head_dim * win)
    assert bench.fine_flops(cfg) == pytest.approx(expect, rel=0, abs=0)
    assert bench.backward_flops(cfg) == 2.5 * bench.fine_flops(cfg)


def test_fine_flops_ns128_figure():
    # 24 x 8 slices of 196 608 tokens, d 64, 16 blocks of 64, window 512
    cfg = CONFIGS["ns128"]
    n = cfg.n_tokens
    t = np.arange(n)
    win = int((np.minimum(t + 256, n) - np.maximum(t - 256, 0)).sum())
    assert bench.fine_flops(cfg) == 4 * 64 * (n * 16 * 64 + win) * 192
    assert bench.fine_flops(cfg) == 14840185749504.0


def test_compress_and_pool_counts():
    cfg = CONFIGS["ns128"]
    m, d, S = cfg.n_blocks, cfg.head_dim, cfg.slices
    assert bench.compress_flops(cfg) == 4.0 * m * m * d * S
    # top-n 16: four bf16 products of 2 m^2 d (three logit pieces and ā·v̄) at 2.5 PFLOP/s
    assert bench.compress_bound_ms(cfg) == pytest.approx(4 * 2.0 * m * m * d * S / 2.5e15 * 1e3)
    e_in, e_out = S * cfg.n_tokens * d, S * m * d
    assert bench.pool_bytes(cfg) == 3 * e_in * 2 + e_out * (8 + 8 + 4 + 4) + S * m * 8


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, env={**os.environ, "HIP_VISIBLE_DEVICES": ""})
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_profile_records_retire_on_source_change(tmp_path, monkeypatch):
    src = tmp_path / "kernel.hip"
    src.write_text("// a kernel\n")
    good = hashlib.sha256(src.read_bytes()).hexdigest()
    traffic = {"k_ok": {"source": str(src), "source_sha256": good, "hbm_bytes": 123.0},
               "k_stale": {"source": str(src), "source_sha256": "0" * 64, "hbm_bytes": 456.0}}
    durations = {"k_ok": {"source": str(src), "source_sha256": good, "avg_ms": 1.5},
                 "k_stale": {"source": str(src), "source_sha256": "0" * 64, "avg_ms": 2.5}}
    (tmp_path / "t.json").write_text(json.dumps(traffic))
    (tmp_path / "d.json").write_text(json.dumps(durations))
    monkeypatch.setattr(bench, "TRAFFIC_JSON", str(tmp_path / "t.json"))
    monkeypatch.setattr(bench, "DURATION_JSON", str(tmp_path / "d.json"))
    # os.path.join(ROOT, absolute) is the absolute path, so the records point at the temporary source
    assert bench.measured_traffic("k_ok") == 123.0
    assert bench.measured_traffic("k_stale") is None
    assert bench.measured_traffic("missing") is None
    assert bench.profiled_ms("k_ok") == 1.5
    assert bench.profiled_ms("k_stale") is None
    src.write_text("// the kernel, edited\n")
    assert bench.measured_traffic("k_ok") is None
    assert bench.profiled_ms("k_ok") is None


def test_committed_profile_records_name_existing_sources():
    for name in ("traffic.json", "kernel_durations.json"):
        recs = json.load(open(os.path.join(ROOT, "profiles", name)))
        assert recs, name
        for key, rec in recs.items():
            assert os.path.isfile(os.path.join(ROOT, rec["source"])), (name, key)
            assert len(rec["source_sha256"]) == 64


def _counter_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"], r)))


def test_traffic_copy_calibration(tmp_path):
    # the copy of 8 MiB reads 8192 KiB and writes 8192 KiB; its counters read 7372.8 and 9011.2 KiB
    # (per-XCD rows of one dispatch are summed), so reads scale by 1/0.9 and writes by 1/1.1
    _counter_csv(tmp_path / "cf.csv", [(1, "copyBuffer", "FETCH_SIZE", 3686.4), (1, "copyBuffer", "FETCH_SIZE", 3686.4)])
    _counter_csv(tmp_path / "cw.csv", [(1, "copyBuffer", "WRITE_SIZE", 9011.2)])
    # two dispatches of the kernel: 900 and 1100 KiB fetched, 220 KiB written each
    _counter_csv(tmp_path / "f.csv", [(5, "fine_kernel<64>", "FETCH_SIZE", 400.0), (5, "fine_kernel<64>", "FETCH_SIZE", 500.0),
                                      (6, "fine_kernel<64>", "FETCH_SIZE", 1100.0), (7, "other", "FETCH_SIZE", 1e9)])
    _counter_csv(tmp_path / "w.csv", [(5, "fine_kernel<64>", "WRITE_SIZE", 220.0), (6, "fine_kernel<64>", "WRITE_SIZE", 220.0)])
    src = tmp_path / "k.hip"
    src.write_text("x")

    class A:
        copy_mib = 8
        copy_fetch = str(tmp_path / "cf.csv")
        copy_write = str(tmp_path / "cw.csv")
        fetch = str(tmp_path / "f.csv")
        write = str(tmp_path / "w.csv")
        kernel = "fine_kernel"
        source = str(src)

    rec = rs.traffic(A)
    assert rec["read_factor"] == pytest.approx(1 / 0.9)
    assert rec["write_factor"] == pytest.approx(1 / 1.1)
    assert rec["fetch_kib_per_dispatch"] == pytest.approx(1000.0)
    assert rec["hbm_read_bytes"] == pytest.approx(1000.0 / 0.9 * 1024)
    assert rec["hbm_write_bytes"] == pytest.approx(220.0 / 1.1 * 1024)
    assert rec["hbm_bytes"] == pytest.approx(rec["hbm_read_bytes"] + rec["hbm_write_bytes"])
    assert rec["source_sha256"] == hashlib.sha256(b"x").hexdigest()


def test_duration_record_and_stats(tmp_path):
    path = tmp_path / "stats.csv"
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs"])
        w.writerow(["void mosaic::(anonymous namespace)::fine_kernel<64, 2, 0>(mosaic::FineArgs)", 19, 4e8, 21059228.1, 60.0, 20406000, 22239000])
        w.writerow(["void mosaic::(anonymous namespace)::fine_kernel<64, 4, 0>(mosaic::FineArgs)", 11, 2.5e8, 22512000, 40.0, 22136000, 23009000])
    src = tmp_path / "k.hip"
    src.write_text("y")

    class A:
        csv = str(path)
        kernel = "fine_kernel<64, 2, 0>"
        source = str(src)

    rec = rs.duration(A)
    assert rec["calls"] == 19 and rec["avg_ms"] == pytest.approx(21.0592281)
    A.kernel = "fine_kernel"
    with pytest.raises(SystemExit):   # two kernels match
        rs.duration(A)
    text = rs.stats(str(path))
    assert "mosaic::fine_kernel<64, 2, 0>" in text and "21.059" in text
    assert "(anonymous namespace)" not in text


def test_counters_sum_rows_of_a_dispatch(tmp_path):
    _counter_csv(tmp_path / "c.csv", [(1, "fine_kernel<64>", "SQ_INSTS_MFMA", 10.0), (1, "fine_kernel<64>", "SQ_INSTS_MFMA", 5.0),
                                      (2, "fine_kernel<64>", "SQ_INSTS_MFMA", 25.0), (3, "pool_kernel", "SQ_INSTS_MFMA", 99.0)])
    text = rs.counters(str(tmp_path / "c.csv"), "fine_kernel")
    lines = text.splitlines()
    assert len(lines) == 4   # header, two dispatches, mean
    assert lines[1].split()[-1] == "15" and lines[2].split()[-1] == "25"
    assert lines[3].split()[-1] == "20"


def test_random_shape_draw_is_valid_and_varied():
    """The seeded shapes of the random-shape GPU test are valid forward
    arguments and reach every kernel path: blocks below 16 (one-wave fine
    kernel), top-n above 16 and above 64 (list, buffered and radix
    selection), both head dims, windows of one token and past the sphere."""
    from test_random_shapes_gpu import CASES
    assert len({c.name for c in CASES}) == len(CASES)
    for c in CASES:
        n_tok = 12 * c.nside ** 2
        assert c.block & (c.block - 1) == 0 and (c.block.bit_length() - 1) % 2 == 0
        assert 1 <= c.block <= c.nside ** 2
        assert 1 <= c.topn <= n_tok // c.block
        assert c.window >= 1 and c.head_dim in (32, 64)
    assert any(c.block < 16 for c in CASES) and any(c.block >= 16 for c in CASES)
    assert any(c.topn > 16 for c in CASES) and any(c.topn <= 16 for c in CASES)
    assert any(c.topn > 64 for c in CASES)
    assert {c.head_dim for c in CASES} == {32, 64}
    assert any(c.window == 1 for c in CASES) and any(c.window > 2 * 12 * c.nside ** 2 for c in CASES)


def test_random_backward_shape_draw_is_valid_and_varied():
    """The seeded shapes of the random-shape backward GPU test lie inside the
    backward's domain (block >= 64, top-n <= 64, m a multiple of 64) and
    reach both head dims, both block sizes, signed and unsigned gates,
    windows of one token and past the sphere, and the largest top-n."""
    from test_random_shapes_backward_gpu import CASES
    assert len({c.name for c, _ in CASES}) == len(CASES)
    for c, _ in CASES:
        m = 12 * c.nside ** 2 // c.block
        assert c.block >= 64 and c.block <= c.nside ** 2 and m % 64 == 0
        assert 1 <= c.topn <= min(m, 64) and c.window >= 1 and c.head_dim in (32, 64)
    assert {c.head_dim for c, _ in CASES} == {32, 64} and {c.block for c, _ in CASES} == {64, 256}
    assert {sg for _, sg in CASES} == {True, False}
    assert any(c.window == 1 for c, _ in CASES)
    assert any(c.window > 2 * 12 * c.nside ** 2 for c, _ in CASES) and any(c.topn == 64 for c, _ in CASES)
