"""CPU checks of bench.py's contract that need no GPU: more than one GPU is
refused with a message (one GPU is measured), the algorithmic byte count of a
launch follows its definition, and the rocprofv3-database summary restricts
to the selected dispatches."""
import os
import sqlite3
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_launch_bytes_definition():
    sys.path.insert(0, ROOT)
    import bench
    # weight K*N, column scales 4N, fp32 output 4MN per item; fp32 activations 4MK once
    assert bench.launch_bytes(16, 1024, [2048]) == 2301952
    assert bench.launch_bytes(1, 3072, [1024]) == 3072 * 1024 + 4 * 1024 + 4 * 3072 + 4 * 1024
    qkv = bench.launch_bytes(16, 1024, [2048, 1024, 1024])
    assert qkv == 1024 * 4096 + 4 * 4096 + 4 * 16 * 4096 + 4 * 16 * 1024
    # every launch of the step quantises inside the product kernel
    for M in (1, 16, 32):
        for K in (1024, 2048, 3072):
            assert bench.fused_quant(M, K)


def test_summarize_restricts_to_the_last_dispatches(tmp_path):
    db = tmp_path / "t.db"
    c = sqlite3.connect(db)
    c.execute("create table kernels (dispatch_id int, name text, start int, duration int)")
    c.execute("create table counters_collection (dispatch_id int, counter_name text, value real)")
    rows = [(i, "void qmm::k_int8_decode_q<1>(x)" if i % 2 else "other", i * 100, 1000 * (i + 1)) for i in range(10)]
    c.executemany("insert into kernels values (?,?,?,?)", rows)
    c.executemany("insert into counters_collection values (?,?,?)", [(i, "FETCH_SIZE", 10.0 * i) for i in range(10)])
    c.commit()
    c.close()
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--summarize", str(db), "--kernel",
                        "k_int8_decode_q", "--last", "2"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    # the last two decode dispatches are ids 7 and 9: 8 and 10 us
    assert "2 selected" in r.stdout
    assert "| 2 | 9.000 | 9.000 |" in r.stdout
    assert "FETCH_SIZE = 80.0 (2 dispatches)" in r.stdout


def test_summarize_cycle_splits_repeating_runs(tmp_path):
    db = tmp_path / "c.db"
    c = sqlite3.connect(db)
    c.execute("create table kernels (dispatch_id int, name text, start int, duration int)")
    # two steps of (3 launches of label a at 1 us, 2 of label b at 5 us)
    durs = [1000, 1000, 1000, 5000, 5000] * 2
    c.executemany("insert into kernels values (?,?,?,?)",
                  [(i, "void qmm::k_int8_decode_q<1>(x)", i * 100, d) for i, d in enumerate(durs)])
    c.commit()
    c.close()
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--summarize", str(db), "--kernel",
                        "k_int8_decode_q", "--cycle", "a:3,b:2"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    out = r.stdout
    assert "a (6 dispatches):" in out and "b (4 dispatches):" in out
    a_part = out.split("a (6 dispatches):")[1].split("b (4 dispatches):")[0]
    assert "| (all selected) | 6 | 1.000 |" in a_part
    assert "| (all selected) | 4 | 5.000 |" in out.split("b (4 dispatches):")[1]
