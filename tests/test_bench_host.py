"""bench.py's host-side contract, without a GPU: one GPU only, the
grouped-query option's check, and the rocprofv3 summary reader on a database
written here."""
import os
import sqlite3
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in (r.stdout + r.stderr)


def test_kv_heads_must_divide_the_query_heads():
    # checked before any input is generated or a device is touched
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--kv-heads", "7"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode != 0
    assert "must divide H = 40" in (r.stdout + r.stderr)


def test_rocprof_summary_reads_kernel_rows(tmp_path):
    db = tmp_path / "k_results.db"
    con = sqlite3.connect(db)
    con.execute("create table kernels (name text, duration integer)")
    con.executemany("insert into kernels values (?, ?)",
                    [("sage::attn_fwd_kernel<128, false, false, 0>(sage::AttnArgs)", 3000000),
                     ("sage::attn_fwd_kernel<128, false, false, 0>(sage::AttnArgs)", 4000000),
                     ("sage::zero_kernel(int __vector(4)*, long)", 5000)])
    con.commit()
    con.close()
    text = bench.rocprof_summary(str(db))
    assert "sage::attn_fwd_kernel<128, false, false, 0> | 2 | 3500.00" in text
    assert "sage::zero_kernel | 1 | 5.00" in text
