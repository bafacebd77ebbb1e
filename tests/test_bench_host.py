"""bench.py's host logic on a machine without a GPU: the byte counts the
roofline divides by, the refusal of more than one GPU, and the summaries it
writes from profiler output (kernel trace, counters, wave timeline), each on
small hand-made inputs whose figures are worked out here."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_weight_and_algorithmic_bytes():
    # 3-bit codes of a 10240 x 5120 weight: 19,660,800 bytes; one bf16 scale
    # and one bf16 bias per group of 64: 2 * 10240 * 80 * 2 = 3,276,800
    assert bench.weight_bytes() == 19_660_800 + 3_276_800 == 22_937_600
    # plus the activations (64 x 5120 bf16) and the output (64 x 10240 bf16)
    assert bench.algorithmic_bytes(64) == 22_937_600 + 655_360 + 1_310_720 == 24_903_680
    assert bench.algorithmic_bytes(1) == 22_937_600 + 10_240 + 20_480


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stdout + r.stderr


def _trace_csv(path, durations_ns, name="void qmm::k<1>(qmm::LaunchArgs)", lds=512):
    with open(path, "w") as f:
        f.write("Kernel_Name,LDS_Block_Size,Grid_Size_X,Workgroup_Size_X,Start_Timestamp,End_Timestamp\n")
        t = 1000
        for d in durations_ns:
            f.write('"%s",%d,%d,%d,%d,%d\n' % (name, lds, 214 * 512, 512, t, t + d))
            t += d + 100


def test_trace_summary_quantiles(tmp_path):
    # ten dispatches of 1..10 us (given out of order): sorted, the median is
    # the 6th value (index 5), p10 the 2nd, p90 the 10th
    p = tmp_path / "kt.csv"
    _trace_csv(p, [d * 1000 for d in (7, 3, 10, 1, 5, 9, 2, 8, 4, 6)])
    out = bench.trace_summary(str(p))
    row = [c.strip() for c in out.splitlines()[2].strip("|").split("|")]
    assert row[0] == "`qmm::k<1>`"
    assert row[1:4] == ["512", "214", "10"]
    assert [float(v) for v in row[4:]] == [6.0, 2.0, 10.0, 1.0, 10.0]


def test_counter_summary_means_per_dispatch(tmp_path):
    # two dispatches of one kernel, each counter reported by two hardware
    # blocks: per dispatch the blocks add up (10 + 30, then 20 + 40), and the
    # table holds the mean over dispatches (50) and of the durations
    p = tmp_path / "pmc.csv"
    rows = [("1", "SQ_WAVES", 10), ("1", "SQ_WAVES", 30), ("2", "SQ_WAVES", 20),
            ("2", "SQ_WAVES", 40)]
    with open(p, "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value,Start_Timestamp,End_Timestamp\n")
        for d, c, v in rows:
            start = 0 if d == "1" else 10_000
            dur = 4_000 if d == "1" else 6_000
            f.write('%s,"void qmm::k<1>(qmm::LaunchArgs)",%s,%d,%d,%d\n' % (d, c, v, start,
                                                                              start + dur))
    out = bench.counter_summary([str(p)])
    lines = out.splitlines()
    assert lines[0] == "| kernel | dispatches | mean us | SQ_WAVES |"
    assert lines[2] == "| `k<1>` | 2 | 5.00 | 50 |"


def test_timeline_summary_tables(tmp_path):
    d = {"resident 9 row(s)": {"workgroups": 214, "waves": 1712,
                               "start": [0.0, 0.04, 0.13, 0.26, 0.3],
                               "compute done": [4.17, 4.66, 5.72, 6.42, 6.88],
                               "compute done, median by wave index": [4.8, 6.3]}}
    p = tmp_path / "tl.json"
    p.write_text(json.dumps(d))
    out = bench.timeline_summary(str(p))
    assert "## resident 9 row(s): 214 workgroups, 1712 waves" in out
    assert "| start | 0.00 | 0.04 | 0.13 | 0.26 | 0.30 |" in out
    assert "| compute done | 4.17 | 4.66 | 5.72 | 6.42 | 6.88 |" in out
    assert "Compute done, median by wave index: 4.80, 6.30" in out


def test_kernel_source_hash_format():
    h = bench.kernel_source_hash()
    assert len(h) == 16 and all(c in "0123456789abcdef" for c in h)
    assert h == bench.kernel_source_hash()
