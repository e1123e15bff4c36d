"""Host-side accounting of bench.py: the algorithmic bytes and flops its roofline
figures divide by, checked against counts made element by element on tiny shapes."""

import dataclasses

import numpy as np

import bench
from workloads import PRESETS


def _tiny(**kw):
    return dataclasses.replace(PRESETS["tiny"], **kw)


def test_attention_flops_count_every_visible_key():
    p = _tiny(B=3, k=2, Hq=4, Hkv=2, D=64)
    L = np.array([5, 0, 17])
    want = 0
    for b in range(p.B):
        for i in range(p.k + 1):            # row i sees keys 0 .. L_b + i
            want += p.Hq * 4 * p.D * (L[b] + i + 1)
    assert bench.attention_flops(p, L) == want


def test_algorithmic_bytes_read_each_examined_row_once():
    p = _tiny(B=2, k=3, V=10, Hq=4, Hkv=2, D=64, block_size=16)
    L = np.array([20, 3])
    a = np.array([1, 3])                    # accepted drafts
    attn, rej, commit = bench.algorithmic_bytes(p, L, a)
    n_keys = L + p.k + 1
    kv = int(np.sum(n_keys)) * p.Hkv * p.D * 2 * 2
    qo = 2 * p.B * (p.k + 1) * p.Hq * p.D * 2
    bt = int(np.sum((n_keys + p.block_size - 1) // p.block_size)) * 4 + p.B * 4
    assert attn == kv + qo + bt
    # sequence 0 rejects at level 1: p_0, p_1, q_0, q_1; sequence 1 accepts all: p_0..p_3, q_0..q_2
    rows = (2 + 2) + (4 + 3)
    small = p.B * p.k * 4 + p.B * (8 + 4) + p.B * (p.k + 1) * 8 + p.B * 4 + p.B * p.k * 4
    assert rej == rows * p.V * 4 + small
    assert commit == p.B * 4 * 3


def test_dense_figure_counts_all_rows():
    p = PRESETS["8b"]
    d = bench.dense_reject_figure(p, 1e-3)
    assert d["bytes"] == p.B * (2 * p.k + 1) * p.V * 4
    assert abs(d["gbs"] - d["bytes"] / 1e-3 / 1e9) < 1e-6


def test_more_than_one_gpu_is_refused_with_a_message():
    """One GPU only: --gpus 2 exits with status 2 and says why, before touching a device."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    res = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2
    assert "exactly one GPU" in res.stderr


def test_each_workload_line_takes_traffic_from_its_own_counter_run():
    # the counter summary a bench line cites must come from a run of that same line: its
    # recorded fetch command names the workload (none for the default, 8b) and no variant
    for workload in ("8b", "7b", "longtail", "262k"):
        path = bench.workload_counters(workload)
        with open(path) as f:
            cmd = next(line for line in f if line.startswith("# fetch command:"))
        args = cmd.split(" -- ", 1)[1].split()
        named = args[args.index("--workload") + 1] if "--workload" in args else "8b"
        assert named == workload, (workload, cmd)
        assert "--variant" not in args and "--sweep" not in args, cmd
    # plain decoding, the ragged step and the trees at the 8B shape have runs of their own,
    # naming that variant
    for variant, tree in (("plain", None), ("ragged", None), ("tree", "2,2"), ("tree", "2,3")):
        path = bench.workload_counters("8b", variant, tree)
        with open(path) as f:
            cmd = next(line for line in f if line.startswith("# fetch command:"))
        args = cmd.split(" -- ", 1)[1].split()
        assert args[args.index("--variant") + 1] == variant, cmd
        assert (args[args.index("--tree") + 1] if "--tree" in args else None) == tree, cmd
        assert "--workload" not in args, cmd
    # other launches (other trees, the fused pass) and other workloads have none
    for variant, tree in (("tree", "3,2"), ("fused", None)):
        assert bench.workload_counters("8b", variant, tree) is None
    assert bench.workload_counters("7b", "ragged") is None
    assert bench.workload_counters("tiny") is None


def test_clock_table_divides_the_die_summed_count_by_the_duration():
    # two dispatches of one kernel at 2.0 and 2.2 GHz (GRBM_COUNT summed over the 8 dies) and a
    # row of another counter, which is ignored; the median of two values is the upper one
    def row(name, counter, value, t0, t1):
        return {"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": str(value),
                "Start_Timestamp": str(t0), "End_Timestamp": str(t1)}
    rows = [row("void k<1>(int)", "GRBM_COUNT", 8 * 2.0 * 1000, 0, 1000),
            row("void k<1>(int)", "GRBM_GUI_ACTIVE", 1.0, 0, 1000),
            row("void k<1>(int)", "GRBM_COUNT", 8 * 2.2 * 500, 5000, 5500)]
    t = bench.clock_table(rows)
    (label,) = t
    n, us, ghz = t[label]
    assert n == 2 and abs(us - 1.0) < 1e-9 and abs(ghz - 2.2) < 1e-9
