"""The bench's host-side accounting, on the CPU: the algorithmic bytes the
roofline divides by, the gate that keeps a counter file taken on other
sources out of `traffic`, and the refusal of more than one GPU."""

import json
import os
import subprocess
import sys

import numpy as np

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_algorithmic_bytes_of_the_gqa_workload():
    """KV + Q + O + block tables (and context lengths) of the bf16 GQA step,
    counted here from the workload's lengths: every context token's key and
    value row of every kv head in bf16, one query and one output row per
    (sequence, query head), one int32 table entry per block and one length
    per sequence."""
    wl = synth.make(3)
    c = wl.cfg
    L = np.asarray(wl.context_lens, dtype=np.int64)
    kv = sum(int(n) * c.H_kv * c.d * 2 * 2 for n in L)
    qo = 2 * c.S * c.H_q * c.d * 2
    tables = sum(-(-int(n) // c.bs) for n in L) * 4 + c.S * 4
    ab = bench.algorithmic_bytes(wl)
    assert ab["kv"] == kv
    assert ab["decode"] == kv + qo + tables == 1_063_927_532
    # the step adds the new rows' store: one key and one value row per (sequence, kv head)
    assert ab["step"] - ab["decode"] == c.S * c.H_kv * c.d * 2 * (2 + 2)


def test_prefix_unique_bytes_count_shared_blocks_once():
    wl = synth.make(4)
    c = wl.cfg
    L = np.asarray(wl.context_lens, dtype=np.int64)
    shared = (c.prefix // c.bs) * c.bs
    row = c.H_kv * c.d * 2 * 2
    ab = bench.algorithmic_bytes(wl)
    assert ab["kv_unique"] == (shared + int((L - shared).sum())) * row
    assert ab["kv"] - ab["kv_unique"] == (c.S - 1) * shared * row


def test_traffic_file_is_used_only_for_its_kernel_and_sources(tmp_path):
    path = tmp_path / "traffic.json"
    rec = {"kernel": "decode (split-K partials)", "kernel_src_sha": bench.src_sha(),
           "hbm_bytes_per_launch": 123.0}
    path.write_text(json.dumps(rec))
    assert bench.load_traffic(str(path), "x", "decode (split-K partials)") == 123.0
    assert bench.load_traffic(str(path), "x", "decode (stream-K)") is None
    path.write_text(json.dumps(dict(rec, kernel_src_sha="0" * 16)))
    assert bench.load_traffic(str(path), "x", "decode (split-K partials)") is None
    assert bench.load_traffic(str(tmp_path / "absent.json"), "x", "decode (split-K partials)") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
