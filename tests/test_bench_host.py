"""Host-side checks of bench.py (no GPU): the arguments it refuses, and the algorithmic
bytes its HBM roofline divides by."""
import math
import subprocess
import sys
from pathlib import Path

import numpy as np

ROOT = Path(__file__).resolve().parents[1]
sys.path.insert(0, str(ROOT))

import bench  # noqa: E402
import workloads as W  # noqa: E402


def _run(*argv):
    return subprocess.run([sys.executable, str(ROOT / "bench.py"), *argv], capture_output=True, text=True,
                          timeout=300)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _run("--gpus", "2")
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_step_counts_below_one_are_refused():
    assert _run("--steps", "0").returncode != 0
    assert _run("--warmup", "-1").returncode != 0


def test_algorithmic_bytes_count_every_token_table_entry_and_scale():
    """Per sequence: its context's K and V rows for every KV head, its query and output
    rows, one table entry per block and its length; E4M3 pools add a K and a V scale per
    (block, KV head).  Summed here sequence by sequence with Python integers."""
    for name in ("llama7b", "llama13b_long", "llama70b_gqa", "llama7b_fp8", "prefix_sharing"):
        w = W.WORKLOADS[name]
        ctx = W.draw_lengths(w)[0].context_lens
        kv_b = 1 if w.kv == "fp8" else w.elem_bytes
        total = 0
        for c in ctx.tolist():
            blocks = math.ceil(c / w.block_size)
            total += c * 2 * w.num_kv_heads * w.head_dim * kv_b
            total += 2 * w.num_q_heads * w.head_dim * w.elem_bytes
            total += 4 * blocks + 4
            if w.kv == "fp8":
                total += 2 * 4 * blocks * w.num_kv_heads
        ab = bench.algorithmic_bytes(w, np.asarray(ctx))
        assert ab["total"] == total, name
        assert ab["kv"] == int(ctx.sum()) * 2 * w.num_kv_heads * w.head_dim * kv_b, name


def test_unique_bytes_count_a_shared_token_once():
    w = W.WORKLOADS["prefix_sharing"]
    ctx = W.draw_lengths(w)[0].context_lens
    ab = bench.algorithmic_bytes(w, np.asarray(ctx), unique_tokens=1000)
    assert ab["kv_unique"] == 1000 * 2 * w.num_kv_heads * w.head_dim * w.elem_bytes
    assert ab["total"] - ab["kv"] == ab["total_unique"] - ab["kv_unique"]
