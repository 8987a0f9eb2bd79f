"""bench.py's host-side pieces: algorithmic byte accounting, workloads and
the one-GPU guard (no GPU needed)."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_history_unit_bytes():
    # 2 x 32 code bytes + 2 x (128 / G) bf16 (scale, zero) pairs per token and KV head
    assert bench.hist_unit_bytes(128) == 72
    assert bench.hist_unit_bytes(64) == 80
    assert bench.hist_unit_bytes(32) == 96


def test_step_bytes_by_hand():
    lens = np.array([100, 320, 1000])
    hkv, hq, g = 2, 8, 128
    hist, total = bench.step_bytes(lens, hkv, hq, g)
    n_hist = 0 + 0 + 680
    assert hist == n_hist * hkv * 72
    bf16 = (100 + 320 + 320) * hkv * 512
    qo = 3 * hq * 128 * 6
    demoted = 1 * hkv * (512 + 72)          # only the request past 320 tokens demotes
    appended = 3 * hkv * 512
    assert total == hist + bf16 + qo + demoted + appended
    assert bench.bf16_bytes(lens, hkv) == bf16


def test_workloads_and_default_steps():
    wl = bench.workloads()
    assert {"b32-100k-g128", "b32-100k-g64", "b32-100k-g128-lloyd", "b1-100k", "b16-128k",
            "b32-ragged-gqa8"} <= set(wl)
    w = wl["b32-100k-g128"]()
    assert (w.batch, w.num_q_heads, w.num_kv_heads, w.group_size) == (32, 32, 8, 128)
    assert set(w.seq_lens) == {100_000} and w.paged and w.codebook == 0
    assert wl["b32-100k-g128-lloyd"]().codebook == 1
    assert wl["b1-100k"]().steps == 100
    r = wl["b32-ragged-gqa8"]()
    assert r.steps == 200 and r.num_q_heads == 64 and r.shared_prefix
    assert min(r.seq_lens) >= 4096 and max(r.seq_lens) <= 131072
    assert bench.default_layers("b1-100k") == 10 and bench.default_layers("b32-100k-g128") == 1


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr


def test_source_sha_ignores_comments_but_not_code(tmp_path):
    from bit_rotated_kv_split_amd.profiling import source_sha
    d = tmp_path / "bit_rotated_kv_split_amd" / "csrc"
    d.mkdir(parents=True)
    (d / "decode_x.hip").write_text("int f() {\n  return 1;  // one\n}\n")
    (d / "other.hip").write_text("int g();\n")
    base = source_sha(str(tmp_path))
    (d / "decode_x.hip").write_text("// header\nint f() {\n  /* the\n     value */ return 1;   // uno\n\n}\n")
    assert source_sha(str(tmp_path)) == base
    (d / "other.hip").write_text("int g(); int h();\n")      # not a decode source
    assert source_sha(str(tmp_path)) == base
    (d / "decode_x.hip").write_text("int f() {\n  return 2;\n}\n")
    assert source_sha(str(tmp_path)) != base


def test_oracle_workers_run_the_oracle_in_parallel_processes():
    """The CPU-baseline workers (spawned processes, one BLAS thread each) run
    the oracle's request_attention on the tasks they are given and report
    their busy time on a shared clock."""
    from oracle import oscar as O
    rng = np.random.default_rng(5)
    L, g = 700, 2

    def bits(shape):
        x = (rng.standard_normal(shape)).astype(np.float32)
        return (x.view(np.uint32) >> 16).astype(np.uint16)

    r = O.composite_rotation(np.eye(128)).astype(np.float32)[None]
    clip = np.full((1, 128), 3.0, np.float32)
    task = ((bits((g, 128)), bits((L, 1, 128)), bits((L, 1, 128)), r, r, clip, clip, 128, "uniform"), 1000)
    ref, _ = O.request_attention(*task[0])
    workers = bench.OracleWorkers(2)
    try:
        nbytes, wall, busy = workers.run([[task, task], [task]])
        assert nbytes == 3000 and wall > 0 and len(busy) == 2
        assert max(busy) <= wall + 1e-6
        nbytes, wall, busy = workers.run([[task], []])
        assert nbytes == 1000 and len(busy) == 1
    finally:
        workers.close()
    assert np.isfinite(ref).all()
    assert bench.cpu_worker_count() >= 1


def test_quarter_means():
    assert bench.quarters([4, 4, 2, 2, 2, 2, 1, 1]) == [4.0, 1.0]
    assert bench.quarters([3.0]) == [3.0, 3.0]


def test_counter_derived_figures():
    """Per-page counts and busy fractions from summed SQ counters: 1024
    SIMDs each issuing 1000 wave64 instructions (4 cycles each) over 8000
    kernel cycles are half busy."""
    from bit_rotated_kv_split_amd.profiling import derived
    vals = {"SQ_INSTS_VALU": 1024 * 1000.0, "SQ_INSTS_MFMA": 512.0, "SQ_VALU_MFMA_BUSY_CYCLES": 1024 * 2000.0,
            "GRBM_GUI_ACTIVE": 8 * 8000.0}
    d = derived(vals, page_heads=256.0)
    assert d["SQ_INSTS_VALU per page-head"] == 4000.0
    assert d["SQ_INSTS_MFMA per page-head"] == 2.0
    assert d["vector ALU busy (4 cycles per instruction)"] == 0.5
    assert d["matrix core busy"] == 0.25
    assert derived({"SQ_INSTS_VALU": 1.0}, page_heads=0.0) == {}
