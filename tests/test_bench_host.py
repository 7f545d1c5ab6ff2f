"""Host logic of bench.py (no GPU): the algorithmic byte counts behind its GB/s and roofline
figures, and its refusal of more than one GPU."""
import importlib.util
import json
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    sys.modules["bench_mod"] = mod          # its process pool names functions by module
    spec.loader.exec_module(mod)
    return mod


def _token_bytes(key_bits, value_bits, d=128, position=True):
    # codes of one token-head, fp16 scale and zero for its key and its value row, and (in the
    # page) its int32 position
    return d * key_bits // 8 + d * value_bits // 8 + 4 * 2 + (4 if position else 0)


HIGH_B, LOW_B = _token_bytes(8, 4), _token_bytes(4, 2)     # K8V4 and K4V2 tiers
HIGH_R, LOW_R = _token_bytes(8, 4, position=False), _token_bytes(4, 2, position=False)


def test_decode_bytes_count_codes_pages_query_and_output():
    b = _bench()
    # two requests x two KV heads; page counts: HIGH pages hold 16 tokens, LOW pages 32; the
    # decode reads codes and scale/zero pairs, not the stored positions
    count = np.array([[[16, 32], [17, 0]], [[0, 33], [0, 0]]], dtype=np.int32)
    Hq = 8
    pages = (1 + 1) + (2 + 0) + (0 + 2) + 0
    want = (16 + 17) * HIGH_R + (32 + 33) * LOW_R + 4 * pages + 2 * Hq * 128 * (2 + 4)
    assert b.decode_algorithmic_bytes(count, 2, Hq) == want
    # the accumulating decode also reads positions and reads + writes one fp32 accumulator
    # per live token and query head (G = 4 here)
    live = 16 + 32 + 17 + 33
    assert b.decode_acc_algorithmic_bytes(count, 2, Hq, 2) == want + live * 4 + live * 4 * 8


def test_compaction_bytes_count_inputs_pages_and_tables():
    b = _bench()
    count = np.array([[[5, 40]]], dtype=np.int32)
    T, Hkv, Hq = 50, 1, 4                  # 5 pruned tokens: their K/V rows are never read
    want = 45 * 128 * 2 * 2 + T * Hq * 4 + 5 * HIGH_B + 40 * LOW_B + 4 * (1 + 2)
    assert b.compaction_algorithmic_bytes(count, T, Hkv, Hq) == want


def test_cold_stats_median_and_min():
    b = _bench()
    st = b.stats([10.0, 30.0, 20.0], 2e6)          # 2 MB per rep
    assert st["us_median"] == 20.0 and st["us_min"] == 10.0
    assert st["GBps_median"] == 100.0 and st["GBps_max"] == 200.0
    assert abs(st["frac_hbm_median"] - 100.0 / 8000.0) < 1e-12


def test_cpu_baseline_one_core_and_pool():
    # the oracle on a small workload: one core, then a process pool; the record names both
    b = _bench()
    from mixed_precision_paged_score_amd import workloads
    w = workloads.Workload("cpu-small", 1, 6, 16, 4, [40, 300, 1, 77, 0, 129], 1.0, 0.2, 16,
                           4096, "zipf", seed=5)
    r = b.cpu_baseline(w)
    assert r["kind"] == "oracle" and r["cores"] >= 1 and r["single_core"]["cores"] == 1
    assert r["value"] > 0 and r["single_core"]["value"] > 0
    assert r["nproc"] >= r["cores"] and isinstance(r["cpu_model"], str)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]
