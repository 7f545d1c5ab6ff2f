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
    spec.loader.exec_module(mod)
    return mod


def _token_bytes(key_bits, value_bits, d=128):
    # codes of one token-head, fp16 scale and zero for its key and its value row, int32 position
    return d * key_bits // 8 + d * value_bits // 8 + 4 * 2 + 4


HIGH_B, LOW_B = _token_bytes(8, 4), _token_bytes(4, 2)     # K8V4 and K4V2 tiers


def test_decode_bytes_count_codes_pages_query_and_output():
    b = _bench()
    # two requests x two KV heads; page counts: HIGH pages hold 16 tokens, LOW pages 32
    count = np.array([[[16, 32], [17, 0]], [[0, 33], [0, 0]]], dtype=np.int32)
    Hq = 8
    pages = (1 + 1) + (2 + 0) + (0 + 2) + 0
    want = (16 + 17) * HIGH_B + (32 + 33) * LOW_B + 4 * pages + 2 * Hq * 128 * (2 + 4)
    assert b.decode_algorithmic_bytes(count, 2, Hq) == want


def test_compaction_bytes_count_inputs_pages_and_tables():
    b = _bench()
    count = np.array([[[5, 40]]], dtype=np.int32)
    T, Hkv, Hq = 50, 1, 4                  # 5 pruned tokens: their K/V rows still count as input
    want = T * Hkv * 128 * 2 * 2 + T * Hq * 4 + 5 * HIGH_B + 40 * LOW_B + 4 * (1 + 2)
    assert b.compaction_algorithmic_bytes(count, T, Hkv, Hq) == want


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]
