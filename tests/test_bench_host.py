"""Host-side arithmetic of bench.py (no GPU): the algorithmic byte counts it divides by."""
import numpy as np

import bench


def test_decode_bytes_counts_kv_q_out_and_table_entries():
    # 2 texts of 5 and 17 tokens, 3 heads over 1 K/V head, D = 4, 2-byte elements, B = 4
    lens = [5, 17]
    want = (5 + 17) * 2 * 1 * 4 * 2 + 2 * 2 * 3 * 4 * 2 + 4 * (2 + 5)
    assert bench.decode_bytes(lens, 3, 4, 4, 2, 1, 2) == want


def test_unique_bytes_count_a_shared_block_once():
    B, Hkv, D, elt = 4, 2, 8, 2
    row = 2 * Hkv * D * elt                       # K and V of one token, all K/V heads
    # texts 0 and 1 share blocks 7 and 3 (3 is partly filled: 2 and 3 places attended);
    # text 1 goes on in block 9; text 2 is alone in block 5
    tables = np.array([[7, 3, -1], [7, 3, 9], [5, -1, -1]])
    lens = [6, 9, 1]
    # block 7: 4 places; block 3: max(2, 4) = 4 (text 1 fills it); block 9: 1; block 5: 1
    assert bench.unique_kv_bytes(tables, lens, B, Hkv, D, elt) == (4 + 4 + 1 + 1) * row
    # without sharing the same texts read every place they attend
    assert bench.decode_bytes(lens, Hkv, D, B, elt, Hkv, elt) - 2 * 3 * Hkv * D * elt \
        - 4 * (2 + 3 + 1) == (6 + 9 + 1) * row


def test_unique_bytes_take_the_most_filled_view_of_a_block():
    tables = np.array([[4], [4]])
    assert bench.unique_kv_bytes(tables, [1, 3], 4, 1, 2, 1) == 3 * 2 * 1 * 2 * 1


def test_config_summary_keeps_the_figures_of_a_configuration():
    line = {"roofline": {"avg_launch_us": 931.3, "median_launch_us": 930.7, "min_launch_us": 922.9,
                         "bytes_per_launch": 5737112369, "achieved": 6160.5, "frac": 0.7701,
                         "kernel": "k"},
            "ms_per_step": 1.9, "steps": 10, "config": {"layers_per_step": 2},
            "seq_layers_per_s": 268588.9, "cache_holding_tokens": 0.9933, "placement": "random"}
    s = bench.config_summary(line)
    assert s["op_us_mean"] == 931.3 and s["frac_of_hbm_peak"] == 0.7701
    assert s["cache_holding_tokens"] == 0.9933 and s["layers_per_step"] == 2


def test_more_than_one_gpu_is_refused():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True,
                       text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr
