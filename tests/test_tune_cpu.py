"""The tuner's table logic and the committed table (no GPU needed)."""
import os
import re

import exact_attention_85_amd as fa2
from exact_attention_85_amd import tune

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_table_rows_pick_the_fastest_and_merge_neighbours():
    results = {(128, 0): {1024: {0: 1.0, 4: 1.2}, 4096: {0: 2.0, 4: 1.5}, 16384: {0: 9.0, 4: 8.0}},
               (64, 1): {1024: {1: 0.5, 3: 0.7}, 4096: {1: 1.0, 3: 0.9}}}
    rows = tune.table_rows(results)
    assert rows[(128, 0)] == [(1, 0), (2048, 4)]      # 4096 and 16384 both pick 4: merged
    assert rows[(64, 1)] == [(1, 1), (2048, 3)]
    # ties (within 2.5 %) go to the previous length's choice, then to the renumbered head-major
    # order (configs 0, 4, 8), then to the faster
    tied = {(128, 0): {1024: {0: 1.00, 2: 0.99}, 4096: {4: 1.00, 6: 0.985, 7: 0.90}, 8192: {4: 1.0, 6: 0.99}}}
    assert tune.table_rows(tied)[(128, 0)] == [(1, 0), (2048, 7), (5793, 4)]
    kept = {(128, 1): {1024: {2: 1.0, 0: 1.1}, 4096: {2: 1.01, 0: 1.0}, 16384: {2: 1.2, 0: 1.0}}}
    assert tune.table_rows(kept)[(128, 1)] == [(1, 2), (8192, 0)]


def test_written_header_round_trips(tmp_path):
    rows = {(64, 0): [(1, 0)], (64, 1): [(1, 1), (2048, 3)], (128, 0): [(1, 0), (2896, 4)], (128, 1): [(1, 5)]}
    path = tmp_path / "t.h"
    tune.write_header(str(path), rows, "test")
    got = re.findall(r"\{(\d+), (\d+), (\d+), (\d+)\},", path.read_text())
    assert [tuple(map(int, g)) for g in got] == [(d, b, m, c) for (d, b), rs in sorted(rows.items()) for m, c in rs]


def test_committed_table_covers_every_shape_class():
    text = open(os.path.join(ROOT, "exact_attention_85_amd", "csrc", "fa2_tune_table.h")).read()
    rows = [tuple(map(int, g)) for g in re.findall(r"\{(\d+), (\d+), (\d+), (\d+)\},", text)]
    n = fa2.num_configs()
    for d in (64, 128):
        for b in (0, 1):
            mins = [m for (dd, bb, m, c) in rows if dd == d and bb == b]
            assert 1 in mins, (d, b)
    assert all(0 <= c < n for (_, _, _, c) in rows)
    # the library answers from the same table
    for (d, b, m, c) in rows:
        assert fa2.default_config(d, b, m) == c
