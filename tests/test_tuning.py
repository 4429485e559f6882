"""The frozen dispatch table (row: offline measured autotune).

The table in csrc/sam_tuned.h must be exactly what tune.py emits from the
committed measurement record, and the dispatcher must return each tuned
(variant, split) for its shape. No GPU needed: the planner is host code.
"""
from pathlib import Path

import pytest

import shape_adaptive_matrix_amd as sam
from shape_adaptive_matrix_amd import tune

RECORD = Path(tune.PKG) / "tuning" / "tuning_sweep.jsonl"


def test_table_is_the_record_emitted(tmp_path):
    out = tmp_path / "sam_tuned.h"
    tune.emit(RECORD, out)
    assert out.read_text() == tune.TUNED_H.read_text()


def _entries():
    rows = []
    for line in tune.TUNED_H.read_text().splitlines():
        line = line.strip()
        if line.startswith("T(") and line.rstrip(" \\").endswith(")"):
            rows.append(tuple(int(x) for x in line.rstrip(" \\")[2:-1].split(",")))
    return rows


def test_table_covers_every_measured_shape():
    assert len(_entries()) == len(tune.load(RECORD)) > 0


@pytest.mark.parametrize("row", _entries())
def test_tuned_plan_is_returned(row):
    dt, M, N, K, vid, split = row
    dtype = {0: "f32", 1: "bf16", 2: "f16", 3: "mxfp8", 4: "mxfp4"}[dt]
    p = sam.plan(M, N, K, dtype)
    assert (p["variant_id"], p["split_k"]) == (vid, split)
    assert p["name"].endswith("_tuned")
    # the fastest measured candidate is what the table holds
    best = tune.load(RECORD)[(dtype, M, N, K)][0]
    assert (best["variant"], best["split"]) == (vid, split)


def test_untuned_shape_uses_the_cost_model():
    p = sam.plan(2040, 2056, 2064, "f32")
    assert not p["name"].endswith("_tuned")
    assert sam.plan(2040, 2056, 2064, "f32") == p   # pure function of the shape
