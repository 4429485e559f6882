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


DTN = {0: "f32", 1: "bf16", 2: "f16", 3: "mxfp8", 4: "mxfp4"}


@pytest.mark.parametrize("row", _entries())
def test_tuned_plan_is_returned(row):
    dt, M, N, K, vid, split, raster = row
    dtype = DTN[dt]
    p = sam.plan(M, N, K, dtype)
    assert (p["variant_id"], p["split_k"], p["raster_n"]) == (vid, split, raster)
    assert p["name"].endswith("_tuned") and p["tuned"] == 1
    # the fastest measured candidate is what the table holds
    best = tune.load(RECORD)[(dtype, M, N, K)][0]
    assert (best["variant"], best["split"], best["raster"]) == (vid, split, raster)


def test_shape_in_a_measured_bucket_takes_its_plan():
    """2040 x 2056 x 2064 shares the half-octave buckets of the measured
    2048^3: it takes that shape's variant and raster order."""
    p = sam.plan(2040, 2056, 2064, "f32")
    ref = sam.plan(2048, 2048, 2048, "f32")
    assert p["tuned"] == 2 and p["name"].endswith("_bucket")
    assert (p["variant_id"], p["raster_n"]) == (ref["variant_id"], ref["raster_n"])
    assert sam.plan(2040, 2056, 2064, "f32") == p   # pure function of the shape


def test_bucket_split_is_replanned_when_the_tile_count_differs():
    """A bucket shape takes the measured split only when its tile count is the
    measured shape's; otherwise the variant's own split or stream-K choice
    (2040 x 2056 x 2064: 272 tiles of 128 x 128 against 2048^3's 256)."""
    p = sam.plan(2040, 2056, 2064, "f32")
    own = sam.variant_plan(p["variant_id"], 2040, 2056, 2064, "f32", 0, p["raster_n"])
    assert p["tuned"] == 2 and (p["split_k"], p["grid_wgs"]) == (own["split_k"], own["grid_wgs"])
    q = sam.plan(3000, 3000, 2990, "f32")                  # 3000^3's tiles: its split kept
    ref = sam.plan(3000, 3000, 3000, "f32")
    assert q["tuned"] == 2 and q["variant_id"] == ref["variant_id"] and q["split_k"] == ref["split_k"]


def test_shape_outside_every_bucket_uses_the_cost_model():
    p = sam.plan(2040, 2056, 700, "f32")
    assert p["tuned"] == 0 and not p["name"].endswith(("_tuned", "_bucket"))
    assert p == sam.plan_model(2040, 2056, 700, "f32")
    assert sam.plan(2040, 2056, 700, "f32") == p


# The cost model alone (no frozen table) against the measured record: on
# every recorded shape its pick was measured too (it is one of the
# candidates), and it must be within this factor of the fastest one.
MODEL_MARGIN = 1.30


def test_cost_model_pick_is_near_the_measured_best():
    worst = []
    for (dtype, M, N, K), rs in tune.load(RECORD).items():
        mp = sam.plan_model(M, N, K, dtype)
        key = (mp["variant_id"], mp["split_k"], mp["raster_n"])
        mine = next((r for r in rs if (r["variant"], r["split"], r["raster"]) == key), None)
        assert mine is not None, f"{dtype} {(M, N, K)}: the model's pick {mp['name']} was never measured"
        worst.append((mine["ms"] / rs[0]["ms"], dtype, (M, N, K), mp["name"], rs[0]["plan"]))
    worst.sort(reverse=True)
    assert worst[0][0] <= MODEL_MARGIN, worst[:3]
