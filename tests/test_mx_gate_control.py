"""Negative control for the block-scaled random-input gate (CPU only).

The full-size block-scaled parity tests accept an output when every compared
element lies within 2^-12 * sum_k |a_k b_k| of the oracle and the rel_rms of
the compared elements is at most 5e-5 (``tests.compare``). This shows the
gate is not vacuous at the workloads' own sizes: an "output" computed by the
oracle itself from inputs with one planted mistake -- a block scale doubled,
or one 32-value block of codes dropped, both in a single row of A -- must be
rejected on the points of that row, while the true result rounded to FP32
passes. Everything here is oracle arithmetic; no GPU is involved.
"""
import numpy as np
import pytest

import oracle
import sam_inputs as si
from tests.compare import MX_REL_RMS, mx_bound_excess, rel_rms

ROW = 1234          # the row that carries the planted mistake
BLOCK = 57          # the 32-value block of K it hits


def _points(w):
    """The parity test's own sample plus every column of ROW."""
    r, c = si.sample_points(w.M, w.N, 1500, seed=w.seed)
    rows = np.concatenate([r, np.full(w.N, ROW, np.int64)])
    cols = np.concatenate([c, np.arange(w.N, dtype=np.int64)])
    return rows, cols


def _eval(o, w, ops, rows, cols):
    A, SA, Bt, SB = ops
    if w.dtype == "mxfp8":
        return o.gemm_mxfp8_points(w.fmt_a, w.fmt_b, A, SA, Bt, SB, rows, cols)
    return o.gemm_mxfp4_points(A, SA, Bt, SB, rows, cols)


def _abs_sum(o, w, ops, rows, cols):
    A, SA, Bt, SB = ops
    mask = 0x7F if w.dtype == "mxfp8" else 0x77   # clear the sign bit of every code
    return _eval(o, w, (A & mask, SA, Bt & mask, SB), rows, cols)


def _plant(w, ops, kind):
    A, SA, Bt, SB = (x.copy() for x in ops)
    if kind == "doubled_scale":
        SA[ROW, BLOCK] += 1                        # E8M0: one more in the code doubles the scale
    else:
        per_byte = 1 if w.dtype == "mxfp8" else 2
        A[ROW, BLOCK * 32 // per_byte:(BLOCK + 1) * 32 // per_byte] = 0
    return A, SA, Bt, SB


@pytest.mark.parametrize("name", ["mxfp8_4096", "mxfp4_4096"])
@pytest.mark.parametrize("kind", ["doubled_scale", "dropped_block"])
def test_gate_rejects_planted_mistake(name, kind):
    w = si.by_name(name)
    o = oracle.get()
    ops = si.make_mx_operands(w)
    rows, cols = _points(w)
    ref = _eval(o, w, ops, rows, cols)
    absum = _abs_sum(o, w, ops, rows, cols)
    # The true result in FP32 passes both gates.
    exact32 = ref.astype(np.float32)
    assert mx_bound_excess(exact32, ref, absum) <= 0
    assert rel_rms(exact32, ref) <= MX_REL_RMS
    # The planted mistake fails both, on the points of its row.
    bad = _eval(o, w, _plant(w, ops, kind), rows, cols)
    on_row = rows == ROW
    assert mx_bound_excess(bad[on_row], ref[on_row], absum[on_row]) > 0
    assert rel_rms(bad[on_row], ref[on_row]) > MX_REL_RMS
    # Many elements of the row are out of bounds one by one (a block whose
    # scale is small next to the row's largest ones moves some of them by
    # less than the bound, so not all).
    err = np.abs(bad[on_row] - ref[on_row])
    share = float(np.mean(err > 2.0 ** -12 * absum[on_row]))
    print(f"{name} {kind}: {share:.2f} of the row's elements out of bounds")
    assert share > 0.1
    # Points off the row are untouched.
    assert np.array_equal(bad[~on_row], ref[~on_row])
