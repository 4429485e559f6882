"""The seeded input generators (CPU): ranges, exactness and the 16-bit
rounding, the last checked against torch's own float32 -> bfloat16 cast."""
import numpy as np
import torch

import sam_inputs as si


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.00390625, 1.01171875, -3.5, 65504.0, 1e-30, -0.0], np.float32)])
    ours = si.bf16_rne_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_uniform_range_and_exactness():
    x = si.uniform_pm1(np.random.default_rng(1), (1000, 100))
    assert x.dtype == np.float32 and x.min() >= -1.0 and x.max() < 1.0
    # multiples of 2^-23: exact in FP32
    assert np.all((x.astype(np.float64) * 2 ** 23) == np.round(x.astype(np.float64) * 2 ** 23))


def test_ints_closed_range():
    x = si.small_ints(np.random.default_rng(2), (100000,), -4, 4)
    assert set(np.unique(x).tolist()) == set(range(-4, 5))


def test_workloads_match_the_stated_configs():
    names = {w.name: w for w in si.WORKLOADS}
    assert names["f32_256_ints"].check == "bitexact" and (names["f32_256_ints"].lo, names["f32_256_ints"].hi) == (-4, 4)
    assert names["f32_2048_ints"].check == "bitexact" and (names["f32_2048_ints"].lo, names["f32_2048_ints"].hi) == (-2, 2)
    shapes = {(w.M, w.N, w.K) for w in si.WORKLOADS}
    for s in [(768, 768, 768), (4097, 3071, 8191), (8191, 8193, 4096), (16, 8192, 8192),
              (8192, 16, 8192), (8192, 8192, 64)]:
        assert s in shapes
    every = si.WORKLOADS + si.MX_WORKLOADS + si.LLM_WORKLOADS + si.LLM_MX_WORKLOADS
    assert len({w.seed for w in every}) == len(every)


def test_mx_recipes():
    """Codes are finite in their format; dyadic codes stay in [1, 4) or are
    zero; scale codes stay in their stated ranges; draws are reproducible."""
    import torch
    for fmt, t in (("e4m3", torch.float8_e4m3fn), ("e5m2", torch.float8_e5m2)):
        for dist in ("mx_normal", "mx_dyadic"):
            w = si.Workload("t", "mxfp8", 37, 29, 96, dist, 5, fmt_a=fmt, fmt_b=fmt)
            A, SA, Bt, SB = si.make_mx_operands(w)
            assert A.shape == (37, 96) and Bt.shape == (29, 96) and SA.shape == (37, 3) and SB.shape == (29, 3)
            for x in (A, Bt):
                v = torch.from_numpy(x).view(t).double().numpy()
                assert np.isfinite(v).all()
                if dist == "mx_dyadic":
                    a = np.abs(v)
                    assert ((a == 0) | ((a >= 1) & (a < 4))).all()
            lo, hi = (123, 131) if dist == "mx_normal" else (126, 128)
            for s in (SA, SB):
                assert s.min() >= lo and s.max() <= hi
            again = si.make_mx_operands(w)
            assert all(np.array_equal(x, y) for x, y in zip((A, SA, Bt, SB), again))


def test_sample_points_distinct_and_cover_tails():
    r, c = si.sample_points(8191, 8193, 4096, seed=3)
    flat = r * 8193 + c
    assert len(np.unique(flat)) == len(flat) >= 4096
    assert (8190, 8192) in set(zip(r.tolist(), c.tolist())) and (0, 0) in set(zip(r.tolist(), c.tolist()))
