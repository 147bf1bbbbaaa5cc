"""Pins for the oracle's grouped store (fp16 scale and zero per 128-token group; a reading
of the blog's "Where this does not work": 68 bytes per token per KV head).

Checked against numpy's IEEE float16 conversion, against the per-channel quantizer in
the cases where the two must agree, against brute-force nearest levels, numpy's var,
and a numpy matmul of the dequantized keys.
"""
import numpy as np
import pytest

import oracle


def test_f16_rounding_matches_numpy():
    rng = np.random.default_rng(0)
    vals = np.concatenate([
        rng.standard_normal(4000).astype(np.float32) * 10.0 ** rng.uniform(-9, 5, 4000),
        np.array([0.0, -0.0, 1.0, 65504.0, 65519.99, 65520.0, 70000.0, -65520.0,
                  2.0 ** -14, 2.0 ** -24, 2.0 ** -25, 1.5 * 2.0 ** -25, 2.0 ** -26,
                  1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 6.1e-5, np.inf, -np.inf],
                 np.float32)])
    with np.errstate(over="ignore"):
        want = vals.astype(np.float16).view(np.uint16)
    got = np.array([oracle.f32_to_f16_bits(v) for v in vals], np.uint16)
    assert np.array_equal(got, want)
    back = np.array([oracle.f16_bits_to_f32(h) for h in want], np.float32)
    assert np.array_equal(back, want.view(np.float16).astype(np.float32))


def test_single_group_with_fp16_exact_tables_is_the_per_channel_quantizer():
    """When a channel's min and (max - min)/15 are exact in fp16, rounding them changes
    nothing and one group spanning all tokens is the per-channel quantizer."""
    rng = np.random.default_rng(1)
    n, d = 300, 8
    x = rng.integers(0, 16, (n, d)).astype(np.float32) * np.float32(0.25) - 2.0
    x[0] = -2.0
    x[1] = 1.75   # every channel spans [-2, 1.75]: s = 0.25, z = -2
    s16, z16, codes = oracle.quantize_grouped(x, group=1024)
    s, z, ref = oracle.quantize(x)
    assert np.array_equal(codes, ref)
    assert np.array_equal(s16[:, 0].view(np.float16).astype(np.float32), s)
    assert np.array_equal(z16[:, 0].view(np.float16).astype(np.float32), z)


def test_grouped_codes_are_nearest_levels_and_groups_are_independent():
    rng = np.random.default_rng(2)
    n, d, group = 400, 5, 128
    x = (rng.standard_normal((n, d)) * [0.1, 1.0, 10.0, 100.0, 3.0]).astype(np.float32)
    s16, z16, codes = oracle.quantize_grouped(x, group)
    ng = (n + group - 1) // group
    assert s16.shape == (d, ng)
    for g in range(ng):
        sl = slice(g * group, min(n, (g + 1) * group))
        sf = s16[:, g].view(np.float16).astype(np.float32)
        zf = z16[:, g].view(np.float16).astype(np.float32)
        levels = zf[None, None, :] + sf[None, None, :] * np.arange(16, dtype=np.float32)[:, None, None]
        err = np.abs(x[sl][None] - levels)             # [16][tokens][d]
        best = err.min(axis=0)
        chosen = np.take_along_axis(err, codes[sl][None].astype(np.int64), 0)[0]
        # the chosen level is a nearest one (fp32 rounding of (x - z)/s may pick either
        # of two levels within one fp32 ulp of a tie)
        assert np.all(chosen <= best + 1e-6 * (np.abs(x[sl]) + sf[None, :]))
    # changing group 1's tokens leaves group 0 alone
    y = x.copy()
    y[group:2 * group] *= 7.0
    s2, z2, c2 = oracle.quantize_grouped(y, group)
    assert np.array_equal(c2[:group], codes[:group])
    assert np.array_equal(s2[:, 0], s16[:, 0]) and np.array_equal(z2[:, 0], z16[:, 0])


def test_grouped_variance_matches_numpy():
    rng = np.random.default_rng(3)
    n, d, group = 1000, 6, 128
    x = (rng.standard_normal((n, d)) * [0.5, 1, 2, 4, 8, 16] + 3.0).astype(np.float32)
    s16, z16, codes = oracle.quantize_grouped(x, group)
    var = oracle.var_grouped(codes, s16, z16, group)
    gi = np.arange(n) // group
    sf = s16.view(np.float16).astype(np.float64)[:, gi].T    # [n][d]
    zf = z16.view(np.float16).astype(np.float64)[:, gi].T
    deq = zf + sf * codes
    assert np.allclose(var, deq.var(axis=0), rtol=1e-6, atol=0)


@pytest.mark.parametrize("depth_kind", ["full", "mixed"])
def test_grouped_scores_match_a_matmul_of_dequantized_keys(depth_kind):
    rng = np.random.default_rng(4)
    n, d, G, group = 700, 128, 3, 128
    x = (rng.standard_normal((n, d)) * 10.0 ** rng.uniform(-1, 1, d)).astype(np.float32)
    q = rng.standard_normal((G, d)).astype(np.float32)
    s16, z16, codes = oracle.quantize_grouped(x, group)
    depth = (np.full(d, 4, np.uint8) if depth_kind == "full"
             else rng.integers(0, 5, d).astype(np.uint8))
    got = oracle.scores_grouped(codes, s16, z16, depth, q, group)
    gi = np.arange(n) // group
    sf = s16.view(np.float16).astype(np.float64)[:, gi].T
    zf = z16.view(np.float16).astype(np.float64)[:, gi].T
    # bin midpoint of the t-plane prefix: p 2^(4-t) + (2^(4-t) - 1) / 2
    w = (1 << (4 - depth.astype(np.int64)))[None, :]
    mid = (codes.astype(np.int64) // w) * w + (w - 1) / 2.0
    want = q.astype(np.float64) @ (zf + sf * mid).T
    assert np.allclose(got, want, rtol=1e-12, atol=1e-9 * np.abs(want).max())
