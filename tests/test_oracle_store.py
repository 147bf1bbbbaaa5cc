"""Pins for the oracle's store build: quantize, bit-plane packing, prefix, variance.

Each test checks the oracle against something other than itself: the pages' worked
example (blog, "Bit planes: how a partial read becomes a valid read"), numpy's
packbits / var, nearest-level brute force, or closed forms.
"""
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from bit_plane_kv_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "plane_diagram.txt")


def _golden():
    rows = {}
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, *vals = line.split()
        rows[key] = vals
    return rows


def test_plane_diagram_worked_example():
    g = _golden()
    codes = np.array([int(b, 2) for b in g["codes"]], np.uint8)       # 11, 6, 13, 2
    planes = oracle.pack_planes(codes[:, None])                        # d = 1
    assert planes.shape == (1, 4, 1)
    for j in range(4):
        bits = g[f"plane{j}"][0]
        # token t of the diagram sits at bit t of the word (low bit = lowest token)
        expect = sum(int(ch) << t for t, ch in enumerate(bits))
        assert int(planes[0, j, 0]) == expect
    # LSB-first words for tokens 0..3
    assert [int(planes[0, j, 0]) for j in range(4)] == [0x5, 0x6, 0xB, 0x5]
    # reading planes 0 and 1 gives the 2-bit version of every number
    assert [oracle.plane_prefix(planes, 0, 2, i) for i in range(4)] == [2, 1, 3, 0]
    # its bin midpoints on the 4-bit scale
    assert [oracle.midpoint_level(int(c), 2) for c in codes] == [9.5, 5.5, 13.5, 1.5]


def test_quantize_reproduces_diagram_codes():
    # range 0..15 gives scale 1 and zero 0, so each value is its own code
    x = np.array([11, 6, 13, 2, 0, 15], np.float32)[:, None]
    s, z, codes = oracle.quantize(x)
    assert s[0] == 1.0 and z[0] == 0.0
    assert codes[:, 0].tolist() == [11, 6, 13, 2, 0, 15]


def _keys(n, d=8, seed=0):
    return synth.keys_np(seed, 99, [0], n, d)[0]


def test_quantize_is_nearest_level():
    x = _keys(5000, 16)
    s, z, codes = oracle.quantize(x)
    assert codes.max() <= 15
    lv = (x.astype(np.float64) - z.astype(np.float64)) / s.astype(np.float64)
    err = np.abs(lv - codes)
    # nearest of the 16 levels z + s*code, up to fp32 rounding of (x - z)/s
    assert err.max() <= 0.5 + 1e-5
    # the extremes map to the end codes
    assert (codes[np.argmin(x, axis=0), np.arange(16)] == 0).all()
    assert (codes[np.argmax(x, axis=0), np.arange(16)] == 15).all()
    # a brute-force nearest level agrees wherever the decision is not a near-tie
    levels = np.arange(16)
    brute = np.argmin(np.abs(lv[..., None] - levels), axis=-1)
    clear = np.abs(np.abs(lv - np.floor(lv)) - 0.5) > 1e-4
    assert (brute[clear] == codes[clear]).all()


def test_constant_channel_gets_code_zero():
    x = np.ones((100, 3), np.float32) * np.array([2.5, -1.0, 0.0], np.float32)
    s, z, codes = oracle.quantize(x)
    assert (s == 0).all() and (codes == 0).all()
    assert z.tolist() == [2.5, -1.0, 0.0]
    assert (oracle.channel_var(codes, s) == 0).all()


def test_packing_matches_numpy_packbits():
    for n in (1, 31, 32, 33, 100, 257):
        rng = np.random.default_rng(n)
        codes = rng.integers(0, 16, (n, 5), dtype=np.uint8)
        planes = oracle.pack_planes(codes)
        W = (n + 31) // 32
        for c in range(5):
            for j in range(4):
                bits = ((codes[:, c] >> (3 - j)) & 1).astype(np.uint8)
                bits = np.concatenate([bits, np.zeros(32 * W - n, np.uint8)])
                words = np.packbits(bits, bitorder="little").view("<u4")
                assert (planes[c, j] == words).all(), (n, c, j)


@settings(max_examples=25, deadline=None)
@given(n=st.integers(1, 300), seed=st.integers(0, 2**31 - 1))
def test_prefix_equals_t_bit_quantizer(n, seed):
    """A t-plane prefix equals the t-bit quantizer of the same value with the same
    scale (blog, "Bit planes"): floor(level / 2^(4-t)), level = the 4-bit rounding."""
    x = _keys(n, 4, seed)
    s, z, codes = oracle.quantize(x)
    planes = oracle.pack_planes(codes)
    f32 = np.float32
    for c in range(4):
        if s[c] == 0:
            continue
        level = np.floor((x[:, c] - z[c]).astype(f32) / s[c] + f32(0.5)).astype(np.int64)
        for t in range(1, 5):
            q_t = np.minimum(level // (1 << (4 - t)), (1 << t) - 1)
            q_t = np.maximum(q_t, 0)
            got = [oracle.plane_prefix(planes, c, t, i) for i in range(n)]
            assert got == q_t.tolist(), (c, t)
        # four planes give the code back
        assert [oracle.plane_prefix(planes, c, 4, i) for i in range(n)] == \
            codes[:, c].tolist()


def test_padding_bits_are_zero():
    n = 70
    codes = np.full((n, 2), 15, np.uint8)
    planes = oracle.pack_planes(codes)
    assert planes.shape[-1] == 3
    assert (planes[:, :, 2] == (1 << (n - 64)) - 1).all()
    assert (planes[:, :, :2] == 0xFFFFFFFF).all()


def test_var_matches_numpy_of_dequantized():
    x = _keys(3000, 32, seed=5)
    s, z, codes = oracle.quantize(x)
    var = oracle.channel_var(codes, s)
    deq = z[None, :].astype(np.float64) + s[None, :].astype(np.float64) * codes
    ref = np.var(deq, axis=0)            # two-pass population variance
    assert np.allclose(var, ref, rtol=1e-6, atol=0)


def test_var_two_level_closed_form():
    n = 1000
    codes = np.zeros((n, 1), np.uint8)
    codes[::2] = 15
    s = np.array([0.25], np.float32)
    # half the codes 0 and half 15: variance of the levels is 7.5^2
    assert oracle.channel_var(codes, s)[0] == np.float32(0.25 * 0.25 * 56.25)


def test_batched_quantize_equals_per_head():
    x = synth.keys_np(3, 0, [0, 1, 2], 200, 8)
    s, z, codes = oracle.quantize(x)
    for h in range(3):
        s1, z1, c1 = oracle.quantize(x[h])
        assert (s1 == s[h]).all() and (z1 == z[h]).all() and (c1 == codes[h]).all()


@settings(max_examples=15, deadline=None)
@given(n=st.integers(1, 200), seed=st.integers(0, 2**31 - 1))
def test_nibbles_hold_the_four_plane_prefix(n, seed):
    """The ordinary token-major layout (blog, "Where this does not work": the plain 4-bit
    scan reads each number whole) holds, for every token and channel, the same number the
    bit planes give when all four are read: checked against the plane packing and its
    prefix, which the pages' diagram pins."""
    d = 6
    x = _keys(n, d, seed)
    _, _, codes = oracle.quantize(x)
    nib = oracle.pack_nibbles(codes)
    planes = oracle.pack_planes(codes)
    assert nib.shape == (n, d // 2) and nib.dtype == np.uint8
    for i in range(n):
        for c in range(d):
            byte = int(nib[i, c // 2])
            number = (byte >> 4) if c % 2 else (byte & 15)
            assert number == oracle.plane_prefix(planes, c, 4, i), (i, c)


def test_nibble_store_is_64_bytes_per_token_at_d128():
    codes = np.zeros((3, 128), np.uint8)
    assert oracle.pack_nibbles(codes).nbytes == 3 * 64
