"""Pins for the oracle's top-k and exact sparse attention, and the bf16 conversions.

Independent checks: numpy lexsort (full sort), order properties, numpy dense softmax
attention on the dequantized keys at k = n, k = 1, equal logits, and torch's CPU bf16
rounding.
"""
import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import oracle
from bit_plane_kv_amd import synth


def _lexsort_topk(s, k):
    s = np.where(s == 0, np.float32(0), s)          # -0 ranks as +0
    order = np.lexsort((np.arange(s.size), -s.astype(np.float64)))
    return np.sort(order[:k])


@settings(max_examples=40, deadline=None)
@given(seed=st.integers(0, 2**31 - 1), n=st.integers(1, 3000), frac=st.floats(0, 1),
       levels=st.sampled_from([0, 2, 7, 1000]))
def test_topk_equals_full_sort(seed, n, frac, levels):
    rng = np.random.default_rng(seed)
    s = rng.standard_normal(n).astype(np.float32)
    if levels:                                      # many exact ties
        s = np.round(s * levels).astype(np.float32)
    k = max(1, min(n, int(round(frac * n))))
    got = oracle.topk(s, k)
    assert (got == _lexsort_topk(s, k)).all()
    assert (np.diff(got) > 0).all()
    sel = np.zeros(n, bool)
    sel[got] = True
    if k < n:
        assert s[sel].min() >= s[~sel].max()
        thr = s[sel].min()
        # among entries equal to the threshold, the selected ones have lower indices
        eq_sel = np.nonzero(sel & (s == thr))[0]
        eq_rest = np.nonzero(~sel & (s == thr))[0]
        if eq_sel.size and eq_rest.size:
            assert eq_sel.max() < eq_rest.min()


def test_topk_signed_zero_and_extremes():
    s = np.array([-0.0, 0.0, -1.0, 3.4e38, -3.4e38, 0.0, -0.0], np.float32)
    assert oracle.topk(s, 1).tolist() == [3]
    assert oracle.topk(s, 3).tolist() == [0, 1, 3]       # -0 ties with +0, lower index
    assert oracle.topk(s, 7).tolist() == list(range(7))
    with pytest.raises(ValueError):
        oracle.topk(s, 0)
    with pytest.raises(ValueError):
        oracle.topk(s, 8)


def test_bf16_conversion_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32) * 100,
                        # exact halfway cases, both parities
                        np.array([1 + 2**-8, 1 + 3 * 2**-8, -(1 + 2**-8), 65504.0],
                                 np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (oracle.f32_to_bf16(x) == ref).all()
    assert (synth.bf16_bits(x) == ref).all()
    back = torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert (oracle.bf16_to_f32(ref) == back).all()


def _dense_attention(q, Kf, Vf, sm_scale):
    l = (Kf.astype(np.float64) @ q.astype(np.float64)) * sm_scale
    p = np.exp(l - l.max())
    p /= p.sum()
    return p @ Vf.astype(np.float64)


def test_k_equals_n_is_dense_attention_on_dequantized_keys():
    n, d = 512, 128
    x = synth.keys_np(0, 5, [0], n, d)[0]
    s, z, codes = oracle.quantize(x)
    deq = oracle.dequantize(codes, s, z).astype(np.float32)
    K = oracle.f32_to_bf16(deq)
    V = synth.values_np(0, 5, [0], n, d)[0]
    q = synth.queries_np(0, 5, [0], 2, d)[0] * np.float32(0.05)
    sm = float(np.float32(1 / np.sqrt(d)))
    idx = np.tile(np.arange(n, dtype=np.int32), (1, 2, 1))
    got = oracle.attention(q[None], K[None], V[None], idx, sm)[0]
    Kf, Vf = oracle.bf16_to_f32(K), oracle.bf16_to_f32(V)
    for g in range(2):
        ref = _dense_attention(q[g], Kf, Vf, sm)
        assert np.allclose(got[g], ref, rtol=1e-10, atol=1e-12)


def test_k_one_returns_the_winner_row():
    n, d = 64, 128
    K = synth.values_np(1, 5, [0], n, d)
    V = synth.values_np(2, 5, [0], n, d)
    q = synth.queries_np(0, 5, [0], 1, d)
    idx = np.array([[[37]]], np.int32)
    out = oracle.attention(q, K, V, idx, 0.1)
    assert (out[0, 0] == oracle.bf16_to_f32(V[0, 37]).astype(np.float64)).all()


def test_equal_logits_average_the_values():
    n, d = 100, 128
    K = synth.values_np(1, 6, [0], n, d)
    V = synth.values_np(2, 6, [0], n, d)
    q = np.zeros((1, 1, d), np.float32)
    idx = np.array([[[3, 10, 11, 50, 99]]], np.int32)
    out = oracle.attention(q, K, V, idx, 0.3)
    ref = oracle.bf16_to_f32(V[0, idx[0, 0]]).astype(np.float64).mean(axis=0)
    assert np.allclose(out[0, 0], ref, rtol=1e-14, atol=1e-15)


def test_attention_ignores_index_order():
    n, d = 300, 128
    K = synth.values_np(3, 6, [0], n, d)
    V = synth.values_np(4, 6, [0], n, d)
    q = synth.queries_np(5, 6, [0], 1, d) * np.float32(0.2)
    idx = np.random.default_rng(0).choice(n, 40, replace=False).astype(np.int32)
    a = oracle.attention(q, K, V, np.sort(idx)[None, None], 0.09)
    b = oracle.attention(q, K, V, idx[None, None], 0.09)
    assert np.allclose(a, b, rtol=1e-13, atol=1e-15)


def _lexsort_topk64(s, k):
    s = np.where(s == 0, 0.0, s)
    order = np.lexsort((np.arange(s.size), -s))
    return np.sort(order[:k])


@settings(max_examples=30, deadline=None)
@given(seed=st.integers(0, 2**31 - 1), n=st.integers(1, 2000), frac=st.floats(0, 1),
       levels=st.sampled_from([0, 3, 50]))
def test_topk_f64_equals_full_sort(seed, n, frac, levels):
    rng = np.random.default_rng(seed)
    s = rng.standard_normal(n)
    if levels:
        s = np.round(s * levels)
    # values that differ below fp32 resolution must still be told apart
    s = s + rng.integers(0, 3, n) * 1e-12
    k = max(1, min(n, int(round(frac * n))))
    assert (oracle.topk_f64(s, k) == _lexsort_topk64(s, k)).all()


def test_topk_f64_signed_zero_and_fine_differences():
    s = np.array([-0.0, 0.0, 1.0, 1.0 + 1e-15, 1.0, -1e-300], np.float64)
    assert oracle.topk_f64(s, 1).tolist() == [3]
    assert oracle.topk_f64(s, 3).tolist() == [2, 3, 4]
    assert oracle.topk_f64(s, 4).tolist() == [0, 2, 3, 4]     # -0 ties +0: lower index


def test_logits_equal_a_library_matmul():
    n, d, G = 777, 128, 3
    K = synth.values_np(8, 6, [0, 1], n, d)
    q = synth.queries_np(9, 6, [0, 1], G, d)
    sm = 0.0883883461356163
    got = oracle.logits(q, K, sm)
    Kf = oracle.bf16_to_f32(K).astype(np.float64)
    for h in range(2):
        ref = (q[h].astype(np.float64) @ Kf[h].T) * sm
        assert np.allclose(got[h], ref, rtol=1e-13, atol=1e-13 * np.abs(ref).max())
    # the attention over every row is the softmax of these logits applied to V
    V = synth.values_np(10, 6, [0, 1], n, d)
    idx = np.tile(np.arange(n, dtype=np.int32), (2, G, 1))
    att = oracle.attention(q, K, V, idx, sm)
    p = np.exp(got - got.max(axis=-1, keepdims=True))
    p /= p.sum(axis=-1, keepdims=True)
    ref = np.einsum("hgn,hnd->hgd", p, oracle.bf16_to_f32(V).astype(np.float64))
    assert np.allclose(att, ref, rtol=1e-10, atol=1e-12)
