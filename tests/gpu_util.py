"""Helpers for the GPU parity tests (inputs, store construction, tolerance checks)."""
import numpy as np
import pytest

from bit_plane_kv_amd import fathom as F
from bit_plane_kv_amd import synth

SCORE_REL_TOL = 1e-5     # per query row: max |diff| <= 1e-5 * max |oracle score|
ATTN_ABS_TOL = 2e-2      # bf16 attention outputs


def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    return torch


def to_dev(a):
    torch = torch_cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def store_from_keys(keys_np, word_stride=None, planes=None):
    """Build a store on the GPU from fp32 keys [H][n][d] with fathom_quantize_store."""
    torch = torch_cuda()
    H, n, _ = keys_np.shape
    st = F.Store.empty(H, n, "cuda", word_stride=word_stride, planes=planes)
    st.planes.fill_(0x5A5A5A5A)   # the build must overwrite every word, tail included
    keys = to_dev(keys_np)
    F.fathom_quantize_store(keys, st)
    torch.cuda.synchronize()
    return st, keys


def u32(t):
    return t.cpu().numpy().view(np.uint32)


def check_rows(got, ref, rel=SCORE_REL_TOL):
    """got, ref [..., n]: per row max|got - ref| <= rel * max|ref|."""
    got = np.asarray(got, np.float64).reshape(-1, got.shape[-1])
    ref = np.asarray(ref, np.float64).reshape(-1, ref.shape[-1])
    err = np.abs(got - ref).max(axis=1)
    scale = np.maximum(np.abs(ref).max(axis=1), np.finfo(np.float32).tiny)
    worst = float((err / scale).max())
    assert worst <= rel, f"score rel error {worst:.3e} > {rel}"
    return worst


def bf16_to_f32(t):
    return t.float().cpu().numpy()


def topk_gate2(gpu_idx, ref_scores, k, tol_abs):
    """End-to-end set check: equal sets, or every index in the symmetric difference has
    an oracle score within 2*tol of the oracle's k-th score.  Returns the count."""
    gi = np.asarray(gpu_idx).reshape(-1, k)
    rs = np.asarray(ref_scores, np.float64).reshape(gi.shape[0], -1)
    flips = 0
    for r in range(gi.shape[0]):
        order = np.lexsort((np.arange(rs.shape[1]), -rs[r]))
        ref_set = set(order[:k].tolist())
        kth = rs[r, order[k - 1]]
        diff = ref_set.symmetric_difference(gi[r].tolist())
        for i in diff:
            assert abs(rs[r, i] - kth) <= 2 * tol_abs[r], (r, i, rs[r, i], kth)
        flips += len(diff)
    return flips


def inputs(cfg_id, H, G, n, seed=0, d=128):
    keys = synth.keys_np(seed, cfg_id, range(H), n, d)
    q = synth.queries_np(seed, cfg_id, range(H), G, d)
    V = synth.values_np(seed, cfg_id, range(H), n, d)
    K = synth.bf16_bits(keys)
    return keys, q, K, V
