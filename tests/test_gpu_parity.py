"""Parity of the HIP path (through the C-ABI) with the CPU oracle.

Bars: bit-exact on plane packing, plans and top-k index sets; per query row
max|diff| <= 1e-5 * max|oracle| on fp32 scores; |diff| <= 2e-2 on bf16 attention.
Shapes span several tiles and ragged tails; edge cases cover n = 1, B = 0 and 4d,
k = 1 and k = n, heavy ties, and the multi-level top-k path.
"""
import numpy as np
import pytest

import oracle
from bit_plane_kv_amd import fathom as F
from bit_plane_kv_amd import synth

from gpu_util import (ATTN_ABS_TOL, SCORE_REL_TOL, bf16_to_f32, check_rows, inputs,
                      store_from_keys, to_dev, topk_gate2, torch_cuda, u32)

pytestmark = pytest.mark.gpu


# ---------------------------------------------------------------------------------
# store build
# ---------------------------------------------------------------------------------
@pytest.mark.parametrize("H,n,extra", [(1, 4096, 0), (3, 1013, 0), (2, 33, 0), (1, 1, 0),
                                       (2, 5000, 4), (1, 70, 8), (4, 2048, 0),
                                       (2, 64 * 9 + 7, 4)])
def test_quantize_store_matches_oracle(H, n, extra):
    print(f"[quantize] H={H} n={n} extra={extra}", flush=True)
    keys = synth.keys_np(1, 50, range(H), n)
    W = (n + 31) // 32
    st, _ = store_from_keys(keys, word_stride=(W + 3) // 4 * 4 + extra)
    s, z, codes = oracle.quantize(keys)
    ref_planes = oracle.pack_planes(codes)
    got = u32(st.planes)
    assert np.array_equal(got[..., :W], ref_planes)
    assert (got[..., W:] == 0).all()
    assert np.array_equal(st.scale.cpu().numpy(), s)
    assert np.array_equal(st.zero.cpu().numpy(), z)
    assert np.array_equal(st.var.cpu().numpy(), oracle.channel_var(codes, s))


def test_quantize_constant_channels():
    keys = synth.keys_np(2, 51, range(2), 300)
    keys[0, :, 5] = 1.25
    keys[1, :, 0] = 0.0
    st, _ = store_from_keys(keys)
    s, z, codes = oracle.quantize(keys)
    ref = oracle.pack_planes(codes)
    got = u32(st.planes)
    assert np.array_equal(got[..., :ref.shape[-1]], ref)
    assert (got[..., ref.shape[-1]:] == 0).all()
    assert st.scale.cpu().numpy()[0, 5] == 0 and st.var.cpu().numpy()[0, 5] == 0


# ---------------------------------------------------------------------------------
# plan
# ---------------------------------------------------------------------------------
def _plan_inputs(G, H=12, seed=3):
    rng = np.random.default_rng(seed + G)
    q = rng.standard_normal((H, G, 128)).astype(np.float32)
    var = (10 ** rng.uniform(-2, 2, (H, 128))).astype(np.float32)
    # heavy ties: equal queries and a few importances, some exactly 4x apart
    q[H // 2:] = 1.0
    var[H // 2:] = rng.choice(np.array([0, 0.25, 1, 4, 16], np.float32), (H - H // 2, 128))
    return q, var


@pytest.mark.parametrize("G", [1, 2, 4, 8])
@pytest.mark.parametrize("B", [0, 1, 7, 68, 92, 136, 300, 511, 512])
def test_plan_matches_oracle(G, B):
    torch = torch_cuda()
    q, var = _plan_inputs(G)
    st = F.Store.empty(q.shape[0], 64, "cuda")
    st.var.copy_(to_dev(var))
    depth = F.fathom_plan(st, to_dev(q), B)
    torch.cuda.synchronize()
    ref = oracle.plan(q, var, B)
    assert np.array_equal(depth.cpu().numpy(), ref)
    assert (depth.cpu().numpy().astype(int).sum(axis=1) == B).all()


@pytest.mark.parametrize("value", [0.0, 3.0])
@pytest.mark.parametrize("B", [0, 1, 92, 127, 128, 129, 136, 384, 511, 512])
def test_plan_all_channels_equal(value, B):
    """Every channel of equal importance: ties everywhere, including the case where
    every channel outranks an item.  Equal nonzero w, B = 136: depth 2 on channels
    0-7 and 1 on the rest; w = 0: every key is 0, so items go by (c, t) and whole
    channels fill in index order."""
    torch = torch_cuda()
    H, G = 3, 4
    q = np.ones((H, G, 128), np.float32)
    var = np.full((H, 128), value, np.float32)
    st = F.Store.empty(H, 64, "cuda")
    st.var.copy_(to_dev(var))
    depth = F.fathom_plan(st, to_dev(q), B).cpu().numpy()
    ref = oracle.plan(q, var, B)
    assert np.array_equal(depth, ref)
    if B == 136 and value > 0:
        assert (ref[:, :8] == 2).all() and (ref[:, 8:] == 1).all()
    if value == 0:
        assert (ref[:, :B // 4] == 4).all() and (ref[:, B // 4 + 1:] == 0).all()


@pytest.mark.parametrize("nc", [0, 1, 34, 128])
def test_plan_fixed_matches_oracle(nc):
    torch = torch_cuda()
    _, var = _plan_inputs(1)
    st = F.Store.empty(var.shape[0], 64, "cuda")
    st.var.copy_(to_dev(var))
    depth = F.fathom_plan_fixed(st, nc)
    torch.cuda.synchronize()
    assert np.array_equal(depth.cpu().numpy(), oracle.plan_fixed(var, nc))


# ---------------------------------------------------------------------------------
# scan
# ---------------------------------------------------------------------------------
def _depths(kind, st, q_t, var, q, rng):
    H = q.shape[0]
    if kind == "plan92":
        d = F.fathom_plan(st, q_t, 92).cpu().numpy()
        assert np.array_equal(d, oracle.plan(q, var, 92))
        return d
    if kind == "b0":
        return np.zeros((H, 128), np.uint8)
    if kind == "b512":
        return np.full((H, 128), 4, np.uint8)
    if kind == "fixed136":
        return oracle.plan_fixed(var, 34)
    return rng.integers(0, 5, (H, 128)).astype(np.uint8)


@pytest.mark.parametrize("H,G,n", [(3, 4, 5000), (2, 1, 4096), (2, 8, 777), (1, 3, 33),
                                   (1, 2, 12345), (1, 4, 1), (2, 5, 4160), (1, 4, 9000)])
@pytest.mark.parametrize("kind", ["plan92", "b0", "b512", "random", "fixed136"])
def test_scan_matches_oracle(H, G, n, kind):
    torch = torch_cuda()
    print(f"[scan] H={H} G={G} n={n} {kind}", flush=True)
    keys, q, _, _ = inputs(60, H, G, n)
    st, _ = store_from_keys(keys)
    s, z, codes = oracle.quantize(keys)
    var = oracle.channel_var(codes, s)
    q_t = to_dev(q)
    depth = _depths(kind, st, q_t, var, q, np.random.default_rng(n))
    scores = F.fathom_scan(st, q_t, to_dev(depth))
    torch.cuda.synchronize()
    ref = oracle.scores(codes, s, z, depth, q)
    check_rows(scores.cpu().numpy(), ref)


@pytest.mark.parametrize("kind", ["plan92", "random"])
def test_scan_long_runs_sampled_heads(kind):
    """72 heads x 32768 tokens: the scan's workgroups take runs of several 256-token
    steps that straddle head boundaries (with different plane counts per head under
    random depths); sampled heads, boundary neighbours included, against the oracle."""
    torch = torch_cuda()
    H, G, n = 72, 4, 32768
    print(f"[scan-long] H={H} G={G} n={n} {kind}", flush=True)
    keys = synth.keys_torch(0, 70, range(H), n, "cuda")
    st = F.Store.empty(H, n, "cuda")
    F.fathom_quantize_store(keys, st)
    del keys
    q = synth.queries_np(0, 70, range(H), G)
    q_t = to_dev(q)
    if kind == "plan92":
        depth_t = F.fathom_plan(st, q_t, 92)
    else:
        depth_t = to_dev(np.random.default_rng(7).integers(0, 5, (H, 128)).astype(np.uint8))
    scores = F.fathom_scan(st, q_t, depth_t)
    torch.cuda.synchronize()
    depth = depth_t.cpu().numpy()
    for h in [0, 1, 35, 36, 70, 71]:
        kh = synth.keys_torch(0, 70, [h], n, "cuda")[0].cpu().numpy()
        s, z, codes = oracle.quantize(kh[None])
        if kind == "plan92":
            assert np.array_equal(depth[h], oracle.plan(q[h][None], oracle.channel_var(codes, s), 92)[0])
        ref = oracle.scores(codes, s, z, depth[h][None], q[h][None])
        check_rows(scores[h].cpu().numpy(), ref[0])


@pytest.mark.parametrize("H,n", [(600, 100), (37, 300)])
def test_scan_many_small_heads(H, n):
    """Heads shorter than one workgroup's run: runs are cut at head boundaries."""
    torch = torch_cuda()
    keys, q, _, _ = inputs(71, H, 4, n)
    st, _ = store_from_keys(keys)
    s, z, codes = oracle.quantize(keys)
    depth = np.random.default_rng(H).integers(0, 5, (H, 128)).astype(np.uint8)
    scores = F.fathom_scan(st, to_dev(q), to_dev(depth))
    torch.cuda.synchronize()
    check_rows(scores.cpu().numpy(), oracle.scores(codes, s, z, depth, q))


@pytest.mark.parametrize("H,G,n", [(2, 4, 5000), (1, 1, 4096), (2, 8, 777), (1, 3, 33)])
@pytest.mark.parametrize("kind", ["plan92", "b512", "random", "b0"])
def test_scan_extract_matches_oracle(H, G, n, kind):
    """The per-bit-extraction comparator gives the same scores to the same tolerance."""
    torch = torch_cuda()
    print(f"[scan-extract] H={H} G={G} n={n} {kind}", flush=True)
    keys, q, _, _ = inputs(62, H, G, n)
    st, _ = store_from_keys(keys)
    s, z, codes = oracle.quantize(keys)
    var = oracle.channel_var(codes, s)
    q_t = to_dev(q)
    depth = _depths(kind, st, q_t, var, q, np.random.default_rng(n + 1))
    got = F.fathom_scan_extract(st, q_t, to_dev(depth))
    torch.cuda.synchronize()
    check_rows(got.cpu().numpy(), oracle.scores(codes, s, z, depth, q))


def test_scan_prepared_equals_scan():
    torch = torch_cuda()
    keys, q, _, _ = inputs(61, 2, 4, 6000)
    st, _ = store_from_keys(keys)
    q_t = to_dev(q)
    depth = F.fathom_plan(st, q_t, 92)
    a = F.fathom_scan(st, q_t, depth)
    ws = F.scan_workspace(st, 4, "cuda")
    F.fathom_scan_prepare(st, q_t, depth, ws)
    b = torch.empty_like(a)
    F.fathom_scan_prepared(st, 4, b, ws)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# ---------------------------------------------------------------------------------
# top-k
# ---------------------------------------------------------------------------------
def _rows(R, n, dist, seed):
    rng = np.random.default_rng(seed)
    s = rng.standard_normal((R, n)).astype(np.float32)
    if dist == "ties":
        s = np.round(s * 4).astype(np.float32)
        s[:, ::7] = -0.0
    elif dist == "equal":
        s[:] = 3.5
    elif dist == "sorted":
        s = np.sort(s, axis=1)
    return s


@pytest.mark.parametrize("R,n,k", [(3, 1, 1), (4, 100, 7), (2, 4097, 512), (2, 32768, 512),
                                   (1, 32768, 32768), (2, 32769, 512), (2, 100000, 1000),
                                   (1, 1 << 20, 512), (1, 70000, 16384), (3, 5000, 5000),
                                   (2, 65536, 1)])
@pytest.mark.parametrize("dist", ["normal", "ties", "equal", "sorted"])
def test_topk_matches_oracle(R, n, k, dist):
    torch = torch_cuda()
    print(f"[topk] R={R} n={n} k={k} {dist}", flush=True)
    s = _rows(R, n, dist, n + k)
    idx = F.fathom_topk(to_dev(s), k)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), oracle.topk(s, k))


# ---------------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------------
@pytest.mark.parametrize("H,G,n,k", [(2, 4, 3000, 512), (1, 1, 4096, 64), (2, 3, 100, 100),
                                     (1, 2, 50, 1), (3, 8, 2000, 77),
                                     (1, 2, 3000, 1300),   # several rounds of 512 rows a slot set
                                     (70, 4, 600, 300)])   # more than 256 rows: 256-thread groups
def test_sparse_attn_matches_oracle(H, G, n, k):
    torch = torch_cuda()
    keys, q, K, V = inputs(70, H, G, n)
    rng = np.random.default_rng(k)
    idx = np.sort(np.stack([np.stack([rng.choice(n, k, replace=False) for _ in range(G)])
                            for _ in range(H)]), axis=-1).astype(np.int32)
    sm = float(np.float32(1 / np.sqrt(128)))
    out = F.fathom_sparse_attn(to_dev(q), to_dev(K).view(torch.bfloat16),
                               to_dev(V).view(torch.bfloat16), to_dev(idx), sm)
    torch.cuda.synchronize()
    ref = oracle.attention(q, K, V, idx, sm)
    err = np.abs(bf16_to_f32(out) - ref).max()
    assert err <= ATTN_ABS_TOL, err


def test_sparse_attn_k_equals_n_is_dense():
    torch = torch_cuda()
    n = 1000
    keys, q, _, V = inputs(71, 1, 2, n)
    s, z, codes = oracle.quantize(keys)
    K = oracle.f32_to_bf16(oracle.dequantize(codes[0], s[0], z[0]).astype(np.float32))[None]
    idx = np.tile(np.arange(n, dtype=np.int32), (1, 2, 1))
    sm = float(np.float32(1 / np.sqrt(128)))
    out = F.fathom_sparse_attn(to_dev(q), to_dev(K).view(torch.bfloat16),
                               to_dev(V).view(torch.bfloat16), to_dev(idx), sm)
    torch.cuda.synchronize()
    Kf = oracle.bf16_to_f32(K[0]).astype(np.float64)
    Vf = oracle.bf16_to_f32(V[0]).astype(np.float64)
    for g in range(2):
        l = Kf @ q[0, g].astype(np.float64) * sm
        p = np.exp(l - l.max())
        dense = (p / p.sum()) @ Vf
        assert np.abs(bf16_to_f32(out)[0, g] - dense).max() <= ATTN_ABS_TOL


# ---------------------------------------------------------------------------------
# the whole step
# ---------------------------------------------------------------------------------
def _step_parity(cfg_id, H, G, n, B, k, seed=0):
    torch = torch_cuda()
    keys, q, K, V = inputs(cfg_id, H, G, n, seed)
    st, _ = store_from_keys(keys)
    depth = torch.empty((H, 128), dtype=torch.uint8, device="cuda")
    scores = torch.empty((H, G, n), dtype=torch.float32, device="cuda")
    idx = torch.empty((H, G, k), dtype=torch.int32, device="cuda")
    sm = float(np.float32(1 / np.sqrt(128)))
    out = F.fathom_step(st, to_dev(q), to_dev(K).view(torch.bfloat16),
                        to_dev(V).view(torch.bfloat16), B, k, sm, depth_out=depth,
                        scores_out=scores, idx_out=idx)
    torch.cuda.synchronize()
    s, z, codes = oracle.quantize(keys)
    var = oracle.channel_var(codes, s)
    ref_depth = oracle.plan(q, var, B)
    assert np.array_equal(depth.cpu().numpy(), ref_depth)
    ref_scores = oracle.scores(codes, s, z, ref_depth, q)
    got_scores = scores.cpu().numpy()
    check_rows(got_scores, ref_scores)
    got_idx = idx.cpu().numpy()
    # gate 1: the GPU top-k of the GPU's own scores is exact
    assert np.array_equal(got_idx.reshape(H * G, k),
                          oracle.topk(got_scores.reshape(H * G, n), k))
    # gate 2: end to end against the oracle's fp64 scores
    tol = SCORE_REL_TOL * np.abs(ref_scores.reshape(H * G, n)).max(axis=1)
    flips = topk_gate2(got_idx, ref_scores, k, tol)
    ref_out = oracle.attention(q, K, V, got_idx, sm)
    assert np.abs(bf16_to_f32(out) - ref_out).max() <= ATTN_ABS_TOL
    return flips


@pytest.mark.parametrize("B", [68, 92, 136, 512])
def test_step_tiny(B):
    cfg = synth.CONFIGS["tiny"]
    print(f"[step] tiny B={B}", flush=True)
    _step_parity(cfg.cfg_id, cfg.H, cfg.G, cfg.n, B, cfg.k)


def test_step_multihead_ragged():
    print("[step] H=6 G=4 n=9000 B=92 k=256", flush=True)
    _step_parity(80, 6, 4, 9000, 92, 256)


def test_step_long_rows_multilevel_topk():
    print("[step] H=1 G=2 n=40000 B=92 k=512", flush=True)
    _step_parity(81, 1, 2, 40000, 92, 512)


# ---------------------------------------------------------------------------------
# host residency: same kernels, planes / K / V in pinned host memory
# ---------------------------------------------------------------------------------
def test_host_resident_store_and_rows_match_hbm():
    torch = torch_cuda()
    H, G, n, k = 2, 4, 5000, 128
    keys, q, K, V = inputs(90, H, G, n)
    st_d, _ = store_from_keys(keys)
    W = ((n + 31) // 32 + 3) // 4 * 4
    pinned = torch.empty((H, 128, 4, W), dtype=torch.int32, pin_memory=True)
    st_h, _ = store_from_keys(keys, planes=pinned)
    assert torch.equal(st_d.planes.cpu(), st_h.planes.cpu())
    q_t = to_dev(q)
    depth = F.fathom_plan(st_d, q_t, 92)
    a = F.fathom_scan(st_d, q_t, depth)
    b = F.fathom_scan(st_h, q_t, depth)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    idx = F.fathom_topk(a, k)
    Kd = to_dev(K).view(torch.bfloat16)
    Vd = to_dev(V).view(torch.bfloat16)
    Kh = torch.from_numpy(K).view(torch.bfloat16).pin_memory()
    Vh = torch.from_numpy(V).view(torch.bfloat16).pin_memory()
    sm = float(np.float32(1 / np.sqrt(128)))
    o1 = F.fathom_sparse_attn(q_t, Kd, Vd, idx, sm)
    o2 = F.fathom_sparse_attn(q_t, Kh, Vh, idx, sm)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_pageable_host_pointer_is_rejected():
    torch = torch_cuda()
    H, n = 1, 256
    keys = synth.keys_np(0, 91, range(H), n)
    st, _ = store_from_keys(keys)
    pageable = torch.empty((H, 128, 4, 8), dtype=torch.int32)   # not pinned
    bad = F.Store(pageable, st.scale, st.zero, st.var, n)
    q = to_dev(synth.queries_np(0, 91, range(H), 1))
    depth = F.fathom_plan(st, q, 16)
    with pytest.raises(F.FathomError) as e:
        F.fathom_scan(bad, q, depth)
    assert e.value.status == F.ERR_NOT_MAPPED


def test_stream_read_runs_stays_in_its_allocation():
    """The run-length measurement read: runs inside a 1 MiB pinned buffer run; a last
    run past its end is refused on the host (nothing is launched)."""
    import ctypes
    torch = torch_cuda()
    L = F.lib()
    p = ctypes.c_void_p()
    assert L.fathom_host_alloc(1 << 20, 0, ctypes.byref(p)) == F.OK
    try:
        sink = torch.zeros(2, dtype=torch.int64, device="cuda")
        sp = ctypes.c_void_p(sink.data_ptr())
        assert L.fathom_stream_read_runs(p, 4096, 8192, 128, sp, None) == F.OK   # ends at 1 MiB - 4 KiB
        assert L.fathom_stream_read_runs(p, 8192, 8192, 128, sp, None) == F.OK   # ends at 1 MiB
        torch.cuda.synchronize()
        assert L.fathom_stream_read_runs(p, 4096, 8192, 129, sp, None) == F.ERR_INVALID_ARG
        off = ctypes.c_void_p(p.value + 16)
        assert L.fathom_stream_read_runs(off, 8192, 8192, 128, sp, None) == F.ERR_INVALID_ARG
    finally:
        assert L.fathom_host_free(p) == F.OK
