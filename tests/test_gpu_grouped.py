"""The grouped store (fp16 scale and zero per 128-token group) against the oracle:
build and decode-time append bit-exact (planes, fp16 tables, variance), the plan
bit-exact, grouped scores within 1e-5 of the oracle's fp64 scores."""
import numpy as np
import pytest

import oracle
from bit_plane_kv_amd import fathom as F

from gpu_util import check_rows, inputs, to_dev, torch_cuda

pytestmark = pytest.mark.gpu


def _build(keys, n_max=None):
    torch = torch_cuda()
    H, n, _ = keys.shape
    gs = F.GStore.empty(H, n_max or n, "cuda", n=n)
    ng = (n + 127) // 128
    F.fathom_quantize_groups(to_dev(keys), gs, 0, ng)
    torch.cuda.synchronize()
    return gs


def _check_against_oracle(gs, keys):
    H, n, _ = keys.shape
    s16, z16, codes = oracle.quantize_grouped(keys)
    ng = (n + 127) // 128
    planes = gs.planes.cpu().numpy().view(np.uint32)
    assert np.array_equal(planes[..., :(n + 31) // 32], oracle.pack_planes(codes))
    assert not planes[..., (n + 31) // 32:4 * ng].any()      # words past n are zero
    # the store's tables are group-major [H][group][channel]; the oracle's [H][channel][group]
    assert np.array_equal(gs.scale16.cpu().numpy().view(np.uint16)[:, :ng].transpose(0, 2, 1), s16)
    assert np.array_equal(gs.zero16.cpu().numpy().view(np.uint16)[:, :ng].transpose(0, 2, 1), z16)
    assert np.array_equal(gs.var.cpu().numpy(), oracle.var_grouped(codes, s16, z16))
    return s16, z16, codes


@pytest.mark.parametrize("H,n,scale", [(1, 4096, 1.0), (3, 1000, 1.0), (2, 1, 1.0),
                                       (2, 130, 1e-6), (1, 777, 300.0), (2, 5000, 1.0)])
def test_grouped_build_matches_oracle(H, n, scale):
    print(f"[grouped build] H={H} n={n} scale={scale}", flush=True)
    keys, _, _, _ = inputs(120, H, 1, n)
    keys = (keys * np.float32(scale)).astype(np.float32)
    _check_against_oracle(_build(keys), keys)


def test_grouped_append_token_by_token_matches_rebuild():
    """Decode-time append: after each new token the partial last group is re-quantized
    from its tokens; every prefix must equal the oracle's build of that prefix."""
    torch = torch_cuda()
    H, n0, steps = 2, 250, 12           # crosses the group boundary at 256
    keys, _, _, _ = inputs(121, H, 1, n0 + steps)
    gs = _build(keys[:, :n0], n_max=n0 + steps)
    kd = to_dev(keys)
    for n in range(n0 + 1, n0 + steps + 1):
        print(f"[grouped append] n={n}", flush=True)
        gs.n_tokens = n
        g = (n - 1) // 128
        F.fathom_quantize_groups(kd[:, 128 * g:n], gs, g, g + 1)
        torch.cuda.synchronize()
        _check_against_oracle(gs, keys[:, :n])


def test_grouped_requantize_an_earlier_group():
    """Re-quantizing a group below the kept running sums restarts the variance from
    group 0; the result must again equal the oracle's build."""
    torch = torch_cuda()
    H, n = 2, 1000
    keys, _, _, _ = inputs(123, H, 1, n)
    gs = _build(keys)
    keys2 = keys.copy()
    keys2[:, 130:250] *= np.float32(3.0)          # group 1 changes
    F.fathom_quantize_groups(to_dev(keys2[:, 128:256]), gs, 1, 2)
    torch.cuda.synchronize()
    _check_against_oracle(gs, keys2)


@pytest.mark.parametrize("H,G,n,kind", [(2, 4, 3000, "plan92"), (1, 1, 4096, "b512"),
                                        (2, 8, 777, "random"), (1, 3, 33, "plan92"),
                                        (1, 4, 9000, "b0"), (2, 6, 5000, "plan92"),
                                        (1, 8, 4100, "b512")])
def test_grouped_plan_and_scan_match_oracle(H, G, n, kind):
    torch = torch_cuda()
    print(f"[grouped scan] H={H} G={G} n={n} {kind}", flush=True)
    keys, q, _, _ = inputs(122, H, G, n)
    gs = _build(keys)
    s16, z16, codes = oracle.quantize_grouped(keys)
    var = oracle.var_grouped(codes, s16, z16)
    q_t = to_dev(q)
    if kind == "plan92":
        depth = F.fathom_plan_grouped(gs, q_t, 92)
        ref_depth = oracle.plan(q, var, 92)
        assert np.array_equal(depth.cpu().numpy(), ref_depth)
    else:
        ref_depth = {"b512": np.full((H, 128), 4, np.uint8), "b0": np.zeros((H, 128), np.uint8),
                     "random": np.random.default_rng(n).integers(0, 5, (H, 128)).astype(
                         np.uint8)}[kind]
        depth = to_dev(ref_depth)
    got = F.fathom_scan_grouped(gs, q_t, depth)
    torch.cuda.synchronize()
    ref = oracle.scores_grouped(codes, s16, z16, ref_depth, q)
    check_rows(got.cpu().numpy(), ref)


def test_grouped_scan_from_pinned_host_memory_equals_hbm():
    """The grouped scan reads planes, fp16 scales and fp16 zeros in place from pinned host
    memory (the blog's setting for this index): the same scores as from HBM, bit for bit,
    over several 2048-token tiles and a ragged last one."""
    torch = torch_cuda()
    H, G, n = 2, 4, 5000
    print(f"[grouped host] H={H} G={G} n={n}", flush=True)
    keys, q, _, _ = inputs(123, H, G, n)
    gs = _build(keys)
    q_t = to_dev(q)
    depth = F.fathom_plan_grouped(gs, q_t, 92)
    ref = F.fathom_scan_grouped(gs, q_t, depth)
    host = {}
    for name in ("planes", "scale16", "zero16"):
        t = getattr(gs, name)
        host[name] = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
        host[name].copy_(t)
    gh = F.GStore(host["planes"], host["scale16"], host["zero16"], gs.sums, gs.var, gs.prefix,
                  gs.prefix_groups, n)
    got = F.fathom_scan_grouped(gh, q_t, depth)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    s16, z16, codes = oracle.quantize_grouped(keys)
    check_rows(got.cpu().numpy(), oracle.scores_grouped(codes, s16, z16, depth.cpu().numpy(), q))


@pytest.mark.parametrize("H,G,n,B,k", [(2, 4, 3000, 92, 64), (1, 8, 777, 136, 100),
                                       (3, 4, 5000, 0, 512), (2, 2, 40000, 92, 512),
                                       (1, 4, 130, 512, 130)])
def test_grouped_step_matches_oracle(H, G, n, B, k):
    """The grouped decode step against the oracle: the plan bit-exact, every score within
    1e-5 of the oracle's fp64 scores, the winners exactly the oracle's top-k of the scores
    the step computed, the output within 2e-2 of the oracle's attention over them."""
    torch = torch_cuda()
    print(f"[grouped step] H={H} G={G} n={n} B={B} k={k}", flush=True)
    keys, q, K, V = inputs(124, H, G, n)
    gs = _build(keys)
    s16, z16, codes = oracle.quantize_grouped(keys)
    var = oracle.var_grouped(codes, s16, z16)
    q_t = to_dev(q)
    Kd = to_dev(K).view(torch.bfloat16)
    Vd = to_dev(V).view(torch.bfloat16)
    sm = float(np.float32(1 / np.sqrt(128)))
    depth = torch.empty((H, 128), dtype=torch.uint8, device="cuda")
    scores = torch.empty((H, G, n), dtype=torch.float32, device="cuda")
    idx = torch.empty((H, G, k), dtype=torch.int32, device="cuda")
    out = F.fathom_step_grouped(gs, q_t, Kd, Vd, B, k, sm, depth_out=depth, scores_out=scores,
                                idx_out=idx)
    torch.cuda.synchronize()
    ref_depth = oracle.plan(q, var, B)
    assert np.array_equal(depth.cpu().numpy(), ref_depth)
    check_rows(scores.cpu().numpy(), oracle.scores_grouped(codes, s16, z16, ref_depth, q))
    got = idx.cpu().numpy()
    assert np.array_equal(got.reshape(H * G, k),
                          oracle.topk(scores.cpu().numpy().reshape(H * G, n), k))
    ref_out = oracle.attention(q, K, V, got, sm)
    assert np.abs(out.float().cpu().numpy() - ref_out).max() <= 2e-2


@pytest.mark.parametrize("H,G,n,k", [(2, 4, 5000, 128), (4, 4, 32768, 512)])
def test_grouped_step_equals_its_four_calls(H, G, n, k):
    """fathom_step_grouped with no optional outputs (intermediates in its workspace) gives
    the outputs, bit for bit, of plan, scan, top-k and attention called one by one, also
    when the same workspace serves a second step of other queries."""
    torch = torch_cuda()
    print(f"[grouped step calls] H={H} G={G} n={n} k={k}", flush=True)
    keys, q, K, V = inputs(125, H, G, n)
    gs = _build(keys)
    Kd = to_dev(K).view(torch.bfloat16)
    Vd = to_dev(V).view(torch.bfloat16)
    sm = float(np.float32(1 / np.sqrt(128)))
    ws = F.step_grouped_workspace(gs, G, k, "cuda")
    for rep in range(2):
        q_t = to_dev(q) if rep == 0 else to_dev(q[:, ::-1].copy())
        out = F.fathom_step_grouped(gs, q_t, Kd, Vd, 92, k, sm, ws=ws)
        depth = F.fathom_plan_grouped(gs, q_t, 92)
        scores = F.fathom_scan_grouped(gs, q_t, depth)
        idx = F.fathom_topk(scores, k)
        ref = F.fathom_sparse_attn(q_t, Kd, Vd, idx, sm)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
