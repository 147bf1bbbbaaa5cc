"""The allocation-free decode step (fathom_step_noalloc, for callers that cannot
allocate: graph capture, tight serving loops) against fathom_step with a workspace of
its own: two calls in a row on the library's static scratch, the second smaller, each
must give the same depths, winners, scores and attention outputs as fathom_step on the
same inputs (identical kernels, so identical bits)."""
import numpy as np
import pytest

from bit_plane_kv_amd import fathom as F

from gpu_util import inputs, store_from_keys, to_dev, torch_cuda

pytestmark = pytest.mark.gpu

SM = float(np.float32(1 / np.sqrt(128)))


def _both(H, G, n, B, k, seed, with_scores):
    torch = torch_cuda()
    print(f"[noalloc] H={H} G={G} n={n} B={B} k={k} scores={with_scores}", flush=True)
    keys, q, K, V = inputs(130 + seed, H, G, n)
    st, _ = store_from_keys(keys)
    q_t = to_dev(q)
    K_t = to_dev(K).view(torch.bfloat16)
    V_t = to_dev(V).view(torch.bfloat16)
    res = []
    for noalloc in (False, True):
        out = torch.empty((H, G, 128), dtype=torch.bfloat16, device="cuda")
        depth = torch.empty((H, 128), dtype=torch.uint8, device="cuda")
        idx = torch.full((H, G, k), -1, dtype=torch.int32, device="cuda")
        scores = (torch.empty((H, G, n), dtype=torch.float32, device="cuda")
                  if with_scores else None)
        if noalloc:
            F.fathom_step_noalloc(st, q_t, K_t, V_t, B, k, SM, out, depth_out=depth,
                                  scores_out=scores, idx_out=idx)
        else:
            F.fathom_step(st, q_t, K_t, V_t, B, k, SM, out=out, depth_out=depth,
                          scores_out=scores, idx_out=idx)
        torch.cuda.synchronize()
        res.append((out, depth, idx, scores))
    (o0, d0, i0, s0), (o1, d1, i1, s1) = res
    assert torch.equal(d0, d1)
    assert torch.equal(i0, i1)
    assert torch.equal(o0.view(torch.int16), o1.view(torch.int16))
    if with_scores:
        assert torch.equal(s0, s1)
    return F.workspace_size(F.OP_STEP, H, G, n, k)


def test_noalloc_step_equals_step_two_calls():
    # first call: one layer of the Qwen3-8B shape (8 KV heads x 4 queries, 32k tokens)
    big = _both(8, 4, 32768, 92, 512, 0, False)
    # second call, smaller, right after: the scratch still holds the first call's data
    small = _both(3, 2, 5000, 68, 64, 1, False)
    assert small < big <= F.STATIC_SCRATCH_BYTES


def test_noalloc_step_every_score_and_multichunk():
    # every score asked for (the full scan and top-k), then rows of several top-k chunks
    _both(2, 4, 20000, 136, 100, 2, True)
    _both(1, 4, 70000, 92, 512, 3, False)


def test_noalloc_step_refuses_too_large():
    torch = torch_cuda()
    H, G, n, k = 8, 4, 1 << 20, 512
    assert F.workspace_size(F.OP_STEP, H, G, n, k) > F.STATIC_SCRATCH_BYTES
    st = F.Store.empty(H, n, "cuda")   # never filled: refused before any GPU work
    q = torch.zeros((H, G, 128), dtype=torch.float32, device="cuda")
    kv = torch.zeros((1, 64, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((H, G, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(F.FathomError) as e:
        F.fathom_step_noalloc(st, q, kv, kv, 92, k, SM, out)
    assert e.value.status == F.ERR_SCRATCH
