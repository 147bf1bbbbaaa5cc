"""The decode step at the benchmark's full sizes, launched as the benchmark launches it.

288 (layer, KV head) pairs x 32768 tokens, G = 4 queries per KV head, B = 92, k = 512
(a Qwen3-8B-shaped cache), one fathom_step on the filtering path with its workspace and
no score output -- the configuration bench.py times.  The oracle cannot redo all 288
heads in seconds, so sampled heads (the first, last and middle ones and their
neighbours) are checked one by one: plan bit-exact; the step's winners equal to the
exact top-k of the full-score scan's fp32 scores (the same arithmetic, computed on its
own path); those scores within the fp32 bar of the oracle's fp64 scores; the winners
within the end-to-end bar of the oracle's own top-k; and the attention output within the
bf16 bar of the oracle's attention over the step's winners.  The one-layer step at a
million tokens (8 KV heads x 1048576 tokens, rows of 32 top-k chunks: the candidate
level, its redo and the final level) is checked the same way, with the store and the
rows in HBM (the same kernels read pinned host memory in the benchmark's host-resident
line; residency itself is tested at small sizes in test_gpu_parity.py).
"""
import numpy as np
import pytest

import oracle
from bit_plane_kv_amd import fathom as F
from bit_plane_kv_amd import synth

from gpu_util import ATTN_ABS_TOL, SCORE_REL_TOL, bf16_to_f32, check_rows, to_dev, \
    topk_gate2, torch_cuda

pytestmark = pytest.mark.gpu

SEED = 11


@pytest.mark.parametrize("name,sampled", [("qwen3_8b_32k_hbm", [0, 1, 143, 144, 286, 287]),
                                          ("qwen3_8b_1m_layer_step", [0, 7])])
def test_step_full_size_sampled_heads(name, sampled):
    torch = torch_cuda()
    cfg = synth.CONFIGS[name]
    H, G, n, B, k = cfg.H, cfg.G, cfg.n, cfg.budgets[0], cfg.k
    print(f"[step full size] {name} H={H} G={G} n={n} B={B} k={k} seed={SEED}", flush=True)
    st = F.Store.empty(H, n, "cuda")
    K = torch.empty((H, n, 128), dtype=torch.bfloat16, device="cuda")
    qws = torch.empty(F.workspace_size(F.OP_QUANTIZE, 32, 1, n, 1), dtype=torch.uint8,
                      device="cuda")
    for h0 in range(0, H, 32):
        h1 = min(H, h0 + 32)
        keys = synth.keys_torch(SEED, cfg.cfg_id, range(h0, h1), n, "cuda")
        F.fathom_quantize_store(keys, st.view_heads(h0, h1), ws=qws)
        K[h0:h1].copy_(keys)
        del keys
    V = synth.values_torch(SEED, cfg.cfg_id, range(H), n, "cuda")
    q = synth.queries_np(SEED, cfg.cfg_id, range(H), G)
    q_t = to_dev(q)
    sm = float(np.float32(1 / np.sqrt(128)))
    ws = F.step_workspace(st, G, k, "cuda")
    depth = torch.empty((H, 128), dtype=torch.uint8, device="cuda")
    idx = torch.empty((H, G, k), dtype=torch.int32, device="cuda")
    out = F.fathom_step(st, q_t, K, V, B, k, sm, depth_out=depth, idx_out=idx, ws=ws)
    # the full-score scan with the step's own plan: the scores the filter and select
    # must have ranked
    full = F.fathom_scan(st, q_t, depth)
    torch.cuda.synchronize()
    depth_np, idx_np, full_np = depth.cpu().numpy(), idx.cpu().numpy(), full.cpu().numpy()
    del qws
    out_np = bf16_to_f32(out)
    del full
    for h in sampled:
        print(f"[step full size] head {h}", flush=True)
        kh = synth.keys_torch(SEED, cfg.cfg_id, [h], n, "cuda")
        s, z, codes = oracle.quantize(kh.cpu().numpy())
        var = oracle.channel_var(codes, s)
        ref_depth = oracle.plan(q[h][None], var, B)
        assert np.array_equal(depth_np[h], ref_depth[0]), h
        ref_scores = oracle.scores(codes, s, z, ref_depth, q[h][None])[0]
        check_rows(full_np[h], ref_scores)
        assert np.array_equal(idx_np[h], oracle.topk(full_np[h], k)), h
        tol = SCORE_REL_TOL * np.abs(ref_scores).max(axis=1)
        topk_gate2(idx_np[h][None], ref_scores[None], k, tol)
        Kh = K[h].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)[None]
        Vh = V[h].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)[None]
        ref_out = oracle.attention(q[h][None], Kh, Vh, idx_np[h][None], sm)[0]
        err = np.abs(out_np[h] - ref_out).max()
        assert err <= ATTN_ABS_TOL, (h, err)
