"""The synthetic accuracy-per-byte sweep's references and its rows, on a small cache
(blog, "What the measurements show -> Accuracy per byte": attention error against the
bits read per token).

The sweep measures the error of each selection against dense attention over all n
tokens and compares it with the exact top-k.  Both references are computed on the GPU
in fp64 (bench.attention_references); here they are checked against the oracle: the
dense output against the oracle's attention over every row, the exact top-k against
the oracle's fp64 top-k of its own logits (ties to the lower index, including rows
made equal on purpose).  The sweep's rows are then run at this size and checked for
what holds at any size.
"""
import numpy as np
import pytest

import bench
import oracle
from bit_plane_kv_amd import fathom as F
from bit_plane_kv_amd import synth

from gpu_util import inputs, store_from_keys, to_dev, torch_cuda

pytestmark = pytest.mark.gpu

SM = float(np.float32(1 / np.sqrt(128)))


def _cache(H, G, n, heavy, ties):
    keys, q, K, V = inputs(120, H, G, n)
    if heavy:
        q = synth.queries_heavy_np(7, 120, range(H), G)
    if ties:  # whole K rows repeated: equal logits at several token indices
        for h in range(H):
            K[h, 100:110] = K[h, 5]
            K[h, n - 20:n] = K[h, 7]
    return keys, q, K, V


@pytest.mark.parametrize("H,G,n,k,heavy,ties", [(2, 4, 4096, 64, False, False),
                                                (2, 4, 4096, 64, True, True),
                                                (1, 2, 3001, 17, False, True),
                                                (1, 1, 777, 777, True, False)])
def test_references_match_oracle(H, G, n, k, heavy, ties):
    torch = torch_cuda()
    print(f"[acc refs] H={H} G={G} n={n} k={k} heavy={heavy} ties={ties}", flush=True)
    keys, q, K, V = _cache(H, G, n, heavy, ties)
    q_t = to_dev(q)
    K_t = to_dev(K).view(torch.bfloat16)
    V_t = to_dev(V).view(torch.bfloat16)
    dense, top = bench.attention_references(q_t, K_t, V_t, k, SM)
    torch.cuda.synchronize()
    every = np.tile(np.arange(n, dtype=np.int32), (H, G, 1))
    ref_dense = oracle.attention(q, K, V, every, SM)
    err = np.abs(dense.cpu().numpy() - ref_dense).max()
    assert err <= 1e-10 * max(1.0, np.abs(ref_dense).max()), err
    ref_top = oracle.topk_f64(oracle.logits(q, K, SM).reshape(H * G, n), k)
    assert np.array_equal(top.cpu().numpy().reshape(H * G, k), ref_top)


def test_accuracy_rows_small():
    """The sweep's rows at a small size: every error finite and non-negative; the exact
    top-k's attention equals the oracle's attention over the oracle's top-k to bf16
    rounding; with every plane read (B = 512) on a cache whose K rows are the
    dequantized keys, the plan ranks by the exact logits up to fp32 rounding, so its
    error matches the exact top-k's."""
    torch = torch_cuda()
    H, G, n, k = 2, 4, 4096, 64
    keys, q, _, V = inputs(121, H, G, n)
    s, z, codes = oracle.quantize(keys)
    deq = np.stack([oracle.dequantize(codes[h], s[h], z[h]) for h in range(H)])
    K = oracle.f32_to_bf16(deq.astype(np.float32))
    st, _ = store_from_keys(keys)
    q_t = to_dev(q)
    K_t = to_dev(K).view(torch.bfloat16)
    V_t = to_dev(V).view(torch.bfloat16)
    dense, top = bench.attention_references(q_t, K_t, V_t, k, SM)
    fixed = F.fathom_plan_fixed(st, 34)
    r = bench.accuracy_rows(F, st, q_t, K_t, V_t, k, SM, fixed, (16, 92, 512), dense, top)
    torch.cuda.synchronize()
    rows = list(r["fathom"].values()) + [r["fixed136"], r["exact_topk"]]
    for e in rows:
        assert np.isfinite(e["max"]) and 0.0 <= e["mean"] <= e["max"]
    ref_top = oracle.topk_f64(oracle.logits(q, K, SM).reshape(H * G, n), k).reshape(H, G, k)
    ref_out = oracle.attention(q, K, V, ref_top, SM)
    ref_dense = oracle.attention(q, K, V, np.tile(np.arange(n, dtype=np.int32), (H, G, 1)), SM)
    e_ref = np.linalg.norm(ref_out - ref_dense, axis=-1) / np.linalg.norm(ref_dense, axis=-1)
    assert abs(r["exact_topk"]["mean"] - float(e_ref.mean())) <= 5e-3
    assert abs(r["fathom"]["512"]["mean"] - r["exact_topk"]["mean"]) <= 5e-3
