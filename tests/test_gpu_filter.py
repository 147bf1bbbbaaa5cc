"""The candidate-filtering scan + select (fathom_scan_topk, and fathom_step without
scores_out) against the full scan + top-k.

Bar: the index sets are bit-exact with the oracle's top-k of the full scan's scores (the
full scan itself is held to the oracle's scores in test_gpu_parity).  The filter's
threshold is a guess; the cases below also force the guess to fail (rows keep fewer than
k tokens), which the select must repair by rescoring, and check through the workspace's
per-query counts that both the filtering and the repair actually ran.
"""
import numpy as np
import pytest

import oracle
from bit_plane_kv_amd import fathom as F
from bit_plane_kv_amd import synth

from gpu_util import bf16_to_f32, inputs, store_from_keys, to_dev, torch_cuda

pytestmark = pytest.mark.gpu

META_BYTES = 4096
CNT_OFFSET = 16 + 3 * 32   # int32 x4, then C[8], S[8], tkey[8]; cnt[8] follows


OVF_OFFSET = CNT_OFFSET + 32 + 4 * 512 + 32   # after cnt[8], plane[512], cnt_exact[8]


def _kept_counts(ws, H, G):
    """Per-(head, query) kept-token counts from the prepared scan workspace."""
    raw = ws[:H * META_BYTES].cpu().numpy().view(np.uint8).reshape(H, META_BYTES)
    return raw[:, CNT_OFFSET:CNT_OFFSET + 32].copy().view(np.uint32)[:, :G]


def _ovf_bits(ws, H):
    """Per-head overflow bits (bit g: row g's candidates are incomplete, rescored)."""
    raw = ws[:H * META_BYTES].cpu().numpy().view(np.uint8).reshape(H, META_BYTES)
    return raw[:, OVF_OFFSET:OVF_OFFSET + 4].copy().view(np.uint32)[:, 0]


def _depth(kind, st, q_t, H, n):
    torch = torch_cuda()
    if kind == "plan92":
        return F.fathom_plan(st, q_t, 92)
    if kind == "b0":
        return torch.zeros((H, 128), dtype=torch.uint8, device="cuda")
    if kind == "b512":
        return torch.full((H, 128), 4, dtype=torch.uint8, device="cuda")
    rng = np.random.default_rng(n)
    return to_dev(rng.integers(0, 5, (H, 128)).astype(np.uint8))


def _sample_words(W):
    """Words the threshold sample reads: every word of a short row, else 8 runs of 4
    words at 4 * floor(r (W // 4 - 1) / 7)."""
    if W <= 32:
        return np.arange(W)
    return np.concatenate([4 * (r * (W // 4 - 1) // 7) + np.arange(4) for r in range(8)])


def _filters(n, k):
    """Whether the sample yields a threshold: its rank m (least m with
    n (m - 5 sqrt(m)) / S >= k) must not exceed the S sampled tokens."""
    W = (n + 31) // 32
    toks = (_sample_words(W)[:, None] * 32 + np.arange(32)[None, :]).ravel()
    S = int((toks < n).sum())
    x = 0.5 * (5.0 + np.sqrt(25.0 + 4.0 * k * S / n))
    return np.ceil(x * x) <= S


def _run(keys, q, k, kind):
    torch = torch_cuda()
    H, G, _ = q.shape
    n = keys.shape[1]
    st, _ = store_from_keys(keys)
    q_t = to_dev(q)
    depth = _depth(kind, st, q_t, H, n)
    full = F.fathom_scan(st, q_t, depth)
    ws = F.scan_topk_workspace(st, G, k, "cuda")
    idx = F.fathom_scan_topk(st, q_t, depth, k, ws=ws)
    torch.cuda.synchronize()
    got = idx.cpu().numpy().reshape(H * G, k)
    ref = oracle.topk(full.cpu().numpy().reshape(H * G, n), k)
    assert np.array_equal(got, ref)
    return _kept_counts(ws, H, G), _ovf_bits(ws, H)


@pytest.mark.parametrize("H,G,n,k,kind", [
    (3, 4, 5000, 64, "plan92"),       # sampled runs (more than 64 words)
    (2, 8, 4096, 100, "random"),      # two query sets
    (1, 3, 33, 5, "plan92"),          # every word sampled
    (2, 1, 32768, 512, "plan92"),     # the Qwen3-8B row length
    (1, 2, 70000, 512, "plan92"),     # several chunks: candidate levels with filler
    (2, 4, 12345, 1, "random"),       # k = 1
    (1, 4, 2000, 2000, "plan92"),     # k = n: no threshold
    (2, 4, 3000, 50, "b0"),           # every score equal: ties to the lower index
    (2, 4, 9000, 300, "b512"),
    (1, 5, 40000, 16384, "plan92"),   # the largest k with several chunks
    (130, 4, 2048, 64, "plan92"),     # more than 512 one-chunk rows: the lean select
    (130, 4, 2048, 64, "b512"),       # ... every row rescored by the full select after it
])
def test_scan_topk_matches_full_scan(H, G, n, k, kind):
    print(f"[scan_topk] H={H} G={G} n={n} k={k} {kind}", flush=True)
    keys, q, _, _ = inputs(100, H, G, n)
    cnt, ovf = _run(keys, q, k, kind)
    if not _filters(n, k):   # k too close to n: the call scans everything
        return
    if kind == "b512":   # heads of more than 480 planes keep no records: all rescored
        assert (cnt == 0).all() and (ovf == (1 << G) - 1).all()
        return
    assert (cnt >= k).all() or kind == "random"   # a random depth may need the repair
    if n == 32768 and kind == "plan92":   # the filter keeps a small share of the row
        assert cnt.max() <= n // 8


TKEY_OFFSET = 16 + 2 * 32   # int32 x4, C[8], S[8], then tkey[8]


def _order_key(v):
    """The select's key of an fp32 score: unsigned order equals the scores' order."""
    b = np.asarray(v, np.float32).view(np.uint32)
    return np.where(b & 0x80000000, ~b, b ^ 0x80000000).astype(np.uint32)


@pytest.mark.parametrize("H,G,n,k,kind", [
    (2, 4, 32768, 512, "plan92"),     # m = 53: the two-stage search
    (2, 4, 32768, 512, "b512"),
    (1, 8, 9000, 300, "plan92"),      # m = 79, two query sets
    (1, 4, 70000, 2000, "random"),    # m = 71, a ragged last sample run
    (1, 5, 40000, 16384, "plan92"),   # m = 536 > 128: every key searched
    (3, 4, 5000, 64, "b0"),           # m = 48, every score equal
])
def test_sample_threshold_is_the_sampled_quantile(H, G, n, k, kind):
    """Each query's threshold key is the m-th largest order key of its scores at the
    sampled tokens (m = the sample rank, scores as the full scan computes them), with
    its low 12 bits cleared."""
    torch = torch_cuda()
    print(f"[sample threshold] H={H} G={G} n={n} k={k} {kind}", flush=True)
    keys, q, _, _ = inputs(103, H, G, n)
    st, _ = store_from_keys(keys)
    q_t = to_dev(q)
    depth = _depth(kind, st, q_t, H, n)
    full = F.fathom_scan(st, q_t, depth).cpu().numpy()
    ws = F.scan_topk_workspace(st, G, k, "cuda")
    F.fathom_scan_topk(st, q_t, depth, k, ws=ws)
    torch.cuda.synchronize()
    raw = ws[:H * META_BYTES].cpu().numpy().view(np.uint8).reshape(H, META_BYTES)
    tkey = raw[:, TKEY_OFFSET:TKEY_OFFSET + 32].copy().view(np.uint32)[:, :G]
    W = (n + 31) // 32
    toks = (_sample_words(W)[:, None] * 32 + np.arange(32)[None, :]).ravel()
    toks = toks[toks < n]
    S = toks.size
    x = 0.5 * (5.0 + np.sqrt(25.0 + 4.0 * k * S / n))
    m = int(np.ceil(x * x))
    assert m <= S
    for h in range(H):
        for g in range(G):
            srt = np.sort(_order_key(full[h, g, toks]))[::-1]
            assert tkey[h, g] == (srt[m - 1] & np.uint32(0xFFFFF000)), (h, g)


def _boost_sampled_tokens(keys, q):
    """Make the tokens the threshold sample reads the best of their rows, so that the
    sampled quantile sits far above the row's k-th score and few tokens clear it."""
    H, n, _ = keys.shape
    W = (n + 31) // 32
    toks = (_sample_words(W)[:, None] * 32 + np.arange(32)[None, :]).ravel()
    toks = toks[toks < n]
    out = keys.copy()
    for h in range(H):
        d = q[h].sum(axis=0)
        out[h, toks, :] += 6.0 * d / np.linalg.norm(d) * np.abs(keys[h]).max()
    return out


@pytest.mark.parametrize("H,G,n,k", [(2, 4, 32768, 512), (1, 2, 70000, 512),
                                     (1, 8, 9000, 300), (65, 8, 8192, 64)])
def test_scan_topk_repairs_rows_that_kept_too_few(H, G, n, k):
    print(f"[scan_topk repair] H={H} G={G} n={n} k={k}", flush=True)
    keys, q, _, _ = inputs(101, H, G, n)
    keys = _boost_sampled_tokens(keys, q)
    cnt, _ = _run(keys, q, k, "plan92")
    assert (cnt < k).any()   # the repair ran on at least one row


@pytest.mark.parametrize("H,G,n,k,boost", [
    (4, 4, 20000, 256, False),   # one layer's shape: select and attention in one kernel
    (2, 4, 32768, 512, True),    # ... and rows it must rescore (the sample boosted)
    (1, 4, 32768, 1024, False),  # the largest k of the fused kernel
    (70, 4, 3000, 64, False),    # more than 256 rows: select, redo, then attention
    # more rows than fill the CUs once with the fused select (8 workgroups a row), at most
    # 256: the fused front, then a workgroup a row for the select, then the split attention
    (16, 4, 20000, 256, False),
    (16, 4, 32768, 512, True),   # ... and rows the select must rescore
    (40, 4, 3000, 64, False),
    (12, 8, 9000, 300, False),   # two query sets: the separate scan, then the same select
])
def test_step_filtered_equals_step_full(H, G, n, k, boost):
    """The filtered step (scan with the keep test, select, attention) against the full
    step (every score written, full top-k, attention): the same winners and outputs."""
    torch = torch_cuda()
    B = 92
    print(f"[step filtered] H={H} G={G} n={n} B={B} k={k} boost={boost}", flush=True)
    keys, q, K, V = inputs(102, H, G, n)
    if boost:
        keys = _boost_sampled_tokens(keys, q)
        K = synth.bf16_bits(keys)
    st, _ = store_from_keys(keys)
    q_t = to_dev(q)
    Kd = to_dev(K).view(torch.bfloat16)
    Vd = to_dev(V).view(torch.bfloat16)
    sm = float(np.float32(1 / np.sqrt(128)))
    scores = torch.empty((H, G, n), dtype=torch.float32, device="cuda")
    i1 = torch.empty((H, G, k), dtype=torch.int32, device="cuda")
    i2 = torch.empty_like(i1)
    o1 = F.fathom_step(st, q_t, Kd, Vd, B, k, sm, scores_out=scores, idx_out=i1)
    o2 = F.fathom_step(st, q_t, Kd, Vd, B, k, sm, idx_out=i2)
    torch.cuda.synchronize()
    assert torch.equal(i1, i2)
    assert torch.equal(o1, o2)
    got = i2.cpu().numpy().reshape(H * G, k)
    assert np.array_equal(got, oracle.topk(scores.cpu().numpy().reshape(H * G, n), k))
    ref_out = oracle.attention(q, K, V, i2.cpu().numpy(), sm)
    assert np.abs(bf16_to_f32(o2) - ref_out).max() <= 2e-2


def test_step_rows_do_not_depend_on_the_kernels_shape():
    """A row's winners and output bits are the same whichever shape the step takes for
    the call: 8 KV heads x 4 queries (32 rows: select and attention in one kernel, eight
    workgroups a row) against the same heads plus one more (36 rows: a select workgroup a
    row, then the split attention), and the first 72 heads (288 rows: the lean select and
    a workgroup a row for the attention, whose softmax merges in another order: there the
    winners are compared exactly and the outputs within a rounding)."""
    torch = torch_cuda()
    H, G, n, B, k = 72, 4, 6000, 92, 256
    print(f"[step shapes] H={H} G={G} n={n} B={B} k={k}", flush=True)
    keys, q, K, V = inputs(131, H, G, n)
    st, _ = store_from_keys(keys)
    q_t = to_dev(q)
    Kd = to_dev(K).view(torch.bfloat16)
    Vd = to_dev(V).view(torch.bfloat16)
    sm = float(np.float32(1 / np.sqrt(128)))
    res = {}
    for h in (8, 9, 72):
        idx = torch.empty((h, G, k), dtype=torch.int32, device="cuda")
        out = F.fathom_step(st.view_heads(0, h), q_t[:h], Kd[:h], Vd[:h], B, k, sm, idx_out=idx)
        res[h] = (idx, out)
    torch.cuda.synchronize()
    for h in (9, 72):
        assert torch.equal(res[h][0][:8], res[8][0])
    assert torch.equal(res[9][1][:8], res[8][1])
    # at most one bf16 rounding step apart (8 significant bits)
    a, b = res[72][1][:9].float(), res[9][1].float()
    assert bool(((a - b).abs() <= torch.maximum(a.abs(), b.abs()) * 2.0 ** -7 + 1e-6).all())
    ref = oracle.attention(q, K, V, res[72][0].cpu().numpy(), sm)
    assert np.abs(bf16_to_f32(res[72][1]) - ref).max() <= 2e-2


@pytest.mark.parametrize("B,n,k", [(0, 9000, 100), (92, 3000, 2900), (92, 40000, 16384),
                                   (512, 33000, 512)])
def test_step_without_scores_out_equals_step_with(B, n, k):
    """The step's own choice of path (filter, or the full scan at B = 0 and when k is
    too close to n for a threshold) gives the winners and outputs of the full path."""
    torch = torch_cuda()
    H, G = 2, 4
    print(f"[step paths] B={B} n={n} k={k}", flush=True)
    keys, q, K, V = inputs(104, H, G, n)
    st, _ = store_from_keys(keys)
    q_t = to_dev(q)
    Kd = to_dev(K).view(torch.bfloat16)
    Vd = to_dev(V).view(torch.bfloat16)
    sm = float(np.float32(1 / np.sqrt(128)))
    scores = torch.empty((H, G, n), dtype=torch.float32, device="cuda")
    i1 = torch.empty((H, G, k), dtype=torch.int32, device="cuda")
    i2 = torch.empty_like(i1)
    o1 = F.fathom_step(st, q_t, Kd, Vd, B, k, sm, scores_out=scores, idx_out=i1)
    o2 = F.fathom_step(st, q_t, Kd, Vd, B, k, sm, idx_out=i2)
    torch.cuda.synchronize()
    assert torch.equal(i1, i2)
    assert torch.equal(o1, o2)
    assert np.array_equal(i1.cpu().numpy().reshape(H * G, k),
                          oracle.topk(scores.cpu().numpy().reshape(H * G, n), k))


def test_scan_topk_host_resident_store():
    torch = torch_cuda()
    H, G, n, k = 2, 4, 20000, 128
    print(f"[scan_topk host] H={H} G={G} n={n} k={k}", flush=True)
    keys, q, _, _ = inputs(103, H, G, n)
    st_d, _ = store_from_keys(keys)
    W = ((n + 31) // 32 + 3) // 4 * 4
    pinned = torch.empty((H, 128, 4, W), dtype=torch.int32, pin_memory=True)
    st_h, _ = store_from_keys(keys, planes=pinned)
    q_t = to_dev(q)
    depth = F.fathom_plan(st_d, q_t, 92)
    a = F.fathom_scan_topk(st_d, q_t, depth, k)
    b = F.fathom_scan_topk(st_h, q_t, depth, k)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def _random_cases(count, seed=7):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < count:
        H = int(rng.integers(1, 4))
        G = int(rng.integers(1, 9))
        n = int(rng.choice([rng.integers(1, 300), rng.integers(300, 40000),
                            rng.integers(40000, 90000)]))
        B = int(rng.choice([0, 4, 37, 92, 136, 300, 512]))
        kmax = n if n <= 32768 else 16384
        k = int(min(kmax, rng.choice([1, 7, 64, 512, 2000, n])))
        cases.append((H, G, n, B, k, int(rng.integers(0, 1 << 30))))
    return cases


@pytest.mark.parametrize("H,G,n,B,k,seed", _random_cases(20))
def test_step_paths_agree_on_random_shapes(H, G, n, B, k, seed):
    """Seeded random shapes, budgets and k: the step's fused path (or its fallback) gives
    exactly the winners and outputs of the full path."""
    torch = torch_cuda()
    print(f"[step random] H={H} G={G} n={n} B={B} k={k} seed={seed}", flush=True)
    keys, q, K, V = inputs(105, H, G, n, seed=seed % 1000)
    st, _ = store_from_keys(keys)
    q_t = to_dev(q)
    Kd = to_dev(K).view(torch.bfloat16)
    Vd = to_dev(V).view(torch.bfloat16)
    sm = float(np.float32(1 / np.sqrt(128)))
    scores = torch.empty((H, G, n), dtype=torch.float32, device="cuda")
    i1 = torch.empty((H, G, k), dtype=torch.int32, device="cuda")
    i2 = torch.empty_like(i1)
    o1 = F.fathom_step(st, q_t, Kd, Vd, B, k, sm, scores_out=scores, idx_out=i1)
    o2 = F.fathom_step(st, q_t, Kd, Vd, B, k, sm, idx_out=i2)
    torch.cuda.synchronize()
    assert torch.equal(i1, i2)
    assert torch.equal(o1, o2)
    assert np.array_equal(i1.cpu().numpy().reshape(H * G, k),
                          oracle.topk(scores.cpu().numpy().reshape(H * G, n), k))


@pytest.mark.parametrize("with_scores", [False, True])
def test_timed_step_equals_step_and_times_its_phases(with_scores):
    """fathom_step_timed: the same winners and output as fathom_step (filtering path and
    full path), with its phase events recorded in order on the stream."""
    torch = torch_cuda()
    H, G, n, B, k = 3, 4, 20000, 92, 256
    print(f"[step timed] with_scores={with_scores}", flush=True)
    keys, q, K, V = inputs(106, H, G, n, seed=3)
    st, _ = store_from_keys(keys)
    q_t = to_dev(q)
    Kd = to_dev(K).view(torch.bfloat16)
    Vd = to_dev(V).view(torch.bfloat16)
    sm = float(np.float32(1 / np.sqrt(128)))
    s1 = torch.empty((H, G, n), dtype=torch.float32, device="cuda") if with_scores else None
    s2 = torch.empty_like(s1) if with_scores else None
    i1 = torch.empty((H, G, k), dtype=torch.int32, device="cuda")
    i2 = torch.empty_like(i1)
    o1 = F.fathom_step(st, q_t, Kd, Vd, B, k, sm, scores_out=s1, idx_out=i1)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(F.STEP_PHASES + 1)]
    o2 = F.fathom_step_timed(st, q_t, Kd, Vd, B, k, sm, ev, scores_out=s2, idx_out=i2)
    torch.cuda.synchronize()
    assert torch.equal(i1, i2) and torch.equal(o1, o2)
    if with_scores:
        assert torch.equal(s1, s2)
    ph = [ev[i].elapsed_time(ev[i + 1]) for i in range(F.STEP_PHASES)]
    assert all(t > 0 for t in ph)
    assert abs(sum(ph) - ev[0].elapsed_time(ev[-1])) < 1e-3 + 1e-3 * sum(ph)
    with pytest.raises(ValueError):
        F.fathom_step_timed(st, q_t, Kd, Vd, B, k, sm, ev[:4])


@pytest.mark.parametrize("H,G,n,k", [
    (2, 4, 20000, 256),   # one-chunk rows, one query set: the fused front
    (1, 4, 70000, 512),   # rows of several chunks: select levels, then the attention
    (3, 8, 5000, 64),     # two query sets: the separate scan, then the select
])
def test_step_with_host_kv_equals_device_kv(H, G, n, k):
    """K/V rows in pinned host memory keep one attention workgroup a row (select and
    attention as separate launches); the winners and outputs are those of the step with
    K/V in device memory, where a row's attention is split over several workgroups, bit
    for bit (the same merge tree)."""
    torch = torch_cuda()
    B = 92
    print(f"[step host kv] H={H} G={G} n={n} k={k}", flush=True)
    keys, q, K, V = inputs(107, H, G, n)
    st, _ = store_from_keys(keys)
    q_t = to_dev(q)
    Kd = to_dev(K).view(torch.bfloat16)
    Vd = to_dev(V).view(torch.bfloat16)
    Kh = torch.from_numpy(K).view(torch.bfloat16).pin_memory()
    Vh = torch.from_numpy(V).view(torch.bfloat16).pin_memory()
    sm = float(np.float32(1 / np.sqrt(128)))
    i1 = torch.empty((H, G, k), dtype=torch.int32, device="cuda")
    i2 = torch.empty_like(i1)
    o1 = F.fathom_step(st, q_t, Kd, Vd, B, k, sm, idx_out=i1)
    o2 = F.fathom_step(st, q_t, Kh, Vh, B, k, sm, idx_out=i2)
    torch.cuda.synchronize()
    assert torch.equal(i1, i2)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    ref = oracle.attention(q, K, V, i1.cpu().numpy(), sm)
    assert np.abs(o2.float().cpu().numpy() - ref).max() <= 2e-2

