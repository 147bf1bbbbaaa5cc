"""The plain 4-bit comparator scan over the ordinary token-major layout (blog, "Where
this does not work"): packing bit-exact with the oracle's nibble layout, scores within
1e-5 of the oracle's fp64 scores with every channel read in full (depth 4)."""
import numpy as np
import pytest

import oracle
from bit_plane_kv_amd import fathom as F

from gpu_util import check_rows, inputs, store_from_keys, to_dev, torch_cuda

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("H,n,extra", [(1, 4096, 0), (3, 1013, 4), (2, 33, 0), (1, 1, 0),
                                       (2, 5000, 8), (1, 70000, 0)])
def test_pack_nibbles_matches_oracle(H, n, extra):
    torch = torch_cuda()
    print(f"[nibbles] H={H} n={n} extra={extra}", flush=True)
    keys, _, _, _ = inputs(110, H, 1, n)
    W = ((n + 31) // 32 + 3) // 4 * 4 + extra
    st, _ = store_from_keys(keys, word_stride=W)
    nib = F.fathom_pack_nibbles(st)
    torch.cuda.synchronize()
    _, _, codes = oracle.quantize(keys)
    assert np.array_equal(nib.cpu().numpy(), oracle.pack_nibbles(codes))


@pytest.mark.parametrize("H,G,n", [(3, 4, 5000), (2, 1, 4096), (2, 8, 777), (1, 3, 33),
                                   (1, 2, 12345), (1, 4, 1), (2, 5, 1030), (1, 4, 40000)])
def test_scan_nibble_matches_oracle(H, G, n):
    torch = torch_cuda()
    print(f"[scan_nibble] H={H} G={G} n={n}", flush=True)
    keys, q, _, _ = inputs(111, H, G, n)
    st, _ = store_from_keys(keys)
    nib = F.fathom_pack_nibbles(st)
    q_t = to_dev(q)
    got = F.fathom_scan_nibble(nib, st.scale, st.zero, q_t)
    torch.cuda.synchronize()
    s, z, codes = oracle.quantize(keys)
    ref = oracle.scores(codes, s, z, np.full((H, 128), 4, np.uint8), q)
    check_rows(got.cpu().numpy(), ref)
