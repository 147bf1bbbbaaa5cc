"""CPU tests of the C-ABI: the library loads, exports every call include/fathom.h
declares, and rejects bad arguments on the host (no GPU needed: these paths return
before any HIP call)."""
import ctypes
import os
import re

import pytest

from bit_plane_kv_amd import fathom as F

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fathom.h")

FAKE = 1 << 20  # a 16-byte aligned non-null address; never dereferenced on these paths


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fathom_\w+)\s*\(", text)))


def test_every_declared_call_is_exported():
    L = F.lib()
    names = _declared()
    assert len(names) >= 14
    for name in names:
        assert hasattr(L, name), name
    # and the binding wraps exactly the declared calls
    assert sorted(F.EXPORTS) == names


def test_word_stride():
    """Rows of at least 16 pages of 4 KiB become an odd number of whole pages; shorter
    rows only round up to 4 words."""
    L = F.lib()
    assert L.fathom_word_stride(1) == 4
    assert L.fathom_word_stride(100) == 4
    assert L.fathom_word_stride(4096) == 128
    assert L.fathom_word_stride(32768) == 1024
    assert L.fathom_word_stride(262144) == 8192
    assert L.fathom_word_stride(524256) == 16384          # 16383 words: below 16 pages
    assert L.fathom_word_stride(524287) == 17 * 1024      # 16384 words: 16 pages -> 17
    assert L.fathom_word_stride(524288) == 17 * 1024
    assert L.fathom_word_stride(1 << 20) == 33 * 1024     # 32 pages -> 33
    assert L.fathom_word_stride((1 << 20) + 1) == 33 * 1024
    for n in [1, 33, 777, 32769, 600000, 1 << 20, 3000000]:
        ws = L.fathom_word_stride(n)
        assert ws >= (n + 31) // 32 and ws % 4 == 0
        if ws >= 16 * 1024:
            assert ws % 1024 == 0 and (ws // 1024) % 2 == 1


def test_version_and_status_strings():
    L = F.lib()
    assert L.fathom_version() == 100
    for s in range(8):
        assert F.status_string(s)
    assert F.status_string(99) == "unknown status"
    assert L.fathom_last_hip_error() == 0


def _st(H=2, n=100, d=128, stride=None, planes=FAKE):
    return F.fathom_store(H, n, d, ((n + 31) // 32 + 3) // 4 * 4 if stride is None else stride,
                          planes, FAKE, FAKE, FAKE)


def test_store_checks():
    L = F.lib()
    r = lambda st: L.fathom_plan(ctypes.byref(st) if st is not None else None, FAKE, 1, 8,
                                 FAKE, None)
    assert r(None) == F.ERR_INVALID_ARG
    assert r(_st(d=64)) == F.ERR_UNSUPPORTED
    assert r(_st(n=0)) == F.ERR_INVALID_ARG
    assert r(_st(H=0)) == F.ERR_INVALID_ARG
    assert r(_st(stride=3)) == F.ERR_INVALID_ARG          # < ceil(100/32)
    assert r(_st(stride=6)) == F.ERR_INVALID_ARG          # rows not 16-byte multiples
    assert r(_st(planes=None)) == F.ERR_INVALID_ARG
    assert r(_st(planes=FAKE + 4)) == F.ERR_INVALID_ARG   # planes must be 16-aligned


def test_plan_checks():
    L = F.lib()
    st = _st()
    assert L.fathom_plan(ctypes.byref(st), FAKE, 1, 513, FAKE, None) == F.ERR_BUDGET
    assert L.fathom_plan(ctypes.byref(st), FAKE, 1, -1, FAKE, None) == F.ERR_BUDGET
    assert L.fathom_plan(ctypes.byref(st), FAKE, 9, 8, FAKE, None) == F.ERR_UNSUPPORTED
    assert L.fathom_plan(ctypes.byref(st), FAKE, 0, 8, FAKE, None) == F.ERR_INVALID_ARG
    assert L.fathom_plan(ctypes.byref(st), None, 1, 8, FAKE, None) == F.ERR_INVALID_ARG
    assert L.fathom_plan(ctypes.byref(st), FAKE, 1, 8, None, None) == F.ERR_INVALID_ARG
    assert L.fathom_plan_fixed(ctypes.byref(st), 129, FAKE, None) == F.ERR_BUDGET
    assert L.fathom_plan_fixed(ctypes.byref(st), 34, None, None) == F.ERR_INVALID_ARG


def test_scan_checks():
    L = F.lib()
    st = _st()
    need = F.workspace_size(F.OP_SCAN, 2, 4)
    assert L.fathom_scan(ctypes.byref(st), FAKE, 4, FAKE, FAKE, FAKE, need - 1,
                         None) == F.ERR_WORKSPACE
    assert L.fathom_scan(ctypes.byref(st), FAKE, 4, FAKE, FAKE, None, need,
                         None) == F.ERR_INVALID_ARG
    assert L.fathom_scan(ctypes.byref(st), FAKE, 4, FAKE, FAKE + 4, FAKE, need,
                         None) == F.ERR_INVALID_ARG
    assert L.fathom_scan_prepared(ctypes.byref(st), 9, FAKE, FAKE, need,
                                  None) == F.ERR_UNSUPPORTED
    assert L.fathom_scan_prepare(ctypes.byref(st), None, 4, FAKE, FAKE, need,
                                 None) == F.ERR_INVALID_ARG


def test_scan_topk_checks():
    L = F.lib()
    st = _st()
    need = F.workspace_size(F.OP_SCAN_TOPK, 2, 4, 100, 10)
    args = lambda G, k, ws, ws_bytes: (ctypes.byref(st), FAKE, G, FAKE, k, FAKE, ws, ws_bytes,
                                       None)
    assert L.fathom_scan_topk(*args(4, 10, FAKE, need - 1)) == F.ERR_WORKSPACE
    assert L.fathom_scan_topk(*args(4, 101, FAKE, need)) == F.ERR_INVALID_ARG
    assert L.fathom_scan_topk(*args(4, 0, FAKE, need)) == F.ERR_INVALID_ARG
    assert L.fathom_scan_topk(*args(9, 10, FAKE, need)) == F.ERR_UNSUPPORTED
    assert L.fathom_scan_topk(*args(4, 10, None, need)) == F.ERR_INVALID_ARG


def test_topk_checks():
    L = F.lib()
    assert L.fathom_topk(FAKE, 4, 100, 0, FAKE, None, 0, None) == F.ERR_INVALID_ARG
    assert L.fathom_topk(FAKE, 4, 100, 101, FAKE, None, 0, None) == F.ERR_INVALID_ARG
    assert L.fathom_topk(FAKE, 0, 100, 10, FAKE, None, 0, None) == F.ERR_INVALID_ARG
    assert L.fathom_topk(FAKE, 4, 40000, 16385, FAKE, FAKE, 1 << 30,
                         None) == F.ERR_UNSUPPORTED
    need = F.workspace_size(F.OP_TOPK, 4, 1, 40000, 512)
    assert need > 0
    assert L.fathom_topk(FAKE, 4, 40000, 512, FAKE, FAKE, need - 1, None) == F.ERR_WORKSPACE
    assert L.fathom_topk(FAKE, 4, 40000, 512, FAKE, None, need, None) == F.ERR_INVALID_ARG


def test_attn_and_step_checks():
    L = F.lib()
    assert L.fathom_sparse_attn(FAKE, FAKE, FAKE, 1, 1, 100, 64, FAKE, 5, 0.1, FAKE,
                                None) == F.ERR_UNSUPPORTED
    assert L.fathom_sparse_attn(FAKE, FAKE, FAKE, 1, 1, 100, 128, FAKE, 101, 0.1, FAKE,
                                None) == F.ERR_INVALID_ARG
    assert L.fathom_sparse_attn(FAKE, FAKE + 2, FAKE, 1, 1, 100, 128, FAKE, 5, 0.1, FAKE,
                                None) == F.ERR_INVALID_ARG
    st = _st()
    need = F.workspace_size(F.OP_STEP, 2, 4, 100, 10)
    args = lambda B, k, ws_bytes: (ctypes.byref(st), FAKE, FAKE, FAKE, 4, B, k, 0.1, FAKE,
                                   None, None, None, FAKE, ws_bytes, None)
    assert L.fathom_step(*args(92, 10, need - 1)) == F.ERR_WORKSPACE
    assert L.fathom_step(*args(600, 10, need)) == F.ERR_BUDGET
    assert L.fathom_step(*args(92, 101, need)) == F.ERR_INVALID_ARG
    # the timed step: the event list is checked first, then everything fathom_step checks
    # (fake handles are never recorded on these paths)
    ev = (ctypes.c_void_p * 5)(*[FAKE + 256 * i for i in range(5)])
    assert L.fathom_step_timed(*args(92, 10, need), None, 5) == F.ERR_INVALID_ARG
    assert L.fathom_step_timed(*args(92, 10, need), ev, 4) == F.ERR_INVALID_ARG
    bad = (ctypes.c_void_p * 5)(FAKE, FAKE, None, FAKE, FAKE)
    assert L.fathom_step_timed(*args(92, 10, need), bad, 5) == F.ERR_INVALID_ARG
    assert L.fathom_step_timed(*args(92, 10, need - 1), ev, 5) == F.ERR_WORKSPACE
    assert L.fathom_step_timed(*args(600, 10, need), ev, 5) == F.ERR_BUDGET
    assert F.STEP_PHASES + 1 == 5


def test_stream_read_and_host_alloc_checks():
    L = F.lib()
    assert L.fathom_stream_read(FAKE, 15, FAKE, None) == F.ERR_INVALID_ARG
    assert L.fathom_stream_read(None, 16, FAKE, None) == F.ERR_INVALID_ARG
    assert L.fathom_stream_read_runs(FAKE, 24, 32, 4, FAKE, None) == F.ERR_INVALID_ARG
    assert L.fathom_stream_read_runs(FAKE, 32, 16, 4, FAKE, None) == F.ERR_INVALID_ARG
    assert L.fathom_stream_read_runs(FAKE, 32, 32, 0, FAKE, None) == F.ERR_INVALID_ARG
    assert L.fathom_stream_read_runs(FAKE, 1 << 20, 1 << 20, 1 << 20, FAKE,
                                     None) == F.ERR_UNSUPPORTED
    # 2^32 vectors of 16 bytes in all: refused (the kernel's run division is 32-bit)
    assert L.fathom_stream_read_runs(FAKE, 16, 16, 1 << 32, FAKE, None) == F.ERR_UNSUPPORTED
    assert L.fathom_stream_read_runs(FAKE, 64, 64, 1 << 30, FAKE, None) == F.ERR_UNSUPPORTED
    p = ctypes.c_void_p()
    assert L.fathom_host_alloc(0, 0, ctypes.byref(p)) == F.ERR_INVALID_ARG
    assert L.fathom_host_alloc(16, 2, ctypes.byref(p)) == F.ERR_INVALID_ARG
    assert L.fathom_host_free(None) == F.ERR_INVALID_ARG


def test_workspace_formulas():
    # scan: 4 KiB meta + 16 K-blocks x 64 lanes x 16 bytes per set of 4 queries, per head
    for G, qs in [(1, 1), (2, 1), (3, 1), (4, 1), (5, 2), (8, 2)]:
        assert F.workspace_size(F.OP_SCAN, 3, G) == 3 * (4096 + 16 * 64 * 16 * qs)
    # top-k: rows that fit one chunk need nothing
    assert F.workspace_size(F.OP_TOPK, 1152, 1, 32768, 512) == 0
    # 1M tokens: 32 chunks x 512 candidates x (4 + 4) bytes per row, one level
    assert F.workspace_size(F.OP_TOPK, 32, 1, 1 << 20, 512) == 32 * 32 * 512 * 8
    # scan + top-k: scan workspace, candidate record area (4 bytes per token, rows
    # rounded up to 256-token blocks), kept-token masks (4 bytes per 32 tokens), the top-k
    # levels and the redo list (8 bytes per row chunk: a chunk may be listed by its own
    # select and again by its row's count check), each rounded up to 256 bytes
    r256 = lambda x: (x + 255) // 256 * 256
    for H, G, n, k in [(2, 4, 100, 10), (288, 4, 32768, 512), (3, 8, 70000, 512)]:
        want = (r256(F.workspace_size(F.OP_SCAN, H, G)) + r256(H * G * r256(n) * 4) +
                r256(H * G * ((n + 31) // 32) * 4) +
                r256(F.workspace_size(F.OP_TOPK, H * G, 1, n, k)) +
                r256(H * G * ((n + 32767) // 32768) * 8))
        assert F.workspace_size(F.OP_SCAN_TOPK, H, G, n, k) == want
    # grouped step: every score (fp32), the top-k levels, the winners, the depths, then (at
    # most 256 rows) the split attention's parts (8 groups x 132 floats a row) and a counter
    # per row
    for H, G, n, k in [(2, 4, 100, 10), (288, 4, 32768, 512), (8, 4, 1 << 20, 512)]:
        part = H * G * 8 * 132 * 4 if H * G <= 256 else 0
        want = (r256(H * G * n * 4) + r256(F.workspace_size(F.OP_TOPK, H * G, 1, n, k)) +
                r256(H * G * k * 4) + r256(H * 128) + r256(part) + r256(H * G * 4))
        assert F.workspace_size(F.OP_STEP_GROUPED, H, G, n, k) == want
    with pytest.raises(F.FathomError):
        F.workspace_size(F.OP_STEP_GROUPED, 8, 9, 100, 10)
    with pytest.raises(F.FathomError):
        F.workspace_size(F.OP_STEP_GROUPED, 8, 4, 100, 101)
    # quantize: min/max partials + integer sums
    q = F.workspace_size(F.OP_QUANTIZE, 2, 1, 4096, 1)
    assert q == 2 * 2 * 2 * 128 * 4 + 2 * 128 * 16
    with pytest.raises(F.FathomError):
        F.workspace_size(F.OP_STEP, 8, 9, 100, 10)
    with pytest.raises(F.FathomError):
        F.workspace_size(7, 8, 1, 100, 10)


def test_step_noalloc_refuses_what_exceeds_its_scratch():
    """The allocation-free step checks its size on the host: a problem whose step
    workspace exceeds the static 64 MiB is refused before any GPU call."""
    L = F.lib()
    assert F.STATIC_SCRATCH_BYTES == 64 << 20

    def store(H, n):
        st = F.fathom_store(H, n, 128, L.fathom_word_stride(n), FAKE, FAKE, FAKE, FAKE)
        return ctypes.byref(st)

    def call(H, n, G=4, B=92, k=512):
        return L.fathom_step_noalloc(store(H, n), FAKE, FAKE, FAKE, G, B, k, 0.088, FAKE,
                                     None, None, None, None)

    assert F.workspace_size(F.OP_STEP, 288, 4, 32768, 512) > F.STATIC_SCRATCH_BYTES
    assert call(288, 32768) == F.ERR_SCRATCH
    assert call(8, 1 << 20) == F.ERR_SCRATCH
    assert call(8, 1 << 20, B=600) == F.ERR_BUDGET
    assert call(8, 32768, G=9) == F.ERR_UNSUPPORTED
    assert call(8, 32768, k=0) == F.ERR_INVALID_ARG
    assert F.status_string(F.ERR_SCRATCH).startswith("problem needs more")

