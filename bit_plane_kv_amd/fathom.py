"""ctypes binding of libfathom.so -- argument marshalling only.

Every function named ``fathom_*`` here calls the C function of the same name declared in
``include/fathom.h``; tensors are passed as device pointers and the current torch stream
as the HIP stream.  torch is used for device memory and streams only: all arithmetic of
the store build, plan, scan, top-k and attention runs in the library's HIP kernels.
The binding raises ``FathomError`` if the library is missing or a call fails; there is
no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfathom.so")

D = 128
PLANES = 4
MAX_G = 8
TOPK_CHUNK = 32768

(OK, ERR_INVALID_ARG, ERR_BUDGET, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_NOT_MAPPED, ERR_HIP,
 ERR_SCRATCH) = range(8)
STATIC_SCRATCH_BYTES = 64 << 20  # the static workspace of fathom_step_noalloc
OP_QUANTIZE, OP_SCAN, OP_TOPK, OP_STEP, OP_SCAN_TOPK, OP_STEP_GROUPED = range(6)


class FathomError(RuntimeError):
    def __init__(self, status: int, call: str, msg: str):
        super().__init__(f"{call}: {msg} (status {status})")
        self.status = status


class fathom_store(ctypes.Structure):
    _fields_ = [("n_heads", ctypes.c_int32), ("n_tokens", ctypes.c_int32),
                ("d", ctypes.c_int32), ("word_stride", ctypes.c_int32),
                ("planes", ctypes.c_void_p), ("scale", ctypes.c_void_p),
                ("zero", ctypes.c_void_p), ("var", ctypes.c_void_p)]


class fathom_gstore(ctypes.Structure):
    _fields_ = [("n_heads", ctypes.c_int32), ("n_tokens", ctypes.c_int32),
                ("d", ctypes.c_int32), ("word_stride", ctypes.c_int32),
                ("group_stride", ctypes.c_int32), ("pad", ctypes.c_int32),
                ("planes", ctypes.c_void_p), ("scale16", ctypes.c_void_p),
                ("zero16", ctypes.c_void_p), ("sums", ctypes.c_void_p),
                ("var", ctypes.c_void_p), ("prefix", ctypes.c_void_p),
                ("prefix_groups", ctypes.c_void_p)]


_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int
_SZ = ctypes.c_size_t
_SIGS = {
    "fathom_version": (_I, []),
    "fathom_word_stride": (_I, [_I]),
    "fathom_last_hip_error": (_I, []),
    "fathom_status_string": (ctypes.c_char_p, [_I]),
    "fathom_workspace_size": (_I, [_I, _I, _I, _I, _I, ctypes.POINTER(_SZ)]),
    "fathom_quantize_store": (_I, [_P, _I, _I, _I, ctypes.POINTER(fathom_store), _P, _SZ, _P]),
    "fathom_plan": (_I, [ctypes.POINTER(fathom_store), _P, _I, _I, _P, _P]),
    "fathom_plan_fixed": (_I, [ctypes.POINTER(fathom_store), _I, _P, _P]),
    "fathom_scan": (_I, [ctypes.POINTER(fathom_store), _P, _I, _P, _P, _P, _SZ, _P]),
    "fathom_scan_prepare": (_I, [ctypes.POINTER(fathom_store), _P, _I, _P, _P, _SZ, _P]),
    "fathom_scan_prepared": (_I, [ctypes.POINTER(fathom_store), _I, _P, _P, _SZ, _P]),
    "fathom_scan_topk": (_I, [ctypes.POINTER(fathom_store), _P, _I, _P, _I, _P, _P, _SZ, _P]),
    "fathom_topk": (_I, [_P, _I, _I, _I, _P, _P, _SZ, _P]),
    "fathom_sparse_attn": (_I, [_P, _P, _P, _I, _I, _I, _I, _P, _I, ctypes.c_float, _P, _P]),
    "fathom_step": (_I, [ctypes.POINTER(fathom_store), _P, _P, _P, _I, _I, _I, ctypes.c_float,
                         _P, _P, _P, _P, _P, _SZ, _P]),
    "fathom_step_timed": (_I, [ctypes.POINTER(fathom_store), _P, _P, _P, _I, _I, _I,
                               ctypes.c_float, _P, _P, _P, _P, _P, _SZ, _P,
                               ctypes.POINTER(ctypes.c_void_p), _I]),
    "fathom_step_noalloc": (_I, [ctypes.POINTER(fathom_store), _P, _P, _P, _I, _I, _I,
                                 ctypes.c_float, _P, _P, _P, _P, _P]),
    "fathom_scan_extract": (_I, [_P, _P, _I, _P, _P, _P]),
    "fathom_pack_nibbles": (_I, [ctypes.POINTER(fathom_store), _P, _P]),
    "fathom_quantize_groups": (_I, [_P, ctypes.c_int64, ctypes.POINTER(fathom_gstore), _I, _I,
                                    _P]),
    "fathom_plan_grouped": (_I, [ctypes.POINTER(fathom_gstore), _P, _I, _I, _P, _P]),
    "fathom_scan_grouped": (_I, [ctypes.POINTER(fathom_gstore), _P, _I, _P, _P, _P]),
    "fathom_step_grouped": (_I, [ctypes.POINTER(fathom_gstore), _P, _P, _P, _I, _I, _I,
                                 ctypes.c_float, _P, _P, _P, _P, _P, _SZ, _P]),
    "fathom_scan_nibble": (_I, [_P, _P, _P, _I, _I, _P, _I, _P, _P]),
    "fathom_stream_read": (_I, [_P, _SZ, _P, _P]),
    "fathom_stream_read_runs": (_I, [_P, _SZ, _SZ, _SZ, _P, _P]),
    "fathom_host_alloc": (_I, [_SZ, _I, ctypes.POINTER(ctypes.c_void_p)]),
    "fathom_host_free": (_I, [_P]),
}
EXPORTS = tuple(_SIGS)


def lib():
    """Load libfathom.so (built by ``python -m bit_plane_kv_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise FathomError(-1, "load", f"{LIB_PATH} is missing; build it with "
                              "`python -m bit_plane_kv_amd.build` (there is no fallback)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().fathom_status_string(status).decode()


def _check(status: int, call: str):
    if status != OK:
        msg = status_string(status)
        if status == ERR_HIP:
            msg += f" (hipError {lib().fathom_last_hip_error()})"
        raise FathomError(status, call, msg)


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def workspace_size(op: int, H: int, G: int = 1, n: int = 1, k: int = 1) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().fathom_workspace_size(op, H, G, n, k, ctypes.byref(out)),
           "fathom_workspace_size")
    return out.value


def _workspace(nbytes: int, device):
    import torch
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


# ---------------------------------------------------------------------------------
# the store: caller-owned buffers (torch tensors) + the C descriptor
# ---------------------------------------------------------------------------------
@dataclass
class Store:
    planes: object        # uint32 viewed as int32 tensor [H][d][4][word_stride]
    scale: object         # fp32 [H][d]
    zero: object
    var: object
    n_tokens: int

    @property
    def n_heads(self) -> int:
        return int(self.planes.shape[0])

    @property
    def word_stride(self) -> int:
        return int(self.planes.shape[-1])

    def descriptor(self) -> fathom_store:
        return fathom_store(self.n_heads, self.n_tokens, D, self.word_stride,
                            _ptr(self.planes), _ptr(self.scale), _ptr(self.zero),
                            _ptr(self.var))

    @staticmethod
    def empty(H: int, n: int, device, word_stride: int | None = None, planes=None) -> "Store":
        """Allocate the store's buffers; `planes` may be supplied (e.g. pinned host)."""
        import torch
        W = int(lib().fathom_word_stride(int(n))) if word_stride is None else word_stride
        if planes is None:
            planes = torch.empty((H, D, PLANES, W), dtype=torch.int32, device=device)
        kw = dict(dtype=torch.float32, device=device)
        return Store(planes, torch.empty((H, D), **kw), torch.empty((H, D), **kw),
                     torch.empty((H, D), **kw), n)

    def view_heads(self, h0: int, h1: int) -> "Store":
        return Store(self.planes[h0:h1], self.scale[h0:h1], self.zero[h0:h1],
                     self.var[h0:h1], self.n_tokens)


GROUP = 128  # tokens per scale/zero group of the grouped store


@dataclass
class GStore:
    """Grouped store: planes as in Store, fp16 scale/zero and int32 code sums per
    (channel, 128-token group), fp32 var.  Capacity: n_max tokens."""
    planes: object        # int32 [H][d][4][word_stride]
    scale16: object       # int16 (fp16 bits) [H][group_stride][d]
    zero16: object
    sums: object          # int32 [H][d][group_stride][2]
    var: object           # fp32 [H][d]
    prefix: object        # fp64 [H][d][2], zeroed
    prefix_groups: object  # int32 [H][d], zeroed
    n_tokens: int

    @property
    def n_heads(self) -> int:
        return int(self.planes.shape[0])

    def descriptor(self) -> fathom_gstore:
        return fathom_gstore(self.n_heads, self.n_tokens, D, int(self.planes.shape[-1]),
                             int(self.scale16.shape[1]), 0, _ptr(self.planes),
                             _ptr(self.scale16), _ptr(self.zero16), _ptr(self.sums),
                             _ptr(self.var), _ptr(self.prefix), _ptr(self.prefix_groups))

    @staticmethod
    def empty(H: int, n_max: int, device, n: int = 0) -> "GStore":
        import torch
        ng = (n_max + GROUP - 1) // GROUP
        i32 = dict(dtype=torch.int32, device=device)
        ws = int(lib().fathom_word_stride(GROUP * ng))  # >= 4 ng words, whole groups
        return GStore(torch.zeros((H, D, PLANES, ws), **i32),
                      torch.zeros((H, ng, D), dtype=torch.int16, device=device),
                      torch.zeros((H, ng, D), dtype=torch.int16, device=device),
                      torch.zeros((H, D, ng, 2), **i32),
                      torch.zeros((H, D), dtype=torch.float32, device=device),
                      torch.zeros((H, D, 2), dtype=torch.float64, device=device),
                      torch.zeros((H, D), **i32), n)


def fathom_quantize_groups(keys, gstore: GStore, g0: int, g1: int, stream=None):
    """keys fp32 [H][m][d] (m = min(n, 128 g1) - 128 g0; any head stride) -> groups g0..g1-1."""
    gs = gstore.descriptor()
    _check(lib().fathom_quantize_groups(_ptr(keys), int(keys.stride(0)), ctypes.byref(gs),
                                        int(g0), int(g1), _stream(stream)),
           "fathom_quantize_groups")


def fathom_plan_grouped(gstore: GStore, q, B: int, depth=None, stream=None):
    import torch
    if depth is None:
        depth = torch.empty((gstore.n_heads, D), dtype=torch.uint8, device=q.device)
    gs = gstore.descriptor()
    _check(lib().fathom_plan_grouped(ctypes.byref(gs), _ptr(q), q.shape[1], int(B),
                                     _ptr(depth), _stream(stream)), "fathom_plan_grouped")
    return depth


def fathom_scan_grouped(gstore: GStore, q, depth, scores=None, stream=None):
    import torch
    H, G, _ = q.shape
    if scores is None:
        scores = torch.empty((H, G, gstore.n_tokens), dtype=torch.float32, device=q.device)
    gs = gstore.descriptor()
    _check(lib().fathom_scan_grouped(ctypes.byref(gs), _ptr(q), G, _ptr(depth), _ptr(scores),
                                     _stream(stream)), "fathom_scan_grouped")
    return scores


# ---------------------------------------------------------------------------------
# calls (same names as the C-ABI)
# ---------------------------------------------------------------------------------
def fathom_quantize_store(keys, store: Store, ws=None, stream=None):
    H, n, d = keys.shape
    need = workspace_size(OP_QUANTIZE, H, 1, n, 1)
    ws = _workspace(need, keys.device) if ws is None else ws
    st = store.descriptor()
    _check(lib().fathom_quantize_store(_ptr(keys), H, n, d, ctypes.byref(st), _ptr(ws),
                                       ws.numel() * ws.element_size(), _stream(stream)),
           "fathom_quantize_store")
    return store


def fathom_plan(store: Store, q, B: int, depth=None, stream=None):
    import torch
    H, G, _ = q.shape
    if depth is None:
        depth = torch.empty((H, D), dtype=torch.uint8, device=q.device)
    st = store.descriptor()
    _check(lib().fathom_plan(ctypes.byref(st), _ptr(q), G, int(B), _ptr(depth),
                             _stream(stream)), "fathom_plan")
    return depth


def fathom_plan_fixed(store: Store, n_channels: int, depth=None, stream=None):
    import torch
    if depth is None:
        depth = torch.empty((store.n_heads, D), dtype=torch.uint8, device=store.var.device)
    st = store.descriptor()
    _check(lib().fathom_plan_fixed(ctypes.byref(st), int(n_channels), _ptr(depth),
                                   _stream(stream)), "fathom_plan_fixed")
    return depth


def scan_workspace(store: Store, G: int, device):
    return _workspace(workspace_size(OP_SCAN, store.n_heads, G), device)


def fathom_scan(store: Store, q, depth, scores=None, ws=None, stream=None):
    import torch
    H, G, _ = q.shape
    if scores is None:
        scores = torch.empty((H, G, store.n_tokens), dtype=torch.float32, device=q.device)
    ws = scan_workspace(store, G, q.device) if ws is None else ws
    st = store.descriptor()
    _check(lib().fathom_scan(ctypes.byref(st), _ptr(q), G, _ptr(depth), _ptr(scores),
                             _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "fathom_scan")
    return scores


def fathom_scan_extract(store: Store, q, depth, scores=None, stream=None):
    """Comparator scan (per-bit extraction on the integer units); same result layout."""
    import torch
    H, G, _ = q.shape
    if scores is None:
        scores = torch.empty((H, G, store.n_tokens), dtype=torch.float32, device=q.device)
    st = store.descriptor()
    _check(lib().fathom_scan_extract(ctypes.byref(st), _ptr(q), G, _ptr(depth), _ptr(scores),
                                     _stream(stream)), "fathom_scan_extract")
    return scores


def fathom_pack_nibbles(store: Store, nib=None, stream=None):
    """The store's codes in the ordinary token-major layout: uint8 [H][n][64]."""
    import torch
    if nib is None:
        nib = torch.empty((store.n_heads, store.n_tokens, D // 2), dtype=torch.uint8,
                          device=store.var.device)
    st = store.descriptor()
    _check(lib().fathom_pack_nibbles(ctypes.byref(st), _ptr(nib), _stream(stream)),
           "fathom_pack_nibbles")
    return nib


def fathom_scan_nibble(nib, scale, zero, q, scores=None, stream=None):
    """Plain 4-bit scan of nibble-packed codes [H][n][64] -> scores [H][G][n] fp32."""
    import torch
    H, n, _ = nib.shape
    G = q.shape[1]
    if scores is None:
        scores = torch.empty((H, G, n), dtype=torch.float32, device=q.device)
    _check(lib().fathom_scan_nibble(_ptr(nib), _ptr(scale), _ptr(zero), H, n, _ptr(q), G,
                                    _ptr(scores), _stream(stream)), "fathom_scan_nibble")
    return scores


def fathom_scan_prepare(store: Store, q, depth, ws, stream=None):
    G = q.shape[1]
    st = store.descriptor()
    _check(lib().fathom_scan_prepare(ctypes.byref(st), _ptr(q), G, _ptr(depth), _ptr(ws),
                                     ws.numel() * ws.element_size(), _stream(stream)),
           "fathom_scan_prepare")


def fathom_scan_prepared(store: Store, G: int, scores, ws, stream=None):
    st = store.descriptor()
    _check(lib().fathom_scan_prepared(ctypes.byref(st), G, _ptr(scores), _ptr(ws),
                                      ws.numel() * ws.element_size(), _stream(stream)),
           "fathom_scan_prepared")
    return scores


def scan_topk_workspace(store: Store, G: int, k: int, device):
    return _workspace(workspace_size(OP_SCAN_TOPK, store.n_heads, G, store.n_tokens, k), device)


def fathom_scan_topk(store: Store, q, depth, k: int, idx=None, ws=None, stream=None):
    """Scan + top-k without writing every score -> idx [H][G][k] int32."""
    import torch
    H, G, _ = q.shape
    if idx is None:
        idx = torch.empty((H, G, k), dtype=torch.int32, device=q.device)
    ws = scan_topk_workspace(store, G, k, q.device) if ws is None else ws
    st = store.descriptor()
    _check(lib().fathom_scan_topk(ctypes.byref(st), _ptr(q), G, _ptr(depth), int(k), _ptr(idx),
                                  _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "fathom_scan_topk")
    return idx


def fathom_topk(scores, k: int, idx=None, ws=None, stream=None):
    """scores [..., n] fp32 (rows = product of leading dims) -> idx [..., k] int32."""
    import torch
    n = scores.shape[-1]
    R = scores.numel() // n
    if idx is None:
        idx = torch.empty((*scores.shape[:-1], k), dtype=torch.int32, device=scores.device)
    need = workspace_size(OP_TOPK, R, 1, n, k)
    if ws is None and need > 0:
        ws = _workspace(need, scores.device)
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().fathom_topk(_ptr(scores), R, n, int(k), _ptr(idx), _ptr(ws), wsb,
                             _stream(stream)), "fathom_topk")
    return idx


def fathom_sparse_attn(q, K, V, idx, sm_scale: float, out=None, stream=None):
    """q fp32 [H][G][d]; K, V bf16 [H][n][d]; idx int32 [H][G][k] -> out bf16 [H][G][d]."""
    import torch
    H, G, d = q.shape
    n = K.shape[1]
    k = idx.shape[-1]
    if out is None:
        out = torch.empty((H, G, d), dtype=torch.bfloat16, device=q.device)
    _check(lib().fathom_sparse_attn(_ptr(q), _ptr(K), _ptr(V), H, G, n, d, _ptr(idx), k,
                                    float(sm_scale), _ptr(out), _stream(stream)),
           "fathom_sparse_attn")
    return out


def step_grouped_workspace(gstore: GStore, G: int, k: int, device):
    return _workspace(workspace_size(OP_STEP_GROUPED, gstore.n_heads, G, gstore.n_tokens, k),
                      device)


def fathom_step_grouped(gstore: GStore, q, K, V, B: int, k: int, sm_scale: float, out=None,
                        depth_out=None, scores_out=None, idx_out=None, ws=None, stream=None):
    import torch
    H, G, d = q.shape
    if out is None:
        out = torch.empty((H, G, d), dtype=torch.bfloat16, device=q.device)
    ws = step_grouped_workspace(gstore, G, k, q.device) if ws is None else ws
    gs = gstore.descriptor()
    _check(lib().fathom_step_grouped(ctypes.byref(gs), _ptr(q), _ptr(K), _ptr(V), G, int(B),
                                     int(k), float(sm_scale), _ptr(out), _ptr(depth_out),
                                     _ptr(scores_out), _ptr(idx_out), _ptr(ws),
                                     ws.numel() * ws.element_size(), _stream(stream)),
           "fathom_step_grouped")
    return out


def step_workspace(store: Store, G: int, k: int, device):
    return _workspace(workspace_size(OP_STEP, store.n_heads, G, store.n_tokens, k), device)


def fathom_step(store: Store, q, K, V, B: int, k: int, sm_scale: float, out=None,
                depth_out=None, scores_out=None, idx_out=None, ws=None, stream=None):
    import torch
    H, G, d = q.shape
    if out is None:
        out = torch.empty((H, G, d), dtype=torch.bfloat16, device=q.device)
    ws = step_workspace(store, G, k, q.device) if ws is None else ws
    st = store.descriptor()
    _check(lib().fathom_step(ctypes.byref(st), _ptr(q), _ptr(K), _ptr(V), G, int(B), int(k),
                             float(sm_scale), _ptr(out), _ptr(depth_out), _ptr(scores_out),
                             _ptr(idx_out), _ptr(ws), ws.numel() * ws.element_size(),
                             _stream(stream)), "fathom_step")
    return out


def fathom_step_noalloc(store: Store, q, K, V, B: int, k: int, sm_scale: float, out,
                        depth_out=None, scores_out=None, idx_out=None, stream=None):
    """fathom_step on the library's static scratch: no workspace argument, and nothing is
    allocated here either, so `out` (bf16 [H][G][128]) must be given."""
    H, G, d = q.shape
    st = store.descriptor()
    _check(lib().fathom_step_noalloc(ctypes.byref(st), _ptr(q), _ptr(K), _ptr(V), G, int(B),
                                     int(k), float(sm_scale), _ptr(out), _ptr(depth_out),
                                     _ptr(scores_out), _ptr(idx_out), _stream(stream)),
           "fathom_step_noalloc")
    return out


STEP_PHASES = 4  # plan + scan preparation, scan, select, attention


def fathom_step_timed(store: Store, q, K, V, B: int, k: int, sm_scale: float, events,
                      out=None, depth_out=None, scores_out=None, idx_out=None, ws=None,
                      stream=None):
    """fathom_step with STEP_PHASES + 1 torch.cuda.Event (enable_timing) recorded on the
    stream at its phase boundaries: events[i].elapsed_time(events[i + 1]) is phase i."""
    import torch
    if len(events) != STEP_PHASES + 1:
        raise ValueError(f"fathom_step_timed needs {STEP_PHASES + 1} events")
    H, G, d = q.shape
    if out is None:
        out = torch.empty((H, G, d), dtype=torch.bfloat16, device=q.device)
    ws = step_workspace(store, G, k, q.device) if ws is None else ws
    st = store.descriptor()
    tstream = stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.current_stream()
    for e in events:  # torch creates an event's handle at its first record
        if not e.cuda_event:
            e.record(tstream)
    handles = (ctypes.c_void_p * len(events))(*[int(e.cuda_event) for e in events])
    _check(lib().fathom_step_timed(ctypes.byref(st), _ptr(q), _ptr(K), _ptr(V), G, int(B),
                                   int(k), float(sm_scale), _ptr(out), _ptr(depth_out),
                                   _ptr(scores_out), _ptr(idx_out), _ptr(ws),
                                   ws.numel() * ws.element_size(), _stream(stream), handles,
                                   len(events)), "fathom_step_timed")
    return out


def fathom_stream_read(src, nbytes: int, sink, stream=None):
    _check(lib().fathom_stream_read(_ptr(src), int(nbytes), _ptr(sink), _stream(stream)),
           "fathom_stream_read")


def fathom_stream_read_runs(src, run_bytes: int, stride_bytes: int, n_runs: int, sink,
                            stream=None):
    _check(lib().fathom_stream_read_runs(_ptr(src), int(run_bytes), int(stride_bytes),
                                         int(n_runs), _ptr(sink), _stream(stream)),
           "fathom_stream_read_runs")
