"""Plain CPU oracle for the Fathom bit-plane key scan -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py``
may import this package.  The product path (``bit_plane_kv_amd`` and ``libfathom.so``)
never imports, links or runs it, and the two share no code.

This module is argument marshalling over ``fathom_oracle.c`` (numpy arrays in, numpy
arrays out); every step of the arithmetic is in that C file, which cites the pages.
Sources cited there: the author's blog post (sections by heading), the Glonce summary
"Fathom speeds long-context KV cache decoding 1.67x with per-query reads", and the
Rootconf proposal "Decoding at a million tokens when the KV cache lives in host memory".

Parity pins: every function here is pinned by ``tests/test_oracle_*.py`` against the
pages' worked example, closed forms, library routines or brute force; none is
"parity unpinned" except the accuracy claims that need real models (not implemented).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fathom_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

PLANES = 4


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no FMA contraction, OpenMP over heads)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC",
               "-shared", "-std=c11", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build(force=True)
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    I = ctypes.c_int
    D = ctypes.c_double
    sig = {
        "oracle_quantize_batch": (None, [P, I, I, I, P, P, P]),
        "oracle_pack_planes_batch": (None, [P, I, I, I, I, P]),
        "oracle_pack_nibbles_batch": (None, [P, I, I, I, P]),
        "oracle_f32_to_f16": (ctypes.c_uint16, [ctypes.c_float]),
        "oracle_f16_to_f32": (ctypes.c_float, [ctypes.c_uint16]),
        "oracle_quantize_grouped_batch": (None, [P, I, I, I, I, P, P, P]),
        "oracle_var_grouped_batch": (None, [P, P, P, I, I, I, I, P]),
        "oracle_scores_grouped_batch": (None, [P, P, P, P, P, I, I, I, I, I, P]),
        "oracle_var_batch": (None, [P, P, I, I, I, P]),
        "oracle_plan_batch": (I, [P, P, I, I, I, I, P]),
        "oracle_plan_fixed": (I, [P, I, I, P]),
        "oracle_scores_batch": (None, [P, P, P, P, P, I, I, I, I, P]),
        "oracle_topk_batch": (I, [P, I, I, I, P]),
        "oracle_attention_batch": (None, [P, P, P, I, I, I, I, P, I, D, P]),
        "oracle_dequantize": (None, [P, P, P, I, I, P]),
        "oracle_plane_prefix": (ctypes.c_uint32, [P, I, I, I, I]),
        "oracle_midpoint_level": (D, [I, I]),
        "oracle_importance": (D, [P, I, I, P, I]),
        "oracle_f32_to_bf16": (ctypes.c_uint16, [ctypes.c_float]),
        "oracle_bf16_to_f32": (ctypes.c_float, [ctypes.c_uint16]),
        "oracle_f32_to_bf16_array": (None, [P, ctypes.c_size_t, P]),
        "oracle_threads": (I, []),
        "oracle_topk_f64_batch": (I, [P, I, I, I, P]),
        "oracle_logits_batch": (None, [P, P, I, I, I, I, D, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def threads() -> int:
    """OpenMP threads the batched oracle calls use."""
    return int(_load().oracle_threads())


def set_threads(n: int) -> None:
    """Set the OpenMP thread count of the batched oracle calls (n >= 1)."""
    _load().oracle_set_threads(ctypes.c_int(int(n)))


def n_words(n: int) -> int:
    return (n + 31) // 32


# ---------------------------------------------------------------------------------
# store build
# ---------------------------------------------------------------------------------
def quantize(keys):
    """keys fp32 [H][n][d] (or [n][d]) -> (scale [H][d], zero [H][d], codes u8 [H][n][d])."""
    x = _c(keys, np.float32)
    squeeze = x.ndim == 2
    if squeeze:
        x = x[None]
    H, n, d = x.shape
    scale = np.empty((H, d), np.float32)
    zero = np.empty((H, d), np.float32)
    codes = np.empty((H, n, d), np.uint8)
    _load().oracle_quantize_batch(_p(x), H, n, d, _p(scale), _p(zero), _p(codes))
    if squeeze:
        return scale[0], zero[0], codes[0]
    return scale, zero, codes


def pack_planes(codes, W: int | None = None):
    """codes u8 [H][n][d] -> planes u32 [H][d][4][W] (W = ceil(n/32) by default)."""
    cd = _c(codes, np.uint8)
    squeeze = cd.ndim == 2
    if squeeze:
        cd = cd[None]
    H, n, d = cd.shape
    W = n_words(n) if W is None else W
    planes = np.empty((H, d, PLANES, W), np.uint32)
    _load().oracle_pack_planes_batch(_p(cd), H, n, d, W, _p(planes))
    return planes[0] if squeeze else planes


def pack_nibbles(codes):
    """codes u8 [H][n][d] -> token-major nibbles u8 [H][n][d/2] (channel 2j low, 2j+1 high)."""
    cd = _c(codes, np.uint8)
    squeeze = cd.ndim == 2
    if squeeze:
        cd = cd[None]
    H, n, d = cd.shape
    nib = np.empty((H, n, d // 2), np.uint8)
    _load().oracle_pack_nibbles_batch(_p(cd), H, n, d, _p(nib))
    return nib[0] if squeeze else nib


GROUP = 128  # tokens per scale/zero group of the grouped store


def f32_to_f16_bits(x: float) -> int:
    return int(_load().oracle_f32_to_f16(float(x)))


def f16_bits_to_f32(h: int) -> float:
    return float(_load().oracle_f16_to_f32(int(h)))


def quantize_grouped(keys, group: int = GROUP):
    """keys fp32 [H][n][d] -> (s16, z16 fp16 bits u16 [H][d][ceil(n/group)], codes u8 [H][n][d])."""
    x = _c(keys, np.float32)
    squeeze = x.ndim == 2
    if squeeze:
        x = x[None]
    H, n, d = x.shape
    ng = (n + group - 1) // group
    s16 = np.empty((H, d, ng), np.uint16)
    z16 = np.empty((H, d, ng), np.uint16)
    codes = np.empty((H, n, d), np.uint8)
    _load().oracle_quantize_grouped_batch(_p(x), H, n, d, int(group), _p(s16), _p(z16),
                                          _p(codes))
    if squeeze:
        return s16[0], z16[0], codes[0]
    return s16, z16, codes


def var_grouped(codes, s16, z16, group: int = GROUP):
    """fp32 [H][d] variance of the group-dequantized channels."""
    cd = _c(codes, np.uint8)
    sh, zh = _c(s16, np.uint16), _c(z16, np.uint16)
    squeeze = cd.ndim == 2
    if squeeze:
        cd, sh, zh = cd[None], sh[None], zh[None]
    H, n, d = cd.shape
    var = np.empty((H, d), np.float32)
    _load().oracle_var_grouped_batch(_p(cd), _p(sh), _p(zh), H, n, d, int(group), _p(var))
    return var[0] if squeeze else var


def scores_grouped(codes, s16, z16, depth, q, group: int = GROUP):
    """fp64 approximate scores [H][G][n] over a grouped store."""
    cd = _c(codes, np.uint8)
    sh, zh = _c(s16, np.uint16), _c(z16, np.uint16)
    dp, qq = _c(depth, np.uint8), _c(q, np.float32)
    squeeze = cd.ndim == 2
    if squeeze:
        cd, sh, zh, dp, qq = cd[None], sh[None], zh[None], dp[None], qq[None]
    H, n, d = cd.shape
    G = qq.shape[1]
    out = np.empty((H, G, n), np.float64)
    _load().oracle_scores_grouped_batch(_p(cd), _p(sh), _p(zh), _p(dp), _p(qq), H, n, d, G,
                                        int(group), _p(out))
    return out[0] if squeeze else out


def plane_prefix(planes_head, c: int, t: int, i: int) -> int:
    """t-plane prefix of token i, channel c, from one head's planes [d][4][W]."""
    pl = _c(planes_head, np.uint32)
    return int(_load().oracle_plane_prefix(_p(pl), pl.shape[-1], c, t, i))


def channel_var(codes, scale):
    """Population variance of the dequantized channels, fp32 [H][d]."""
    cd = _c(codes, np.uint8)
    sc = _c(scale, np.float32)
    squeeze = cd.ndim == 2
    if squeeze:
        cd, sc = cd[None], sc[None]
    H, n, d = cd.shape
    var = np.empty((H, d), np.float32)
    _load().oracle_var_batch(_p(cd), _p(sc), H, n, d, _p(var))
    return var[0] if squeeze else var


def importance(q_head, var_head, c: int) -> float:
    """w_c = var_c * sum_g q_gc^2 in fp64 for one head (q [G][d], var [d])."""
    q = _c(q_head, np.float32)
    v = _c(var_head, np.float32)
    G, d = q.shape
    return float(_load().oracle_importance(_p(q), G, d, _p(v), c))


def plan(q, var, B: int):
    """q fp32 [H][G][d], var fp32 [H][d] -> depth u8 [H][d] (greedy water-filling)."""
    qq = _c(q, np.float32)
    vv = _c(var, np.float32)
    squeeze = qq.ndim == 2
    if squeeze:
        qq, vv = qq[None], vv[None]
    H, G, d = qq.shape
    depth = np.empty((H, d), np.uint8)
    rc = _load().oracle_plan_batch(_p(qq), _p(vv), H, G, d, int(B), _p(depth))
    if rc != 0:
        raise ValueError(f"oracle plan rejected B={B} for d={d}")
    return depth[0] if squeeze else depth


def plan_fixed(var, n_channels: int):
    """Comparator plan: depth 4 on the n_channels largest-variance channels [H][d]."""
    vv = _c(var, np.float32)
    squeeze = vv.ndim == 1
    if squeeze:
        vv = vv[None]
    H, d = vv.shape
    depth = np.empty((H, d), np.uint8)
    for h in range(H):
        rc = _load().oracle_plan_fixed(_p(vv[h]), d, int(n_channels), _p(depth[h]))
        if rc != 0:
            raise ValueError(f"oracle fixed plan rejected n_channels={n_channels}")
    return depth[0] if squeeze else depth


def midpoint_level(code: int, t: int) -> float:
    return float(_load().oracle_midpoint_level(int(code), int(t)))


def scores(codes, scale, zero, depth, q):
    """fp64 approximate scores [H][G][n] from the oracle's own codes."""
    cd = _c(codes, np.uint8)
    sc, zr = _c(scale, np.float32), _c(zero, np.float32)
    dp, qq = _c(depth, np.uint8), _c(q, np.float32)
    squeeze = cd.ndim == 2
    if squeeze:
        cd, sc, zr, dp, qq = cd[None], sc[None], zr[None], dp[None], qq[None]
    H, n, d = cd.shape
    G = qq.shape[1]
    out = np.empty((H, G, n), np.float64)
    _load().oracle_scores_batch(_p(cd), _p(sc), _p(zr), _p(dp), _p(qq), H, n, d, G,
                                _p(out))
    return out[0] if squeeze else out


def dequantize(codes_head, scale_head, zero_head):
    """z + s*code in fp64 for one head: [n][d]."""
    cd = _c(codes_head, np.uint8)
    sc, zr = _c(scale_head, np.float32), _c(zero_head, np.float32)
    n, d = cd.shape
    out = np.empty((n, d), np.float64)
    _load().oracle_dequantize(_p(cd), _p(sc), _p(zr), n, d, _p(out))
    return out


def topk(scores_rows, k: int):
    """fp32 scores [R][n] -> int32 idx [R][k], ascending by index."""
    s = _c(scores_rows, np.float32)
    squeeze = s.ndim == 1
    if squeeze:
        s = s[None]
    R, n = s.shape
    idx = np.empty((R, k), np.int32)
    rc = _load().oracle_topk_batch(_p(s), R, n, int(k), _p(idx))
    if rc != 0:
        raise ValueError(f"oracle top-k rejected k={k} for n={n}")
    return idx[0] if squeeze else idx


def topk_f64(scores_rows, k: int):
    """fp64 scores [R][n] -> int32 idx [R][k], ascending by index (same order rule as
    topk: larger first, equal values to the lower index, -0 as +0)."""
    s = _c(scores_rows, np.float64)
    squeeze = s.ndim == 1
    if squeeze:
        s = s[None]
    R, n = s.shape
    idx = np.empty((R, k), np.int32)
    rc = _load().oracle_topk_f64_batch(_p(s), R, n, int(k), _p(idx))
    if rc != 0:
        raise ValueError(f"oracle top-k rejected k={k} for n={n}")
    return idx[0] if squeeze else idx


def logits(q, K, sm_scale: float):
    """q fp32 [H][G][d]; K bf16 bits (uint16) [H][n][d] -> fp64 logits [H][G][n] of
    every token (the attention's first step over all n rows)."""
    qq = _c(q, np.float32)
    KK = _c(K, np.uint16)
    H, G, d = qq.shape
    n = KK.shape[1]
    out = np.empty((H, G, n), np.float64)
    _load().oracle_logits_batch(_p(qq), _p(KK), H, G, n, d, float(sm_scale), _p(out))
    return out


def attention(q, K, V, idx, sm_scale: float):
    """q fp32 [H][G][d]; K,V bf16 bits (uint16) [H][n][d]; idx int32 [H][G][k]
    -> fp64 [H][G][d]."""
    qq = _c(q, np.float32)
    KK, VV = _c(K, np.uint16), _c(V, np.uint16)
    ii = _c(idx, np.int32)
    H, G, d = qq.shape
    n = KK.shape[1]
    k = ii.shape[2]
    out = np.empty((H, G, d), np.float64)
    _load().oracle_attention_batch(_p(qq), _p(KK), _p(VV), H, G, n, d, _p(ii), k,
                                   float(sm_scale), _p(out))
    return out


def f32_to_bf16(x):
    """Round fp32 values to bf16 (ties to even); returns uint16 bit patterns."""
    flat = np.ascontiguousarray(x, np.float32).ravel()
    out = np.empty(flat.size, np.uint16)
    _load().oracle_f32_to_bf16_array(_p(flat), flat.size, _p(out))
    return out.reshape(np.shape(x))


def bf16_to_f32(h):
    lib = _load()
    flat = np.ascontiguousarray(h, np.uint16).ravel()
    out = np.fromiter((lib.oracle_bf16_to_f32(int(v)) for v in flat), np.float32,
                      count=flat.size)
    return out.reshape(np.shape(h))
