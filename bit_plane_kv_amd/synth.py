"""Seeded synthetic inputs shaped like the pages' workloads.

This module only draws random numbers; it holds none of the method's arithmetic, and
it is the one piece that both the library's tests/benchmarks and the oracle's callers
share.  The pages measure on real models (Llama-3.1-8B ... Qwen2.5-7B-Instruct-1M) and
real sessions, which are not available; these caches stand in for them with the
Qwen3-8B shape the blog uses ("How big the cache actually gets": 36 layers, 8 KV heads,
128 channels):

* per (layer, KV head, channel) a spread s_c = 10**U(-1, 1)  (log-uniform in [0.1, 10]);
* keys  = s_c * N(0, 1)                  fp32 [H][n][d]
* query = N(0, 1)                        fp32 [H][G][d]   (G query heads per KV head)
* K rows = the keys rounded to bf16      (the 16-bit cache the winners are read from)
* V rows = N(0, 1) rounded to bf16

Every stream comes from numpy's PCG64 seeded with SeedSequence([seed, config, head,
role]), so any head can be regenerated alone.  Large configurations are drawn on the
GPU with torch's Philox generator instead (``*_torch``), again seeded per head.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

D = 128          # channels per KV head (Qwen3-8B)
LAYERS = 36
KV_HEADS = 8

ROLE_SPREAD, ROLE_KEYS, ROLE_QUERY, ROLE_VALUE, ROLE_QGAIN = 0, 1, 2, 3, 4


@dataclass(frozen=True)
class Config:
    name: str
    cfg_id: int
    H: int            # (layer, KV head) pairs in one call
    G: int            # queries per KV head
    n: int            # tokens
    budgets: tuple    # bit budgets B per token per KV head
    k: int            # winners per query
    residency: str    # "hbm" or "host"
    fixed136: bool = False
    note: str = field(default="", compare=False)


CONFIGS = {
    "tiny": Config("tiny", 0, 1, 1, 4096, (68, 92, 136, 512), 64, "hbm",
                   note="1 KV head, 1 query, n=4096"),
    "qwen3_8b_32k_hbm": Config("qwen3_8b_32k_hbm", 1, LAYERS * KV_HEADS, 4, 32768, (92,),
                               512, "hbm", fixed136=True,
                               note="36 layers x 8 KV heads x 4 queries, n=32768, in HBM"),
    "qwen3_8b_256k_host": Config("qwen3_8b_256k_host", 2, LAYERS * KV_HEADS, 4, 262144,
                                 (68, 92, 136), 512, "host",
                                 note="n=262144, store in pinned host memory"),
    "qwen3_8b_1m_host": Config("qwen3_8b_1m_host", 3, LAYERS * KV_HEADS, 4, 1048576, (92,),
                               512, "host", fixed136=True,
                               note="n=1048576, store in pinned host memory"),
    "qwen3_8b_1m_layer_step": Config("qwen3_8b_1m_layer_step", 4, KV_HEADS, 4, 1048576,
                                     (92,), 512, "host",
                                     note="one layer's decode step at n=1048576"),
}


def _rng(seed: int, cfg_id: int, head: int, role: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(
        [int(seed), int(cfg_id), int(head), int(role)])))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even) and return the uint16 bits.
    Input formatting for the 16-bit cache rows; finite inputs only."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    lower = u & 0xFFFF
    upper = u >> 16
    bump = (lower > 0x8000) | ((lower == 0x8000) & ((upper & 1) == 1))
    return (upper + bump.astype(np.uint64)).astype(np.uint16)


def spreads(seed: int, cfg_id: int, head: int, d: int = D) -> np.ndarray:
    return (10.0 ** _rng(seed, cfg_id, head, ROLE_SPREAD).uniform(-1.0, 1.0, d)).astype(
        np.float32)


def keys_np(seed: int, cfg_id: int, heads, n: int, d: int = D) -> np.ndarray:
    """fp32 keys [len(heads)][n][d]."""
    heads = list(heads)
    out = np.empty((len(heads), n, d), np.float32)
    for a, h in enumerate(heads):
        s = spreads(seed, cfg_id, h, d)
        z = _rng(seed, cfg_id, h, ROLE_KEYS).standard_normal((n, d), dtype=np.float32)
        out[a] = z * s[None, :]
    return out


def queries_np(seed: int, cfg_id: int, heads, G: int, d: int = D) -> np.ndarray:
    heads = list(heads)
    out = np.empty((len(heads), G, d), np.float32)
    for a, h in enumerate(heads):
        out[a] = _rng(seed, cfg_id, h, ROLE_QUERY).standard_normal((G, d), dtype=np.float32)
    return out


def queries_heavy_np(seed: int, cfg_id: int, heads, G: int, d: int = D,
                     sigma: float = 1.5) -> np.ndarray:
    """Queries whose channel magnitudes are heavy-tailed: N(0, 1) times a per-(KV head,
    channel) gain exp(sigma N(0, 1)) shared by the head's G queries, so that a few
    channels dominate each head's scores (the regime a per-query plan is for)."""
    heads = list(heads)
    out = np.empty((len(heads), G, d), np.float32)
    for a, h in enumerate(heads):
        gain = np.exp(sigma * _rng(seed, cfg_id, h, ROLE_QGAIN).standard_normal(d))
        z = _rng(seed, cfg_id, h, ROLE_QUERY).standard_normal((G, d), dtype=np.float32)
        out[a] = (z * gain[None, :]).astype(np.float32)
    return out


def values_np(seed: int, cfg_id: int, heads, n: int, d: int = D) -> np.ndarray:
    """bf16 bits [len(heads)][n][d] of N(0, 1) values."""
    heads = list(heads)
    out = np.empty((len(heads), n, d), np.uint16)
    for a, h in enumerate(heads):
        out[a] = bf16_bits(_rng(seed, cfg_id, h, ROLE_VALUE).standard_normal(
            (n, d), dtype=np.float32))
    return out


# ---------------------------------------------------------------------------------
# device-side generation for the large configurations (torch is plumbing here)
# ---------------------------------------------------------------------------------
def _torch_seed(seed: int, cfg_id: int, head: int, role: int) -> int:
    ss = np.random.SeedSequence([int(seed), int(cfg_id), int(head), int(role)])
    return int(ss.generate_state(1, np.uint64)[0] & 0x7FFFFFFFFFFFFFFF)


def keys_torch(seed: int, cfg_id: int, heads, n: int, device, d: int = D):
    """fp32 keys [len(heads)][n][d] drawn on `device` (spreads from numpy, so a head's
    spreads match keys_np)."""
    import torch
    heads = list(heads)
    out = torch.empty((len(heads), n, d), dtype=torch.float32, device=device)
    gen = torch.Generator(device=device)
    for a, h in enumerate(heads):
        gen.manual_seed(_torch_seed(seed, cfg_id, h, ROLE_KEYS))
        s = torch.from_numpy(spreads(seed, cfg_id, h, d)).to(device)
        out[a].normal_(generator=gen)
        out[a].mul_(s[None, :])
    return out


def values_torch(seed: int, cfg_id: int, heads, n: int, device, d: int = D, out=None):
    """bf16 [len(heads)][n][d] of N(0, 1) values drawn on `device`."""
    import torch
    heads = list(heads)
    if out is None:
        out = torch.empty((len(heads), n, d), dtype=torch.bfloat16, device=device)
    gen = torch.Generator(device=device)
    tmp = torch.empty((n, d), dtype=torch.float32, device=device)
    for a, h in enumerate(heads):
        gen.manual_seed(_torch_seed(seed, cfg_id, h, ROLE_VALUE))
        tmp.normal_(generator=gen)
        out[a].copy_(tmp)
    return out
