"""Seeded synthetic inputs for the MoE layer (the only module shared by the tests, the bench
and the CPU oracle's callers).

This module draws numbers and changes their storage format; it computes nothing of the
layer itself.

Recipe (one independent stream per tensor block):
  * stream key ``SeedSequence([seed, tensor_id, block])``, PCG64, ``standard_normal`` in
    float32; tensor ids: 0 x, 1 router weight, 2 gate bias, 3 gate projection,
    4 up projection, 5 down projection; ``block`` is the expert for expert weights and a
    4096-row chunk for x;
  * x ~ N(0, 1); router weight ~ N(0, 1/hidden) unless the config overrides the std;
    gate/up projections ~ N(0, 1/hidden); down projection ~ N(0, 1/inter)
    ("N(0, v)" is read as variance v);
  * gate bias: none, N(0, v), or the Zipf(s) popularity log-prior -s*ln(e+1);
  * bf16 tensors are rounded from float32 to nearest-even and kept as raw uint16 bits.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

from .configs import MoEConfig, BF16, SWIGLU

TID_X, TID_ROUTER, TID_BIAS, TID_GATE, TID_UP, TID_DOWN = range(6)
X_CHUNK_ROWS = 4096


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); NaN stays a quiet NaN."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint32, copy=True)
    nan = np.isnan(a)
    u += np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    out = (u >> np.uint32(16)).astype(np.uint16)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(seed: int, tid: int, block: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tid, block])))


def _normal(seed, tid, block, shape, std, bf16: bool) -> np.ndarray:
    z = _rng(seed, tid, block).standard_normal(int(np.prod(shape)), dtype=np.float32)
    z = z.reshape(shape)
    if std != 1.0:
        z *= np.float32(std)
    return f32_to_bf16_bits(z) if bf16 else z


def _experts(seed, tid, E, shape, std, bf16, pool) -> np.ndarray:
    dt = np.uint16 if bf16 else np.float32
    out = np.empty((E,) + tuple(shape), dtype=dt)

    def one(e):
        out[e] = _normal(seed, tid, e, shape, std, bf16)

    list(pool.map(one, range(E)))
    return out


def gate_bias(cfg: MoEConfig, seed: int = 0) -> Optional[np.ndarray]:
    if cfg.bias is None:
        return None
    kind, p = cfg.bias
    if kind == "normal":
        return _normal(seed, TID_BIAS, 0, (cfg.experts,), math.sqrt(p), False)
    if kind == "zipf":
        # popularity p_e proportional to (e+1)^-s; the log-prior differs from ln p_e by a
        # constant, which softmax and top-k ignore.
        return (-float(p) * np.log(np.arange(1, cfg.experts + 1, dtype=np.float64))).astype(
            np.float32)
    raise ValueError(f"unknown bias recipe {cfg.bias!r}")


def make_inputs(cfg: MoEConfig, seed: int = 0, threads: int = 8, weights: bool = True) -> dict:
    """All inputs of one layer call. bf16 tensors are uint16 bit arrays, fp32 ones float32."""
    bf16 = cfg.dtype == BF16
    T, H, I, E = cfg.tokens, cfg.hidden, cfg.inter, cfg.experts
    out = {}
    with ThreadPoolExecutor(max(1, threads)) as pool:
        x = np.empty((T, H), dtype=np.uint16 if bf16 else np.float32)

        def xchunk(c):
            r0 = c * X_CHUNK_ROWS
            r1 = min(T, r0 + X_CHUNK_ROWS)
            x[r0:r1] = _normal(seed, TID_X, c, (r1 - r0, H), 1.0, bf16)

        list(pool.map(xchunk, range((T + X_CHUNK_ROWS - 1) // X_CHUNK_ROWS)))
        out["x"] = x
        rstd = cfg.router_std if cfg.router_std is not None else 1.0 / math.sqrt(H)
        out["w_router"] = _normal(seed, TID_ROUTER, 0, (H, E), rstd, bf16)
        out["bias"] = gate_bias(cfg, seed)
        if weights:
            out["w_gate"] = (_experts(seed, TID_GATE, E, (H, I), 1.0 / math.sqrt(H), bf16, pool)
                             if cfg.activation == SWIGLU else None)
            out["w_up"] = _experts(seed, TID_UP, E, (H, I), 1.0 / math.sqrt(H), bf16, pool)
            out["w_down"] = _experts(seed, TID_DOWN, E, (I, H), 1.0 / math.sqrt(I), bf16, pool)
    return out


def as_float(cfg: MoEConfig, a):
    """float32 view of an input array (bf16 bits are widened exactly)."""
    if a is None:
        return None
    return bf16_bits_to_f32(a) if (cfg.dtype == BF16 and a.dtype == np.uint16) else a


class ExpertView:
    """Lazy per-expert float32 view of a stacked [E, ...] weight array (bounds host memory)."""

    def __init__(self, cfg: MoEConfig, stacked: np.ndarray):
        self.cfg, self.a = cfg, stacked

    def __len__(self):
        return self.a.shape[0]

    def __getitem__(self, e):
        return as_float(self.cfg, self.a[e])
