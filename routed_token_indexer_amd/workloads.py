"""Seeded synthetic workloads for the routed token indexer.

This module only draws inputs. It holds none of the indexer's arithmetic (no
pooling, routing, scoring or selection), so that the CPU oracle and the GPU
path can both be fed from it without sharing any of the method.

Shapes follow the two inference phases the MISA pages describe (decode with one
query per sequence over a long prefix; causal prefill where every position is
a query), with the head counts of the two models the pages evaluate
(MISA pages, "Experimentele Resultaten": H_I = 64 for DeepSeek-V3.2 and
H_I = 32 for GLM-5, h = 8 routed heads).

Two value modes:

* ``gauss``: q ~ N(0, 1/d) per coordinate; w = softmax over heads of N(0, 1);
  keys either i.i.d. N(0, 1/d) or a stationary AR(1) along the sequence with
  rho = 0.9; optional planted "needle" keys of norm 4 aligned with a random
  query head of a query that can see them.
* ``grid``: q, k = U{-2..2} * 2^-4 and w = U{1..4} / 4, so every product and
  every partial sum of the indexer is a small multiple of a power of two and
  fp32 arithmetic is exact in any order.

All q/k values are rounded to bf16 (round to nearest even) before either side
sees them: ``q``/``k`` hold the bf16 values as float32, ``q_bf16``/``k_bf16``
the raw 16-bit patterns for upload. Generation order is q, w, keys, needles;
the seed is 1000 + config index (gauss) or 2000 + config index (grid).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

__all__ = ["Config", "CONFIGS", "config", "make_inputs", "bf16_round", "bf16_bits", "bits_to_f32"]


@dataclass(frozen=True)
class Config:
    name: str
    index: int
    nseq: int            # sequences whose keys are stored
    L: int               # stored prefix length per sequence (Lmax)
    T: int               # number of queries
    H: int               # indexer heads
    d: int               # head dimension
    B: int               # pooling block size
    h: int               # routed heads per query
    topk: int            # final selected tokens per query
    kc: Optional[int]    # candidate count of the hierarchical coarse pass (None: not used)
    needles: int         # planted needle keys per sequence (gauss mode only)
    ar1: bool            # AR(1) keys (True) or i.i.d. keys (False)
    phase: str           # "decode", "mtp" (several consecutive decode positions per sequence) or "prefill"
    q_len0: int = 0      # decode: first query's visible prefix when queries share one sequence
    description: str = ""

    @property
    def queries_per_seq(self) -> int:
        return self.T // self.nseq


# The five workload shapes. c0 is small enough for the pure-Python brute force;
# c1..c4 are the decode / prefill / long-context shapes the pages' models use.
CONFIGS = {
    "c0": Config("c0", 0, nseq=1, L=512, T=16, H=8, d=32, B=32, h=2, topk=64, kc=None,
                 needles=0, ar1=False, phase="decode", q_len0=497,
                 description="tiny: one 512-token sequence, 16 queries at prefixes 497..512, "
                             "H=8, d=32, B=32, h=2, k=64"),
    "c1": Config("c1", 1, nseq=4, L=32768, T=4, H=64, d=128, B=64, h=8, topk=2048, kc=None,
                 needles=32, ar1=True, phase="decode",
                 description="DeepSeek-V3.2-like decode: 4 sequences x 1 query, L=32768, H=64, "
                             "d=128, B=64, h=8, k=2048"),
    "c2": Config("c2", 2, nseq=1, L=16384, T=16384, H=64, d=128, B=64, h=8, topk=2048, kc=None,
                 needles=32, ar1=True, phase="prefill",
                 description="causal prefill: L=16384, every position a query, H=64, d=128, "
                             "B=64, h=8, k=2048"),
    "c3": Config("c3", 3, nseq=16, L=65536, T=16, H=32, d=128, B=64, h=8, topk=2048, kc=None,
                 needles=0, ar1=True, phase="decode",
                 description="GLM-5-like decode: 16 sequences x 1 query, L=65536, H=32, d=128, "
                             "B=64, h=8, k=2048"),
    "c4": Config("c4", 4, nseq=4, L=131072, T=4, H=64, d=128, B=128, h=8, topk=2048, kc=8192,
                 needles=64, ar1=True, phase="decode",
                 description="hierarchical MISA at 128K: 4 sequences x 1 query, L=131072, H=64, "
                             "d=128, B=128, h=8, k'=8192, k=2048"),
    # not one of the five shapes: a multi-token-prediction decode step on c1's
    # sequences (4 consecutive positions of each), for the shared key pass
    "c1m": Config("c1m", 5, nseq=4, L=32768, T=16, H=64, d=128, B=64, h=8, topk=2048, kc=None,
                  needles=32, ar1=True, phase="mtp",
                  description="multi-token decode: 4 sequences x 4 consecutive queries, L=32768, H=64, "
                              "d=128, B=64, h=8, k=2048"),
}


def config(name: str) -> Config:
    return CONFIGS[name]


# ---------------------------------------------------------------- bf16 encoding
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit pattern, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    return bits_to_f32(bf16_bits(x))


# ---------------------------------------------------------------- query layout
def query_layout(cfg: Config):
    """q_seq[t] (sequence of query t) and q_len[t] (its visible prefix length p)."""
    T = cfg.T
    if cfg.phase == "prefill":
        # every position is a query; a query sees itself, so p = t + 1
        q_seq = np.zeros(T, np.int32)
        q_len = np.arange(1, T + 1, dtype=np.int32)
    elif cfg.phase == "mtp":
        # m = T / nseq consecutive positions per sequence, queries of a sequence
        # adjacent: query i of sequence n sees L - m + 1 + i tokens
        m = T // cfg.nseq
        q_seq = np.repeat(np.arange(cfg.nseq, dtype=np.int32), m)
        q_len = np.tile(cfg.L - m + 1 + np.arange(m, dtype=np.int32), cfg.nseq).astype(np.int32)
    elif cfg.nseq == 1 and T > 1:
        # several decode queries on one sequence at consecutive prefixes
        q_seq = np.zeros(T, np.int32)
        q_len = (cfg.q_len0 + np.arange(T)).astype(np.int32)
    else:
        q_seq = np.arange(T, dtype=np.int32)
        q_len = np.full(T, cfg.L, np.int32)
    return q_seq, q_len


@dataclass
class Inputs:
    cfg: Config
    mode: str
    seed: int
    q: np.ndarray        # [T, H, d] float32 (bf16 values)
    w: np.ndarray        # [T, H] float32
    k: np.ndarray        # [nseq, L, d] float32 (bf16 values)
    q_seq: np.ndarray    # [T] int32
    q_len: np.ndarray    # [T] int32
    q_bf16: np.ndarray = field(repr=False, default=None)   # [T, H, d] uint16
    k_bf16: np.ndarray = field(repr=False, default=None)   # [nseq, L, d] uint16
    needle_pos: Optional[np.ndarray] = None               # [nseq, needles] planted positions


def _softmax_rows(x: np.ndarray) -> np.ndarray:
    z = x - x.max(axis=1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=1, keepdims=True)


def _ar1_keys(rng: np.random.Generator, nseq: int, L: int, d: int, rho: float, sigma: float) -> np.ndarray:
    """Stationary AR(1) per coordinate: k_0 = sigma*e_0, k_s = rho*k_{s-1} + sqrt(1-rho^2)*sigma*e_s."""
    from scipy.signal import lfilter

    out = np.empty((nseq, L, d), np.float32)
    c = np.sqrt(1.0 - rho * rho)
    for n in range(nseq):
        e = rng.standard_normal((L, d))
        e[0] /= c                    # makes the filter's first output sigma*e_0
        out[n] = lfilter([c * sigma], [1.0, -rho], e, axis=0).astype(np.float32)
    return out


def make_inputs(cfg, mode: str = "gauss", seed: Optional[int] = None, **overrides) -> Inputs:
    """Draw one seeded batch for ``cfg``.

    ``overrides`` replace fields of the config (e.g. ``L=4096, T=4, nseq=4``)
    for parity cases at reduced size; the caller keeps them consistent
    (prefill: T == L; one query per sequence: T == nseq). The seed defaults to
    1000+index (gauss) / 2000+index (grid).
    """
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    if overrides:
        cfg = Config(**{**cfg.__dict__, **overrides})
    if cfg.phase == "prefill" and cfg.T != cfg.L:
        raise ValueError("prefill: every position is a query (T == L)")
    if cfg.phase == "decode" and cfg.nseq > 1 and cfg.T != cfg.nseq:
        raise ValueError("decode over several sequences: one query per sequence (T == nseq)")
    if cfg.phase == "mtp" and (cfg.T % cfg.nseq or cfg.T // cfg.nseq > cfg.L):
        raise ValueError("multi-token decode: the same number (at most L) of queries per sequence")
    if cfg.nseq == 1 and cfg.phase == "decode" and cfg.q_len0 + cfg.T - 1 > cfg.L:
        raise ValueError("decode prefixes exceed the stored length")
    if seed is None:
        seed = (1000 if mode == "gauss" else 2000) + cfg.index
    rng = np.random.Generator(np.random.PCG64(seed))
    T, H, d, L, nseq = cfg.T, cfg.H, cfg.d, cfg.L, cfg.nseq
    q_seq, q_len = query_layout(cfg)
    sigma = 1.0 / np.sqrt(d)
    needle_pos = None
    if mode == "gauss":
        q = (rng.standard_normal((T, H, d)) * sigma).astype(np.float32)
        q = bf16_round(q)
        w = _softmax_rows(rng.standard_normal((T, H))).astype(np.float32)
        if cfg.ar1:
            k = _ar1_keys(rng, nseq, L, d, 0.9, sigma)
        else:
            k = (rng.standard_normal((nseq, L, d)) * sigma).astype(np.float32)
        if cfg.needles:
            needle_pos = np.zeros((nseq, cfg.needles), np.int64)
            for n in range(nseq):
                qs = np.nonzero(q_seq == n)[0]
                if cfg.phase == "prefill":
                    # a needle at s is aimed at a later query t* > s (which can see it)
                    # (query index t* sees tokens 0..t*)
                    pos = rng.choice(L - 1, size=cfg.needles, replace=False)
                    tq = np.array([rng.integers(s + 1, L) for s in pos])
                else:
                    pos = rng.choice(L, size=cfg.needles, replace=False)
                    tq = rng.choice(qs, size=cfg.needles)
                g = rng.integers(0, H, size=cfg.needles)
                for s, t, gg in zip(pos, tq, g):
                    v = q[t, gg].astype(np.float64)
                    k[n, s] = (4.0 * v / np.linalg.norm(v)).astype(np.float32)
                needle_pos[n] = pos
        k = bf16_round(k)
    elif mode == "grid":
        q = (rng.integers(-2, 3, size=(T, H, d)).astype(np.float32) * np.float32(1.0 / 16))
        w = (rng.integers(1, 5, size=(T, H)).astype(np.float32) * np.float32(0.25))
        k = (rng.integers(-2, 3, size=(nseq, L, d)).astype(np.float32) * np.float32(1.0 / 16))
    else:
        raise ValueError(f"unknown mode {mode!r}")
    return Inputs(cfg=cfg, mode=mode, seed=seed, q=q, w=w, k=k, q_seq=q_seq, q_len=q_len,
                  q_bf16=bf16_bits(q), k_bf16=bf16_bits(k), needle_pos=needle_pos)
