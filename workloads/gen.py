"""Seeded synthetic inputs for the TokenGate gated-prefill workloads.

This module only draws random numbers and lays them out.  It holds none of
the method's arithmetic (no scoring, normalisation, selection or attention),
so both the fp64 oracle and the HIP path can take their inputs from here.

Each workload stands in for a setting of the TokenGate paper ("TokenGate:
Adapting LLMs for Fast and Memory-Efficient Prefill with Learned Token
Pruning"): §3.1 splits the prompt into a request part that is never pruned
and a prunable document part; App. C.2 runs budgets of 64-8192 kept document
tokens; App. D.3 (Table 3) goes to 128k context on a Qwen3-1.7B backbone.
The pages' datasets are not used: every value below is a Gaussian or uniform
draw from ``numpy.random.default_rng``.

Conventions
-----------
* bf16 tensors are stored as ``uint16`` bit patterns, rounded from float32
  draws with round-to-nearest-even.  ``bf16_to_f64`` widens them exactly.
* ``w1`` has shape ``[h, d]``: row ``j`` holds the input weights of hidden
  unit ``j`` (the ``nn.Linear`` weight layout).
* ``wq/wk/wv`` have shape ``[d, H*dh]`` so that ``Q = X @ wq``.
* Layout of the prompt: every sequence is its document tokens followed by its
  prompt tokens (``prunable`` is 1 then 0).

Draw order per workload (one ``default_rng(seed)`` stream unless noted):
  prompt lengths (ragged batch only), x, w1, w2, wq, wk, wv, gain, temp,
  then workload-specific draws (budgets / preset scores).
Large Gaussian arrays (``x``) are drawn in fixed 2^22-element chunks, chunk
``i`` from ``default_rng(SeedSequence(seed).spawn(n_chunks)[i])``, so the
result does not depend on how many threads fill it.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Optional

import numpy as np

CHUNK = 1 << 22


# --------------------------------------------------------------------------
# bf16 helpers (storage format only)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (RNE); returns uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).reshape(-1).view(np.uint32)
    out = np.empty(u.shape, np.uint16)
    for s in range(0, u.size, CHUNK):
        v = u[s:s + CHUNK]
        t = (v >> 16) & np.uint32(1)
        t += np.uint32(0x7FFF)
        t += v
        t >>= 16
        out[s:s + CHUNK] = t
    return out.reshape(np.shape(a))


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return bf16_to_f32(bits).astype(np.float64)


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def _gauss_chunked(seed_seq: np.random.SeedSequence, n: int, std: float,
                   to_bf16: bool, threads: int = 8) -> np.ndarray:
    """n Gaussian draws N(0, std^2) as float32 (or bf16 bits)."""
    n_chunks = max(1, -(-n // CHUNK))
    kids = seed_seq.spawn(n_chunks)
    out = np.empty(n, np.uint16 if to_bf16 else np.float32)

    def fill(i):
        lo, hi = i * CHUNK, min(n, (i + 1) * CHUNK)
        g = np.random.default_rng(kids[i])
        buf = g.standard_normal(hi - lo, dtype=np.float32)
        if std != 1.0:
            buf *= np.float32(std)
        out[lo:hi] = f32_to_bf16_bits(buf) if to_bf16 else buf

    if n_chunks == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(min(threads, n_chunks)) as ex:
            list(ex.map(fill, range(n_chunks)))
    return out


# --------------------------------------------------------------------------
# workload description
# --------------------------------------------------------------------------
@dataclasses.dataclass
class Workload:
    name: str
    seed: int
    dtype: str                      # "f32" or "bf16"
    seq_doc: List[int]              # document (prunable) tokens per sequence
    seq_prompt: List[int]           # prompt (non-prunable) tokens per sequence
    d: int
    h: int
    hq: int
    hkv: int
    dh: int
    budgets: List[List[int]]        # one list of per-sequence K per call
    temp_lo: float = 1.0
    temp_hi: float = 1.0
    preset_scores: bool = False     # scores drawn directly (scorer not run)
    n_calls: int = 1

    @property
    def seqlens(self) -> List[int]:
        return [a + b for a, b in zip(self.seq_doc, self.seq_prompt)]

    @property
    def t_in(self) -> int:
        return sum(self.seqlens)

    @property
    def n_seq(self) -> int:
        return len(self.seq_doc)

    def cu_seqlens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.seqlens)]).astype(np.int32)

    def prunable(self) -> np.ndarray:
        parts = []
        for a, b in zip(self.seq_doc, self.seq_prompt):
            parts.append(np.ones(a, np.uint8))
            parts.append(np.zeros(b, np.uint8))
        return np.concatenate(parts)


def _ragged_prompt_lengths(rng: np.random.Generator, n: int) -> List[int]:
    # integer prompt length drawn uniformly from [256, 1024], inclusive
    return [int(v) for v in rng.integers(256, 1025, size=n)]


def describe(cfg: int) -> Workload:
    """Shapes of workload ``cfg`` (0..4); no large arrays are drawn."""
    if cfg == 0:
        return Workload("tiny-fp32-1k", 0, "f32", [960], [64], 256, 64, 4, 4, 64,
                        [[128]])
    if cfg == 1:
        return Workload("qwen3-1.7b-16k", 1, "bf16", [15872], [512], 2048, 256, 16, 8,
                        128, [[1984]], 0.8, 1.2)
    if cfg == 2:
        w = Workload("budget-sweep-32k", 2, "bf16", [32256], [512], 2048, 256, 16, 8,
                     128, [], 0.8, 1.2, preset_scores=True, n_calls=8)
        return w
    if cfg == 3:
        return Workload("qwen3-1.7b-128k", 3, "bf16", [130560], [512], 2048, 256, 16, 8,
                        128, [[8192]], 0.8, 1.2)
    if cfg == 4:
        lens = [8192, 24576, 49152, 65536]
        rng = np.random.default_rng(4)
        prompts = _ragged_prompt_lengths(rng, 4)
        docs = [L - p for L, p in zip(lens, prompts)]
        return Workload("ragged-varlen-4seq", 4, "bf16", docs, prompts, 2048, 256, 16, 8,
                        128, [[dd // 16 for dd in docs]], 0.8, 1.2)
    raise ValueError(f"unknown workload {cfg}")


def generate(cfg: int, *, with_x: bool = True, with_proj: bool = True) -> Dict[str, object]:
    """Draw every array of workload ``cfg``.

    Returns a dict with the Workload under ``"wl"`` and arrays:
    x, w1 (bf16 bits or f32), b1, w2 (f32), b2 (float), wq, wk, wv,
    gain, temp (f32, post-softplus effective values), prunable (u8),
    cu_seqlens (i32), budgets (list of int32 arrays, one per call) and,
    for the budget sweep, ``b_preset`` (f32).
    """
    wl = describe(cfg)
    rng = np.random.default_rng(wl.seed)
    bf = wl.dtype == "bf16"
    out: Dict[str, object] = {"wl": wl}
    if cfg == 4:
        _ragged_prompt_lengths(rng, 4)          # keep the draw order documented above
    t_in, d, h = wl.t_in, wl.d, wl.h
    # x: one child SeedSequence of the workload seed (chunked, thread-invariant)
    x_seq = np.random.SeedSequence([wl.seed, 1])
    if with_x:
        out["x"] = _gauss_chunked(x_seq, t_in * d, 1.0, bf).reshape(t_in, d)
    conv = (lambda a: f32_to_bf16_bits(a)) if bf else (lambda a: a)
    w1 = rng.standard_normal((h, d), dtype=np.float32) * np.float32(1.0 / math.sqrt(d))
    out["w1"] = conv(w1)
    out["b1"] = np.zeros(h, np.float32)
    out["w2"] = (rng.standard_normal(h, dtype=np.float32) *
                 np.float32(1.0 / math.sqrt(h))).astype(np.float32)
    out["b2"] = 0.0
    nq, nk = wl.hq * wl.dh, wl.hkv * wl.dh
    if with_proj:
        s = np.float32(1.0 / math.sqrt(d))
        out["wq"] = conv(rng.standard_normal((d, nq), dtype=np.float32) * s)
        out["wk"] = conv(rng.standard_normal((d, nk), dtype=np.float32) * s)
        out["wv"] = conv(rng.standard_normal((d, nk), dtype=np.float32) * s)
    else:
        # advance the stream exactly as if the projections had been drawn
        for cols in (nq, nk, nk):
            rng.standard_normal((d, cols), dtype=np.float32)
    out["gain"] = rng.uniform(0.5, 1.5, wl.hq).astype(np.float32)
    if wl.temp_lo == wl.temp_hi:
        out["temp"] = np.full(wl.hq, wl.temp_lo, np.float32)
    else:
        out["temp"] = rng.uniform(wl.temp_lo, wl.temp_hi, wl.hq).astype(np.float32)
    out["prunable"] = wl.prunable()
    out["cu_seqlens"] = wl.cu_seqlens()
    if wl.preset_scores:
        n_doc = wl.seq_doc[0]
        half = n_doc // 2                       # |P|/2, upper end of the budget range
        u = rng.uniform(0.0, math.log(half), wl.n_calls)
        ks = np.clip(np.rint(np.exp(u)), 1, half).astype(np.int32)
        wl.budgets = [[int(k)] for k in ks]
        # Gaussian scores of variance 2 on the bf16 grid (so exact ties occur),
        # then exactly +6.0 on 5% of document tokens chosen without replacement.
        sd = rng.standard_normal(n_doc, dtype=np.float32) * np.float32(math.sqrt(2.0))
        sd = bf16_to_f32(f32_to_bf16_bits(sd))
        n_spike = int(round(0.05 * n_doc))
        spikes = rng.choice(n_doc, size=n_spike, replace=False)
        sd[spikes] = np.float32(6.0)
        b = np.zeros(t_in, np.float32)
        b[:n_doc] = sd
        out["b_preset"] = b
    out["budgets"] = [np.asarray(kk, np.int32) for kk in wl.budgets]
    return out


def random_qkv(seed: int, t: int, hq: int, hkv: int, dh: int, bf16: bool = True):
    """Stand-in Q/K/V of a projected layer: N(0, 1) entries, the distribution
    that X @ W gives for X ~ N(0,1) rows and W ~ N(0, 1/d) weights.
    Used where projecting every row would be too slow for the host."""
    ss = np.random.SeedSequence([seed, 7])
    a, b, c = ss.spawn(3)
    q = _gauss_chunked(a, t * hq * dh, 1.0, bf16).reshape(t, hq, dh)
    k = _gauss_chunked(b, t * hkv * dh, 1.0, bf16).reshape(t, hkv, dh)
    v = _gauss_chunked(c, t * hkv * dh, 1.0, bf16).reshape(t, hkv, dh)
    return q, k, v


def digests(arrs: Dict[str, object]) -> Dict[str, str]:
    return {k: sha256(v)[:16] for k, v in arrs.items() if isinstance(v, np.ndarray)}
