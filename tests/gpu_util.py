"""Helpers for the GPU parity tests (marshalling and error measures only)."""
import functools
import math
import sys

import numpy as np
import torch

import oracle as O
from workloads import bf16_to_f64, f32_to_bf16_bits, generate

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None


def say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def f32_dev(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def i32_dev(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def u8_dev(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(DEV)


def to_f64(t: torch.Tensor) -> np.ndarray:
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return bf16_to_f64(t.view(torch.int16).cpu().numpy().view(np.uint16))
    return t.cpu().numpy().astype(np.float64)


def round_bf16(a: np.ndarray) -> np.ndarray:
    """fp64 -> bf16 bits (via fp32, RNE)."""
    return f32_to_bf16_bits(np.asarray(a, np.float64).astype(np.float32))


def rel_l2(got: np.ndarray, ref: np.ndarray) -> float:
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def score_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max_j |got - ref| / max(|ref_j|, rms(ref)); the parity bar is 1e-5."""
    floor = math.sqrt(float(np.mean(ref ** 2))) if ref.size else 1.0
    den = np.maximum(np.abs(ref), floor)
    return float(np.max(np.abs(got - ref) / den)) if ref.size else 0.0


def ref_score_chunked(x_bits_or_f32, w1, b1, w2, b2, bf16: bool, rows=65536):
    """Oracle scores of every row, evaluated in row chunks to bound memory."""
    T = x_bits_or_f32.shape[0]
    out = np.empty(T)
    w1d = bf16_to_f64(w1) if bf16 else np.asarray(w1, np.float64)
    for s in range(0, T, rows):
        xs = x_bits_or_f32[s:s + rows]
        xd = bf16_to_f64(xs) if bf16 else xs.astype(np.float64)
        out[s:s + rows] = O.ref_score(xd, w1d, b1, w2, b2)
    return out


@functools.lru_cache(maxsize=2)
def workload(cfg: int):
    return generate(cfg)
