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
    """max_j |got - ref| / max(|ref_j|, rms(ref)); the parity bar is 1e-5.

    When every reference value is 0 (a sequence of prompt tokens only: their
    normalised score is set to 0 by Eq. 3) there is no scale to divide by,
    and the result must be exactly 0: the error is 0 if it is, inf if not."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    floor = math.sqrt(float(np.mean(ref ** 2)))
    if not floor > 0.0:
        return 0.0 if np.array_equal(got, ref) else math.inf
    den = np.maximum(np.abs(ref), floor)
    return float(np.max(np.abs(got - ref) / den))


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


# The forward's lse2 (log2 of the softmax normaliser) sums probabilities that
# were rounded to bf16 before the sum.  bf16 keeps 8 significant bits, so
# round-to-nearest is within 2^-8 relative per term, and so is the sum of
# such positive terms: its base-2 log is within log2(1 + 2^-8) = 5.6e-3 of
# the exact one.  The fp32 logits add an error proportional to their size
# (the gain term enters as a bf16 hi/lo pair, 2^-18 relative): the bar is
# |got - ref| <= LSE2_ABS + LSE2_REL |ref|.
LSE2_ABS = math.log2(1.0 + 2.0 ** -8)
LSE2_REL = 1e-5


def lse2_excess(got, ref):
    """max over entries of |got - ref| - LSE2_REL |ref| (to compare with LSE2_ABS)."""
    return float(np.max(np.abs(got - ref) - LSE2_REL * np.abs(ref)))


# Attention parity figures.  The global rel-L2 is the bar the workloads are
# quoted at; per head and per row the same error is measured again, so that
# a defect confined to one head (each head has its own gain and temperature,
# Eq. 6-7) or to one block of query rows cannot hide inside the global norm.
ATTN_BARS = {
    "bf16": dict(glob=1e-2, head=1e-2, row=2e-2),
    "f32": dict(glob=1e-5, head=1e-5, row=1e-4),
}


def attn_errors(got: np.ndarray, ref: np.ndarray) -> dict:
    """got, ref: [rows, heads, dh].  Global, worst per-head and worst per-row
    rel-L2, and the largest absolute difference."""
    d = got - ref
    rn = np.linalg.norm(ref)
    head_ref = np.sqrt(np.sum(ref ** 2, axis=(0, 2)))
    head_err = np.sqrt(np.sum(d ** 2, axis=(0, 2)))
    row_ref = np.sqrt(np.sum(ref ** 2, axis=(1, 2)))
    row_err = np.sqrt(np.sum(d ** 2, axis=(1, 2)))
    tiny = 1e-300
    return dict(glob=float(np.linalg.norm(d) / max(rn, tiny)),
                head=float(np.max(head_err / np.maximum(head_ref, tiny), initial=0.0)),
                row=float(np.max(row_err / np.maximum(row_ref, tiny), initial=0.0)),
                max_abs=float(np.max(np.abs(d), initial=0.0)))


def check_attn(got: np.ndarray, ref: np.ndarray, dtype: str, tag: str, bars=("glob", "head", "row")):
    """Print every figure and assert the chosen bars for `dtype`."""
    e = attn_errors(got, ref)
    say(f"attn {tag}: rel-L2 {e['glob']:.3e}, worst head {e['head']:.3e}, "
        f"worst row {e['row']:.3e}, max abs {e['max_abs']:.3e}")
    lim = ATTN_BARS[dtype]
    for b in bars:
        assert e[b] <= lim[b], f"{tag}: {b} rel-L2 {e[b]:.3e} > {lim[b]:.0e}"
    assert np.all(np.isfinite(got)), f"{tag}: non-finite output"
    return e
