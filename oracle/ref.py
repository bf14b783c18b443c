"""Plain fp64 CPU oracle of the TokenGate gated-prefill step.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call
this module: only the tests, the package smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code with the HIP library.

Source: "TokenGate: Adapting LLMs for Fast and Memory-Efficient Prefill with
Learned Token Pruning" (Patel, Ranjan, Stoica, Zaharia, Guestrin), cited
below as [TG] with its section and equation numbers.  Equation numbers are
recovered by order of appearance (Eq. 1-2 in §3, Eq. 3-4 in §4.1, Eq. 5-8 in
§4.2, Eq. 9-10 in §4.3).

Every function computes the plain definition in float64 with numpy; there
is no blocking, fusion or reordering beyond splitting query rows into
batches to bound memory.  Where the pages leave a step open, the reading is
named in the docstring (R-numbers match ``readings.py``).

Pinning status: every function here is pinned by the not-gpu tests against
closed forms, library routines (torch autograd for the backward), central
differences, independent formulations of the paper's equations or brute force -- except the two documented readings marked
"parity unpinned" in ``readings.py`` (the length factor of the temperature
and the values of epsilon in the score normalisation and in LN2), whose only
pinned consequence is that the length factor is 1 when nothing is pruned.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence, Tuple

import numpy as np

from . import readings as R


# ---------------------------------------------------------------------------
# gate module: scoring network and normalisation ([TG] §4.1, Eq. 3)
# ---------------------------------------------------------------------------
def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z * sigmoid(z) = z / (1 + e^-z)."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def ref_score(x: np.ndarray, w1: np.ndarray, b1: Optional[np.ndarray],
              w2: np.ndarray, b2: float) -> np.ndarray:
    """Raw gate scores b~_j = MLP_theta(a~_j^L), [TG] §4.1 Eq. 3 (left part).

    The pages call the scorer a small MLP without giving its shape (R4); the
    workloads fix it as d -> h (SiLU) -> 1 with biases:
        u_j  = SiLU(W1 x_j + b1)          (w1 is [h, d], row = hidden unit)
        b~_j = w2 . u_j + b2
    x holds the scorer's input rows a~^L = LN2(a^L) directly (R5).
    """
    x = np.asarray(x, dtype=np.float64)
    w1 = np.asarray(w1, dtype=np.float64)
    pre = x @ w1.T
    if b1 is not None:
        pre = pre + np.asarray(b1, dtype=np.float64)[None, :]
    u = silu(pre)
    return u @ np.asarray(w2, dtype=np.float64) + float(b2)


def ref_rmsnorm(a: np.ndarray, gamma: Optional[np.ndarray], eps: float) -> np.ndarray:
    """The block's second norm, a~ = LN2(a), [TG] §3 Eq. 1, read as the
    RMSNorm of the Qwen3 family (R22): each row divided by the root of its
    mean square plus eps, then scaled by gamma (None = ones)."""
    a = np.asarray(a, dtype=np.float64)
    r = np.sqrt(np.mean(a * a, axis=-1, keepdims=True) + float(eps))
    out = a / r
    if gamma is not None:
        out = out * np.asarray(gamma, dtype=np.float64)
    return out


def ref_score_prenorm(a: np.ndarray, gamma: Optional[np.ndarray], norm_eps: float,
                      w1: np.ndarray, b1: Optional[np.ndarray], w2: np.ndarray,
                      b2: float) -> np.ndarray:
    """Raw gate scores from the post-attention residual a^L itself:
    b~_j = MLP_theta(LN2(a_j^L)), [TG] §4.1 Eq. 3 with §3 Eq. 1's LN2 (R22)."""
    return ref_score(ref_rmsnorm(a, gamma, norm_eps), w1, b1, w2, b2)


def ref_normalise(b_raw: np.ndarray, prunable: np.ndarray, cu_seqlens: Sequence[int],
                  eps: float = R.EPS) -> Tuple[np.ndarray, np.ndarray]:
    """Normalised scores, [TG] §4.1 Eq. 3 (right part), per sequence s:

        r_s = sqrt( (1/|P_s|) * sum_{j in P_s} b~_j^2 + eps )     (R2: RMS)
        b_j = b~_j / r_s   for j in P_s,     b_j = 0 for j in N_s (prompt).

    A sequence with no prunable token has every b_j = 0 and r_s = 1.
    Returns (b, r) with r one value per sequence.
    """
    b_raw = np.asarray(b_raw, dtype=np.float64)
    prunable = np.asarray(prunable).astype(bool)
    b = np.zeros_like(b_raw)
    r = np.ones(len(cu_seqlens) - 1)
    for s in range(len(cu_seqlens) - 1):
        lo, hi = int(cu_seqlens[s]), int(cu_seqlens[s + 1])
        P = np.nonzero(prunable[lo:hi])[0] + lo
        if P.size == 0:
            continue
        mean_sq = np.mean(b_raw[P] ** 2)
        r[s] = math.sqrt(mean_sq + eps)
        b[P] = b_raw[P] / r[s]
    return b, r


# ---------------------------------------------------------------------------
# top-K selector ([TG] §4.1 Eq. 4)
# ---------------------------------------------------------------------------
def rank_order(values: np.ndarray, index: np.ndarray) -> np.ndarray:
    """Permutation that sorts candidates best-first under the strict order
    (value descending, index ascending), with -0.0 equal to +0.0 and NaN
    ranked below -inf (R11).  ``np.lexsort`` takes its last key as primary."""
    v = np.asarray(values, dtype=np.float64).copy()
    nan = np.isnan(v)
    v[nan] = 0.0
    v = v + 0.0                      # -0.0 -> +0.0
    return np.lexsort((np.asarray(index), -v, nan.astype(np.int8)))


def ref_select(b: np.ndarray, prunable: np.ndarray, cu_seqlens: Sequence[int],
               k: Sequence[int]):
    """Kept set S_s = top-K_{j in P_s}(b_j)  U  N_s, [TG] §4.1 Eq. 4.

    K counts prunable tokens only (R12): K' = min(K_s, |P_s|); K >= |P_s| keeps
    every document token, K = 0 keeps the prompt only; K < 0 is an error.
    Ties are broken by lower index (R11).  The kept tokens of each sequence
    are emitted in ascending original index (R14), sequences in input order.

    Returns (kept_idx, kept_pos, kept_b, kept_cu_seqlens):
      kept_idx -- global token index, kept_pos -- index within its sequence,
      kept_b   -- b at the kept token, kept_cu_seqlens -- offsets per sequence.
    """
    b = np.asarray(b)
    prunable = np.asarray(prunable).astype(bool)
    idx_all, cu = [], [0]
    for s in range(len(cu_seqlens) - 1):
        lo, hi = int(cu_seqlens[s]), int(cu_seqlens[s + 1])
        ks = int(k[s])
        if ks < 0:
            raise ValueError("budget K must be >= 0")
        seq = np.arange(lo, hi)
        P = seq[prunable[lo:hi]]
        Nset = seq[~prunable[lo:hi]]
        kp = min(ks, P.size)
        top = P[rank_order(b[P], P)[:kp]]
        S = np.sort(np.concatenate([top, Nset]))
        idx_all.append(S)
        cu.append(cu[-1] + S.size)
    kept_idx = np.concatenate(idx_all).astype(np.int64) if idx_all else np.zeros(0, np.int64)
    seq_of = np.searchsorted(np.asarray(cu_seqlens), kept_idx, side="right") - 1
    kept_pos = kept_idx - np.asarray(cu_seqlens)[seq_of]
    return kept_idx, kept_pos, b[kept_idx], np.asarray(cu, dtype=np.int64)


def ref_kept_sizes(cu_seqlens: Sequence[int], n_prunable: Sequence[int],
                   k: Sequence[int]) -> np.ndarray:
    """|S_s| = min(K_s, |P_s|) + |N_s| as offsets (Eq. 4 with R12)."""
    cu = [0]
    for s in range(len(cu_seqlens) - 1):
        n = int(cu_seqlens[s + 1]) - int(cu_seqlens[s])
        cu.append(cu[-1] + min(int(k[s]), int(n_prunable[s])) + n - int(n_prunable[s]))
    return np.asarray(cu, dtype=np.int64)


# ---------------------------------------------------------------------------
# compaction of the kept rows ([TG] §4.1: pruned residuals stop at layer L)
# ---------------------------------------------------------------------------
def ref_gather(src: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """X_S = X[S]: the kept rows, in kept order, copied unchanged."""
    return np.asarray(src)[np.asarray(idx, dtype=np.int64)].copy()


# ---------------------------------------------------------------------------
# token-gated attention ([TG] §4.2 Eq. 5-8)
# ---------------------------------------------------------------------------
def length_factor(m: np.ndarray, p: np.ndarray, mode: str = R.LEN_SCALE) -> np.ndarray:
    """The length term of the temperature in [TG] Eq. 7 (R6).

    m = kept keys visible to the query (itself included), p = the query's
    1-based original position in its sequence.
      "log_ratio": log m / log max(2, p)   (the reading used everywhere)
      "swap":      log p / log max(2, m)   (rejected alternative, for study)
      "off":       1
    """
    m = np.asarray(m, dtype=np.float64)
    p = np.asarray(p, dtype=np.float64)
    if mode == "log_ratio":
        return np.log(m) / np.log(np.maximum(2.0, p))
    if mode == "swap":
        return np.log(p) / np.log(np.maximum(2.0, m))
    if mode == "off":
        return np.ones_like(m)
    raise ValueError(mode)


def _softmax_rows(logits: np.ndarray) -> np.ndarray:
    mx = np.max(logits, axis=-1, keepdims=True)
    e = np.exp(logits - mx)
    return e / np.sum(e, axis=-1, keepdims=True)


def ref_gated_attn(q, k, v, kept_b, kept_pos, kept_cu, gain, temp,
                   sm_scale: Optional[float] = None, len_scale: str = R.LEN_SCALE,
                   rows: Optional[np.ndarray] = None, row_block: int = 512) -> np.ndarray:
    """Token-gated causal attention over the kept tokens, [TG] Eq. 8:

        alpha_ij = softmax_{j in S, j <= i} ( tau_i^h * ( s * q_i.k_j + gain_h * b_j ) )
        tau_i^h  = temp_h * length_factor(m_i, p_i)                (Eq. 7, R6)
        O_i^h    = sum_j alpha_ij v_j

    s = 1/sqrt(d_head) (R1); gain and temp are the post-softplus values (R7);
    query head h reads KV head floor(h / (Hq/Hkv)) (R9); causality is by
    original position, which equals compacted order because S is ascending
    (R10).  m_i = compacted index within the sequence + 1, p_i = kept_pos + 1.

    q: [T, Hq, dh], k/v: [T, Hkv, dh]; kept_b: [T]; kept_pos: [T] or None
    (None means length factor 1); kept_cu: [n_seq+1].
    ``rows``: optional global row indices to evaluate (others are left 0).
    Returns O: [T, Hq, dh] float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    kb = np.asarray(kept_b, dtype=np.float64)
    T, Hq, dh = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(dh) if sm_scale is None else float(sm_scale)
    out = np.zeros((T, Hq, dh))
    want = None if rows is None else set(int(r) for r in rows)
    for s in range(len(kept_cu) - 1):
        lo, hi = int(kept_cu[s]), int(kept_cu[s + 1])
        n = hi - lo
        if n == 0:
            continue
        a = np.arange(n)
        m = a + 1.0
        if kept_pos is None:
            lam = np.ones(n)
        else:
            p = np.asarray(kept_pos[lo:hi], dtype=np.float64) + 1.0
            lam = length_factor(m, p, len_scale)
        sel = a if want is None else np.array([r - lo for r in range(lo, hi) if r in want],
                                               dtype=np.int64)
        for h in range(Hq):
            kv = h // G
            K = k[lo:hi, kv, :]
            V = v[lo:hi, kv, :]
            bias = float(gain[h]) * kb[lo:hi]
            for c0 in range(0, sel.size, row_block):
                rr = sel[c0:c0 + row_block]
                if rr.size == 0:
                    continue
                last = int(rr.max()) + 1                  # keys beyond are all masked
                z = scale * (q[lo + rr, h, :] @ K[:last].T) + bias[None, :last]
                tau = float(temp[h]) * lam[rr]
                logits = tau[:, None] * z
                logits[np.arange(last)[None, :] > rr[:, None]] = -np.inf
                out[lo + rr, h, :] = _softmax_rows(logits) @ V[:last]
    return out


def ref_gated_attn_lse2(q, k, kept_b, kept_pos, kept_cu, gain, temp,
                        sm_scale: Optional[float] = None, len_scale: str = R.LEN_SCALE) -> np.ndarray:
    """The softmax normaliser of [TG] Eq. 8 per query row and head, in base 2:
    lse2[i, h] = log2 sum_{j in S, j <= i} exp(tau_i^h (s q_i.k_j + gain_h b_j)),
    the logits exactly as in ref_gated_attn.  alpha_ij = 2^(logit_ij log2 e -
    lse2_i) is then the attention weight.  Returns [T, Hq] float64 (rows past
    kept_cu[-1] are 0)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    kb = np.asarray(kept_b, dtype=np.float64)
    T, Hq, dh = q.shape
    G = Hq // k.shape[1]
    scale = 1.0 / math.sqrt(dh) if sm_scale is None else float(sm_scale)
    out = np.zeros((T, Hq))
    for s in range(len(kept_cu) - 1):
        lo, hi = int(kept_cu[s]), int(kept_cu[s + 1])
        n = hi - lo
        if n == 0:
            continue
        m = np.arange(n) + 1.0
        lam = np.ones(n) if kept_pos is None else length_factor(
            m, np.asarray(kept_pos[lo:hi], dtype=np.float64) + 1.0, len_scale)
        for h in range(Hq):
            z = scale * (q[lo:hi, h, :] @ k[lo:hi, h // G, :].T) + float(gain[h]) * kb[None, lo:hi]
            logits = (float(temp[h]) * lam)[:, None] * z
            logits[np.arange(n)[None, :] > np.arange(n)[:, None]] = -np.inf
            mx = np.max(logits, axis=1)
            out[lo:hi, h] = (mx + np.log(np.sum(np.exp(logits - mx[:, None]), axis=1))) / math.log(2.0)
    return out


# --- independent formulations used to pin ref_gated_attn ------------------
def ref_gated_attn_masked(q_full, k_full, v_full, b_full, keep_mask, cu_seqlens, gain, temp,
                          sm_scale=None, len_scale: str = R.LEN_SCALE):
    """Mask form of [TG] Eq. 8 on the full, uncompacted sequence: keys outside S
    get -inf, m_i = #{j in S_s : j <= i}, p_i = i - start + 1; evaluated on the
    rows of S only (other rows are returned as NaN)."""
    q_full = np.asarray(q_full, np.float64)
    k_full = np.asarray(k_full, np.float64)
    v_full = np.asarray(v_full, np.float64)
    N, Hq, dh = q_full.shape
    G = Hq // k_full.shape[1]
    scale = 1.0 / math.sqrt(dh) if sm_scale is None else sm_scale
    out = np.full((N, Hq, dh), np.nan)
    keep_mask = np.asarray(keep_mask).astype(bool)
    for s in range(len(cu_seqlens) - 1):
        lo, hi = int(cu_seqlens[s]), int(cu_seqlens[s + 1])
        km = keep_mask[lo:hi]
        if not km.any():                             # no kept rows: nothing to evaluate
            continue
        counts = np.cumsum(km)                       # m_i for every position
        pos = np.arange(1, hi - lo + 1, dtype=np.float64)
        lam = length_factor(counts.astype(np.float64).clip(min=1), pos, len_scale)
        for h in range(Hq):
            kv = h // G
            z = scale * q_full[lo:hi, h] @ k_full[lo:hi, kv].T + gain[h] * b_full[lo:hi][None, :]
            logits = (temp[h] * lam)[:, None] * z
            allowed = np.tril(np.ones((hi - lo, hi - lo), bool)) & km[None, :]
            logits = np.where(allowed, logits, -np.inf)
            rows = np.nonzero(km)[0]
            out[lo + rows, h] = _softmax_rows(logits[rows]) @ v_full[lo:hi, kv]
    return out


def ref_gated_attn_multiplicative(q, k, v, kept_b, kept_pos, kept_cu, gain, temp,
                                  sm_scale=None, len_scale: str = R.LEN_SCALE):
    """[TG] Eq. 5 with the head-wise gate of Eq. 6 and the temperature of Eq. 7
    applied as a power of the gate value:

        g_j^h  = softmax_{j in S}( gain_h * b_j )              (over the whole S_s)
        alpha_ij ∝ exp(tau_i * s * q_i.k_j) * (g_j^h)^tau_i,   j <= i

    Equal to Eq. 8 because the softmax normaliser of g is constant in j."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    T, Hq, dh = q.shape
    G = Hq // k.shape[1]
    scale = 1.0 / math.sqrt(dh) if sm_scale is None else sm_scale
    out = np.zeros_like(q)
    for s in range(len(kept_cu) - 1):
        lo, hi = int(kept_cu[s]), int(kept_cu[s + 1])
        n = hi - lo
        if n == 0:
            continue
        m = np.arange(1, n + 1, dtype=np.float64)
        p = np.asarray(kept_pos[lo:hi], np.float64) + 1.0
        lam = length_factor(m, p, len_scale)
        for h in range(Hq):
            gb = gain[h] * np.asarray(kept_b[lo:hi], np.float64)
            g = np.exp(gb - gb.max())
            g = g / g.sum()
            tau = temp[h] * lam
            for i in range(n):
                w = np.exp(tau[i] * scale * (k[lo:lo + i + 1, h // G] @ q[lo + i, h]))
                w = w * g[:i + 1] ** tau[i]
                out[lo + i, h] = (w / w.sum()) @ v[lo:lo + i + 1, h // G]
    return out


def ref_gated_attn_loggate(q, k, v, kept_b, kept_pos, kept_cu, gain, temp,
                           sm_scale=None, len_scale: str = R.LEN_SCALE):
    """Additive-bias form: logits tau_i * (s q.k + gain_h * log g_j) with
    g = softmax_{j in S}(b) taken once over the whole kept set S_s."""
    q = np.asarray(q, np.float64)
    kb = np.asarray(kept_b, np.float64)
    T = q.shape[0]
    logg = np.zeros(T)
    for s in range(len(kept_cu) - 1):
        lo, hi = int(kept_cu[s]), int(kept_cu[s + 1])
        if hi > lo:
            z = kb[lo:hi]
            mx = z.max()
            logg[lo:hi] = z - (mx + math.log(np.sum(np.exp(z - mx))))
    return ref_gated_attn(q, k, v, logg, kept_pos, kept_cu, gain, temp, sm_scale, len_scale)


def ref_gated_attn_bruteforce(q, k, v, kept_b, kept_pos, kept_cu, gain, temp,
                              sm_scale=None, len_scale: str = R.LEN_SCALE):
    """Explicit scalar loops over (sequence, head, query, key), for tiny T."""
    T, Hq, dh = np.shape(q)
    Hkv = np.shape(k)[1]
    scale = 1.0 / math.sqrt(dh) if sm_scale is None else sm_scale
    out = np.zeros((T, Hq, dh))
    for s in range(len(kept_cu) - 1):
        lo, hi = int(kept_cu[s]), int(kept_cu[s + 1])
        for h in range(Hq):
            kvh = (h * Hkv) // Hq
            for i in range(lo, hi):
                m = i - lo + 1
                p = int(kept_pos[i]) + 1
                if len_scale == "log_ratio":
                    lam = math.log(m) / math.log(max(2, p))
                elif len_scale == "swap":
                    lam = math.log(p) / math.log(max(2, m))
                else:
                    lam = 1.0
                tau = float(temp[h]) * lam
                logits = []
                for j in range(lo, i + 1):
                    dot = 0.0
                    for e in range(dh):
                        dot += float(q[i][h][e]) * float(k[j][kvh][e])
                    logits.append(tau * (scale * dot + float(gain[h]) * float(kept_b[j])))
                mx = max(logits)
                w = [math.exp(t - mx) for t in logits]
                tot = sum(w)
                for e in range(dh):
                    acc = 0.0
                    for jj, j in enumerate(range(lo, i + 1)):
                        acc += w[jj] * float(v[j][kvh][e])
                    out[i, h, e] = acc / tot
    return out


# ---------------------------------------------------------------------------
# backward of token-gated attention ([TG] §4.3: the gate's scores receive a
# gradient through the attention of Eq. 8)
# ---------------------------------------------------------------------------
def ref_gated_attn_bwd(q, k, v, kept_b, kept_pos, kept_cu, gain, temp, dout,
                       sm_scale: Optional[float] = None, len_scale: str = R.LEN_SCALE,
                       row_block: int = 512, error_scales: bool = False):
    """Gradients of L = sum(O * dout) through the token-gated attention of
    [TG] Eq. 8 (gain of Eq. 6, temperature of Eq. 7), by the chain rule on

        z_ij = s q_i.k_j + gain_h b_j,   l_ij = tau_i z_ij   (j <= i),
        P_i  = softmax_j(l_i),           O_i  = sum_j P_ij v_j:

        dP_ij  = dout_i . v_j
        dl_ij  = P_ij (dP_ij - sum_j' P_ij' dP_ij')
        dv_j   = sum_i P_ij dout_i
        dq_i   = s tau_i sum_j dl_ij k_j
        dk_j   = s sum_i tau_i dl_ij q_i
        db_j   = sum_{h,i} tau_i gain_h dl_ij          (the gate's gradient path)
        dgain_h = sum_{i,j} tau_i b_j dl_ij
        dtemp_h = sum_{i,j} lambda_i z_ij dl_ij          (tau_i = temp_h lambda_i)

    KV gradients add up over the query heads that share a KV head (R9);
    tau_i's length factor depends on positions only, so it carries no
    gradient.  Query rows are processed in blocks of ``row_block``.
    Returns (dq [T,Hq,dh], dk [T,Hkv,dh], dv [T,Hkv,dh], db [T], dgain [Hq],
    dtemp [Hq]), float64.

    dgain and dtemp sum terms of both signs over every (query, key) pair
    (each row of dl sums to zero).  With ``error_scales`` the function also
    returns, per head, the sums over the pairs of |weight| * P (|dP| + |D|)
    (weight tau b for gain, lambda z for temperature): a rounding error of
    relative size u in dP or D moves each sum by at most u times that scale,
    which is what a tolerance for a finite-precision result is measured by.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(dout, dtype=np.float64)
    kb = np.asarray(kept_b, dtype=np.float64)
    T, Hq, dh = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(dh) if sm_scale is None else float(sm_scale)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    db = np.zeros(T)
    dgain, dtemp = np.zeros(Hq), np.zeros(Hq)
    sgain, stemp = np.zeros(Hq), np.zeros(Hq)
    for s in range(len(kept_cu) - 1):
        lo, hi = int(kept_cu[s]), int(kept_cu[s + 1])
        n = hi - lo
        if n == 0:
            continue
        a = np.arange(n)
        if kept_pos is None:
            lam = np.ones(n)
        else:
            lam = length_factor(a + 1.0, np.asarray(kept_pos[lo:hi], np.float64) + 1.0, len_scale)
        for h in range(Hq):
            kvh = h // G
            K, V = k[lo:hi, kvh, :], v[lo:hi, kvh, :]
            g = float(gain[h])
            for r0 in range(0, n, row_block):
                rr = a[r0:r0 + row_block]
                last = int(rr[-1]) + 1
                Q, dO = q[lo + rr, h, :], do[lo + rr, h, :]
                tau = float(temp[h]) * lam[rr]
                z = scale * (Q @ K[:last].T) + g * kb[lo:lo + last][None, :]
                causal = np.arange(last)[None, :] <= rr[:, None]
                logits = np.where(causal, tau[:, None] * z, -np.inf)
                P = _softmax_rows(logits)
                dP = dO @ V[:last].T
                dl = P * (dP - np.sum(P * dP, axis=1, keepdims=True))
                dv[lo:lo + last, kvh, :] += P.T @ dO
                tdl = tau[:, None] * dl
                dq[lo + rr, h, :] = scale * (tdl @ K[:last])
                dk[lo:lo + last, kvh, :] += scale * (tdl.T @ Q)
                db[lo:lo + last] += g * np.sum(tdl, axis=0)
                dgain[h] += float(np.sum(tdl * kb[lo:lo + last][None, :]))
                zc = np.where(causal, z, 0.0)
                dtemp[h] += float(np.sum(lam[rr][:, None] * zc * dl))
                if error_scales:
                    sens = P * (np.abs(dP) + np.abs(np.sum(P * dP, axis=1, keepdims=True)))
                    sgain[h] += float(np.sum(np.abs(tau[:, None] * kb[lo:lo + last][None, :]) * sens))
                    stemp[h] += float(np.sum(np.abs(lam[rr][:, None] * zc) * sens))
    if error_scales:
        return dq, dk, dv, db, dgain, dtemp, sgain, stemp
    return dq, dk, dv, db, dgain, dtemp


def ref_gated_attn_bwd_rows(q, k, v, kept_b, kept_pos, kept_cu, gain, temp, dout,
                            query_rows, key_rows, sm_scale: Optional[float] = None,
                            len_scale: str = R.LEN_SCALE, row_block: int = 512):
    """The gradients of ref_gated_attn_bwd at a sample of rows, for inputs
    too large for every gradient row: dq at ``query_rows`` and dk, dv, db at
    ``key_rows`` (global row indices).  The same definitions, evaluated the
    same way block by block: every query row's softmax and D_i still need all
    of its keys, but only the sampled rows of dq and columns of the dk, dv
    and db sums are formed.  Returns (dq [len(query_rows), Hq, dh],
    dk [len(key_rows), Hkv, dh], dv [len(key_rows), Hkv, dh], db [len(key_rows)]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(dout, dtype=np.float64)
    kb = np.asarray(kept_b, dtype=np.float64)
    T, Hq, dh = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(dh) if sm_scale is None else float(sm_scale)
    qrows = np.asarray(query_rows, dtype=np.int64)
    krows = np.asarray(key_rows, dtype=np.int64)
    dq = np.zeros((len(qrows), Hq, dh))
    dk = np.zeros((len(krows), Hkv, dh))
    dv = np.zeros((len(krows), Hkv, dh))
    db = np.zeros(len(krows))
    for s in range(len(kept_cu) - 1):
        lo, hi = int(kept_cu[s]), int(kept_cu[s + 1])
        n = hi - lo
        if n == 0:
            continue
        qsel = np.nonzero((qrows >= lo) & (qrows < hi))[0]     # positions in query_rows
        ksel = np.nonzero((krows >= lo) & (krows < hi))[0]
        if qsel.size == 0 and ksel.size == 0:
            continue
        a = np.arange(n)
        if kept_pos is None:
            lam = np.ones(n)
        else:
            lam = length_factor(a + 1.0, np.asarray(kept_pos[lo:hi], np.float64) + 1.0, len_scale)
        kl = krows[ksel] - lo                                    # sampled keys, local
        for h in range(Hq):
            kvh = h // G
            K, V = k[lo:hi, kvh, :], v[lo:hi, kvh, :]
            g = float(gain[h])
            for r0 in range(0, n, row_block):
                rr = a[r0:r0 + row_block]
                last = int(rr[-1]) + 1
                Q, dO = q[lo + rr, h, :], do[lo + rr, h, :]
                tau = float(temp[h]) * lam[rr]
                z = scale * (Q @ K[:last].T) + g * kb[lo:lo + last][None, :]
                causal = np.arange(last)[None, :] <= rr[:, None]
                logits = np.where(causal, tau[:, None] * z, -np.inf)
                P = _softmax_rows(logits)
                dP = dO @ V[:last].T
                dl = P * (dP - np.sum(P * dP, axis=1, keepdims=True))
                tdl = tau[:, None] * dl
                for pos in qsel:
                    i = int(qrows[pos]) - lo
                    if r0 <= i < r0 + len(rr):
                        dq[pos, h, :] = scale * (tdl[i - r0] @ K[:last])
                for m, j in zip(ksel, kl):
                    if j < last:
                        dv[m, kvh, :] += P[:, j] @ dO
                        dk[m, kvh, :] += scale * (tdl[:, j] @ Q)
                        db[m] += g * float(np.sum(tdl[:, j]))
    return dq, dk, dv, db


# ---------------------------------------------------------------------------
# backward of the gate's scorer ([TG] §4.1 Eq. 3 read backwards: the gradient
# that reaches the kept scores b through the attention flows on to the
# scoring network's weights)
# ---------------------------------------------------------------------------
def ref_score_bwd(x, w1, b1, w2, b2, prunable, cu_seqlens, kept_idx, kept_cu, db_kept,
                  eps: float = R.EPS, error_scales: bool = False):
    """Gradients of L = sum_r db_kept[r] * b[kept_idx[r]] w.r.t. the scorer's
    input rows and parameters, by the chain rule through Eq. 3:

      normalisation, per sequence s with prunable set P and
      r = sqrt(mean_P b~^2 + eps), C = sum_{j in P} db_j b~_j:
        db~_k = db_k / r - b~_k C / (|P| r^3)      for k in P
        db~_k = 0                                   for prompt tokens (b := 0)
      (db_j is db_kept at kept tokens and 0 at pruned ones: the selection
      passes no gradient, and pruned tokens still feel r.)
      scorer, z = W1 x + b1, u = SiLU(z), b~ = w2 . u + b2:
        dz = db~ w2 * SiLU'(z),  SiLU'(z) = sigma(z) (1 + z (1 - sigma(z)))
        dW1 = sum_j dz_j x_j^T,  db1 = sum_j dz_j,  dw2 = sum_j db~_j u_j,
        db2 = sum_j db~_j,       dx_j = W1^T dz_j.

    x [T, d], w1 [h, d], b1 [h] or None, w2 [h], b2 scalar; kept_idx,
    kept_cu, db_kept as returned by the selector and the attention's backward.
    Returns (dx [T, d], dw1 [h, d], db1 [h], dw2 [h], db2), float64; with
    ``error_scales`` also sum_k |db~_k|, the scale of db2's sum of terms of
    both signs (a finite-precision result is measured against it).
    """
    x = np.asarray(x, dtype=np.float64)
    w1 = np.asarray(w1, dtype=np.float64)
    w2 = np.asarray(w2, dtype=np.float64)
    T = x.shape[0]
    pre = x @ w1.T
    if b1 is not None:
        pre = pre + np.asarray(b1, dtype=np.float64)[None, :]
    sig = 1.0 / (1.0 + np.exp(-pre))
    u = pre * sig
    b_raw = u @ w2 + float(b2)
    db = np.zeros(T)
    db[np.asarray(kept_idx, dtype=np.int64)] = np.asarray(db_kept, dtype=np.float64)
    prunable = np.asarray(prunable).astype(bool)
    dbt = np.zeros(T)
    for s in range(len(cu_seqlens) - 1):
        lo, hi = int(cu_seqlens[s]), int(cu_seqlens[s + 1])
        P = np.nonzero(prunable[lo:hi])[0] + lo
        if P.size == 0:
            continue
        r = math.sqrt(np.mean(b_raw[P] ** 2) + eps)
        C = float(np.sum(db[P] * b_raw[P]))
        dbt[P] = db[P] / r - b_raw[P] * C / (P.size * r ** 3)
    dz = dbt[:, None] * w2[None, :] * sig * (1.0 + pre * (1.0 - sig))
    out = (dz @ w1, dz.T @ x, dz.sum(axis=0), u.T @ dbt, float(dbt.sum()))
    if error_scales:
        return out + (float(np.sum(np.abs(dbt))),)
    return out


def ref_score_prenorm_bwd(a, gamma, norm_eps: float, w1, b1, w2, b2, prunable, cu_seqlens,
                          kept_idx, kept_cu, db_kept, eps: float = R.EPS,
                          error_scales: bool = False):
    """The same gradients when the scorer reads the residual a^L and applies
    the block's second norm itself, b~_j = MLP(LN2(a_j)) ([TG] §4.1 Eq. 3
    with §3 Eq. 1's LN2, read as an RMSNorm, R22).  With
    r_j = sqrt(mean_c a_jc^2 + norm_eps) and x_j = gamma * a_j / r_j,
    ref_score_bwd at x gives dx, dW1, db1, dw2, db2; the norm then passes
        dgamma = sum_j dx_j * a_j / r_j
        da_j   = gamma * dx_j / r_j - a_j (sum_c gamma_c dx_jc a_jc) / (d r_j^3)
    (the derivative of a_j / r_j is I / r_j - a_j a_j^T / (d r_j^3)).
    gamma None means ones (dgamma is still returned).
    Returns (da [T, d], dw1 [h, d], dgamma [d], db1 [h], dw2 [h], db2); with
    ``error_scales`` also ref_score_bwd's scale of db2.
    """
    a = np.asarray(a, dtype=np.float64)
    d = a.shape[1]
    g = np.ones(d) if gamma is None else np.asarray(gamma, dtype=np.float64)
    r = np.sqrt(np.mean(a * a, axis=1) + float(norm_eps))
    x = ref_rmsnorm(a, g, norm_eps)
    got = ref_score_bwd(x, w1, b1, w2, b2, prunable, cu_seqlens, kept_idx, kept_cu, db_kept,
                        eps=eps, error_scales=error_scales)
    dx, dw1, db1, dw2, db2 = got[:5]
    dgamma = np.sum(dx * a / r[:, None], axis=0)
    gdx = dx * g[None, :]
    da = gdx / r[:, None] - a * (np.sum(gdx * a, axis=1) / (d * r ** 3))[:, None]
    out = (da, dw1, dgamma, db1, dw2, db2)
    return out + tuple(got[5:])


# ---------------------------------------------------------------------------
# harness-level projection (outside the four library calls)
# ---------------------------------------------------------------------------
def ref_project(xs: np.ndarray, wq, wk, wv, hq: int, hkv: int, dh: int):
    """Q = X_S Wq, K = X_S Wk, V = X_S Wv in fp64, reshaped to heads."""
    xs = np.asarray(xs, np.float64)
    T = xs.shape[0]
    q = (xs @ np.asarray(wq, np.float64)).reshape(T, hq, dh)
    k = (xs @ np.asarray(wk, np.float64)).reshape(T, hkv, dh)
    v = (xs @ np.asarray(wv, np.float64)).reshape(T, hkv, dh)
    return q, k, v


def ref_rope(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotary position embedding, rotate-half layout (R23): for every head
    vector x of row t (x[t, h, :], length dh) and pair e < dh/2 with angle
    a = pos[t] * theta**(-2e/dh):
        x[e]        -> x[e] cos a - x[e + dh/2] sin a
        x[e + dh/2] -> x[e + dh/2] cos a + x[e] sin a."""
    x = np.asarray(x, np.float64)
    dh = x.shape[-1]
    half = dh // 2
    inv = float(theta) ** (-2.0 * np.arange(half) / dh)
    ang = np.asarray(pos, np.float64)[:, None] * inv[None, :]          # [T, dh/2]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    lo, hi = x[..., :half], x[..., half:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


def ref_project_qk_rope(xs: np.ndarray, wq, wk, wv, hq: int, hkv: int, dh: int, pos,
                        q_norm: Optional[np.ndarray], k_norm: Optional[np.ndarray],
                        norm_eps: float, theta: float):
    """The projections with the Qwen3-style per-head RMSNorm of q and k and
    the rotary embedding at the kept tokens' original positions (R23): Q, K, V
    as in ref_project, then q <- RMSNorm_dh(q) * q_norm, k <- RMSNorm_dh(k) *
    k_norm (skipped when the weight is None), then RoPE on q and k (skipped
    when theta <= 0).  v is the plain projection."""
    q, k, v = ref_project(xs, wq, wk, wv, hq, hkv, dh)
    if q_norm is not None:
        q = ref_rmsnorm(q, q_norm, norm_eps)
    if k_norm is not None:
        k = ref_rmsnorm(k, k_norm, norm_eps)
    if theta > 0:
        q = ref_rope(q, pos, theta)
        k = ref_rope(k, pos, theta)
    return q, k, v


# ---------------------------------------------------------------------------
# whole step
# ---------------------------------------------------------------------------
def ref_gate(x, w1, b1, w2, b2, prunable, cu_seqlens, k, eps: float = R.EPS):
    """Score -> normalise -> select -> gather for one gated layer."""
    b_raw = ref_score(x, w1, b1, w2, b2)
    b, _ = ref_normalise(b_raw, prunable, cu_seqlens, eps)
    kept_idx, kept_pos, kept_b, kept_cu = ref_select(b.astype(np.float32), prunable,
                                                     cu_seqlens, k)
    return b_raw, b, kept_idx, kept_pos, kept_b, kept_cu, ref_gather(x, kept_idx)
