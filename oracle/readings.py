"""Readings the oracle takes where the TokenGate pages are silent, garbled or
ambiguous.  TEST INFRASTRUCTURE ONLY (see ``oracle/ref.py``).

R1  logit scale: the extracted text prints q.k / d_head; read as 1/sqrt(d_head)
    (scaled dot-product attention; §3 Eq. 2 and §4.2 Eq. 8).
R2  Eq. 3 normaliser: read as the RMS, b~ / sqrt(mean_P b~^2 + eps).
R3  eps: not given; EPS below (a parameter of every scoring call).
R4  scorer shape: d -> h (SiLU) -> 1 with biases, from the workloads.
R5  scorer input: the workloads' hidden rows are a~^L = LN2(a^L) already.
R6  Eq. 7 symbols m_i, p_i (undefined on the pages): m_i = kept keys visible
    to query i including itself, p_i = its 1-based original position.
    LEN_SCALE = "log_ratio" gives tau_i = temp_h * log m_i / log max(2, p_i).
    PARITY UNPINNED beyond its consequence tau = temp when nothing is pruned.
R7  gain, temp are post-softplus positive values, one per query head.
R8  gain placement: Eq. 8 literally; the Eq. 5/6 multiplicative form and the
    additive gain * log softmax(b) form give the same weights (pinned).
R9  GQA: query head h reads KV head floor(h / (Hq / Hkv)).
R10 causality by original position == compacted order (S is ascending).
R11 selection order: (b descending, index ascending); -0.0 == +0.0; NaN ranks
    below -inf.
R12 K counts prunable tokens; K >= |P| keeps all of P; K = 0 keeps only the
    prompt; K < 0 is an error.
R13 prompt tokens carry b = 0 and take part in every softmax.
R14 kept tokens are emitted in ascending original index per sequence.
R20 selection runs on the normalised scores rounded to fp32.
R21 a decode step over a (pruned) cache is the last query row of the prefill
    attention over the cache rows, with the new token's key and value
    appended as the last row: m = cache length, p = its original position + 1,
    and generated tokens carry b = 0 like prompt tokens (neither is pruned).
R22 LN2 (named, not defined, in §3 Eq. 1) is the RMSNorm of the Qwen3 family:
    a / sqrt(mean(a^2) + eps) * gamma per row; eps is passed explicitly
    (PARITY UNPINNED as a value, like EPS).
R23 the projections of the kept rows (before the gated attention) may apply
    the Qwen3 family's per-head RMSNorm to q and k (over head_dim, one
    [head_dim] weight shared by all heads of q, another for k) and then the
    rotary embedding in the rotate-half layout at each kept token's original
    position in its sequence: pair (e, e + dh/2) of a head rotates by
    pos * theta^(-2e/dh).  Neither is on the pages; the oracle's form is
    pinned by an independent complex-number rotation, by the relative-position
    property of rotated dot products and by the norm's closed forms.
EPS is PARITY UNPINNED (a choice, passed explicitly to both sides).
"""
EPS = 1e-6
LEN_SCALE = "log_ratio"
