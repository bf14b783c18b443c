"""Pins of the fp64 oracle against what the TokenGate pages and plain
mathematics fix: closed forms, library routines, independent formulations of
the paper's equations, invariants and brute force.  CPU only."""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
from hypothesis import given, settings
from hypothesis import strategies as st

import oracle as O
from oracle import readings as R
from workloads import generate

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed=0):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------------------
# scoring network ([TG] §4.1 Eq. 3, scorer shape from the workloads)
# ---------------------------------------------------------------------------
def test_silu_special_values():
    assert O.silu(0.0) == 0.0
    assert O.silu(1.0) == pytest.approx(1.0 / (1.0 + math.exp(-1.0)), rel=1e-15)
    assert O.silu(-1.0) == pytest.approx(-1.0 / (1.0 + math.e), rel=1e-15)
    assert O.silu(800.0) == 800.0          # sigmoid saturates to 1
    assert O.silu(-800.0) == 0.0           # e^800 overflows: z / inf = -0


def test_score_one_hot_picks_silu_of_one_input():
    rng = _rng(1)
    T, d, h = 37, 12, 5
    x = rng.standard_normal((T, d))
    w1 = np.zeros((h, d))
    w1[3, 7] = 1.0                      # hidden unit 3 reads input 7
    w2 = np.zeros(h)
    w2[3] = 1.0
    b1 = np.zeros(h)
    got = O.ref_score(x, w1, b1, w2, 0.0)
    assert np.array_equal(got, x[:, 7] / (1.0 + np.exp(-x[:, 7])))
    # biases enter before (b1) and after (b2) the activation
    b1[3] = 0.25
    got = O.ref_score(x, w1, b1, w2, -2.0)
    z = x[:, 7] + 0.25
    assert np.allclose(got, z / (1.0 + np.exp(-z)) - 2.0, rtol=0, atol=1e-15)


def test_score_matches_torch_fp64():
    rng = _rng(2)
    T, d, h = 50, 24, 9
    x = rng.standard_normal((T, d))
    w1 = rng.standard_normal((h, d))
    b1 = rng.standard_normal(h)
    w2 = rng.standard_normal(h)
    lin1 = torch.nn.Linear(d, h).double()
    lin2 = torch.nn.Linear(h, 1).double()
    with torch.no_grad():
        lin1.weight.copy_(torch.from_numpy(w1))
        lin1.bias.copy_(torch.from_numpy(b1))
        lin2.weight.copy_(torch.from_numpy(w2)[None])
        lin2.bias.fill_(0.3)
        want = lin2(torch.nn.functional.silu(lin1(torch.from_numpy(x))))[:, 0].numpy()
    got = O.ref_score(x, w1, b1, w2, 0.3)
    assert np.allclose(got, want, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------------------
# LN2 before the scorer (§3 Eq. 1, RMSNorm reading R22)
# ---------------------------------------------------------------------------
def test_rmsnorm_closed_form_and_invariants():
    # [3, 4]: mean square 12.5, so the row becomes [3, 4] / sqrt(12.5)
    got = O.ref_rmsnorm(np.array([[3.0, 4.0]]), None, 0.0)
    assert np.allclose(got, [[3.0 / math.sqrt(12.5), 4.0 / math.sqrt(12.5)]], rtol=1e-15, atol=0)
    rng = _rng(40)
    a = rng.standard_normal((20, 64)) * rng.uniform(0.1, 10.0, (20, 1))
    y = O.ref_rmsnorm(a, None, 0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=1)), 1.0, rtol=1e-14)     # unit RMS
    assert np.allclose(O.ref_rmsnorm(7.5 * a, None, 0.0), y, rtol=1e-13)     # scale-free
    g = rng.uniform(0.5, 2.0, 64)
    assert np.allclose(O.ref_rmsnorm(a, g, 0.0), y * g[None, :], rtol=1e-15)
    # eps enters under the root: a zero row stays zero, a tiny row is damped
    z = O.ref_rmsnorm(np.zeros((1, 8)), None, 1e-6)
    assert np.array_equal(z, np.zeros((1, 8)))


def test_rmsnorm_matches_torch_fp64():
    rng = _rng(41)
    a = rng.standard_normal((33, 48)) * 3.0
    g = rng.uniform(0.5, 1.5, 48)
    want = torch.nn.functional.rms_norm(torch.from_numpy(a), (48,), torch.from_numpy(g),
                                        eps=1e-6).numpy()
    assert np.allclose(O.ref_rmsnorm(a, g, 1e-6), want, rtol=1e-13, atol=1e-13)


def test_prenorm_score_folds_gamma_into_w1():
    """W1 (gamma * a / r) = (W1 diag(gamma)) (a / r): the norm weight folds
    into the scorer's first layer, leaving only the division by the row RMS."""
    rng = _rng(42)
    T, d, h = 40, 32, 8
    a = rng.standard_normal((T, d)) * rng.uniform(0.2, 5.0, (T, 1))
    g = rng.uniform(0.5, 1.5, d)
    w1 = rng.standard_normal((h, d)) / math.sqrt(d)
    b1 = rng.standard_normal(h)
    w2 = rng.standard_normal(h)
    got = O.ref_score_prenorm(a, g, 1e-6, w1, b1, w2, 0.1)
    folded = O.ref_score_prenorm(a, None, 1e-6, w1 * g[None, :], b1, w2, 0.1)
    assert np.allclose(got, folded, rtol=1e-12, atol=1e-12)
    # and it is the plain scorer on the normalised rows
    r = np.sqrt(np.mean(a * a, axis=1, keepdims=True) + 1e-6)
    assert np.allclose(got, O.ref_score(a / r * g, w1, b1, w2, 0.1), rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------------------
# normalisation (Eq. 3, RMS reading R2)
# ---------------------------------------------------------------------------
def test_normalise_closed_forms():
    b_raw = np.array([3.0, 4.0, 100.0, -7.0])
    prunable = np.array([1, 1, 0, 0], np.uint8)
    b, r = O.ref_normalise(b_raw, prunable, [0, 4], eps=0.0)
    assert r[0] == math.sqrt(12.5)
    assert b[0] == 3.0 / math.sqrt(12.5) and b[1] == 4.0 / math.sqrt(12.5)
    assert b[2] == 0.0 and b[3] == 0.0                   # prompt tokens: b := 0
    rng = _rng(3)
    x = rng.standard_normal(200) * 3.0
    pr = (rng.random(200) < 0.8).astype(np.uint8)
    for eps in (0.0, 1e-6, 0.5):
        b, _ = O.ref_normalise(x, pr, [0, 200], eps)
        P = pr.astype(bool)
        M = np.mean(x[P] ** 2)
        assert np.mean(b[P] ** 2) == pytest.approx(M / (M + eps), rel=1e-13)
        assert np.all(b[~P] == 0.0)
    # positive rescaling of the scorer output leaves b unchanged when eps = 0
    b1, _ = O.ref_normalise(x, pr, [0, 200], 0.0)
    b2, _ = O.ref_normalise(7.5 * x, pr, [0, 200], 0.0)
    assert np.allclose(b1, b2, rtol=1e-14, atol=0)
    # all-zero raw scores give all-zero b
    bz, _ = O.ref_normalise(np.zeros(10), np.ones(10, np.uint8), [0, 10], 1e-6)
    assert np.all(bz == 0.0)


def test_normalise_is_per_sequence():
    x = np.array([1.0, 1.0, 10.0, 10.0, 10.0])
    pr = np.ones(5, np.uint8)
    b, r = O.ref_normalise(x, pr, [0, 2, 5], eps=0.0)
    assert np.allclose(b, 1.0) and np.allclose(r, [1.0, 10.0])
    # a sequence with no prunable token: nothing to normalise, b = 0
    b, r = O.ref_normalise(x, np.array([0, 0, 1, 1, 1], np.uint8), [0, 2, 5], 0.0)
    assert b[0] == 0.0 and b[1] == 0.0 and r[0] == 1.0


# ---------------------------------------------------------------------------
# top-K selector (Eq. 4, readings R11, R12, R14)
# ---------------------------------------------------------------------------
def _beats(bt, t, bu, u):
    """t ranks strictly before u: larger value first, NaN last, lower index on ties."""
    nt, nu = math.isnan(bt), math.isnan(bu)
    if nt != nu:
        return nu
    if not nt and bt != bu:
        return bt > bu
    return t < u


def _brute_select(b, prunable, k):
    P = [j for j in range(len(b)) if prunable[j]]
    Nset = [j for j in range(len(b)) if not prunable[j]]
    kp = min(k, len(P))
    found = []
    for T in itertools.combinations(P, kp):
        rest = [u for u in P if u not in T]
        if all(_beats(b[t], t, b[u], u) for t in T for u in rest):
            found.append(T)
    assert len(found) == 1                  # the strict order makes the subset unique
    return sorted(list(found[0]) + Nset)


@pytest.mark.parametrize("seed", range(40))
def test_select_bruteforce_small(seed):
    rng = _rng(100 + seed)
    n = int(rng.integers(1, 11))
    pool = np.array([0.0, -0.0, 1.0, -1.0, 2.5, np.inf, -np.inf, np.nan, 0.5, 0.5])
    b = rng.choice(pool, n) if seed % 2 else rng.standard_normal(n).round(1)
    pr = (rng.random(n) < 0.7).astype(np.uint8)
    for k in range(0, n + 2):
        idx, pos, kb, cu = O.ref_select(b, pr, [0, n], [k])
        assert list(idx) == _brute_select(list(b), list(pr), k)
        assert np.array_equal(pos, idx)
        assert cu[-1] == len(idx)


@settings(max_examples=300, derandomize=True, deadline=None, database=None)
@given(vals=st.lists(st.sampled_from([0.0, -0.0, 1.0, -1.0, 0.5, 2.5, math.inf, -math.inf,
                                      math.nan]), max_size=9),
       mask_bits=st.integers(0, 2 ** 9 - 1), extra=st.integers(0, 2))
def test_select_bruteforce_hypothesis(vals, mask_bits, extra):
    """Every budget from 0 to |P| + 2 on hypothesis-drawn tiny inputs drawn
    from a tie-heavy pool with signed zeros, infinities and NaN."""
    n = len(vals)
    b = np.array(vals, np.float64)
    pr = np.array([(mask_bits >> j) & 1 for j in range(n)], np.uint8)
    for k in range(0, int(pr.sum()) + 1 + extra):
        idx, _, _, cu = O.ref_select(b, pr, [0, n], [k])
        assert list(idx) == _brute_select(list(b), list(pr), k)
        assert cu[-1] == len(idx)


def test_select_invariants_and_special_cases():
    rng = _rng(7)
    cu = [0, 50, 50, 130, 131]
    n = cu[-1]
    b = rng.standard_normal(n)
    b[rng.random(n) < 0.1] = -np.inf
    b[rng.random(n) < 0.05] = np.nan
    pr = (rng.random(n) < 0.75).astype(np.uint8)
    for ks in ([0, 0, 0, 0], [3, 5, 10, 1], [1000, 1, 1000, 1000], [40, 0, 2, 0]):
        idx, pos, kb, kcu = O.ref_select(b, pr, cu, ks)
        for s in range(4):
            lo, hi = cu[s], cu[s + 1]
            sel = idx[kcu[s]:kcu[s + 1]]
            assert np.all((sel >= lo) & (sel < hi))
            assert np.all(np.diff(sel) > 0)                       # ascending (R14)
            nP = int(pr[lo:hi].sum())
            prompt = np.arange(lo, hi)[pr[lo:hi] == 0]
            assert set(prompt) <= set(sel)                         # prompt always kept
            assert sel.size == min(ks[s], nP) + (hi - lo - nP)
            assert np.array_equal(pos[kcu[s]:kcu[s + 1]], sel - lo)
        assert np.array_equal(kcu, O.ref_kept_sizes(cu, [int(pr[cu[s]:cu[s + 1]].sum())
                                                         for s in range(4)], ks))
        assert np.array_equal(kb, b[idx], equal_nan=True)
    # all-equal scores keep the first K document tokens
    idx, *_ = O.ref_select(np.full(20, 0.3), np.ones(20, np.uint8), [0, 20], [6])
    assert list(idx) == list(range(6))
    # -0.0 and +0.0 are equal: the lower index wins
    idx, *_ = O.ref_select(np.array([-0.0, 0.0, -0.0]), np.ones(3, np.uint8), [0, 3], [1])
    assert list(idx) == [0]
    with pytest.raises(ValueError):
        O.ref_select(b, pr, cu, [-1, 0, 0, 0])


def test_select_preset_budget_sweep_spikes_and_ties():
    g = generate(2, with_x=False, with_proj=False)
    b = g["b_preset"]
    pr = g["prunable"]
    n_doc = int(pr.sum())
    spikes = np.nonzero(b == 6.0)[0]
    assert spikes.size == round(0.05 * n_doc)
    for kk in g["budgets"]:
        idx, pos, kb, cu = O.ref_select(b, pr, g["cu_seqlens"], kk)
        k = int(kk[0])
        doc_kept = idx[idx < n_doc]
        assert doc_kept.size == k
        assert np.all(idx[doc_kept.size:] == np.arange(n_doc, b.size))
        above = np.nonzero(b[:n_doc] > 6.0)[0]      # rare Gaussian draws beyond the spikes
        if above.size <= k <= above.size + spikes.size:
            # every +6 spike ties: after the larger values, the lowest indices win
            want = np.sort(np.concatenate([above, spikes[:k - above.size]]))
            assert np.array_equal(doc_kept, want)


# ---------------------------------------------------------------------------
# gather
# ---------------------------------------------------------------------------
def test_gather_bytewise_and_identity():
    rng = _rng(9)
    src = rng.integers(0, 2 ** 16, (40, 24), dtype=np.uint16)
    idx = np.array([0, 3, 3, 39, 17])
    out = O.ref_gather(src, idx)
    for r, i in enumerate(idx):
        assert out[r].tobytes() == src[i].tobytes()
    idx, *_ = O.ref_select(rng.standard_normal(40), np.ones(40, np.uint8), [0, 40], [40])
    assert np.array_equal(O.ref_gather(src, idx), src)


# ---------------------------------------------------------------------------
# token-gated attention (Eq. 5-8)
# ---------------------------------------------------------------------------
def _attn_case(seed, seqlens=(13, 1, 29), hq=4, hkv=2, dh=16, keep_frac=0.5, n_prompt=3):
    rng = _rng(seed)
    cu = np.concatenate([[0], np.cumsum(seqlens)]).astype(np.int64)
    N = int(cu[-1])
    pr = np.ones(N, np.uint8)
    for s in range(len(seqlens)):
        pr[max(cu[s], cu[s + 1] - n_prompt):cu[s + 1]] = 0
    b = rng.standard_normal(N)
    b[pr == 0] = 0.0
    ks = [int(keep_frac * int(pr[cu[s]:cu[s + 1]].sum())) for s in range(len(seqlens))]
    idx, pos, kb, kcu = O.ref_select(b, pr, cu, ks)
    qf = rng.standard_normal((N, hq, dh))
    kf = rng.standard_normal((N, hkv, dh))
    vf = rng.standard_normal((N, hkv, dh))
    gain = rng.uniform(0.5, 1.5, hq)
    temp = rng.uniform(0.8, 1.2, hq)
    return dict(cu=cu, pr=pr, b=b, idx=idx, pos=pos, kb=kb, kcu=kcu, qf=qf, kf=kf, vf=vf,
                q=qf[idx], k=kf[idx], v=vf[idx], gain=gain, temp=temp)


def _sdpa(q, k, v, cu, scale=None):
    """torch scaled_dot_product_attention (fp64, CPU) per sequence, GQA by
    repeating consecutive KV heads."""
    G = q.shape[1] // k.shape[1]
    out = np.zeros_like(q)
    for s in range(len(cu) - 1):
        lo, hi = int(cu[s]), int(cu[s + 1])
        if hi == lo:
            continue
        tq = torch.from_numpy(q[lo:hi]).permute(1, 0, 2)
        tk = torch.from_numpy(k[lo:hi]).repeat_interleave(G, dim=1).permute(1, 0, 2)
        tv = torch.from_numpy(v[lo:hi]).repeat_interleave(G, dim=1).permute(1, 0, 2)
        o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True,
                                                             scale=scale)
        out[lo:hi] = o.permute(1, 0, 2).numpy()
    return out


def test_zero_scores_reduce_to_topk_causal_sdpa():
    c = _attn_case(11)
    hq = c["q"].shape[1]
    zeros = np.zeros_like(c["kb"])
    got = O.ref_gated_attn(c["q"], c["k"], c["v"], zeros, c["pos"], c["kcu"], c["gain"],
                           np.ones(hq), len_scale="off")
    assert np.allclose(got, _sdpa(c["q"], c["k"], c["v"], c["kcu"]), rtol=0, atol=1e-12)
    # gain = 0 silences any score vector in the same way
    got = O.ref_gated_attn(c["q"], c["k"], c["v"], c["kb"], c["pos"], c["kcu"], np.zeros(hq),
                           np.ones(hq), len_scale="off")
    assert np.allclose(got, _sdpa(c["q"], c["k"], c["v"], c["kcu"]), rtol=0, atol=1e-12)


def test_full_context_reduces_to_causal_sdpa_with_temperature():
    c = _attn_case(12, keep_frac=1.0)
    hq, dh = c["q"].shape[1], c["q"].shape[2]
    assert c["idx"].size == c["cu"][-1]
    zeros = np.zeros_like(c["kb"])
    # the length factor is 1 at every position when nothing is pruned (R6)
    got = O.ref_gated_attn(c["q"], c["k"], c["v"], zeros, c["pos"], c["kcu"], c["gain"],
                           np.ones(hq))
    assert np.allclose(got, _sdpa(c["q"], c["k"], c["v"], c["kcu"]), rtol=0, atol=1e-12)
    # a uniform temperature t multiplies the logit scale
    got = O.ref_gated_attn(c["q"], c["k"], c["v"], zeros, c["pos"], c["kcu"], c["gain"],
                           np.full(hq, 0.7))
    want = _sdpa(c["q"], c["k"], c["v"], c["kcu"], scale=0.7 / math.sqrt(dh))
    assert np.allclose(got, want, rtol=0, atol=1e-12)


def test_uniform_kept_bias_cancels():
    c = _attn_case(13)
    base = O.ref_gated_attn(c["q"], c["k"], c["v"], np.zeros_like(c["kb"]), c["pos"], c["kcu"],
                            c["gain"], c["temp"])
    for cst in (0.37, -2.0, 5.0):
        got = O.ref_gated_attn(c["q"], c["k"], c["v"], np.full_like(c["kb"], cst), c["pos"],
                               c["kcu"], c["gain"], c["temp"])
        assert np.allclose(got, base, rtol=0, atol=1e-12)


def test_zero_queries_give_closed_form_score_weights():
    """With q = 0 the logits are tau_i * gain_h * b_j, so each output row is the
    softmax-of-scores average of the visible values."""
    c = _attn_case(14)
    q0 = np.zeros_like(c["q"])
    got = O.ref_gated_attn(q0, c["k"], c["v"], c["kb"], c["pos"], c["kcu"], c["gain"], c["temp"])
    from scipy.special import softmax
    hq, hkv = c["q"].shape[1], c["k"].shape[1]
    for s in range(len(c["kcu"]) - 1):
        lo, hi = int(c["kcu"][s]), int(c["kcu"][s + 1])
        for i in range(lo, hi):
            m, p = i - lo + 1, int(c["pos"][i]) + 1
            for h in range(hq):
                tau = c["temp"][h] * math.log(m) / math.log(max(2, p))
                w = softmax(tau * c["gain"][h] * c["kb"][lo:i + 1])
                assert np.allclose(got[i, h], w @ c["v"][lo:i + 1, h // (hq // hkv)],
                                   rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", [21, 22, 23])
def test_mask_form_equals_compacted_form(seed):
    c = _attn_case(seed, seqlens=(40, 7, 25), keep_frac=0.4)
    got = O.ref_gated_attn(c["q"], c["k"], c["v"], c["kb"], c["pos"], c["kcu"], c["gain"],
                           c["temp"])
    keep = np.zeros(c["cu"][-1], bool)
    keep[c["idx"]] = True
    full = O.ref_gated_attn_masked(c["qf"], c["kf"], c["vf"], c["b"], keep, c["cu"], c["gain"],
                                   c["temp"])
    assert np.allclose(got, full[c["idx"]], rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", [31, 32])
def test_multiplicative_and_loggate_forms_equal_eq8(seed):
    c = _attn_case(seed)
    args = (c["q"], c["k"], c["v"], c["kb"], c["pos"], c["kcu"], c["gain"], c["temp"])
    eq8 = O.ref_gated_attn(*args)
    assert np.allclose(O.ref_gated_attn_multiplicative(*args), eq8, rtol=0, atol=1e-12)
    assert np.allclose(O.ref_gated_attn_loggate(*args), eq8, rtol=0, atol=1e-12)


@settings(max_examples=60, derandomize=True, deadline=None, database=None)
@given(seqlens=st.lists(st.integers(0, 12), min_size=1, max_size=3),
       heads=st.sampled_from([(1, 1), (2, 1), (4, 2), (4, 4)]), dh=st.integers(1, 6),
       keep_frac=st.sampled_from([0.0, 0.3, 0.7, 1.0]), n_prompt=st.integers(0, 4),
       seed=st.integers(0, 2 ** 31 - 1))
def test_attention_forms_agree_hypothesis(seqlens, heads, dh, keep_frac, n_prompt, seed):
    """On hypothesis-drawn tiny cases the vectorised oracle, the explicit
    double loop, and the full-length masked form evaluated on the kept rows
    agree (empty sequences, no prompt tokens, nothing pruned included)."""
    hq, hkv = heads
    c = _attn_case(seed, seqlens=tuple(seqlens), hq=hq, hkv=hkv, dh=dh, keep_frac=keep_frac,
                   n_prompt=n_prompt)
    args = (c["q"], c["k"], c["v"], c["kb"], c["pos"], c["kcu"], c["gain"], c["temp"])
    got = O.ref_gated_attn(*args)
    assert np.allclose(got, O.ref_gated_attn_bruteforce(*args), rtol=0, atol=1e-12)
    keep = np.zeros(c["cu"][-1], bool)
    keep[c["idx"]] = True
    full = O.ref_gated_attn_masked(c["qf"], c["kf"], c["vf"], c["b"], keep, c["cu"], c["gain"],
                                   c["temp"])
    assert np.allclose(got, full[c["idx"]], rtol=0, atol=1e-12)


def test_bruteforce_tiny():
    c = _attn_case(41, seqlens=(8, 3, 6), hq=2, hkv=1, dh=5)
    args = (c["q"], c["k"], c["v"], c["kb"], c["pos"], c["kcu"], c["gain"], c["temp"])
    for mode in ("log_ratio", "swap", "off"):
        assert np.allclose(O.ref_gated_attn(*args, len_scale=mode),
                           O.ref_gated_attn_bruteforce(*args, len_scale=mode), rtol=0, atol=1e-12)


def test_causality_and_sequence_independence():
    c = _attn_case(51, seqlens=(30, 20))
    args = [c["q"], c["k"], c["v"], c["kb"], c["pos"], c["kcu"], c["gain"], c["temp"]]
    base = O.ref_gated_attn(*args)
    lo, hi = int(c["kcu"][0]), int(c["kcu"][1])
    cut = lo + (hi - lo) // 2
    k2, v2, kb2 = c["k"].copy(), c["v"].copy(), c["kb"].copy()
    k2[cut + 1:hi] += 3.0
    v2[cut + 1:hi] -= 1.0
    kb2[cut + 1:hi] += 2.0
    pert = O.ref_gated_attn(c["q"], k2, v2, kb2, *args[4:])
    assert np.array_equal(pert[lo:cut + 1], base[lo:cut + 1])
    # each sequence run alone gives the same rows as the packed batch
    for s in range(2):
        a, b_ = int(c["kcu"][s]), int(c["kcu"][s + 1])
        alone = O.ref_gated_attn(c["q"][a:b_], c["k"][a:b_], c["v"][a:b_], c["kb"][a:b_],
                                 c["pos"][a:b_], [0, b_ - a], c["gain"], c["temp"])
        assert np.allclose(alone, base[a:b_], rtol=0, atol=1e-13)
    # evaluating a subset of rows gives the same rows
    rows = np.array([0, 3, hi + 2, hi + 5])
    sub = O.ref_gated_attn(*args, rows=rows, row_block=2)
    assert np.allclose(sub[rows], base[rows], rtol=0, atol=1e-14)


def test_first_query_attends_to_itself_only():
    c = _attn_case(61)
    got = O.ref_gated_attn(c["q"], c["k"], c["v"], c["kb"], c["pos"], c["kcu"], c["gain"],
                           c["temp"])
    G = c["q"].shape[1] // c["k"].shape[1]
    for s in range(len(c["kcu"]) - 1):
        lo = int(c["kcu"][s])
        if c["kcu"][s + 1] > lo:
            for h in range(c["q"].shape[1]):
                assert np.array_equal(got[lo, h], c["v"][lo, h // G])


def test_length_factor_values():
    m = np.array([1, 2, 5, 10])
    p = np.array([1, 2, 20, 10])
    lam = O.length_factor(m, p, "log_ratio")
    assert lam[0] == 0.0 and lam[1] == 1.0 and lam[3] == 1.0
    assert lam[2] == pytest.approx(math.log(5) / math.log(20), rel=1e-15)
    assert np.all(O.length_factor(m, p, "off") == 1.0)


# ---------------------------------------------------------------------------
# pass-count cost model: the explainer page's worked example
# ---------------------------------------------------------------------------
def test_worked_example_pass_counts():
    g = json.load(open(os.path.join(GOLDEN, "pass_counts_worked_example.json")))
    i, e = g["inputs"], g["expected"]
    full, gated = O.token_layer_passes(i["n_layers"], i["n_tokens"], i["gate_after_layer"],
                                       i["kept"])
    assert full == e["unpruned_token_layer_passes"]
    assert gated == e["gated_token_layer_passes"]
    assert (i["gate_after_layer"] + 1) * i["n_tokens"] == e["passes_below_gate"]
    assert gated - e["passes_below_gate"] == e["passes_above_gate"]
    assert round(full / gated, 1) == e["reduction_rounded_1dp"]
    assert O.attention_pair_ratio(i["n_tokens"], i["kept"]) == e[
        "attention_pair_reduction_per_upper_layer"]


def test_causal_flop_count_matches_pair_count():
    # 4*dh flops per (query head, causal pair); T(T+1)/2 pairs
    T, hq, dh = 8704, 16, 128
    assert O.causal_attention_flops([T], hq, dh) == 4 * dh * hq * (T * (T + 1) // 2)
    assert O.causal_attention_flops([T], hq, dh) == 310_347_038_720


# ---------------------------------------------------------------------------
# whole gate on the tiny workload
# ---------------------------------------------------------------------------
def test_gate_on_tiny_workload():
    g = generate(0)
    out = O.ref_gate(g["x"], g["w1"], g["b1"], g["w2"], g["b2"], g["prunable"],
                     g["cu_seqlens"], g["budgets"][0])
    b_raw, b, idx, pos, kb, kcu, xs = out
    assert idx.size == 192 and kcu[-1] == 192
    assert np.all(idx[-64:] == np.arange(960, 1024))
    assert np.all(b[960:] == 0.0)
    assert np.array_equal(xs, g["x"][idx])
    # the kept document tokens are exactly the 128 best normalised scores
    order = np.argsort(-b[:960].astype(np.float32), kind="stable")
    assert set(order[:128]) == set(idx[:128])


# ---------------------------------------------------------------------------
# projection of the kept rows (the step between gather and attention)
# ---------------------------------------------------------------------------
def test_projection_identity_weights_return_the_rows():
    rng = np.random.default_rng(31)
    T, hq, hkv, dh = 5, 2, 1, 4
    d = hq * dh
    x = rng.standard_normal((T, d))
    eye = np.eye(d)
    q, k, v = O.ref_project(x, eye, eye[:, :hkv * dh], eye[:, hkv * dh:2 * hkv * dh], hq, hkv, dh)
    assert np.array_equal(q.reshape(T, d), x)
    assert np.array_equal(k.reshape(T, hkv * dh), x[:, :hkv * dh])
    assert np.array_equal(v.reshape(T, hkv * dh), x[:, hkv * dh:])


# rotary embedding and q/k norm of the projections (reading R23)
def test_rope_tiny_worked_example():
    """dh = 4, theta = 10000: pair (x0, x2) turns at frequency 1, pair (x1, x3)
    at 10000**(-1/2) = 0.01; position 1."""
    x = np.array([1.0, 2.0, 3.0, 4.0]).reshape(1, 1, 4)
    got = O.ref_rope(x, np.array([1]), 10000.0).reshape(4)
    c1, s1, c2, s2 = math.cos(1.0), math.sin(1.0), math.cos(0.01), math.sin(0.01)
    want = [1 * c1 - 3 * s1, 2 * c2 - 4 * s2, 3 * c1 + 1 * s1, 4 * c2 + 2 * s2]
    assert np.allclose(got, want, rtol=0, atol=1e-15)


def test_rope_equals_complex_rotation_and_preserves_pairs():
    rng = _rng(61)
    T, H, dh, theta = 7, 3, 16, 1e6
    x = rng.standard_normal((T, H, dh))
    pos = rng.integers(0, 200000, T)
    got = O.ref_rope(x, pos, theta)
    half = dh // 2
    z = (x[..., :half] + 1j * x[..., half:]) * np.exp(
        1j * np.outer(pos, theta ** (-np.arange(0, dh, 2) / dh)))[:, None, :]
    assert np.allclose(got[..., :half], z.real, rtol=0, atol=1e-12)
    assert np.allclose(got[..., half:], z.imag, rtol=0, atol=1e-12)
    pair_norm = lambda a: np.hypot(a[..., :half], a[..., half:])
    assert np.allclose(pair_norm(got), pair_norm(x), rtol=1e-13)
    assert np.array_equal(O.ref_rope(x, np.zeros(T, np.int64), theta), x)


def test_rope_dot_products_depend_on_relative_position():
    rng = _rng(62)
    dh = 64
    q = rng.standard_normal((1, 1, dh))
    k = rng.standard_normal((1, 1, dh))
    for m, n in [(0, 5), (17, 400), (1000, 1001), (90000, 131071)]:
        a = float(np.sum(O.ref_rope(q, [m], 1e6) * O.ref_rope(k, [n], 1e6)))
        b = float(np.sum(O.ref_rope(q, [0], 1e6) * O.ref_rope(k, [n - m], 1e6)))
        assert abs(a - b) <= 1e-9 * (1 + abs(b))


def test_project_qk_rope_composition():
    """No norm weights and theta <= 0 give the plain projection; the norm
    leaves each q and k head with unit RMS (unit weight, eps 0) and the
    rotation keeps it."""
    rng = _rng(63)
    T, d, hq, hkv, dh = 9, 24, 4, 2, 8
    xs = rng.standard_normal((T, d))
    wq, wk, wv = (rng.standard_normal((d, h * dh)) for h in (hq, hkv, hkv))
    pos = rng.integers(0, 5000, T)
    plain = O.ref_project(xs, wq, wk, wv, hq, hkv, dh)
    same = O.ref_project_qk_rope(xs, wq, wk, wv, hq, hkv, dh, pos, None, None, 1e-6, 0.0)
    for a, b in zip(plain, same):
        assert np.array_equal(a, b)
    q, k, v = O.ref_project_qk_rope(xs, wq, wk, wv, hq, hkv, dh, pos, np.ones(dh), np.ones(dh),
                                    0.0, 1e6)
    for a in (q, k):
        assert np.allclose(np.sqrt(np.mean(a * a, axis=-1)), 1.0, rtol=1e-12)
    assert np.array_equal(v, plain[2])


def test_qk_norm_worked_example():
    """One head of dh = 4, [3, 4, 0, 0]: mean square 25/4, RMS 2.5, so the
    normalised head is [1.2, 1.6, 0, 0]; the weight [1, 2, 3, 4] scales it
    element by element to [1.2, 3.2, 0, 0].  Rotation off."""
    xs = np.array([[1.0, 0.0]])
    wq = np.array([[3.0, 4.0, 0.0, 0.0], [0.0, 0.0, 0.0, 0.0]])
    wk = np.array([[0.0, 0.0, 0.0, 2.0], [0.0, 0.0, 0.0, 0.0]])
    q, k, _ = O.ref_project_qk_rope(xs, wq, wk, wk, 1, 1, 4, [0], np.array([1.0, 2.0, 3.0, 4.0]),
                                    None, 0.0, 0.0)
    assert np.allclose(q.reshape(4), [1.2, 3.2, 0.0, 0.0], rtol=0, atol=1e-15)
    assert np.array_equal(k.reshape(4), [0.0, 0.0, 0.0, 2.0])        # no k weight: untouched


def test_projection_head_layout_and_linearity():
    rng = np.random.default_rng(32)
    T, d, hq, hkv, dh = 4, 6, 3, 1, 2
    wq = rng.standard_normal((d, hq * dh))
    wk = rng.standard_normal((d, hkv * dh))
    wv = rng.standard_normal((d, hkv * dh))
    x1, x2 = rng.standard_normal((T, d)), rng.standard_normal((T, d))
    q1, k1, v1 = O.ref_project(x1, wq, wk, wv, hq, hkv, dh)
    # head h, element e of row r is the dot product of row r with column h*dh+e
    for r in range(T):
        for h in range(hq):
            for e in range(dh):
                want = sum(x1[r, c] * wq[c, h * dh + e] for c in range(d))
                assert abs(q1[r, h, e] - want) < 1e-12
    q2, k2, v2 = O.ref_project(x2, wq, wk, wv, hq, hkv, dh)
    q3, k3, v3 = O.ref_project(2.5 * x1 - x2, wq, wk, wv, hq, hkv, dh)
    for a, b, c in ((q1, q2, q3), (k1, k2, k3), (v1, v2, v3)):
        assert np.allclose(c, 2.5 * a - b, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# backward of token-gated attention (§4.3 gradient path through Eq. 8)
# ---------------------------------------------------------------------------
def _bwd_case(seed, lens=(5, 7), hq=4, hkv=2, dh=8):
    rng = _rng(seed)
    kc = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T = int(kc[-1])
    q = rng.standard_normal((T, hq, dh))
    k = rng.standard_normal((T, hkv, dh))
    v = rng.standard_normal((T, hkv, dh))
    kb = rng.standard_normal(T)
    pos = np.concatenate([np.sort(rng.choice(40, n, replace=False)) for n in lens]).astype(np.int64)
    gain = rng.uniform(0.5, 1.5, hq)
    temp = rng.uniform(0.8, 1.2, hq)
    do = rng.standard_normal((T, hq, dh))
    return q, k, v, kb, pos, kc, gain, temp, do


def _loss(q, k, v, kb, pos, kc, gain, temp, do):
    return float(np.sum(O.ref_gated_attn(q, k, v, kb, pos, kc, gain, temp) * do))


def test_attn_bwd_matches_central_differences():
    """Every gradient against (L(x+h) - L(x-h)) / 2h of L = sum(O * dout),
    on several entries of each input."""
    args = list(_bwd_case(50))
    dq, dk, dv, db, dg, dt = O.ref_gated_attn_bwd(*args)
    grads = {0: dq, 1: dk, 2: dv, 3: db, 6: dg, 7: dt}
    rng = _rng(51)
    eps = 1e-6
    for ai, gr in grads.items():
        for _ in range(6):
            idx = tuple(int(rng.integers(0, n)) for n in np.shape(args[ai]))
            plus = [np.array(a, dtype=np.float64, copy=True) if i == ai else a for i, a in enumerate(args)]
            minus = [np.array(a, dtype=np.float64, copy=True) if i == ai else a for i, a in enumerate(args)]
            plus[ai][idx] += eps
            minus[ai][idx] -= eps
            fd = (_loss(*plus) - _loss(*minus)) / (2 * eps)
            assert abs(fd - gr[idx]) <= 1e-6 * max(1.0, abs(fd)), (ai, idx, fd, gr[idx])


def test_attn_bwd_matches_torch_autograd_fp64():
    """The same loss written with torch ops (masked softmax attention with an
    additive bias and a per-query temperature), differentiated by autograd."""
    q, k, v, kb, pos, kc, gain, temp, do = _bwd_case(52, lens=(9, 1, 6), hq=6, hkv=3, dh=4)
    T, hq, dh = q.shape
    G = hq // k.shape[1]
    tq, tk, tv, tb, tg, tt = (torch.tensor(a, dtype=torch.float64, requires_grad=True)
                              for a in (q, k, v, kb, gain, temp))
    out = []
    for s in range(len(kc) - 1):
        lo, hi = int(kc[s]), int(kc[s + 1])
        n = hi - lo
        m = torch.arange(1, n + 1, dtype=torch.float64)
        p = torch.tensor(pos[lo:hi] + 1, dtype=torch.float64)
        lam = torch.log(m) / torch.log(torch.clamp(p, min=2.0))
        for h in range(hq):
            z = tq[lo:hi, h] @ tk[lo:hi, h // G].T / math.sqrt(dh) + tg[h] * tb[lo:hi][None, :]
            lg = (tt[h] * lam)[:, None] * z
            lg = lg.masked_fill(torch.triu(torch.ones(n, n, dtype=torch.bool), 1), float("-inf"))
            out.append((torch.softmax(lg, dim=1) @ tv[lo:hi, h // G] * torch.tensor(do[lo:hi, h])).sum())
    torch.stack(out).sum().backward()
    got = O.ref_gated_attn_bwd(q, k, v, kb, pos, kc, gain, temp, do)
    for g_np, t in zip(got, (tq, tk, tv, tb, tg, tt)):
        assert np.allclose(g_np, t.grad.numpy(), rtol=1e-11, atol=1e-12)


def test_attn_bwd_invariants():
    """Shifting every b of a sequence by c shifts each row's logits by a
    constant, so the scores' gradient sums to zero per sequence; and since
    each row of P sums to 1, dv summed over keys equals dout summed over the
    queries and query heads of each KV head."""
    q, k, v, kb, pos, kc, gain, temp, do = _bwd_case(53, lens=(11, 4, 8), hq=4, hkv=2, dh=8)
    dq, dk, dv, db, dg, dt = O.ref_gated_attn_bwd(q, k, v, kb, pos, kc, gain, temp, do)
    for s in range(len(kc) - 1):
        assert abs(np.sum(db[kc[s]:kc[s + 1]])) < 1e-12
        for kvh in range(2):
            want = do[kc[s]:kc[s + 1], 2 * kvh:2 * kvh + 2].sum(axis=(0, 1))
            assert np.allclose(dv[kc[s]:kc[s + 1], kvh].sum(axis=0), want, rtol=1e-12, atol=1e-12)
    # row blocks do not change the result
    again = O.ref_gated_attn_bwd(q, k, v, kb, pos, kc, gain, temp, do, row_block=3)
    for a, b in zip(again, (dq, dk, dv, db, dg, dt)):
        assert np.allclose(a, b, rtol=1e-13, atol=1e-14)


# ---------------------------------------------------------------------------
# backward of the scorer (Eq. 3 through the normalisation and the MLP)
# ---------------------------------------------------------------------------
def _score_bwd_case(seed, lens=(9, 7), d=6, h=5):
    rng = _rng(seed)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T = int(cu[-1])
    x = rng.standard_normal((T, d))
    w1 = rng.standard_normal((h, d)) / math.sqrt(d)
    b1 = 0.1 * rng.standard_normal(h)
    w2 = rng.standard_normal(h) / math.sqrt(h)
    pr = np.ones(T, np.uint8)
    for s in range(len(lens)):
        pr[cu[s + 1] - 2:cu[s + 1]] = 0                   # two prompt tokens per sequence
    k = [3, 2, 4][:len(lens)]
    raw = O.ref_score(x, w1, b1, w2, 0.2)
    b, _ = O.ref_normalise(raw, pr, cu, 1e-6)
    kept_idx, _, _, kept_cu = O.ref_select(b, pr, cu, k)
    db_kept = rng.standard_normal(len(kept_idx))
    return x, w1, b1, w2, pr, cu, kept_idx, kept_cu, db_kept


def _score_loss(x, w1, b1, w2, b2, pr, cu, kept_idx, db_kept):
    b, _ = O.ref_normalise(O.ref_score(x, w1, b1, w2, b2), pr, cu, 1e-6)
    return float(np.sum(np.asarray(db_kept) * b[np.asarray(kept_idx)]))


def test_score_bwd_matches_central_differences():
    """The kept set is held fixed (selection passes no gradient); the loss is
    sum_r db_kept[r] * b[kept_idx[r]], and every pruned token still enters
    through the sequence's normaliser."""
    x, w1, b1, w2, pr, cu, ki, kc, dbk = _score_bwd_case(60)
    dx, dw1, db1, dw2, db2 = O.ref_score_bwd(x, w1, b1, w2, 0.2, pr, cu, ki, kc, dbk, eps=1e-6)
    base = dict(x=x, w1=w1, b1=b1, w2=w2)
    grads = dict(x=dx, w1=dw1, b1=db1, w2=dw2)
    rng = _rng(61)
    e = 1e-6
    for name, g in grads.items():
        for _ in range(6):
            idx = tuple(int(rng.integers(0, n)) for n in np.shape(base[name]))
            vals = []
            for sgn in (1, -1):
                a = {n: np.array(v, copy=True) for n, v in base.items()}
                a[name][idx] += sgn * e
                vals.append(_score_loss(a["x"], a["w1"], a["b1"], a["w2"], 0.2, pr, cu, ki, dbk))
            fd = (vals[0] - vals[1]) / (2 * e)
            assert abs(fd - g[idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, g[idx])
    # b2 shifts every raw score of a sequence equally, which the RMS does not cancel
    fd = (_score_loss(x, w1, b1, w2, 0.2 + e, pr, cu, ki, dbk)
          - _score_loss(x, w1, b1, w2, 0.2 - e, pr, cu, ki, dbk)) / (2 * e)
    assert abs(fd - db2) <= 1e-6 * max(1.0, abs(fd))


def test_score_bwd_matches_torch_autograd_fp64():
    x, w1, b1, w2, pr, cu, ki, kc, dbk = _score_bwd_case(62, lens=(12, 5, 9), d=8, h=4)
    tx, tw1, tb1, tw2 = (torch.tensor(a, dtype=torch.float64, requires_grad=True)
                         for a in (x, w1, b1, w2))
    tb2 = torch.tensor(0.2, dtype=torch.float64, requires_grad=True)
    raw = torch.nn.functional.silu(tx @ tw1.T + tb1) @ tw2 + tb2
    parts = []
    for s in range(len(cu) - 1):
        lo, hi = int(cu[s]), int(cu[s + 1])
        m = torch.tensor(pr[lo:hi].astype(bool))
        rs = torch.sqrt(torch.mean(raw[lo:hi][m] ** 2) + 1e-6)
        parts.append(torch.where(m, raw[lo:hi] / rs, torch.zeros_like(raw[lo:hi])))
    b = torch.cat(parts)
    (b[torch.tensor(ki)] * torch.tensor(dbk)).sum().backward()
    got = O.ref_score_bwd(x, w1, b1, w2, 0.2, pr, cu, ki, kc, dbk, eps=1e-6)
    for g, t in zip(got, (tx, tw1, tb1, tw2, tb2)):
        assert np.allclose(g, t.grad.numpy(), rtol=1e-11, atol=1e-12)


def _prenorm_loss(a, g, ne, w1, b1, w2, b2, pr, cu, kept_idx, db_kept):
    raw = O.ref_score_prenorm(a, g, ne, w1, b1, w2, b2)
    b, _ = O.ref_normalise(raw, pr, cu, 1e-6)
    return float(np.sum(np.asarray(db_kept) * b[np.asarray(kept_idx)]))


def test_score_prenorm_bwd_matches_central_differences():
    """The LN2-fused scorer's gradients w.r.t. the residual rows, W1, the
    norm's weight, b1, w2 and b2 against central differences of the loss
    through the forward oracle (kept set fixed, as for the plain form)."""
    x, w1, b1, w2, pr, cu, ki, kc, dbk = _score_bwd_case(63)
    rng = _rng(64)
    a = 3.0 * x + 0.5                                # rows far from unit RMS
    g = rng.uniform(0.5, 1.5, a.shape[1])
    ne = 1e-3
    da, dw1, dg, db1, dw2, db2 = O.ref_score_prenorm_bwd(a, g, ne, w1, b1, w2, 0.2, pr, cu, ki,
                                                         kc, dbk, eps=1e-6)
    base = dict(a=a, g=g, w1=w1, b1=b1, w2=w2)
    grads = dict(a=da, g=dg, w1=dw1, b1=db1, w2=dw2)
    e = 1e-6
    for name, grad in grads.items():
        for _ in range(6):
            idx = tuple(int(rng.integers(0, n)) for n in np.shape(base[name]))
            vals = []
            for sgn in (1, -1):
                p = {n: np.array(v, copy=True) for n, v in base.items()}
                p[name][idx] += sgn * e
                vals.append(_prenorm_loss(p["a"], p["g"], ne, p["w1"], p["b1"], p["w2"], 0.2, pr,
                                          cu, ki, dbk))
            fd = (vals[0] - vals[1]) / (2 * e)
            assert abs(fd - grad[idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, grad[idx])
    fd = (_prenorm_loss(a, g, ne, w1, b1, w2, 0.2 + e, pr, cu, ki, dbk)
          - _prenorm_loss(a, g, ne, w1, b1, w2, 0.2 - e, pr, cu, ki, dbk)) / (2 * e)
    assert abs(fd - db2) <= 1e-6 * max(1.0, abs(fd))


def test_score_prenorm_bwd_matches_torch_rms_norm_autograd():
    """Against autograd through torch's own RMSNorm routine in fp64."""
    x, w1, b1, w2, pr, cu, ki, kc, dbk = _score_bwd_case(65, lens=(12, 5, 9), d=8, h=4)
    rng = _rng(66)
    a = 2.0 * x - 0.3
    g = rng.uniform(0.5, 1.5, a.shape[1])
    ta, tg, tw1, tb1, tw2 = (torch.tensor(v, dtype=torch.float64, requires_grad=True)
                             for v in (a, g, w1, b1, w2))
    tb2 = torch.tensor(0.2, dtype=torch.float64, requires_grad=True)
    xn = torch.nn.functional.rms_norm(ta, (a.shape[1],), weight=tg, eps=1e-3)
    raw = torch.nn.functional.silu(xn @ tw1.T + tb1) @ tw2 + tb2
    parts = []
    for s in range(len(cu) - 1):
        lo, hi = int(cu[s]), int(cu[s + 1])
        m = torch.tensor(pr[lo:hi].astype(bool))
        rs = torch.sqrt(torch.mean(raw[lo:hi][m] ** 2) + 1e-6)
        parts.append(torch.where(m, raw[lo:hi] / rs, torch.zeros_like(raw[lo:hi])))
    b = torch.cat(parts)
    (b[torch.tensor(ki)] * torch.tensor(dbk)).sum().backward()
    got = O.ref_score_prenorm_bwd(a, g, 1e-3, w1, b1, w2, 0.2, pr, cu, ki, kc, dbk, eps=1e-6)
    for v, t in zip(got, (ta, tw1, tg, tb1, tw2, tb2)):
        assert np.allclose(v, t.grad.numpy(), rtol=1e-11, atol=1e-12)


def test_score_prenorm_bwd_fold_and_scale_invariance():
    """Folding the norm's weight into W1 (W1' = W1 diag(gamma), gamma = ones)
    leaves da unchanged and gives dW1 = dW1' diag(gamma) and
    dgamma = sum over hidden units of W1 * dW1'.  With norm_eps = 0 the norm
    is blind to the scale of a row, so every row of da is orthogonal to its
    row of a."""
    x, w1, b1, w2, pr, cu, ki, kc, dbk = _score_bwd_case(67)
    rng = _rng(68)
    a = 1.7 * x
    g = rng.uniform(0.5, 1.5, a.shape[1])
    da, dw1, dg, db1, dw2, db2 = O.ref_score_prenorm_bwd(a, g, 1e-3, w1, b1, w2, 0.2, pr, cu,
                                                         ki, kc, dbk, eps=1e-6)
    fa, fw1, _, fb1, fw2, fb2 = O.ref_score_prenorm_bwd(a, None, 1e-3, w1 * g[None, :], b1, w2,
                                                        0.2, pr, cu, ki, kc, dbk, eps=1e-6)
    assert np.allclose(fa, da, rtol=1e-12, atol=1e-14)
    assert np.allclose(fw1 * g[None, :], dw1, rtol=1e-12, atol=1e-14)
    assert np.allclose(np.sum(w1 * fw1, axis=0), dg, rtol=1e-12, atol=1e-14)
    assert np.allclose(fb1, db1, rtol=1e-12) and np.allclose(fw2, dw2, rtol=1e-12)
    assert abs(fb2 - db2) <= 1e-12 * max(1.0, abs(db2))
    z, *_ = O.ref_score_prenorm_bwd(a, g, 0.0, w1, b1, w2, 0.2, pr, cu, ki, kc, dbk, eps=1e-6)
    assert np.max(np.abs(np.sum(z * a, axis=1))) <= 1e-12 * np.max(np.abs(z) * np.abs(a)) * a.shape[1]
    assert np.max(np.abs(z)) > 1e-3                   # not orthogonal by being zero


def test_attn_bwd_rows_match_the_full_backward():
    """The sampled-rows form gives the full backward's dq rows and dk, dv, db
    rows exactly (same definitions), across row blocks and sequences, with
    positions and GQA."""
    rng = _rng(91)
    lens = [37, 0, 70, 1]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T, hq, hkv, dh = int(cu[-1]), 4, 2, 8
    q = rng.standard_normal((T, hq, dh))
    k = rng.standard_normal((T, hkv, dh))
    v = rng.standard_normal((T, hkv, dh))
    do = rng.standard_normal((T, hq, dh))
    kb = rng.standard_normal(T)
    pos = np.concatenate([np.sort(rng.choice(500, n, replace=False)) for n in lens]).astype(np.int64)
    gain = rng.uniform(0.5, 1.5, hq)
    temp = rng.uniform(0.8, 1.2, hq)
    full = O.ref_gated_attn_bwd(q, k, v, kb, pos, cu, gain, temp, do, row_block=16)
    qr = [0, 15, 16, 36, 37, 60, 106, 107]
    kr = [0, 1, 16, 36, 37, 52, 106, 107]
    dq, dk, dv, db = O.ref_gated_attn_bwd_rows(q, k, v, kb, pos, cu, gain, temp, do, qr, kr,
                                               row_block=16)
    assert np.allclose(dq, full[0][qr], rtol=1e-12, atol=1e-13)
    assert np.allclose(dk, full[1][kr], rtol=1e-12, atol=1e-13)
    assert np.allclose(dv, full[2][kr], rtol=1e-12, atol=1e-13)
    assert np.allclose(db, full[3][kr], rtol=1e-12, atol=1e-13)


# softmax normaliser of the gated attention, base 2 (the backward's statistic)
def test_attn_lse2_closed_forms():
    """Zero queries and zero scores make every visible logit 0, so row i of a
    sequence has lse2 = log2(i + 1); a sequence's first row sees only itself,
    so lse2 = tau (s q.k + gain b) / ln 2, here with s = 1/sqrt(2),
    q.k = 2, gain 1.5, b 0.5, temp 0.75: 0.75 (sqrt 2 + 0.75) / ln 2."""
    T, hq, hkv, dh = 7, 2, 1, 2
    cu = np.array([0, 3, 7])
    z = O.ref_gated_attn_lse2(np.zeros((T, hq, dh)), np.ones((T, hkv, dh)), np.zeros(T), None, cu,
                              np.ones(hq), np.ones(hq))
    want = np.log2(np.array([1, 2, 3, 1, 2, 3, 4], np.float64))
    assert np.allclose(z, want[:, None], rtol=0, atol=1e-15)
    q = np.zeros((1, 1, 2)); q[0, 0, 0] = 1.0
    k = np.zeros((1, 1, 2)); k[0, 0, 0] = 2.0
    got = O.ref_gated_attn_lse2(q, k, np.array([0.5]), None, np.array([0, 1]), np.array([1.5]),
                                np.array([0.75]))
    assert abs(got[0, 0] - 0.75 * (math.sqrt(2.0) + 0.75) / math.log(2.0)) <= 1e-14


def test_attn_lse2_normalises_the_attention():
    """2^(logit log2 e - lse2) are the attention weights: they sum to one over
    the visible keys, and applied to V they give ref_gated_attn's output."""
    rng = _rng(71)
    T, hq, hkv, dh = 40, 4, 2, 8
    cu = np.array([0, 13, 13, 40])
    q, k, v = (rng.standard_normal((T, h, dh)) for h in (hq, hkv, hkv))
    kb = rng.standard_normal(T)
    pos = np.concatenate([np.sort(rng.choice(100, 13, replace=False)),
                          np.sort(rng.choice(300, 27, replace=False))])
    gain, temp = rng.uniform(0.5, 1.5, hq), rng.uniform(0.8, 1.2, hq)
    lse2 = O.ref_gated_attn_lse2(q, k, kb, pos, cu, gain, temp)
    ref = O.ref_gated_attn(q, k, v, kb, pos, cu, gain, temp)
    s = 1.0 / math.sqrt(dh)
    for a, b in ((0, 13), (13, 40)):
        n = b - a
        lam = O.length_factor(np.arange(n) + 1.0, pos[a:b] + 1.0)
        for h in range(hq):
            logit = (temp[h] * lam)[:, None] * (s * q[a:b, h] @ k[a:b, h // 2].T + gain[h] * kb[None, a:b])
            w = np.exp2(logit * math.log2(math.e) - lse2[a:b, h, None])
            w[np.triu_indices(n, 1)] = 0.0
            assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-12)
            assert np.allclose(w @ v[a:b, h // 2], ref[a:b, h], rtol=0, atol=1e-12)
