"""Property-based parity: hypothesis draws the shapes, sequence lengths,
budgets and value patterns, and every drawn case goes through the C ABI and
is compared with the oracle at the usual bars: tg_select_topk and tg_gather
bit-exact, tg_score within 1e-5, tg_gated_attn rel-L2 <= 1e-2 (bf16) and
<= 1e-5 (fp32).  Draws are derandomized, so every run sees the same cases;
lengths are biased towards the kernels' block edges (chunks of 2048 tokens
in the selector, 64-key tiles and 128-query blocks in the attention)."""
import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle as O
from gpu_util import i32_dev, rel_l2, say
from test_parity_attn import TOL as ATTN_TOL
from test_parity_attn import run_attn, synth_case
from test_parity_gather_score import _check_score
from test_parity_select import check_select
from workloads import f32_to_bf16_bits

pytestmark = pytest.mark.gpu

SETTINGS = dict(derandomize=True, deadline=None, database=None,
                suppress_health_check=list(HealthCheck))

SEL_LEN = st.one_of(st.sampled_from([0, 1, 2, 63, 64, 65, 2047, 2048, 2049, 4096]),
                    st.integers(0, 6000))


@settings(max_examples=40, **SETTINGS)
@given(lens=st.lists(SEL_LEN, min_size=1, max_size=5), mode=st.integers(0, 4),
       density=st.sampled_from([0.0, 0.3, 0.9, 1.0]), seed=st.integers(0, 2 ** 31 - 1),
       kpick=st.lists(st.integers(0, 5), min_size=5, max_size=5))
def test_select_hypothesis(lens, mode, density, seed, kpick):
    rng = np.random.default_rng(seed)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    if mode == 0:
        b = rng.standard_normal(T)
    elif mode == 1:                      # many exact ties
        b = rng.integers(-3, 4, T).astype(np.float64)
    elif mode == 2:                      # signed zeros, infinities, NaN, denormals
        b = rng.choice(np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 1.0, -1.0, 1e-40]), T)
    elif mode == 3:                      # all equal
        b = np.full(T, -0.25)
    else:                                # bf16-grid values: ties between distinct draws
        b = f32_to_bf16_bits(rng.standard_normal(T).astype(np.float32)).astype(np.uint32)
        b = (b << 16).view(np.float32).astype(np.float64)
    pr = (rng.random(T) < density).astype(np.uint8)
    k = []
    for s in range(len(lens)):
        n_p = int(pr[cu[s]:cu[s + 1]].sum())
        k.append([0, 1, max(n_p - 1, 0), n_p, n_p + 7, n_p // 3][kpick[s]])
    say(f"select hypothesis: lens={lens} mode={mode} density={density} k={k}")
    check_select(b, pr, cu, k, f"lens={lens}")


@settings(max_examples=10, **SETTINGS)
@given(lens=st.lists(st.integers(0, 700), min_size=65, max_size=90),
       mode=st.integers(0, 4), seed=st.integers(0, 2 ** 31 - 1),
       kpick=st.integers(0, 5))
def test_select_hypothesis_many_sequences(lens, mode, seed, kpick):
    """65 .. 90 short sequences per batch (many sequences share a chunk
    boundary region and the kept_cu offsets run over all of them)."""
    rng = np.random.default_rng(seed)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    b = rng.standard_normal(T) if mode < 3 else rng.integers(-2, 3, T).astype(np.float64)
    pr = (rng.random(T) < 0.8).astype(np.uint8)
    k = []
    for s in range(len(lens)):
        n_p = int(pr[cu[s]:cu[s + 1]].sum())
        k.append([0, 1, max(n_p - 1, 0), n_p, n_p + 7, n_p // 3][(kpick + s) % 6])
    say(f"select hypothesis: {len(lens)} sequences, T={T}")
    check_select(b, pr, cu, k, f"{len(lens)} sequences")


@settings(max_examples=25, **SETTINGS)
@given(n_src=st.integers(1, 4000), n_rows=st.integers(1, 4000), row_words=st.integers(1, 700),
       seed=st.integers(0, 2 ** 31 - 1))
def test_gather_hypothesis(n_src, n_rows, row_words, seed):
    """Rows of 4 .. 2800 bytes: multiples of 16 take the vector path, the
    others the 4-byte path."""
    from learned_token_pruning_06_amd import ops
    rng = np.random.default_rng(seed)
    src = rng.integers(-2 ** 31, 2 ** 31, (n_src, row_words), dtype=np.int64).astype(np.int32)
    idx = rng.integers(0, n_src, n_rows).astype(np.int32)
    say(f"gather hypothesis: {n_rows} of {n_src} rows, {4 * row_words} B")
    out = ops.gather(torch.from_numpy(src).cuda(), i32_dev(idx))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), O.ref_gather(src, idx))


@settings(max_examples=20, **SETTINGS)
@given(T=st.integers(1, 3000), d=st.sampled_from([64, 128, 192, 256, 512]),
       h=st.sampled_from([32, 64, 96, 128, 160, 192, 224, 256]),
       cuts=st.lists(st.floats(0.0, 1.0), max_size=3), seed=st.integers(0, 2 ** 31 - 1))
def test_score_hypothesis(T, d, h, cuts, seed):
    rng = np.random.default_rng(seed)
    inner = sorted({int(c * T) for c in cuts})
    cu = np.array([0] + inner + [T], np.int32)
    g = dict(x=f32_to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32)),
             w1=f32_to_bf16_bits((rng.standard_normal((h, d)) / np.sqrt(d)).astype(np.float32)),
             b1=(0.1 * rng.standard_normal(h)).astype(np.float32),
             w2=(rng.standard_normal(h) / np.sqrt(h)).astype(np.float32),
             b2=float(rng.uniform(-1, 1)),
             prunable=(rng.random(T) < 0.85).astype(np.uint8), cu_seqlens=cu)
    say(f"score hypothesis: T={T} d={d} h={h} cu={cu.tolist()}")
    _check_score(g, True, f"T={T} d={d} h={h}")


ATTN_LEN = st.one_of(st.sampled_from([0, 1, 63, 64, 65, 127, 128, 129]), st.integers(0, 600))
HEADS = [(16, 8), (8, 8), (16, 4), (32, 4), (4, 1), (8, 2)]


@settings(max_examples=25, **SETTINGS)
@given(lens=st.lists(ATTN_LEN, min_size=1, max_size=3).filter(lambda l: 0 < sum(l) <= 1200),
       heads=st.sampled_from(HEADS), dh=st.sampled_from([64, 128]),
       dtype=st.sampled_from(["bf16", "bf16", "f32"]), with_pos=st.booleans(),
       prompt=st.sampled_from([0, 8, 64]), seed=st.integers(0, 2 ** 31 - 1))
def test_attn_hypothesis(lens, heads, dh, dtype, with_pos, prompt, seed):
    hq, hkv = heads
    say(f"attn hypothesis: lens={lens} hq={hq} hkv={hkv} dh={dh} {dtype} pos={with_pos}")
    q, k, v, kb, pos, kc, gain, temp = synth_case(seed, lens, hq, hkv, dh, dtype,
                                                  with_pos=with_pos, prompt=prompt)
    got = run_attn(q, k, v, kb, pos, kc, gain, temp, dtype)
    ref = O.ref_gated_attn(q, k, v, kb, pos, kc, gain, temp)
    err = rel_l2(got, ref)
    assert err <= ATTN_TOL[dtype], f"rel-L2 {err:.3e}"


# head layouts the fused norm + rotary projection takes: hq * dh and hkv * dh
# multiples of 128, (hq + 2 hkv) * dh a multiple of 256
ROPE_HEADS = [(4, 2, 64), (2, 1, 128), (8, 4, 64), (4, 1, 128), (8, 2, 64), (6, 1, 128)]


@settings(max_examples=15, **SETTINGS)
@given(t=st.one_of(st.sampled_from([1, 255, 256, 257, 511]), st.integers(1, 700)),
       d=st.sampled_from([64, 128, 192, 256, 512]), heads=st.sampled_from(ROPE_HEADS),
       norm=st.sampled_from(["none", "q", "k", "both"]),
       theta=st.sampled_from([0.0, 1e4, 5e5, 1e6]), seed=st.integers(0, 2 ** 31 - 1))
def test_proj_rope_hypothesis(t, d, heads, norm, theta, seed):
    """tg_qkv_proj_rope on drawn shapes, norm weights and rotary bases, with
    positions anywhere below 2^20, against ref_project_qk_rope under the
    element bound of test_parity_proj (one bf16 rounding plus 1e-3 of the
    RMS)."""
    from test_parity_proj import _check_rope
    hq, hkv, dh = heads
    rng = np.random.default_rng(seed)
    bf = lambda a: f32_to_bf16_bits(np.asarray(a, np.float32))
    x = bf(rng.standard_normal((t, d)))
    s = 1.0 / np.sqrt(d)
    wq, wk, wv = (bf(rng.standard_normal((d, n * dh)) * s) for n in (hq, hkv, hkv))
    pos = rng.integers(0, 1 << 20, t).astype(np.int32)
    wts = lambda: (1.0 + 0.3 * rng.standard_normal(dh)).astype(np.float32)
    qn = wts() if norm in ("q", "both") else None
    kn = wts() if norm in ("k", "both") else None
    say(f"proj+rope hypothesis: t={t} d={d} {hq}/{hkv}x{dh} norm={norm} theta={theta:g}")
    _check_rope(x, wq, wk, wv, hq, hkv, dh, pos if theta > 0 else None, qn, kn, theta,
                f"t={t} d={d}")
