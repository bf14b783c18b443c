"""tg_qkv_proj (the projections of the kept rows) against the fp64 oracle.
The kernel rounds its fp32 accumulators to bf16, so besides the rel-L2 bar of
1e-2 every element must lie within one bf16 rounding (2^-8 relative) plus a
small accumulation allowance of the fp64 result."""
import numpy as np
import pytest

import oracle as O
from gpu_util import bf16_dev, rel_l2, say, to_f64, workload
from workloads import bf16_to_f64, f32_to_bf16_bits

pytestmark = pytest.mark.gpu

REL_L2 = 1e-2


def _weights_rows(wq, wk, wv):
    """[d, n] projection matrices (bf16 bits) -> one [(nq + 2 nkv), d] weight, rows = features."""
    return np.ascontiguousarray(np.concatenate([wq.T, wk.T, wv.T], axis=0))


def _check(x_bits, wq, wk, wv, hq, hkv, dh, tag, rows=None):
    from learned_token_pruning_06_amd import ops
    w = _weights_rows(wq, wk, wv)
    q, k, v = ops.qkv_proj(bf16_dev(x_bits), bf16_dev(w), hq, hkv, dh)
    sel = np.arange(x_bits.shape[0]) if rows is None else rows
    xr = bf16_to_f64(x_bits[sel])
    rq, rk, rv = O.ref_project(xr, bf16_to_f64(wq), bf16_to_f64(wk), bf16_to_f64(wv), hq, hkv, dh)
    worst = 0.0
    for name, got, ref in (("q", q, rq), ("k", k, rk), ("v", v, rv)):
        g = to_f64(got)[sel]
        err = rel_l2(g, ref)
        scale = np.sqrt(np.mean(ref ** 2))
        bound = 2.0 ** -8 * np.abs(ref) + 1e-3 * scale
        over = float(np.max(np.abs(g - ref) - bound))
        say(f"proj {tag} {name}: rel-L2 {err:.2e}, worst excess over the element bound {over:.2e}")
        assert err <= REL_L2
        assert over <= 0.0
        worst = max(worst, err)
    return worst


@pytest.mark.parametrize("t,d,hq,hkv,dh", [(1, 64, 2, 1, 64), (300, 256, 4, 2, 64),
                                          (257, 128, 4, 4, 64), (511, 512, 8, 4, 64),
                                          (640, 256, 2, 1, 128)])
def test_proj_synthetic_shapes(t, d, hq, hkv, dh):
    rng = np.random.default_rng(t * 7 + d)
    bf = lambda a: f32_to_bf16_bits(np.asarray(a, np.float32))
    x = bf(rng.standard_normal((t, d)))
    s = 1.0 / np.sqrt(d)
    wq = bf(rng.standard_normal((d, hq * dh)) * s)
    wk = bf(rng.standard_normal((d, hkv * dh)) * s)
    wv = bf(rng.standard_normal((d, hkv * dh)) * s)
    _check(x, wq, wk, wv, hq, hkv, dh, f"t={t} d={d} {hq}/{hkv}x{dh}")


def test_proj_16k_workload_kept_rows():
    """Rows shaped like the 16k layer's kept set (every prompt row and a spread
    of document rows); the projection does not depend on which rows are kept."""
    g = workload(1)
    wl = g["wl"]
    rows = np.concatenate([np.arange(0, wl.t_in - 512, 8), np.arange(wl.t_in - 512, wl.t_in)])
    x = np.ascontiguousarray(g["x"][rows])
    _check(x, g["wq"], g["wk"], g["wv"], wl.hq, wl.hkv, wl.dh, f"16k kept rows ({rows.size})")


def test_proj_128k_kept_size_sampled_rows():
    """The 128k layer's kept size (8192 document + 512 prompt rows) with its own
    weights; the oracle is evaluated on a sample of output rows."""
    g = workload(3)
    wl = g["wl"]
    doc = np.linspace(0, wl.t_in - 513, 8192).astype(np.int64)
    rows_in = np.concatenate([doc, np.arange(wl.t_in - 512, wl.t_in)])
    x = np.ascontiguousarray(g["x"][rows_in])
    t = rows_in.size
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([rng.integers(0, t, 96), [0, 255, 256, t - 1]]))
    _check(x, g["wq"], g["wk"], g["wv"], wl.hq, wl.hkv, wl.dh, f"t={t} sampled", rows=rows)


def test_proj_is_deterministic():
    import torch
    from learned_token_pruning_06_amd import ops
    g = workload(1)
    wl = g["wl"]
    x = bf16_dev(g["x"][:1000])
    w = bf16_dev(_weights_rows(g["wq"], g["wk"], g["wv"]))
    a = ops.qkv_proj(x, w, wl.hq, wl.hkv, wl.dh)
    b = ops.qkv_proj(x, w, wl.hq, wl.hkv, wl.dh)
    for u, v in zip(a, b):
        assert torch.equal(u.view(torch.int16), v.view(torch.int16))


# --------------------------------------------------------------------------
# tg_qkv_proj_rope: per-head RMSNorm of q and k, then the rotary embedding at
# the kept tokens' original positions, fused into the projection's epilogue
# (the oracle's ref_project_qk_rope).  The kernel normalises and rotates the
# fp32 accumulators and rounds once, so the same element bound applies: one
# bf16 rounding of the result plus the accumulation allowance (the angle is
# reduced in fp64, so the rotation adds no error of its order).
# --------------------------------------------------------------------------
def _check_rope(x_bits, wq, wk, wv, hq, hkv, dh, pos, qn, kn, theta, tag, rows=None):
    from learned_token_pruning_06_amd import ops
    from gpu_util import f32_dev, i32_dev
    w = _weights_rows(wq, wk, wv)
    q, k, v = ops.qkv_proj_rope(bf16_dev(x_bits), bf16_dev(w), hq, hkv, dh,
                                pos=None if pos is None else i32_dev(pos),
                                q_norm=None if qn is None else f32_dev(qn),
                                k_norm=None if kn is None else f32_dev(kn),
                                norm_eps=1e-6, rope_theta=theta)
    sel = np.arange(x_bits.shape[0]) if rows is None else rows
    rq, rk, rv = O.ref_project_qk_rope(
        bf16_to_f64(x_bits[sel]), bf16_to_f64(wq), bf16_to_f64(wk), bf16_to_f64(wv), hq, hkv, dh,
        None if pos is None else np.asarray(pos)[sel],
        None if qn is None else qn.astype(np.float64),
        None if kn is None else kn.astype(np.float64), 1e-6, theta)
    for name, got, ref in (("q", q, rq), ("k", k, rk), ("v", v, rv)):
        g = to_f64(got)[sel]
        err = rel_l2(g, ref)
        scale = np.sqrt(np.mean(ref ** 2))
        bound = 2.0 ** -8 * np.abs(ref) + 1e-3 * scale
        over = float(np.max(np.abs(g - ref) - bound))
        say(f"proj+rope {tag} {name}: rel-L2 {err:.2e}, worst excess {over:.2e}")
        assert err <= REL_L2
        assert over <= 0.0


def _rope_case(seed, t, d, hq, hkv, dh, max_pos):
    rng = np.random.default_rng(seed)
    bf = lambda a: f32_to_bf16_bits(np.asarray(a, np.float32))
    x = bf(rng.standard_normal((t, d)))
    s = 1.0 / np.sqrt(d)
    wq = bf(rng.standard_normal((d, hq * dh)) * s)
    wk = bf(rng.standard_normal((d, hkv * dh)) * s)
    wv = bf(rng.standard_normal((d, hkv * dh)) * s)
    # kept positions: increasing with gaps, the first one 0
    pos = np.sort(rng.choice(max_pos, size=t, replace=False)).astype(np.int32)
    pos[0] = 0
    qn = (1.0 + 0.2 * rng.standard_normal(dh)).astype(np.float32)
    kn = (1.0 + 0.2 * rng.standard_normal(dh)).astype(np.float32)
    return x, wq, wk, wv, pos, qn, kn


@pytest.mark.parametrize("t,d,hq,hkv,dh,norm,theta", [
    (1, 64, 4, 2, 64, True, 1e6),          # one row
    (300, 256, 4, 2, 64, True, 1e6),       # two heads per 128 columns
    (257, 128, 2, 1, 128, True, 0.0),      # norm only
    (511, 512, 8, 4, 64, False, 1e4),      # rotation only
    (640, 256, 4, 1, 128, True, 1e6),      # 4 query heads per KV head
    (384, 192, 16, 8, 64, False, 5e5),
])
def test_proj_rope_synthetic_shapes(t, d, hq, hkv, dh, norm, theta):
    x, wq, wk, wv, pos, qn, kn = _rope_case(t + d + dh, t, d, hq, hkv, dh, 1 << 17)
    if not norm:
        qn = kn = None
    _check_rope(x, wq, wk, wv, hq, hkv, dh, pos if theta > 0 else None, qn, kn, theta,
                f"t={t} d={d} {hq}/{hkv}x{dh} norm={norm} theta={theta:g}")


def test_proj_rope_only_k_norm_and_far_positions():
    """A k weight without a q weight, and positions far beyond the 128k
    context (up to 2^30) where the angle runs over many thousands of turns."""
    x, wq, wk, wv, _, _, kn = _rope_case(11, 300, 256, 4, 2, 128, 1 << 17)
    pos = np.random.default_rng(12).integers(0, 1 << 30, 300).astype(np.int32)
    _check_rope(x, wq, wk, wv, 4, 2, 128, pos, None, kn, 1e6, "k norm only, far positions")


def test_proj_rope_off_matches_plain_projection():
    """Neither norm nor rotation: the same accumulators rounded the same way
    as tg_qkv_proj, bit for bit."""
    import torch
    from learned_token_pruning_06_amd import ops
    x, wq, wk, wv, _, _, _ = _rope_case(13, 700, 512, 8, 4, 128, 1 << 17)
    xd, wd = bf16_dev(x), bf16_dev(_weights_rows(wq, wk, wv))
    a = ops.qkv_proj(xd, wd, 8, 4, 128)
    b = ops.qkv_proj_rope(xd, wd, 8, 4, 128)
    for u, w_ in zip(a, b):
        assert torch.equal(u.view(torch.int16), w_.view(torch.int16))


def test_proj_rope_16k_workload_kept_rows():
    """The 16k layer's kept rows at their original positions, with the
    layer's head shape, a rotary base of 10^6 and random norm weights."""
    g = workload(1)
    wl = g["wl"]
    rows = np.concatenate([np.arange(0, wl.t_in - 512, 8), np.arange(wl.t_in - 512, wl.t_in)])
    x = np.ascontiguousarray(g["x"][rows])
    rng = np.random.default_rng(14)
    qn = (1.0 + 0.2 * rng.standard_normal(wl.dh)).astype(np.float32)
    kn = (1.0 + 0.2 * rng.standard_normal(wl.dh)).astype(np.float32)
    _check_rope(x, g["wq"], g["wk"], g["wv"], wl.hq, wl.hkv, wl.dh, rows.astype(np.int32),
                qn, kn, 1e6, f"16k kept rows ({rows.size})")


def test_proj_rope_128k_kept_size_sampled_rows():
    """The 128k layer's kept size at original positions up to 131071; the
    oracle is evaluated on a sample of output rows."""
    g = workload(3)
    wl = g["wl"]
    doc = np.linspace(0, wl.t_in - 513, 8192).astype(np.int64)
    rows_in = np.concatenate([doc, np.arange(wl.t_in - 512, wl.t_in)])
    x = np.ascontiguousarray(g["x"][rows_in])
    t = rows_in.size
    rng = np.random.default_rng(15)
    rows = np.unique(np.concatenate([rng.integers(0, t, 96), [0, 255, 256, t - 1]]))
    qn = (1.0 + 0.2 * rng.standard_normal(wl.dh)).astype(np.float32)
    kn = (1.0 + 0.2 * rng.standard_normal(wl.dh)).astype(np.float32)
    _check_rope(x, g["wq"], g["wk"], g["wv"], wl.hq, wl.hkv, wl.dh, rows_in.astype(np.int32),
                qn, kn, 1e6, f"t={t} sampled", rows=rows)
