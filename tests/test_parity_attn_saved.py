"""The forward's row statistic and the backward that takes it.

tg_gated_attn's optional lse2 output against ref_gated_attn_lse2 (fp64).
The kernel forms the normaliser from bf16-rounded probabilities (the ones
that enter P.V, each within 2^-8 relative: bf16 keeps 8 significant bits),
so its base-2 log is within log2(1 + 2^-8) = 5.6e-3 of the exact one, plus
the fp32 error of the logits; the bar is |got - ref| <= 5.6e-3 + 1e-5 |ref|
(gpu_util.LSE2_ABS, LSE2_REL).

tg_gated_attn_bwd with fwd_out and fwd_lse2 against ref_gated_attn_bwd,
with the saved state taken (a) from the oracle (its output rounded to bf16,
its lse2 to fp32) and (b) from tg_gated_attn itself, the pipeline a training
step runs.  D = dout . out then carries out's bf16 rounding (2^-8 relative),
which reaches every gradient through dl = P (dP - D): all six take the bf16
bar, rel-L2 <= 1e-2, and dgain, dtemp the same bar relative to the oracle's
error scale plus the value."""
import math

import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import (LSE2_ABS, bf16_dev, f32_dev, i32_dev, lse2_excess, rel_l2, round_bf16,
                      say)
from test_parity_attn_bwd import NAMES, bwd_case
from workloads import bf16_to_f64

pytestmark = pytest.mark.gpu

BAR = 1e-2


def _dev(case):
    q, k, v, do, kb, pos, kc, gain, temp = case
    return ([bf16_dev(round_bf16(a)) for a in (q, k, v, do)], f32_dev(kb),
            None if pos is None else i32_dev(pos), i32_dev(kc), f32_dev(gain), f32_dev(temp))


@pytest.mark.parametrize("dh,hq,hkv,lens", [(128, 16, 8, [1, 5, 31, 64, 65, 130]),
                                            (64, 4, 1, [300, 0, 77]),
                                            (128, 8, 8, [2496])])
def test_forward_lse2_matches_oracle(dh, hq, hkv, lens):
    from learned_token_pruning_06_amd import ops
    case = bwd_case(200 + dh + hq, lens, hq, hkv, dh, "bf16")
    q, k, v, do, kb, pos, kc, gain, temp = case
    (qd, kd, vd, _), kbd, posd, kcd, gd, td = _dev(case)
    t = q.shape[0]
    lse2 = torch.full((hq, t), float("nan"), device=qd.device)
    say(f"attn lse2: dh={dh} {hq}/{hkv} lens={lens}")
    ops.gated_attn(qd, kd, vd, kbd, posd, kcd, gd, td, lse2=lse2)
    torch.cuda.synchronize()
    got = lse2.cpu().numpy().astype(np.float64).T
    ref = O.ref_gated_attn_lse2(q, k, kb, pos, kc, gain, temp)
    err = lse2_excess(got, ref)
    say(f"  worst |d lse2| beyond 1e-5 |ref|: {err:.2e}")
    assert np.all(np.isfinite(got))
    assert err <= LSE2_ABS


def _check(got, case, tag):
    q, k, v, do, kb, pos, kc, gain, temp = case
    *ref, sgain, stemp = O.ref_gated_attn_bwd(q, k, v, kb, pos, kc, gain, temp, do,
                                              error_scales=True)
    scale = {"dgain": sgain, "dtemp": stemp}
    errs = {}
    for name, g, r in zip(NAMES, got, ref):
        g = g.cpu().numpy().astype(np.float64)
        errs[name] = (float(np.max(np.abs(g - r) / (np.abs(r) + scale[name])))
                      if name in scale else rel_l2(g, r))
    say(f"  {tag}: " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    for name, e in errs.items():
        assert e <= BAR, f"{name}: {e:.3e} > {BAR}"


@pytest.mark.parametrize("source", ["oracle", "forward"])
@pytest.mark.parametrize("dh,hq,hkv,lens", [(128, 16, 8, [1, 5, 31, 32, 33, 64, 65, 130]),
                                            (64, 16, 2, [200, 57]),
                                            (128, 16, 8, [2496])])
def test_bwd_with_saved_state_matches_oracle(source, dh, hq, hkv, lens):
    from learned_token_pruning_06_amd import ops
    case = bwd_case(300 + dh + hq + len(lens), lens, hq, hkv, dh, "bf16")
    q, k, v, do, kb, pos, kc, gain, temp = case
    (qd, kd, vd, dod), kbd, posd, kcd, gd, td = _dev(case)
    t = q.shape[0]
    say(f"attn bwd, saved state from the {source}: dh={dh} {hq}/{hkv} lens={lens}")
    if source == "oracle":
        fo = bf16_dev(round_bf16(O.ref_gated_attn(q, k, v, kb, pos, kc, gain, temp)))
        fl = f32_dev(np.ascontiguousarray(O.ref_gated_attn_lse2(q, k, kb, pos, kc, gain, temp).T))
    else:
        fl = torch.empty((hq, t), dtype=torch.float32, device=qd.device)
        fo = ops.gated_attn(qd, kd, vd, kbd, posd, kcd, gd, td, lse2=fl)
    got = ops.gated_attn_bwd(qd, kd, vd, dod, kbd, posd, kcd, gd, td, fwd_out=fo, fwd_lse2=fl)
    torch.cuda.synchronize()
    _check(got, case, source)


def test_bwd_saved_state_close_to_recomputed():
    """Both modes on the same inputs agree to the bf16 bar, and the saved-state
    mode is deterministic."""
    from learned_token_pruning_06_amd import ops
    case = bwd_case(400, [700, 301], 16, 8, 128, "bf16")
    (qd, kd, vd, dod), kbd, posd, kcd, gd, td = _dev(case)
    fl = torch.empty((16, qd.shape[0]), dtype=torch.float32, device=qd.device)
    fo = ops.gated_attn(qd, kd, vd, kbd, posd, kcd, gd, td, lse2=fl)
    a = ops.gated_attn_bwd(qd, kd, vd, dod, kbd, posd, kcd, gd, td)
    b = ops.gated_attn_bwd(qd, kd, vd, dod, kbd, posd, kcd, gd, td, fwd_out=fo, fwd_lse2=fl)
    c = ops.gated_attn_bwd(qd, kd, vd, dod, kbd, posd, kcd, gd, td, fwd_out=fo, fwd_lse2=fl)
    torch.cuda.synchronize()
    for name, x, y, z in zip(NAMES, a, b, c):
        assert torch.equal(y, z), name
        if name in ("dq", "dk", "dv", "db"):
            e = rel_l2(y.cpu().numpy().astype(np.float64), x.cpu().numpy().astype(np.float64))
            say(f"  {name}: saved vs recomputed rel-L2 {e:.2e}")
            assert e <= BAR


# ---- the 128k step's attention backward at full size, on sampled rows
_STEP = {}


def _step_case():
    """The 128k step's kept rows: 8192 document tokens at sorted random
    positions below 130560 and the 512 prompt tokens after them (b = 0),
    16 query / 8 KV heads of dim 128, bf16 operands."""
    if "case" not in _STEP:
        rng = np.random.default_rng(4242)
        T, hq, hkv, dh = 8704, 16, 8, 128
        grid = lambda shape, sc=1.0: bf16_to_f64(round_bf16(rng.standard_normal(shape) * sc))
        q, k, v = grid((T, hq, dh)), grid((T, hkv, dh)), grid((T, hkv, dh))
        do = grid((T, hq, dh), 0.5)
        pos = np.concatenate([np.sort(rng.choice(130560, 8192, replace=False)),
                              np.arange(130560, 131072)]).astype(np.int64)
        kb = rng.standard_normal(T).astype(np.float32).astype(np.float64)
        kb[8192:] = 0.0
        kc = np.array([0, T], np.int64)
        gain = rng.uniform(0.5, 1.5, hq).astype(np.float32)
        temp = rng.uniform(0.8, 1.2, hq).astype(np.float32)
        samp = np.unique(np.concatenate([[0, 1, 63, 64, 127, 128, 129, 4095, 4096, 8191, 8192,
                                          8703], rng.choice(T, 20, replace=False)]))
        _STEP["case"] = (q, k, v, do, kb, pos, kc, gain, temp)
        _STEP["rows"] = samp
    return _STEP["case"], _STEP["rows"]


def _step_ref():
    if "ref" not in _STEP:
        (q, k, v, do, kb, pos, kc, gain, temp), rows = _step_case()
        say("  oracle: 128k step backward at the sampled rows (all rows' statistics)")
        _STEP["ref"] = O.ref_gated_attn_bwd_rows(q, k, v, kb, pos, kc, gain, temp, do, rows, rows)
    return _STEP["ref"]


@pytest.mark.parametrize("mode", ["saved", "recompute"])
def test_bwd_128k_step_sampled_rows(mode):
    """All 8704 kept rows of the 128k step through the GPU backward (with the
    forward's output and lse2, as the benchmark times it, or recomputing the
    statistics); dq at 32 sampled query rows and dk, dv, db at the same
    rows as keys, against the oracle, per tensor and per head: rel-L2 <= 1e-2
    (P and dS enter the products in bf16; with the saved state D also carries
    out's bf16 rounding); db without the saved state within 1e-5 (fp32)."""
    from learned_token_pruning_06_amd import ops
    case, rows = _step_case()
    q, k, v, do, kb, pos, kc, gain, temp = case
    (qd, kd, vd, dod), kbd, posd, kcd, gd, td = _dev(case)
    say(f"attn bwd 128k step ({mode}): T=8704, 16/8 heads, dh=128")
    if mode == "saved":
        lse2 = torch.empty((16, 8704), dtype=torch.float32, device=qd.device)
        out = ops.gated_attn(qd, kd, vd, kbd, posd, kcd, gd, td, lse2=lse2)
        got = ops.gated_attn_bwd(qd, kd, vd, dod, kbd, posd, kcd, gd, td, fwd_out=out,
                                 fwd_lse2=lse2)
    else:
        got = ops.gated_attn_bwd(qd, kd, vd, dod, kbd, posd, kcd, gd, td)
    torch.cuda.synchronize()
    rq, rk, rv, rb = _step_ref()
    idx = torch.as_tensor(rows, device=qd.device)
    g = [got[i].index_select(0, idx).cpu().numpy().astype(np.float64) for i in range(4)]
    errs = {"dq": rel_l2(g[0], rq), "dk": rel_l2(g[1], rk), "dv": rel_l2(g[2], rv),
            "db": rel_l2(g[3], rb)}
    heads = {"dq": max(rel_l2(g[0][:, h], rq[:, h]) for h in range(16)),
             "dk": max(rel_l2(g[1][:, h], rk[:, h]) for h in range(8)),
             "dv": max(rel_l2(g[2][:, h], rv[:, h]) for h in range(8))}
    say("  " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()) + "  worst head "
        + " ".join(f"{n}={e:.2e}" for n, e in heads.items()))
    bars = {"dq": 1e-2, "dk": 1e-2, "dv": 1e-2, "db": 1e-2 if mode == "saved" else 1e-5}
    for n, e in errs.items():
        assert e <= bars[n], f"{n}: {e:.3e} > {bars[n]}"
    for n, e in heads.items():
        assert e <= 1e-2, f"worst head of {n}: {e:.3e}"
