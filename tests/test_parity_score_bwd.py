"""tg_score_bwd against the oracle's scorer backward (ref_score_bwd, fp64,
pinned by central differences and torch autograd).

The oracle is fed the values the kernel reads (bf16 rows and weights
rounded the same way, the forward's raw scores rounded to fp32 as the
kernel receives them).  fp32 arithmetic (fp32 inputs, or shapes outside the
matrix-core path): rel-L2 <= 1e-5 for dx, dW1, db1 and dw2 (fp32 sums over
<= 2^14 terms).  bf16 inputs with h = 256 and d % 256 == 0 run dW1 and dx on
the matrix cores with dz rounded to bf16 (relative 2^-8 per term): those two
take the bf16 bar, rel-L2 <= 1e-2; db1 and dw2 come from the fp32 values.
db2 is a sum of terms of both signs over every prunable token, so its bar
is |got - ref| <= 1e-5 (|ref| + sum |db~|).

The LN2-fused form (norm_eps >= 0) is checked against
ref_score_prenorm_bwd with the norm's weight folded into W1 (gamma None in
the oracle, the folded weights as the kernel reads them), at the same bars:
dx is then the gradient at the residual rows, dW1 the one at the folded
weight (the unfolding is pinned on the CPU)."""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import bf16_dev, f32_dev, i32_dev, rel_l2, round_bf16, say, u8_dev
from workloads import bf16_to_f64

pytestmark = pytest.mark.gpu

TOL = 1e-5
EPS = 1e-6


def sbwd_case(seed, T, d, h, lens, budgets, dtype, norm_eps=None):
    """norm_eps set: x rows are residual rows (mean 0.5, RMS about 3, row 0
    all zeros when T > 2) and w1 carries a folded norm weight in [0.5, 1.5]."""
    rng = np.random.default_rng(seed)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    assert cu[-1] == T

    def grid(a):
        return bf16_to_f64(round_bf16(a)) if dtype == "bf16" else a.astype(np.float32).astype(np.float64)
    if norm_eps is None:
        x = grid(rng.standard_normal((T, d)))
        w1 = grid(rng.standard_normal((h, d)) / np.sqrt(d))
    else:
        a = 3.0 * rng.standard_normal((T, d)) + 0.5
        if T > 2:
            a[0] = 0.0
        x = grid(a)
        gamma = rng.uniform(0.5, 1.5, d)
        w1 = grid(rng.standard_normal((h, d)) / np.sqrt(d) * gamma[None, :])
    b1 = (0.1 * rng.standard_normal(h)).astype(np.float32)
    w2 = (rng.standard_normal(h) / np.sqrt(h)).astype(np.float32)
    b2 = 0.125
    pr = (rng.random(T) < 0.85).astype(np.uint8)
    if norm_eps is None:
        raw = O.ref_score(x, w1, b1, w2, b2)
    else:
        raw = O.ref_score_prenorm(x, None, norm_eps, w1, b1, w2, b2)
    raw32 = raw.astype(np.float32)
    b, _ = O.ref_normalise(raw32.astype(np.float64), pr, cu, EPS)
    kept_idx, _, _, kept_cu = O.ref_select(b.astype(np.float32), pr, cu, budgets)
    db_kept = rng.standard_normal(len(kept_idx)).astype(np.float32)
    return dict(x=x, w1=w1, b1=b1, w2=w2, b2=b2, pr=pr, cu=cu, raw32=raw32,
                kept_idx=np.asarray(kept_idx, np.int32), kept_cu=np.asarray(kept_cu, np.int32),
                db_kept=db_kept, norm_eps=norm_eps)


def run(c, dtype):
    from learned_token_pruning_06_amd import ops
    dev = (lambda a: bf16_dev(round_bf16(a))) if dtype == "bf16" else f32_dev
    out = ops.score_bwd(dev(c["x"]), dev(c["w1"]), f32_dev(c["w2"]), u8_dev(c["pr"]),
                        i32_dev(c["cu"]), f32_dev(c["raw32"]), i32_dev(c["kept_idx"]),
                        i32_dev(c["kept_cu"]), f32_dev(c["db_kept"]), b1=f32_dev(c["b1"]), eps=EPS,
                        norm_eps=-1.0 if c["norm_eps"] is None else c["norm_eps"])
    torch.cuda.synchronize()
    return [t.cpu().numpy().astype(np.float64) for t in out]


def check(c, dtype):
    mfma = dtype == "bf16" and c["w1"].shape[0] == 256 and c["x"].shape[1] % 256 == 0
    got = run(c, dtype)
    if c["norm_eps"] is None:
        *ref, scale = O.ref_score_bwd(c["x"], c["w1"], c["b1"], c["w2"], c["b2"], c["pr"],
                                      c["cu"], c["kept_idx"], c["kept_cu"], c["db_kept"], eps=EPS,
                                      error_scales=True)
    else:
        da, dw1, _, db1, dw2, db2, scale = O.ref_score_prenorm_bwd(
            c["x"], None, c["norm_eps"], c["w1"], c["b1"], c["w2"], c["b2"], c["pr"], c["cu"],
            c["kept_idx"], c["kept_cu"], c["db_kept"], eps=EPS, error_scales=True)
        ref = [da, dw1, db1, dw2, db2]
    errs = {n: rel_l2(g, r) for n, g, r in zip(("dx", "dw1", "db1", "dw2"), got[:4], ref[:4])}
    errs["db2"] = abs(float(got[4][0]) - ref[4]) / (abs(ref[4]) + scale)
    say("  " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    for n, e in errs.items():
        bar = 1e-2 if (mfma and n in ("dx", "dw1")) else TOL
        assert e <= bar, f"{n}: {e:.3e} > {bar}"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_score_bwd_small(dtype):
    say(f"score bwd {dtype}: T=300 d=64 h=64, three sequences (one empty)")
    check(sbwd_case(1, 300, 64, 64, [100, 0, 200], [10, 5, 30], dtype), dtype)


def test_score_bwd_ragged_bf16():
    say("score bwd bf16: T=2560 d=2048 h=256, ragged sequences")
    check(sbwd_case(2, 2560, 2048, 256, [1, 255, 256, 257, 1791], [1, 16, 0, 300, 200], "bf16"),
          "bf16")


def test_score_bwd_16k_layer():
    """The 16k-token gated layer: 15872 document + 512 prompt tokens (here a
    random 85% prunable mask), K = 1984."""
    say("score bwd bf16: 16384 tokens, d 2048, h 256")
    check(sbwd_case(3, 16384, 2048, 256, [16384], [1984], "bf16"), "bf16")


@pytest.mark.parametrize("d", [256, 512])
def test_score_bwd_256_row_tiles(d):
    """70000 tokens: the recomputation of z takes 256-row tiles (the ragged
    last one holds 112 rows); bf16 rows on the matrix-core path."""
    say(f"score bwd bf16: 70000 tokens, d {d}, h 256")
    check(sbwd_case(5 + d, 70000, d, 256, [1, 40000, 29999], [1, 3000, 2000], "bf16"), "bf16")


def test_score_bwd_deterministic():
    c = sbwd_case(4, 3000, 2048, 256, [3000], [400], "bf16")
    a, b = run(c, "bf16"), run(c, "bf16")
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


# ---- the LN2-fused form (norm_eps >= 0)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_score_bwd_ln2_small(dtype):
    """Vector path (h = 64): three sequences (one empty), an all-zero
    residual row (its 1 / RMS is 1 / sqrt(norm_eps))."""
    say(f"score bwd LN2 {dtype}: T=300 d=64 h=64")
    check(sbwd_case(11, 300, 64, 64, [100, 0, 200], [10, 5, 30], dtype, norm_eps=1e-6), dtype)


def test_score_bwd_ln2_f32_wide():
    """Vector path with several 64-unit hidden blocks (h = 192: the row's
    norm term sums three partials) and d = 320."""
    say("score bwd LN2 f32: T=700 d=320 h=192")
    check(sbwd_case(12, 700, 320, 192, [1, 699], [1, 100], "f32", norm_eps=1e-5), "f32")


def test_score_bwd_ln2_ragged_bf16():
    """Matrix-core path, 64-row tiles: the norm term is subtracted in the dx
    product's epilogue."""
    say("score bwd LN2 bf16: T=2560 d=2048 h=256, ragged sequences")
    check(sbwd_case(13, 2560, 2048, 256, [1, 255, 256, 257, 1791], [1, 16, 0, 300, 200], "bf16",
                    norm_eps=1e-6), "bf16")


def test_score_bwd_ln2_128_row_tiles():
    """70000 tokens: the recomputation takes 128-row tiles (the row's norm
    term sums the four waves that split its hidden units)."""
    say("score bwd LN2 bf16: 70000 tokens, d 512, h 256")
    check(sbwd_case(14, 70000, 512, 256, [1, 40000, 29999], [1, 3000, 2000], "bf16",
                    norm_eps=1e-6), "bf16")


def test_score_bwd_ln2_deterministic():
    c = sbwd_case(15, 3000, 2048, 256, [3000], [400], "bf16", norm_eps=1e-6)
    a, b = run(c, "bf16"), run(c, "bf16")
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("norm_eps", [None, 1e-5])
def test_score_bwd_single_token_sequences(norm_eps):
    """500 sequences of one token each, all budgets 1.  For a prunable token
    the two terms of db~ nearly cancel (db eps / r^3 is left, r^2 = b~^2 +
    eps), so they are formed in fp64 and rounded once.  Besides the usual
    bars, every row of dx is held to 1e-4 of its own norm: the rows with
    |b~| >> sqrt(eps) have tiny gradients that rel-L2 over all rows does not
    see, and an fp32 difference of the two terms measured ~1e-2 on them."""
    lens, budgets = [1] * 500, [1] * 500
    tag = "plain" if norm_eps is None else "LN2"
    say(f"score bwd {tag} f32: 500 sequences of one token")
    c = sbwd_case(17, 500, 128, 64, lens, budgets, "f32", norm_eps=norm_eps)
    check(c, "f32")
    got = run(c, "f32")[0]
    if norm_eps is None:
        ref = O.ref_score_bwd(c["x"], c["w1"], c["b1"], c["w2"], c["b2"], c["pr"], c["cu"],
                              c["kept_idx"], c["kept_cu"], c["db_kept"], eps=EPS)[0]
    else:
        ref = O.ref_score_prenorm_bwd(c["x"], None, norm_eps, c["w1"], c["b1"], c["w2"],
                                      c["b2"], c["pr"], c["cu"], c["kept_idx"], c["kept_cu"],
                                      c["db_kept"], eps=EPS)[0]
    rn = np.linalg.norm(ref, axis=1)
    live = rn > 0
    assert np.all(np.linalg.norm(got, axis=1)[~live] == 0.0)       # prompt tokens
    worst = float(np.max(np.linalg.norm(got - ref, axis=1)[live] / rn[live]))
    say(f"  worst row of dx: {worst:.2e} of its norm")
    assert worst <= 1e-4


@pytest.mark.parametrize("norm_eps", [None, 1e-6])
def test_score_bwd_128k_step(norm_eps):
    """The benchmark's configuration: 131072 tokens (the last 512 prompt
    tokens), d 2048, h 256, K = 8192, bf16 rows on the matrix-core path; dW1,
    db1, dw2, db2 in full, dx on 64 sampled rows (first and last rows, tile
    edges, the last document and first prompt row, random), at the bars of
    the smaller cases."""
    T, d, h = 131072, 2048, 256
    rng = np.random.default_rng(99 if norm_eps is None else 98)
    tag = "plain" if norm_eps is None else "LN2"
    say(f"score bwd {tag} bf16: the 128k step, T={T} d={d} h={h} K=8192")
    c = sbwd_case(21 if norm_eps is None else 22, T, d, h, [T], [8192], "bf16", norm_eps=norm_eps)
    c["pr"][:] = 1
    c["pr"][T - 512:] = 0
    # the kept set and db for this prompt layout (the case drew its own mask)
    if norm_eps is None:
        raw = O.ref_score(c["x"], c["w1"], c["b1"], c["w2"], c["b2"])
    else:
        raw = O.ref_score_prenorm(c["x"], None, norm_eps, c["w1"], c["b1"], c["w2"], c["b2"])
    c["raw32"] = raw.astype(np.float32)
    b, _ = O.ref_normalise(c["raw32"].astype(np.float64), c["pr"], c["cu"], EPS)
    ki, _, _, kc = O.ref_select(b.astype(np.float32), c["pr"], c["cu"], [8192])
    c["kept_idx"], c["kept_cu"] = np.asarray(ki, np.int32), np.asarray(kc, np.int32)
    c["db_kept"] = rng.standard_normal(len(ki)).astype(np.float32)
    got = run(c, "bf16")
    if norm_eps is None:
        *ref, scale = O.ref_score_bwd(c["x"], c["w1"], c["b1"], c["w2"], c["b2"], c["pr"],
                                      c["cu"], c["kept_idx"], c["kept_cu"], c["db_kept"], eps=EPS,
                                      error_scales=True)
    else:
        da, dw1, _, db1, dw2, db2, scale = O.ref_score_prenorm_bwd(
            c["x"], None, norm_eps, c["w1"], c["b1"], c["w2"], c["b2"], c["pr"], c["cu"],
            c["kept_idx"], c["kept_cu"], c["db_kept"], eps=EPS, error_scales=True)
        ref = [da, dw1, db1, dw2, db2]
    rows = np.unique(np.concatenate([[0, 1, 127, 128, 255, 256, T - 513, T - 512, T - 1],
                                     rng.choice(T, 55, replace=False)]))
    errs = {"dx": rel_l2(got[0][rows], ref[0][rows]), "dw1": rel_l2(got[1], ref[1]),
            "db1": rel_l2(got[2], ref[2]), "dw2": rel_l2(got[3], ref[3]),
            "db2": abs(float(got[4][0]) - ref[4]) / (abs(ref[4]) + scale)}
    say("  " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    for n, e in errs.items():
        bar = 1e-2 if n in ("dx", "dw1") else TOL
        assert e <= bar, f"{n}: {e:.3e} > {bar}"
