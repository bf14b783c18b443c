"""tg_score_bwd against the oracle's scorer backward (ref_score_bwd, fp64,
pinned by central differences and torch autograd).

The oracle is fed the values the kernel reads (bf16 rows and weights
rounded the same way, the forward's raw scores rounded to fp32 as the
kernel receives them).  fp32 arithmetic (fp32 inputs, or shapes outside the
matrix-core path): rel-L2 <= 1e-5 for dx, dW1, db1 and dw2 (fp32 sums over
<= 2^14 terms).  bf16 inputs with h = 256 and d % 256 == 0 run dW1 and dx on
the matrix cores with dz rounded to bf16 (relative 2^-9 per term): those two
take the bf16 bar, rel-L2 <= 1e-2; db1 and dw2 come from the fp32 values.
db2 is a sum of terms of both signs over every prunable token, so its bar
is |got - ref| <= 1e-5 (|ref| + sum |db~|)."""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import bf16_dev, f32_dev, i32_dev, rel_l2, round_bf16, say, u8_dev
from workloads import bf16_to_f64

pytestmark = pytest.mark.gpu

TOL = 1e-5
EPS = 1e-6


def sbwd_case(seed, T, d, h, lens, budgets, dtype):
    rng = np.random.default_rng(seed)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    assert cu[-1] == T

    def grid(a):
        return bf16_to_f64(round_bf16(a)) if dtype == "bf16" else a.astype(np.float32).astype(np.float64)
    x = grid(rng.standard_normal((T, d)))
    w1 = grid(rng.standard_normal((h, d)) / np.sqrt(d))
    b1 = (0.1 * rng.standard_normal(h)).astype(np.float32)
    w2 = (rng.standard_normal(h) / np.sqrt(h)).astype(np.float32)
    b2 = 0.125
    pr = (rng.random(T) < 0.85).astype(np.uint8)
    raw = O.ref_score(x, w1, b1, w2, b2)
    raw32 = raw.astype(np.float32)
    b, _ = O.ref_normalise(raw32.astype(np.float64), pr, cu, EPS)
    kept_idx, _, _, kept_cu = O.ref_select(b.astype(np.float32), pr, cu, budgets)
    db_kept = rng.standard_normal(len(kept_idx)).astype(np.float32)
    return dict(x=x, w1=w1, b1=b1, w2=w2, b2=b2, pr=pr, cu=cu, raw32=raw32,
                kept_idx=np.asarray(kept_idx, np.int32), kept_cu=np.asarray(kept_cu, np.int32),
                db_kept=db_kept)


def run(c, dtype):
    from learned_token_pruning_06_amd import ops
    dev = (lambda a: bf16_dev(round_bf16(a))) if dtype == "bf16" else f32_dev
    out = ops.score_bwd(dev(c["x"]), dev(c["w1"]), f32_dev(c["w2"]), u8_dev(c["pr"]),
                        i32_dev(c["cu"]), f32_dev(c["raw32"]), i32_dev(c["kept_idx"]),
                        i32_dev(c["kept_cu"]), f32_dev(c["db_kept"]), b1=f32_dev(c["b1"]), eps=EPS)
    torch.cuda.synchronize()
    return [t.cpu().numpy().astype(np.float64) for t in out]


def check(c, dtype):
    mfma = dtype == "bf16" and c["w1"].shape[0] == 256 and c["x"].shape[1] % 256 == 0
    got = run(c, dtype)
    *ref, scale = O.ref_score_bwd(c["x"], c["w1"], c["b1"], c["w2"], c["b2"], c["pr"], c["cu"],
                                  c["kept_idx"], c["kept_cu"], c["db_kept"], eps=EPS,
                                  error_scales=True)
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
