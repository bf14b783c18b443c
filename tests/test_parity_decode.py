"""tg_gated_decode against the oracle.

A decode step of token-gated attention is the last query row of the prefill
attention over the same cache rows (the new token's key and value are the
sequence's last cache row; m = cache length, p = its original position + 1),
so the oracle is ref_gated_attn evaluated at those rows only.  The bar is the
bf16 attention bar, rel-L2 <= 1e-2, here per sequence.  Pruning the cache of
a layer to the kept tokens is tg_gather over its rows, checked bit-exact."""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import DEV, bf16_dev, f32_dev, i32_dev, rel_l2, round_bf16, say, to_f64
from workloads import bf16_to_f64

pytestmark = pytest.mark.gpu

TOL = 1e-2


def decode_case(seed, lens, hq, hkv, dh, with_pos=True, with_b=True):
    rng = np.random.default_rng(seed)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T, n_seq = int(cu[-1]), len(lens)
    grid = lambda shape: bf16_to_f64(round_bf16(rng.standard_normal(shape)))
    q, k, v = grid((n_seq, hq, dh)), grid((T, hkv, dh)), grid((T, hkv, dh))
    cb = rng.standard_normal(T).astype(np.float32).astype(np.float64) if with_b else np.zeros(T)
    for s in range(n_seq):
        if lens[s]:
            cb[cu[s + 1] - 1] = 0.0                  # the generated token carries no score
    qpos = np.array([n - 1 + int(rng.integers(0, 4 * n + 1)) if n else 0 for n in lens],
                    np.int64) if with_pos else None
    gain = rng.uniform(0.5, 1.5, hq).astype(np.float32)
    temp = rng.uniform(0.8, 1.2, hq).astype(np.float32)
    return q, k, v, (cb if with_b else None), qpos, cu, gain, temp


def oracle_decode(q, k, v, cb, qpos, cu, gain, temp, seqs=None):
    """Row c_{s+1}-1 of the oracle's prefill attention, with that row's query
    set to the decode query of sequence s."""
    n_seq, hq, dh = q.shape
    T = int(cu[-1])
    qf = np.zeros((T, hq, dh))
    pos = np.zeros(T, np.int64)
    rows = []
    for s in (range(n_seq) if seqs is None else seqs):
        if cu[s + 1] > cu[s]:
            r = int(cu[s + 1]) - 1
            qf[r] = q[s]
            pos[r] = 0 if qpos is None else qpos[s]
            rows.append(r)
    kb = np.zeros(T) if cb is None else cb
    o = O.ref_gated_attn(qf, k, v, kb, None if qpos is None else pos, cu, gain, temp,
                         rows=np.array(rows, np.int64))
    out = np.zeros((n_seq, hq, dh))
    for s in range(n_seq):
        if cu[s + 1] > cu[s]:
            out[s] = o[int(cu[s + 1]) - 1]
    return out


def run_decode(q, k, v, cb, qpos, cu, gain, temp, max_len=None):
    from learned_token_pruning_06_amd import ops
    out = ops.gated_decode(bf16_dev(round_bf16(q)), bf16_dev(round_bf16(k)),
                           bf16_dev(round_bf16(v)), None if cb is None else f32_dev(cb),
                           None if qpos is None else i32_dev(qpos), i32_dev(cu), f32_dev(gain),
                           f32_dev(temp),
                           max_cache_len=int(np.diff(cu).max(initial=0)) if max_len is None
                           else max_len)
    torch.cuda.synchronize()
    return to_f64(out)


def check_per_seq(got, ref, cu, tol=TOL, seqs=None):
    worst = 0.0
    for s in (range(len(cu) - 1) if seqs is None else seqs):
        if cu[s + 1] == cu[s]:
            assert np.all(got[s] == 0.0), f"empty sequence {s} must give zeros"
            continue
        e = rel_l2(got[s], ref[s])
        worst = max(worst, e)
        assert e <= tol, f"sequence {s} (len {cu[s + 1] - cu[s]}): rel-L2 {e:.3e}"
    return worst


LENS = [1, 2, 63, 64, 65, 255, 256, 257, 1000, 3001]


@pytest.mark.parametrize("dh", [128, 64])
@pytest.mark.parametrize("hq,hkv", [(16, 8), (8, 8), (16, 4), (16, 2)])
def test_decode_is_last_prefill_row(dh, hq, hkv):
    say(f"decode dh={dh} hq={hq} hkv={hkv} lens={LENS}")
    case = decode_case(10 + dh + hq + hkv, LENS, hq, hkv, dh)
    got = run_decode(*case)
    ref = oracle_decode(*case)
    worst = check_per_seq(got, ref, case[5])
    assert rel_l2(got, ref) <= TOL
    say(f"  worst per-sequence rel-L2 {worst:.2e}")


def test_decode_without_positions_or_scores():
    """q_pos = NULL gives length factor 1; cache_b = NULL gives b = 0."""
    say("decode q_pos=None cache_b=None")
    case = decode_case(3, [5, 300, 777], 16, 8, 128, with_pos=False, with_b=False)
    check_per_seq(run_decode(*case), oracle_decode(*case), case[5])


def test_decode_single_key_returns_its_value():
    """m = 1: the softmax has one term, the output is v of the new token."""
    case = decode_case(4, [1, 1, 1], 16, 8, 128)
    got = run_decode(*case)
    v, cu = case[2], case[5]
    for s in range(3):
        want = np.repeat(v[cu[s]], 2, axis=0)        # GQA: heads 2h, 2h+1 read KV head h
        np.testing.assert_array_equal(got[s], bf16_to_f64(round_bf16(want)))


def test_decode_empty_sequences_give_zeros():
    say("decode with empty sequences")
    case = decode_case(5, [0, 40, 0, 0, 513, 0], 16, 8, 128)
    check_per_seq(run_decode(*case), oracle_decode(*case), case[5])


def test_decode_any_max_len_is_correct():
    """max_cache_len only sizes the key split: a short value makes each
    workgroup walk more chunks, the result stays within the bar."""
    say("decode with max_cache_len below the longest sequence")
    case = decode_case(6, [700, 2049, 31], 16, 8, 128)
    ref = oracle_decode(*case)
    for mx in (0, 1, 256, 5000):
        check_per_seq(run_decode(*case, max_len=mx), ref, case[5])


def test_decode_large_batch_walks_chunks():
    """64 sequences x 8 KV heads fill the grid with few chunks per sequence,
    so every workgroup loops over several 256-key chunks."""
    rng = np.random.default_rng(7)
    lens = [int(x) for x in rng.integers(1500, 3500, 64)]
    say(f"decode batch of 64, lens {min(lens)}..{max(lens)}")
    case = decode_case(7, lens, 16, 8, 128)
    got = run_decode(*case)
    seqs = list(range(0, 64, 7))
    check_per_seq(got, oracle_decode(*case, seqs=seqs), case[5], seqs=seqs)


def test_decode_deterministic():
    case = decode_case(8, [4000, 123], 16, 8, 128)
    a, b = run_decode(*case), run_decode(*case)
    np.testing.assert_array_equal(a, b)


def test_decode_matches_prefill_kernel_last_rows():
    """The same rows through tg_gated_attn (every row a query) and
    tg_gated_decode (the last row only) agree to bf16 rounding."""
    from learned_token_pruning_06_amd import ops
    lens = [300, 1, 2500]
    q, k, v, cb, qpos, cu, gain, temp = decode_case(9, lens, 16, 8, 128)
    rng = np.random.default_rng(90)
    T = int(cu[-1])
    qf = bf16_to_f64(round_bf16(rng.standard_normal((T, 16, 128))))
    pos = np.zeros(T, np.int64)
    for s in range(len(lens)):
        lo, hi = int(cu[s]), int(cu[s + 1])
        qf[hi - 1] = q[s]
        pos[lo:hi] = np.arange(hi - lo)
        pos[hi - 1] = qpos[s]
    pre = ops.gated_attn(bf16_dev(round_bf16(qf)), bf16_dev(round_bf16(k)),
                         bf16_dev(round_bf16(v)), f32_dev(cb), i32_dev(pos), i32_dev(cu),
                         f32_dev(gain), f32_dev(temp), max_len=max(lens))
    torch.cuda.synchronize()
    pre = to_f64(pre)
    got = run_decode(q, k, v, cb, qpos, cu, gain, temp)
    for s in range(len(lens)):
        assert rel_l2(got[s], pre[int(cu[s + 1]) - 1]) <= TOL


def test_kv_cache_pruning_is_a_gather_then_decode():
    """After prefill, the cache of a layer below the gate is pruned to the
    kept tokens (a gather of its K and V rows, bit-exact), the new token is
    appended, and the decode step runs over the pruned cache."""
    from learned_token_pruning_06_amd import ops
    rng = np.random.default_rng(11)
    N, hq, hkv, dh = 4096, 16, 8, 128
    prunable = np.ones(N, np.uint8)
    prunable[-128:] = 0
    b = rng.standard_normal(N).astype(np.float32).astype(np.float64)
    b[-128:] = 0.0
    kept_idx, kept_pos, kept_b, kept_cu = O.ref_select(b, prunable, [0, N], [512])
    kf = round_bf16(rng.standard_normal((N, hkv, dh)))
    vf = round_bf16(rng.standard_normal((N, hkv, dh)))
    idx = i32_dev(kept_idx)
    kp = ops.gather(bf16_dev(kf), idx)
    vp = ops.gather(bf16_dev(vf), idx)
    torch.cuda.synchronize()
    kp_bits = kp.view(torch.int16).cpu().numpy().view(np.uint16)
    vp_bits = vp.view(torch.int16).cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(kp_bits, O.ref_gather(kf, kept_idx))
    np.testing.assert_array_equal(vp_bits, O.ref_gather(vf, kept_idx))
    # append the generated token (b = 0, original position N)
    knew, vnew = round_bf16(rng.standard_normal((1, hkv, dh))), round_bf16(rng.standard_normal((1, hkv, dh)))
    kc = np.concatenate([kp_bits, knew])
    vc = np.concatenate([vp_bits, vnew])
    cb = np.concatenate([np.asarray(kept_b, np.float64), [0.0]])
    cu = np.array([0, kc.shape[0]], np.int64)
    q = bf16_to_f64(round_bf16(rng.standard_normal((1, hq, dh))))
    gain = rng.uniform(0.5, 1.5, hq).astype(np.float32)
    temp = rng.uniform(0.8, 1.2, hq).astype(np.float32)
    qpos = np.array([N], np.int64)
    got = run_decode(q, bf16_to_f64(kc), bf16_to_f64(vc), cb, qpos, cu, gain, temp)
    ref = oracle_decode(q, bf16_to_f64(kc), bf16_to_f64(vc), cb, qpos, cu, gain, temp)
    check_per_seq(got, ref, cu)


@pytest.mark.parametrize("cache", [8705, 131073])
def test_decode_after_128k_prefill(cache):
    """One decode step after the 128k-token gated prefill: the pruned cache
    (8192 kept document + 512 prompt tokens + the new one) and, as the
    unpruned reference point, the full 131072-token cache + the new one."""
    say(f"decode over a {cache}-row cache")
    case = decode_case(12, [cache], 16, 8, 128)
    check_per_seq(run_decode(*case), oracle_decode(*case), case[5])


def test_decode_rejects_bad_arguments():
    from learned_token_pruning_06_amd import ops
    from learned_token_pruning_06_amd._lib import TokenGateError
    q = torch.zeros((1, 16, 128), dtype=torch.bfloat16, device=DEV)
    kc = torch.zeros((4, 8, 128), dtype=torch.bfloat16, device=DEV)
    cu = i32_dev([0, 4])
    g = f32_dev(np.ones(16))
    with pytest.raises(TokenGateError):                 # hq/hkv = 16/3
        ops.gated_decode(q, kc[:, :3].contiguous(), kc[:, :3].contiguous(), None, None, cu, g, g)
    with pytest.raises(TokenGateError):                 # workspace too small
        ops.gated_decode(q, kc, kc, None, None, cu, g, g, max_cache_len=4096,
                         ws=torch.empty(16, dtype=torch.uint8, device=DEV))
