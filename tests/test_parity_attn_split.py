"""tg_gated_attn_split against the oracle, at the same bars as tg_gated_attn.

The split form plans its work on the GPU (the query blocks, and the key
chunks of the longest ones, sorted largest first for the workgroups) and
merges the split blocks' partial results in a second launch; the attention it
computes is Eq. 8's, unchanged.  Each case first checks that its sizes make
the call split (a workspace that holds partial results) and then
compares the output with ref_gated_attn (rel-L2 <= 1e-2 globally and per
head, 2e-2 per row, as for the unsplit form) and lse2 with
ref_gated_attn_lse2 (|d| <= 5.6e-3 + 1e-5 |ref|, the bar of the unsplit lse2
test: bf16-rounded probabilities in the normaliser).  Where no block is
split, the output must match tg_gated_attn bit for bit (only the order in
which the blocks run differs)."""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import (LSE2_ABS, bf16_dev, check_attn, f32_dev, i32_dev, lse2_excess, round_bf16,
                      say, to_f64, workload)
from test_parity_attn import synth_case
from workloads import bf16_to_f64

pytestmark = pytest.mark.gpu


def _ws_bytes(t, n_seq, max_len, hq, hkv, dh):
    from learned_token_pruning_06_amd import _lib
    return _lib.load().tg_gated_attn_split_workspace_size(t, n_seq, max_len, hq, hkv, dh)


def _has_partials(nbytes, t, hq, dh):
    """The workspace holds partial results (some block is split): at least
    two chunks' (bf16 output, f32 max and sum) per row and head."""
    return nbytes >= 2 * t * hq * (dh * 2 + 8)


def _dev_args(q, k, v, kb, pos, kc, gain, temp):
    return (bf16_dev(round_bf16(q)), bf16_dev(round_bf16(k)), bf16_dev(round_bf16(v)),
            f32_dev(kb), None if pos is None else i32_dev(pos), i32_dev(kc), f32_dev(gain),
            f32_dev(temp))


def _run_split(case, sm_scale=None):
    from learned_token_pruning_06_amd import ops
    q, k, v, kb, pos, kc, gain, temp = case
    t, hq, dh = q.shape
    hkv = k.shape[1]
    ml = int(np.diff(kc).max(initial=0))
    nbytes = _ws_bytes(t, kc.size - 1, ml, hq, hkv, dh)
    lse2 = torch.full((hq, t), float("nan"), device="cuda")
    out = ops.gated_attn(*_dev_args(*case), max_len=ml, sm_scale=sm_scale, lse2=lse2, split=True)
    torch.cuda.synchronize()
    return to_f64(out), lse2.cpu().numpy().astype(np.float64).T, nbytes


def _check_lse2(got, case, tag, sm_scale=None):
    q, k, v, kb, pos, kc, gain, temp = case
    ref = O.ref_gated_attn_lse2(q, k, kb, pos, kc, gain, temp, sm_scale=sm_scale)
    err = lse2_excess(got, ref)
    say(f"  {tag}: worst |d lse2| beyond 1e-5 |ref|: {err:.2e}")
    assert np.all(np.isfinite(got)), f"{tag}: non-finite lse2"
    assert err <= LSE2_ABS, f"{tag}: lse2 error {err:.2e}"


SPLIT_CASES = [
    # seed, kept lengths, hq, hkv, dh (chunk tiles and chunks of the longest
    # block, as planned)
    (41, [2496], 16, 8, 128),                   # 14 x 3
    (42, [1, 5, 31, 64, 65, 1300], 16, 8, 128),  # short sequences unsplit, 8 x 3
    (43, [2496], 8, 8, 128),                    # MHA, 8 x 5
    (44, [1800, 0, 77], 4, 1, 64),              # 4 query heads per KV head, dh 64, 8 x 4
    (45, [2000, 333], 32, 4, 128),              # 8 query heads per KV head, 18 x 2
    (46, [1400], 16, 8, 128),                   # 8 x 3
    (47, [1600, 64, 129], 16, 8, 128),          # 8 x 4, last chunk shorter
]


@pytest.mark.parametrize("case", SPLIT_CASES,
                         ids=[f"s{c[0]}-g{c[2] // c[3]}-dh{c[4]}" for c in SPLIT_CASES])
def test_split_matches_oracle(case):
    seed, lens, hq, hkv, dh = case
    say(f"attn split: seed={seed} lens={lens} hq={hq} hkv={hkv} dh={dh}")
    c = synth_case(seed, lens, hq, hkv, dh, "bf16", prompt=5)
    got, lse2, nbytes = _run_split(c)
    assert _has_partials(nbytes, sum(lens), hq, dh), "these sizes should split the keys"
    q, k, v, kb, pos, kc, gain, temp = c
    check_attn(got, O.ref_gated_attn(q, k, v, kb, pos, kc, gain, temp), "bf16", f"split {seed}")
    _check_lse2(lse2, c, f"split {seed}")


def test_split_wide_scores_without_positions():
    """A wide score range moves the running maximum often inside every
    chunk, so the chunks' maxima differ widely and the merge's weights span
    many orders of magnitude; no positions (length factor 1), explicit
    scale."""
    say("attn split: wide score range, kept_pos NULL, sm_scale 0.05")
    q, k, v, kb, _, kc, gain, temp = synth_case(48, [1500], 16, 8, 128, "bf16", with_pos=False)
    kb = np.linspace(-20, 20, kb.size)
    c = (q, k, v, kb, None, kc, gain, temp * 3)
    got, lse2, nbytes = _run_split(c, sm_scale=0.05)
    assert _has_partials(nbytes, 1500, 16, 128)
    check_attn(got, O.ref_gated_attn(q, k, v, kb, None, kc, gain, temp * 3, sm_scale=0.05),
               "bf16", "split, wide scores")
    _check_lse2(lse2, c, "split, wide scores", sm_scale=0.05)
    # the unsplit form on the same inputs, for comparison: few keys dominate
    # each row here, so the probabilities' rounding does not average out
    from learned_token_pruning_06_amd import ops
    l0 = torch.full((16, q.shape[0]), float("nan"), device="cuda")
    ops.gated_attn(*_dev_args(*c), max_len=1500, sm_scale=0.05, lse2=l0)
    torch.cuda.synchronize()
    _check_lse2(l0.cpu().numpy().astype(np.float64).T, c, "unsplit, wide scores", sm_scale=0.05)


def test_split_is_deterministic():
    from learned_token_pruning_06_amd import ops
    say("attn split: repeat runs identical")
    c = synth_case(49, [1900, 100], 16, 8, 128, "bf16")
    args = _dev_args(*c)
    o1 = ops.gated_attn(*args, split=True)
    o2 = ops.gated_attn(*args, split=True)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    q, k, v, kb, pos, kc, gain, temp = c
    check_attn(to_f64(o1), O.ref_gated_attn(q, k, v, kb, pos, kc, gain, temp), "bf16",
               "split, two sequences")


def test_split_leaves_rows_past_the_last_sequence():
    """Rows past kept_cu[n_seq] are left alone, as by tg_gated_attn."""
    from learned_token_pruning_06_amd import ops
    say("attn split: 40 rows past the last sequence untouched")
    q, k, v, kb, pos, kc, gain, temp = synth_case(50, [1400, 40], 16, 8, 128, "bf16")
    kc_short = kc[:-1]                                # the 40 rows of the last length dropped
    assert _has_partials(_ws_bytes(1440, 1, 1400, 16, 8, 128), 1440, 16, 128)
    args = list(_dev_args(q, k, v, kb, pos, kc_short, gain, temp))
    out = torch.full_like(args[0], 7.0)
    ops.gated_attn(*args, max_len=1400, out=out, split=True)
    torch.cuda.synchronize()
    tail = out[1400:].float()
    assert torch.all(tail == 7.0)
    want = O.ref_gated_attn(q[:1400], k[:1400], v[:1400], kb[:1400], pos[:1400], kc_short, gain,
                            temp)
    check_attn(to_f64(out[:1400]), want, "bf16", "split, head rows")


def test_split_with_max_len_understated():
    """max_kept_seqlen below a sequence's real length (a broken promise): the
    split is planned for the stated length, so the long sequence's blocks
    have more key tiles than the planned chunks cover and the last chunk
    runs to the block's end.  The result must still be the attention."""
    from learned_token_pruning_06_amd import ops
    say("attn split: max_len 1300 stated for a 2600-row sequence")
    c = synth_case(52, [300, 2600], 16, 8, 128, "bf16")
    t = 2900
    assert _has_partials(_ws_bytes(t, 2, 1300, 16, 8, 128), t, 16, 128)
    out = ops.gated_attn(*_dev_args(*c), max_len=1300, split=True)
    torch.cuda.synchronize()
    q, k, v, kb, pos, kc, gain, temp = c
    check_attn(to_f64(out), O.ref_gated_attn(q, k, v, kb, pos, kc, gain, temp), "bf16",
               "split, understated max_len")


@pytest.mark.parametrize("lens", [[20000], [589, 1602, 3141, 7048], [700, 333, 5, 64]],
                         ids=["one-20000", "ragged-4", "short-4"])
def test_unsplit_sizes_match_the_plain_path(lens):
    """No block outweighs a workgroup's share: nothing is split, the blocks
    only run in another order, and every one is computed as tg_gated_attn
    computes it (identical bits)."""
    from learned_token_pruning_06_amd import ops
    say(f"attn split: lengths {lens} planned without a split")
    t, ml = sum(lens), max(lens)
    assert not _has_partials(_ws_bytes(t, len(lens), ml, 16, 8, 128), t, 16, 128)
    c = synth_case(51, lens, 16, 8, 128, "bf16")
    args = _dev_args(*c)
    l1 = torch.full((16, t), float("nan"), device="cuda")
    l0 = torch.full((16, t), float("nan"), device="cuda")
    o1 = ops.gated_attn(*args, max_len=ml, split=True, lse2=l1)
    o0 = ops.gated_attn(*args, max_len=ml, lse2=l0)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o0.view(torch.int16))
    assert torch.equal(l1, l0)


def test_split_16k_workload_all_rows():
    """The 16k workload's kept rows (2496 of them after top-K), through the
    split form: every row against the oracle on the same rounded inputs."""
    say("attn split: 16k workload, every kept row")
    g = workload(1)
    wl = g["wl"]
    xd = bf16_to_f64(g["x"])
    w1 = bf16_to_f64(g["w1"])
    b_raw = np.concatenate([O.ref_score(xd[s:s + 32768], w1, g["b1"], g["w2"], g["b2"])
                            for s in range(0, xd.shape[0], 32768)])
    b, _ = O.ref_normalise(b_raw, g["prunable"], g["cu_seqlens"])
    idx, pos, kb, kc = O.ref_select(b.astype(np.float32), g["prunable"], g["cu_seqlens"],
                                    g["budgets"][0])
    q, k, v = O.ref_project(xd[idx], bf16_to_f64(g["wq"]), bf16_to_f64(g["wk"]),
                            bf16_to_f64(g["wv"]), wl.hq, wl.hkv, wl.dh)
    q, k, v = (bf16_to_f64(round_bf16(a)) for a in (q, k, v))
    c = (q, k, v, kb, pos, kc, g["gain"], g["temp"])
    got, lse2, nbytes = _run_split(c)
    say(f"  {q.shape[0]} kept rows, workspace {nbytes} bytes")
    assert _has_partials(nbytes, q.shape[0], q.shape[1], q.shape[2])
    check_attn(got, O.ref_gated_attn(*c), "bf16", "split, 16k workload")
    _check_lse2(lse2, c, "split, 16k workload")


def _random_configs(n=10, seed=77):
    """Seeded random shapes: 1-5 sequences, the longest 1280-1700 rows (at
    least 20 key tiles, so most draws split), the others 0-1700; every
    head grouping the attention supports, dh 64 and 128."""
    rng = np.random.default_rng(seed)
    heads = [(16, 8, 128), (8, 8, 128), (16, 4, 128), (32, 4, 128), (4, 1, 64), (8, 4, 64)]
    out = []
    for i in range(n):
        n_seq = int(rng.integers(1, 6))
        lens = [int(x) for x in rng.integers(0, 1701, n_seq)]
        lens[int(rng.integers(0, n_seq))] = int(rng.integers(1280, 1701))
        hq, hkv, dh = heads[i % len(heads)]
        out.append((1000 + i, lens, hq, hkv, dh))
    return out


@pytest.mark.parametrize("case", _random_configs(),
                         ids=[f"r{c[0]}-n{len(c[1])}-g{c[2] // c[3]}-dh{c[4]}"
                              for c in _random_configs()])
def test_split_random_shapes(case):
    seed, lens, hq, hkv, dh = case
    say(f"attn split (random): seed={seed} lens={lens} hq={hq} hkv={hkv} dh={dh}")
    c = synth_case(seed, lens, hq, hkv, dh, "bf16", prompt=7)
    got, lse2, nbytes = _run_split(c)
    say(f"  partial results: {_has_partials(nbytes, sum(lens), hq, dh)}")
    q, k, v, kb, pos, kc, gain, temp = c
    check_attn(got, O.ref_gated_attn(q, k, v, kb, pos, kc, gain, temp), "bf16",
               f"split random {seed}")
    _check_lse2(lse2, c, f"split random {seed}")


def test_budget_sweep_every_budget_plain_and_split():
    """The 32k budget sweep (preset scores with ties and +6 spikes, eight
    budgets drawn log-uniformly): for every budget, the oracle's kept set and
    projections, then both tg_gated_attn and tg_gated_attn_split on every
    kept row against the oracle on the same rounded inputs, and the split
    form's lse2.  Kept sets of one score vector are nested (ties go to the
    lower index), so the rows are projected once, for the largest budget.
    Budgets past 8192 kept document tokens are left to the plain path's
    largest-budget test (test_parity_attn.py): one sequence that long leaves
    no block longer than a workgroup's share, so both forms make the same
    single launch."""
    from test_parity_attn import run_attn
    g = workload(2)
    wl = g["wl"]
    b = g["b_preset"].astype(np.float32)
    budgets = [np.asarray(k, np.int32) for k in g["budgets"]]
    big = max(budgets, key=lambda k: int(k[0]))
    idx_all, _, _, _ = O.ref_select(b, g["prunable"], g["cu_seqlens"], big)
    xd = bf16_to_f64(g["x"][idx_all])
    q_all, k_all, v_all = O.ref_project(xd, bf16_to_f64(g["wq"]), bf16_to_f64(g["wk"]),
                                        bf16_to_f64(g["wv"]), wl.hq, wl.hkv, wl.dh)
    q_all, k_all, v_all = (bf16_to_f64(round_bf16(a)) for a in (q_all, k_all, v_all))
    for kk in budgets:
        if int(kk[0]) > 8192:
            continue
        idx, pos, kb, kc = O.ref_select(b, g["prunable"], g["cu_seqlens"], kk)
        at = np.searchsorted(idx_all, idx)
        assert np.array_equal(idx_all[at], idx), "kept sets are nested"
        c = (q_all[at], k_all[at], v_all[at], kb, pos, kc, g["gain"], g["temp"])
        say(f"attn sweep: K={int(kk[0])}, {idx.size} kept rows")
        ref = O.ref_gated_attn(*c)
        check_attn(run_attn(*c, "bf16"), ref, "bf16", f"sweep K={int(kk[0])}, plain")
        got, lse2, _ = _run_split(c)
        check_attn(got, ref, "bf16", f"sweep K={int(kk[0])}, split")
        _check_lse2(lse2, c, f"sweep K={int(kk[0])}, split")
