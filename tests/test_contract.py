"""Device-side contract checks (tg_set_contract_checks / tg_contract_status).

Valid inputs raise no flag; each broken precondition raises its own bit.
Only breaches the kernels already handle inside their buffers are used: a
capacity below the kept count (outputs past it are dropped), a negative
budget (read as 0), gather indices outside the source (zero rows), kept
positions that do not increase, and packing offsets past the end (clamped to
the row count).  The results of the valid parts are checked as well."""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import DEV, f32_dev, i32_dev, say, u8_dev

pytestmark = pytest.mark.gpu


@pytest.fixture
def checks():
    from learned_token_pruning_06_amd import ops
    ops.set_contract_checks(True)
    ops.contract_status()                        # start from a clear word
    try:
        yield ops
    finally:
        ops.set_contract_checks(False)
        ops.contract_status()


def _scores(seed, T, n_prompt):
    rng = np.random.default_rng(seed)
    b = rng.standard_normal(T).astype(np.float32)
    pr = np.ones(T, np.uint8)
    pr[-n_prompt:] = 0
    b[pr == 0] = 0.0
    return b, pr


def test_valid_calls_raise_nothing(checks):
    ops = checks
    say("contract checks: valid selection, gather and attention")
    b, pr = _scores(1, 5000, 64)
    cu = np.array([0, 3000, 5000], np.int32)
    k = [700, 1]
    npr = [int(pr[0:3000].sum()), int(pr[3000:].sum())]
    _, tk = ops.kept_sizes(cu, npr, k)
    idx, pos, kb, kc = ops.select_topk(f32_dev(b), u8_dev(pr), i32_dev(cu), i32_dev(k), tk)
    src = torch.randn(5000, 64, device=DEV)
    ops.gather(src, idx)
    q = torch.randn(tk, 4, 64, device=DEV).bfloat16()
    kv = torch.randn(tk, 2, 64, device=DEV).bfloat16()
    ops.gated_attn(q, kv, kv, kb, pos, kc, f32_dev(np.ones(4)), f32_dev(np.ones(4)))
    assert ops.contract_status() == set()
    want = O.ref_select(b, pr, cu, k)
    assert np.array_equal(idx.cpu().numpy(), want[0])


def test_small_capacity_and_negative_budget(checks):
    ops = checks
    b, pr = _scores(2, 4096, 32)
    cu = np.array([0, 4096], np.int32)
    say("contract checks: capacity below the kept count")
    idx, _, _, kc = ops.select_topk(f32_dev(b), u8_dev(pr), i32_dev(cu), i32_dev([1000]), 500)
    assert ops.contract_status() == {"capacity"}
    want = O.ref_select(b, pr, cu, [1000])
    assert np.array_equal(idx.cpu().numpy(), want[0][:500])   # the first 500 still written
    assert ops.contract_status() == set()                       # the read cleared the word
    say("contract checks: negative budget")
    idx, _, _, kc = ops.select_topk(f32_dev(b), u8_dev(pr), i32_dev(cu), i32_dev([-3]), 32)
    assert ops.contract_status() == {"negative_budget"}
    assert np.array_equal(idx.cpu().numpy(), O.ref_select(b, pr, cu, [0])[0])


def test_offsets_past_the_end(checks):
    ops = checks
    b, pr = _scores(3, 3000, 16)
    say("contract checks: cu_seqlens past t_in")
    ops.select_topk(f32_dev(b), u8_dev(pr), i32_dev([0, 3100]), i32_dev([10]), 26)
    assert ops.contract_status() == {"offsets"}
    say("contract checks: kept_cu_seqlens past the kept rows")
    T = 200
    q = torch.randn(T, 4, 64, device=DEV).bfloat16()
    kv = torch.randn(T, 2, 64, device=DEV).bfloat16()
    ops.gated_attn(q, kv, kv, f32_dev(np.zeros(T)), i32_dev(np.arange(T)), i32_dev([0, T + 64]),
                   f32_dev(np.ones(4)), f32_dev(np.ones(4)))
    assert ops.contract_status() == {"kept_offsets"}


def test_bad_indices_and_positions(checks):
    ops = checks
    say("contract checks: gather index outside the source")
    src = torch.arange(40 * 8, dtype=torch.float32, device=DEV).reshape(40, 8)
    out = ops.gather(src, i32_dev([3, 40, -1, 39]))
    assert ops.contract_status() == {"index"}
    assert not out[1].any() and not out[2].any()
    say("contract checks: kept positions not increasing")
    T = 130
    q = torch.randn(T, 4, 64, device=DEV).bfloat16()
    kv = torch.randn(T, 2, 64, device=DEV).bfloat16()
    pos = np.arange(T)
    pos[70] = pos[69]                              # a repeat inside sequence 0
    cu = i32_dev([0, 100, T])
    ops.gated_attn(q, kv, kv, f32_dev(np.zeros(T)), i32_dev(pos), cu, f32_dev(np.ones(4)),
                   f32_dev(np.ones(4)))
    assert ops.contract_status() == {"positions"}
    pos2 = np.concatenate([np.arange(100), np.arange(30)])   # restarts at a sequence start: fine
    ops.gated_attn(q, kv, kv, f32_dev(np.zeros(T)), i32_dev(pos2), cu, f32_dev(np.ones(4)),
                   f32_dev(np.ones(4)))
    assert ops.contract_status() == set()
