"""The four calls only enqueue kernels (no allocation, memset or sync inside),
so a whole gated layer can be captured into a HIP graph.  Replays must be
bit-equal to the eager run, with eager work and synchronisations between
them (several replays, as stale graph state shows only after the first)."""
import numpy as np
import pytest
import torch

from gpu_util import bf16_dev, f32_dev, i32_dev, say, u8_dev, workload

pytestmark = pytest.mark.gpu


def test_gated_layer_graph_replay_matches_eager():
    from learned_token_pruning_06_amd import ops
    g = workload(1)
    wl = g["wl"]
    lib = ops.load()
    x = bf16_dev(g["x"])
    w1 = bf16_dev(g["w1"])
    w2, b1 = f32_dev(g["w2"]), f32_dev(g["b1"])
    pr, cu = u8_dev(g["prunable"]), i32_dev(g["cu_seqlens"])
    kdev = i32_dev(g["budgets"][0])
    gain, temp = f32_dev(g["gain"]), f32_dev(g["temp"])
    _, t_kept = ops.kept_sizes(g["cu_seqlens"], [int(g["prunable"].sum())], g["budgets"][0])
    w_all = bf16_dev(np.ascontiguousarray(np.concatenate([g["wq"].T, g["wk"].T, g["wv"].T], 0)))
    dev = x.device
    # every buffer allocated up front, so the captured region allocates nothing
    b_raw = torch.empty(wl.t_in, dtype=torch.float32, device=dev)
    b = torch.empty_like(b_raw)
    ws_s = ops.workspace(lib.tg_score_workspace_size(wl.t_in, 1), dev)
    ws_k = ops.workspace(lib.tg_select_workspace_size(wl.t_in, 1), dev)
    kept_idx = torch.empty(t_kept, dtype=torch.int32, device=dev)
    kept_pos = torch.empty_like(kept_idx)
    kept_b = torch.empty(t_kept, dtype=torch.float32, device=dev)
    kept_cu = torch.empty(2, dtype=torch.int32, device=dev)
    x_kept = torch.empty(t_kept, wl.d, dtype=torch.bfloat16, device=dev)
    q = torch.empty(t_kept, wl.hq, wl.dh, dtype=torch.bfloat16, device=dev)
    k = torch.empty(t_kept, wl.hkv, wl.dh, dtype=torch.bfloat16, device=dev)
    v = torch.empty_like(k)
    o = torch.empty_like(q)

    def layer():
        ops.score(x, w1, w2, pr, cu, b1=b1, b2=g["b2"], eps=1e-6, b_raw=b_raw, b=b, ws=ws_s)
        ops.select_topk(b, pr, cu, kdev, t_kept, kept_idx, kept_pos, kept_b, kept_cu, ws_k)
        ops.gather(x, kept_idx, out=x_kept)
        ops.qkv_proj(x_kept, w_all, wl.hq, wl.hkv, wl.dh, q=q, k=k, v=v)
        ops.gated_attn(q, k, v, kept_b, kept_pos, kept_cu, gain, temp, max_len=t_kept, out=o)

    outs = (b, kept_idx, kept_pos, kept_b, kept_cu, x_kept, q, k, v, o)
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        layer()                                   # eager reference (and warm-up)
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer()
    torch.cuda.synchronize()
    for rep in range(4):
        for t in outs:                            # eager work between replays
            t.view(torch.uint8).fill_(0xA5)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, t, r in zip(("b", "kept_idx", "kept_pos", "kept_b", "kept_cu", "x_kept", "q", "k",
                               "v", "o"), outs, ref):
            assert torch.equal(t.view(torch.uint8), r.view(torch.uint8)), f"replay {rep}: {name}"
        say(f"graph replay {rep}: all ten outputs bit-equal to eager")


def test_padded_bucket_graph_serves_several_budgets():
    """One graph per padded kept length (the paper's prefill captures one
    graph per padded length, App. C.2): the 128k layer is captured once with
    every buffer sized for 9216 kept rows, then replayed for budgets of 7000,
    8700, 8192 and again 7000 document tokens, only the device budget changing
    between replays.  The kernels read the real kept count from
    kept_cu_seqlens on the device; rows past it are padding.  Each replay is
    checked against the oracle: the scores within 1e-5, the kept set and the
    gathered rows exactly, q/k/v at the bf16 bar of the projection, and the
    attention output at the bf16 bars (global, per head, per row) against the
    oracle's attention on the replay's own q/k/v."""
    import oracle as O
    from gpu_util import check_attn, rel_l2, score_err, to_f64
    from learned_token_pruning_06_amd import ops
    from workloads import bf16_to_f64
    g = workload(3)
    wl = g["wl"]
    lib = ops.load()
    cap = 9216
    x = bf16_dev(g["x"])
    w1 = bf16_dev(g["w1"])
    w2, b1 = f32_dev(g["w2"]), f32_dev(g["b1"])
    pr, cu = u8_dev(g["prunable"]), i32_dev(g["cu_seqlens"])
    gain, temp = f32_dev(g["gain"]), f32_dev(g["temp"])
    w_all = bf16_dev(np.ascontiguousarray(np.concatenate([g["wq"].T, g["wk"].T, g["wv"].T], 0)))
    dev = x.device
    kdev = torch.tensor([8192], dtype=torch.int32, device=dev)
    b_raw = torch.empty(wl.t_in, dtype=torch.float32, device=dev)
    b = torch.empty_like(b_raw)
    ws_s = ops.workspace(lib.tg_score_workspace_size(wl.t_in, 1), dev)
    ws_k = ops.workspace(lib.tg_select_workspace_size(wl.t_in, 1), dev)
    kept_idx = torch.empty(cap, dtype=torch.int32, device=dev)
    kept_pos = torch.empty_like(kept_idx)
    kept_b = torch.empty(cap, dtype=torch.float32, device=dev)
    kept_cu = torch.empty(2, dtype=torch.int32, device=dev)
    x_kept = torch.empty(cap, wl.d, dtype=torch.bfloat16, device=dev)
    q = torch.empty(cap, wl.hq, wl.dh, dtype=torch.bfloat16, device=dev)
    k = torch.empty(cap, wl.hkv, wl.dh, dtype=torch.bfloat16, device=dev)
    v = torch.empty_like(k)
    o = torch.empty_like(q)

    def layer():
        ops.score(x, w1, w2, pr, cu, b1=b1, b2=g["b2"], eps=O.readings.EPS, b_raw=b_raw, b=b,
                  ws=ws_s)
        ops.select_topk(b, pr, cu, kdev, cap, kept_idx, kept_pos, kept_b, kept_cu, ws_k)
        ops.gather(x, kept_idx, out=x_kept)
        ops.qkv_proj(x_kept, w_all, wl.hq, wl.hkv, wl.dh, q=q, k=k, v=v)
        ops.gated_attn(q, k, v, kept_b, kept_pos, kept_cu, gain, temp, max_len=cap, out=o)

    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        layer()                                   # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer()
    torch.cuda.synchronize()

    # the oracle's scores once (they do not depend on the budget)
    w1d = bf16_to_f64(g["w1"])
    ref_raw = np.concatenate([O.ref_score(bf16_to_f64(g["x"][s:s + 32768]), w1d, g["b1"], g["w2"],
                                          g["b2"]) for s in range(0, wl.t_in, 32768)])
    ref_b, _ = O.ref_normalise(ref_raw, g["prunable"], g["cu_seqlens"], O.readings.EPS)
    conv = bf16_to_f64
    for rep, K in enumerate((7000, 8700, 8192, 7000)):
        say(f"bucket graph replay {rep}: K = {K}, capacity {cap}")
        for t in (b, kept_idx, kept_pos, kept_b, kept_cu, x_kept, q, k, v, o):
            t.view(torch.uint8).fill_(0xA5)       # eager work between replays
        kdev.fill_(K)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got_b = b.cpu().numpy()
        assert score_err(got_b.astype(np.float64), ref_b) <= 1e-5, f"K={K}: scores"
        want = O.ref_select(got_b, g["prunable"], g["cu_seqlens"], [K])
        tk = int(want[3][-1])
        assert tk == K + 512 <= cap
        assert np.array_equal(kept_cu.cpu().numpy(), want[3]), f"K={K}: kept_cu"
        for name, got, ref in (("kept_idx", kept_idx, want[0]), ("kept_pos", kept_pos, want[1])):
            assert np.array_equal(got[:tk].cpu().numpy(), ref), f"K={K}: {name}"
        assert np.array_equal(kept_b[:tk].cpu().numpy().view(np.uint32),
                              np.asarray(want[2], np.float32).view(np.uint32)), f"K={K}: kept_b"
        xk = x_kept[:tk].view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(xk, O.ref_gather(g["x"], want[0])), f"K={K}: gathered rows"
        rq, rk, rv = O.ref_project(conv(xk), conv(g["wq"]), conv(g["wk"]), conv(g["wv"]), wl.hq,
                                   wl.hkv, wl.dh)
        qg, kg, vg = (to_f64(t[:tk]) for t in (q, k, v))
        for name, got, ref in (("q", qg, rq), ("k", kg, rk), ("v", vg, rv)):
            e = rel_l2(got, ref)
            assert e <= 1e-2, f"K={K}: {name} rel-L2 {e:.2e}"
        ref_o = O.ref_gated_attn(qg, kg, vg, want[2], want[1], want[3], g["gain"], g["temp"])
        check_attn(to_f64(o[:tk]), ref_o, "bf16", f"bucket replay K={K}")


def test_split_attention_graph_serves_several_lengths():
    """tg_gated_attn_split captured once for a capacity of 3000 kept rows and
    replayed for sequences of 2496, 1500, 2999 and again 2496 rows, only
    kept_cu_seqlens changing on the device between replays.  Its plan runs on
    the GPU from the device offsets, so each replay splits the blocks it
    really has.  Each replay must equal an eager split call bit for bit,
    match the oracle at the bf16 bars, and leave the padding rows alone."""
    import oracle as O
    from gpu_util import check_attn, round_bf16, to_f64
    from learned_token_pruning_06_amd import ops
    from workloads import bf16_to_f64
    cap, hq, hkv, dh = 3000, 16, 8, 128
    rng = np.random.default_rng(91)
    qh, kh, vh = (round_bf16(rng.standard_normal((cap, n, dh))) for n in (hq, hkv, hkv))
    kbh = rng.standard_normal(cap).astype(np.float32)
    posh = (3 * np.arange(cap)).astype(np.int32)
    gainh = rng.uniform(0.5, 1.5, hq).astype(np.float32)
    temph = rng.uniform(0.8, 1.2, hq).astype(np.float32)
    q, k, v = bf16_dev(qh), bf16_dev(kh), bf16_dev(vh)
    kb, kp, gain, temp = f32_dev(kbh), i32_dev(posh), f32_dev(gainh), f32_dev(temph)
    kc = i32_dev(np.array([0, cap], np.int32))
    lib = ops.load()
    dev = q.device
    ws = ops.workspace(lib.tg_gated_attn_split_workspace_size(cap, 1, cap, hq, hkv, dh), dev)
    o = torch.empty_like(q)
    o_eager = torch.empty_like(q)

    def attn(out):
        ops.gated_attn(q, k, v, kb, kp, kc, gain, temp, max_len=cap, out=out, split=True, ws=ws)

    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        attn(o)                                   # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        attn(o)
    torch.cuda.synchronize()
    for rep, n in enumerate((2496, 1500, 2999, 2496)):
        say(f"split graph replay {rep}: {n} kept rows, capacity {cap}")
        kc[1].fill_(n)                            # eager work between replays
        o.view(torch.uint8).fill_(0xA5)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        attn(o_eager)
        torch.cuda.synchronize()
        assert torch.equal(o[:n].view(torch.int16), o_eager[:n].view(torch.int16)), \
            f"replay {rep}: differs from the eager call"
        assert torch.all(o[n:].view(torch.uint8) == 0xA5), f"replay {rep}: padding rows written"
        want = O.ref_gated_attn(bf16_to_f64(qh[:n]), bf16_to_f64(kh[:n]), bf16_to_f64(vh[:n]),
                                kbh[:n].astype(np.float64), posh[:n], np.array([0, n]), gainh,
                                temph)
        check_attn(to_f64(o[:n]), want, "bf16", f"split graph replay, {n} rows")
