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
