"""Benchmark of the TokenGate gated-prefill hot path on one MI355X.

One step = tg_score + tg_select_topk + tg_gather + tg_gated_attn over the
128k-token gated layer (Qwen3-1.7B shapes: hidden 2048, scorer 2048->256->1,
16 query / 8 KV heads of dim 128, 130560 document + 512 prompt tokens, K=8192
document tokens kept -> 8704 kept tokens), bf16, synthetic seeded inputs
resident in HBM.  The Q/K/V projection of the kept rows is not one of the
four calls: it is computed once before timing and the step reads it.

Prints one JSON line (see the keys below).  --gpus N > 1 is refused: the
path runs on one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "gated-prefill tokens/s at 128k ctx; gated-attn MFMA % peak; gate HBM GB/s"
PEAK_BF16_TFLOPS = 2500.0           # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0               # MI355X HBM3E
PEAK_FP32_TFLOPS = 157.3            # MI355X fp32 vector ALU
WORKLOAD = 3                        # 128k-token gated layer (the metric's configuration)
WORKLOAD_NAMES = {
    1: "gated layer 16k: 15872 doc + 512 prompt tokens, K=1984",
    2: "budget sweep 32k: 32256 doc + 512 prompt tokens, 8 calls with K log-uniform in [1, 16128], "
       "preset scores with ties and +6 spikes",
    3: "gated layer 128k: 130560 doc + 512 prompt tokens, K=8192",
    4: "ragged batch: 4 sequences of 8192/24576/49152/65536 tokens, K = 1/16 of each doc part",
}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_code(text: str) -> str:
    """The code of a C++/HIP source without its comments and blank lines, so
    that an edit of the comments alone keeps the counters taken on it."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def source_sha(names):
    """Digest of the named kernel sources' code (comments excluded)."""
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "learned_token_pruning_06_amd", "csrc", n)) as f:
            h.update(source_code(f.read()).encode())
    return h.hexdigest()[:16]


def traffic_for(kernel: str, src_files):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    try:
        d = json.load(open(p))[kernel]
    except Exception:
        return None
    if d.get("source_sha") != source_sha(src_files):
        return None
    return d.get("bytes_per_launch")


def mfma_counters_for(kernel: str, src_files):
    """Matrix-core counters per launch from committed rocprofv3 runs
    (SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE x 1024 SIMDs, and the bf16
    MFMA flops the hardware counted), if they were taken on the current kernel
    source; else None."""
    p = os.path.join(ROOT, "profiles", "pmc_mfma.json")
    try:
        d = json.load(open(p))[kernel]
    except Exception:
        return None
    if d.get("source_sha") != source_sha(src_files):
        return None
    return {k: d[k] for k in ("mfma_busy", "mfma_flops_per_launch") if k in d}


def budget_sweep(g, dev, reps=10):
    """The 32k budget sweep: for each of the 8 drawn budgets, tg_select_topk on
    the preset scores, tg_gather of the kept rows and the attention over them
    (Q/K/V: seeded stand-ins of the kept shape; the attention's cost depends
    only on the shapes).  attn_us is tg_gated_attn_split, the path the step
    takes (it splits the keys of long query blocks when the blocks are too
    few for the GPU); attn_plain_us is tg_gated_attn.  Mean us per call over
    `reps` back-to-back calls (the attention: the lower of two such means)."""
    import numpy as np
    import torch
    from learned_token_pruning_06_amd import ops
    from workloads import random_qkv
    wl = g["wl"]
    lib = ops.load()
    T = wl.t_in
    tb = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
        torch.bfloat16).to(dev)
    b = torch.from_numpy(np.asarray(g["b_preset"], np.float32)).to(dev)
    pr = torch.from_numpy(g["prunable"]).to(dev)
    cu = torch.from_numpy(g["cu_seqlens"]).to(dev)
    x = tb(g["x"])
    gain = torch.from_numpy(g["gain"]).to(dev)
    temp = torch.from_numpy(g["temp"]).to(dev)
    n_pr = int(g["prunable"].sum())
    kmax = max(int(k[0]) for k in g["budgets"])
    tmax = min(kmax, n_pr) + (T - n_pr)
    q_all, k_all, v_all = (tb(a) for a in random_qkv(22, tmax, wl.hq, wl.hkv, wl.dh))
    ws = ops.workspace(lib.tg_select_workspace_size(T, 1), dev)

    def time_it(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e3
    rows = []
    for kk in g["budgets"]:
        K = int(kk[0])
        _, tk = ops.kept_sizes(g["cu_seqlens"], [n_pr], [K])
        kdev = torch.tensor([K], dtype=torch.int32, device=dev)
        ki = torch.empty(tk, dtype=torch.int32, device=dev)
        kp, kb = torch.empty_like(ki), torch.empty(tk, dtype=torch.float32, device=dev)
        kc = torch.empty(2, dtype=torch.int32, device=dev)
        xk = torch.empty(tk, wl.d, dtype=torch.bfloat16, device=dev)
        q, k, v = q_all[:tk], k_all[:tk], v_all[:tk]
        o = torch.empty_like(q)
        t_sel = time_it(lambda: ops.select_topk(b, pr, cu, kdev, tk, ki, kp, kb, kc, ws))
        t_gat = time_it(lambda: ops.gather(x, ki, out=xk))
        ws_a = ops.workspace(
            lib.tg_gated_attn_split_workspace_size(tk, 1, tk, wl.hq, wl.hkv, wl.dh), dev)
        # the two attention forms alternate, twice each; each takes the lower
        # of its two batch means (a clock that is still ramping up would
        # otherwise favour whichever runs second)
        ta, tp = [], []
        for _ in range(2):
            ta.append(time_it(lambda: ops.gated_attn(q, k, v, kb, kp, kc, gain, temp, max_len=tk,
                                                     out=o, split=True, ws=ws_a)))
            tp.append(time_it(lambda: ops.gated_attn(q, k, v, kb, kp, kc, gain, temp, max_len=tk,
                                                     out=o)))
        t_att, t_pl = min(ta), min(tp)
        fl = 2.0 * wl.dh * wl.hq * tk * (tk + 1)
        rows.append({"k": K, "t_kept": int(tk), "select_us": round(t_sel, 2),
                     "gather_us": round(t_gat, 2), "attn_us": round(t_att, 2),
                     "attn_plain_us": round(t_pl, 2),
                     "attn_tflops": round(fl / (t_att * 1e-6) / 1e12, 1),
                     "attn_frac_of_bf16_peak": round(fl / (t_att * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4)})
    del q_all, k_all, v_all, x
    return rows


def short_inputs(dev, reps=10):
    """The attention alone on the kept shapes of the 16k layer (one sequence,
    2496 kept rows) and of the ragged 4-sequence batch (12380 kept rows):
    tg_gated_attn_split (the step's path) against tg_gated_attn.  Q/K/V and
    the kept scores are seeded stand-ins, positions ascending with a stride
    of 16 (the cost depends on the shapes); the two forms alternate, twice
    each, and each keeps its lower mean over `reps` back-to-back calls."""
    import numpy as np
    import torch
    from learned_token_pruning_06_amd import ops
    from workloads import generate, random_qkv
    lib = ops.load()
    rows = []
    for cfg in (1, 4):
        g = generate(cfg, with_x=False, with_proj=False)
        wl = g["wl"]
        cu_h = np.asarray(g["cu_seqlens"], np.int64)
        n_seq = len(cu_h) - 1
        npr = [int(g["prunable"][cu_h[s]:cu_h[s + 1]].sum()) for s in range(n_seq)]
        kc_h, tk = ops.kept_sizes(g["cu_seqlens"], npr, g["budgets"][0])
        kc_h = np.asarray(kc_h, np.int64)
        lens = np.diff(kc_h)
        ml = int(lens.max(initial=0))
        tb = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
            torch.bfloat16).to(dev)
        q, k, v = (tb(a) for a in random_qkv(40 + cfg, tk, wl.hq, wl.hkv, wl.dh))
        rng = np.random.default_rng(40 + cfg)
        kb = torch.from_numpy(rng.standard_normal(tk).astype(np.float32)).to(dev)
        pos = np.concatenate([16 * np.arange(n) for n in lens]).astype(np.int32)
        kp = torch.from_numpy(pos).to(dev)
        kc = torch.from_numpy(kc_h.astype(np.int32)).to(dev)
        gain = torch.from_numpy(g["gain"]).to(dev)
        temp = torch.from_numpy(g["temp"]).to(dev)
        o = torch.empty_like(q)
        ws = ops.workspace(lib.tg_gated_attn_split_workspace_size(tk, n_seq, ml, wl.hq, wl.hkv,
                                                                  wl.dh), dev)
        fs = {"split": lambda: ops.gated_attn(q, k, v, kb, kp, kc, gain, temp, max_len=ml, out=o,
                                              split=True, ws=ws),
              "plain": lambda: ops.gated_attn(q, k, v, kb, kp, kc, gain, temp, max_len=ml, out=o)}
        best = {}
        for _ in range(2):
            for name, f in fs.items():
                f()
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(reps):
                    f()
                e1.record()
                torch.cuda.synchronize()
                best[name] = min(best.get(name, 1e30), e0.elapsed_time(e1) / reps * 1e3)
        fl = 2.0 * wl.dh * wl.hq * float(np.sum(lens * (lens + 1)))
        rows.append({"workload": WORKLOAD_NAMES[cfg], "t_kept": int(tk),
                     "kept_seqlens": [int(x) for x in lens], "split_us": round(best["split"], 2),
                     "plain_us": round(best["plain"], 2),
                     "split_tflops": round(fl / (best["split"] * 1e-6) / 1e12, 1),
                     "split_frac_of_bf16_peak": round(fl / (best["split"] * 1e-6) / 1e12 /
                                                      PEAK_BF16_TFLOPS, 4),
                     "plain_frac_of_bf16_peak": round(fl / (best["plain"] * 1e-6) / 1e12 /
                                                      PEAK_BF16_TFLOPS, 4)})
        del q, k, v
    return rows


def cpu_baseline(g, t_kept_cu, score_chunk=16384):
    """The fp64 oracle on the whole step of the same workload: score and
    normalise all 131072 tokens (x upcast in chunks of score_chunk rows),
    select, gather, and the gated attention over all kept query rows and
    heads.  Q/K/V are seeded stand-ins of the kept shape (the projection is
    not part of the step)."""
    import numpy as np
    import oracle as O
    from workloads import bf16_to_f64, random_qkv
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas = os.cpu_count()
    wl = g["wl"]
    T = wl.t_in
    w1 = bf16_to_f64(g["w1"])
    t0 = time.perf_counter()
    b_raw = np.empty(T)
    for r0 in range(0, T, score_chunk):
        b_raw[r0:r0 + score_chunk] = O.ref_score(bf16_to_f64(g["x"][r0:r0 + score_chunk]), w1,
                                                 g["b1"], g["w2"], g["b2"])
    t_score = time.perf_counter() - t0
    t0 = time.perf_counter()
    b, _ = O.ref_normalise(b_raw, g["prunable"], g["cu_seqlens"])
    idx, pos, kb, kc = O.ref_select(b.astype(np.float32), g["prunable"], g["cu_seqlens"],
                                    g["budgets"][0])
    xk = O.ref_gather(g["x"], idx)
    t_gate = time.perf_counter() - t0
    tk = int(kc[-1])
    q, k, v = random_qkv(11, tk, wl.hq, wl.hkv, wl.dh)
    qd, kd, vd = bf16_to_f64(q), bf16_to_f64(k), bf16_to_f64(v)
    t0 = time.perf_counter()
    O.ref_gated_attn(qd, kd, vd, kb, pos, kc, g["gain"], g["temp"])
    t_attn = time.perf_counter() - t0
    total = t_score + t_gate + t_attn
    del xk
    return {
        "value": T / total, "unit": "tokens/s", "cores": int(blas), "kind": "oracle",
        "sample": (f"the whole step, not a sample: fp64 numpy oracle scores and normalises all {T} "
                   f"tokens, selects, gathers, and runs the gated attention over all {tk} kept query "
                   f"rows x {wl.hq} heads; Q/K/V projection excluded as on the GPU"),
        "seconds": {"score": t_score, "normalise_select_gather": t_gate, "attention": t_attn},
        "host_cores_visible": len(os.sched_getaffinity(0)),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-full-context", action="store_true")
    ap.add_argument("--kernels-only", action="store_true",
                    help="skip the CPU baseline and the full-context lane (for profiling)")
    ap.add_argument("--workload", type=int, default=WORKLOAD, choices=sorted(WORKLOAD_NAMES),
                    help="input configuration; the side lanes run on the default one only")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MB",
                    help="after timing, copy MB MiB 3 times with tg_gather and identity indices "
                         "(reference for hardware byte counters); not part of the metric")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the gated-prefill "
              "path has no multi-GPU mode here", file=sys.stderr)
        sys.exit(2)
    if args.kernels_only:
        args.no_cpu_baseline = True
        args.no_full_context = True

    import numpy as np
    import torch
    from learned_token_pruning_06_amd import ops
    from workloads import generate, random_qkv

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.time()
    if args.workload == 2:
        run_sweep(args, dev)
        return
    g = generate(args.workload)
    lanes = args.workload == WORKLOAD
    wl = g["wl"]
    log(f"inputs generated in {time.time() - t0:.1f}s")

    def tb(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    x = tb(g["x"])
    w1 = tb(g["w1"])
    b1 = torch.from_numpy(g["b1"]).to(dev)
    w2 = torch.from_numpy(g["w2"]).to(dev)
    pr = torch.from_numpy(g["prunable"]).to(dev)
    cu = torch.from_numpy(g["cu_seqlens"]).to(dev)
    kdev = torch.from_numpy(g["budgets"][0]).to(dev)
    gain = torch.from_numpy(g["gain"]).to(dev)
    temp = torch.from_numpy(g["temp"]).to(dev)
    T = wl.t_in
    cu_h = np.asarray(g["cu_seqlens"], np.int64)
    n_seq = len(cu_h) - 1
    n_prunable = [int(g["prunable"][cu_h[s]:cu_h[s + 1]].sum()) for s in range(n_seq)]
    kept_cu_h, t_kept = ops.kept_sizes(g["cu_seqlens"], n_prunable, g["budgets"][0])
    kept_lens = np.diff(np.asarray(kept_cu_h, np.int64))
    max_kept = int(kept_lens.max(initial=0))
    lib = ops.load()
    b_raw = torch.empty(T, dtype=torch.float32, device=dev)
    b = torch.empty(T, dtype=torch.float32, device=dev)
    ws_s = ops.workspace(lib.tg_score_workspace_size(T, n_seq), dev)
    ws_k = ops.workspace(lib.tg_select_workspace_size(T, n_seq), dev)
    kept_idx = torch.empty(t_kept, dtype=torch.int32, device=dev)
    kept_pos = torch.empty(t_kept, dtype=torch.int32, device=dev)
    kept_b = torch.empty(t_kept, dtype=torch.float32, device=dev)
    kept_cu = torch.empty(n_seq + 1, dtype=torch.int32, device=dev)
    x_kept = torch.empty(t_kept, wl.d, dtype=torch.bfloat16, device=dev)

    def gate():
        ops.score(x, w1, w2, pr, cu, b1=b1, eps=1e-6, b_raw=b_raw, b=b, ws=ws_s)
        ops.select_topk(b, pr, cu, kdev, t_kept, kept_idx, kept_pos, kept_b, kept_cu, ws_k)
        ops.gather(x, kept_idx, out=x_kept)

    # projection of the kept rows with tg_qkv_proj: outside the timed step (not
    # one of the four calls of the metric); timed on its own further below
    gate()
    w_all = tb(np.ascontiguousarray(np.concatenate([g["wq"].T, g["wk"].T, g["wv"].T], axis=0)))
    q, k, v = ops.qkv_proj(x_kept, w_all, wl.hq, wl.hkv, wl.dh)
    o = torch.empty_like(q)
    # the attention takes tg_gated_attn_split: with one long sequence (the
    # 128k layer) it is the plain launch; short or ragged inputs get their
    # work planned and the keys of long query blocks split
    ws_a = ops.workspace(lib.tg_gated_attn_split_workspace_size(t_kept, n_seq, max_kept, wl.hq,
                                                                wl.hkv, wl.dh), dev)
    torch.cuda.synchronize()
    assert int(kept_cu[-1].item()) == t_kept

    names = ["score", "select", "gather", "attn"]

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        ops.score(x, w1, w2, pr, cu, b1=b1, eps=1e-6, b_raw=b_raw, b=b, ws=ws_s)
        if ev is not None:
            ev[1].record()
        ops.select_topk(b, pr, cu, kdev, t_kept, kept_idx, kept_pos, kept_b, kept_cu, ws_k)
        if ev is not None:
            ev[2].record()
        ops.gather(x, kept_idx, out=x_kept)
        if ev is not None:
            ev[3].record()
        ops.gated_attn(q, k, v, kept_b, kept_pos, kept_cu, gain, temp, max_len=max_kept, out=o,
                       split=True, ws=ws_a)
        if ev is not None:
            ev[4].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log("warmup done")
    # timed region: exactly K steps, events on the stream the kernels run on
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    per = {n: [] for n in names}
    for e in evs:
        for j, n in enumerate(names):
            per[n].append(e[j].elapsed_time(e[j + 1]) * 1e3)      # us
    avg = {n: float(np.mean(per[n])) for n in names}
    med = {n: float(np.median(per[n])) for n in names}
    ms_per_step = wall * 1e3 / args.steps
    tokens_per_s = T / (wall / args.steps)
    log(f"per-kernel mean us: {avg}; step {ms_per_step:.3f} ms")

    # algorithmic work (what the method must move / compute)
    attn_flops = 2.0 * wl.dh * wl.hq * float(np.sum(kept_lens * (kept_lens + 1)))
    score_bytes = T * wl.d * 2 + wl.h * wl.d * 2 + T * (1 + 4 + 4 + 4 + 4)
    select_bytes = T * (4 + 1) + t_kept * 12
    gather_bytes = 2 * t_kept * wl.d * 2
    attn_tflops = attn_flops / (avg["attn"] * 1e-6) / 1e12
    score_gbs = score_bytes / (avg["score"] * 1e-6) / 1e9
    gate_gbs = (score_bytes + select_bytes + gather_bytes) / (
        (avg["score"] + avg["select"] + avg["gather"]) * 1e-6) / 1e9
    kern = {"attn": ("mfma", attn_tflops, PEAK_BF16_TFLOPS, "TFLOP/s", ["attn.hip", "common.h"]),
            "score": ("hbm", score_gbs, PEAK_HBM_GBS, "GB/s", ["score.hip", "common.h"])}
    dom = "attn" if avg["attn"] >= avg["score"] else "score"
    bound, ach, peak, unit, srcs = kern[dom]
    roofline = {"bound": bound, "achieved": round(ach, 2), "peak": peak, "unit": unit,
                "frac": round(ach / peak, 4), "traffic": traffic_for(dom, srcs),
                "kernel": "gated_attn_bf16" if dom == "attn" else "score_mlp_bf16",
                "avg_launch_us": round(avg[dom], 2)}
    mc = mfma_counters_for(dom, srcs)
    if mc is not None:
        roofline.update(mc)

    def time_it(fn, reps=10):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e3      # us

    proj = score_ln2 = attn_bwd = score_bwd = decode = None
    if lanes:
        # the projection of the kept rows (tg_qkv_proj), beside the step: our
        # kernel and the torch (hipBLASLt) GEMMs on the same operands
        proj_flops = 2.0 * t_kept * wl.d * (wl.hq + 2 * wl.hkv) * wl.dh
        wq_t, wk_t, wv_t = tb(g["wq"]), tb(g["wk"]), tb(g["wv"])
        t_proj = time_it(lambda: ops.qkv_proj(x_kept, w_all, wl.hq, wl.hkv, wl.dh, q=q, k=k, v=v))
        t_proj_torch = time_it(lambda: (x_kept @ wq_t, x_kept @ wk_t, x_kept @ wv_t))
        proj = {"kernel": "tg_qkv_proj", "us": round(t_proj, 2),
                "tflops": round(proj_flops / (t_proj * 1e-6) / 1e12, 1),
                "torch_matmul_us": round(t_proj_torch, 2),
                "note": "not part of the step: Q/K/V of the kept rows, 8704 x 2048 -> 2048+1024+1024"}
        del wq_t, wk_t, wv_t

        # LN2 fused into the scorer (norm_eps >= 0, the norm weight folded into
        # W1): the same rows taken as residuals, beside torch's separate RMSNorm
        # pass over them, which the fusion removes
        gam = torch.ones(wl.d, dtype=torch.bfloat16, device=dev)
        t_score_ln2 = time_it(lambda: ops.score(x, w1, w2, pr, cu, b1=b1, eps=1e-6, b_raw=b_raw, b=b,
                                                ws=ws_s, norm_eps=1e-6))
        t_rms_torch = time_it(lambda: torch.nn.functional.rms_norm(x, (wl.d,), gam, 1e-6))
        score_ln2 = {"kernel": "tg_score (norm_eps >= 0)", "us": round(t_score_ln2, 2),
                     "plain_score_us": round(avg["score"], 2),
                     "torch_rms_norm_us": round(t_rms_torch, 2),
                     "note": "scorer with the block's RMSNorm fused; the torch time is the extra "
                             "pass an unfused norm costs"}

        # the attention's backward (tg_gated_attn_bwd) on the step's kept rows:
        # bf16 inputs run on the matrix cores; algorithmic work 10 dh flop
        # per (query, key) pair and head (the five products of the backward)
        # The forward hands the backward its output and row statistic (lse2),
        # as a training step does; the time without them is reported beside.
        dout = torch.randn_like(q)
        ws_b = ops.workspace(lib.tg_gated_attn_bwd_workspace_size(t_kept, 1, wl.hq, wl.hkv), dev)
        fwd_lse2 = torch.empty((wl.hq, t_kept), dtype=torch.float32, device=dev)
        fwd_out = ops.gated_attn(q, k, v, kept_b, kept_pos, kept_cu, gain, temp, max_len=max_kept,
                                 lse2=fwd_lse2)
        t_bwd = time_it(lambda: ops.gated_attn_bwd(q, k, v, dout, kept_b, kept_pos, kept_cu, gain,
                                                   temp, ws=ws_b, fwd_out=fwd_out,
                                                   fwd_lse2=fwd_lse2), reps=3)
        t_bwd_re = time_it(lambda: ops.gated_attn_bwd(q, k, v, dout, kept_b, kept_pos, kept_cu,
                                                      gain, temp, ws=ws_b), reps=3)
        bwd_flops = 10.0 * wl.dh * wl.hq * t_kept * (t_kept + 1) / 2
        bwd_tf = bwd_flops / (t_bwd * 1e-6) / 1e12
        attn_bwd = {"kernel": "tg_gated_attn_bwd", "us": round(t_bwd, 1), "tflops": round(bwd_tf, 1),
                    "bound": "mfma", "peak_tflops": PEAK_BF16_TFLOPS,
                    "frac_of_bf16_peak": round(bwd_tf / PEAK_BF16_TFLOPS, 4),
                    "us_statistics_recomputed": round(t_bwd_re, 1),
                    "note": "8704 kept rows, bf16 inputs on the matrix cores (P, dS in bf16), "
                            "fp32 gradients; the forward's output and lse2 are passed in, so the "
                            "scores are recomputed in 2 passes (14 dh flop per pair done); "
                            "without them a third pass recomputes the statistics"}
        del dout, ws_b, fwd_lse2, fwd_out

        # the scorer's backward (tg_score_bwd) from a gradient at the kept scores:
        # recompute z, then dW1 and dx (3 products of 2 d h flop per token),
        # on the matrix cores for these bf16 shapes
        db_k = torch.randn(t_kept, dtype=torch.float32, device=dev)
        ws_sb = ops.workspace(lib.tg_score_bwd_workspace_size(T, 1, wl.d, wl.h), dev)
        t_sbwd = time_it(lambda: ops.score_bwd(x, w1, w2, pr, cu, b_raw, kept_idx, kept_cu, db_k,
                                               b1=b1, ws=ws_sb), reps=3)
        # the same with the block's RMSNorm fused in front of the scorer (the
        # rows taken as residuals): dx is then the gradient at the residual
        t_sbwd_ln2 = time_it(lambda: ops.score_bwd(x, w1, w2, pr, cu, b_raw, kept_idx, kept_cu,
                                                   db_k, b1=b1, ws=ws_sb, norm_eps=1e-6), reps=3)
        sbwd_flops = 3 * 2.0 * T * wl.d * wl.h
        sbwd_tf = sbwd_flops / (t_sbwd * 1e-6) / 1e12
        score_bwd = {"kernel": "tg_score_bwd", "us": round(t_sbwd, 1), "tflops": round(sbwd_tf, 1),
                     "bound": "mfma", "peak_tflops": PEAK_BF16_TFLOPS,
                     "frac_of_bf16_peak": round(sbwd_tf / PEAK_BF16_TFLOPS, 4),
                     "us_ln2_fused": round(t_sbwd_ln2, 1),
                     "note": "131072 tokens, d 2048, h 256, bf16 rows; dz in bf16 for the dW1 and "
                             "dx products, fp32 outputs; dx included; us_ln2_fused with the "
                             "block's RMSNorm in front (norm_eps >= 0)"}
        del db_k, ws_sb

        # one decode step after the prefill (tg_gated_decode): the new token's
        # query against the pruned cache of this layer (the kept rows' K/V plus
        # the token itself).  The calls are replayed from a HIP graph so that the
        # time is the GPU's, not the host's launch rate.
        def decode_lane(kc, vc, cb, qpos, reps):
            n = kc.shape[0]
            qd = q[-1:].contiguous()
            od = torch.empty_like(qd)
            cud = torch.tensor([0, n], dtype=torch.int32, device=dev)
            wsd = ops.workspace(lib.tg_gated_decode_workspace_size(1, wl.hq, wl.hkv, wl.dh, n), dev)
            call = lambda: ops.gated_decode(qd, kc, vc, cb, qpos, cud, gain, temp, max_cache_len=n,
                                            out=od, ws=wsd)
            call()
            torch.cuda.synchronize()
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                for _ in range(reps):
                    call()
            gr.replay()
            torch.cuda.synchronize()
            t_us = time_it(gr.replay, reps=5) / reps
            nbytes = 2.0 * n * wl.hkv * wl.dh * 2 + n * 4 + 2 * wl.hq * wl.dh * 2
            return {"cache_rows": n, "us": round(t_us, 2), "gbs": round(nbytes / (t_us * 1e-6) / 1e9, 1),
                    "frac_of_hbm_peak": round(nbytes / (t_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
        kc = torch.cat([k, k[-1:]]).contiguous()
        vc = torch.cat([v, v[-1:]]).contiguous()
        cbd = torch.cat([kept_b, torch.zeros(1, dtype=torch.float32, device=dev)])
        qpos = torch.tensor([T], dtype=torch.int32, device=dev)
        decode = {"kernel": "tg_gated_decode", "pruned_cache": decode_lane(kc, vc, cbd, qpos, 50),
                  "note": "1 sequence, the new token against the kept rows + itself; "
                          "graph replay of 50 steps, 2 launches each"}
        del kc, vc

    sweep = None
    short = None
    if lanes:
        # the 32k budget sweep (8 drawn budgets on preset scores) as a lane
        sweep = budget_sweep(generate(2), dev)
        short = short_inputs(dev)

    full = None
    if lanes and not args.no_full_context:
        # unpruned reference point: all 131072 tokens kept (stand-in Q/K/V)
        qf, kf, vf = random_qkv(3, T, wl.hq, wl.hkv, wl.dh)
        qf, kf, vf = tb(qf), tb(kf), tb(vf)
        bf_ = b.clone()
        posf = torch.arange(T, dtype=torch.int32, device=dev)
        cuf = torch.tensor([0, T], dtype=torch.int32, device=dev)
        of = torch.empty_like(qf)
        ops.gated_attn(qf, kf, vf, bf_, posf, cuf, gain, temp, max_len=T, out=of)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 3
        e0.record()
        for _ in range(reps):
            ops.gated_attn(qf, kf, vf, bf_, posf, cuf, gain, temp, max_len=T, out=of)
        e1.record()
        torch.cuda.synchronize()
        t_full = e0.elapsed_time(e1) / reps * 1e-3
        fl = 2.0 * wl.dh * wl.hq * T * (T + 1)
        # decode over the unpruned cache (the same 131072 rows, the last one new)
        decode["full_cache"] = decode_lane(kf, vf, bf_, qpos, 10)
        full = {"attn_ms": round(t_full * 1e3, 3), "attn_tflops": round(fl / t_full / 1e12, 1),
                "attn_frac_of_peak": round(fl / t_full / 1e12 / PEAK_BF16_TFLOPS, 4),
                "tokens_per_s_gate_plus_attn": round(
                    T / (t_full + (avg["score"] + avg["select"]) * 1e-6), 1),
                "note": "K = all tokens; gather is the identity and not run"}
        del qf, kf, vf, of

    if args.calibrate_copy > 0:
        # a plain copy of known size through tg_gather with identity indices:
        # MB MiB read and MB MiB written per launch (counter calibration)
        rows = args.calibrate_copy * (1 << 20) // 4096
        src = torch.ones(rows, 2048, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        ident = torch.arange(rows, dtype=torch.int32, device=dev)
        for _ in range(3):
            ops.gather(src, ident, out=dst)
        torch.cuda.synchronize()
        log(f"calibration copies: 3 x {args.calibrate_copy} MiB read + written by gather_vec16 "
            f"({rows} rows of 4096 B)")
        del src, dst, ident

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the oracle on the whole step (cpu_baseline)")
        cpu = cpu_baseline(g, kept_cu_h)

    out = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded Gaussian hidden states and random-init weights)",
        "config": {"workload": WORKLOAD_NAMES[args.workload],
                   "t_in": T, "k": [int(v) for v in g["budgets"][0]], "t_kept": t_kept, "d": wl.d,
                   "h": wl.h, "hq": wl.hq, "hkv": wl.hkv, "dh": wl.dh,
                   "step": "score+select+gather+gated_attn (Q/K/V projection excluded)"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels_us_mean": {n: round(avg[n], 2) for n in names},
        "kernels_us_median": {n: round(med[n], 2) for n in names},
        "attn_tflops": round(attn_tflops, 1),
        "attn_frac_of_bf16_peak": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
        "score_gbs": round(score_gbs, 1),
        "gate_gbs": round(gate_gbs, 1),
        "gate_frac_of_hbm_peak": round(gate_gbs / PEAK_HBM_GBS, 4),
        "full_context": full,
        "qkv_proj": proj,
        "decode": decode,
        "score_ln2": score_ln2,
        "attn_bwd": attn_bwd,
        "score_bwd": score_bwd,
        "budget_sweep": sweep,
        "attn_short_inputs": short,
    }
    print(json.dumps(out), flush=True)


def run_sweep(args, dev):
    """--workload 2: the 8-call budget sweep as the measured step (the scores
    are preset, so a call is select + gather + attention)."""
    import numpy as np
    import torch
    from workloads import generate
    g = generate(2)
    wl = g["wl"]
    log("inputs generated (budget sweep)")
    for _ in range(max(args.warmup, 1)):
        budget_sweep(g, dev, reps=1)
    t0 = time.perf_counter()
    rows = budget_sweep(g, dev, reps=args.steps)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_call = [r["select_us"] + r["gather_us"] + r["attn_us"] for r in rows]
    T = wl.t_in
    value = T * len(rows) / (sum(per_call) * 1e-6)
    fl = sum(2.0 * wl.dh * wl.hq * r["t_kept"] * (r["t_kept"] + 1) for r in rows)
    att = sum(r["attn_us"] for r in rows)
    ach = fl / (att * 1e-6) / 1e12
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(sum(per_call) * 1e-3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (preset bf16-grid Gaussian scores with +6 spikes; stand-in Q/K/V)",
        "config": {"workload": WORKLOAD_NAMES[2], "t_in": T, "k": [r["k"] for r in rows],
                   "d": wl.d, "hq": wl.hq, "hkv": wl.hkv, "dh": wl.dh,
                   "step": "8 calls of select+gather+gated_attn (scores preset, no scorer)"},
        "roofline": {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                     "traffic": None, "kernel": "gated_attn_bf16",
                     "avg_launch_us": round(att / len(rows), 2)},
        "cpu_baseline": None,
        "budget_sweep": rows,
        "wall_s": round(wall, 3),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
