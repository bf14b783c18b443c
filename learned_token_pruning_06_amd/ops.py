"""Python binding of the TokenGate gated-prefill C ABI.

Argument marshalling only: torch supplies device memory and the current
stream, every step of the computation runs in libtokengate's HIP kernels.
Each function mirrors the C call of the same name in include/tokengate.h.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence

import numpy as np
import torch

from . import _lib
from ._lib import TG_BF16, TG_F32, check, load

_DT = {torch.bfloat16: TG_BF16, torch.float32: TG_F32}


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype=None, dim=None):
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if dim is not None and t.dim() != dim:
        raise ValueError(f"{name} must have {dim} dims")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# --------------------------------------------------------------------- score
def score(x: torch.Tensor, w1: torch.Tensor, w2: torch.Tensor, prunable: torch.Tensor,
          cu_seqlens: torch.Tensor, b1: Optional[torch.Tensor] = None, b2: float = 0.0,
          eps: float = 1e-6, b_raw: Optional[torch.Tensor] = None,
          b: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
          norm_eps: Optional[float] = None):
    """tg_score: raw scores b~ and normalised scores b (f32, one per token).
    With norm_eps set, x holds the residual rows and the scorer applies the
    RMSNorm first (its weight already folded into w1)."""
    lib = load()
    _need(x, "x", (torch.bfloat16, torch.float32), 2)
    _need(w1, "w1", x.dtype, 2)
    _need(w2, "w2", torch.float32, 1)
    _need(prunable, "prunable", torch.uint8, 1)
    _need(cu_seqlens, "cu_seqlens", torch.int32, 1)
    if b1 is not None:
        _need(b1, "b1", torch.float32, 1)
    t_in, d = x.shape
    h = w1.shape[0]
    n_seq = cu_seqlens.numel() - 1
    dev = x.device
    if b_raw is None:
        b_raw = torch.empty(t_in, dtype=torch.float32, device=dev)
    if b is None:
        b = torch.empty(t_in, dtype=torch.float32, device=dev)
    need = lib.tg_score_workspace_size(t_in, n_seq)
    if ws is None:
        ws = workspace(need, dev)
    st = lib.tg_score(_p(x), _DT[x.dtype], x.stride(0), t_in, d, h, _p(w1), _p(b1), _p(w2),
                      float(b2), _p(prunable), _p(cu_seqlens), n_seq, float(eps),
                      float(-1.0 if norm_eps is None else norm_eps), _p(b_raw), _p(b),
                      _p(ws), ws.numel(), _stream(dev))
    check("tg_score", st)
    return b_raw, b


# -------------------------------------------------------------------- select
def kept_sizes(cu_seqlens_host: Sequence[int], n_prunable_host: Sequence[int],
               k_host: Sequence[int]):
    """tg_kept_sizes (host arithmetic): (kept_cu_seqlens as int32 array, t_kept)."""
    lib = load()
    cu = np.ascontiguousarray(cu_seqlens_host, dtype=np.int32)
    npr = np.ascontiguousarray(n_prunable_host, dtype=np.int32)
    kk = np.ascontiguousarray(k_host, dtype=np.int32)
    n_seq = cu.size - 1
    if npr.size != n_seq or kk.size != n_seq:
        raise ValueError("n_prunable and k need one entry per sequence")
    out = np.zeros(n_seq + 1, np.int32)
    tk = ctypes.c_int64(0)
    st = lib.tg_kept_sizes(cu.ctypes.data_as(ctypes.c_void_p), npr.ctypes.data_as(ctypes.c_void_p),
                           kk.ctypes.data_as(ctypes.c_void_p), n_seq,
                           out.ctypes.data_as(ctypes.c_void_p), ctypes.byref(tk))
    check("tg_kept_sizes", st)
    return out, int(tk.value)


def select_topk(b: torch.Tensor, prunable: torch.Tensor, cu_seqlens: torch.Tensor,
                k: torch.Tensor, t_kept: int, kept_idx: Optional[torch.Tensor] = None,
                kept_pos: Optional[torch.Tensor] = None, kept_b: Optional[torch.Tensor] = None,
                kept_cu: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                with_pos: bool = True, with_b: bool = True):
    """tg_select_topk: (kept_idx, kept_pos, kept_b, kept_cu_seqlens), all on device."""
    lib = load()
    _need(b, "b", torch.float32, 1)
    _need(prunable, "prunable", torch.uint8, 1)
    _need(cu_seqlens, "cu_seqlens", torch.int32, 1)
    _need(k, "k", torch.int32, 1)
    t_in = b.numel()
    n_seq = cu_seqlens.numel() - 1
    dev = b.device
    cap = int(t_kept)
    if kept_idx is None:
        kept_idx = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    if kept_pos is None and with_pos:
        kept_pos = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    if kept_b is None and with_b:
        kept_b = torch.empty(max(cap, 1), dtype=torch.float32, device=dev)
    if kept_cu is None:
        kept_cu = torch.empty(n_seq + 1, dtype=torch.int32, device=dev)
    need = lib.tg_select_workspace_size(t_in, n_seq)
    if ws is None:
        ws = workspace(need, dev)
    st = lib.tg_select_topk(_p(b), _p(prunable), _p(cu_seqlens), _p(k), n_seq, t_in, cap,
                            _p(kept_idx), _p(kept_pos), _p(kept_b), _p(kept_cu), _p(ws), ws.numel(),
                            _stream(dev))
    check("tg_select_topk", st)
    sl = slice(0, cap)
    return (kept_idx[sl], None if kept_pos is None else kept_pos[sl],
            None if kept_b is None else kept_b[sl], kept_cu)


def select_topk_noalloc(b: torch.Tensor, prunable: torch.Tensor, cu_seqlens: torch.Tensor,
                        k: torch.Tensor, kept_idx: torch.Tensor, kept_pos: Optional[torch.Tensor],
                        kept_b: Optional[torch.Tensor], kept_cu: torch.Tensor):
    """tg_select_topk_noalloc: the selection into caller-provided outputs
    (capacity = kept_idx.numel()), with the library's static scratch memory
    instead of a workspace; nothing is allocated."""
    lib = load()
    _need(b, "b", torch.float32, 1)
    _need(prunable, "prunable", torch.uint8, 1)
    _need(cu_seqlens, "cu_seqlens", torch.int32, 1)
    _need(k, "k", torch.int32, 1)
    _need(kept_idx, "kept_idx", torch.int32, 1)
    _need(kept_cu, "kept_cu", torch.int32, 1)
    n_seq = cu_seqlens.numel() - 1
    st = lib.tg_select_topk_noalloc(_p(b), _p(prunable), _p(cu_seqlens), _p(k), n_seq, b.numel(),
                                    kept_idx.numel(), _p(kept_idx), _p(kept_pos), _p(kept_b),
                                    _p(kept_cu), _stream(b.device))
    check("tg_select_topk_noalloc", st)


def set_contract_checks(on: bool = True):
    """tg_set_contract_checks: enqueue device-side contract checks with every
    later call (debugging aid)."""
    check("tg_set_contract_checks", load().tg_set_contract_checks(1 if on else 0))


def contract_status(device=None):
    """tg_contract_status: the set of broken rules since the last read (names
    from _lib.CONTRACT_BITS), after the current stream's work; clears them."""
    from ._lib import CONTRACT_BITS
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else device
    flags = ctypes.c_uint32(0)
    check("tg_contract_status", load().tg_contract_status(ctypes.byref(flags), _stream(dev)))
    return {name for name, bit in CONTRACT_BITS.items() if flags.value & bit}


# -------------------------------------------------------------------- gather
def gather(src: torch.Tensor, idx: torch.Tensor, out: Optional[torch.Tensor] = None):
    """tg_gather: out[r] = src[idx[r]] over the first axis of a contiguous src."""
    lib = load()
    _need(src, "src")
    _need(idx, "idx", torch.int32, 1)
    if src.dim() < 1:
        raise ValueError("src needs at least one dimension")
    row_bytes = int(np.prod(src.shape[1:], dtype=np.int64)) * src.element_size()
    n_rows = idx.numel()
    if out is None:
        out = torch.empty((n_rows,) + tuple(src.shape[1:]), dtype=src.dtype, device=src.device)
    else:
        _need(out, "out", src.dtype)
    st = lib.tg_gather(_p(src), row_bytes, src.shape[0], row_bytes, _p(idx), n_rows, _p(out),
                       row_bytes, _stream(src.device))
    check("tg_gather", st)
    return out


# ----------------------------------------------------------------- attention
def qkv_proj(x: torch.Tensor, w: torch.Tensor, hq: int, hkv: int, dh: int,
             q: Optional[torch.Tensor] = None, k: Optional[torch.Tensor] = None,
             v: Optional[torch.Tensor] = None):
    """tg_qkv_proj: q [T,Hq,dh], k/v [T,Hkv,dh] from the kept rows x [T,d] and the
    concatenated weight w [(Hq+2Hkv)*dh, d] (rows of Wq, then Wk, then Wv)."""
    lib = load()
    _need(x, "x", torch.bfloat16, 2)
    _need(w, "w", torch.bfloat16, 2)
    t, d = x.shape
    dev = x.device
    if q is None:
        q = torch.empty(t, hq, dh, dtype=x.dtype, device=dev)
    if k is None:
        k = torch.empty(t, hkv, dh, dtype=x.dtype, device=dev)
    if v is None:
        v = torch.empty(t, hkv, dh, dtype=x.dtype, device=dev)
    st = lib.tg_qkv_proj(_p(x), _DT[x.dtype], x.stride(0), t, d, _p(w), hq, hkv, dh, _p(q), _p(k),
                         _p(v), _stream(dev))
    check("tg_qkv_proj", st)
    return q, k, v


def qkv_proj_rope(x: torch.Tensor, w: torch.Tensor, hq: int, hkv: int, dh: int,
                  pos: Optional[torch.Tensor] = None, q_norm: Optional[torch.Tensor] = None,
                  k_norm: Optional[torch.Tensor] = None, norm_eps: float = 1e-6,
                  rope_theta: float = 0.0, q: Optional[torch.Tensor] = None,
                  k: Optional[torch.Tensor] = None, v: Optional[torch.Tensor] = None):
    """tg_qkv_proj_rope: qkv_proj plus the per-head RMSNorm of q and k
    (q_norm, k_norm [dh] fp32, None to skip) and the rotary embedding at
    positions pos [T] int32 (rope_theta > 1; 0 for none)."""
    lib = load()
    _need(x, "x", torch.bfloat16, 2)
    _need(w, "w", torch.bfloat16, 2)
    if pos is not None:
        _need(pos, "pos", torch.int32, 1)
    if q_norm is not None:
        _need(q_norm, "q_norm", torch.float32, 1)
    if k_norm is not None:
        _need(k_norm, "k_norm", torch.float32, 1)
    t, d = x.shape
    dev = x.device
    if q is None:
        q = torch.empty(t, hq, dh, dtype=x.dtype, device=dev)
    if k is None:
        k = torch.empty(t, hkv, dh, dtype=x.dtype, device=dev)
    if v is None:
        v = torch.empty(t, hkv, dh, dtype=x.dtype, device=dev)
    st = lib.tg_qkv_proj_rope(_p(x), _DT[x.dtype], x.stride(0), t, d, _p(w), hq, hkv, dh,
                              _p(pos), _p(q_norm), _p(k_norm), float(norm_eps),
                              float(rope_theta), _p(q), _p(k), _p(v), _stream(dev))
    check("tg_qkv_proj_rope", st)
    return q, k, v


def gated_attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, kept_b: torch.Tensor,
               kept_pos: Optional[torch.Tensor], kept_cu: torch.Tensor, gain: torch.Tensor,
               temp: torch.Tensor, max_len: Optional[int] = None,
               sm_scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
               lse2: Optional[torch.Tensor] = None, split: bool = False,
               ws: Optional[torch.Tensor] = None):
    """tg_gated_attn: token-gated causal attention, q [T,Hq,dh], k/v [T,Hkv,dh].
    lse2 (optional, f32 [Hq, T], bf16 only) receives each row's softmax
    normaliser in base 2, which gated_attn_bwd can take instead of
    recomputing it.  split=True calls tg_gated_attn_split (bf16 only), which
    splits the keys of each query block over workgroups when the query
    blocks are too few; ws is its workspace (allocated when omitted)."""
    lib = load()
    _need(q, "q", (torch.bfloat16, torch.float32), 3)
    _need(k, "k", q.dtype, 3)
    _need(v, "v", q.dtype, 3)
    _need(kept_b, "kept_b", torch.float32, 1)
    _need(kept_cu, "kept_cu", torch.int32, 1)
    _need(gain, "gain", torch.float32, 1)
    _need(temp, "temp", torch.float32, 1)
    if kept_pos is not None:
        _need(kept_pos, "kept_pos", torch.int32, 1)
    t, hq, dh = q.shape
    hkv = k.shape[1]
    if lse2 is not None:
        _need(lse2, "lse2", torch.float32, 2)
        if tuple(lse2.shape) != (hq, t):
            raise ValueError(f"lse2 must be [{hq}, {t}], got {tuple(lse2.shape)}")
    if out is None:
        out = torch.empty_like(q)
    n_seq = kept_cu.numel() - 1
    ml = int(max_len if max_len else t)
    if split:
        nbytes = lib.tg_gated_attn_split_workspace_size(t, n_seq, ml, hq, hkv, dh)
        if ws is None and nbytes > 0:
            ws = workspace(nbytes, q.device)
        st = lib.tg_gated_attn_split(_p(q), _p(k), _p(v), _DT[q.dtype], _p(out), t, _p(kept_b),
                                     _p(kept_pos), _p(kept_cu), n_seq, ml, hq, hkv, dh, _p(gain),
                                     _p(temp), float(sm_scale or 0.0), _p(lse2), _p(ws),
                                     0 if ws is None else ws.numel() * ws.element_size(),
                                     _stream(q.device))
        check("tg_gated_attn_split", st)
        return out
    st = lib.tg_gated_attn(_p(q), _p(k), _p(v), _DT[q.dtype], _p(out), t, _p(kept_b),
                           _p(kept_pos), _p(kept_cu), n_seq, ml, hq, hkv,
                           dh, _p(gain), _p(temp), float(sm_scale or 0.0), _p(lse2),
                           _stream(q.device))
    check("tg_gated_attn", st)
    return out


def score_bwd(x: torch.Tensor, w1: torch.Tensor, w2: torch.Tensor, prunable: torch.Tensor,
              cu_seqlens: torch.Tensor, b_raw: torch.Tensor, kept_idx: torch.Tensor,
              kept_cu: torch.Tensor, db_kept: torch.Tensor, b1: Optional[torch.Tensor] = None,
              eps: float = 1e-6, want_dx: bool = True, ws: Optional[torch.Tensor] = None,
              norm_eps: float = -1.0):
    """tg_score_bwd: returns (dx or None, dw1, db1, dw2, db2), all f32.

    norm_eps >= 0: x holds the residual rows and the scorer applies the
    block's second norm (w1 with the norm's weight folded in, as for
    score); dx is then the gradient at the residual rows and dw1 the one at
    the folded weight."""
    lib = load()
    _need(x, "x", (torch.bfloat16, torch.float32), 2)
    _need(w1, "w1", x.dtype, 2)
    _need(w2, "w2", torch.float32, 1)
    _need(prunable, "prunable", torch.uint8, 1)
    _need(cu_seqlens, "cu_seqlens", torch.int32, 1)
    _need(b_raw, "b_raw", torch.float32, 1)
    _need(kept_idx, "kept_idx", torch.int32, 1)
    _need(kept_cu, "kept_cu", torch.int32, 1)
    _need(db_kept, "db_kept", torch.float32, 1)
    if b1 is not None:
        _need(b1, "b1", torch.float32, 1)
    t, d = x.shape
    h = w1.shape[0]
    n_seq = cu_seqlens.numel() - 1
    f32 = dict(dtype=torch.float32, device=x.device)
    dx = torch.empty((t, d), **f32) if want_dx else None
    dw1 = torch.empty((h, d), **f32)
    db1 = torch.empty(h, **f32)
    dw2 = torch.empty(h, **f32)
    db2 = torch.empty(1, **f32)
    nbytes = lib.tg_score_bwd_workspace_size(t, n_seq, d, h)
    if ws is None:
        ws = workspace(nbytes, x.device)
    st = lib.tg_score_bwd(_p(x), _DT[x.dtype], x.stride(0), t, d, h, _p(w1), _p(b1), _p(w2),
                          _p(prunable), _p(cu_seqlens), n_seq, float(eps), float(norm_eps),
                          _p(b_raw),
                          _p(kept_idx), _p(kept_cu), kept_idx.numel(), _p(db_kept), _p(dx),
                          _p(dw1), _p(db1), _p(dw2), _p(db2), _p(ws),
                          ws.numel() * ws.element_size(), _stream(x.device))
    check("tg_score_bwd", st)
    return dx, dw1, db1, dw2, db2


def gated_attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, dout: torch.Tensor,
                   kept_b: torch.Tensor, kept_pos: Optional[torch.Tensor], kept_cu: torch.Tensor,
                   gain: torch.Tensor, temp: torch.Tensor, sm_scale: Optional[float] = None,
                   ws: Optional[torch.Tensor] = None, fwd_out: Optional[torch.Tensor] = None,
                   fwd_lse2: Optional[torch.Tensor] = None):
    """tg_gated_attn_bwd: returns (dq, dk, dv, db, dgain, dtemp), all f32.
    fwd_out and fwd_lse2 (both or neither, bf16 only): the forward's output
    and lse2, which replace the recomputation of the softmax statistics."""
    lib = load()
    _need(q, "q", (torch.bfloat16, torch.float32), 3)
    _need(k, "k", q.dtype, 3)
    _need(v, "v", q.dtype, 3)
    _need(dout, "dout", q.dtype, 3)
    _need(kept_b, "kept_b", torch.float32, 1)
    _need(kept_cu, "kept_cu", torch.int32, 1)
    _need(gain, "gain", torch.float32, 1)
    _need(temp, "temp", torch.float32, 1)
    if kept_pos is not None:
        _need(kept_pos, "kept_pos", torch.int32, 1)
    t, hq, dh = q.shape
    hkv = k.shape[1]
    if fwd_out is not None:
        _need(fwd_out, "fwd_out", q.dtype, 3)
        if fwd_out.shape != q.shape:
            raise ValueError("fwd_out must have q's shape")
    if fwd_lse2 is not None:
        _need(fwd_lse2, "fwd_lse2", torch.float32, 2)
        if tuple(fwd_lse2.shape) != (hq, t):
            raise ValueError(f"fwd_lse2 must be [{hq}, {t}]")
    n_seq = kept_cu.numel() - 1
    f32 = dict(dtype=torch.float32, device=q.device)
    dq = torch.empty((t, hq, dh), **f32)
    dk = torch.empty((t, hkv, dh), **f32)
    dv = torch.empty((t, hkv, dh), **f32)
    db = torch.empty(t, **f32)
    dgain = torch.empty(hq, **f32)
    dtemp = torch.empty(hq, **f32)
    nbytes = lib.tg_gated_attn_bwd_workspace_size(t, n_seq, hq, hkv)
    if ws is None:
        ws = workspace(nbytes, q.device)
    st = lib.tg_gated_attn_bwd(_p(q), _p(k), _p(v), _p(dout), _DT[q.dtype], t, _p(kept_b),
                               _p(kept_pos), _p(kept_cu), n_seq, hq, hkv, dh, _p(gain), _p(temp),
                               float(sm_scale or 0.0), _p(dq), _p(dk), _p(dv), _p(db), _p(dgain),
                               _p(dtemp), _p(fwd_out), _p(fwd_lse2), _p(ws),
                               ws.numel() * ws.element_size(), _stream(q.device))
    check("tg_gated_attn_bwd", st)
    return dq, dk, dv, db, dgain, dtemp


def gated_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                 cache_b: Optional[torch.Tensor], q_pos: Optional[torch.Tensor],
                 cache_cu: torch.Tensor, gain: torch.Tensor, temp: torch.Tensor,
                 max_cache_len: Optional[int] = None, sm_scale: Optional[float] = None,
                 out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None):
    """tg_gated_decode: one new token per sequence, q [n_seq,Hq,dh], against
    the caches k/v [T,Hkv,dh] whose last row per sequence is that token."""
    lib = load()
    _need(q, "q", torch.bfloat16, 3)
    _need(k_cache, "k_cache", torch.bfloat16, 3)
    _need(v_cache, "v_cache", torch.bfloat16, 3)
    _need(cache_cu, "cache_cu", torch.int32, 1)
    _need(gain, "gain", torch.float32, 1)
    _need(temp, "temp", torch.float32, 1)
    if cache_b is not None:
        _need(cache_b, "cache_b", torch.float32, 1)
    if q_pos is not None:
        _need(q_pos, "q_pos", torch.int32, 1)
    n_seq, hq, dh = q.shape
    t, hkv = k_cache.shape[0], k_cache.shape[1]
    mx = int(max_cache_len if max_cache_len is not None else t)
    if out is None:
        out = torch.empty_like(q)
    nbytes = lib.tg_gated_decode_workspace_size(n_seq, hq, hkv, dh, mx)
    if ws is None:
        ws = workspace(nbytes, q.device)
    st = lib.tg_gated_decode(_p(q), _p(k_cache), _p(v_cache), _DT[q.dtype], _p(out), t,
                             _p(cache_b), _p(q_pos), _p(cache_cu), n_seq, mx, hq, hkv, dh,
                             _p(gain), _p(temp), float(sm_scale or 0.0), _p(ws),
                             ws.numel() * ws.element_size(), _stream(q.device))
    check("tg_gated_decode", st)
    return out


# ------------------------------------------------------------------ pipeline
def gate_prefill(x, w1, w2, prunable, cu_seqlens, k, cu_seqlens_host, n_prunable_host, k_host,
                 b1=None, b2: float = 0.0, eps: float = 1e-6):
    """Score, select and gather one gated layer; returns a dict of device tensors
    plus the host-side kept sizes."""
    kept_cu_host, t_kept = kept_sizes(cu_seqlens_host, n_prunable_host, k_host)
    b_raw, b = score(x, w1, w2, prunable, cu_seqlens, b1=b1, b2=b2, eps=eps)
    kept_idx, kept_pos, kept_b, kept_cu = select_topk(b, prunable, cu_seqlens, k, t_kept)
    x_kept = gather(x, kept_idx)
    return dict(b_raw=b_raw, b=b, kept_idx=kept_idx, kept_pos=kept_pos, kept_b=kept_b,
                kept_cu=kept_cu, kept_cu_host=kept_cu_host, t_kept=t_kept, x_kept=x_kept)
