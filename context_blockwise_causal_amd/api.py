"""Torch-facing binding of libringattn: tensors in, tensors out, every step in the HIP library.

PyTorch supplies device memory and streams only.  The functions named ``ra_*`` mirror the C
entry points one to one (shape checks and pointer marshalling, nothing else); the
convenience functions at the end (``rank_view_fwd`` / ``rank_view_bwd`` /
``scaled_dot_product_attention``) allocate outputs and the workspace with torch and call the
rank-view entry points.
"""
from __future__ import annotations

import ctypes
import dataclasses

import torch

from . import _lib as L

_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class Problem:
    batch: int
    seq_len: int
    heads_q: int
    heads_kv: int
    head_dim: int
    cp: int = 1
    layout: str = "contiguous"
    dtype: str = "bf16"
    scale: float = 0.0
    window: int = 0       # sliding window (0 = off)
    attn_chunk: int = 0   # attention chunk (0 = off)

    @property
    def chunk(self) -> int:
        return self.seq_len // self.cp

    @property
    def torch_dtype(self):
        return _DT[self.dtype]

    def c(self):
        return L.problem(self.batch, self.seq_len, self.heads_q, self.heads_kv, self.head_dim,
                         self.cp, self.layout, self.dtype, self.scale, self.window, self.attn_chunk)


def to_device(store_array, dtype: str, device="cuda"):
    """A store-form numpy array (float32, or uint16 bf16 bit patterns as drawn by ``inputs``) as
    a device tensor of the problem dtype, bits unchanged."""
    import numpy as np
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(store_array).view(np.int16))
        return t.to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(store_array, dtype=np.float32)).to(device)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, shape, dtype, name):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


class Context:
    """Owns an ra_context (events) for one device."""

    def __init__(self, device: int = 0):
        lib = L.load()
        h = ctypes.c_void_p()
        L.check("ra_create", lib.ra_create(device, ctypes.byref(h)))
        self.handle = h
        self.device = device

    def set_debug(self, flags: int):
        """ra_set_debug: L.RA_DEBUG_POISON_SLOTS | L.RA_DEBUG_ROCTX, or 0."""
        L.call("ra_set_debug", self.handle, flags)

    def close(self):
        if self.handle:
            L.load().ra_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ----------------------------------------------------------------------------- host-only


def ra_validate(prob: Problem, rank: int = 0):
    p = prob.c()
    L.call("ra_validate", ctypes.byref(p), rank)


def ra_plan_step(prob: Problem, rank: int, step: int, positions: bool = False):
    """(owner, pairs): pairs as (q_row0, kv_row0, q_len, kv_len, mask), plus (q_pos0, kv_pos0)
    when positions=True."""
    p = prob.c()
    owner = ctypes.c_int32()
    n = ctypes.c_int32()
    arr = (L.ra_pair * 4)()
    L.call("ra_plan_step", ctypes.byref(p), rank, step, ctypes.byref(owner), arr, ctypes.byref(n))
    if positions:
        return owner.value, [(a.q_row0, a.kv_row0, a.q_len, a.kv_len, a.mask, a.q_pos0, a.kv_pos0)
                             for a in arr[:n.value]]
    return owner.value, [(a.q_row0, a.kv_row0, a.q_len, a.kv_len, a.mask) for a in arr[:n.value]]


def ra_workspace_size(prob: Problem, pass_: int) -> int:
    p = prob.c()
    b = ctypes.c_size_t()
    L.call("ra_workspace_size", ctypes.byref(p), pass_, ctypes.byref(b))
    return b.value


# ----------------------------------------------------------------------------- device calls


def ra_layout_gather(ctx, prob: Problem, rank_begin: int, rank_count: int, full, out=None,
                     stream=None):
    B, H, S, D = full.shape
    _need(full, (prob.batch, H, prob.seq_len, prob.head_dim), prob.torch_dtype, "full")
    if out is None:
        out = torch.empty((B, H, rank_count * prob.chunk, D), dtype=full.dtype, device=full.device)
    _need(out, (B, H, rank_count * prob.chunk, D), prob.torch_dtype, "out")
    p = prob.c()
    L.call("ra_layout_gather", ctx.handle, ctypes.byref(p), rank_begin, rank_count, H, _ptr(full),
           _ptr(out), _stream(stream))
    return out


def ra_layout_scatter(ctx, prob: Problem, rank_begin: int, rank_count: int, part, full,
                      stream=None):
    B, H, R, D = part.shape
    _need(part, (prob.batch, H, rank_count * prob.chunk, prob.head_dim), prob.torch_dtype, "part")
    _need(full, (B, H, prob.seq_len, D), prob.torch_dtype, "full")
    p = prob.c()
    L.call("ra_layout_scatter", ctx.handle, ctypes.byref(p), rank_begin, rank_count, H, _ptr(part),
           _ptr(full), _stream(stream))
    return full


def reshard_shapes(prob: Problem, step: int, heads: int):
    """(src shape, dst shape) of a Ulysses re-shard step over `heads` heads."""
    cp, B, S, D = prob.cp, prob.batch, prob.seq_len, prob.head_dim
    Hh, Sc = heads // cp, S // cp
    seq, xbuf, head = (B, heads, Sc, D), (cp, B, Hh, Sc, D), (B, Hh, S, D)
    return {L.RA_A2A_SEQ_PACK: (seq, xbuf), L.RA_A2A_HEAD_UNPACK: (xbuf, head),
            L.RA_A2A_HEAD_PACK: (head, xbuf), L.RA_A2A_SEQ_UNPACK: (xbuf, seq)}[step]


def ra_ulysses_reshard(ctx, prob: Problem, step: int, heads: int, src, dst=None, stream=None):
    """One Ulysses re-shard step (see include/ra.h); allocates dst when not given."""
    if heads % prob.cp or prob.seq_len % prob.cp:
        raise ValueError("heads and seq_len must be divisible by cp")
    if step not in (L.RA_A2A_SEQ_PACK, L.RA_A2A_HEAD_UNPACK, L.RA_A2A_HEAD_PACK, L.RA_A2A_SEQ_UNPACK):
        raise ValueError(f"unknown re-shard step {step}")
    ss, ds = reshard_shapes(prob, step, heads)
    _need(src, ss, prob.torch_dtype, "src")
    if dst is None:
        dst = torch.empty(ds, dtype=prob.torch_dtype, device=src.device)
    _need(dst, ds, prob.torch_dtype, "dst")
    p = prob.c()
    L.call("ra_ulysses_reshard", ctx.handle, ctypes.byref(p), step, heads, _ptr(src), _ptr(dst),
           _stream(stream))
    return dst


def ra_stage_kv(ctx, prob: Problem, owner: int, k_ring, v_ring, dst=None, stream=None):
    """Owner's K and V chunk out of the ring tensors into `dst` (K then V): a uint8-viewable
    device tensor of 2 * batch * heads_kv * chunk * head_dim elements of the problem dtype
    (allocated here when None, shaped (2, batch, heads_kv, chunk, head_dim))."""
    kshp = (prob.batch, prob.heads_kv, prob.seq_len, prob.head_dim)
    _need(k_ring, kshp, prob.torch_dtype, "k_ring")
    _need(v_ring, kshp, prob.torch_dtype, "v_ring")
    shp = (2, prob.batch, prob.heads_kv, prob.chunk, prob.head_dim)
    if dst is None:
        dst = torch.empty(shp, dtype=prob.torch_dtype, device=k_ring.device)
    _need(dst, shp, prob.torch_dtype, "dst")
    p = prob.c()
    L.call("ra_stage_kv", ctx.handle, ctypes.byref(p), owner, _ptr(k_ring), _ptr(v_ring), _ptr(dst),
           _stream(stream))
    return dst


def new_state(prob: Problem, rows: int, device="cuda"):
    U = torch.empty((prob.batch, prob.heads_q, rows, prob.head_dim), dtype=torch.float32, device=device)
    m = torch.empty((prob.batch, prob.heads_q, rows), dtype=torch.float32, device=device)
    l = torch.empty_like(m)
    return U, m, l


def ra_state_init(ctx, prob: Problem, U, m, l, stream=None):
    rows = U.shape[2]
    _need(U, (prob.batch, prob.heads_q, rows, prob.head_dim), torch.float32, "U")
    _need(m, (prob.batch, prob.heads_q, rows), torch.float32, "m")
    _need(l, (prob.batch, prob.heads_q, rows), torch.float32, "l")
    p = prob.c()
    L.call("ra_state_init", ctx.handle, ctypes.byref(p), rows, _ptr(U), _ptr(m), _ptr(l),
           _stream(stream))


def ra_chunk_fwd(ctx, prob: Problem, q, k, v, pairs, U, m, l, stream=None):
    B, Hq, q_rows, D = q.shape
    kv_rows = k.shape[2]
    _need(q, (prob.batch, prob.heads_q, q_rows, prob.head_dim), prob.torch_dtype, "q")
    _need(k, (prob.batch, prob.heads_kv, kv_rows, prob.head_dim), prob.torch_dtype, "k")
    _need(v, (prob.batch, prob.heads_kv, kv_rows, prob.head_dim), prob.torch_dtype, "v")
    _need(U, (B, Hq, q_rows, D), torch.float32, "U")
    _need(m, (B, Hq, q_rows), torch.float32, "m")
    _need(l, (B, Hq, q_rows), torch.float32, "l")
    p = prob.c()
    arr = L.pairs_array(pairs)
    L.call("ra_chunk_fwd", ctx.handle, ctypes.byref(p), _ptr(q), q_rows, _ptr(k), _ptr(v), kv_rows,
           arr, len(pairs), _ptr(U), _ptr(m), _ptr(l), _stream(stream))


def ra_lse_merge(ctx, prob: Problem, o_part, lse_part, U, m, l, stream=None):
    rows = U.shape[2]
    shp = (prob.batch, prob.heads_q, rows)
    _need(o_part, shp + (prob.head_dim,), torch.float32, "o_part")
    _need(lse_part, shp, torch.float32, "lse_part")
    _need(U, shp + (prob.head_dim,), torch.float32, "U")
    _need(m, shp, torch.float32, "m")
    _need(l, shp, torch.float32, "l")
    p = prob.c()
    L.call("ra_lse_merge", ctx.handle, ctypes.byref(p), rows, _ptr(o_part), _ptr(lse_part), _ptr(U),
           _ptr(m), _ptr(l), _stream(stream))


def ra_fwd_finalize(ctx, prob: Problem, U, m, l, o=None, lse=None, stream=None):
    rows = U.shape[2]
    shp = (prob.batch, prob.heads_q, rows)
    _need(U, shp + (prob.head_dim,), torch.float32, "U")
    _need(m, shp, torch.float32, "m")
    _need(l, shp, torch.float32, "l")
    if o is None:
        o = torch.empty(shp + (prob.head_dim,), dtype=prob.torch_dtype, device=U.device)
    if lse is None:
        lse = torch.empty(shp, dtype=torch.float32, device=U.device)
    p = prob.c()
    L.call("ra_fwd_finalize", ctx.handle, ctypes.byref(p), rows, _ptr(U), _ptr(m), _ptr(l), _ptr(o),
           _ptr(lse), _stream(stream))
    return o, lse


def ra_bwd_preprocess(ctx, prob: Problem, o, dO, delta=None, stream=None):
    rows = o.shape[2]
    shp = (prob.batch, prob.heads_q, rows)
    _need(o, shp + (prob.head_dim,), prob.torch_dtype, "o")
    _need(dO, shp + (prob.head_dim,), prob.torch_dtype, "dO")
    if delta is None:
        delta = torch.empty(shp, dtype=torch.float32, device=o.device)
    p = prob.c()
    L.call("ra_bwd_preprocess", ctx.handle, ctypes.byref(p), rows, _ptr(o), _ptr(dO), _ptr(delta),
           _stream(stream))
    return delta


def ra_chunk_bwd(ctx, prob: Problem, q, dO, lse, delta, k, v, pairs, dq_acc, dk_acc, dv_acc,
                 stream=None):
    q_rows = q.shape[2]
    kv_rows = k.shape[2]
    qs = (prob.batch, prob.heads_q, q_rows)
    ks = (prob.batch, prob.heads_kv, kv_rows, prob.head_dim)
    _need(q, qs + (prob.head_dim,), prob.torch_dtype, "q")
    _need(dO, qs + (prob.head_dim,), prob.torch_dtype, "dO")
    _need(lse, qs, torch.float32, "lse")
    _need(delta, qs, torch.float32, "delta")
    _need(k, ks, prob.torch_dtype, "k")
    _need(v, ks, prob.torch_dtype, "v")
    if dq_acc is not None:
        _need(dq_acc, qs + (prob.head_dim,), torch.float32, "dq_acc")
    if dk_acc is not None:
        _need(dk_acc, ks, torch.float32, "dk_acc")
    if dv_acc is not None:
        _need(dv_acc, ks, torch.float32, "dv_acc")
    p = prob.c()
    arr = L.pairs_array(pairs)
    L.call("ra_chunk_bwd", ctx.handle, ctypes.byref(p), _ptr(q), _ptr(dO), _ptr(lse), _ptr(delta),
           q_rows, _ptr(k), _ptr(v), kv_rows, arr, len(pairs), _ptr(dq_acc), _ptr(dk_acc),
           _ptr(dv_acc), _stream(stream))


def ra_chunk_bwd_ds_size(prob: Problem, q_rows: int, kv_rows: int, pairs) -> int:
    """Scratch bytes of ra_chunk_bwd_ds for this pair list (0 for fp32 problems)."""
    p = prob.c()
    arr = L.pairs_array(pairs)
    n = ctypes.c_size_t()
    L.call("ra_chunk_bwd_ds_size", ctypes.byref(p), q_rows, kv_rows, arr, len(pairs), ctypes.byref(n))
    return n.value


def ra_chunk_bwd_ds(ctx, prob: Problem, q, dO, lse, delta, k, v, pairs, dq_acc, dk_acc, dv_acc,
                    scratch=None, stream=None):
    """Chunk backward with stored dS: dK/dV kernel (which stores dS) then dQ = dS K.  dq_acc =
    None runs the first kernel only, dk_acc = dv_acc = None the second only (reading the scratch
    of an earlier first-phase call).  `scratch` is a uint8 device tensor of at least
    ra_chunk_bwd_ds_size bytes (allocated here when None)."""
    q_rows = q.shape[2]
    kv_rows = k.shape[2]
    qs = (prob.batch, prob.heads_q, q_rows)
    ks = (prob.batch, prob.heads_kv, kv_rows, prob.head_dim)
    _need(q, qs + (prob.head_dim,), prob.torch_dtype, "q")
    _need(dO, qs + (prob.head_dim,), prob.torch_dtype, "dO")
    _need(lse, qs, torch.float32, "lse")
    _need(delta, qs, torch.float32, "delta")
    _need(k, ks, prob.torch_dtype, "k")
    _need(v, ks, prob.torch_dtype, "v")
    if dq_acc is not None:
        _need(dq_acc, qs + (prob.head_dim,), torch.float32, "dq_acc")
    if dk_acc is not None:
        _need(dk_acc, ks, torch.float32, "dk_acc")
    if dv_acc is not None:
        _need(dv_acc, ks, torch.float32, "dv_acc")
    if scratch is None:
        nbytes = ra_chunk_bwd_ds_size(prob, q_rows, kv_rows, pairs)
        scratch = torch.empty(max(16, nbytes), dtype=torch.uint8, device=q.device)
    p = prob.c()
    arr = L.pairs_array(pairs)
    L.call("ra_chunk_bwd_ds", ctx.handle, ctypes.byref(p), _ptr(q), _ptr(dO), _ptr(lse), _ptr(delta),
           q_rows, _ptr(k), _ptr(v), kv_rows, arr, len(pairs), _ptr(dq_acc), _ptr(dk_acc),
           _ptr(dv_acc), _ptr(scratch), scratch.numel(), _stream(stream))
    return scratch


def ra_chunk_bwd_ds_noalloc(ctx, prob: Problem, q, dO, lse, delta, k, v, pairs, dq_acc, dk_acc, dv_acc,
                            stream=None):
    """ra_chunk_bwd_ds with the library's static scratch (no device allocation by the call): at most
    RA_NOALLOC_SCRATCH_BYTES of stored dS; calls that overlap on one GPU race for it."""
    q_rows = q.shape[2]
    kv_rows = k.shape[2]
    qs = (prob.batch, prob.heads_q, q_rows)
    ks = (prob.batch, prob.heads_kv, kv_rows, prob.head_dim)
    _need(q, qs + (prob.head_dim,), prob.torch_dtype, "q")
    _need(dO, qs + (prob.head_dim,), prob.torch_dtype, "dO")
    _need(lse, qs, torch.float32, "lse")
    _need(delta, qs, torch.float32, "delta")
    _need(k, ks, prob.torch_dtype, "k")
    _need(v, ks, prob.torch_dtype, "v")
    if dq_acc is not None:
        _need(dq_acc, qs + (prob.head_dim,), torch.float32, "dq_acc")
    if dk_acc is not None:
        _need(dk_acc, ks, torch.float32, "dk_acc")
    if dv_acc is not None:
        _need(dv_acc, ks, torch.float32, "dv_acc")
    p = prob.c()
    arr = L.pairs_array(pairs)
    L.call("ra_chunk_bwd_ds_noalloc", ctx.handle, ctypes.byref(p), _ptr(q), _ptr(dO), _ptr(lse), _ptr(delta),
           q_rows, _ptr(k), _ptr(v), kv_rows, arr, len(pairs), _ptr(dq_acc), _ptr(dk_acc), _ptr(dv_acc),
           _stream(stream))


def ra_cast_from_f32(ctx, prob: Problem, src, dst=None, stream=None):
    if src.dtype != torch.float32 or not src.is_contiguous():
        raise ValueError("src must be a contiguous float32 tensor")
    if dst is None:
        dst = torch.empty(src.shape, dtype=prob.torch_dtype, device=src.device)
    _need(dst, tuple(src.shape), prob.torch_dtype, "dst")
    p = prob.c()
    L.call("ra_cast_from_f32", ctx.handle, ctypes.byref(p), src.numel(), _ptr(src), _ptr(dst),
           _stream(stream))
    return dst


def ra_rank_view_fwd(ctx, prob: Problem, rank: int, q_slice, k_ring, v_ring, o_slice, lse_slice,
                     workspace, compute=None, staging=None):
    shp = (prob.batch, prob.heads_q, prob.chunk)
    kshp = (prob.batch, prob.heads_kv, prob.seq_len, prob.head_dim)
    _need(q_slice, shp + (prob.head_dim,), prob.torch_dtype, "q_slice")
    _need(k_ring, kshp, prob.torch_dtype, "k_ring")
    _need(v_ring, kshp, prob.torch_dtype, "v_ring")
    _need(o_slice, shp + (prob.head_dim,), prob.torch_dtype, "o_slice")
    _need(lse_slice, shp, torch.float32, "lse_slice")
    p = prob.c()
    cs = _stream(compute)
    ss = _stream(staging) if staging is not None else cs
    L.call("ra_rank_view_fwd", ctx.handle, ctypes.byref(p), rank, _ptr(q_slice), _ptr(k_ring),
           _ptr(v_ring), _ptr(o_slice), _ptr(lse_slice), _ptr(workspace),
           workspace.numel() * workspace.element_size(), cs, ss)


def ra_rank_view_bwd(ctx, prob: Problem, rank: int, q_slice, k_ring, v_ring, o_slice, lse_slice,
                     dO_slice, dq_slice, dk_ring, dv_ring, workspace, compute=None, staging=None):
    shp = (prob.batch, prob.heads_q, prob.chunk)
    kshp = (prob.batch, prob.heads_kv, prob.seq_len, prob.head_dim)
    for name, t in (("q_slice", q_slice), ("o_slice", o_slice), ("dO_slice", dO_slice),
                    ("dq_slice", dq_slice)):
        _need(t, shp + (prob.head_dim,), prob.torch_dtype, name)
    for name, t in (("k_ring", k_ring), ("v_ring", v_ring), ("dk_ring", dk_ring), ("dv_ring", dv_ring)):
        _need(t, kshp, prob.torch_dtype, name)
    _need(lse_slice, shp, torch.float32, "lse_slice")
    p = prob.c()
    cs = _stream(compute)
    ss = _stream(staging) if staging is not None else cs
    L.call("ra_rank_view_bwd", ctx.handle, ctypes.byref(p), rank, _ptr(q_slice), _ptr(k_ring),
           _ptr(v_ring), _ptr(o_slice), _ptr(lse_slice), _ptr(dO_slice), _ptr(dq_slice),
           _ptr(dk_ring), _ptr(dv_ring), _ptr(workspace), workspace.numel() * workspace.element_size(),
           cs, ss)


# ----------------------------------------------------------------------------- convenience


def workspace(prob: Problem, pass_: int, device="cuda"):
    n = ra_workspace_size(prob, pass_)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device)


def rank_view_fwd(ctx, prob: Problem, rank: int, q_slice, k_ring, v_ring, ws=None, compute=None,
                  staging=None):
    o = torch.empty_like(q_slice)
    lse = torch.empty((prob.batch, prob.heads_q, prob.chunk), dtype=torch.float32, device=q_slice.device)
    if ws is None:
        ws = workspace(prob, 0, q_slice.device)
    ra_rank_view_fwd(ctx, prob, rank, q_slice, k_ring, v_ring, o, lse, ws, compute, staging)
    return o, lse


def rank_view_fwd_split(ctx, prob: Problem, rank: int, q_slice, k_all, v_all, ws=None, compute=None,
                        merge=None, out=None):
    """All-gather mode with split-KV (see include/ra.h): returns (o, lse)."""
    B, Hq, C, D = prob.batch, prob.heads_q, prob.chunk, prob.head_dim
    _need(q_slice, (B, Hq, C, D), prob.torch_dtype, "q_slice")
    _need(k_all, (B, prob.heads_kv, prob.seq_len, D), prob.torch_dtype, "k_all")
    _need(v_all, (B, prob.heads_kv, prob.seq_len, D), prob.torch_dtype, "v_all")
    if out is None:
        o = torch.empty_like(q_slice)
        lse = torch.empty((B, Hq, C), dtype=torch.float32, device=q_slice.device)
    else:
        o, lse = out
    if ws is None:
        ws = workspace(prob, 2, q_slice.device)
    p = prob.c()
    L.call("ra_rank_view_fwd_split", ctx.handle, ctypes.byref(p), rank, _ptr(q_slice), _ptr(k_all),
           _ptr(v_all), _ptr(o), _ptr(lse), _ptr(ws), ws.numel(), _stream(compute), _stream(merge))
    return o, lse


def rank_view_bwd(ctx, prob: Problem, rank: int, q_slice, k_ring, v_ring, o, lse, dO, ws=None,
                  compute=None, staging=None):
    dq = torch.empty_like(q_slice)
    dk = torch.empty_like(k_ring)
    dv = torch.empty_like(v_ring)
    if ws is None:
        ws = workspace(prob, 1, q_slice.device)
    ra_rank_view_bwd(ctx, prob, rank, q_slice, k_ring, v_ring, o, lse, dO, dq, dk, dv, ws, compute,
                     staging)
    return dq, dk, dv


def scaled_dot_product_attention(ctx, q, k, v, n_rep: int, scale: float = 0.0):
    """Causal attention of full sequences on one GPU (cp = 1): q (B,Hq,S,D), k/v (B,Hq/n_rep,S,D).

    The call shape of the attention helper in "Feat: Context Parallel" (n_rep = Hq / Hkv, the
    head grouping done inside the kernel).  Returns (o, lse).
    """
    B, Hq, S, D = q.shape
    if Hq % n_rep or k.shape[1] != Hq // n_rep:
        raise ValueError("k/v must have heads_q / n_rep heads")
    dt = {torch.bfloat16: "bf16", torch.float32: "f32"}[q.dtype]
    prob = Problem(B, S, Hq, Hq // n_rep, D, 1, "contiguous", dt, scale)
    return rank_view_fwd(ctx, prob, 0, q, k, v)
