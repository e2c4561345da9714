"""FP64 CPU oracle for one context-parallel rank's share of blockwise causal self-attention.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import this module.  The product path (the HIP library and its
Python binding) never imports, calls or links it, and this module imports nothing from the
product: it takes plain numpy arrays and returns plain numpy arrays.

What it computes, and from which passage of the pages:

* Attention is the plain definition softmax(Q K^T * scale + causal mask) V, with the safe
  (max-subtracted) softmax -- lecture note "上下文并行", section "朴素 Ring Attention", the
  softmax and safe-softmax equations and the per-step partial-attention equation; the
  InfiniTrain pull request "Feat: Context Parallel" review thread that spells the chain
  q@k^T * 1/sqrt(D) -> MaskedFill -> Softmax -> @v.
* Causal visibility: a query at global position t sees the keys at positions j <= t, itself
  included (lecture note "上下文并行", section "Zig-Zag Ring Attention", the statement of which
  tokens each token attends to).
* GQA: query head h reads key/value head h // n_rep, n_rep = Hq / Hkv.  This is the grouping
  that the RepeatKVHeads gradient reshape (B, H/n_rep, n_rep, T, D).Sum(2) implies
  ("Feat: Context Parallel", review thread on the attention helper).
* Sequence layouts: contiguous (default) or zigzag head/tail pairing where, for 2*cp chunks,
  rank r holds chunks r and 2*cp-1-r ("Feat: Context Parallel" section 主要改动; lecture
  note "Zig-Zag Ring Attention", the cp_size = 4 example).
* Ring order: each round a rank sends its K/V to the next rank and receives from the
  previous one ("朴素 Ring Attention", the 4-GPU walk-through), so at step i rank r holds the
  chunk owned by rank (r - i) mod cp.
* Online-softmax state (running max m, running sum l, unnormalised output U) and its update
  per K/V block, which the lecture note derives from FlashAttention-2 ("朴素 Ring Attention",
  the order-independence argument).  The oracle's attention itself does NOT use this update:
  it computes every row with two passes (max, then exp / sum / PV) over the row's whole causal
  key set.  The online functions below exist only to be pinned against that definition and to
  serve as the reference for the library's state-merge entry point.
* Backward: the analytic gradient of sum_t <dO_t, O_t> over the rank's rows, i.e. the
  recompute backward the "Feat: Context Parallel" p2p mode describes (probabilities recomputed
  from the saved log-sum-exp; K/V gradients returned to the owner).

Readings where the pages are silent or garbled:
  scale = 1/sqrt(head_dim); the softmax sum runs over the row's visible keys; masked scores are
  excluded exactly (probability 0); LSE is the natural log; a rank view's dK/dV is the
  contribution of that rank's query rows only.

Every function works in float64 and is written for a reader to check against the
definitions, not for speed: rows are processed in blocks only to bound memory.
"""
from __future__ import annotations

import math

import numpy as np

FULL = "FULL"
DIAG = "DIAG"
SKIP = "SKIP"

# ----------------------------------------------------------------------------- layouts


def n_chunks(cp: int, layout: str) -> int:
    """Number of sequence chunks: cp for contiguous, 2*cp for zigzag."""
    if layout == "contiguous":
        return cp
    if layout == "zigzag":
        return 2 * cp
    raise ValueError(f"unknown layout {layout!r}")


def rank_chunks(cp: int, layout: str, rank: int) -> list:
    """Chunk indices a rank holds, in slice order (early chunk first for zigzag)."""
    if not 0 <= rank < cp:
        raise ValueError("rank out of range")
    if layout == "contiguous":
        return [rank]
    return [rank, 2 * cp - 1 - rank]


def rank_positions(seq_len: int, cp: int, layout: str, rank: int) -> np.ndarray:
    """Global token positions of a rank's slice, in slice order."""
    nc = n_chunks(cp, layout)
    if seq_len % nc:
        raise ValueError("sequence length must split into equal chunks")
    c = seq_len // nc
    return np.concatenate([np.arange(ch * c, (ch + 1) * c, dtype=np.int64)
                           for ch in rank_chunks(cp, layout, rank)])


def ring_owner(cp: int, rank: int, step: int) -> int:
    """Owner of the K/V chunk a rank holds at ring step ``step`` (received from rank-1 each step)."""
    return (rank - step) % cp


# ----------------------------------------------------------------------------- step plans


def classify(q_pos: np.ndarray, k_pos: np.ndarray) -> str:
    """Mask kind of a (Q block, K/V block) pair, read off its causal visibility matrix.

    FULL: every key visible to every query.  SKIP: no key visible.  DIAG: the blocks have
    equal length and key j is visible to query i exactly when j <= i (local indices).
    """
    vis = k_pos[None, :] <= q_pos[:, None]
    if vis.all():
        return FULL
    if not vis.any():
        return SKIP
    if len(q_pos) == len(k_pos) and np.array_equal(vis, np.tril(np.ones_like(vis))):
        return DIAG
    raise ValueError("pair is neither full, diagonal nor empty")


def plan_step(seq_len: int, cp: int, layout: str, rank: int, step: int):
    """Pairs one rank computes at one ring step, by brute-force classification of positions.

    Returns (owner, pairs) where each pair is (q_row0, kv_row0, q_len, kv_len, kind); q rows
    are offsets in the rank's Q slice and kv rows are offsets in the owner's K/V chunk.
    """
    owner = ring_owner(cp, rank, step)
    c = seq_len // n_chunks(cp, layout)
    pairs = []
    for qi, qch in enumerate(rank_chunks(cp, layout, rank)):
        for ki, kch in enumerate(rank_chunks(cp, layout, owner)):
            qp = np.arange(qch * c, (qch + 1) * c)
            kp = np.arange(kch * c, (kch + 1) * c)
            pairs.append((qi * c, ki * c, c, c, classify(qp, kp)))
    return owner, pairs


def pair_positions(kind: str, q_len: int, kv_len: int):
    """Positions that realise a single pair of the given kind (for chunk-level references)."""
    if kind == FULL:
        return kv_len + np.arange(q_len), np.arange(kv_len)
    if kind == DIAG:
        if q_len != kv_len:
            raise ValueError("a diagonal pair needs q_len == kv_len")
        return np.arange(q_len), np.arange(kv_len)
    if kind == SKIP:
        return np.arange(q_len), q_len + np.arange(kv_len)
    raise ValueError(kind)


# ----------------------------------------------------------------------------- attention


def _scale(d: int, scale):
    return 1.0 / math.sqrt(d) if not scale else float(scale)


def _row_block(n_keys: int) -> int:
    return int(max(16, min(512, (1 << 25) // max(1, n_keys))))


def _key_limit(k_pos: np.ndarray, k_sorted: bool, qmax: int) -> int:
    if k_sorted:
        return int(np.searchsorted(k_pos, qmax, side="right"))
    return len(k_pos)


def visible(q_pos, k_pos, window: int = 0, attn_chunk: int = 0):
    """Visibility matrix (len(q_pos), len(k_pos)) of the causal mask and its two restrictions.

    Causal: key j is visible to query t iff j <= t, the diagonal included ("Zig-Zag Ring
    Attention" section of the lecture note).  The transformers context-parallel page names two further masks the attention
    call must rebuild over the whole sequence, sliding-window and chunked attention; read as
    the usual definitions: with a window W > 0 the query also needs t - j < W (itself and the
    W - 1 keys before it), with an attention chunk C > 0 it needs j // C == t // C (keys of its
    own chunk of C positions).  0 disables either restriction.
    """
    q_pos = np.asarray(q_pos, np.int64)[:, None]
    k_pos = np.asarray(k_pos, np.int64)[None, :]
    vis = k_pos <= q_pos
    if window:
        vis = vis & (q_pos - k_pos < window)
    if attn_chunk:
        vis = vis & (k_pos // attn_chunk == q_pos // attn_chunk)
    return vis


def attention_rows(q, k, v, q_pos, k_pos, scale=None, window: int = 0, attn_chunk: int = 0):
    """Causal attention for the query rows ``q_pos`` against keys at ``k_pos``, optionally with
    a sliding window or attention chunks (``visible``).

    q: (B, Hq, T, D); k, v: (B, Hkv, Tk, D); float64.  Returns O (B, Hq, T, D) and the
    natural-log LSE (B, Hq, T).  Rows with no visible key get O = 0 and LSE = -inf.
    Two passes per row block: the row max of the visible scores, then exp / sum / PV.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    q_pos = np.asarray(q_pos, np.int64)
    k_pos = np.asarray(k_pos, np.int64)
    B, Hq, T, D = q.shape
    Hkv = k.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    n_rep = Hq // Hkv
    sc = _scale(D, scale)
    k_sorted = bool(np.all(np.diff(k_pos) >= 0))
    o = np.zeros((B, Hq, T, D))
    lse = np.full((B, Hq, T), -np.inf)
    rb = _row_block(len(k_pos))
    for b in range(B):
        for h in range(Hq):
            g = h // n_rep
            for r0 in range(0, T, rb):
                qp = q_pos[r0:r0 + rb]
                kn = _key_limit(k_pos, k_sorted, int(qp.max()))
                if kn == 0:
                    continue
                s = sc * (q[b, h, r0:r0 + rb] @ k[b, g, :kn].T)
                vis = visible(qp, k_pos[:kn], window, attn_chunk)
                s = np.where(vis, s, -np.inf)
                m = s.max(axis=1)
                has = np.isfinite(m)
                m_safe = np.where(has, m, 0.0)
                p = np.where(vis, np.exp(s - m_safe[:, None]), 0.0)
                l = p.sum(axis=1)
                with np.errstate(divide="ignore", invalid="ignore"):
                    o[b, h, r0:r0 + rb] = np.where(has[:, None], (p @ v[b, g, :kn]) / l[:, None], 0.0)
                    lse[b, h, r0:r0 + rb] = np.where(has, m_safe + np.log(l), -np.inf)
    return o, lse


def attention_rows_bwd(q, k, v, do, q_pos, k_pos, scale=None, window: int = 0, attn_chunk: int = 0):
    """Analytic gradient of sum over the given rows of <dO_t, O_t>.

    Returns dq (B, Hq, T, D) and dk, dv (B, Hkv, Tk, D); dk/dv of a key/value head sum the
    contributions of all query heads that read it.  Per row t and key j:
      D_t = <dO_t, O_t>,  P_tj = exp(s_tj - LSE_t),  dP_tj = <dO_t, v_j>,
      dS_tj = P_tj (dP_tj - D_t),  dq_t = scale sum_j dS_tj k_j,
      dk_j = scale sum_t dS_tj q_t,  dv_j = sum_t P_tj dO_t.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(do, np.float64)
    q_pos = np.asarray(q_pos, np.int64)
    k_pos = np.asarray(k_pos, np.int64)
    B, Hq, T, D = q.shape
    Hkv = k.shape[1]
    n_rep = Hq // Hkv
    sc = _scale(D, scale)
    o, lse = attention_rows(q, k, v, q_pos, k_pos, scale, window, attn_chunk)
    delta = np.sum(do * o, axis=-1)
    k_sorted = bool(np.all(np.diff(k_pos) >= 0))
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    rb = _row_block(len(k_pos))
    for b in range(B):
        for h in range(Hq):
            g = h // n_rep
            for r0 in range(0, T, rb):
                qp = q_pos[r0:r0 + rb]
                kn = _key_limit(k_pos, k_sorted, int(qp.max()))
                if kn == 0:
                    continue
                qb = q[b, h, r0:r0 + rb]
                dob = do[b, h, r0:r0 + rb]
                s = sc * (qb @ k[b, g, :kn].T)
                vis = visible(qp, k_pos[:kn], window, attn_chunk)
                lb = lse[b, h, r0:r0 + rb]
                lb_safe = np.where(np.isfinite(lb), lb, 0.0)
                p = np.where(vis, np.exp(s - lb_safe[:, None]), 0.0)
                dp = dob @ v[b, g, :kn].T
                ds = p * (dp - delta[b, h, r0:r0 + rb][:, None])
                dq[b, h, r0:r0 + rb] = sc * (ds @ k[b, g, :kn])
                dk[b, g, :kn] += sc * (ds.T @ qb)
                dv[b, g, :kn] += p.T @ dob
    return dq, dk, dv


def key_grads(q, k, v, do, q_pos, k_pos, o, lse, scale=None, window: int = 0, attn_chunk: int = 0):
    """dK and dV of the keys at ``k_pos`` from the query rows at ``q_pos``, given those rows'
    output O and LSE over their whole visible key set (from ``attention_rows``).

    The same gradient as ``attention_rows_bwd`` restricted to a subset of keys: a key's gradient
    needs, besides its own scores, only the row statistics LSE_t and D_t = <dO_t, O_t>, so the
    rows' keys outside the subset enter through O and LSE alone.  Per row t and key j:
      P_tj = exp(s_tj - LSE_t),  dS_tj = P_tj (<dO_t, v_j> - D_t),
      dk_j = scale sum_t dS_tj q_t,  dv_j = sum_t P_tj dO_t  (summed over the query heads
    that read the key's head).  q, do, o: (B, Hq, T, D); lse: (B, Hq, T); k, v: the subset's
    keys and values (B, Hkv, Tk, D).  Returns dk, dv (B, Hkv, Tk, D).
    """
    q, k, v, do, o, lse = (np.asarray(a, np.float64) for a in (q, k, v, do, o, lse))
    B, Hq, T, D = q.shape
    n_rep = Hq // k.shape[1]
    sc = _scale(D, scale)
    delta = np.sum(do * o, axis=-1)
    vis = visible(q_pos, k_pos, window, attn_chunk)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            g = h // n_rep
            lb = np.where(np.isfinite(lse[b, h]), lse[b, h], 0.0)
            p = np.where(vis, np.exp(sc * (q[b, h] @ k[b, g].T) - lb[:, None]), 0.0)
            ds = p * (do[b, h] @ v[b, g].T - delta[b, h][:, None])
            dk[b, g] += sc * (ds.T @ q[b, h])
            dv[b, g] += p.T @ do[b, h]
    return dk, dv


# ----------------------------------------------------------------------------- rank views


def rank_view_fwd(q, k, v, cp: int, layout: str, rank: int, scale=None, window: int = 0,
                  attn_chunk: int = 0):
    """O and LSE of one rank's Q slice, from full-sequence Q (B,Hq,S,D), K, V (B,Hkv,S,D).

    Rows are independent, so this is the full-sequence causal attention restricted to the
    rank's positions (slice order).
    """
    S = q.shape[2]
    pos = rank_positions(S, cp, layout, rank)
    return attention_rows(np.asarray(q)[:, :, pos], k, v, pos, np.arange(S), scale, window, attn_chunk)


def rank_view_bwd(q, k, v, do_slice, cp: int, layout: str, rank: int, scale=None, window: int = 0,
                  attn_chunk: int = 0):
    """dQ of the rank's slice and the rank's full-sequence dK, dV contributions.

    ``do_slice`` is dO for the rank's rows (B, Hq, S/cp, D) in slice order.  dK and dV are
    returned in full-sequence order (B, Hkv, S, D); summing them over all ranks gives the
    full-sequence dK and dV.
    """
    S = q.shape[2]
    pos = rank_positions(S, cp, layout, rank)
    return attention_rows_bwd(np.asarray(q)[:, :, pos], k, v, do_slice, pos, np.arange(S), scale,
                              window, attn_chunk)


def ring_order(seq_len: int, cp: int, layout: str) -> np.ndarray:
    """Global positions in owner-major ring order: owner 0's slice, then owner 1's, ..."""
    return np.concatenate([rank_positions(seq_len, cp, layout, r) for r in range(cp)])


# ----------------------------------------------------------------------------- online state


def state_empty(lead_shape, d: int):
    """Empty online-softmax state: U = 0, m = -inf, l = 0."""
    return (np.zeros(tuple(lead_shape) + (d,)), np.full(tuple(lead_shape), -np.inf),
            np.zeros(tuple(lead_shape)))


def _rescale(m_old, m_new):
    """exp(m_old - m_new), taken as 0 when the old state is empty (m_old = -inf)."""
    with np.errstate(invalid="ignore"):
        return np.where(np.isfinite(m_old), np.exp(m_old - np.where(np.isfinite(m_new), m_new, 0.0)), 0.0)


def fold_block(state, s, v_blk):
    """Fold one K/V block into a row state, FlashAttention-2 style.

    ``s``: (..., T, Nk) scaled scores with -inf where masked; ``v_blk``: (..., Nk, D).
      m' = max(m, rowmax s);  P = exp(s - m');  l' = exp(m - m') l + rowsum P;
      U' = exp(m - m') U + P V.
    """
    U, m, l = state
    m_new = np.maximum(m, s.max(axis=-1))
    alpha = _rescale(m, m_new)
    base = np.where(np.isfinite(m_new), m_new, 0.0)
    p = np.where(np.isfinite(s), np.exp(s - base[..., None]), 0.0)
    return (alpha[..., None] * U + p @ v_blk, m_new, alpha * l + p.sum(axis=-1))


def merge_partial(state, o_part, lse_part):
    """Fold a normalised partial result (O_p, LSE_p) into a row state.

    The partial is the state (U = O_p, m = LSE_p, l = 1); an empty partial has LSE_p = -inf.
    """
    U, m, l = state
    m_new = np.maximum(m, lse_part)
    a = _rescale(m, m_new)
    b = _rescale(lse_part, m_new)
    return (a[..., None] * U + b[..., None] * o_part, m_new, a * l + b)


def finalize(state):
    """O = U / l and LSE = m + ln l; empty rows give O = 0, LSE = -inf."""
    U, m, l = state
    with np.errstate(divide="ignore", invalid="ignore"):
        o = np.where((l > 0)[..., None], U / l[..., None], 0.0)
        lse = np.where(l > 0, m + np.log(l), -np.inf)
    return o, lse
