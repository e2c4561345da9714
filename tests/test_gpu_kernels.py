"""GPU parity of the individual C-ABI entry points against the FP64 oracle (and exact numpy
definitions for the byte-moving kernels).  Sizes span several tiles and end in ragged tails."""
import itertools
import math

import numpy as np
import pytest
import torch

from context_blockwise_causal_amd import _lib as L
from context_blockwise_causal_amd import api
from context_blockwise_causal_amd.inputs import bf16_bits_from_f32, draw_like
from oracle import attn64 as O
from tests.gpu_util import assert_close, bits, round_like, to_dev, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ctx():
    c = api.Context(0)
    yield c
    c.close()


def rand_store(shape, dtype, seed):
    return draw_like(shape, dtype, seed)


# ----------------------------------------------------------------------------- layout


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("layout", ["contiguous", "zigzag"])
@pytest.mark.parametrize("cp", [1, 2, 4, 8])
def test_layout_gather_scatter_bit_exact(ctx, dtype, layout, cp):
    B, H, D = 2, 3, 64
    S = 2 * cp * 40
    prob = api.Problem(B, S, H, H, D, cp, layout, dtype)
    x = to_dev(rand_store((B, H, S, D), dtype, 7 + cp), dtype)
    ring = api.ra_layout_gather(ctx, prob, 0, cp, x)
    torch.cuda.synchronize()
    order = O.ring_order(S, cp, layout)
    assert np.array_equal(bits(ring), bits(x[:, :, torch.from_numpy(order).cuda()]))
    for r in range(cp):
        sl = api.ra_layout_gather(ctx, prob, r, 1, x)
        pos = torch.from_numpy(O.rank_positions(S, cp, layout, r)).cuda()
        assert np.array_equal(bits(sl), bits(x[:, :, pos]))
    back = torch.zeros_like(x)
    api.ra_layout_scatter(ctx, prob, 0, cp, ring, back)
    torch.cuda.synchronize()
    assert np.array_equal(bits(back), bits(x))
    if cp > 1:  # scattering one rank writes only that rank's rows
        part = torch.zeros_like(x)
        api.ra_layout_scatter(ctx, prob, 1, 1, api.ra_layout_gather(ctx, prob, 1, 1, x), part)
        torch.cuda.synchronize()
        pos = O.rank_positions(S, cp, layout, 1)
        mask = np.zeros(S, bool)
        mask[pos] = True
        assert np.array_equal(bits(part[:, :, torch.from_numpy(mask).cuda()]), bits(x[:, :, torch.from_numpy(mask).cuda()]))
        assert torch.count_nonzero(part[:, :, torch.from_numpy(~mask).cuda()].float()) == 0


# ----------------------------------------------------------------------------- state helpers


def test_state_init_and_finalize(ctx):
    prob = api.Problem(2, 64, 4, 2, 128, 1, "contiguous", "bf16")
    U, m, l = api.new_state(prob, 50)
    api.ra_state_init(ctx, prob, U, m, l)
    torch.cuda.synchronize()
    assert torch.all(U == 0) and torch.all(l == 0) and torch.all(torch.isneginf(m))
    rng = np.random.default_rng(3)
    Un = rng.standard_normal(U.shape)
    mn = rng.standard_normal(m.shape)
    ln = rng.uniform(0.5, 9.0, l.shape)
    ln[0, 1, :7] = 0.0
    mn[0, 1, :7] = -np.inf
    Un[0, 1, :7] = 0.0
    for dtype in ("bf16", "f32"):
        p2 = api.Problem(2, 64, 4, 2, 128, 1, "contiguous", dtype)
        Ud = torch.tensor(Un, dtype=torch.float32, device="cuda")
        md = torch.tensor(mn, dtype=torch.float32, device="cuda")
        ld = torch.tensor(ln, dtype=torch.float32, device="cuda")
        o, lse = api.ra_fwd_finalize(ctx, p2, Ud, md, ld)
        torch.cuda.synchronize()
        ro, rl = O.finalize((to_f64(Ud), to_f64(md), to_f64(ld)))
        assert_close(to_f64(o), ro, dtype, "O")
        fin = np.isfinite(rl)
        assert np.array_equal(np.isfinite(to_f64(lse)), fin)
        assert np.max(np.abs(to_f64(lse)[fin] - rl[fin])) < 1e-5


def test_lse_merge_matches_oracle(ctx):
    prob = api.Problem(1, 96, 4, 4, 64, 1, "contiguous", "bf16")
    rows = 96
    rng = np.random.default_rng(11)
    U = rng.standard_normal((1, 4, rows, 64))
    m = rng.standard_normal((1, 4, rows)) * 3
    l = rng.uniform(0.1, 5, (1, 4, rows))
    op = rng.standard_normal((1, 4, rows, 64))
    lp = rng.standard_normal((1, 4, rows)) * 3
    # empty state rows, empty partial rows, and rows where both are empty
    U[0, 0, :10], m[0, 0, :10], l[0, 0, :10] = 0, -np.inf, 0
    lp[0, 0, 5:15] = -np.inf
    op[0, 0, 5:15] = 0
    dev = lambda a: torch.tensor(a, dtype=torch.float32, device="cuda")
    Ud, md, ld = dev(U), dev(m), dev(l)
    api.ra_lse_merge(ctx, prob, dev(op), dev(lp), Ud, md, ld)
    torch.cuda.synchronize()
    f32 = lambda a: np.asarray(a, np.float32).astype(np.float64)
    rU, rm, rl = O.merge_partial((f32(U), f32(m), f32(l)), f32(op), f32(lp))
    gm = to_f64(md)
    assert np.array_equal(np.isneginf(gm), np.isneginf(rm))
    fin = np.isfinite(rm)
    assert np.max(np.abs(gm[fin] - rm[fin])) < 1e-6
    assert np.max(np.abs(to_f64(ld) - rl) / np.maximum(1, rl)) < 1e-5
    assert np.max(np.abs(to_f64(Ud) - rU)) < 1e-5


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_preprocess_and_cast(ctx, dtype, D):
    prob = api.Problem(2, 80, 3, 3, D, 1, "contiguous", dtype)
    o = to_dev(rand_store((2, 3, 80, D), dtype, 21), dtype)
    do = to_dev(rand_store((2, 3, 80, D), dtype, 22), dtype)
    delta = api.ra_bwd_preprocess(ctx, prob, o, do)
    torch.cuda.synchronize()
    ref = np.sum(to_f64(o) * to_f64(do), axis=-1)
    assert np.max(np.abs(to_f64(delta) - ref)) < 1e-4
    src = torch.randn(2, 3, 80, D, device="cuda") * 5
    out = api.ra_cast_from_f32(ctx, prob, src)
    torch.cuda.synchronize()
    if dtype == "bf16":
        expect = bf16_bits_from_f32(src.cpu().numpy())
        assert np.array_equal(out.view(torch.int16).cpu().numpy().view(np.uint16), expect)
    else:
        assert torch.equal(out, src)


# ----------------------------------------------------------------------------- chunk forward


def run_pairs_fwd(ctx, prob, q, k, v, pairs, state=None):
    B, Hq, qr, D = q.shape
    if state is None:
        state = api.new_state(prob, qr)
        api.ra_state_init(ctx, prob, *state)
    api.ra_chunk_fwd(ctx, prob, q, k, v, pairs, *state)
    return state


CASES = [  # (D, Hq, Hkv, dtype)
    (128, 4, 2, "bf16"), (64, 3, 3, "bf16"), (128, 2, 1, "f32"), (64, 2, 2, "f32"),
]


@pytest.mark.parametrize("D,Hq,Hkv,dtype", CASES)
@pytest.mark.parametrize("kind", ["FULL", "DIAG"])
def test_chunk_fwd_single_pair(ctx, D, Hq, Hkv, dtype, kind):
    B = 2
    qlen = 261 if kind == "DIAG" else 200
    kvlen = 261 if kind == "DIAG" else 333
    q_rows, kv_rows, q0, k0 = qlen + 50, kvlen + 31, 20, 17
    prob = api.Problem(B, 2 * q_rows, Hq, Hkv, D, 1, "contiguous", dtype)
    qs = rand_store((B, Hq, q_rows, D), dtype, 31)
    ks = rand_store((B, Hkv, kv_rows, D), dtype, 32)
    vs = rand_store((B, Hkv, kv_rows, D), dtype, 33)
    q, k, v = to_dev(qs, dtype), to_dev(ks, dtype), to_dev(vs, dtype)
    mask = {"FULL": L.RA_MASK_FULL, "DIAG": L.RA_MASK_DIAG}[kind]
    U, m, l = api.new_state(prob, q_rows)
    api.ra_state_init(ctx, prob, U, m, l)
    # rows outside the pair carry arbitrary state that must come back bit-unchanged
    U[:, :, :q0] = 1.5
    m[:, :, :q0] = 0.25
    l[:, :, :q0] = 3.0
    before = [bits(t[:, :, :q0]) for t in (U, m, l)] + [bits(t[:, :, q0 + qlen:]) for t in (U, m, l)]
    api.ra_chunk_fwd(ctx, prob, q, k, v, [(q0, k0, qlen, kvlen, mask)], U, m, l)
    o, lse = api.ra_fwd_finalize(ctx, prob, U, m, l)
    torch.cuda.synchronize()
    after = [bits(t[:, :, :q0]) for t in (U, m, l)] + [bits(t[:, :, q0 + qlen:]) for t in (U, m, l)]
    for a, b in zip(before, after):
        assert np.array_equal(a, b)
    qp, kp = O.pair_positions(O.FULL if kind == "FULL" else O.DIAG, qlen, kvlen)
    ro, rl = O.attention_rows(to_f64(q)[:, :, q0:q0 + qlen], to_f64(k)[:, :, k0:k0 + kvlen],
                              to_f64(v)[:, :, k0:k0 + kvlen], qp, kp)
    assert_close(to_f64(o)[:, :, q0:q0 + qlen], ro, dtype, "O")
    assert np.max(np.abs(to_f64(lse)[:, :, q0:q0 + qlen] - rl)) < (1e-5 if dtype == "f32" else 2e-3)


@pytest.mark.parametrize("D,Hq,Hkv,dtype", CASES)
def test_chunk_fwd_skip_and_empty_leave_state(ctx, D, Hq, Hkv, dtype):
    prob = api.Problem(1, 256, Hq, Hkv, D, 1, "contiguous", dtype)
    q = to_dev(rand_store((1, Hq, 128, D), dtype, 41), dtype)
    k = to_dev(rand_store((1, Hkv, 128, D), dtype, 42), dtype)
    U, m, l = api.new_state(prob, 128)
    U.normal_()
    m.normal_()
    l.uniform_(1, 2)
    before = [bits(t) for t in (U, m, l)]
    api.ra_chunk_fwd(ctx, prob, q, k, k, [(0, 0, 128, 128, L.RA_MASK_SKIP), (0, 0, 0, 5, L.RA_MASK_FULL)],
                     U, m, l)
    torch.cuda.synchronize()
    assert all(np.array_equal(b, bits(t)) for b, t in zip(before, (U, m, l)))


@pytest.mark.parametrize("D,Hq,Hkv,dtype", CASES)
@pytest.mark.parametrize("L_", [150, 256])
def test_chunk_fwd_zigzag_local_step_and_second_chunk(ctx, D, Hq, Hkv, dtype, L_):
    """The step-0 pattern (pairs sharing Q rows) then a FULL step from a second K/V chunk."""
    B = 1
    prob = api.Problem(B, 4 * L_, Hq, Hkv, D, 1, "contiguous", dtype)
    q = to_dev(rand_store((B, Hq, 2 * L_, D), dtype, 51), dtype)
    k = to_dev(rand_store((B, Hkv, 2 * L_, D), dtype, 52), dtype)
    v = to_dev(rand_store((B, Hkv, 2 * L_, D), dtype, 53), dtype)
    k2 = to_dev(rand_store((B, Hkv, L_, D), dtype, 54), dtype)
    v2 = to_dev(rand_store((B, Hkv, L_, D), dtype, 55), dtype)
    pairs0 = [(0, 0, L_, L_, L.RA_MASK_DIAG), (0, L_, L_, L_, L.RA_MASK_SKIP),
              (L_, 0, L_, L_, L.RA_MASK_FULL), (L_, L_, L_, L_, L.RA_MASK_DIAG)]
    st = run_pairs_fwd(ctx, prob, q, k, v, pairs0)
    o, lse = api.ra_fwd_finalize(ctx, prob, *st)
    torch.cuda.synchronize()
    pos = np.arange(2 * L_)
    ro, rl = O.attention_rows(to_f64(q), to_f64(k), to_f64(v), pos, pos)
    assert_close(to_f64(o), ro, dtype, "O step 0")
    # a second chunk lying wholly before both Q halves: keys at positions -L..-1
    api.ra_chunk_fwd(ctx, prob, q, k2, v2, [(0, 0, L_, L_, L.RA_MASK_FULL), (L_, 0, L_, L_, L.RA_MASK_FULL)], *st)
    o, lse = api.ra_fwd_finalize(ctx, prob, *st)
    torch.cuda.synchronize()
    kk = np.concatenate([to_f64(k2), to_f64(k)], axis=2)
    vv = np.concatenate([to_f64(v2), to_f64(v)], axis=2)
    kpos = np.arange(-L_, 2 * L_)
    ro, rl = O.attention_rows(to_f64(q), kk, vv, pos, kpos)
    assert_close(to_f64(o), ro, dtype, "O two chunks")
    assert np.max(np.abs(to_f64(lse) - rl)) < (1e-5 if dtype == "f32" else 2e-3)


# ----------------------------------------------------------------------------- chunk backward


def oracle_stats(q64, k64, v64, do64, qp, kp):
    o, lse = O.attention_rows(q64, k64, v64, qp, kp)
    return o, lse, np.sum(do64 * o, axis=-1)


def chunk_bwd(entry, ctx, prob, q, do, lse, delta, k, v, pairs, dq, dk, dv):
    """The chunk backward through one of its two entry points: "recompute" (ra_chunk_bwd: the dQ
    kernel recomputes S and dP) or "stored" (ra_chunk_bwd_ds: dQ from the dS the dK/dV kernel
    stored).  The stored path's scratch starts filled with NaN bit patterns, so that an entry
    the dQ pass reads without the dK/dV kernel having written it shows up as non-finite."""
    if entry == "recompute":
        return api.ra_chunk_bwd(ctx, prob, q, do, lse, delta, k, v, pairs, dq, dk, dv)
    n = api.ra_chunk_bwd_ds_size(prob, q.shape[2], k.shape[2], pairs)
    scratch = torch.full((max(16, n),), 0xFF, dtype=torch.uint8, device="cuda")
    api.ra_chunk_bwd_ds(ctx, prob, q, do, lse, delta, k, v, pairs, dq, dk, dv, scratch)
    return scratch


@pytest.mark.parametrize("entry", ["recompute", "stored"])
@pytest.mark.parametrize("D,Hq,Hkv,dtype", CASES)
@pytest.mark.parametrize("kind", ["FULL", "DIAG"])
def test_chunk_bwd_single_pair(ctx, D, Hq, Hkv, dtype, kind, entry):
    B = 1 if dtype == "f32" else 2
    qlen = 200 if kind == "DIAG" else 190
    kvlen = 200 if kind == "DIAG" else 300
    if dtype == "f32":
        qlen, kvlen = (qlen // 2, qlen // 2) if kind == "DIAG" else (80, 100)
    prob = api.Problem(B, 2 * max(qlen, kvlen), Hq, Hkv, D, 1, "contiguous", dtype)
    q = to_dev(rand_store((B, Hq, qlen, D), dtype, 61), dtype)
    k = to_dev(rand_store((B, Hkv, kvlen, D), dtype, 62), dtype)
    v = to_dev(rand_store((B, Hkv, kvlen, D), dtype, 63), dtype)
    do = to_dev(rand_store((B, Hq, qlen, D), dtype, 64), dtype)
    qp, kp = O.pair_positions(O.FULL if kind == "FULL" else O.DIAG, qlen, kvlen)
    q64, k64, v64, do64 = (to_f64(t) for t in (q, k, v, do))
    o, lse, delta = oracle_stats(q64, k64, v64, do64, qp, kp)
    lse_d = torch.tensor(lse, dtype=torch.float32, device="cuda")
    dl_d = torch.tensor(delta, dtype=torch.float32, device="cuda")
    dq = torch.zeros(B, Hq, qlen, D, device="cuda")
    dk = torch.zeros(B, Hkv, kvlen, D, device="cuda")
    dv = torch.zeros_like(dk)
    mask = {"FULL": L.RA_MASK_FULL, "DIAG": L.RA_MASK_DIAG}[kind]
    chunk_bwd(entry, ctx, prob, q, do, lse_d, dl_d, k, v, [(0, 0, qlen, kvlen, mask)], dq, dk, dv)
    torch.cuda.synchronize()
    rdq, rdk, rdv = O.attention_rows_bwd(q64, k64, v64, do64, qp, kp)
    for got, ref, name in ((dq, rdq, "dQ"), (dk, rdk, "dK"), (dv, rdv, "dV")):
        assert_close(to_f64(got), ref, dtype, name)


@pytest.mark.parametrize("Hkv", [32, 16])
@pytest.mark.parametrize("kind", ["FULL", "DIAG"])
def test_chunk_bwd_two_query_heads_per_workgroup(ctx, kind, Hkv):
    """With more than 256 dK/dV workgroups and an even number of query heads per key/value head,
    each D = 128 workgroup takes two query heads of its group in turn (one K/V prologue, one
    set of dK/dV atomics): 64 query heads, groups of 2 and 4, 5 key tiles of 256 (the last ragged),
    both entries, every element against the oracle."""
    B, Hq, D, dtype = 1, 64, 128, "bf16"
    kvlen = 1100
    qlen = 100 if kind == "FULL" else kvlen
    mask = {"FULL": L.RA_MASK_FULL, "DIAG": L.RA_MASK_DIAG}[kind]
    prob = api.Problem(B, 2 * kvlen, Hq, Hkv, D, 1, "contiguous", dtype)
    q = to_dev(rand_store((B, Hq, qlen, D), dtype, 121), dtype)
    k = to_dev(rand_store((B, Hkv, kvlen, D), dtype, 122), dtype)
    v = to_dev(rand_store((B, Hkv, kvlen, D), dtype, 123), dtype)
    do = to_dev(rand_store((B, Hq, qlen, D), dtype, 124), dtype)
    qp, kp = O.pair_positions(O.FULL if kind == "FULL" else O.DIAG, qlen, kvlen)
    q64, k64, v64, do64 = (to_f64(t) for t in (q, k, v, do))
    _, lse, delta = oracle_stats(q64, k64, v64, do64, qp, kp)
    lse_d = torch.tensor(lse, dtype=torch.float32, device="cuda")
    dl_d = torch.tensor(delta, dtype=torch.float32, device="cuda")
    rdq, rdk, rdv = O.attention_rows_bwd(q64, k64, v64, do64, qp, kp)
    for entry in ("recompute", "stored"):
        dq = torch.zeros(B, Hq, qlen, D, device="cuda")
        dk = torch.zeros(B, Hkv, kvlen, D, device="cuda")
        dv = torch.zeros_like(dk)
        chunk_bwd(entry, ctx, prob, q, do, lse_d, dl_d, k, v, [(0, 0, qlen, kvlen, mask)], dq, dk, dv)
        torch.cuda.synchronize()
        for got, ref, name in ((dq, rdq, "dQ"), (dk, rdk, "dK"), (dv, rdv, "dV")):
            assert_close(to_f64(got), ref, dtype, f"{name} ({entry})")


@pytest.mark.parametrize("kind,window,D", [("FULL", 0, 128), ("DIAG", 0, 128), ("DIAG", 150, 128),
                                           ("FULL", 0, 64), ("DIAG", 0, 64)])
def test_chunk_bwd_dq_two_query_blocks_per_wavefront(ctx, kind, window, D):
    """With at least 1024 dQ workgroups at 256 query rows each, the dQ kernel of the stored-dS
    entry takes two 32-query blocks per wavefront (tiles of 32 keys x 256 queries, each K^T operand
    feeding two MFMAs): 2 x 256 query heads over 500 query rows (two tiles per head, the second
    ragged), a FULL pair with 300 keys and a DIAG pair, also with a sliding window, every element
    of dQ, dK and dV against the oracle."""
    B, Hq, dtype = 2, 256, "bf16"
    Hkv = Hq // 2 if D == 128 else Hq
    qlen = 500
    kvlen = 300 if kind == "FULL" else qlen
    mask = {"FULL": L.RA_MASK_FULL, "DIAG": L.RA_MASK_DIAG}[kind]
    prob = api.Problem(B, 2 * qlen, Hq, Hkv, D, 1, "contiguous", dtype, 0.0, window, 0)
    q = to_dev(rand_store((B, Hq, qlen, D), dtype, 131), dtype)
    k = to_dev(rand_store((B, Hkv, kvlen, D), dtype, 132), dtype)
    v = to_dev(rand_store((B, Hkv, kvlen, D), dtype, 133), dtype)
    do = to_dev(rand_store((B, Hq, qlen, D), dtype, 134), dtype)
    qp, kp = O.pair_positions(O.FULL if kind == "FULL" else O.DIAG, qlen, kvlen)
    q64, k64, v64, do64 = (to_f64(t) for t in (q, k, v, do))
    o, lse = O.attention_rows(q64, k64, v64, qp, kp, window=window)
    delta = np.sum(do64 * o, axis=-1)
    lse_d = torch.tensor(lse, dtype=torch.float32, device="cuda")
    dl_d = torch.tensor(delta, dtype=torch.float32, device="cuda")
    rdq, rdk, rdv = O.attention_rows_bwd(q64, k64, v64, do64, qp, kp, window=window)
    dq = torch.zeros(B, Hq, qlen, D, device="cuda")
    dk = torch.zeros(B, Hkv, kvlen, D, device="cuda")
    dv = torch.zeros_like(dk)
    chunk_bwd("stored", ctx, prob, q, do, lse_d, dl_d, k, v,
              [(0, 0, qlen, kvlen, mask, int(qp[0]), int(kp[0]))], dq, dk, dv)
    torch.cuda.synchronize()
    for got, ref, name in ((dq, rdq, "dQ"), (dk, rdk, "dK"), (dv, rdv, "dV")):
        assert_close(to_f64(got), ref, dtype, name)


@pytest.mark.parametrize("kind", ["FULL", "DIAG"])
@pytest.mark.parametrize("n", [1, 2, 3])
def test_short_loops_of_the_d128_kernels(ctx, n, kind):
    """The D = 128 bf16 kernels run their main loops in ping-pong form, whose prologue and tail
    differ for one, two and three iterations (tiles of 64 keys in the forward, steps of 32 query
    rows in the dK/dV kernel): pairs of those lengths, ragged, forward and both backward entries."""
    B, Hq, Hkv, D, dtype = 1, 4, 2, 128, "bf16"
    kvlen = 64 * (n - 1) + 23  # forward: n key tiles
    qlen = 32 * (n - 1) + 11   # backward: n query steps
    if kind == "DIAG":  # one length: 1, 2, 3 key tiles and 1, 3, 5 query steps
        kvlen = qlen = {1: 11, 2: 75, 3: 150}[n]
    mask = {"FULL": L.RA_MASK_FULL, "DIAG": L.RA_MASK_DIAG}[kind]
    qp, kp = O.pair_positions(O.FULL if kind == "FULL" else O.DIAG, qlen, kvlen)
    prob = api.Problem(B, 2 * max(qlen, kvlen), Hq, Hkv, D, 1, "contiguous", dtype)
    q = to_dev(rand_store((B, Hq, qlen, D), dtype, 81 + n), dtype)
    k = to_dev(rand_store((B, Hkv, kvlen, D), dtype, 91 + n), dtype)
    v = to_dev(rand_store((B, Hkv, kvlen, D), dtype, 101 + n), dtype)
    do = to_dev(rand_store((B, Hq, qlen, D), dtype, 111 + n), dtype)
    q64, k64, v64, do64 = (to_f64(t) for t in (q, k, v, do))
    U, m, l = run_pairs_fwd(ctx, prob, q, k, v, [(0, 0, qlen, kvlen, mask)])
    o, lse = api.ra_fwd_finalize(ctx, prob, U, m, l)
    torch.cuda.synchronize()
    ro, rl, rdelta = oracle_stats(q64, k64, v64, do64, qp, kp)
    assert_close(to_f64(o), ro, dtype, f"O ({n} tiles)")
    assert np.max(np.abs(to_f64(lse) - rl)) < 2e-3
    lse_d = torch.tensor(rl, dtype=torch.float32, device="cuda")
    dl_d = torch.tensor(rdelta, dtype=torch.float32, device="cuda")
    rdq, rdk, rdv = O.attention_rows_bwd(q64, k64, v64, do64, qp, kp)
    for entry in ("recompute", "stored"):
        dq = torch.zeros(B, Hq, qlen, D, device="cuda")
        dk = torch.zeros(B, Hkv, kvlen, D, device="cuda")
        dv = torch.zeros_like(dk)
        chunk_bwd(entry, ctx, prob, q, do, lse_d, dl_d, k, v, [(0, 0, qlen, kvlen, mask)], dq, dk, dv)
        torch.cuda.synchronize()
        for got, ref, name in ((dq, rdq, "dQ"), (dk, rdk, "dK"), (dv, rdv, "dV")):
            assert_close(to_f64(got), ref, dtype, f"{name} ({entry}, {n} steps)")


@pytest.mark.parametrize("entry", ["recompute", "stored"])
@pytest.mark.parametrize("D,Hq,Hkv,dtype", CASES[:2])
def test_chunk_bwd_zigzag_local_step_accumulates(ctx, D, Hq, Hkv, dtype, entry):
    """Step-0 pairs share K/V rows; accumulators are added to, not overwritten."""
    B, L_ = 1, 200
    prob = api.Problem(B, 4 * L_, Hq, Hkv, D, 1, "contiguous", dtype)
    q = to_dev(rand_store((B, Hq, 2 * L_, D), dtype, 71), dtype)
    k = to_dev(rand_store((B, Hkv, 2 * L_, D), dtype, 72), dtype)
    v = to_dev(rand_store((B, Hkv, 2 * L_, D), dtype, 73), dtype)
    do = to_dev(rand_store((B, Hq, 2 * L_, D), dtype, 74), dtype)
    pos = np.arange(2 * L_)
    q64, k64, v64, do64 = (to_f64(t) for t in (q, k, v, do))
    o, lse, delta = oracle_stats(q64, k64, v64, do64, pos, pos)
    pairs0 = [(0, 0, L_, L_, L.RA_MASK_DIAG), (0, L_, L_, L_, L.RA_MASK_SKIP),
              (L_, 0, L_, L_, L.RA_MASK_FULL), (L_, L_, L_, L_, L.RA_MASK_DIAG)]
    rng = np.random.default_rng(75)
    base = [rng.standard_normal(s) for s in ((B, Hq, 2 * L_, D), (B, Hkv, 2 * L_, D), (B, Hkv, 2 * L_, D))]
    dq, dk, dv = (torch.tensor(b, dtype=torch.float32, device="cuda") for b in base)
    chunk_bwd(entry, ctx, prob, q, do, torch.tensor(lse, dtype=torch.float32, device="cuda"),
              torch.tensor(delta, dtype=torch.float32, device="cuda"), k, v, pairs0, dq, dk, dv)
    torch.cuda.synchronize()
    rdq, rdk, rdv = O.attention_rows_bwd(q64, k64, v64, do64, pos, pos)
    f32 = lambda a: np.asarray(a, np.float32).astype(np.float64)
    for got, b, ref, name in ((dq, base[0], rdq, "dQ"), (dk, base[1], rdk, "dK"), (dv, base[2], rdv, "dV")):
        assert_close(to_f64(got) - f32(b), ref, dtype, name)


@pytest.mark.parametrize("D,Hq,Hkv,dtype", CASES)
def test_chunk_bwd_partial_gradients(ctx, D, Hq, Hkv, dtype):
    """dq_acc = NULL gives dK, dV only; dk_acc = dv_acc = NULL gives dQ only; each matches the
    oracle and leaves the gradient it was not asked for alone."""
    B, qlen, kvlen = 1, (96 if dtype == "f32" else 190), (96 if dtype == "f32" else 260)
    prob = api.Problem(B, 2 * max(qlen, kvlen), Hq, Hkv, D, 1, "contiguous", dtype)
    q = to_dev(rand_store((B, Hq, qlen, D), dtype, 81), dtype)
    k = to_dev(rand_store((B, Hkv, kvlen, D), dtype, 82), dtype)
    v = to_dev(rand_store((B, Hkv, kvlen, D), dtype, 83), dtype)
    do = to_dev(rand_store((B, Hq, qlen, D), dtype, 84), dtype)
    qp, kp = O.pair_positions(O.FULL, qlen, kvlen)
    q64, k64, v64, do64 = (to_f64(t) for t in (q, k, v, do))
    o, lse, delta = oracle_stats(q64, k64, v64, do64, qp, kp)
    lse_d = torch.tensor(lse, dtype=torch.float32, device="cuda")
    dl_d = torch.tensor(delta, dtype=torch.float32, device="cuda")
    pairs = [(0, 0, qlen, kvlen, L.RA_MASK_FULL)]
    rdq, rdk, rdv = O.attention_rows_bwd(q64, k64, v64, do64, qp, kp)
    dk = torch.zeros(B, Hkv, kvlen, D, device="cuda")
    dv = torch.zeros_like(dk)
    api.ra_chunk_bwd(ctx, prob, q, do, lse_d, dl_d, k, v, pairs, None, dk, dv)
    dq = torch.zeros(B, Hq, qlen, D, device="cuda")
    api.ra_chunk_bwd(ctx, prob, q, do, lse_d, dl_d, k, v, pairs, dq, None, None)
    torch.cuda.synchronize()
    for got, ref, name in ((dq, rdq, "dQ"), (dk, rdk, "dK"), (dv, rdv, "dV")):
        assert_close(to_f64(got), ref, dtype, name)
    with pytest.raises(ValueError):
        api.ra_chunk_bwd(ctx, prob, q, do, lse_d, dl_d, k, v, pairs, dq, dk, None)
    with pytest.raises(ValueError):
        api.ra_chunk_bwd(ctx, prob, q, do, lse_d, dl_d, k, v, pairs, None, None, None)
    if dtype != "bf16":
        return
    # the stored-dS entry point as two calls: dK/dV (storing dS), then dQ from the stored dS
    dk2 = torch.zeros_like(dk)
    dv2 = torch.zeros_like(dv)
    dq2 = torch.zeros_like(dq)
    n = api.ra_chunk_bwd_ds_size(prob, qlen, kvlen, pairs)
    scratch = torch.full((n,), 0xFF, dtype=torch.uint8, device="cuda")
    api.ra_chunk_bwd_ds(ctx, prob, q, do, lse_d, dl_d, k, v, pairs, None, dk2, dv2, scratch)
    assert torch.count_nonzero(dq2) == 0
    api.ra_chunk_bwd_ds(ctx, prob, q, do, lse_d, dl_d, k, v, pairs, dq2, None, None, scratch)
    torch.cuda.synchronize()
    for got, ref, name in ((dq2, rdq, "dQ"), (dk2, rdk, "dK"), (dv2, rdv, "dV")):
        assert_close(to_f64(got), ref, dtype, name + " (stored dS, two calls)")
    with pytest.raises(ValueError):
        api.ra_chunk_bwd_ds(ctx, prob, q, do, lse_d, dl_d, k, v, pairs, dq2, dk2, None, scratch)
    with pytest.raises(ValueError):  # scratch too small: RA_ERR_WORKSPACE
        api.ra_chunk_bwd_ds(ctx, prob, q, do, lse_d, dl_d, k, v, pairs, dq2, dk2, dv2, scratch[:n - 256])


# ----------------------------------------------------------------------------- merge order


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("layout,cp", [("contiguous", 2), ("contiguous", 3), ("contiguous", 4),
                                       ("zigzag", 2), ("zigzag", 4)])
def test_lse_merge_of_chunk_partials_in_every_order(ctx, dtype, layout, cp):
    """The online merge does not depend on the order of the chunks ("上下文并行", 朴素 Ring
    Attention: the (Q, K_j, V_j) blocks may be folded in any order).  The per-owner partials
    (O_p, LSE_p) of a rank view come from the oracle (attention of the rank's rows against one
    owner's chunk, empty rows LSE = -inf); ra_lse_merge folds them into an empty state in every
    order of the owners (cp! orders), and the finalized result must match the oracle's full
    attention to the stated tolerance each time."""
    B, Hq, Hkv, D = 1, 4, 2, 64
    chunk = 48 if layout == "zigzag" else 40
    S = chunk * cp
    prob = api.Problem(B, S, Hq, Hkv, D, cp, layout, dtype)
    q64, k64, v64 = (to_f64(to_dev(rand_store(sh, dtype, 90 + i), dtype)) for i, sh in
                     enumerate(((B, Hq, S, D), (B, Hkv, S, D), (B, Hkv, S, D))))
    rank = cp - 1  # the last rank sees every owner's chunk
    pos = O.rank_positions(S, cp, layout, rank)
    ro, rl = O.attention_rows(q64[:, :, pos], k64, v64, pos, np.arange(S))
    parts = []
    for owner in range(cp):
        kp = O.rank_positions(S, cp, layout, owner)
        op, lp = O.attention_rows(q64[:, :, pos], k64[:, :, kp], v64[:, :, kp], pos, kp)
        parts.append((torch.tensor(op, dtype=torch.float32, device="cuda"),
                      torch.tensor(lp, dtype=torch.float32, device="cuda")))
    rows = len(pos)
    for order in itertools.permutations(range(cp)):
        U, m, l = api.new_state(prob, rows)
        api.ra_state_init(ctx, prob, U, m, l)
        for o_ in order:
            api.ra_lse_merge(ctx, prob, parts[o_][0], parts[o_][1], U, m, l)
        o, lse = api.ra_fwd_finalize(ctx, prob, U, m, l)
        torch.cuda.synchronize()
        assert_close(to_f64(o), ro, dtype, f"O order {order}")
        assert np.max(np.abs(to_f64(lse) - rl)) < 1e-5, order


@pytest.mark.parametrize("layout,cp", [("contiguous", 4), ("zigzag", 3)])
def test_gpu_chunk_partials_merge_in_every_order(ctx, layout, cp):
    """The same with partials the GPU computes: every ring step of a rank view folded by
    ra_chunk_fwd into its own empty state and finalized (fp32, so O_p is not rounded), then
    merged in every order of the steps."""
    B, Hq, Hkv, D, dtype = 1, 2, 1, 64, "f32"
    chunk = 40
    S = chunk * cp
    prob = api.Problem(B, S, Hq, Hkv, D, cp, layout, dtype)
    stores = [rand_store(sh, dtype, 70 + i) for i, sh in
              enumerate(((B, Hq, S, D), (B, Hkv, S, D), (B, Hkv, S, D)))]
    q, k, v = (to_dev(s_, dtype) for s_ in stores)
    q64, k64, v64 = (to_f64(x) for x in (q, k, v))
    rank = cp - 1
    q_sl = api.ra_layout_gather(ctx, prob, rank, 1, q)
    k_ring = api.ra_layout_gather(ctx, prob, 0, cp, k)
    v_ring = api.ra_layout_gather(ctx, prob, 0, cp, v)
    rows = prob.chunk
    parts = []
    for i in range(cp):
        owner, pairs = api.ra_plan_step(prob, rank, i)
        kc = k_ring[:, :, owner * rows:(owner + 1) * rows].contiguous()
        vc = v_ring[:, :, owner * rows:(owner + 1) * rows].contiguous()
        U, m, l = api.new_state(prob, rows)
        api.ra_state_init(ctx, prob, U, m, l)
        api.ra_chunk_fwd(ctx, prob, q_sl, kc, vc, pairs, U, m, l)
        parts.append(api.ra_fwd_finalize(ctx, prob, U, m, l))
    ro, rl = O.rank_view_fwd(q64, k64, v64, cp, layout, rank)
    for order in itertools.permutations(range(cp)):
        U, m, l = api.new_state(prob, rows)
        api.ra_state_init(ctx, prob, U, m, l)
        for i in order:
            api.ra_lse_merge(ctx, prob, parts[i][0], parts[i][1], U, m, l)
        o, lse = api.ra_fwd_finalize(ctx, prob, U, m, l)
        torch.cuda.synchronize()
        assert_close(to_f64(o), ro, dtype, f"O order {order}")
        assert np.max(np.abs(to_f64(lse) - rl)) < 1e-5, order


# ----------------------------------------------------------------------------- staging copy


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("layout,cp", [("contiguous", 4), ("zigzag", 3)])
def test_stage_kv_bit_exact(ctx, dtype, layout, cp):
    """ra_stage_kv copies owner o's K and V chunk (rows [o S/cp, (o+1) S/cp) of the ring
    tensors) into the destination, K then V, bit for bit."""
    B, Hq, Hkv, D = 2, 4, 2, 64
    S = 2 * cp * 36
    prob = api.Problem(B, S, Hq, Hkv, D, cp, layout, dtype)
    k = to_dev(rand_store((B, Hkv, S, D), dtype, 141), dtype)
    v = to_dev(rand_store((B, Hkv, S, D), dtype, 142), dtype)
    k_ring = api.ra_layout_gather(ctx, prob, 0, cp, k)
    v_ring = api.ra_layout_gather(ctx, prob, 0, cp, v)
    c = prob.chunk
    for owner in range(cp):
        dst = api.ra_stage_kv(ctx, prob, owner, k_ring, v_ring)
        torch.cuda.synchronize()
        assert np.array_equal(bits(dst[0]), bits(k_ring[:, :, owner * c:(owner + 1) * c]))
        assert np.array_equal(bits(dst[1]), bits(v_ring[:, :, owner * c:(owner + 1) * c]))
    with pytest.raises(ValueError):
        api.ra_stage_kv(ctx, prob, cp, k_ring, v_ring)


def test_reshard_rejects_overlapping_buffers(ctx):
    """Validation rejects src / dst ranges that overlap anywhere (not only equal pointers);
    nothing is enqueued."""
    prob = api.Problem(1, 256, 8, 8, 64, 4, "contiguous", "bf16")
    n = 1 * 8 * 64 * 64  # batch * heads * S/cp * head_dim
    buf = torch.zeros(2 * n + 64, dtype=torch.bfloat16, device="cuda")
    src = buf[:n]
    for off in (8, n - 8):
        with pytest.raises(ValueError):
            L.call("ra_ulysses_reshard", ctx.handle, __import__("ctypes").byref(prob.c()), 0, 8,
                   api._ptr(src), api._ptr(buf[off:off + n]), None)
    L.call("ra_ulysses_reshard", ctx.handle, __import__("ctypes").byref(prob.c()), 0, 8,
           api._ptr(src), api._ptr(buf[n:2 * n]), None)
    torch.cuda.synchronize()
