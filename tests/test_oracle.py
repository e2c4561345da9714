"""Pins of the FP64 oracle against things other than itself (CPU only).

Each test checks the oracle against an independent route: pure-Python brute force on tiny
inputs, torch's float64 scaled_dot_product_attention and autograd (a library routine for the
textbook definition), closed forms, finite differences, invariants, and values printed on
the pages (the zigzag assignment and exclusion table under tests/golden/).
"""
import itertools
import math
import os

import numpy as np
import pytest
import torch

from oracle import attn64 as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# ----------------------------------------------------------------------------- brute force


def brute_attention(q, k, v, q_pos, k_pos, n_rep):
    """Pure-Python loops: softmax over visible keys, one row at a time."""
    B, Hq, T, D = q.shape
    out = np.zeros_like(q)
    lse = np.zeros((B, Hq, T))
    sc = 1.0 / math.sqrt(D)
    for b in range(B):
        for h in range(Hq):
            g = h // n_rep
            for t in range(T):
                scores = []
                for j in range(k.shape[2]):
                    if k_pos[j] <= q_pos[t]:
                        scores.append((j, sc * sum(q[b, h, t, e] * k[b, g, j, e] for e in range(D))))
                mx = max(s for _, s in scores)
                w = [(j, math.exp(s - mx)) for j, s in scores]
                tot = sum(x for _, x in w)
                for e in range(D):
                    out[b, h, t, e] = sum(x * v[b, g, j, e] for j, x in w) / tot
                lse[b, h, t] = mx + math.log(tot)
    return out, lse


@pytest.mark.parametrize("hq,hkv", [(2, 2), (4, 2), (3, 1)])
def test_forward_matches_brute_force(hq, hkv):
    B, S, D = 2, 11, 5
    q, k, v = rnd((B, hq, S, D), 1), rnd((B, hkv, S, D), 2), rnd((B, hkv, S, D), 3)
    pos = np.arange(S)
    o, lse = O.attention_rows(q, k, v, pos, pos)
    ob, lb = brute_attention(q, k, v, pos, pos, hq // hkv)
    assert np.max(np.abs(o - ob)) < 1e-12
    assert np.max(np.abs(lse - lb)) < 1e-12


def test_forward_brute_force_permuted_positions():
    """Rows given in zigzag order and keys in ring order: same values per position."""
    B, H, S, D, cp = 1, 2, 16, 4, 2
    q, k, v = rnd((B, H, S, D), 4), rnd((B, H, S, D), 5), rnd((B, H, S, D), 6)
    for r in range(cp):
        qp = O.rank_positions(S, cp, "zigzag", r)
        kp = O.ring_order(S, cp, "zigzag")
        o, lse = O.attention_rows(q[:, :, qp], k[:, :, kp], v[:, :, kp], qp, kp)
        ob, lb = brute_attention(q[:, :, qp], k[:, :, kp], v[:, :, kp], qp, kp, 1)
        assert np.max(np.abs(o - ob)) < 1e-12 and np.max(np.abs(lse - lb)) < 1e-12


# ----------------------------------------------------------------------------- torch pin


def torch_reference(q, k, v, do, n_rep):
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    kr = tk.repeat_interleave(n_rep, dim=1)
    vr = tv.repeat_interleave(n_rep, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(tq, kr, vr, is_causal=True)
    o.backward(torch.tensor(do, dtype=torch.float64))
    return o.detach().numpy(), tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("hq,hkv,S,D", [(2, 2, 37, 16), (8, 2, 64, 32), (4, 1, 50, 8)])
def test_forward_and_backward_match_torch_fp64(hq, hkv, S, D):
    B = 2
    q, k, v, do = (rnd((B, hq, S, D), 10), rnd((B, hkv, S, D), 11),
                   rnd((B, hkv, S, D), 12), rnd((B, hq, S, D), 13))
    pos = np.arange(S)
    o, _ = O.attention_rows(q, k, v, pos, pos)
    dq, dk, dv = O.attention_rows_bwd(q, k, v, do, pos, pos)
    to, tdq, tdk, tdv = torch_reference(q, k, v, do, hq // hkv)
    for a, b in ((o, to), (dq, tdq), (dk, tdk), (dv, tdv)):
        assert np.max(np.abs(a - b)) < 1e-11


# ----------------------------------------------------------------------------- closed forms


def test_zero_queries_give_prefix_means():
    B, H, S, D = 1, 2, 20, 6
    q = np.zeros((B, H, S, D))
    k, v = rnd((B, H, S, D), 20), rnd((B, H, S, D), 21)
    pos = np.arange(S)
    o, lse = O.attention_rows(q, k, v, pos, pos)
    means = np.cumsum(v, axis=2) / np.arange(1, S + 1)[None, None, :, None]
    assert np.max(np.abs(o - means)) < 1e-13
    assert np.max(np.abs(lse - np.log(np.arange(1, S + 1))[None, None, :])) < 1e-13


def test_first_row_and_constant_values():
    B, H, S, D = 1, 3, 9, 4
    q, k = rnd((B, H, S, D), 22), rnd((B, H, S, D), 23)
    v = np.broadcast_to(rnd((1, 1, 1, D), 24), (B, H, S, D)).copy()
    pos = np.arange(S)
    o, lse = O.attention_rows(q, k, v, pos, pos)
    assert np.max(np.abs(o - v)) < 1e-13                       # constant V rows pass through
    v2 = rnd((B, H, S, D), 25)
    o2, lse2 = O.attention_rows(q, k, v2, pos, pos)
    assert np.max(np.abs(o2[:, :, 0] - v2[:, :, 0])) < 1e-14   # row 0 sees only key 0
    s00 = np.sum(q[:, :, 0] * k[:, :, 0], axis=-1) / math.sqrt(D)
    assert np.max(np.abs(lse2[:, :, 0] - s00)) < 1e-14


def test_rows_sum_to_one_and_shift_invariance():
    B, H, S, D = 2, 2, 40, 8
    q, k, v = rnd((B, H, S, D), 30), rnd((B, H, S, D), 31), rnd((B, H, S, D), 32)
    pos = np.arange(S)
    o, lse = O.attention_rows(q, k, v, pos, pos)
    s = np.einsum("bhtd,bhjd->bhtj", q, k) / math.sqrt(D)
    p = np.where(np.tril(np.ones((S, S), bool)), np.exp(s - lse[..., None]), 0.0)
    assert np.max(np.abs(p.sum(-1) - 1.0)) < 1e-13
    # safe-softmax shift: adding the same vector to every key moves each score of a row by
    # the same amount, so O is unchanged and LSE moves by scale * <q_t, u>.
    u = rnd((1, 1, 1, D), 33) * 3.0
    o2, lse2 = O.attention_rows(q, k + u, v, pos, pos)
    assert np.max(np.abs(o2 - o)) < 1e-12
    expect = lse + np.sum(q * u, axis=-1) / math.sqrt(D)
    assert np.max(np.abs(lse2 - expect)) < 1e-11


def test_large_scores_do_not_overflow():
    """Scores far beyond exp's range: the max-subtracted softmax stays finite (hard argmax)."""
    B, H, S, D = 1, 1, 24, 8
    q, k, v = rnd((B, H, S, D), 34) * 400.0, rnd((B, H, S, D), 35), rnd((B, H, S, D), 36)
    pos = np.arange(S)
    o, lse = O.attention_rows(q, k, v, pos, pos)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    s = np.einsum("td,jd->tj", q[0, 0], k[0, 0]) / math.sqrt(D)
    s = np.where(np.tril(np.ones((S, S), bool)), s, -np.inf)
    arg = s.argmax(-1)
    gap = np.sort(s, -1)[:, -1] - np.sort(s, -1)[:, -2]
    ok = gap > 50  # rows whose winner is separated by > 50 nats are one-hot in fp64
    assert ok.sum() > S // 2
    assert np.max(np.abs(o[0, 0][ok] - v[0, 0][arg[ok]])) < 1e-15


# ----------------------------------------------------------------------------- backward


def test_backward_finite_differences():
    B, Hq, Hkv, S, D = 1, 4, 2, 13, 4
    q, k, v, do = (rnd((B, Hq, S, D), 40), rnd((B, Hkv, S, D), 41),
                   rnd((B, Hkv, S, D), 42), rnd((B, Hq, S, D), 43))
    rows = np.array([2, 3, 5, 8, 12])      # a subset of query rows, as for one rank
    f = lambda qq, kk, vv: np.sum(do[:, :, rows] * O.attention_rows(qq[:, :, rows], kk, vv, rows, np.arange(S))[0])
    dq, dk, dv = O.attention_rows_bwd(q[:, :, rows], k, v, do[:, :, rows], rows, np.arange(S))
    eps = 1e-5
    rng = np.random.default_rng(44)
    for which, arr, grad in (("q", q, None), ("k", k, dk), ("v", v, dv)):
        for _ in range(12):
            idx = tuple(int(rng.integers(0, n)) for n in arr.shape)
            if which == "q":
                if idx[2] not in rows:
                    continue
                g = dq[idx[0], idx[1], int(np.where(rows == idx[2])[0][0]), idx[3]]
            else:
                g = grad[idx]
            plus, minus = arr.copy(), arr.copy()
            plus[idx] += eps
            minus[idx] -= eps
            args_p = {"q": (plus, k, v), "k": (q, plus, v), "v": (q, k, plus)}[which]
            args_m = {"q": (minus, k, v), "k": (q, minus, v), "v": (q, k, minus)}[which]
            fd = (f(*args_p) - f(*args_m)) / (2 * eps)
            assert abs(fd - g) <= 1e-6 * max(1.0, abs(g)), (which, idx, fd, g)


def test_backward_invariants():
    B, Hq, Hkv, S, D = 2, 6, 2, 30, 8
    q, k, v, do = (rnd((B, Hq, S, D), 50), rnd((B, Hkv, S, D), 51),
                   rnd((B, Hkv, S, D), 52), rnd((B, Hq, S, D), 53))
    pos = np.arange(S)
    dq, dk, dv = O.attention_rows_bwd(q, k, v, do, pos, pos)
    # sum_j dS_tj = 0 for every row, so the key gradients of a head sum to zero
    assert np.max(np.abs(dk.sum(axis=2))) < 1e-11
    # sum_j P_tj = 1, so the value gradients sum to the group's total dO
    grp = do.reshape(B, Hkv, Hq // Hkv, S, D).sum(axis=(2, 3))
    assert np.max(np.abs(dv.sum(axis=2) - grp)) < 1e-11
    z = O.attention_rows_bwd(q, k, v, np.zeros_like(do), pos, pos)
    assert all(np.max(np.abs(x)) == 0.0 for x in z)


def test_gqa_equals_repeated_mha():
    """Head h reads kv head h // n_rep; K/V grads sum over the (Hkv, n_rep) grouping."""
    B, Hq, Hkv, S, D = 1, 6, 2, 21, 8
    n_rep = Hq // Hkv
    q, k, v, do = (rnd((B, Hq, S, D), 60), rnd((B, Hkv, S, D), 61),
                   rnd((B, Hkv, S, D), 62), rnd((B, Hq, S, D), 63))
    pos = np.arange(S)
    kr, vr = np.repeat(k, n_rep, axis=1), np.repeat(v, n_rep, axis=1)
    o1, l1 = O.attention_rows(q, k, v, pos, pos)
    o2, l2 = O.attention_rows(q, kr, vr, pos, pos)
    assert np.max(np.abs(o1 - o2)) < 1e-14 and np.max(np.abs(l1 - l2)) < 1e-14
    g1 = O.attention_rows_bwd(q, k, v, do, pos, pos)
    g2 = O.attention_rows_bwd(q, kr, vr, do, pos, pos)
    assert np.max(np.abs(g1[0] - g2[0])) < 1e-13
    for a, b in ((g1[1], g2[1]), (g1[2], g2[2])):
        assert np.max(np.abs(a - b.reshape(B, Hkv, n_rep, S, D).sum(2))) < 1e-13


# ----------------------------------------------------------------------------- layouts and plans


def read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                rows.append(line.split())
    return rows


def test_zigzag_assignment_matches_pages():
    for r, a, b in read_golden("zigzag_cp4_assignment.txt"):
        assert O.rank_chunks(4, "zigzag", int(r)) == [int(a), int(b)]


@pytest.mark.parametrize("layout", ["contiguous", "zigzag"])
@pytest.mark.parametrize("cp", [1, 2, 4, 8, 16])
def test_positions_partition_the_sequence(layout, cp):
    S = 4 * cp * 3
    allpos = np.concatenate([O.rank_positions(S, cp, layout, r) for r in range(cp)])
    assert np.array_equal(np.sort(allpos), np.arange(S))
    assert np.array_equal(O.ring_order(S, cp, layout), allpos)
    if layout == "contiguous":
        assert np.array_equal(allpos, np.arange(S))


@pytest.mark.parametrize("cp", [2, 4, 8, 16])
def test_zigzag_plan_follows_exclusion_table(cp):
    rules = {cond: excl for cond, excl in read_golden("zigzag_step_rules.txt")}
    S = 2 * cp * 4
    for rank in range(cp):
        for i in range(cp):
            owner, pairs = O.plan_step(S, cp, "zigzag", rank, i)
            assert owner == (rank - i) % cp
            kinds = {(p[0] // 4 // 1, p[1] // 4): p[4] for p in pairs}
            kinds = {("Q_lo" if p[0] == 0 else "Q_hi", "K_lo" if p[1] == 0 else "K_hi"): p[4] for p in pairs}
            if i == 0:
                assert rules["i==0"] == "none"
                # the local step is causal attention over the rank's own [chunk r | chunk 2cp-1-r]
                assert kinds == {("Q_lo", "K_lo"): O.DIAG, ("Q_lo", "K_hi"): O.SKIP,
                                 ("Q_hi", "K_lo"): O.FULL, ("Q_hi", "K_hi"): O.DIAG}
            elif i <= rank:
                assert rules["1<=i<=rank"] == "K_hi"
                assert all((kind == O.SKIP) == (qk[1] == "K_hi") for qk, kind in kinds.items())
                assert all(kind in (O.FULL, O.SKIP) for kind in kinds.values())
            else:
                assert rules["i>rank"] == "Q_lo"
                assert all((kind == O.SKIP) == (qk[0] == "Q_lo") for qk, kind in kinds.items())
                assert all(kind in (O.FULL, O.SKIP) for kind in kinds.values())


@pytest.mark.parametrize("cp", [1, 2, 4, 8, 16])
def test_contiguous_plan_and_work_totals(cp):
    S = cp * 3
    total_full = total_diag = 0
    for rank in range(cp):
        full = diag = 0
        for i in range(cp):
            _, pairs = O.plan_step(S, cp, "contiguous", rank, i)
            (kind,) = [p[4] for p in pairs]
            expect = O.DIAG if i == 0 else (O.FULL if i <= rank else O.SKIP)
            assert kind == expect
            full += kind == O.FULL
            diag += kind == O.DIAG
        assert (full, diag) == (rank, 1)
        total_full += full
        total_diag += diag
    # all ranks together cover the causal triangle of cp x cp chunk pairs
    assert total_full == cp * (cp - 1) // 2 and total_diag == cp


@pytest.mark.parametrize("cp", [2, 4, 8, 16])
def test_zigzag_work_is_balanced(cp):
    S = 2 * cp * 2
    for rank in range(cp):
        full = diag = 0
        for i in range(cp):
            for p in O.plan_step(S, cp, "zigzag", rank, i)[1]:
                full += p[4] == O.FULL
                diag += p[4] == O.DIAG
        assert (full, diag) == (2 * cp - 1, 2)


# ----------------------------------------------------------------------------- rank views


def test_four_gpus_one_token_each():
    """The ring walk-through: 4 ranks, 1 token each; after 4 rounds each Q saw every K/V."""
    B, H, S, D, cp = 1, 1, 4, 3, 4
    q, k, v = rnd((B, H, S, D), 70), rnd((B, H, S, D), 71), rnd((B, H, S, D), 72)
    full, _ = brute_attention(q, k, v, np.arange(S), np.arange(S), 1)
    for r in range(cp):
        o_r, _ = O.rank_view_fwd(q, k, v, cp, "contiguous", r)
        assert np.max(np.abs(o_r[:, :, 0] - full[:, :, r])) < 1e-14
        # and by folding the chunks in ring order through the online state
        st = O.state_empty((B, H, 1), D)
        for i in range(cp):
            own = O.ring_owner(cp, r, i)
            s = np.einsum("bhd,bhd->bh", q[:, :, r], k[:, :, own])[..., None, None] / math.sqrt(D)
            if own > r:
                s = np.full_like(s, -np.inf)
            st = O.fold_block(st, s, v[:, :, own:own + 1])
        o_f, _ = O.finalize(st)
        assert np.max(np.abs(o_f[:, :, 0] - full[:, :, r])) < 1e-14


@pytest.mark.parametrize("layout", ["contiguous", "zigzag"])
@pytest.mark.parametrize("cp", [2, 4])
def test_rank_views_reassemble_full_attention(layout, cp):
    B, Hq, Hkv, D = 1, 4, 2, 8
    S = 2 * cp * 6
    q, k, v, do = (rnd((B, Hq, S, D), 80), rnd((B, Hkv, S, D), 81),
                   rnd((B, Hkv, S, D), 82), rnd((B, Hq, S, D), 83))
    pos = np.arange(S)
    o_full, lse_full = O.attention_rows(q, k, v, pos, pos)
    dq_full, dk_full, dv_full = O.attention_rows_bwd(q, k, v, do, pos, pos)
    dk_sum, dv_sum = np.zeros_like(k), np.zeros_like(v)
    for r in range(cp):
        p = O.rank_positions(S, cp, layout, r)
        o, lse = O.rank_view_fwd(q, k, v, cp, layout, r)
        assert np.max(np.abs(o - o_full[:, :, p])) < 1e-13
        assert np.max(np.abs(lse - lse_full[:, :, p])) < 1e-13
        dq, dk, dv = O.rank_view_bwd(q, k, v, do[:, :, p], cp, layout, r)
        assert np.max(np.abs(dq - dq_full[:, :, p])) < 1e-12
        dk_sum += dk
        dv_sum += dv
    assert np.max(np.abs(dk_sum - dk_full)) < 1e-12
    assert np.max(np.abs(dv_sum - dv_full)) < 1e-12


# ----------------------------------------------------------------------------- online merge


def _fold_chunks_in_order(q, k, v, q_pos, order, chunk):
    B, H, T, D = q.shape
    st = O.state_empty((B, H, T), D)
    for c in order:
        ks = slice(c * chunk, (c + 1) * chunk)
        s = np.einsum("bhtd,bhjd->bhtj", q, k[:, :, ks]) / math.sqrt(D)
        kp = np.arange(c * chunk, (c + 1) * chunk)
        s = np.where(kp[None, None, None, :] <= q_pos[None, None, :, None], s, -np.inf)
        st = O.fold_block(st, s, v[:, :, ks])
    return O.finalize(st)


@pytest.mark.parametrize("cp", [2, 3, 4])
def test_online_fold_is_order_independent_all_permutations(cp):
    B, H, D, c = 1, 2, 6, 5
    S = cp * c
    q, k, v = rnd((B, H, S, D), 90), rnd((B, H, S, D), 91), rnd((B, H, S, D), 92)
    pos = np.arange(S)
    o_ref, lse_ref = O.attention_rows(q, k, v, pos, pos)
    for order in itertools.permutations(range(cp)):
        o, lse = _fold_chunks_in_order(q, k, v, pos, order, c)
        assert np.max(np.abs(o - o_ref)) < 1e-12 and np.max(np.abs(lse - lse_ref)) < 1e-12


@pytest.mark.parametrize("cp", [8, 16])
def test_online_merge_of_partials_random_orders(cp):
    B, H, D, c = 1, 2, 4, 3
    S = cp * c
    q, k, v = rnd((B, H, S, D), 93), rnd((B, H, S, D), 94), rnd((B, H, S, D), 95)
    pos = np.arange(S)
    o_ref, lse_ref = O.attention_rows(q, k, v, pos, pos)
    parts = []
    for ch in range(cp):
        kp = np.arange(ch * c, (ch + 1) * c)
        parts.append(O.attention_rows(q, k[:, :, kp], v[:, :, kp], pos, kp))
    rng = np.random.default_rng(96)
    for _ in range(6):
        st = O.state_empty((B, H, S), D)
        for ch in rng.permutation(cp):
            st = O.merge_partial(st, *parts[ch])
        o, lse = O.finalize(st)
        assert np.max(np.abs(o - o_ref)) < 1e-12 and np.max(np.abs(lse - lse_ref)) < 1e-12


def test_merge_of_empty_states_stays_empty():
    st = O.state_empty((3,), 2)
    st = O.merge_partial(st, np.zeros((3, 2)), np.full(3, -np.inf))
    assert np.all(st[0] == 0) and np.all(np.isneginf(st[1])) and np.all(st[2] == 0)
    o, lse = O.finalize(st)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def _pair_positions_pinned(fn) -> bool:
    """True when ``fn(kind, q_len, kv_len)`` returns positions whose causal visibility matrix is
    exactly the pair kind it was asked for ("上下文并行", Zig-Zag Ring Attention: causal means key
    j is visible to query i iff j <= i).  The check computes the visibility matrix itself rather
    than calling ``classify``, so that a mistake shared by the two functions would still show."""
    for n, m in ((1, 1), (5, 5), (16, 16), (7, 3), (3, 9)):
        kinds = [O.FULL, O.SKIP] + ([O.DIAG] if n == m else [])
        for kind in kinds:
            qp, kp = (np.asarray(a, np.int64) for a in fn(kind, n, m))
            if qp.shape != (n,) or kp.shape != (m,):
                return False
            vis = np.array([[int(kp[j]) <= int(qp[i]) for j in range(m)] for i in range(n)])
            want = {O.FULL: np.ones((n, m), bool), O.SKIP: np.zeros((n, m), bool),
                    O.DIAG: np.tril(np.ones((n, m), bool))}[kind]
            if not np.array_equal(vis, want):
                return False
            # a 1 x 1 diagonal pair is also a full one, which classify reports first
            if O.classify(qp, kp) != (O.FULL if (kind == O.DIAG and n == 1) else kind):
                return False
    return True


def test_pair_positions_realise_each_kind():
    """pair_positions builds the position sets behind every single-pair GPU reference: each kind
    must come out with exactly that visibility (brute force over tiny pairs)."""
    assert _pair_positions_pinned(O.pair_positions)


def test_pair_positions_pin_catches_planted_offsets():
    """Planted mistakes in the positions (queries placed so the first one misses the last key for FULL, keys one
    row too early for SKIP, a diagonal shifted by one) must fail the pin."""
    def early_full(kind, n, m):
        if kind == O.FULL:
            return m - 2 + np.arange(n), np.arange(m)
        return O.pair_positions(kind, n, m)

    def early_skip(kind, n, m):
        if kind == O.SKIP:
            return np.arange(n), n - 1 + np.arange(m)
        return O.pair_positions(kind, n, m)

    def shifted_diag(kind, n, m):
        if kind == O.DIAG:
            return np.arange(n), 1 + np.arange(m)
        return O.pair_positions(kind, n, m)

    for bad in (early_full, early_skip, shifted_diag):
        assert not _pair_positions_pinned(bad), bad.__name__


@pytest.mark.parametrize("hq,hkv,window", [(4, 2, 0), (2, 2, 0), (3, 1, 5)])
def test_key_grads_equal_full_backward_on_key_subsets(hq, hkv, window):
    """key_grads (the gradient of a subset of keys from given row statistics) equals the pinned
    full backward restricted to that subset, for scattered rows and keys."""
    rng = np.random.default_rng(31)
    S, D = 40, 8
    q = rng.standard_normal((2, hq, S, D))
    k = rng.standard_normal((2, hkv, S, D))
    v = rng.standard_normal((2, hkv, S, D))
    rows = np.sort(rng.choice(S, 17, replace=False))
    do = rng.standard_normal((2, hq, len(rows), D))
    kpos = np.arange(S)
    _, rdk, rdv = O.attention_rows_bwd(q[:, :, rows], k, v, do, rows, kpos, window=window)
    o, lse = O.attention_rows(q[:, :, rows], k, v, rows, kpos, window=window)
    sel = np.sort(rng.choice(S, 11, replace=False))
    dk, dv = O.key_grads(q[:, :, rows], k[:, :, sel], v[:, :, sel], do, rows, sel, o, lse, window=window)
    assert np.max(np.abs(dk - rdk[:, :, sel])) < 1e-12
    assert np.max(np.abs(dv - rdv[:, :, sel])) < 1e-12
