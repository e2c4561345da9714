"""Pins of the oracle's sliding-window and chunked-attention masks against closed forms and
brute force: W = 1 or C = 1 leaves each query only itself (O = its own V row); W >= S and C >= S
reduce to plain causal attention; a brute-force softmax over an explicitly built mask matches;
gradients match finite differences; a planted off-by-one in the window fails."""
import numpy as np
import pytest

from oracle import attn64 as O


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def brute(q, k, v, qp, kp, scale, window, chunk):
    B, Hq, T, D = q.shape
    n_rep = Hq // k.shape[1]
    o = np.zeros_like(q)
    for b in range(B):
        for h in range(Hq):
            for i, t in enumerate(qp):
                js = [j for j, kpos in enumerate(kp) if kpos <= t and (not window or t - kpos < window)
                      and (not chunk or kpos // chunk == t // chunk)]
                s = np.array([scale * q[b, h, i] @ k[b, h // n_rep, j] for j in js])
                p = np.exp(s - s.max())
                o[b, h, i] = (p / p.sum()) @ v[b, h // n_rep, js]
    return o


@pytest.mark.parametrize("window,chunk", [(1, 0), (0, 1)])
def test_self_only(window, chunk):
    q, k, v = rand((1, 2, 12, 8), 1), rand((1, 1, 12, 8), 2), rand((1, 1, 12, 8), 3)
    pos = np.arange(12)
    o, lse = O.attention_rows(q, k, v, pos, pos, None, window, chunk)
    np.testing.assert_allclose(o, np.repeat(v, 2, axis=1), rtol=0, atol=1e-15)
    s = np.einsum("bhtd,bhtd->bht", q, np.repeat(k, 2, axis=1)) / np.sqrt(8)
    np.testing.assert_allclose(lse, s, rtol=0, atol=1e-12)


@pytest.mark.parametrize("window,chunk", [(40, 0), (0, 40), (64, 64)])
def test_wide_masks_are_causal(window, chunk):
    q, k, v = rand((1, 2, 40, 8), 4), rand((1, 2, 40, 8), 5), rand((1, 2, 40, 8), 6)
    pos = np.arange(40)
    a = O.attention_rows(q, k, v, pos, pos, None, window, chunk)
    c = O.attention_rows(q, k, v, pos, pos)
    np.testing.assert_array_equal(a[0], c[0])
    np.testing.assert_array_equal(a[1], c[1])


@pytest.mark.parametrize("window,chunk", [(5, 0), (0, 6), (7, 4), (3, 8)])
def test_brute_force(window, chunk):
    q, k, v = rand((1, 4, 20, 8), 7), rand((1, 2, 20, 8), 8), rand((1, 2, 20, 8), 9)
    qp = np.array([3, 9, 10, 19, 0, 14])
    kp = np.arange(20)
    o, _ = O.attention_rows(q[:, :, qp], k, v, qp, kp, 0.3, window, chunk)
    np.testing.assert_allclose(o, brute(q[:, :, qp], k, v, qp, kp, 0.3, window, chunk), rtol=1e-12, atol=1e-12)


def test_visibility_counts():
    vis = O.visible(np.arange(10), np.arange(10), 3, 0)
    assert vis.sum(axis=1).tolist() == [1, 2, 3, 3, 3, 3, 3, 3, 3, 3]
    vis = O.visible(np.arange(10), np.arange(10), 0, 4)
    assert vis.sum(axis=1).tolist() == [1, 2, 3, 4, 1, 2, 3, 4, 1, 2]


def test_backward_matches_finite_differences():
    q, k, v, do = rand((1, 2, 10, 4), 11), rand((1, 1, 10, 4), 12), rand((1, 1, 10, 4), 13), rand((1, 2, 10, 4), 14)
    pos = np.arange(10)
    W, C = 3, 6
    dq, dk, dv = O.attention_rows_bwd(q, k, v, do, pos, pos, None, W, C)

    def f(q_, k_, v_):
        return float(np.sum(do * O.attention_rows(q_, k_, v_, pos, pos, None, W, C)[0]))
    eps = 1e-6
    for arr, grad in ((q, dq), (k, dk), (v, dv)):
        for idx in [(0, 0, 4, 1), (0, 0, 9, 3), (0, 0, 6, 0)]:
            if idx[1] >= arr.shape[1]:
                continue
            a1, a2 = arr.copy(), arr.copy()
            a1[idx] += eps
            a2[idx] -= eps
            args1 = [a1 if x is arr else x for x in (q, k, v)]
            args2 = [a2 if x is arr else x for x in (q, k, v)]
            num = (f(*args1) - f(*args2)) / (2 * eps)
            assert abs(num - grad[idx]) < 1e-6, (idx, num, grad[idx])


def test_planted_window_off_by_one_is_caught():
    """A window rule t - j <= W (one key too many) disagrees with the brute force."""
    q, k, v = rand((1, 1, 12, 4), 15), rand((1, 1, 12, 4), 16), rand((1, 1, 12, 4), 17)
    pos = np.arange(12)
    ref = brute(q, k, v, pos, pos, 0.5, 4, 0)
    wrong = O.attention_rows(q, k, v, pos, pos, 0.5, 5, 0)[0]
    assert not np.allclose(wrong, ref, atol=1e-9)
