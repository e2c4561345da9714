"""Pins of the Ulysses re-shard oracle against what the definition fixes: the all-to-all of
sequence shards yields each rank's head shard of the full tensor, the reverse yields the
sequence shards, the round trip is the identity, and a hand-checked tiny case."""
import numpy as np
import pytest

from oracle import attn64 as O
from oracle import reshard as R


def full_tensor(B, H, S, D, seed):
    return np.random.default_rng(seed).standard_normal((B, H, S, D))


@pytest.mark.parametrize("cp,B,H,S,D", [(2, 1, 2, 8, 4), (4, 2, 8, 16, 3), (8, 1, 32, 64, 2), (1, 1, 3, 5, 2)])
def test_seq_to_head_is_head_shard(cp, B, H, S, D):
    x = full_tensor(B, H, S, D, cp * 100 + H)
    send = [R.pack_seq(R.seq_shard(x, cp, r), cp) for r in range(cp)]
    recv = R.exchange(send)
    for r in range(cp):
        np.testing.assert_array_equal(R.unpack_to_head(recv[r]), R.head_shard(x, cp, r))


@pytest.mark.parametrize("cp,B,H,S,D", [(2, 1, 2, 8, 4), (4, 2, 8, 16, 3), (8, 1, 16, 32, 2)])
def test_head_to_seq_is_seq_shard_and_round_trip(cp, B, H, S, D):
    x = full_tensor(B, H, S, D, cp * 7 + S)
    send = [R.pack_head(R.head_shard(x, cp, r), cp) for r in range(cp)]
    recv = R.exchange(send)
    for r in range(cp):
        np.testing.assert_array_equal(R.unpack_to_seq(recv[r]), R.seq_shard(x, cp, r))
    # seq -> head -> seq
    heads = [R.unpack_to_head(b) for b in R.exchange([R.pack_seq(R.seq_shard(x, cp, r), cp) for r in range(cp)])]
    back = [R.unpack_to_seq(b) for b in R.exchange([R.pack_head(h, cp) for h in heads])]
    for r in range(cp):
        np.testing.assert_array_equal(back[r], R.seq_shard(x, cp, r))


def test_tiny_case_by_hand():
    # B=1, H=2, S=4, D=1, cp=2; value = 10*head + position
    x = np.array([[[[0], [1], [2], [3]], [[10], [11], [12], [13]]]])
    # rank 0 holds positions 0,1 of both heads; after the exchange it holds head 0, all positions
    send0 = R.pack_seq(R.seq_shard(x, 2, 0), 2)
    assert send0.shape == (2, 1, 1, 2, 1)
    assert send0[:, 0, 0, :, 0].tolist() == [[0, 1], [10, 11]]
    recv = R.exchange([send0, R.pack_seq(R.seq_shard(x, 2, 1), 2)])
    assert R.unpack_to_head(recv[0])[0, :, :, 0].tolist() == [[0, 1, 2, 3]]
    assert R.unpack_to_head(recv[1])[0, :, :, 0].tolist() == [[10, 11, 12, 13]]


def test_planted_mistake_is_caught():
    """An exchange that forgets the transpose (recv[r] = send[r]) must fail the defining pin."""
    x = full_tensor(1, 4, 8, 2, 5)
    send = [R.pack_seq(R.seq_shard(x, 2, r), 2) for r in range(2)]
    wrong = [send[r] for r in range(2)]
    assert not np.array_equal(R.unpack_to_head(wrong[0]), R.head_shard(x, 2, 0))


@pytest.mark.parametrize("layout", ["contiguous", "zigzag"])
@pytest.mark.parametrize("a2a,ring", [(1, 4), (2, 2), (2, 4), (4, 2), (3, 1)])
def test_usp_positions_partition_and_reduce(layout, a2a, ring):
    """The a2a+p2p token assignment: the A * R ranks' positions partition the sequence; each ring
    group's members together hold exactly that group's ring slice, in slice order; A = 1 is the
    ring layout itself and R = 1 the plain contiguous Ulysses split."""
    S = 2 * a2a * ring * 6
    allpos = np.concatenate([R.usp_positions(S, a2a, ring, layout, g, u)
                             for g in range(ring) for u in range(a2a)])
    assert np.array_equal(np.sort(allpos), np.arange(S))
    for g in range(ring):
        group = np.concatenate([R.usp_positions(S, a2a, ring, layout, g, u) for u in range(a2a)])
        assert np.array_equal(group, O.rank_positions(S, ring, layout, g))
    if a2a == 1:
        for g in range(ring):
            assert np.array_equal(R.usp_positions(S, 1, ring, layout, g, 0), O.rank_positions(S, ring, layout, g))
    if ring == 1:
        for u in range(a2a):
            assert np.array_equal(R.usp_positions(S, a2a, 1, layout, 0, u),
                                  np.arange(u * S // a2a, (u + 1) * S // a2a))


def test_usp_positions_zigzag_example():
    """By hand: 2 ring groups x 2 members, zigzag, 16 tokens (4 chunks of 4): group 0 holds chunks
    0 and 3 = positions 0-3, 12-15, split between its members; group 1 chunks 1 and 2."""
    want = {(0, 0): [0, 1, 2, 3], (0, 1): [12, 13, 14, 15], (1, 0): [4, 5, 6, 7], (1, 1): [8, 9, 10, 11]}
    for (g, u), w in want.items():
        assert list(R.usp_positions(16, 2, 2, "zigzag", g, u)) == w
