"""Oracle of the Ulysses re-shard: the sequence-shard <-> head-shard exchange of the all-to-all.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import this module; the product never imports it and it imports
nothing from the product.  Plain numpy, any dtype (the operations are pure data movement).

What it computes (lecture note "上下文并行", section Ulysses): before attention every rank
holds a contiguous sequence shard with all heads; an all-to-all leaves every rank with all
positions of its own 1/cp of the heads; after attention a second all-to-all restores the
sequence sharding.  Written here as the definition:

* ``seq_shard(full, cp, r)``  -- positions [r S/cp, (r+1) S/cp) of every head;
* ``head_shard(full, cp, r)`` -- heads [r H/cp, (r+1) H/cp) at every position;
* the all-to-all: rank r sends block j of its send buffer to rank j, and block j of its
  receive buffer is what rank j sent to it (``exchange``);
* the pack / unpack steps on either side of it, each a slicing or concatenation.

Tensors are (B, H, S, D); send / receive buffers are (cp, B, H/cp, S/cp, D).

The a2a+p2p composition ("Feat: Context Parallel", 主要改动, the mode table: an all-to-all
layout change inside sub-groups, then ring attention; "上下文并行", section USP: all-to-all inside
a node, ring across nodes) arranges A * R ranks as R ring groups of A members.  Reading taken
where the pages leave the token assignment open: the ring layout (contiguous or zigzag over R)
gives ring group g its tokens, in slice order, and member u of the group holds the u-th of A
equal contiguous pieces of them (``usp_positions``).  The all-to-all inside a group leaves member
u with all the group's tokens for heads [u H/A, (u+1) H/A); the ring then runs across the groups
among the members that hold the same heads.
"""
from __future__ import annotations

import numpy as np

from oracle import attn64 as _attn


def seq_shard(full, cp, r):
    S = full.shape[2]
    c = S // cp
    return full[:, :, r * c:(r + 1) * c]


def head_shard(full, cp, r):
    H = full.shape[1]
    h = H // cp
    return full[:, r * h:(r + 1) * h]


def pack_seq(shard, cp):
    """Sequence shard (B, H, S/cp, D) -> send buffer: block j holds the heads of rank j."""
    h = shard.shape[1] // cp
    return np.stack([shard[:, j * h:(j + 1) * h] for j in range(cp)])


def unpack_to_head(recv):
    """Receive buffer (block j = rank j's positions of this rank's heads) -> head shard."""
    return np.concatenate([recv[j] for j in range(recv.shape[0])], axis=2)


def pack_head(shard, cp):
    """Head shard (B, H/cp, S, D) -> send buffer: block j holds the positions of rank j."""
    c = shard.shape[2] // cp
    return np.stack([shard[:, :, j * c:(j + 1) * c] for j in range(cp)])


def unpack_to_seq(recv):
    """Receive buffer (block j = rank j's heads at this rank's positions) -> sequence shard."""
    return np.concatenate([recv[j] for j in range(recv.shape[0])], axis=1)


def exchange(send):
    """The all-to-all on a list of per-rank send buffers: recv[r][j] = send[j][r]."""
    cp = len(send)
    return [np.stack([send[j][r] for j in range(cp)]) for r in range(cp)]


def usp_positions(seq_len, a2a, ring, layout, group, member):
    """Sequence positions rank (group, member) holds before the all-to-all: the member-th of
    ``a2a`` contiguous pieces of ring group ``group``'s slice (ring layout over ``ring``)."""
    pos = _attn.rank_positions(seq_len, ring, layout, group)
    n = len(pos) // a2a
    return pos[member * n:(member + 1) * n]
