"""GPU parity of the a2a+p2p composition (USP): A * R simulated ranks as R ring groups of A
members.  Inside each group the Ulysses re-shard (ra_ulysses_reshard) and a simulated all-to-all
turn every member's sequence shard into the group's tokens for 1/A of the heads; the ring rank
views (ra_rank_view_fwd / _bwd) then run across the groups among members holding the same heads;
a second re-shard returns O and dQ to the sequence shards.  dK / dV: each ring rank view returns
its contribution to every owner's K/V gradient; the contributions are summed over the ring (the
return to the owner) and re-sharded back inside the owner's group.  Every rank's O, dQ, dK and dV
shard is compared with the FP64 oracle's full-sequence attention at the rank's positions."""
import numpy as np
import pytest
import torch

from context_blockwise_causal_amd import _lib as L
from context_blockwise_causal_amd import api
from context_blockwise_causal_amd.inputs import draw
from oracle import attn64 as O
from oracle import reshard as R
from tests.gpu_util import assert_close, to_dev, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ctx():
    c = api.Context(0)
    yield c
    c.close()


def exchange(send):
    """The all-to-all inside one group of simulated ranks: recv[u][j] = send[j][u]."""
    n = len(send)
    return [torch.stack([send[j][u] for j in range(n)]).contiguous() for u in range(n)]


CASES = [  # A (all-to-all), R (ring), layout, Hq, Hkv, D, dtype
    (2, 2, "contiguous", 4, 4, 64, "bf16"),
    (2, 2, "zigzag", 8, 4, 128, "bf16"),
    (2, 4, "contiguous", 8, 2, 128, "bf16"),
    (2, 4, "zigzag", 4, 4, 64, "bf16"),
    (2, 4, "zigzag", 8, 4, 64, "f32"),
]


@pytest.mark.parametrize("A,Rg,layout,Hq,Hkv,D,dtype", CASES)
def test_a2a_plus_ring_matches_oracle(ctx, A, Rg, layout, Hq, Hkv, D, dtype):
    B = 1
    P = A * Rg
    S = 2 * P * (24 if dtype == "bf16" else 8)
    n_rep = Hq // Hkv
    t = draw(B, S, Hq, Hkv, D, dtype, 700 + P)
    full = {n: to_dev(t.store[n], dtype) for n in ("q", "k", "v", "do")}
    Sg = S // Rg                      # tokens of one ring group
    # re-shard problem: one group's tokens, all-to-all degree A
    gprob = api.Problem(B, Sg, Hq, Hkv, D, A, "contiguous", dtype)
    # ring problem: the whole sequence over R ring ranks, on 1/A of the heads
    rprob = api.Problem(B, S, Hq // A, Hkv // A, D, Rg, layout, dtype)
    ring_lay = api.Problem(B, S, Hq, Hkv, D, Rg, layout, dtype)

    def to_heads(name, H):
        """Sequence shards of every rank -> per (group, member) head shards (B, H/A, Sg, D)."""
        out = {}
        for g in range(Rg):
            gslice = api.ra_layout_gather(ctx, ring_lay, g, 1, full[name])   # group's tokens, slice order
            shards = [gslice[:, :, u * (Sg // A):(u + 1) * (Sg // A)].contiguous() for u in range(A)]
            send = [api.ra_ulysses_reshard(ctx, gprob, L.RA_A2A_SEQ_PACK, H, sh) for sh in shards]
            for u, rb in enumerate(exchange(send)):
                out[(g, u)] = api.ra_ulysses_reshard(ctx, gprob, L.RA_A2A_HEAD_UNPACK, H, rb)
        return out

    def to_seq(parts, H):
        """Per (group, member) head shards -> every rank's sequence shard (B, H, Sg/A, D)."""
        out = {}
        for g in range(Rg):
            send = [api.ra_ulysses_reshard(ctx, gprob, L.RA_A2A_HEAD_PACK, H, parts[(g, u)]) for u in range(A)]
            for u, rb in enumerate(exchange(send)):
                out[(g, u)] = api.ra_ulysses_reshard(ctx, gprob, L.RA_A2A_SEQ_UNPACK, H, rb)
        return out

    qh, kh, vh, doh = to_heads("q", Hq), to_heads("k", Hkv), to_heads("v", Hkv), to_heads("do", Hq)
    o_h, dq_h, dk_sum, dv_sum = {}, {}, {}, {}
    for u in range(A):
        # the ring tensors of head shard u: owner g's rows are group g's tokens (owner-major)
        k_ring = torch.cat([kh[(g, u)] for g in range(Rg)], dim=2).contiguous()
        v_ring = torch.cat([vh[(g, u)] for g in range(Rg)], dim=2).contiguous()
        dk_sum[u] = torch.zeros(k_ring.shape, dtype=torch.float32, device="cuda")
        dv_sum[u] = torch.zeros_like(dk_sum[u])
        for g in range(Rg):
            o, lse = api.rank_view_fwd(ctx, rprob, g, qh[(g, u)], k_ring, v_ring, staging=torch.cuda.Stream())
            dq, dk, dv = api.rank_view_bwd(ctx, rprob, g, qh[(g, u)], k_ring, v_ring, o, lse, doh[(g, u)],
                                           staging=torch.cuda.Stream())
            o_h[(g, u)], dq_h[(g, u)] = o, dq
            dk_sum[u] += dk.float()   # the return of K/V gradients to their owners
            dv_sum[u] += dv.float()
    cast = (lambda x: x.to(torch.bfloat16)) if dtype == "bf16" else (lambda x: x)
    dk_h = {(g, u): cast(dk_sum[u][:, :, g * Sg:(g + 1) * Sg]).contiguous() for g in range(Rg) for u in range(A)}
    dv_h = {(g, u): cast(dv_sum[u][:, :, g * Sg:(g + 1) * Sg]).contiguous() for g in range(Rg) for u in range(A)}
    o_s, dq_s = to_seq(o_h, Hq), to_seq(dq_h, Hq)
    dk_s, dv_s = to_seq(dk_h, Hkv), to_seq(dv_h, Hkv)
    torch.cuda.synchronize()

    q64, k64, v64, do64 = (t.as_f64(n) for n in ("q", "k", "v", "do"))
    pos_all = np.arange(S)
    ro, _ = O.attention_rows(q64, k64, v64, pos_all, pos_all)
    rdq, rdk, rdv = O.attention_rows_bwd(q64, k64, v64, do64, pos_all, pos_all)
    for g in range(Rg):
        for u in range(A):
            pos = R.usp_positions(S, A, Rg, layout, g, u)
            assert_close(to_f64(o_s[(g, u)]), ro[:, :, pos], dtype, f"O rank ({g},{u})")
            assert_close(to_f64(dq_s[(g, u)]), rdq[:, :, pos], dtype, f"dQ rank ({g},{u})")
            assert_close(to_f64(dk_s[(g, u)]), rdk[:, :, pos], dtype, f"dK rank ({g},{u})")
            assert_close(to_f64(dv_s[(g, u)]), rdv[:, :, pos], dtype, f"dV rank ({g},{u})")
