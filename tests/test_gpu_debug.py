"""GPU checks of the rank views' debugging aids (ra_set_debug).  With slot poisoning and roctx
ranges on, the results are bitwise those of the production setting (no correct read of a slot
sees the NaN fill), and once the call's stream has drained the staging slots in the workspace hold
the fill word and nothing else does (the fill ran, after the slots' last readers)."""
import numpy as np
import pytest
import torch

from context_blockwise_causal_amd import _lib as L
from context_blockwise_causal_amd import api
from context_blockwise_causal_amd.inputs import draw
from tests.gpu_util import bits, to_dev

pytestmark = pytest.mark.gpu

FILL = 0x7FC07FC0  # NaN as two bf16 values and as one fp32


def staged_steps(prob, rank):
    """Ring steps after the local one that compute something (the steps the ring stages)."""
    n = 0
    for step in range(1, prob.cp):
        _, pairs = api.ra_plan_step(prob, rank, step)
        n += any(p[4] != L.RA_MASK_SKIP and p[2] > 0 and p[3] > 0 for p in pairs)
    return n


def fill_words(ws):
    return int((ws.view(torch.int32) == FILL).sum().item())


@pytest.mark.parametrize("B,C,Hq,Hkv,D,cp,layout,dtype,own_staging", [
    (1, 128, 4, 2, 128, 4, "zigzag", "bf16", True),      # both slots, refills
    (1, 64, 2, 2, 64, 2, "contiguous", "bf16", True),    # one staged step: one slot
    (1, 64, 2, 1, 64, 3, "zigzag", "f32", True),         # fp32 slots
    (1, 96, 2, 1, 128, 4, "contiguous", "bf16", False),  # staging on the compute stream
])
def test_debug_modes_keep_results_and_poison_slots(B, C, Hq, Hkv, D, cp, layout, dtype, own_staging):
    S = C * cp
    prob = api.Problem(B, S, Hq, Hkv, D, cp, layout, dtype)
    t = draw(B, S, Hq, Hkv, D, dtype, 11)
    plain, debug = api.Context(0), api.Context(0)
    debug.set_debug(L.RA_DEBUG_POISON_SLOTS | L.RA_DEBUG_ROCTX)
    esize = 2 if dtype == "bf16" else 4
    slot_words = 2 * B * Hkv * C * D * esize // 4  # K and V of one chunk
    try:
        dev = {n: to_dev(t.store[n], dtype) for n in ("q", "k", "v", "do")}
        k_ring = api.ra_layout_gather(plain, prob, 0, cp, dev["k"])
        v_ring = api.ra_layout_gather(plain, prob, 0, cp, dev["v"])
        for rank in range(cp):
            q_sl = api.ra_layout_gather(plain, prob, rank, 1, dev["q"])
            do_sl = api.ra_layout_gather(plain, prob, rank, 1, dev["do"])
            runs = []
            for ctx in (plain, debug):
                stg = torch.cuda.Stream() if own_staging else None
                wsf = torch.zeros(max(api.ra_workspace_size(prob, 0), 16), dtype=torch.uint8, device="cuda")
                wsb = torch.zeros(max(api.ra_workspace_size(prob, 1), 16), dtype=torch.uint8, device="cuda")
                o, lse = api.rank_view_fwd(ctx, prob, rank, q_sl, k_ring, v_ring, ws=wsf, staging=stg)
                dq, dk, dv = api.rank_view_bwd(ctx, prob, rank, q_sl, k_ring, v_ring, o, lse, do_sl, ws=wsb,
                                               staging=stg)
                torch.cuda.synchronize()
                runs.append(((o, lse, dq, dk, dv), wsf, wsb))
            # O, LSE and dQ are formed in a fixed order: bit for bit.  dK and dV sum the query heads
            # of a group by fp32 atomics, whose order varies from run to run: to their rounding.
            for name, a, b in zip(("O", "LSE", "dQ"), runs[0][0][:3], runs[1][0][:3]):
                assert np.array_equal(bits(a), bits(b)), f"{name} rank {rank}: debug mode changed the result"
            tol = 1e-2 if dtype == "bf16" else 1e-5
            for name, a, b in zip(("dK", "dV"), runs[0][0][3:], runs[1][0][3:]):
                a, b = a.float(), b.float()
                assert torch.isfinite(b).all(), f"{name} rank {rank}: non-finite values in debug mode"
                assert (a - b).abs().max().item() <= tol * max(a.abs().max().item(), 1e-30), name
            nslots = min(2, staged_steps(prob, rank))
            for i, name in ((1, "forward"), (2, "backward")):
                assert fill_words(runs[0][i]) == 0, f"{name} rank {rank}: fill word without the debug flag"
                assert fill_words(runs[1][i]) == nslots * slot_words, \
                    f"{name} rank {rank}: {fill_words(runs[1][i])} fill words, expected {nslots} slots"
    finally:
        plain.close()
        debug.close()
