"""The no-allocation chunk backward (ra_chunk_bwd_ds_noalloc) against ra_chunk_bwd_ds on the same
inputs: two calls in a row on one GPU, the second smaller than the first (it reuses the static
scratch the first one filled), and the size limit of the static scratch."""
import numpy as np
import pytest
import torch

from context_blockwise_causal_amd import _lib as L
from context_blockwise_causal_amd import api
from context_blockwise_causal_amd.inputs import draw_like
from oracle import attn64 as O
from tests.gpu_util import assert_close, bits, to_dev, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ctx():
    c = api.Context(0)
    yield c
    c.close()


def case(kind, B, Hq, Hkv, D, L_, seed):
    """Inputs of one chunk backward: the zigzag local step's three half-chunk pairs ("step0") or
    one full pair with ragged lengths ("full"), with lse and delta from the FP64 oracle."""
    dtype = "bf16"
    if kind == "step0":
        qlen = kvlen = 2 * L_
        pairs = [(0, 0, L_, L_, L.RA_MASK_DIAG), (L_, 0, L_, L_, L.RA_MASK_FULL),
                 (L_, L_, L_, L_, L.RA_MASK_DIAG), (0, L_, L_, L_, L.RA_MASK_SKIP)]
        qpos = kpos = np.arange(2 * L_)
    else:
        qlen, kvlen = L_, L_ + 70
        pairs = [(0, 0, qlen, kvlen, L.RA_MASK_FULL)]
        qpos, kpos = O.pair_positions(O.FULL, qlen, kvlen)
    q = to_dev(draw_like((B, Hq, qlen, D), dtype, seed), dtype)
    k = to_dev(draw_like((B, Hkv, kvlen, D), dtype, seed + 1), dtype)
    v = to_dev(draw_like((B, Hkv, kvlen, D), dtype, seed + 2), dtype)
    do = to_dev(draw_like((B, Hq, qlen, D), dtype, seed + 3), dtype)
    q64, k64, v64, do64 = (to_f64(t) for t in (q, k, v, do))
    o, lse = O.attention_rows(q64, k64, v64, qpos, kpos)
    delta = np.sum(do64 * o, axis=-1)
    prob = api.Problem(B, 2 * max(qlen, kvlen), Hq, Hkv, D, 1, "contiguous", dtype)
    lse_d = torch.tensor(lse, dtype=torch.float32, device="cuda")
    dl_d = torch.tensor(delta, dtype=torch.float32, device="cuda")
    return prob, q, do, lse_d, dl_d, k, v, pairs


def zeros_like_grads(q, k):
    return torch.zeros(q.shape, device="cuda"), torch.zeros(k.shape, device="cuda"), \
        torch.zeros(k.shape, device="cuda")


def test_noalloc_matches_chunk_bwd_ds_on_two_calls(ctx):
    cases = [("step0", 2, 8, 2, 128, 300, 901), ("full", 1, 4, 2, 64, 190, 911)]
    sizes = []
    for kind, B, Hq, Hkv, D, L_, seed in cases:
        print(f"no-alloc case {kind} B{B} Hq{Hq} Hkv{Hkv} D{D} L{L_}", flush=True)
        prob, q, do, lse, dl, k, v, pairs = case(kind, B, Hq, Hkv, D, L_, seed)
        n = api.ra_chunk_bwd_ds_size(prob, q.shape[2], k.shape[2], pairs)
        assert 0 < n <= L.RA_NOALLOC_SCRATCH_BYTES
        sizes.append(n)
        dq1, dk1, dv1 = zeros_like_grads(q, k)
        scratch = torch.full((n,), 0xFF, dtype=torch.uint8, device="cuda")
        api.ra_chunk_bwd_ds(ctx, prob, q, do, lse, dl, k, v, pairs, dq1, dk1, dv1, scratch)
        dq2, dk2, dv2 = zeros_like_grads(q, k)
        api.ra_chunk_bwd_ds_noalloc(ctx, prob, q, do, lse, dl, k, v, pairs, dq2, dk2, dv2)
        torch.cuda.synchronize()
        # dQ has no atomics: the same kernels on the same stored dS give the same bits
        assert (bits(dq2) == bits(dq1)).all(), "dQ differs from ra_chunk_bwd_ds"
        # dK / dV add the query heads of a group with fp32 atomics, whose order may differ
        for got, ref, name in ((dk2, dk1, "dK"), (dv2, dv1, "dV")):
            assert_close(to_f64(got), to_f64(ref), "bf16", name)
            assert np.max(np.abs(to_f64(got) - to_f64(ref))) <= 1e-5 * max(1.0, np.max(np.abs(to_f64(ref))))
    assert sizes[1] < sizes[0]


def test_noalloc_rejects_more_than_the_static_scratch(ctx):
    B, Hq, Hkv, D, Lq = 1, 1, 1, 128, 8192
    prob = api.Problem(B, 2 * Lq, Hq, Hkv, D, 1, "contiguous", "bf16")
    pairs = [(0, 0, Lq, Lq, L.RA_MASK_FULL)]
    assert api.ra_chunk_bwd_ds_size(prob, Lq, Lq, pairs) > L.RA_NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, Hq, Lq, D), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((B, Hkv, Lq, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((B, Hq, Lq), device="cuda")
    dq, dk, dv = zeros_like_grads(q, k)
    with pytest.raises(L.RAValueError) as e:
        api.ra_chunk_bwd_ds_noalloc(ctx, prob, q, q, lse, lse, k, k, pairs, dq, dk, dv)
    assert e.value.status == L.RA_ERR_WORKSPACE
