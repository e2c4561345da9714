"""GPU parity at the workloads' full sizes, in the launch configuration the benchmark times.

The oracle cannot afford every row at these sizes, so each rank view is checked on:
  * sampled query rows of O, LSE and dQ (rows are independent: the oracle computes exactly
    those rows, for one whole key/value group of query heads and one more head);
  * dK, dV of the keys at the end of the rank's last chunk, which only the queries after them
    in that chunk can see (so the oracle needs only those query rows);
  * properties that hold at any size: sum_j dV_j = sum over the group's heads and the rank's rows
    of dO, sum_j dK_j = 0, and exact zeros in the rows of chunks the rank never attends to.
The smallest workloads (tiny fp32, GPT-2-shaped) are compared on every element.
"""
import functools

import numpy as np
import pytest
import torch

from context_blockwise_causal_amd import api
from context_blockwise_causal_amd.inputs import draw, f32_from_bf16_bits
from context_blockwise_causal_amd.workloads import WORKLOADS
from oracle import attn64 as O
from tests.gpu_util import (assert_close, oracle_dq_rows, oracle_fwd_rows, stratified_rows, to_dev,
                             to_f64)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ctx():
    c = api.Context(0)
    yield c
    c.close()


@functools.lru_cache(maxsize=1)
def _drawn(key):
    return draw(*key)


def drawn(name):
    wl = WORKLOADS[name]  # the two long-ring layouts share one draw
    return _drawn((wl.batch, wl.seq_len, wl.heads_q, wl.heads_kv, wl.head_dim, wl.dtype, wl.seed))


def f64_sub(t, name, heads=None, rows=None):
    a = t.store[name]
    if heads is not None:
        a = a[:, heads]
    if rows is not None:
        a = a[:, :, rows]
    return (f32_from_bf16_bits(a) if t.dtype == "bf16" else np.asarray(a, np.float32)).astype(np.float64)


def run_rank(ctx, prob, dev, k_ring, v_ring, rank, backward):
    q_sl = api.ra_layout_gather(ctx, prob, rank, 1, dev["q"])
    o, lse = api.rank_view_fwd(ctx, prob, rank, q_sl, k_ring, v_ring, staging=torch.cuda.Stream())
    out = {"o": o, "lse": lse}
    if backward:
        do_sl = api.ra_layout_gather(ctx, prob, rank, 1, dev["do"])
        out["dq"], out["dk"], out["dv"] = api.rank_view_bwd(ctx, prob, rank, q_sl, k_ring, v_ring, o, lse,
                                                            do_sl, staging=torch.cuda.Stream())
    torch.cuda.synchronize()
    return out


def setup(ctx, name):
    wl = WORKLOADS[name]
    prob = api.Problem(wl.batch, wl.seq_len, wl.heads_q, wl.heads_kv, wl.head_dim, wl.cp, wl.layout, wl.dtype)
    t = drawn(name)
    dev = {n: to_dev(t.store[n], wl.dtype) for n in ("q", "k", "v", "do")}
    k_ring = api.ra_layout_gather(ctx, prob, 0, wl.cp, dev["k"])
    v_ring = api.ra_layout_gather(ctx, prob, 0, wl.cp, dev["v"])
    return wl, prob, t, dev, k_ring, v_ring


@pytest.mark.parametrize("name", ["tiny-f32-cp2", "gpt2s-bf16-cp4"])
def test_small_workloads_every_element(ctx, name):
    wl, prob, t, dev, k_ring, v_ring = setup(ctx, name)
    q64, k64, v64 = (t.as_f64(n) for n in ("q", "k", "v"))
    for rank in wl.ranks:
        print(f"[{name}] rank {rank}", flush=True)
        out = run_rank(ctx, prob, dev, k_ring, v_ring, rank, wl.backward)
        ro, rl = O.rank_view_fwd(q64, k64, v64, wl.cp, wl.layout, rank)
        assert_close(to_f64(out["o"]), ro, wl.dtype, f"O rank {rank}")
        assert np.max(np.abs(to_f64(out["lse"]) - rl)) < (1e-5 if wl.dtype == "f32" else 2e-3)


@pytest.mark.parametrize("name", ["llama-gqa-cp8-zigzag", "qwen3-ulysses-share", "long-ring-cp16-zigzag",
                                  "long-ring-cp16-contiguous"])
def test_large_workloads_sampled(ctx, name):
    wl, prob, t, dev, k_ring, v_ring = setup(ctx, name)
    S, cp, n_rep = wl.seq_len, wl.cp, wl.heads_q // wl.heads_kv
    g_extra = wl.heads_kv - 1
    heads = sorted(set(list(range(n_rep)) + [g_extra * n_rep + n_rep - 1]))
    kv_heads = sorted({h // n_rep for h in heads})
    kpos = np.arange(S)
    k64 = {g: f64_sub(t, "k", [g]) for g in kv_heads}
    v64 = {g: f64_sub(t, "v", [g]) for g in kv_heads}
    order = O.ring_order(S, cp, wl.layout)
    ring_index = np.empty(S, np.int64)
    ring_index[order] = np.arange(S)
    rng = np.random.default_rng(wl.seed)
    for rank in wl.ranks:
        print(f"[{name}] rank {rank}", flush=True)
        out = run_rank(ctx, prob, dev, k_ring, v_ring, rank, wl.backward)
        pos = O.rank_positions(S, cp, wl.layout, rank)
        n = len(pos)
        # two rows of every 128-row query tile (the tile of the forward and dQ kernels)
        sample = stratified_rows(n, 128, 2, rng)
        got = {k: to_f64(v) for k, v in out.items() if k in ("o", "lse", "dq")}
        for h in heads:
            g = h // n_rep
            rows = pos[sample]
            q = f64_sub(t, "q", [h], rows)
            do = f64_sub(t, "do", [h], rows)
            ro, rl = oracle_fwd_rows(q, k64[g], v64[g], rows, kpos, block=32)
            assert_close(got["o"][:, h][:, sample], ro[:, 0], wl.dtype, f"O rank {rank} head {h}")
            assert np.max(np.abs(got["lse"][:, h][:, sample] - rl[:, 0])) < 2e-3
            if wl.backward:
                rdq = oracle_dq_rows(q, k64[g], v64[g], do, rows, kpos, block=16)
                assert_close(got["dq"][:, h][:, sample], rdq[:, 0], wl.dtype, f"dQ rank {rank} head {h}")
        if not wl.backward:
            continue
        dk = out["dk"]
        dv = out["dv"]
        # keys at the end of the rank's last chunk: only the rank's rows after them see them
        last_chunk_end = int(pos[-1]) + 1
        tail = np.arange(last_chunk_end - 256, last_chunk_end)
        for g in kv_heads:
            grp = list(range(g * n_rep, (g + 1) * n_rep))
            q = f64_sub(t, "q", grp, tail)
            do = f64_sub(t, "do", grp, tail)
            _, rdk, rdv = O.attention_rows_bwd(q, k64[g], v64[g], do, tail, kpos)
            sel = torch.from_numpy(ring_index[tail]).cuda()
            assert_close(to_f64(dk[:, g][:, sel]), rdk[:, 0, tail], wl.dtype, f"dK tail rank {rank} kv {g}")
            assert_close(to_f64(dv[:, g][:, sel]), rdv[:, 0, tail], wl.dtype, f"dV tail rank {rank} kv {g}")
        # sum_j dV_j = the group's sum of dO over the rank's rows; sum_j dK_j = 0
        dv_sum = dv.float().sum(dim=2).double().cpu().numpy()          # (B, Hkv, D)
        do_sl = api.ra_layout_gather(ctx, prob, rank, 1, dev["do"]).float()
        expect = do_sl.view(wl.batch, wl.heads_kv, n_rep, n, wl.head_dim).sum(dim=(2, 3)).double().cpu().numpy()
        rel = np.linalg.norm(dv_sum - expect) / np.linalg.norm(expect)
        assert rel < 2e-2, f"sum dV rank {rank}: rel {rel:.3e}"
        dk_f = dk.float()
        dk_sum = dk_f.sum(dim=2).double().cpu().numpy()
        scale = torch.linalg.vector_norm(dk_f).item()
        assert np.linalg.norm(dk_sum) < 0.1 * scale, f"sum dK rank {rank} not ~0"
        # chunks the rank never attends to carry exact zeros
        if wl.layout == "contiguous":
            zero_from = (rank + 1) * prob.chunk
            if zero_from < S:
                assert torch.count_nonzero(dk[:, :, zero_from:]) == 0
                assert torch.count_nonzero(dv[:, :, zero_from:]) == 0
        del out, dk, dv
        torch.cuda.empty_cache()


@pytest.mark.parametrize("name,rank", [("llama-gqa-cp8-zigzag", 0), ("llama-gqa-cp8-zigzag", 7),
                                       ("long-ring-cp16-zigzag", 0)])
def test_staged_owner_grads_every_element(ctx, name, rank):
    """dK and dV of staged (FULL-pair) owners at full size, element by element: the owners of
    ring steps 1 and 2, whose chunks were staged into slot 0 and slot 1 and whose dK/dV kernels
    ran on the compute stream and on the second stream, with the per-owner zeroing and cast.
    For each owner 64 keys at the start and 64 at the end of its chunk are compared for one
    key/value group; the oracle takes every rank row that sees them (O and LSE over each row's
    whole causal key prefix), then the keys' gradients from those rows (key_grads)."""
    wl, prob, t, dev, k_ring, v_ring = setup(ctx, name)
    S, cp, n_rep = wl.seq_len, wl.cp, wl.heads_q // wl.heads_kv
    out = run_rank(ctx, prob, dev, k_ring, v_ring, rank, True)
    dk, dv = to_f64(out["dk"][:, :1]), to_f64(out["dv"][:, :1])   # kv group 0, ring order
    del out
    torch.cuda.empty_cache()
    g, grp = 0, list(range(n_rep))
    pos = O.rank_positions(S, cp, wl.layout, rank)
    kpos = np.arange(S)
    k64, v64 = f64_sub(t, "k", [g]), f64_sub(t, "v", [g])
    chunk = prob.chunk
    for step in (1, 2):
        owner, pairs = api.ra_plan_step(prob, rank, step)
        assert any(p_[4] == 0 for p_ in pairs), "step must have a FULL pair"
        opos = O.rank_positions(S, cp, wl.layout, owner)
        sel_idx = np.concatenate([np.arange(64), np.arange(chunk - 64, chunk)])
        sel = opos[sel_idx]                                    # sequence positions of the keys
        rows = pos[pos >= sel.min()]                           # the rank rows that can see them
        print(f"[{name}] rank {rank} step {step} owner {owner}: {len(rows)} rows", flush=True)
        q = f64_sub(t, "q", grp, rows)
        do = f64_sub(t, "do", grp, rows)
        o, lse = oracle_fwd_rows(q, k64, v64, rows, kpos, block=64)
        rdk, rdv = O.key_grads(q, k64[:, :, sel], v64[:, :, sel], do, rows, sel, o, lse)
        ring_rows = owner * chunk + sel_idx
        assert_close(dk[:, :, ring_rows], rdk, wl.dtype, f"dK owner {owner}")
        assert_close(dv[:, :, ring_rows], rdv, wl.dtype, f"dV owner {owner}")
