"""CPU tests of libringattn: the library loads, exports every symbol include/ra.h declares, and
its host-only logic (validation, ring step plans, workspace sizes) is right.  No GPU calls."""
import ctypes
import os
import re

import numpy as np
import pytest

from context_blockwise_causal_amd import _lib as L
from context_blockwise_causal_amd import api
from oracle import attn64 as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KIND = {O.FULL: L.RA_MASK_FULL, O.DIAG: L.RA_MASK_DIAG, O.SKIP: L.RA_MASK_SKIP}


def declared_functions():
    text = open(os.path.join(ROOT, "include", "ra.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ra_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = L.load()
    names = declared_functions()
    assert len(names) == 26
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(L.SIGNATURES) | set(L.OTHER)
    assert lib.ra_version().startswith(b"libringattn")
    assert L.status_str(L.RA_ERR_WORKSPACE) == "RA_ERR_WORKSPACE"


@pytest.mark.parametrize("layout", ["contiguous", "zigzag"])
@pytest.mark.parametrize("cp", [1, 2, 4, 8, 16])
def test_plan_matches_oracle_brute_force(layout, cp):
    S = 2 * cp * 8
    prob = api.Problem(1, S, 2, 1, 64, cp, layout, "bf16")
    for rank in range(cp):
        for step in range(cp):
            owner, pairs = api.ra_plan_step(prob, rank, step)
            o_owner, o_pairs = O.plan_step(S, cp, layout, rank, step)
            assert owner == o_owner
            assert sorted(pairs) == sorted((a, b, c, d, KIND[k]) for a, b, c, d, k in o_pairs)


def test_workspace_sizes():
    p = api.Problem(2, 4096, 12, 4, 64, 4, "contiguous", "bf16")
    rows = 2 * 12 * 1024
    slot = 2 * 4 * 1024 * 64 * 2 * 2
    state = rows * 64 * 4 + 2 * rows * 4
    assert api.ra_workspace_size(p, 0) == 2 * state + 2 * slot  # two states with two slots
    kvel = 2 * 4 * 4096 * 64
    # bf16 backward: two stored-dS buffers of one step's pair (B * Hq * 1024 keys * 1024 queries)
    ds = 2 * 12 * 1024 * 1024 * 2
    assert api.ra_workspace_size(p, 1) == rows * 64 * 4 + 2 * kvel * 4 + rows * 4 + 2 * slot + 2 * ds
    # the scratch of one step, through the chunk-level query: dS^T blocks of key rows x query
    # columns, both padded to 128; SKIP pairs take none
    assert api.ra_chunk_bwd_ds_size(p, 1024, 1024, [(0, 0, 1024, 1024, 0)]) == ds
    assert api.ra_chunk_bwd_ds_size(p, 300, 200, [(0, 0, 150, 100, 0), (150, 0, 150, 100, 2)]) == \
        2 * 12 * 128 * 256 * 2
    assert api.ra_chunk_bwd_ds_size(p, 300, 300, [(0, 0, 150, 150, 1), (150, 0, 150, 150, 0)]) == \
        2 * (2 * 12 * 256 * 256 * 2)
    f32 = api.Problem(2, 4096, 12, 4, 64, 4, "contiguous", "f32")
    assert api.ra_chunk_bwd_ds_size(f32, 1024, 1024, [(0, 0, 1024, 1024, 0)]) == 0
    assert api.ra_workspace_size(p, 2) == (1 + 4) * (rows * 64 * 4 + 2 * rows * 4)  # running + 4 partials
    two = api.Problem(2, 4096, 12, 4, 64, 2, "contiguous", "bf16")  # one staging slot, one state
    rows2 = 2 * 12 * 2048
    assert api.ra_workspace_size(two, 0) == rows2 * 64 * 4 + 2 * rows2 * 4 + 2 * 4 * 2048 * 64 * 2 * 2
    one = api.Problem(1, 512, 2, 2, 128, 1, "contiguous", "f32")
    assert api.ra_workspace_size(one, 0) == 2 * 512 * 128 * 4 + 2 * 4096  # no staging slots at cp=1


@pytest.mark.parametrize("kw,code", [
    (dict(heads_q=6, heads_kv=4), L.RA_ERR_INVALID),            # Hq % Hkv
    (dict(seq_len=100, cp=3), L.RA_ERR_INVALID),                # S % cp
    (dict(seq_len=96, cp=4, layout="zigzag"), L.RA_ERR_INVALID),  # S % 2cp (96 % 8 = 0 ok) -> use 100
    (dict(head_dim=96), L.RA_ERR_UNSUPPORTED),
    (dict(batch=0), L.RA_ERR_INVALID),
    (dict(scale=-1.0), L.RA_ERR_INVALID),
])
def test_validation_errors(kw, code):
    base = dict(batch=1, seq_len=64, heads_q=4, heads_kv=2, head_dim=64, cp=2, layout="contiguous",
                dtype="bf16", scale=0.0)
    base.update(kw)
    if kw.get("layout") == "zigzag":
        base["seq_len"] = 100  # 100 % 8 != 0
    p = api.Problem(**base)
    with pytest.raises(ValueError) as e:
        api.ra_validate(p, 0)
    assert e.value.status == code
    assert L.last_error()


def test_rank_and_step_errors():
    p = api.Problem(1, 64, 2, 2, 64, 4, "zigzag", "bf16")
    for rank in (-1, 4):
        with pytest.raises(ValueError):
            api.ra_validate(p, rank)
    with pytest.raises(ValueError):
        api.ra_plan_step(p, 0, 4)
    bad = L.problem(1, 64, 2, 2, 64, 2, 7, L.RA_BF16)
    assert L.load().ra_validate(ctypes.byref(bad), 0) == L.RA_ERR_INVALID
    assert L.load().ra_validate(None, 0) == L.RA_ERR_INVALID


def test_device_entry_points_reject_null_context_without_enqueueing():
    p = L.problem(1, 64, 2, 2, 64, 1, L.RA_CONTIGUOUS, L.RA_BF16)
    lib = L.load()
    st = lib.ra_layout_gather(None, ctypes.byref(p), 0, 1, 2, None, None, None)
    assert st == L.RA_ERR_INVALID
    arr = L.pairs_array([(0, 0, 8, 8, L.RA_MASK_DIAG)])
    st = lib.ra_chunk_fwd(None, ctypes.byref(p), None, 8, None, None, 8, arr, 1, None, None, None, None)
    assert st == L.RA_ERR_INVALID
    # the debug switch, too: no context, whatever the flags
    assert lib.ra_set_debug(None, 0) == L.RA_ERR_INVALID
    assert lib.ra_set_debug(None, L.RA_DEBUG_POISON_SLOTS | L.RA_DEBUG_ROCTX) == L.RA_ERR_INVALID


@pytest.mark.parametrize("layout", ["contiguous", "zigzag"])
@pytest.mark.parametrize("cp,window,chunk", [(4, 5, 0), (4, 0, 8), (8, 40, 0), (8, 0, 16), (2, 3, 12)])
def test_plan_positions_and_window_skips(layout, cp, window, chunk):
    """Pair positions are the rows' sequence positions; a pair is SKIP exactly when the oracle's
    visibility (causal, window, attention chunk) has no visible (query, key) in it."""
    S = 2 * cp * 16
    prob = api.Problem(1, S, 2, 1, 64, cp, layout, "bf16", 0.0, window, chunk)
    for rank in range(cp):
        qpos = O.rank_positions(S, cp, layout, rank)
        for step in range(cp):
            owner, pairs = api.ra_plan_step(prob, rank, step, positions=True)
            kpos = O.rank_positions(S, cp, layout, owner)
            for q0, k0, ql, kl, mask, qp0, kp0 in pairs:
                assert np.array_equal(qpos[q0:q0 + ql], np.arange(qp0, qp0 + ql))
                assert np.array_equal(kpos[k0:k0 + kl], np.arange(kp0, kp0 + kl))
                vis = O.visible(qpos[q0:q0 + ql], kpos[k0:k0 + kl], window, chunk)
                causal = O.classify(qpos[q0:q0 + ql], kpos[k0:k0 + kl])
                if mask == L.RA_MASK_SKIP:
                    assert not vis.any()
                else:
                    assert vis.any()
                    assert KIND[causal] == mask  # the causal kind is kept; the kernel applies the rest


def test_grid_row_limit_is_validated():
    """The row-wise kernels put one (batch, head) per grid row (at most 65535): larger problems
    are rejected by validation, before anything could be enqueued."""
    big = api.Problem(65536, 256, 1, 1, 64, 1, "contiguous", "bf16")
    with pytest.raises(ValueError) as e:
        api.ra_validate(big)
    assert e.value.status == L.RA_ERR_UNSUPPORTED
    api.ra_validate(api.Problem(65535, 256, 1, 1, 64, 1, "contiguous", "bf16"))
    with pytest.raises(ValueError):
        api.ra_workspace_size(api.Problem(8192, 256, 16, 16, 64, 1, "contiguous", "bf16"), 0)
