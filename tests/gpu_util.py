"""Helpers shared by the GPU tests: device tensors from the seeded inputs, tolerance checks."""
import numpy as np
import torch

from context_blockwise_causal_amd import api
from context_blockwise_causal_amd.inputs import bf16_bits_from_f32, f32_from_bf16_bits

# Tolerances against the FP64 oracle.  bf16 inputs: elementwise |got - ref| <= 2e-2 + 1e-2 |ref|
# (absolute and relative bounds combined as in allclose) and, per tensor,
# ||got - ref||_2 <= 1e-2 ||ref||_2.  fp32 inputs: max |got - ref| <= 1e-5.
BF16_ATOL, BF16_RTOL, BF16_L2 = 2e-2, 1e-2, 1e-2
F32_ATOL = 1e-5


to_dev = api.to_device


def to_f64(t) -> np.ndarray:
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return f32_from_bf16_bits(t.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    return t.float().cpu().numpy().astype(np.float64)


def bits(t) -> np.ndarray:
    """Raw bytes of a device tensor, for bit-exact comparisons."""
    return t.detach().contiguous().view(torch.uint8).cpu().numpy()


def assert_close(got, ref, dtype: str, name: str):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    err = np.abs(got - ref)
    if dtype == "f32":
        mx = float(err.max()) if err.size else 0.0
        assert mx <= F32_ATOL, f"{name}: max abs err {mx:.3e} > {F32_ATOL}"
        return mx
    bound = BF16_ATOL + BF16_RTOL * np.abs(ref)
    worst = float((err / bound).max()) if err.size else 0.0
    assert worst <= 1.0, f"{name}: elementwise error {worst:.3f} x the bf16 bound (max abs {err.max():.3e})"
    nref = float(np.linalg.norm(ref))
    if nref > 0:
        rel = float(np.linalg.norm(got - ref)) / nref
        assert rel <= BF16_L2, f"{name}: relative L2 error {rel:.3e} > {BF16_L2}"
    return worst


def round_like(x64: np.ndarray, dtype: str) -> np.ndarray:
    """Store form of an fp64 array after rounding to the problem dtype (for building inputs)."""
    x32 = np.asarray(x64, np.float32)
    return bf16_bits_from_f32(x32) if dtype == "bf16" else x32


def problem_for(B, S, Hq, Hkv, D, cp, layout, dtype):
    return api.Problem(B, S, Hq, Hkv, D, cp, layout, dtype)



def _parallel_blocks(fn, n, block):
    """fn(row slice) over blocks of rows in parallel threads, one BLAS thread each."""
    import concurrent.futures
    import os

    from threadpoolctl import threadpool_limits

    starts = list(range(0, n, block))
    workers = max(1, min(16, len(os.sched_getaffinity(0)), len(starts)))

    def one(s):
        with threadpool_limits(1):
            return fn(slice(s, s + block))

    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        return list(ex.map(one, starts))


def oracle_fwd_rows(q, k, v, rows, kpos, block=256, **kw):
    """O.attention_rows over blocks of query rows in parallel (rows are independent, so this
    only splits the work): returns O and LSE for all rows."""
    from oracle import attn64 as O
    parts = _parallel_blocks(lambda sl: O.attention_rows(q[:, :, sl], k, v, rows[sl], kpos, **kw),
                             len(rows), block)
    return np.concatenate([p_[0] for p_ in parts], axis=2), np.concatenate([p_[1] for p_ in parts], axis=2)


def oracle_dq_rows(q, k, v, do, rows, kpos, block=128, **kw):
    """dQ of the given rows from O.attention_rows_bwd, over blocks of rows in parallel."""
    from oracle import attn64 as O
    parts = _parallel_blocks(
        lambda sl: O.attention_rows_bwd(q[:, :, sl], k, v, do[:, :, sl], rows[sl], kpos, **kw)[0],
        len(rows), block)
    return np.concatenate(parts, axis=2)


def stratified_rows(n, tile, per_tile, rng):
    """Row sample hitting every `tile`-row tile `per_tile` times (plus the first and last row)."""
    picks = [0, n - 1]
    for t0 in range(0, n, tile):
        m = min(tile, n - t0)
        picks.extend(t0 + rng.choice(m, min(per_tile, m), replace=False))
    return np.unique(np.asarray(picks, np.int64))
