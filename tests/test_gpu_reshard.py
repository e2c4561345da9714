"""GPU parity of the Ulysses re-shard steps (bit-exact against the oracle's definition) and of
their composition with attention: sequence shards -> all-to-all -> per-rank attention on a
head shard -> all-to-all back, against the FP64 oracle's full-sequence attention."""
import numpy as np
import pytest
import torch

from context_blockwise_causal_amd import _lib as L
from context_blockwise_causal_amd import api
from context_blockwise_causal_amd.inputs import draw_like
from oracle import attn64 as O
from oracle import reshard as R
from tests.gpu_util import assert_close, bits, to_dev, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ctx():
    c = api.Context(0)
    yield c
    c.close()


def exchange_dev(send):
    """The all-to-all between simulated ranks on one device: recv[r][j] = send[j][r]."""
    cp = len(send)
    return [torch.stack([send[j][r] for j in range(cp)]).contiguous() for r in range(cp)]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("cp,B,H,S,D", [(2, 1, 2, 64, 64), (4, 2, 8, 96, 128), (8, 1, 32, 128, 64), (1, 1, 4, 48, 128)])
def test_reshard_steps_bit_exact(ctx, dtype, cp, B, H, S, D):
    prob = api.Problem(B, S, H, H, D, cp, "contiguous", dtype)
    x_store = draw_like((B, H, S, D), dtype, 500 + cp)
    x = to_dev(x_store, dtype)
    x_np = np.asarray(x_store)
    # sequence shards -> send buffers -> exchange -> head shards
    send = [api.ra_ulysses_reshard(ctx, prob, L.RA_A2A_SEQ_PACK, H, x[:, :, r * (S // cp):(r + 1) * (S // cp)].contiguous())
            for r in range(cp)]
    recv = exchange_dev(send)
    heads = [api.ra_ulysses_reshard(ctx, prob, L.RA_A2A_HEAD_UNPACK, H, recv[r]) for r in range(cp)]
    torch.cuda.synchronize()
    for r in range(cp):
        ref_send = R.pack_seq(R.seq_shard(x_np, cp, r), cp)
        np.testing.assert_array_equal(bits(send[r]).reshape(-1), np.ascontiguousarray(ref_send).view(np.uint8).reshape(-1))
        ref_head = R.head_shard(x_np, cp, r)
        np.testing.assert_array_equal(bits(heads[r]).reshape(-1), np.ascontiguousarray(ref_head).view(np.uint8).reshape(-1))
    # and back: head shards -> send buffers -> exchange -> sequence shards
    send2 = [api.ra_ulysses_reshard(ctx, prob, L.RA_A2A_HEAD_PACK, H, heads[r]) for r in range(cp)]
    recv2 = exchange_dev(send2)
    seqs = [api.ra_ulysses_reshard(ctx, prob, L.RA_A2A_SEQ_UNPACK, H, recv2[r]) for r in range(cp)]
    torch.cuda.synchronize()
    for r in range(cp):
        ref_send2 = R.pack_head(R.head_shard(x_np, cp, r), cp)
        np.testing.assert_array_equal(bits(send2[r]).reshape(-1), np.ascontiguousarray(ref_send2).view(np.uint8).reshape(-1))
        ref_seq = R.seq_shard(x_np, cp, r)
        np.testing.assert_array_equal(bits(seqs[r]).reshape(-1), np.ascontiguousarray(ref_seq).view(np.uint8).reshape(-1))


def test_reshard_rejects_bad_arguments(ctx):
    prob = api.Problem(1, 64, 6, 6, 64, 4, "contiguous", "bf16")
    x = torch.zeros((1, 6, 16, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        api.ra_ulysses_reshard(ctx, prob, L.RA_A2A_SEQ_PACK, 6, x)   # 6 heads over cp = 4
    prob2 = api.Problem(1, 64, 8, 8, 64, 4, "contiguous", "bf16")
    with pytest.raises(ValueError):
        api.ra_ulysses_reshard(ctx, prob2, 7, 8, torch.zeros((1, 8, 16, 64), dtype=torch.bfloat16, device="cuda"))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ulysses_attention_composition(ctx, dtype):
    """a2a, then causal attention of full sequences on each rank's heads (GQA: the q and kv
    heads are split alike), then a2a back: the output's sequence shards match the oracle."""
    cp, B, Hq, Hkv, S, D = 4, 1, 8, 4, 256, 64
    n_rep = Hq // Hkv
    q_s, k_s, v_s = (draw_like((B, h, S, D), dtype, 600 + i) for i, h in enumerate((Hq, Hkv, Hkv)))
    q, k, v = (to_dev(a, dtype) for a in (q_s, k_s, v_s))
    prob = api.Problem(B, S, Hq, Hkv, D, cp, "contiguous", dtype)
    Sc = S // cp

    def seq_to_head(t, H):
        send = [api.ra_ulysses_reshard(ctx, prob, L.RA_A2A_SEQ_PACK, H, t[:, :, r * Sc:(r + 1) * Sc].contiguous())
                for r in range(cp)]
        return [api.ra_ulysses_reshard(ctx, prob, L.RA_A2A_HEAD_UNPACK, H, b) for b in exchange_dev(send)]

    qh, kh, vh = seq_to_head(q, Hq), seq_to_head(k, Hkv), seq_to_head(v, Hkv)
    oh = [api.scaled_dot_product_attention(ctx, qh[r], kh[r], vh[r], n_rep)[0] for r in range(cp)]
    send = [api.ra_ulysses_reshard(ctx, prob, L.RA_A2A_HEAD_PACK, Hq, oh[r]) for r in range(cp)]
    o_seq = [api.ra_ulysses_reshard(ctx, prob, L.RA_A2A_SEQ_UNPACK, Hq, b) for b in exchange_dev(send)]
    torch.cuda.synchronize()
    pos = np.arange(S)
    ref, _ = O.attention_rows(to_f64(q), to_f64(k), to_f64(v), pos, pos)
    for r in range(cp):
        assert_close(to_f64(o_seq[r]), ref[:, :, r * Sc:(r + 1) * Sc], dtype, f"O seq shard {r}")
