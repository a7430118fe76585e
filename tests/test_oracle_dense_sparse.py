"""Pins for the oracle's dense and sparse attention.

O-dense is checked against torch's scaled-dot-product attention in float64
(a library routine); O-sparse against the same routine on the gathered rows
with the log-weights as an additive score bias (vAttention page, eq. 3), and
against the invariants the definition implies.
"""
import numpy as np
import pytest
import torch

from long_context_sparse_gathered_amd import synth


def _rand(rng, B, Hq, Hkv, n, d, dtype):
    q = rng.standard_normal((B, Hq, d)).astype(np.float32)
    K = (rng.standard_normal((B, Hkv, n, d)) + 0.5).astype(np.float32)
    V = rng.standard_normal((B, Hkv, n, d)).astype(np.float32)
    if dtype == "bf16":
        return synth.round_bf16_bits(q), synth.round_bf16_bits(K), synth.round_bf16_bits(V)
    return q, K, V


def _f64(x):
    x = np.asarray(x)
    return synth.bf16_bits_to_f32(x).astype(np.float64) if x.dtype == np.uint16 else x.astype(np.float64)


def _torch_sdpa(q, K, V, scale, bias=None):
    """Reference attention from torch, float64, GQA by repeating KV heads."""
    qt = torch.from_numpy(_f64(q))[:, :, None, :]              # [B,Hq,1,d]
    Kt, Vt = torch.from_numpy(_f64(K)), torch.from_numpy(_f64(V))
    G = qt.shape[1] // Kt.shape[1]
    Kt, Vt = Kt.repeat_interleave(G, dim=1), Vt.repeat_interleave(G, dim=1)
    mask = None if bias is None else torch.from_numpy(bias)[:, :, None, :]
    o = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, attn_mask=mask, scale=float(scale))
    return o[:, :, 0, :].numpy()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(1, 1, 1, 37, 16), (2, 8, 2, 300, 128), (1, 4, 4, 5, 8)])
def test_dense_matches_torch_sdpa(orc, dtype, shape):
    rng = np.random.default_rng(11)
    B, Hq, Hkv, n, d = shape
    q, K, V = _rand(rng, B, Hq, Hkv, n, d, dtype)
    scale = np.float32(1 / np.sqrt(d))
    out, lse = orc.dense(q, K, V)
    ref = _torch_sdpa(q, K, V, scale)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    # lse = log sum_j exp(s_j): check against logsumexp of explicit fp64 logits
    G = Hq // Hkv
    s = np.einsum("bhd,bhnd->bhn", _f64(q), np.repeat(_f64(K), G, axis=1)) * np.float64(scale)
    np.testing.assert_allclose(lse, torch.logsumexp(torch.from_numpy(s), dim=-1).numpy(), rtol=1e-13)


def _gather_bias(q, K, V, idx, logw, G):
    """Rows of the index list gathered per KV head, and their log-weights."""
    Kg = np.take_along_axis(K, idx[..., None].astype(np.int64), axis=2)
    Vg = np.take_along_axis(V, idx[..., None].astype(np.int64), axis=2)
    bias = np.repeat(logw.astype(np.float64), G, axis=1)
    return Kg, Vg, bias


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_sparse_matches_torch_on_gathered_rows(orc, dtype):
    rng = np.random.default_rng(5)
    B, Hq, Hkv, n, d, m = 2, 8, 2, 500, 64, 40
    q, K, V = _rand(rng, B, Hq, Hkv, n, d, dtype)
    idx = rng.integers(0, n, size=(B, Hkv, m)).astype(np.int32)  # duplicates allowed
    logw = rng.normal(0, 2, size=(B, Hkv, m)).astype(np.float32)
    out, _ = orc.sparse(q, K, V, idx, logw=logw)
    Kg, Vg, bias = _gather_bias(q, K, V, idx, logw, Hq // Hkv)
    ref = _torch_sdpa(q, Kg, Vg, np.float32(1 / np.sqrt(d)), bias=bias)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_full_index_set_equals_dense(orc):
    rng = np.random.default_rng(2)
    B, Hq, Hkv, n, d = 2, 4, 2, 257, 128
    q, K, V = _rand(rng, B, Hq, Hkv, n, d, "bf16")
    idx = np.broadcast_to(np.arange(n, dtype=np.int32), (B, Hkv, n)).copy()
    o_s, l_s = orc.sparse(q, K, V, idx)
    o_d, l_d = orc.dense(q, K, V)
    np.testing.assert_allclose(o_s, o_d, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(l_s, l_d, rtol=1e-13)


def test_sparse_invariances(orc):
    rng = np.random.default_rng(3)
    B, Hq, Hkv, n, d, m = 1, 4, 1, 200, 32, 30
    q, K, V = _rand(rng, B, Hq, Hkv, n, d, "f32")
    idx = rng.choice(n, size=m, replace=False).astype(np.int32)[None, None]
    # log-weights on a 1/8 grid so that adding 3 is exact in fp32
    logw = (np.round(rng.normal(0, 1, size=(1, 1, m)) * 8) / 8).astype(np.float32)
    base, lse = orc.sparse(q, K, V, idx, logw=logw)
    # a constant added to every log-weight changes the output not at all
    o2, lse2 = orc.sparse(q, K, V, idx, logw=logw + np.float32(3.0))
    np.testing.assert_allclose(o2, base, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse2, lse + 3.0, rtol=1e-12)
    # permuting the list changes nothing
    p = rng.permutation(m)
    o3, _ = orc.sparse(q, K, V, idx[..., p], logw=logw[..., p])
    np.testing.assert_allclose(o3, base, rtol=1e-12, atol=1e-13)
    # duplicates count as separate terms: two copies of a row at log-weight 0
    # equal one copy at log-weight ln 2 (up to the fp32 rounding of ln 2)
    lw = logw.copy()
    lw[..., 0] = 0.0
    idx2 = np.concatenate([idx, idx[..., :1]], axis=-1)
    lw2 = np.concatenate([lw, lw[..., :1]], axis=-1)
    lw1 = lw.copy()
    lw1[..., 0] = np.float32(np.log(2.0))
    o4, _ = orc.sparse(q, K, V, idx2, logw=lw2)
    o5, _ = orc.sparse(q, K, V, idx, logw=lw1)
    np.testing.assert_allclose(o4, o5, rtol=0, atol=1e-6 * np.abs(o5).max())


def test_ragged_lengths_and_empty_unit(orc):
    rng = np.random.default_rng(4)
    B, Hq, Hkv, n, d, m = 2, 2, 2, 100, 16, 12
    q, K, V = _rand(rng, B, Hq, Hkv, n, d, "f32")
    idx = rng.integers(0, n, size=(B, Hkv, m)).astype(np.int32)
    lens = np.array([[12, 5], [0, 1]], np.int32)
    out, lse = orc.sparse(q, K, V, idx, idx_len=lens)
    for s in range(B):
        for g in range(Hkv):
            L = lens[s, g]
            sub_q = q[s:s + 1, g:g + 1]
            if L == 0:
                assert np.all(out[s, g] == 0) and np.isneginf(lse[s, g])
                continue
            o1, l1 = orc.sparse(sub_q, K[s:s + 1, g:g + 1], V[s:s + 1, g:g + 1], idx[s:s + 1, g:g + 1, :L])
            np.testing.assert_allclose(out[s, g], o1[0, 0], rtol=1e-14, atol=1e-15)


def test_rejects_out_of_range(orc):
    q = np.zeros((1, 1, 8), np.float32)
    K = np.zeros((1, 1, 10, 8), np.float32)
    with pytest.raises(ValueError):
        orc.sparse(q, K, K, np.array([[[3, 10]]], np.int32))
