"""The decode entry point that allocates nothing (its scratch is the library's
per-GPU static array) gives the same bits as the entry point with a caller
workspace, on the paths that use scratch: split-K with the rank-1 prior,
the sampled tail, and a long plain list.  Two calls in a row, the second on
a smaller input, so the second reads scratch the first left behind."""
import numpy as np
import pytest
import torch

from long_context_sparse_gathered_amd import sda, synth
from tests.gpu_util import case_to_dev, dev, to_dev

pytestmark = pytest.mark.gpu


def _same(a, b, what):
    a, b = a.cpu(), b.cpu()
    assert torch.equal(a, b), f"{what}: max |diff| {(a.double() - b.double()).abs().max().item()}"


def _both(call):
    """Run `call(noalloc)` with the workspace entry point and without it."""
    ref = call(False)
    torch.cuda.synchronize()
    got = call(True)
    torch.cuda.synchronize()
    return ref, got


def _decode(noalloc, q, K, V, idx, tail, lam=1.0, idx_len=None):
    B, Hq, d = q.shape
    out = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device=q.device)
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=q.device)
    if noalloc:
        return sda.sparse_decode_attn_noalloc(q, K, V, idx, out, lse, tail=tail, lam=lam, idx_len=idx_len)
    return sda.sparse_decode_attn(q, K, V, idx, tail=tail, lam=lam, idx_len=idx_len, out=out, lse=lse)


@pytest.mark.parametrize("shape", [(4, 16384, 700), (2, 8192, 450)])
def test_prior_split_k(shape):
    B, n, top = shape
    w = synth.WORKLOADS["prior_bf16_b16_n128k"].replace(B=B, n=n, n_top=top)
    c = synth.make_case(w)
    d = case_to_dev(c)
    ps = sda.build_prior(d["K"], d["V"], d["mu_Q"])
    need = sda.workspace_bytes(sda.make_dims(d["K"], w.Hq), sda.OP_SPARSE, sda.TAIL_PRIOR, c.idx.shape[-1])
    assert 0 < need <= sda.NOALLOC_SCRATCH_BYTES
    for lam in (1.0, 0.37):
        ref, got = _both(lambda na: _decode(na, d["q"], d["K"], d["V"], d["idx"], ps, lam))
        _same(ref[0], got[0], f"out lam={lam}")
        _same(ref[1], got[1], f"lse lam={lam}")


@pytest.mark.parametrize("shape", [(2, 16384, 160), (1, 8192, 80)])
def test_sampled(shape):
    B, n, top = shape
    w = synth.WORKLOADS["sampled_bf16_b8_n64k"].replace(B=B, n=n, n_top=top)
    c = synth.make_case(w)
    d = case_to_dev(c)
    need = sda.workspace_bytes(sda.make_dims(d["K"], w.Hq), sda.OP_SPARSE, sda.TAIL_SAMPLED, c.idx.shape[-1])
    assert 0 < need <= sda.NOALLOC_SCRATCH_BYTES

    def call(na):
        t = sda.SampledTail(eps=w.eps, delta=w.delta, b0=w.b0, seed=w.sampler_seed, b_cap=64,
                            b=torch.zeros((w.B, w.Hkv), dtype=torch.int32, device=dev()),
                            bstar=torch.zeros((w.B, w.Hkv), dtype=torch.float64, device=dev()),
                            samples=torch.full((w.B, w.Hkv, 64), -1, dtype=torch.int32, device=dev()))
        out, lse = _decode(na, d["q"], d["K"], d["V"], d["idx"], t)
        return out, lse, t.b, t.bstar, t.samples

    ref, got = _both(call)
    for name, a, b in zip(("out", "lse", "b", "bstar", "samples"), ref, got):
        _same(a, b, name)


@pytest.mark.parametrize("shape", [(2, 5000, 3001), (1, 3000, 1200)])
def test_long_plain_list_fp32(shape):
    B, n, m = shape
    rng = np.random.default_rng(m)
    q = rng.standard_normal((B, 4, 128)).astype(np.float32)
    K = (rng.standard_normal((B, 2, n, 128)) + 0.2).astype(np.float32)
    V = rng.standard_normal((B, 2, n, 128)).astype(np.float32)
    idx = np.sort(rng.choice(n, size=(B, 2, m)), axis=-1).astype(np.int32)
    qd, Kd, Vd, idxd = to_dev(q), to_dev(K), to_dev(V), to_dev(idx)
    assert sda.workspace_bytes(sda.make_dims(Kd, 4), sda.OP_SPARSE, sda.TAIL_NONE, m) > 0
    ref, got = _both(lambda na: _decode(na, qd, Kd, Vd, idxd, None))
    _same(ref[0], got[0], "out")
    _same(ref[1], got[1], "lse")
