"""Split-K calls (the streaming kernel writes one partial record per split,
then the merge launch combines them) that share one workspace, whatever it
holds beforehand, and replays of a captured call with other calls on the
same workspace between them: every result must equal, bit for bit, that of
a separate eager call with a workspace of its own ("RESA", Online
Aggregator: the merge of partial softmax sums, here in a fixed order)."""
import numpy as np
import pytest
import torch

from long_context_sparse_gathered_amd import sda, synth
from tests.gpu_util import case_to_dev, to_dev

pytestmark = pytest.mark.gpu


def _prior_problem():
    w = synth.WORKLOADS["prior_bf16_b16_n128k"].replace(B=2, n=16384, n_top=600)
    c = synth.make_case(w)
    d = case_to_dev(c)
    ps = sda.build_prior(d["K"], d["V"], d["mu_Q"])
    return d, ps


def _plain_problem(seed=11, B=1, n=6000, m=2500):
    w = synth.WORKLOADS["proxy_bf16_b1_n32k"].replace(B=B, n=n, n_top=40, C=0)
    c = synth.make_case(w)
    rng = np.random.default_rng(seed)
    idx = np.sort(rng.integers(0, n, size=(B, w.Hkv, m)), axis=-1).astype(np.int32)
    d = case_to_dev(c)
    d["idx"] = to_dev(idx)
    return d


def _ws_bytes(d, tail_kind, m):
    dims = sda.make_dims(d["K"], d["q"].shape[1])
    return sda.workspace_bytes(dims, sda.OP_SPARSE, tail_kind, m)


def test_shared_workspace_alternating_calls():
    dp, ps = _prior_problem()
    dn = _plain_problem()
    need = max(_ws_bytes(dp, sda.TAIL_PRIOR, dp["idx"].shape[-1]), _ws_bytes(dn, sda.TAIL_NONE, dn["idx"].shape[-1]))
    assert need > 0  # both calls take the split-K path
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device=dp["K"].device)  # not initialised by the library
    refp = [t.clone() for t in sda.sparse_decode_attn(dp["q"], dp["K"], dp["V"], dp["idx"], tail=ps, lam=0.7)]
    refn = [t.clone() for t in sda.sparse_decode_attn(dn["q"], dn["K"], dn["V"], dn["idx"])]
    torch.cuda.synchronize()
    for _ in range(3):
        op, lp = sda.sparse_decode_attn(dp["q"], dp["K"], dp["V"], dp["idx"], tail=ps, lam=0.7, ws=ws)
        op, lp = op.clone(), lp.clone()
        on, ln = sda.sparse_decode_attn(dn["q"], dn["K"], dn["V"], dn["idx"], ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(op, refp[0]) and torch.equal(lp, refp[1])
        assert torch.equal(on, refn[0]) and torch.equal(ln, refn[1])


def test_graph_replays_with_other_calls_between():
    dp, ps = _prior_problem()
    dn = _plain_problem(seed=12)
    need = max(_ws_bytes(dp, sda.TAIL_PRIOR, dp["idx"].shape[-1]), _ws_bytes(dn, sda.TAIL_NONE, dn["idx"].shape[-1]))
    ws = torch.zeros((need,), dtype=torch.uint8, device=dp["K"].device)
    q = dp["q"].clone()
    out = torch.empty((q.shape[0], q.shape[1], q.shape[2]), dtype=torch.float32, device=q.device)
    lse = torch.empty((q.shape[0], q.shape[1]), dtype=torch.float32, device=q.device)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):  # warm-up outside the capture
        sda.sparse_decode_attn(q, dp["K"], dp["V"], dp["idx"], tail=ps, lam=0.7, out=out, lse=lse, ws=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        sda.sparse_decode_attn(q, dp["K"], dp["V"], dp["idx"], tail=ps, lam=0.7, out=out, lse=lse, ws=ws)
    torch.cuda.synchronize()
    gen = torch.Generator(device="cpu").manual_seed(3)
    for r in range(4):
        qr = (torch.randn(q.shape, generator=gen) * 0.5).to(torch.bfloat16).to(q.device)
        q.copy_(qr)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (out.clone(), lse.clone())
        ref = sda.sparse_decode_attn(qr, dp["K"], dp["V"], dp["idx"], tail=ps, lam=0.7)
        # another call on the same workspace between replays
        sda.sparse_decode_attn(dn["q"], dn["K"], dn["V"], dn["idx"], ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(got[0], ref[0]), f"replay {r}"
        assert torch.equal(got[1], ref[1]), f"replay {r}"
    del g


def test_dense_split_merge_shared_workspace():
    w = synth.WORKLOADS["proxy_bf16_b1_n32k"].replace(B=2, n=9000, n_top=40, C=0)
    c = synth.make_case(w)
    d = case_to_dev(c)
    dims = sda.make_dims(d["K"], d["q"].shape[1])
    need = sda.workspace_bytes(dims, sda.OP_DENSE)
    assert need > 0
    ws = torch.full((need,), 0x5A, dtype=torch.uint8, device=d["K"].device)
    ref = [t.clone() for t in sda.dense_decode_attn(d["q"], d["K"], d["V"])]
    q2 = (d["q"].float() * -0.75).to(torch.bfloat16)
    ref2 = [t.clone() for t in sda.dense_decode_attn(q2, d["K"], d["V"])]
    for _ in range(3):
        a = [t.clone() for t in sda.dense_decode_attn(d["q"], d["K"], d["V"], ws=ws)]
        b = [t.clone() for t in sda.dense_decode_attn(q2, d["K"], d["V"], ws=ws)]
        torch.cuda.synchronize()
        assert all(torch.equal(x, y) for x, y in zip(a, ref))
        assert all(torch.equal(x, y) for x, y in zip(b, ref2))
