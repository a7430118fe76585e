"""Helpers shared by the GPU tests: moving generated inputs to the device and
the error metric (max over rows of max |o - o*| / max |o*|, per (seq, head))."""
import numpy as np
import torch


def dev():
    return torch.device("cuda:0")


def to_dev(a: np.ndarray) -> torch.Tensor:
    """numpy -> device tensor; uint16 arrays are bf16 bit patterns."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev())
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def rel_err(got, ref) -> float:
    got = got.detach().cpu().double().numpy() if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.abs(ref).max(axis=-1)
    den = np.where(den > 0, den, 1.0)
    return float((np.abs(got - ref).max(axis=-1) / den).max())


def lse_err(got, ref) -> float:
    got = got.detach().cpu().double().numpy()
    ref = np.asarray(ref, np.float64)
    both_inf = np.isneginf(got) & np.isneginf(ref)
    d = np.where(both_inf, 0.0, np.abs(got - ref))
    return float(d.max())


def case_to_dev(c):
    out = {"q": to_dev(c.q), "K": to_dev(c.K), "V": to_dev(c.V), "idx": to_dev(c.idx)}
    if c.cid is not None:
        out["cid"] = to_dev(c.cid)
        out["idx_cluster"] = to_dev(c.idx_cluster)
    if c.mu_Q is not None:
        out["mu_Q"] = to_dev(c.mu_Q)
    return out
