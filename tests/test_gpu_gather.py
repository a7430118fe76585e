"""The row-gather measurement aid (sda_gather_rows): every wave's checksum,
the XOR of every 32-bit word it loaded, against the same XOR on the host
over the documented partition of the list and of the per-unit state
(bit-exact), with invalid list entries skipped, ragged shares and state
shares that do not divide evenly."""
import numpy as np
import pytest
import torch

from long_context_sparse_gathered_amd import sda
from tests.gpu_util import dev

pytestmark = pytest.mark.gpu


def _cdiv(a, b):
    return -(-a // b)


def _expected(Kb, Vb, idx, state, waves, parts):
    """Kb, Vb: [B, Hkv, n, 128] uint16; idx [B, Hkv, m]; state [units, bytes] uint8."""
    B, Hkv, n, _ = Kb.shape
    m = idx.shape[-1]
    units = B * Hkv
    out = np.zeros((units, parts, waves), np.uint32)
    kw = Kb.reshape(units, n, 64, 2).astype(np.uint32)
    vw = Vb.reshape(units, n, 64, 2).astype(np.uint32)
    kx = np.bitwise_xor.reduce(kw[..., 0] | (kw[..., 1] << 16), axis=-1)   # [units, n] XOR of a row's words
    vx = np.bitwise_xor.reduce(vw[..., 0] | (vw[..., 1] << 16), axis=-1)
    EP = _cdiv(m, parts)
    EW = _cdiv(EP, waves)
    sbytes = state.shape[1] if state is not None else 0
    SP = _cdiv(_cdiv(sbytes, parts), 16) * 16 if sbytes else 0
    for u in range(units):
        lst = idx.reshape(units, m)[u]
        for p in range(parts):
            e0, e1 = p * EP, min(m, (p + 1) * EP)
            for w in range(waves):
                x = np.uint32(0)
                for e in range(e0 + w * EW, min(e1, e0 + (w + 1) * EW)):
                    j = int(lst[e])
                    if 0 <= j < n:
                        x ^= kx[u, j] ^ vx[u, j]
                out[u, p, w] = x
            if sbytes:
                s0, s1 = p * SP, min(sbytes, (p + 1) * SP)
                words = state[u].view(np.uint32)
                for t in range(64 * waves):
                    b = s0 + 16 * t
                    while b + 16 <= s1:
                        out[u, p, t // 64] ^= np.bitwise_xor.reduce(words[b // 4:b // 4 + 4])
                        b += 16 * 64 * waves
    return out.reshape(-1)


@pytest.mark.parametrize("waves,parts,sbytes", [(8, 1, 0), (4, 3, 1040), (16, 2, 4096), (8, 5, 32)])
def test_gather_checksums_bit_exact(waves, parts, sbytes):
    rng = np.random.default_rng(waves * 100 + parts)
    B, Hkv, n, m = 2, 2, 3000, 150
    Kb = rng.integers(0, 1 << 16, size=(B, Hkv, n, 128), dtype=np.uint16)
    Vb = rng.integers(0, 1 << 16, size=(B, Hkv, n, 128), dtype=np.uint16)
    idx = np.sort(rng.choice(n, size=(B, Hkv, m)), axis=-1).astype(np.int32)
    idx[0, 0, 3] = -1          # skipped
    idx[1, 1, 7] = n + 5       # skipped
    state = rng.integers(0, 256, size=(B * Hkv, sbytes), dtype=np.uint8) if sbytes else None
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev())  # noqa: E731
    K, V = to(Kb), to(Vb)
    st = torch.from_numpy(state).to(dev()) if sbytes else None
    got = sda.gather_rows(K, V, torch.from_numpy(idx).to(dev()), waves=waves, parts=parts, state=st)
    torch.cuda.synchronize()
    got = got.cpu().numpy().view(np.uint32)
    np.testing.assert_array_equal(got, _expected(Kb, Vb, idx, state, waves, parts))
