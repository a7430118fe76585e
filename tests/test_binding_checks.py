"""The Python binding checks every tensor against the shapes, element types and
strides the kernels assume, and raises before calling the library (host only:
the library entry points are replaced by a stub that fails the test if reached;
CPU tensors stand in for device tensors, and a call whose arguments are all
consistent stops at the final "must be on a GPU" check)."""
import pytest
import torch

from long_context_sparse_gathered_amd import sda

B, Hq, Hkv, n, d, m, C = 2, 8, 2, 64, 128, 12, 4


@pytest.fixture(autouse=True)
def no_library(monkeypatch):
    def boom():
        raise AssertionError("the library was called despite a bad argument")
    monkeypatch.setattr(sda, "lib", boom)


def kv(dtype=torch.bfloat16):
    return torch.zeros((B, Hkv, n, d), dtype=dtype), torch.zeros((B, Hkv, n, d), dtype=dtype)


def args(**over):
    K, V = kv()
    a = dict(q=torch.zeros((B, Hq, d), dtype=torch.bfloat16), K=K, V=V,
             idx=torch.zeros((B, Hkv, m), dtype=torch.int32))
    a.update(over)
    return a


def proxies(**over):
    st = dict(C=C, count=torch.zeros((B, Hkv, C), dtype=torch.int32),
              sumK=torch.zeros((B, Hkv, C, d)), sumV=torch.zeros((B, Hkv, C, d)))
    st.update(over)
    return sda.ProxyState(**st)


def prior(**over):
    st = dict(mu_Q=torch.zeros((B, Hq, d)), mu_K=torch.zeros((B, Hkv, d)), O_est=torch.zeros((B, Hq, d)),
              maxP=torch.zeros((B, Hq)), sumP=torch.zeros((B, Hq)))
    st.update(over)
    return sda.PriorState(**st)


def sparse(**kw):
    a = args(**{k: kw.pop(k) for k in list(kw) if k in ("q", "K", "V", "idx")})
    return sda.sparse_decode_attn(a["q"], a["K"], a["V"], a["idx"], **kw)


def raises_on(name, fn):
    with pytest.raises((TypeError, ValueError)) as e:
        fn()
    assert name in str(e.value), str(e.value)


def test_consistent_arguments_reach_the_device_check():
    raises_on("GPU", lambda: sparse())
    raises_on("GPU", lambda: sparse(tail=proxies(), idx_cluster=torch.zeros((B, Hkv, m), dtype=torch.int32)))
    raises_on("GPU", lambda: sparse(tail=prior()))
    raises_on("GPU", lambda: sparse(tail=sda.SampledTail(b_cap=4)))
    K, V = kv()
    raises_on("GPU", lambda: sda.dense_decode_attn(torch.zeros((B, Hq, d), dtype=torch.bfloat16), K, V))


def test_value_cache_must_match_keys():
    K, _ = kv()
    raises_on("V", lambda: sparse(V=torch.zeros((B, Hkv, n + 1, d), dtype=torch.bfloat16)))       # shape
    raises_on("V", lambda: sparse(V=torch.zeros((B, Hkv, n, d), dtype=torch.float32)))            # dtype
    kvbuf = torch.zeros((B, Hkv, n, 2, d), dtype=torch.bfloat16)
    raises_on("V", lambda: sparse(V=kvbuf[:, :, :, 1, :]))                                         # strides
    raises_on("K", lambda: sparse(K=torch.zeros((B, Hkv, n, d), dtype=torch.float16),
                                  V=torch.zeros((B, Hkv, n, d), dtype=torch.float16)))


def test_query_checks():
    raises_on("q", lambda: sparse(q=torch.zeros((B, Hq, d), dtype=torch.float32)))                # dtype
    raises_on("q", lambda: sparse(q=torch.zeros((B, Hq, 2 * d), dtype=torch.bfloat16)[..., ::2]))  # strided
    raises_on("q", lambda: sparse(q=torch.zeros((B, Hq + 1, d), dtype=torch.bfloat16)))           # heads
    raises_on("q", lambda: sparse(q=torch.zeros((B + 1, Hq, d), dtype=torch.bfloat16)))           # batch


def test_list_checks():
    raises_on("idx", lambda: sparse(idx=torch.zeros((B, Hkv, m), dtype=torch.int64)))
    raises_on("idx", lambda: sparse(idx=torch.zeros((B, Hkv + 1, m), dtype=torch.int32)))
    raises_on("m", lambda: sparse(m=m + 1))                                                       # m beyond idx
    raises_on("m", lambda: sparse(m=m - 1))
    raises_on("m", lambda: sparse(idx=None, m=3))
    raises_on("idx_len", lambda: sparse(idx_len=torch.zeros((B, Hkv + 1), dtype=torch.int32)))
    raises_on("logw", lambda: sparse(logw=torch.zeros((B, Hkv, m - 1))))
    raises_on("logw", lambda: sparse(logw=torch.zeros((B, Hkv, m), dtype=torch.float64)))
    raises_on("flags", lambda: sparse(flags=torch.zeros((B, Hkv), dtype=torch.int64)))


def test_output_checks():
    raises_on("out", lambda: sparse(out=torch.zeros((B, Hq, d), dtype=torch.bfloat16)))
    raises_on("out", lambda: sparse(out=torch.zeros((B, Hq, d - 1))))
    raises_on("out", lambda: sparse(out=torch.zeros((B, d, Hq)).transpose(1, 2)))
    raises_on("lse", lambda: sparse(lse=torch.zeros((B, Hq), dtype=torch.float64)))
    raises_on("lse", lambda: sparse(lse=torch.zeros((B, Hq + 1))))


def test_proxy_state_checks():
    icl = torch.zeros((B, Hkv, m), dtype=torch.int32)
    raises_on("idx_cluster", lambda: sparse(tail=proxies(), idx_cluster=torch.zeros((B, Hkv, m + 1), dtype=torch.int32)))
    raises_on("cluster_id", lambda: sparse(tail=proxies(), cluster_id=torch.zeros((B, Hkv, n - 1), dtype=torch.int32)))
    raises_on("count", lambda: sparse(tail=proxies(count=torch.zeros((B, Hkv, C + 1), dtype=torch.int32)),
                                      idx_cluster=icl))
    raises_on("sumK", lambda: sparse(tail=proxies(sumK=torch.zeros((B, Hkv, C, d), dtype=torch.bfloat16)),
                                     idx_cluster=icl))
    raises_on("sumV", lambda: sparse(tail=proxies(sumV=torch.zeros((B, Hkv, C + 1, d))), idx_cluster=icl))


def test_prior_state_checks():
    raises_on("mu_Q", lambda: sparse(tail=prior(mu_Q=torch.zeros((B, Hkv, d)))))
    raises_on("mu_K", lambda: sparse(tail=prior(mu_K=torch.zeros((B, Hq, d)))))
    raises_on("O_est", lambda: sparse(tail=prior(O_est=torch.zeros((B, Hq, d), dtype=torch.float64))))
    raises_on("maxP", lambda: sparse(tail=prior(maxP=torch.zeros((B, Hkv)))))
    raises_on("sumP", lambda: sparse(tail=prior(sumP=torch.zeros((B, Hq, 1)))))


def test_sampled_output_checks():
    raises_on("b", lambda: sparse(tail=sda.SampledTail(b=torch.zeros((B, Hkv + 1), dtype=torch.int32))))
    raises_on("bstar", lambda: sparse(tail=sda.SampledTail(bstar=torch.zeros((B, Hkv)))))
    raises_on("samples", lambda: sparse(tail=sda.SampledTail(b_cap=8,
                                                             samples=torch.zeros((B, Hkv, 4), dtype=torch.int32))))


def test_builder_and_dense_checks():
    K, V = kv()
    raises_on("cluster_id", lambda: sda.build_tail_proxies(K, V, torch.zeros((B, Hkv, n), dtype=torch.int64), C))
    raises_on("V", lambda: sda.build_tail_proxies(K, torch.zeros((B, Hkv, n, d)), torch.zeros((B, Hkv, n),
                                                                                                 dtype=torch.int32), C))
    raises_on("q", lambda: sda.build_prior(K, V, torch.zeros((B, Hq, d), dtype=torch.bfloat16)))
    raises_on("q", lambda: sda.build_prior(K, V, torch.zeros((B, Hq + 1, d))))
    q = torch.zeros((B, Hq, d), dtype=torch.bfloat16)
    raises_on("out", lambda: sda.dense_decode_attn(q, K, V, out=torch.zeros((B, Hq, d), dtype=torch.bfloat16)))
    raises_on("V", lambda: sda.dense_decode_attn(q, K, V[:, :1]))
    raises_on("ws", lambda: sda.dense_decode_attn(q, K, V, ws=torch.zeros(16, dtype=torch.int32)))


def test_selector_and_clustering_checks():
    K, _ = kv()
    q = torch.zeros((B, Hq, d), dtype=torch.bfloat16)
    cid = torch.zeros((B, Hkv, n), dtype=torch.int32)
    st = proxies(sumK2=torch.zeros((B, Hkv, C, d)))
    qc = sda.QgsCodes(U=torch.zeros((B, Hkv, d, sda.QGS_RANK)),
                      codes=torch.zeros((B, Hkv, n, sda.QGS_RANK), dtype=torch.int8),
                      kmax=torch.zeros((B, Hkv, sda.QGS_RANK), dtype=torch.float64))
    raises_on("GPU", lambda: sda.select_qgs(q, K, cid, st, qc, 4, 8, 10))
    raises_on("codes", lambda: sda.select_qgs(q, K, cid, st, sda.QgsCodes(U=qc.U, codes=qc.codes[:, :, :-1],
                                                                          kmax=qc.kmax), 4, 8, 10))
    raises_on("kmax", lambda: sda.select_qgs(q, K, cid, st, sda.QgsCodes(U=qc.U, codes=qc.codes,
                                                                         kmax=qc.kmax.float()), 4, 8, 10))
    raises_on("sumK2", lambda: sda.select_qgs(q, K, cid, proxies(sumK2=torch.zeros((B, Hkv, C, d - 1))), qc,
                                              4, 8, 10))
    raises_on("budget", lambda: sda.select_qgs(q, K, cid, st, qc, 4, 8, 10,
                                               budget=torch.zeros((B, Hkv, C + 1), dtype=torch.int32)))
    raises_on("idx", lambda: sda.select_qgs(q, K, cid, st, qc, 4, 8, 10, out=(
        torch.zeros((B, Hkv, 21), dtype=torch.int32), torch.zeros((B, Hkv), dtype=torch.int32),
        torch.zeros((B, Hkv, 22), dtype=torch.int32))))
    raises_on("U", lambda: sda.build_qgs_codes(K, torch.zeros((B, Hkv, d, sda.QGS_RANK - 1))))
    raises_on("V", lambda: sda.build_qgc_clusters(K, torch.zeros((B, Hkv, d, sda.QGC_RANK), dtype=torch.float64), 8))
    raises_on("GPU", lambda: sda.build_qgc_clusters(K, torch.zeros((B, Hkv, d, sda.QGC_RANK)), 8))
