"""Benchmark of sparse decode attention with a tail estimate on one MI355X.

Default: one decode step with count-aware mean proxies at batch 32, 32K
context, 1% read (32 query / 8 KV heads, d = 128, bf16; 328 listed rows and
32 cluster proxies per KV head).  Prints ONE JSON line.

* `value` is the gathered-row throughput (GB/s) of the decode step, inputs
  resident in HBM.  The timed region replays a HIP graph of `--steps`
  captured launches (one per step) between HIP events on the launch stream,
  so `ms_per_step` is the average launch duration on the GPU without host
  launch overhead.
* `roofline` relates the kernel's algorithmic bytes per launch to the 8 TB/s
  HBM peak; `traffic` comes from the committed rocprofv3 counter summary when
  it was taken on the current kernel source, else null.
* `cpu_baseline` times the fp64 CPU oracle on a bounded sample of the same
  workload.

To keep the 256 MB last-level cache from serving the rows, consecutive steps
read different copies of the KV cache and proxy state (standing in for the
other layers of a decode step); a copy comes back only after the other
copies have streamed several times the cache size.

The other hot-path rows (sampled tail at batch 8 / 64K, rank-1 prior at
batch 16 / 128K, the selector at batch 32 / 32K, the builders) are measured
too and reported under `secondary` (`--no-rows` skips them).  `--copy-calibration` runs only a plain 1 GiB device copy (the
reference kernel for scaling the HBM byte counters).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
COUNTERS = os.path.join(ROOT, "profiles", "counters.json")
KERNEL_SOURCES = ["long_context_sparse_gathered_amd/csrc/sda_attn.hip",
                  "long_context_sparse_gathered_amd/csrc/sda_device.hpp",
                  "long_context_sparse_gathered_amd/csrc/sda_kernels.hpp"]


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--copies", type=int, default=12, help="KV-cache copies rotated through (cache defeat)")
    ap.add_argument("--dense-steps", type=int, default=10)
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead of a graph replay")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--check-units", type=int, default=4, help="units checked against the oracle")
    ap.add_argument("--rows", action="store_true", default=True,
                    help="also measure the sampled, prior and selector rows and the builders (default)")
    ap.add_argument("--no-rows", dest="rows", action="store_false", help="the headline step only")
    ap.add_argument("--copy-calibration", action="store_true")
    return ap.parse_args()


def _timer():
    import torch
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def time_steps(step, steps: int, warmup: int, graph: bool) -> float:
    """Average milliseconds per call of step(i), i = 0..steps-1."""
    import torch
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        for i in range(warmup):
            step(i)
    torch.cuda.synchronize()
    e0, e1 = _timer()
    if graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(steps):
                step(i)
        g.replay()          # untimed replay (first-touch of the graph)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            e0.record(stream)
            g.replay()
            e1.record(stream)
    else:
        with torch.cuda.stream(stream):
            e0.record(stream)
            for i in range(steps):
                step(i)
            e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def to_dev(x, dev):
    import numpy as np
    import torch
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(x).to(dev)


def main():
    a = _args()
    if a.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {a.gpus}); this build has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from long_context_sparse_gathered_amd import sda, synth

    dev = torch.device("cuda:0")
    if a.copy_calibration:
        copy_calibration(dev)
        return

    w = synth.WORKLOADS["proxy_bf16_b32_n32k"]
    t0 = time.time()
    c = synth.make_case(w)
    print(f"# generated {w.name} in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    q, K, V = to_dev(c.q, dev), to_dev(c.K, dev), to_dev(c.V, dev)
    idx, cid, icl = to_dev(c.idx, dev), to_dev(c.cid, dev), to_dev(c.idx_cluster, dev)
    st = sda.build_tail_proxies(K, V, cid, w.C)
    torch.cuda.synchronize()

    # builder (once per request, off the per-step clock)
    ws_b = torch.empty(sda.workspace_bytes(sda.make_dims(K, w.Hq), sda.OP_BUILD_PROXIES, C=w.C), dtype=torch.uint8,
                       device=dev)
    build_ms = time_steps(lambda i: sda.build_tail_proxies(K, V, cid, w.C, ws=ws_b), 3, 1, graph=False)

    copies = [(K, V, st)]
    for _ in range(a.copies - 1):
        copies.append((K.clone(), V.clone(), sda.ProxyState(C=w.C, count=st.count.clone(),
                                                             sumK=st.sumK.clone(), sumV=st.sumV.clone())))
    out = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device=dev)
    lse = torch.empty((w.B, w.Hq), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def step(i):
        Kc, Vc, sc = copies[i % len(copies)]
        sda.sparse_decode_attn(q, Kc, Vc, idx, tail=sc, idx_cluster=icl, out=out, lse=lse)

    ms = time_steps(step, a.steps, a.warmup, graph=not a.no_graph)
    ms_eager = None if a.no_graph else time_steps(step, a.steps, 2, graph=False)

    # parity spot check of the timed configuration
    max_err = None
    if a.check_units > 0:
        from oracle import oracle
        step(0)
        torch.cuda.synchronize()
        got = out.cpu().double().numpy()
        errs = []
        rng = np.random.default_rng(0)
        for u in rng.choice(w.B * w.Hkv, size=a.check_units, replace=False):
            s, g = divmod(int(u), w.Hkv)
            uc = synth.unit_case(w, s, g)
            ref, _ = oracle.sparse_proxy_def(uc.q, uc.K, uc.V, uc.idx, uc.cid, w.C)
            o = got[s, g * w.G:(g + 1) * w.G]
            errs.append(float((np.abs(o - ref[0]).max(axis=-1) / np.abs(ref[0]).max(axis=-1)).max()))
        max_err = max(errs)

    # dense decode over the same tensors (speedup reference)
    dense_ms = None
    if not a.no_dense:
        ws_d = torch.empty(sda.workspace_bytes(sda.make_dims(K, w.Hq), sda.OP_DENSE), dtype=torch.uint8, device=dev)

        def dstep(i):
            Kc, Vc, _ = copies[i % len(copies)]
            sda.dense_decode_attn(q, Kc, Vc, out=out, lse=lse, ws=ws_d)
        dense_ms = time_steps(dstep, a.dense_steps, 2, graph=False)

    bytes_ = step_bytes(w)
    gbs = bytes_["gathered"] / (ms * 1e-3) / 1e9
    tot_gbs = bytes_["total"] / (ms * 1e-3) / 1e9

    traffic = None
    if os.path.exists(COUNTERS):
        cnt = json.load(open(COUNTERS))
        rec = cnt.get("sparse_proxy_b32_n32k")
        if rec and rec.get("kernel_source_sha") == kernel_source_sha():
            traffic = rec["hbm_bytes_per_launch"]

    cpu = None if a.no_cpu else cpu_baseline(w, c, a.cpu_seconds)
    secondary = measure_rows(a, dev) if a.rows else None

    res = {
        "metric": "sparse decode attn µs/step & HBM GB/s (% peak), B=32 n=32K 1% read",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms, 5),
        "us_per_step": round(ms * 1e3, 3),
        "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "total_gbs": round(tot_gbs, 1),
        "us_per_step_eager_launches": None if ms_eager is None else round(ms_eager * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded generator; stands in for RULER/LongBench decode at 32K)",
        "config": {"workload": f"B={w.B} Hq={w.Hq} Hkv={w.Hkv} d={w.d} {w.dtype} n={w.n} "
                               f"m={w.m} (4 sink + 64 local + {w.n_top} top-k) proxies C={w.C}",
                   "tail": "count-aware mean proxies", "kv_copies_rotated": a.copies,
                   "timing": "eager launches" if a.no_graph else "HIP graph replay of the timed steps"},
        "roofline": {"bound": "hbm", "achieved": round(tot_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(tot_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "sparse_unit_vt_kernel<4, proxy, 3>", "bytes_per_launch": bytes_["total"],
                     "bytes_breakdown": bytes_},
        "dense_us_per_step": None if dense_ms is None else round(dense_ms * 1e3, 2),
        "speedup_vs_dense": None if dense_ms is None else round(dense_ms / ms, 2),
        "proxy_build_us": round(build_ms * 1e3, 2),
        "max_rel_err_sampled_units": max_err,
        "cpu_baseline": cpu,
    }
    if secondary is not None:
        res["secondary"] = secondary
    print(json.dumps(res), flush=True)


def step_bytes(w, m=None, state_bytes=None):
    """Algorithmic HBM bytes of one decode step: the listed K/V rows, the list
    (position + per-entry cluster id), the tail state, q in, out and lse out."""
    units = w.B * w.Hkv
    m = w.m if m is None else m
    row = w.d * w.elem_bytes
    gathered = units * m * 2 * row
    listed = units * m * (4 + (4 if w.tail == "proxy" else 0))
    if state_bytes is None:
        state_bytes = units * w.C * (4 + 2 * w.d * 4) if w.tail == "proxy" else 0
    qo = w.B * w.Hq * (w.d * w.elem_bytes + w.d * 4 + 4)
    return {"gathered": gathered, "list": listed, "state": state_bytes, "q_out": qo,
            "total": gathered + listed + state_bytes + qo}


def cpu_baseline(w, c, seconds):
    """fp64 oracle, O(|I|) proxy path, on whole units of the same step."""
    from oracle import oracle
    threads = oracle.get_threads()
    sample_units = min(32, w.B * w.Hkv)
    B1 = sample_units // w.Hkv
    q, K, V, idx, cid = c.q[:B1], c.K[:B1], c.V[:B1], c.idx[:B1], c.cid[:B1]
    cnt, sK, sV = oracle.proxy_build(K, V, cid, w.C)
    t0 = time.time()
    reps = 0
    while True:
        oracle.sparse_proxy(q, K, V, idx, cid, w.C, cnt, sK, sV)
        reps += 1
        if time.time() - t0 > seconds:
            break
    dt = (time.time() - t0) / reps
    gathered = sample_units * w.m * 2 * w.d * w.elem_bytes
    step_s = dt * (w.B * w.Hkv) / sample_units
    return {"value": round(gathered / dt / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "us_per_step": round(step_s * 1e6, 1),
            "sample": f"{sample_units} of {w.B * w.Hkv} (sequence, KV head) units of the same step, "
                      f"O(|I|) proxy path from prebuilt fp64 cluster sums, {reps} repetitions"}


def measure_rows(a, dev):
    """Sampled tail (batch 8, 64K) and rank-1 prior (batch 16, 128K) decode
    steps, the prior build, and the selector (QGS + ErrorGate, batch 32, 32K)
    with its builders, each on its own synthetic workload."""
    import torch

    from long_context_sparse_gathered_amd import sda, synth
    out = {}

    # sampled tail
    w = synth.WORKLOADS["sampled_bf16_b8_n64k"]
    c = synth.make_case(w)
    q, K, V, idx = to_dev(c.q, dev), to_dev(c.K, dev), to_dev(c.V, dev), to_dev(c.idx, dev)
    ncopy = 6
    copies = [(K, V)] + [(K.clone(), V.clone()) for _ in range(ncopy - 1)]
    tail = sda.SampledTail(eps=w.eps, delta=w.delta, b0=w.b0, seed=w.sampler_seed, b_cap=0)
    o = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device=dev)
    ws = torch.empty(sda.workspace_bytes(sda.make_dims(K, w.Hq), sda.OP_SPARSE, sda.TAIL_SAMPLED, w.m), dtype=torch.uint8,
                     device=dev)
    sda.sparse_decode_attn(q, K, V, idx, tail=tail, out=o, ws=ws)
    torch.cuda.synchronize()
    b_sum = int(tail.b.sum().item())
    ms = time_steps(lambda i: sda.sparse_decode_attn(q, copies[i % ncopy][0], copies[i % ncopy][1], idx, tail=tail,
                                                     out=o, ws=ws), 50, 5, graph=not a.no_graph)
    units = w.B * w.Hkv
    rows = units * (w.m + w.b0) * 2 + b_sum * 2
    by = rows * w.d * w.elem_bytes + units * w.m * 4 + w.B * w.Hq * (w.d * 2 + w.d * 4 + 4)
    out["sampled_b8_n64k"] = {"us_per_step": round(ms * 1e3, 2), "mean_budget_b": round(b_sum / units, 1),
                              "bytes_per_step": by, "gbs": round(by / (ms * 1e-3) / 1e9, 1),
                              "frac_hbm_peak": round(by / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    del copies, K, V, c
    torch.cuda.empty_cache()

    # rank-1 prior
    w = synth.WORKLOADS["prior_bf16_b16_n128k"]
    c = synth.make_case(w)
    q, K, V, idx, muQ = (to_dev(x, dev) for x in (c.q, c.K, c.V, c.idx, c.mu_Q))
    ws_p = torch.empty(sda.workspace_bytes(sda.make_dims(K, w.Hq), sda.OP_BUILD_PRIOR), dtype=torch.uint8, device=dev)
    build_ms = time_steps(lambda i: sda.build_prior(K, V, muQ, ws=ws_p), 3, 1, graph=False)
    ps = sda.build_prior(K, V, muQ, ws=ws_p)
    ncopy = 3
    copies = [(K, V)] + [(K.clone(), V.clone()) for _ in range(ncopy - 1)]
    o = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, sda.workspace_bytes(sda.make_dims(K, w.Hq), sda.OP_SPARSE, sda.TAIL_PRIOR, w.m)),
                     dtype=torch.uint8, device=dev)
    ms_p = time_steps(lambda i: sda.sparse_decode_attn(q, copies[i % ncopy][0], copies[i % ncopy][1], idx, tail=ps,
                                                       out=o, ws=ws), 50, 5, graph=not a.no_graph)
    ms_none = time_steps(lambda i: sda.sparse_decode_attn(q, copies[i % ncopy][0], copies[i % ncopy][1], idx, out=o,
                                                          ws=ws), 50, 5, graph=not a.no_graph)
    units = w.B * w.Hkv
    state = w.B * w.Hq * (w.d * 4 * 2 + 8) + units * w.d * 4
    by = units * w.m * (2 * w.d * w.elem_bytes + 4) + state + w.B * w.Hq * (w.d * 2 + w.d * 4 + 4)
    dense_by = units * w.n * 2 * w.d * w.elem_bytes
    out["prior_b16_n128k"] = {"us_per_step": round(ms_p * 1e3, 2), "no_tail_us_per_step": round(ms_none * 1e3, 2),
                              "prior_overhead_pct": round(100 * (ms_p / ms_none - 1), 2),
                              "bytes_per_step": by, "gbs": round(by / (ms_p * 1e-3) / 1e9, 1),
                              "frac_hbm_peak": round(by / (ms_p * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                              "build_prior_us": round(build_ms * 1e3, 1),
                              "build_prior_gbs": round(dense_by / (build_ms * 1e-3) / 1e9, 1)}
    del copies, K, V, c, ps
    torch.cuda.empty_cache()

    # the selector in front of the proxy decode (QGS codes + ErrorGate + per-cluster top-q)
    w = synth.WORKLOADS["qgs_bf16_b32_n32k"]
    c = synth.make_case(w)
    q, K, V, U, cid = (to_dev(x, dev) for x in (c.q, c.K, c.V, c.U, c.cid))
    ws_b = torch.empty(sda.workspace_bytes(sda.make_dims(K, w.Hq), sda.OP_BUILD_PROXIES, C=w.C), dtype=torch.uint8,
                       device=dev)
    pbuild_ms = time_steps(lambda i: sda.build_tail_proxies(K, V, cid, w.C, ws=ws_b, with_sumK2=True), 3, 1,
                           graph=False)
    st = sda.build_tail_proxies(K, V, cid, w.C, ws=ws_b, with_sumK2=True)
    ws_c = torch.empty(sda.workspace_bytes(sda.make_dims(K, w.Hq), sda.OP_BUILD_QGS), dtype=torch.uint8, device=dev)
    cbuild_ms = time_steps(lambda i: sda.build_qgs_codes(K, U, ws=ws_c), 3, 1, graph=False)
    qc = sda.build_qgs_codes(K, U, ws=ws_c)
    del V
    ncopy = 2
    copies = [(qc, cid)] + [(sda.QgsCodes(U=U, codes=qc.codes.clone(), kmax=qc.kmax), cid.clone())
                            for _ in range(ncopy - 1)]
    units = w.B * w.Hkv
    outs = (torch.empty((w.B, w.Hkv, w.m), dtype=torch.int32, device=dev),
            torch.empty((w.B, w.Hkv), dtype=torch.int32, device=dev),
            torch.empty((w.B, w.Hkv, w.m), dtype=torch.int32, device=dev))
    ws = torch.empty(sda.workspace_bytes(sda.make_dims(K, w.Hq), sda.OP_SELECT_QGS, C=w.C), dtype=torch.uint8,
                     device=dev)
    ms_s = time_steps(lambda i: sda.select_qgs(q, K, copies[i % ncopy][1], st, copies[i % ncopy][0], w.n_sink,
                                               w.n_local, w.n_top, out=outs, ws=ws), 50, 5, graph=not a.no_graph)
    per_unit = (w.n * (w.r + 4) + w.C * (4 + 2 * w.d * 4) + w.d * w.r * 4 + w.r * 8 + w.m * 8 + 4)
    by = units * per_unit + w.B * w.Hq * w.d * w.elem_bytes
    # query-geometry clustering (C = 64, 10 passes) and the selector on its clusters
    V16 = U[..., :sda.QGC_RANK].contiguous()
    ws_q = torch.empty(sda.workspace_bytes(sda.make_dims(K, w.Hq), sda.OP_BUILD_QGC, C=64), dtype=torch.uint8,
                       device=dev)
    qgc_ms = time_steps(lambda i: sda.build_qgc_clusters(K, V16, 64, T=10, ws=ws_q), 3, 1, graph=False)
    cid64 = sda.build_qgc_clusters(K, V16, 64, T=10, ws=ws_q)
    del ws_q
    Vfull = to_dev(c.V, dev)
    st64 = sda.build_tail_proxies(K, Vfull, cid64, 64, with_sumK2=True)
    del Vfull
    ws64 = torch.empty(sda.workspace_bytes(sda.make_dims(K, w.Hq), sda.OP_SELECT_QGS, C=64), dtype=torch.uint8,
                       device=dev)
    ms_s64 = time_steps(lambda i: sda.select_qgs(q, K, cid64, st64, copies[i % ncopy][0], w.n_sink, w.n_local,
                                                 w.n_top, out=outs, ws=ws64), 50, 5, graph=not a.no_graph)
    out["qgs_select_b32_n32k"] = {"us_per_step": round(ms_s * 1e3, 2), "bytes_per_step": by,
                                  "gbs": round(by / (ms_s * 1e-3) / 1e9, 1),
                                  "frac_hbm_peak": round(by / (ms_s * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                  "rows_scored": units * w.n, "rows_picked": units * w.n_top,
                                  "build_codes_us": round(cbuild_ms * 1e3, 1),
                                  "build_proxies_with_sq_us": round(pbuild_ms * 1e3, 1),
                                  "qgc_clusters_c64_t10_us": round(qgc_ms * 1e3, 1),
                                  "us_per_step_on_qgc_c64": round(ms_s64 * 1e3, 2)}
    return out


def copy_calibration(dev):
    """A plain device-to-device copy of 1 GiB, five times: the kernel whose
    FETCH_SIZE / WRITE_SIZE per dispatch calibrate the byte counters."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev)
    src.fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "copies": 5}), flush=True)


if __name__ == "__main__":
    main()
