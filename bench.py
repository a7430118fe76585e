"""Benchmark of sparse decode attention with a tail estimate on one MI355X.

Default: one decode step with count-aware mean proxies at batch 32, 32K
context, 1% read (32 query / 8 KV heads, d = 128, bf16; 328 listed rows and
32 cluster proxies per KV head).  Prints ONE JSON line.

* `value` is the gathered-row throughput (GB/s) of the decode step, inputs
  resident in HBM.  A timed pass replays a HIP graph of `--steps` captured
  launches (one per step) between HIP events on the launch stream; the
  reported time per step is the median of `--repeats` such passes.
* `roofline` relates the kernel's algorithmic bytes per launch to the 8 TB/s
  HBM peak; `traffic` comes from the committed rocprofv3 counter summary when
  it was taken on the current kernel source, else null.
* `gather_ceiling` times a plain gather of the same rows and proxy state in
  the decode kernel's launch shape (one 8-wave workgroup per unit), with no
  arithmetic: the floor that launch shape puts under the step.
* `cpu_baseline` times the fp64 CPU oracle on a bounded sample of the same
  workload; `cpu_oracle` times each tail's oracle path at all host threads
  and at one thread.
* `configs` holds one line per measured workload: the single-head fp32
  correctness case, batch 1, the headline shape at 3% read (lists longer
  than the one-pass kernel holds), the sampled tail (batch 8, 64K), the rank-1
  prior (batch 16, 128K) and the selector (batch 32, 32K), each with
  µs/step, gathered and total GB/s, the dense speedup, the max relative
  error against the oracle and, where the path computes integers, bit-exact
  flags.  `--no-rows` skips them.

To keep the 256 MB last-level cache from serving the rows, consecutive steps
read different copies of the KV cache and tail state (standing in for the
other layers of a decode step); a copy comes back only after the other
copies have streamed several times the cache size.

`--gather-ceiling` prints only the gather timings (several launch shapes);
`--copy-calibration` runs only a plain 1 GiB device copy (the reference
kernel for scaling the HBM byte counters).
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
    ap.add_argument("--repeats", type=int, default=5, help="timed passes; the median is reported")
    ap.add_argument("--copies", type=int, default=12, help="KV-cache copies rotated through (cache defeat)")
    ap.add_argument("--dense-steps", type=int, default=10)
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead of a graph replay")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--path-seconds", type=float, default=2.0, help="CPU time per oracle path and thread count")
    ap.add_argument("--check-units", type=int, default=4, help="units checked against the oracle")
    ap.add_argument("--rows", action="store_true", default=True,
                    help="also measure the other workloads and the builders (default)")
    ap.add_argument("--no-rows", dest="rows", action="store_false", help="the headline step only")
    ap.add_argument("--gather-ceiling", action="store_true", help="only the plain-gather timings")
    ap.add_argument("--copy-calibration", action="store_true")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# timing and checking helpers

def time_steps(step, steps: int, warmup: int, graph: bool, repeats: int = 5):
    """Milliseconds per call of step(i), i = 0..steps-1: (median over
    `repeats` timed passes, every pass's figure)."""
    import numpy as np
    import torch
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        for i in range(warmup):
            step(i)
    torch.cuda.synchronize()
    per = []
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(steps):
                step(i)
        g.replay()          # untimed replay (first-touch of the graph)
        torch.cuda.synchronize()
        for _ in range(repeats):
            with torch.cuda.stream(stream):
                e0.record(stream)
                g.replay()
                e1.record(stream)
            torch.cuda.synchronize()
            per.append(e0.elapsed_time(e1) / steps)
        del g
    else:
        for _ in range(repeats):
            with torch.cuda.stream(stream):
                e0.record(stream)
                for i in range(steps):
                    step(i)
                e1.record(stream)
            torch.cuda.synchronize()
            per.append(e0.elapsed_time(e1) / steps)
    return float(np.median(per)), per


def to_dev(x, dev):
    import numpy as np
    import torch
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev)


def rel_err(got, ref) -> float:
    """max over (seq, head) rows of max |o - o*| / max |o*|."""
    import numpy as np
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.abs(ref).max(axis=-1)
    den = np.where(den > 0, den, 1.0)
    return float((np.abs(got - ref).max(axis=-1) / den).max())


def timed_cpu(fn, seconds: float):
    """(seconds per call, calls) of fn, repeated for at least `seconds`."""
    t0 = time.time()
    reps = 0
    while True:
        fn()
        reps += 1
        if time.time() - t0 > seconds:
            break
    return (time.time() - t0) / reps, reps


def oracle_path(name, fn, gathered_bytes, units_sampled, units_step, seconds, note):
    """One oracle path timed at all host threads and at one thread."""
    from oracle import oracle
    nmax = oracle.get_threads()
    rec = {"sample": note, "units_sampled": units_sampled}
    for th in (nmax, 1):
        oracle.set_threads(th)
        dt, reps = timed_cpu(fn, seconds)
        key = "all_threads" if th == nmax else "one_thread"
        rec[key] = {"threads": th, "ms_per_call": round(dt * 1e3, 3), "repetitions": reps,
                    "us_per_step": round(dt * units_step / units_sampled * 1e6, 1),
                    "gathered_gbs": None if gathered_bytes is None else round(gathered_bytes / dt / 1e9, 3)}
    oracle.set_threads(nmax)
    return name, rec


def line(ms, gathered, total, dense_ms=None, **extra):
    r = {"us_per_step": round(ms * 1e3, 3), "gathered_bytes": gathered,
         "gathered_gbs": None if gathered is None else round(gathered / (ms * 1e-3) / 1e9, 1),
         "pct_hbm_peak_gathered": None if gathered is None else round(100 * gathered / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
         "total_bytes": total, "total_gbs": round(total / (ms * 1e-3) / 1e9, 1),
         "frac_hbm_peak_total": round(total / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    if dense_ms is not None:
        r["dense_us_per_step"] = round(dense_ms * 1e3, 2)
        r["speedup_vs_dense"] = round(dense_ms / ms, 2)
    r.update(extra)
    return r


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


def dense_time(dev, q, copies, Hq, steps, out, lse):
    import torch

    from long_context_sparse_gathered_amd import sda
    K0 = copies[0][0]
    ws = torch.empty(max(1, sda.workspace_bytes(sda.make_dims(K0, Hq), sda.OP_DENSE)), dtype=torch.uint8, device=dev)

    def dstep(i):
        Kc, Vc = copies[i % len(copies)][:2]
        sda.dense_decode_attn(q, Kc, Vc, out=out, lse=lse, ws=ws)
    ms, _ = time_steps(dstep, steps, 2, graph=False, repeats=3)
    return ms


# ---------------------------------------------------------------------------
# the headline step (batch 32, 32K, 1% read) and its 3% variant

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
    units = w.B * w.Hkv
    state_words = w.C * (1 + 2 * w.d)      # count + sumK + sumV per unit, 4-byte words

    copies = [(K, V, st)]
    for _ in range(a.copies - 1):
        copies.append((K.clone(), V.clone(), sda.ProxyState(C=w.C, count=st.count.clone(),
                                                             sumK=st.sumK.clone(), sumV=st.sumV.clone())))
    gstate = [torch.zeros((units, state_words), dtype=torch.int32, device=dev) for _ in copies]
    torch.cuda.synchronize()

    if a.gather_ceiling:
        res = {"gather_ceiling": {}}
        for waves, parts in [(8, 1), (4, 1), (16, 1), (8, 2), (4, 2)]:
            res["gather_ceiling"][f"{waves}w_x{parts}"] = gather_ceiling(a, copies, gstate, idx, w, waves, parts)
        print(json.dumps(res), flush=True)
        return

    # builder (once per request, off the per-step clock)
    ws_b = torch.empty(sda.workspace_bytes(sda.make_dims(K, w.Hq), sda.OP_BUILD_PROXIES, C=w.C), dtype=torch.uint8,
                       device=dev)
    build_ms, _ = time_steps(lambda i: sda.build_tail_proxies(K, V, cid, w.C, ws=ws_b), 3, 1, graph=False, repeats=1)
    del ws_b

    out = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device=dev)
    lse = torch.empty((w.B, w.Hq), dtype=torch.float32, device=dev)

    def step(i):
        Kc, Vc, sc = copies[i % len(copies)]
        sda.sparse_decode_attn(q, Kc, Vc, idx, tail=sc, idx_cluster=icl, out=out, lse=lse)

    ms, per = time_steps(step, a.steps, a.warmup, graph=not a.no_graph, repeats=a.repeats)
    ms_eager = None if a.no_graph else time_steps(step, a.steps, 2, graph=False, repeats=1)[0]

    # parity spot check of the timed configuration, and two runs bit for bit
    max_err = None
    twice_equal = None
    check_units = []
    if a.check_units > 0:
        from oracle import oracle
        step(0)
        torch.cuda.synchronize()
        got = out.cpu().double().numpy()
        first = (out.clone(), lse.clone())
        step(0)
        torch.cuda.synchronize()
        twice_equal = bool(torch.equal(first[0], out) and torch.equal(first[1], lse))
        errs = []
        rng = np.random.default_rng(0)
        for u in rng.choice(units, size=a.check_units, replace=False):
            s, g = divmod(int(u), w.Hkv)
            check_units.append(int(u))
            uc = synth.unit_case(w, s, g)
            ref, _ = oracle.sparse_proxy_def(uc.q, uc.K, uc.V, uc.idx, uc.cid, w.C)
            errs.append(rel_err(got[s, g * w.G:(g + 1) * w.G], ref[0]))
        max_err = max(errs)

    dense_ms = None if a.no_dense else dense_time(dev, q, copies, w.Hq, a.dense_steps, out, lse)
    ceiling = gather_ceiling(a, copies, gstate, idx, w, 8, 1)

    bytes_ = step_bytes(w)
    gbs = bytes_["gathered"] / (ms * 1e-3) / 1e9
    tot_gbs = bytes_["total"] / (ms * 1e-3) / 1e9

    traffic = None
    if os.path.exists(COUNTERS):
        cnt = json.load(open(COUNTERS))
        rec = cnt.get("sparse_proxy_b32_n32k")
        if rec and rec.get("kernel_source_sha") == kernel_source_sha():
            traffic = rec["hbm_bytes_per_launch"]

    configs = {}
    cpu_paths = {}
    if a.rows:
        configs["C3_3pct_proxy_bf16_b32_n32k"] = measure_three_percent(a, dev, w, c, q, copies, out, lse, dense_ms)
    del copies, gstate
    torch.cuda.empty_cache()

    cpu = None
    if not a.no_cpu:
        cpu = cpu_baseline(w, c, a.cpu_seconds)
        from oracle import oracle
        B1 = 2
        cnt_, sK_, sV_ = oracle.proxy_build(c.K[:B1], c.V[:B1], c.cid[:B1], w.C)
        name, rec = oracle_path(
            "proxy_o_of_I", lambda: oracle.sparse_proxy(c.q[:B1], c.K[:B1], c.V[:B1], c.idx[:B1], c.cid[:B1], w.C,
                                                        cnt_, sK_, sV_),
            B1 * w.Hkv * w.m * 2 * w.d * w.elem_bytes, B1 * w.Hkv, units, a.path_seconds,
            f"{B1 * w.Hkv} units of the batch-32 32K 1% step, O(|I|) proxy path from prebuilt fp64 cluster sums")
        cpu_paths[name] = rec
    del c

    if a.rows:
        configs.update(measure_small_configs(a, dev))
        rows_out, paths = measure_rows(a, dev)
        configs.update(rows_out)
        cpu_paths.update(paths)

    res = {
        "metric": "sparse decode attn µs/step & HBM GB/s (% peak), B=32 n=32K 1% read",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms, 5),
        "us_per_step": round(ms * 1e3, 3),
        "repeats_us_per_step": [round(x * 1e3, 3) for x in per],
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
                   "timing": ("eager launches" if a.no_graph else "HIP graph replay of the timed steps")
                             + f", median of {a.repeats} passes"},
        "roofline": {"bound": "hbm", "achieved": round(tot_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(tot_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "sparse_unit_vt_kernel<4, proxy, 3>", "bytes_per_launch": bytes_["total"],
                     "bytes_breakdown": bytes_},
        "gather_ceiling": ceiling,
        "dense_us_per_step": None if dense_ms is None else round(dense_ms * 1e3, 2),
        "speedup_vs_dense": None if dense_ms is None else round(dense_ms / ms, 2),
        "proxy_build_us": round(build_ms * 1e3, 2),
        "max_rel_err_sampled_units": max_err,
        "units_checked": check_units,
        "run_twice_bit_equal": twice_equal,
        "cpu_baseline": cpu,
        "cpu_oracle": cpu_paths or None,
    }
    if configs:
        res["configs"] = configs
    print(json.dumps(res), flush=True)


def gather_ceiling(a, copies, gstate, idx, w, waves, parts):
    """A plain gather of the listed K/V rows and each unit's proxy state, no
    arithmetic, in the given launch shape (`waves` waves per workgroup,
    `parts` workgroups per unit)."""
    import torch

    from long_context_sparse_gathered_amd import sda
    units = w.B * w.Hkv
    chk = torch.zeros(units * parts * waves, dtype=torch.int32, device=copies[0][0].device)

    def gstep(i):
        j = i % len(copies)
        sda.gather_rows(copies[j][0], copies[j][1], idx, waves=waves, parts=parts, state=gstate[j], checksum=chk)
    ms, _ = time_steps(gstep, a.steps, a.warmup, graph=not a.no_graph, repeats=a.repeats)
    by = units * w.m * 2 * w.d * w.elem_bytes
    st = gstate[0].numel() * gstate[0].element_size()
    return {"shape": f"{waves} waves x {parts} workgroup(s) per unit", "us_per_step": round(ms * 1e3, 3),
            "gathered_gbs": round(by / (ms * 1e-3) / 1e9, 1),
            "total_gbs": round((by + st) / (ms * 1e-3) / 1e9, 1)}


def draws_gather_ceiling(a, copies, b_sum, slices=32, waves=8):
    """A plain gather of as many uniformly random K/V rows as the sampled
    tail's fresh draws read (b_sum row pairs spread over the whole cache), no
    arithmetic: each (sequence, KV head) range of n rows is cut into `slices`
    slices of n/slices rows, and every slice is a unit of the gather aid with
    the same number of random rows (one workgroup of `waves` waves each)."""
    import numpy as np
    import torch

    from long_context_sparse_gathered_amd import sda
    K0 = copies[0][0]
    B, Hkv, n, d = K0.shape
    if not K0.is_contiguous() or n % slices:
        return None
    H2, n2 = Hkv * slices, n // slices
    units = B * H2
    m = -(-b_sum // units)
    if m > waves * 4 * (12 if waves == 16 else 24):
        return None
    rng = np.random.default_rng(7)
    idx = torch.from_numpy(rng.integers(0, n2, size=(B, H2, m), dtype=np.int32)).to(K0.device)
    views = [(K.view(B, H2, n2, d), V.view(B, H2, n2, d)) for K, V in copies]
    chk = torch.zeros(units * waves, dtype=torch.int32, device=K0.device)

    def gstep(i):
        Kv, Vv = views[i % len(views)]
        sda.gather_rows(Kv, Vv, idx, waves=waves, parts=1, checksum=chk)
    ms, _ = time_steps(gstep, 50, 5, graph=not a.no_graph, repeats=a.repeats)
    by = units * m * 2 * d * K0.element_size()
    return {"shape": f"{units} slices of {n2} rows, {m} random rows each, {waves} waves x 1 workgroup per slice",
            "us": round(ms * 1e3, 3), "gathered_gbs": round(by / (ms * 1e-3) / 1e9, 1)}


def measure_three_percent(a, dev, w, c, q, copies, out, lse, dense_ms):
    """The headline shape at 3% read (984 listed rows per KV head): the proxy
    tail on the long-list kernel, over the same KV-cache copies."""
    import numpy as np
    import torch

    from long_context_sparse_gathered_amd import sda, synth
    from oracle import oracle
    n_top = int(np.ceil(w.n * 0.03 - 1e-9)) - w.n_sink - w.n_local
    w3 = w.replace(n_top=n_top)
    idx3 = synth.index_sets(c, n_top)
    icl3 = np.take_along_axis(c.cid, idx3.astype(np.int64), axis=2).astype(np.int32)
    idx_d, icl_d = to_dev(idx3, dev), to_dev(icl3, dev)
    ws = torch.empty(max(1, sda.workspace_bytes(sda.make_dims(copies[0][0], w.Hq), sda.OP_SPARSE, sda.TAIL_PROXY,
                                                w3.m, w.C)), dtype=torch.uint8, device=dev)

    def step(i):
        Kc, Vc, sc = copies[i % len(copies)]
        sda.sparse_decode_attn(q, Kc, Vc, idx_d, tail=sc, idx_cluster=icl_d, out=out, lse=lse, ws=ws)
    ms, per = time_steps(step, 100, 10, graph=not a.no_graph, repeats=a.repeats)
    step(0)
    torch.cuda.synchronize()
    got = out.cpu().double().numpy()
    errs = []
    rng = np.random.default_rng(1)
    for u in rng.choice(w.B * w.Hkv, size=max(1, a.check_units), replace=False):
        s, g = divmod(int(u), w.Hkv)
        uc = synth.unit_case(w3, s, g)
        assert np.array_equal(uc.idx[0, 0], idx3[s, g])
        ref, _ = oracle.sparse_proxy_def(uc.q, uc.K, uc.V, uc.idx, uc.cid, w.C)
        errs.append(rel_err(got[s, g * w.G:(g + 1) * w.G], ref[0]))
    by = step_bytes(w3)
    return line(ms, by["gathered"], by["total"], dense_ms, m=w3.m, path="one workgroup per unit, value rows requested as the key tiles are consumed",
                repeats_us=[round(x * 1e3, 3) for x in per], max_rel_err=max(errs), units_checked=len(errs))


# ---------------------------------------------------------------------------
# the small correctness configurations

def measure_small_configs(a, dev):
    """C1 (single head, fp32, 4K, cache-resident and launch-bound) and C2
    (batch 1, 32K, bf16) with the full oracle on every unit."""
    import torch

    from long_context_sparse_gathered_amd import sda, synth
    from oracle import oracle
    res = {}
    for key, wname, ncopy in [("C1_proxy_f32_b1_n4k", "proxy_f32_b1_n4k", 1),
                              ("C2_proxy_bf16_b1_n32k", "proxy_bf16_b1_n32k", 12)]:
        w = synth.WORKLOADS[wname]
        c = synth.make_case(w)
        q, K, V = to_dev(c.q, dev), to_dev(c.K, dev), to_dev(c.V, dev)
        cid, icl, idx = to_dev(c.cid, dev), to_dev(c.idx_cluster, dev), to_dev(c.idx, dev)
        st = sda.build_tail_proxies(K, V, cid, w.C)
        copies = [(K, V, st)] + [(K.clone(), V.clone(), sda.ProxyState(C=w.C, count=st.count.clone(),
                                                                       sumK=st.sumK.clone(), sumV=st.sumV.clone()))
                                 for _ in range(ncopy - 1)]
        out = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device=dev)
        lse = torch.empty((w.B, w.Hq), dtype=torch.float32, device=dev)

        def step(i):
            Kc, Vc, sc = copies[i % len(copies)]
            sda.sparse_decode_attn(q, Kc, Vc, idx, tail=sc, idx_cluster=icl, out=out, lse=lse)
        ms, per = time_steps(step, a.steps, a.warmup, graph=not a.no_graph, repeats=a.repeats)
        step(0)
        torch.cuda.synchronize()
        ref, _ = oracle.sparse_proxy_def(c.q, c.K, c.V, c.idx, c.cid, w.C)
        err = rel_err(out.cpu().double().numpy(), ref)
        dms = None if a.no_dense else dense_time(dev, q, copies, w.Hq, 20, out, lse)
        by = step_bytes(w)
        res[key] = line(ms, by["gathered"], by["total"], dms, m=w.m, dtype=w.dtype,
                        repeats_us=[round(x * 1e3, 3) for x in per], max_rel_err=err,
                        tolerance=1e-5 if w.dtype == "f32" else 2e-3, units_checked=w.B * w.Hkv,
                        note="latency-bound: the rows fit in the last-level cache" if ncopy == 1 else
                        f"{ncopy} KV copies rotated")
        del copies, K, V, st
        torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------------------
# the other tails and the selector

def measure_rows(a, dev):
    """Sampled tail (batch 8, 64K) and rank-1 prior (batch 16, 128K) decode
    steps, the prior build, and the selector (QGS + ErrorGate, batch 32, 32K)
    with its builders, each on its own synthetic workload; returns the lines
    and the oracle timings of those paths."""
    import numpy as np
    import torch

    from long_context_sparse_gathered_amd import sda, synth
    from oracle import oracle
    out = {}
    paths = {}

    # sampled tail ------------------------------------------------------------
    w = synth.WORKLOADS["sampled_bf16_b8_n64k"]
    c = synth.make_case(w)
    q, K, V, idx = to_dev(c.q, dev), to_dev(c.K, dev), to_dev(c.V, dev), to_dev(c.idx, dev)
    ncopy = 6
    copies = [(K, V)] + [(K.clone(), V.clone()) for _ in range(ncopy - 1)]
    tail = sda.SampledTail(eps=w.eps, delta=w.delta, b0=w.b0, seed=w.sampler_seed, b_cap=0)
    o = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device=dev)
    lse = torch.empty((w.B, w.Hq), dtype=torch.float32, device=dev)
    ws = torch.empty(sda.workspace_bytes(sda.make_dims(K, w.Hq), sda.OP_SPARSE, sda.TAIL_SAMPLED, w.m), dtype=torch.uint8,
                     device=dev)
    sda.sparse_decode_attn(q, K, V, idx, tail=tail, out=o, ws=ws)
    torch.cuda.synchronize()
    b_sum = int(tail.b.sum().item())
    ms, per = time_steps(lambda i: sda.sparse_decode_attn(q, copies[i % ncopy][0], copies[i % ncopy][1], idx,
                                                          tail=tail, out=o, ws=ws), 50, 5, graph=not a.no_graph,
                         repeats=a.repeats)
    # every unit's budget and drawn positions against the oracle
    b_cap = w.n
    chk = sda.SampledTail(eps=w.eps, delta=w.delta, b0=w.b0, seed=w.sampler_seed, b_cap=b_cap)
    sda.sparse_decode_attn(q, K, V, idx, tail=chk, out=o, lse=lse, ws=ws)
    torch.cuda.synchronize()
    ref = oracle.sampled(c.q, c.K, c.V, c.idx, w.eps, w.z, w.b0, w.sampler_seed, b_cap)
    b_gpu = chk.b.cpu().numpy()
    r = np.round(ref["bstar"])
    ties = int(((np.abs(ref["bstar"] - r) < 1e-9 * np.maximum(ref["bstar"], 1.0)) & (r >= 1)).sum())
    b_exact = bool(np.array_equal(b_gpu, ref["b"]))
    samp = chk.samples.cpu().numpy()
    draws_exact = b_exact and all(np.array_equal(samp[s, g, :int(ref["b"][s, g])],
                                                 ref["samples"][s, g, :int(ref["b"][s, g])])
                                  for s in range(w.B) for g in range(w.Hkv))
    err = rel_err(o.cpu().double().numpy(), ref["out"])
    # the verified budget (eps and delta bound the output; the smallest budget
    # over 31 splits of delta): timed on the same step, budgets and draws
    # of every unit against the oracle's verified estimator
    vt = sda.SampledTail(eps=w.eps, delta=w.delta, b0=w.b0, seed=w.sampler_seed, b_cap=b_cap, verified=True)
    sda.sparse_decode_attn(q, K, V, idx, tail=vt, out=o, lse=lse, ws=ws)
    torch.cuda.synchronize()
    vref = oracle.sampled_verified(c.q, c.K, c.V, c.idx, w.eps, vt.z_split, w.b0, w.sampler_seed, b_cap)
    vb = vt.b.cpu().numpy()
    vsamp = vt.samples.cpu().numpy()
    v_exact = bool(np.array_equal(vb, vref["b"])) and all(
        np.array_equal(vsamp[s, g, :int(vb[s, g])], vref["samples"][s, g, :int(vb[s, g])])
        for s in range(w.B) for g in range(w.Hkv))
    v_err = rel_err(o.cpu().double().numpy(), vref["out"])
    vtime = sda.SampledTail(eps=w.eps, delta=w.delta, b0=w.b0, seed=w.sampler_seed, b_cap=0, verified=True)
    vms, vper = time_steps(lambda i: sda.sparse_decode_attn(q, copies[i % ncopy][0], copies[i % ncopy][1], idx,
                                                            tail=vtime, out=o, ws=ws), 20, 3, graph=not a.no_graph,
                           repeats=a.repeats)
    verified = {"us_per_step": round(vms * 1e3, 3), "mean_budget_b": round(float(vb.mean()), 1),
                "units_reading_whole_tail": int((vb >= w.n - w.m).sum()),
                "budget_and_draws_bit_exact": v_exact, "max_rel_err": v_err,
                "note": "eps = delta = 0.05 on the attention output (Lemma 4.2 + Theorem 4.3 allocation)"}
    del vref, vsamp
    dms = None if a.no_dense else dense_time(dev, q, copies, w.Hq, 5, o, lse)
    units = w.B * w.Hkv
    rows = units * (w.m + w.b0) * 2 + b_sum * 2
    gathered = rows * w.d * w.elem_bytes
    by = gathered + units * w.m * 4 + w.B * w.Hq * (w.d * 2 + w.d * 4 + 4)
    out["C4_sampled_bf16_b8_n64k"] = line(
        ms, gathered, by, dms, m=w.m, mean_budget_b=round(b_sum / units, 1),
        repeats_us=[round(x * 1e3, 3) for x in per], max_rel_err=err, units_checked=units,
        budget_bit_exact=b_exact, draws_bit_exact=draws_exact, budget_ties=ties,
        draws_gather_ceiling=draws_gather_ceiling(a, copies, b_sum), verified_budget=verified,
        note="gathered = I_f, the b0 base draws and the b fresh draws (K and V rows)")
    B1 = 2
    name, rec = oracle_path(
        "sampled", lambda: oracle.sampled(c.q[:B1], c.K[:B1], c.V[:B1], c.idx[:B1], w.eps, w.z, w.b0,
                                          w.sampler_seed, 0),
        None, B1 * w.Hkv, units, a.path_seconds,
        f"{B1 * w.Hkv} units of the batch-8 64K step: exact part, base draws, budget, fresh draws")
    paths[name] = rec
    del copies, K, V, c, chk
    torch.cuda.empty_cache()

    # rank-1 prior ------------------------------------------------------------
    w = synth.WORKLOADS["prior_bf16_b16_n128k"]
    c = synth.make_case(w)
    q, K, V, idx, muQ = (to_dev(x, dev) for x in (c.q, c.K, c.V, c.idx, c.mu_Q))
    ws_p = torch.empty(sda.workspace_bytes(sda.make_dims(K, w.Hq), sda.OP_BUILD_PRIOR), dtype=torch.uint8, device=dev)
    build_ms, _ = time_steps(lambda i: sda.build_prior(K, V, muQ, ws=ws_p), 3, 1, graph=False, repeats=1)
    ps = sda.build_prior(K, V, muQ, ws=ws_p)
    ncopy = 3
    copies = [(K, V)] + [(K.clone(), V.clone()) for _ in range(ncopy - 1)]
    o = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device=dev)
    lse = torch.empty((w.B, w.Hq), dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, sda.workspace_bytes(sda.make_dims(K, w.Hq), sda.OP_SPARSE, sda.TAIL_PRIOR, w.m)),
                     dtype=torch.uint8, device=dev)
    ms_p, per = time_steps(lambda i: sda.sparse_decode_attn(q, copies[i % ncopy][0], copies[i % ncopy][1], idx,
                                                            tail=ps, out=o, ws=ws), 50, 5, graph=not a.no_graph,
                           repeats=a.repeats)
    ms_none, _ = time_steps(lambda i: sda.sparse_decode_attn(q, copies[i % ncopy][0], copies[i % ncopy][1], idx,
                                                             out=o, ws=ws), 50, 5, graph=not a.no_graph,
                            repeats=a.repeats)
    sda.sparse_decode_attn(q, K, V, idx, tail=ps, out=o, lse=lse, ws=ws)
    torch.cuda.synchronize()
    got = o.cpu().double().numpy()
    errs = []
    rng = np.random.default_rng(2)
    units = w.B * w.Hkv
    for u in rng.choice(units, size=max(1, a.check_units), replace=False):
        s, g = divmod(int(u), w.Hkv)
        uc = synth.unit_case(w, s, g)
        ref, _ = oracle.sparse_prior_def(uc.q, uc.K, uc.V, uc.idx, uc.mu_Q, w.lam)
        errs.append(rel_err(got[s, g * w.G:(g + 1) * w.G], ref[0]))
    dms = None if a.no_dense else dense_time(dev, q, copies, w.Hq, 3, o, lse)
    state = w.B * w.Hq * (w.d * 4 * 2 + 8) + units * w.d * 4
    gathered = units * w.m * 2 * w.d * w.elem_bytes
    by = gathered + units * w.m * 4 + state + w.B * w.Hq * (w.d * 2 + w.d * 4 + 4)
    dense_by = units * w.n * 2 * w.d * w.elem_bytes
    out["C5_prior_bf16_b16_n128k"] = line(
        ms_p, gathered, by, dms, m=w.m, repeats_us=[round(x * 1e3, 3) for x in per],
        no_tail_us_per_step=round(ms_none * 1e3, 2), prior_overhead_pct=round(100 * (ms_p / ms_none - 1), 2),
        max_rel_err=max(errs), units_checked=len(errs),
        build_prior_us=round(build_ms * 1e3, 1), build_prior_gbs=round(dense_by / (build_ms * 1e-3) / 1e9, 1))
    B1 = 2
    pst = oracle.prior_build(c.K[:B1], c.V[:B1], c.mu_Q[:B1])
    name, rec = oracle_path(
        "prior_delta_form", lambda: oracle.sparse_prior(c.q[:B1], c.K[:B1], c.V[:B1], c.idx[:B1], c.mu_Q[:B1],
                                                        w.lam, *pst),
        B1 * w.Hkv * w.m * 2 * w.d * w.elem_bytes, B1 * w.Hkv, units, a.path_seconds,
        f"{B1 * w.Hkv} units of the batch-16 128K 3% step, O(|I|) delta form from a prebuilt fp64 prior")
    paths[name] = rec
    name, rec = oracle_path(
        "prior_definition_o_of_n", lambda: oracle.sparse_prior_def(c.q[:B1], c.K[:B1], c.V[:B1], c.idx[:B1],
                                                                   c.mu_Q[:B1], w.lam),
        None, B1 * w.Hkv, units, a.path_seconds,
        f"{B1 * w.Hkv} units of the batch-16 128K 3% step, the O(n) definition (every unlisted row weighed)")
    paths[name] = rec
    del copies, K, V, c, ps, pst
    torch.cuda.empty_cache()

    # the selector in front of the proxy decode (QGS codes + ErrorGate + per-cluster top-q)
    out.update(measure_selector(a, dev))
    return out, paths


def measure_selector(a, dev):
    import numpy as np
    import torch

    from long_context_sparse_gathered_amd import sda, synth
    from oracle import qgs
    w = synth.WORKLOADS["qgs_bf16_b32_n32k"]
    c = synth.make_case(w)
    q, K, V, U, cid = (to_dev(x, dev) for x in (c.q, c.K, c.V, c.U, c.cid))
    ws_b = torch.empty(sda.workspace_bytes(sda.make_dims(K, w.Hq), sda.OP_BUILD_PROXIES, C=w.C), dtype=torch.uint8,
                       device=dev)
    pbuild_ms, _ = time_steps(lambda i: sda.build_tail_proxies(K, V, cid, w.C, ws=ws_b, with_sumK2=True), 3, 1,
                              graph=False, repeats=1)
    st = sda.build_tail_proxies(K, V, cid, w.C, ws=ws_b, with_sumK2=True)
    ws_c = torch.empty(sda.workspace_bytes(sda.make_dims(K, w.Hq), sda.OP_BUILD_QGS), dtype=torch.uint8, device=dev)
    cbuild_ms, _ = time_steps(lambda i: sda.build_qgs_codes(K, U, ws=ws_c), 3, 1, graph=False, repeats=1)
    qc = sda.build_qgs_codes(K, U, ws=ws_c)
    del V
    ncopy = 2
    copies = [(qc, cid)] + [(sda.QgsCodes(U=U, codes=qc.codes.clone(), kmax=qc.kmax), cid.clone())
                            for _ in range(ncopy - 1)]
    units = w.B * w.Hkv
    outs = (torch.empty((w.B, w.Hkv, w.m), dtype=torch.int32, device=dev),
            torch.empty((w.B, w.Hkv), dtype=torch.int32, device=dev),
            torch.empty((w.B, w.Hkv, w.m), dtype=torch.int32, device=dev))
    budget = torch.zeros((w.B, w.Hkv, w.C), dtype=torch.int32, device=dev)
    ws = torch.empty(sda.workspace_bytes(sda.make_dims(K, w.Hq), sda.OP_SELECT_QGS, C=w.C), dtype=torch.uint8,
                     device=dev)
    ms_s, per = time_steps(lambda i: sda.select_qgs(q, K, copies[i % ncopy][1], st, copies[i % ncopy][0], w.n_sink,
                                                    w.n_local, w.n_top, out=outs, ws=ws), 50, 5,
                           graph=not a.no_graph, repeats=a.repeats)
    # bit-exact lists and budgets on sampled units, the oracle fed the
    # builder's own cluster sums (decisions within a few fp64 roundings of a
    # tie are counted, not compared)
    sda.select_qgs(q, K, cid, st, qc, w.n_sink, w.n_local, w.n_top, out=outs, budget=budget, ws=ws)
    torch.cuda.synchronize()
    sc = np.float32(1.0 / np.sqrt(w.d))
    exact, fragile, checked = True, 0, []
    rng = np.random.default_rng(3)
    for u in rng.choice(units, size=2, replace=False):
        s, g = divmod(int(u), w.Hkv)
        checked.append(int(u))
        stats = (st.count[s, g].cpu().numpy().astype(np.int64), st.sumK[s, g].cpu().double().numpy(),
                 st.sumK2[s, g].cpu().double().numpy())
        og = qgs.select_unit(c.q[s, g * w.G:(g + 1) * w.G], c.K[s, g], c.cid[s, g], w.C, c.U[s, g], w.n_sink,
                             w.n_local, w.n_top, sc, stats=stats)
        if og["margin"] < 1e-9:
            fragile += 1
            continue
        L = int(outs[1][s, g])
        exact &= bool(np.array_equal(budget[s, g].cpu().numpy(), og["budget"]))
        exact &= bool(np.array_equal(outs[0][s, g, :L].cpu().numpy(), og["idx"]))
    per_unit = (w.n * (w.r + 4) + w.C * (4 + 2 * w.d * 4) + w.d * w.r * 4 + w.r * 8 + w.m * 8 + 4)
    by = units * per_unit + w.B * w.Hq * w.d * w.elem_bytes
    # query-geometry clustering (C = 64, 10 passes) and the selector on its clusters
    V16 = U[..., :sda.QGC_RANK].contiguous()
    ws_q = torch.empty(sda.workspace_bytes(sda.make_dims(K, w.Hq), sda.OP_BUILD_QGC, C=64), dtype=torch.uint8,
                       device=dev)
    qgc_ms, _ = time_steps(lambda i: sda.build_qgc_clusters(K, V16, 64, T=10, ws=ws_q), 3, 1, graph=False, repeats=1)
    cid64 = sda.build_qgc_clusters(K, V16, 64, T=10, ws=ws_q)
    del ws_q
    Vfull = to_dev(c.V, dev)
    st64 = sda.build_tail_proxies(K, Vfull, cid64, 64, with_sumK2=True)
    del Vfull
    ws64 = torch.empty(sda.workspace_bytes(sda.make_dims(K, w.Hq), sda.OP_SELECT_QGS, C=64), dtype=torch.uint8,
                       device=dev)
    ms_s64, _ = time_steps(lambda i: sda.select_qgs(q, K, cid64, st64, copies[i % ncopy][0], w.n_sink, w.n_local,
                                                    w.n_top, out=outs, ws=ws64), 50, 5, graph=not a.no_graph,
                           repeats=a.repeats)
    return {"qgs_select_b32_n32k": line(
        ms_s, None, by, None, repeats_us=[round(x * 1e3, 3) for x in per],
        rows_scored=units * w.n, rows_picked=units * w.n_top,
        lists_and_budgets_bit_exact=exact, units_checked=checked, fragile_units_skipped=fragile,
        build_codes_us=round(cbuild_ms * 1e3, 1), build_proxies_with_sq_us=round(pbuild_ms * 1e3, 1),
        qgc_clusters_c64_t10_us=round(qgc_ms * 1e3, 1), us_per_step_on_qgc_c64=round(ms_s64 * 1e3, 2),
        note="total bytes: int8 codes, ids, cluster state, basis and lists; no K/V rows are gathered")}


def cpu_baseline(w, c, seconds):
    """fp64 oracle, O(|I|) proxy path, on whole units of the same step, all
    host threads."""
    from oracle import oracle
    threads = oracle.get_threads()
    sample_units = min(32, w.B * w.Hkv)
    B1 = sample_units // w.Hkv
    q, K, V, idx, cid = c.q[:B1], c.K[:B1], c.V[:B1], c.idx[:B1], c.cid[:B1]
    cnt, sK, sV = oracle.proxy_build(K, V, cid, w.C)
    dt, reps = timed_cpu(lambda: oracle.sparse_proxy(q, K, V, idx, cid, w.C, cnt, sK, sV), seconds)
    gathered = sample_units * w.m * 2 * w.d * w.elem_bytes
    step_s = dt * (w.B * w.Hkv) / sample_units
    return {"value": round(gathered / dt / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "us_per_step": round(step_s * 1e6, 1), "host_cpus": os.cpu_count(),
            "sample": f"{sample_units} of {w.B * w.Hkv} (sequence, KV head) units of the same step, "
                      f"O(|I|) proxy path from prebuilt fp64 cluster sums, {reps} repetitions"}


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
