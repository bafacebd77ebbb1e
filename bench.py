"""Benchmark of the 3-bit group-64 affine matmul, K=5120 -> N=10240, at
M = 1, 9, 16, 32, 64 activation rows on one MI355X.

One step = one matmul at each of the five row counts (the whole hot path:
native weights streamed from HBM, unpacked, dequantized, multiplied, reduced,
written), each on a different copy of the weights: the copies form a ring of
more than 1 GiB, four times the 256 MB Infinity Cache, so every matmul reads
its weights cold from HBM.  Inputs are resident in device memory before the
timed region starts; the one-time repack to the native layout is outside it.

Prints one JSON line (stdout).  Progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

K, N, BITS = 5120, 10240, 3
ROWS = (1, 9, 16, 32, 64)
HBM_PEAK_GBPS = 8000.0      # MI355X published HBM3E read+write peak
RING_BYTES = 1 << 30


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def weight_bytes() -> int:
    return N * K * BITS // 8 + 2 * N * (K // 64) * 2


def algorithmic_bytes(m: int) -> int:
    """Bytes one matmul must move: weights once, activations once, output once."""
    return weight_bytes() + m * K * 2 + m * N * 2


def _oracle_steps(problem, threads: int, seconds: float):
    """Full steps of the float64 oracle (all five row counts, every output)
    until about `seconds` have passed: (steps, seconds)."""
    import oracle
    t0 = time.perf_counter()
    reps = 0
    while True:
        for m in ROWS:
            p = problem.rows(m)
            oracle.matmul(BITS, K, p.x, p.w, p.scales, p.biases, threads=threads)
        reps += 1
        if time.perf_counter() - t0 >= seconds or reps >= 200:
            break
    return reps, time.perf_counter() - t0


def cpu_baseline(problem, seconds: float = 10.0):
    """The float64 oracle on the host cores, timed on all of them (the value)
    and on one thread; the same weight-stream GB/s formula as the GPU line."""
    threads = len(os.sched_getaffinity(0))
    reps, dt = _oracle_steps(problem, threads, seconds)
    reps1, dt1 = _oracle_steps(problem, 1, seconds)
    gbps = reps * len(ROWS) * weight_bytes() / dt / 1e9
    gbps1 = reps1 * len(ROWS) * weight_bytes() / dt1 / 1e9
    return {"value": round(gbps, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "%d full step(s): all %d outputs at each of M=%s, float64 oracle, %.1f s"
                      % (reps, N, ",".join(map(str, ROWS)), dt),
            "us_per_step": round(dt / reps * 1e6, 1),
            "one_thread": {"value": round(gbps1, 4), "unit": "GB/s", "cores": 1,
                           "us_per_step": round(dt1 / reps1 * 1e6, 1),
                           "sample": "%d full step(s) on one thread, %.1f s" % (reps1, dt1)}}


def trace_summary(path: str) -> str:
    """Per-dispatch kernel durations from a rocprofv3 kernel trace (CSV): one
    row per (kernel, dynamic LDS size) -- the LDS size tells the row counts of
    one kernel apart -- with the count, median, p10, p90, min and max in us."""
    import csv
    groups = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            key = (r["Kernel_Name"], int(r.get("LDS_Block_Size") or 0),
                   int(r.get("Grid_Size_X") or 0) // max(1, int(r.get("Workgroup_Size_X") or 1)))
            d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0
            groups.setdefault(key, []).append(d)

    def q(v, f):
        return v[min(len(v) - 1, int(f * len(v)))]

    lines = ["| kernel | LDS bytes | workgroups | dispatches | median us | p10 us | p90 us | min us | max us |",
             "|---|---|---|---|---|---|---|---|---|"]
    for (name, lds, wgs), v in sorted(groups.items(), key=lambda kv: -len(kv[1])):
        v.sort()
        short = name.replace("void ", "").split("(")[0]
        lines.append("| `%s` | %d | %d | %d | %.2f | %.2f | %.2f | %.2f | %.2f |" % (
            short, lds, wgs, len(v), q(v, 0.5), q(v, 0.1), q(v, 0.9), v[0], v[-1]))
    return "\n".join(lines)


def kernel_source_hash() -> str:
    """sha256[:16] over the matmul kernels' sources (the shared device header
    and every family's file, in name order)."""
    import hashlib
    csrc = os.path.join(ROOT, "bit_quantized_matmul_affine_amd", "csrc")
    h = hashlib.sha256()
    for name in ("qmm_device.h", "qmm_formats.h", "qmm_internal.h", "qmm_layout.hip",
                 "qmm_mfma.hip", "qmm_resident.hip", "qmm_slab.hip", "qmm_stream.hip",
                 "qmm_wide.hip"):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


MATMUL_KERNELS = ("stream_kernel", "resident_kernel", "slab_kernel", "split_slab_kernel",
                  "mfma_kernel", "gemv_kernel", "wide_kernel")


def _counter_means(path: str, counter: str):
    """Mean value of one counter per kernel name over a rocprofv3 --pmc CSV
    (one row per dispatch and counter): {name: (dispatches, mean)}."""
    import csv
    acc = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r.get("Counter_Name") != counter:
                continue
            name = r["Kernel_Name"].replace("void ", "").split("(")[0].replace("qmm::", "")
            n, tot = acc.get(name, (0, 0.0))
            acc[name] = (n + 1, tot + float(r["Counter_Value"]))
    return {k: (n, tot / n) for k, (n, tot) in acc.items()}


def traffic_summary(probe_csv: str, runs) -> str:
    """HBM bytes per dispatch of the matmul kernel of each bench run.  runs:
    (rows, FETCH_SIZE csv, WRITE_SIZE csv) of `bench.py --rows rows` under
    `rocprofv3 --pmc FETCH_SIZE` / `--pmc WRITE_SIZE`; probe_csv: FETCH_SIZE
    of `bench.py --probe-only` (1 GiB read per launch), which scales the
    FETCH_SIZE KiB to bytes.  WRITE_SIZE is taken at face value (KiB).
    Writes profiles/hbm_traffic.json and returns a markdown table."""
    probe = [v for k, v in _counter_means(probe_csv, "FETCH_SIZE").items() if "probe_kernel" in k]
    assert probe, "no probe_kernel dispatch in " + probe_csv
    fetch_factor = (1 << 30) / 1024.0 / probe[0][1]
    kernels = {}
    for rows, fcsv, wcsv in runs:
        fm = {k: v for k, v in _counter_means(fcsv, "FETCH_SIZE").items()
              if k.split("<")[0] in MATMUL_KERNELS}
        wm = {k: v for k, v in _counter_means(wcsv, "WRITE_SIZE").items()
              if k.split("<")[0] in MATMUL_KERNELS}
        assert len(fm) == 1 and list(fm) == list(wm), "one matmul kernel per run: %s" % list(fm)
        name = next(iter(fm))
        fk, wk = fm[name][1], wm[name][1]
        e = kernels.setdefault(name, {"rows": [], "fetch_kib": [], "write_kib": []})
        e["rows"].append(rows)
        e["fetch_kib"].append(fk)
        e["write_kib"].append(wk)
    lines = ["| kernel | M | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes (scaled) | "
             "algorithmic bytes | ratio |", "|---|---|---|---|---|---|---|"]
    out = {}
    for name, e in kernels.items():
        fk = sum(e["fetch_kib"]) / len(e["fetch_kib"])
        wk = sum(e["write_kib"]) / len(e["write_kib"])
        hbm = fk * 1024.0 * fetch_factor + wk * 1024.0
        alg = sum(algorithmic_bytes(m) for m in e["rows"]) / len(e["rows"])
        out[name] = {"rows": e["rows"], "fetch_kib": fk, "write_kib": wk, "hbm_bytes": hbm}
        lines.append("| `%s` | %s | %.1f | %.1f | %d | %d | %.3f |" % (
            name, ",".join(map(str, e["rows"])), fk, wk, hbm, alg, hbm / alg))
    rec = {"kernel_source_sha256_16": kernel_source_hash(), "fetch_factor": fetch_factor,
           "write_factor": 1.0, "kernels": out}
    with open(os.path.join(ROOT, "profiles", "hbm_traffic.json"), "w") as f:
        json.dump(rec, f, indent=1)
    lines.append("")
    lines.append("FETCH_SIZE scale: the probe reads 1 GiB per launch and FETCH_SIZE reports "
                 "%.1f KiB for it: bytes = KiB x 1024 x %.4f.  Kernel sources: %s."
                 % (probe[0][1], fetch_factor, rec["kernel_source_sha256_16"]))
    return "\n".join(lines)


def measured_traffic(rows: int):
    """HBM bytes per launch of the kernel that serves `rows` rows, from the
    committed FETCH_SIZE/WRITE_SIZE measurement, or None when the kernel
    source has changed since it was taken."""
    try:
        with open(os.path.join(ROOT, "profiles", "hbm_traffic.json")) as f:
            rec = json.load(f)
        h = kernel_source_hash()
    except OSError:
        return None
    if rec.get("kernel_source_sha256_16") != h:
        return None
    for k in rec["kernels"].values():
        if rows in k["rows"]:
            return int(k["hbm_bytes"])
    return None


def measure_hbm(torch, binding, gib: int = 4, reps: int = 5):
    buf = torch.empty(gib << 30, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    best = 0.0
    for _ in range(reps):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        binding.hbm_probe(buf, grid=4096)
        e.record()
        e.synchronize()
        best = max(best, buf.numel() / (s.elapsed_time(e) * 1e-3) / 1e9)
    del buf
    return best


def time_workload(torch, binding, prob, rows, reps=5, cold=True):
    """Mean us per matmul of `prob` at `rows` rows: a graph of R launches, each
    on its own weight copy (R copies >= 1 GiB, so reads are cold), replayed
    `reps` times; with cold=False one copy is reused (cache-resident)."""
    lin = binding.QuantizedLinear(prob, max_rows=max(rows, 1))
    wb = prob.weight_bytes
    ring = max(2, -(-RING_BYTES // wb)) if cold else 1
    copies = [(lin.codes, lin.sb)] + [(lin.codes.clone(), lin.sb.clone()) for _ in range(ring - 1)]
    x = binding.to_device(prob.x[:rows])
    y = torch.empty(rows, prob.N, dtype=torch.bfloat16 if prob.x_dtype == "bf16" else torch.float32,
                    device="cuda")
    plan = lin.plan
    ws = plan.workspace(max(256, plan.workspace_bytes(rows)), x.device)
    n = max(ring, 16)

    def calls():
        for i in range(n):
            c, sbv = copies[i % ring]
            plan.run(x, c, sbv, out=y, workspace=ws)

    calls()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    g.replay()
    torch.cuda.synchronize()
    d = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        e1.synchronize()
        d.append(e0.elapsed_time(e1) * 1e3 / n)
    variant = plan.stats()["last_variant"]
    del g, copies, lin
    torch.cuda.synchronize()
    return sum(d) / len(d), variant


def time_gate_up(torch, binding, gate, up, reps=5):
    """Mean us per fused gate/up call (qmm_run_gate_up) of the MLP's gate and up
    projections, cold as in time_workload (a ring of weight-pair copies)."""
    lg = binding.QuantizedLinear(gate, max_rows=gate.M)
    lu = binding.QuantizedLinear(up, max_rows=up.M)
    wb = gate.weight_bytes + up.weight_bytes
    ring = max(2, -(-RING_BYTES // wb))
    copies = [(lg.codes, lg.sb, lu.codes, lu.sb)] + [
        (lg.codes.clone(), lg.sb.clone(), lu.codes.clone(), lu.sb.clone()) for _ in range(ring - 1)]
    x = binding.to_device(gate.x)
    h = torch.empty(gate.M, gate.N, dtype=torch.bfloat16, device="cuda")
    n = max(ring, 16)

    def calls():
        for i in range(n):
            gc, gs, uc, us_ = copies[i % ring]
            lg.plan.run_gate_up(x, gc, gs, uc, us_, out=h)

    calls()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    g.replay()
    torch.cuda.synchronize()
    d = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        e1.synchronize()
        d.append(e0.elapsed_time(e1) * 1e3 / n)
    del g, copies, lg, lu
    torch.cuda.synchronize()
    return sum(d) / len(d), wb


def time_norm(torch, binding, synth, rows, D, reps=5):
    """Mean us per residual add + RMS norm call (qmm_residual_rms_norm) over
    bf16 [rows, D]; algorithmic bytes: x, update read, residual, normalized
    written (2 bytes each) plus the weight vector."""
    xr, ur, wr = synth.norm_inputs(7, rows, D, "bf16")
    x, u, w = binding.to_device(xr), binding.to_device(ur), binding.to_device(wr)
    res, norm = torch.empty_like(x), torch.empty_like(x)
    n = 32 if rows * D < (1 << 24) else 4

    def calls():
        for _ in range(n):
            binding.residual_rms_norm(x, u, w, 1e-5, residual=res, normalized=norm)

    calls()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    g.replay()
    torch.cuda.synchronize()
    d = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        e1.synchronize()
        d.append(e0.elapsed_time(e1) * 1e3 / n)
    del g, x, u, res, norm
    torch.cuda.synchronize()
    us = sum(d) / len(d)
    nbytes = 4 * rows * D * 2 + D * 2
    return {"us": round(us, 3), "bytes": nbytes, "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
            "frac_of_8TBps": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}


def time_attention(torch, binding, synth, H, KV, N, D, bits, gs, reps=5):
    """Mean us per decode-attention call (qmm_decode_attention, both kernels)
    over a cache of KV heads x N rows; algorithmic bytes: the key and value
    codes, scales and biases once, plus q and the output.  Cold: each call
    reads its own copy of the cache from a ring of copies of at least 1 GiB
    (four times the 256 MB last-level cache); also a warm figure with one
    cache reused (resident in the last-level cache)."""
    q, k, v = synth.attention_inputs(13, H=H, KV=KV, N=N, D=D, bits=bits, group_size=gs)
    qd = binding.to_device(q)
    kd = tuple(binding.to_device(x) for x in k)
    vd = tuple(binding.to_device(x) for x in v)
    nbytes = sum(x.nbytes for x in k) + sum(x.nbytes for x in v) + 2 * q.nbytes
    ring = max(2, -(-RING_BYTES // nbytes))
    caches = [(kd, vd)] + [(tuple(x.clone() for x in kd), tuple(x.clone() for x in vd))
                           for _ in range(ring - 1)]
    out = torch.empty_like(qd)
    need = binding.lib().qmm_attention_workspace_bytes(H, N, D)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")

    def timed(n, pick):
        def calls():
            for i in range(n):
                kc, vc = pick(i)
                binding.decode_attention(qd, kc, vc, bits, gs, out=out, workspace=ws)

        calls()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            calls()
        g.replay()
        torch.cuda.synchronize()
        d = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            e1.synchronize()
            d.append(e0.elapsed_time(e1) * 1e3 / n)
        del g
        return sum(d) / len(d)

    cold = timed(ring, lambda i: caches[i])
    warm = timed(32, lambda i: caches[0])
    del caches
    torch.cuda.synchronize()
    gb = nbytes / (cold * 1e-6) / 1e9
    return {"us": round(cold, 3), "bytes": nbytes, "GBps": round(gb, 1),
            "frac_of_8TBps": round(gb / HBM_PEAK_GBPS, 4),
            "cold": "a ring of %d cache copies (%.2f GiB): each call reads its cache from HBM"
                    % (ring, ring * nbytes / 2**30),
            "us_cache_resident": round(warm, 3),
            "GBps_cache_resident": round(nbytes / (warm * 1e-6) / 1e9, 1)}


def wave_timeline(torch, binding, synth):
    """Per-wave phase times of the streaming kernel (1 row), the resident
    kernel (9 and 16 rows) and the split slab kernel (64 rows) on the 3-bit
    5120 -> 10240 workload, cold (a ring of weight copies), from the timing
    build: each wave stamps a 100 MHz device-wide counter at its phase
    boundaries and writes the stamps at its end.  Times in us from the
    earliest wave start of the last launch, percentiles 0/10/50/90/100 over
    waves (the split slab kernel's: over its compute waves).  The timing
    build waits for each chunk's weights explicitly before stamping them (the
    ordinary build waits at the first use); the split slab kernel's stamps
    add no waits."""
    import numpy as np
    names = {"stream": {0: "start", 1: "activation loads issued", 2: "weight loads issued",
                        3: "activations landed (in LDS with sums)", 12: "compute done",
                        13: "workgroup barrier", 14: "stores issued (storing wave)"},
             "resident": {0: "start", 1: "loads issued", 2: "activations landed",
                          12: "compute done", 13: "workgroup barrier",
                          14: "stores issued (storing waves)"},
             "slab": {0: "start", 1: "slice 0 landed (first barrier)", 10: "fold barrier",
                      11: "partial tiles added in LDS", 12: "partials stored (coherent)",
                      13: "ticket taken", 14: "y stored (second arrivals)"}}
    first_chunk = {"stream": 4, "resident": 3}
    (prob,) = synth.workload(2, M=64)
    out = {}
    for fam, rows in (("stream", 1), ("resident", 9), ("resident", 16), ("slab", 64)):
        lin = binding.QuantizedLinear(prob, max_rows=64)
        ring = max(2, -(-RING_BYTES // weight_bytes()))
        copies = [(lin.codes, lin.sb)] + [(lin.codes.clone(), lin.sb.clone())
                                          for _ in range(ring - 1)]
        x = binding.to_device(prob.x[:rows])
        y = torch.empty(rows, N, dtype=torch.bfloat16, device="cuda")
        ws = torch.zeros(8 << 20, dtype=torch.uint8, device="cuda")
        for _ in range(2):
            for c, sbv in copies:
                lin.plan.run(x, c, sbv, out=y, variant=fam, workspace=ws)
        torch.cuda.synchronize()
        st = lin.plan.stats()
        if fam == "slab":
            # 12 compute waves and 4 loader waves; 5 slices of 512 k; the
            # stamps follow the kernel's own tickets and partial tiles
            assert st["last_splitk"] == 2, "64 rows run on the split slab kernel"
            nw, nsl, skip = 16, 5, lin.plan.workspace_bytes(rows)
        else:
            nw, cpw = 8, 5
            skip = ((N // 16) * 4 + 255) // 256 * 256
        grid = st["last_grid"] if fam != "stream" else N // 16
        raw = ws.cpu().numpy()[skip:].view(np.uint64)[: grid * nw * 16]
        s16 = raw.reshape(grid, nw, 16).astype(np.int64)
        t0 = s16[:, :, 0].min()
        rel = (s16 - t0) * 0.01                      # 100 MHz ticks -> us
        rec = {"family": fam, "rows": rows, "workgroups": grid, "waves": grid * nw}
        stamps = dict(names[fam])
        if fam == "slab":
            for j in range(nsl):
                stamps[2 + j] = "slice %d done (barrier)" % j
            comp = rel[:, :12, :]
            cs16 = s16[:, :12, :]
        else:
            for j in range(cpw):
                stamps[first_chunk[fam] + j] = "chunk %d weights landed" % j
            comp, cs16 = rel, s16
        for k in sorted(stamps):
            v = comp[:, :, k][cs16[:, :, k] > 0]
            rec[stamps[k]] = [round(float(np.percentile(v, q)), 2) for q in (0, 10, 50, 90, 100)]
        rec["workgroup start"] = [round(float(np.percentile(rel[:, :, 0].min(axis=1), q)), 2)
                                  for q in (0, 10, 50, 90, 100)]
        if fam == "slab":
            rec["slice time, median over workgroups (us)"] = [
                round(float(np.median(rel[:, 0, 2 + j] - rel[:, 0, 1 + j])), 3)
                for j in range(nsl)]
        else:
            land = 3 if fam == "stream" else 2
            rec["activations landed, median by wave index"] = [
                round(float(np.median(rel[:, w, land])), 2) for w in range(nw)]
            rec["compute done, median by wave index"] = [
                round(float(np.median(rel[:, w, 12])), 2) for w in range(nw)]
        out["%s %d row(s)" % (fam, rows)] = rec
        del copies, lin
        torch.cuda.synchronize()
    return out


def counter_summary(paths) -> str:
    """Markdown table of rocprofv3 --pmc CSVs (no GPU needed): per kernel, the
    mean over its dispatches of each counter (the rows of one dispatch, one
    per hardware block instance, added) and of the dispatch duration."""
    import csv
    from collections import defaultdict
    per = defaultdict(lambda: defaultdict(float))  # (kernel, dispatch) -> counter -> value
    dur = {}
    for path in paths:
        with open(path) as f:
            for r in csv.DictReader(f):
                name = r["Kernel_Name"].split("(")[0].replace("void ", "").replace("qmm::", "")
                key = (name, path, r["Dispatch_Id"])
                per[key][r["Counter_Name"]] += float(r["Counter_Value"])
                dur[key] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3
    kernels = defaultdict(list)
    for key in per:
        kernels[key[0]].append(key)
    counters = sorted({c for v in per.values() for c in v})
    lines = ["| kernel | dispatches | mean us | " + " | ".join(counters) + " |",
             "|---|---|---|" + "---|" * len(counters)]
    for name, keys in sorted(kernels.items()):
        if name.startswith("at::") or name.startswith("__amd"):
            continue
        cells = []
        for c in counters:
            vals = [per[k][c] for k in keys if c in per[k]]
            cells.append("%.4g" % (sum(vals) / len(vals)) if vals else "")
        lines.append("| `%s` | %d | %.2f | %s |" % (name, len(keys),
                                                   sum(dur[k] for k in keys) / len(keys),
                                                   " | ".join(cells)))
    return "\n".join(lines)


def timeline_summary(path: str) -> str:
    """Markdown tables of a --wave-timeline JSON (no GPU needed): per family
    and row count, p0 / p10 / p50 / p90 / p100 of every phase, then the
    per-wave-index medians."""
    with open(path) as f:
        d = json.load(f)
    out = []
    for name, r in d.items():
        out.append("## %s: %d workgroups, %d waves\n" % (name, r["workgroups"], r["waves"]))
        out.append("| phase | p0 | p10 | p50 | p90 | p100 |")
        out.append("|---|---|---|---|---|---|")
        extra = []
        for k, v in r.items():
            if not isinstance(v, list):
                continue
            if "median" in k:
                extra.append("%s: %s" % (k[0].upper() + k[1:], ", ".join("%.2f" % x for x in v)))
                continue
            out.append("| %s | %s |" % (k, " | ".join("%.2f" % x for x in v)))
        out.append("")
        for e in extra:
            out.append(e + "\n")
    return "\n".join(out)


def crossover(torch, binding, synth, reps=3):
    """The 4-bit 8192 -> 28672 block of 128 rows (the compute/bandwidth
    crossover), cold as in time_workload."""
    (p4,) = synth.workload(4)
    us, v = time_workload(torch, binding, p4, p4.M, reps=reps)
    tf = 2.0 * p4.M * p4.N * p4.K / (us * 1e-6) / 1e12
    return {"us": round(us, 3), "weight_GBps": round(p4.weight_bytes / (us * 1e-6) / 1e9, 1),
            "tflops": round(tf, 2), "frac_of_bf16_mfma_peak": round(tf / 2500.0, 4), "variant": v}


def other_workloads(torch, binding, synth, probe):
    """The remaining configurations, each cold-read as above."""
    out = {}
    (p1,) = synth.workload(1)
    us, v = time_workload(torch, binding, p1, 1)
    gb = p1.weight_bytes / (us * 1e-6) / 1e9
    out["4-bit 5120->10240, 1 row, bf16"] = {
        "us": round(us, 3), "weight_GBps": round(gb, 1), "variant": v,
        "frac_of_measured_peak": round(gb / probe, 4) if probe else None}
    trio = {}
    total_us, total_bytes = 0.0, 0
    for p in synth.workload(3):
        us, v = time_workload(torch, binding, p, p.M)
        total_us += us
        total_bytes += p.weight_bytes
        trio[p.name] = {"us": round(us, 3), "weight_GBps": round(p.weight_bytes / (us * 1e-6) / 1e9, 1),
                        "variant": v}
    gb = total_bytes / (total_us * 1e-6) / 1e9
    gate, up, down = synth.workload(3)
    gu_us, gu_bytes = time_gate_up(torch, binding, gate, up)
    fused_us = gu_us + trio["c3_down"]["us"]
    fgb = total_bytes / (fused_us * 1e-6) / 1e9
    out["4-bit MLP trio 3840->15360 x2, 15360->3840, 4 rows, bf16"] = {
        "per_projection": trio, "trio_us": round(total_us, 3), "weight_GBps": round(gb, 1),
        "frac_of_measured_peak": round(gb / probe, 4) if probe else None,
        "fused_gate_up": {"us": round(gu_us, 3),
                          "weight_GBps": round(gu_bytes / (gu_us * 1e-6) / 1e9, 1),
                          "what": "silu(x.Wg^T)*(x.Wu^T) in one kernel (qmm_run_gate_up)"},
        "trio_fused_us": round(fused_us, 3), "weight_GBps_fused": round(fgb, 1),
        "frac_of_measured_peak_fused": round(fgb / probe, 4) if probe else None}
    out["4-bit 8192->28672, 128 rows, bf16"] = crossover(torch, binding, synth)
    fmt = {}
    for bits, gs in ((2, 64), (2, 32), (8, 64), (8, 128), (3, 32), (4, 32), (4, 128), (3, 128)):
        pf = synth.small(900 + bits + gs, bits=bits, K=5120, N=10240, M=16, group_size=gs)
        for rows in (1, 16):
            us, v = time_workload(torch, binding, pf, rows)
            gb = pf.weight_bytes / (us * 1e-6) / 1e9
            fmt["%d-bit group-%d, %d row%s" % (bits, gs, rows, "s" if rows > 1 else "")] = {
                "us": round(us, 3), "weight_bytes": pf.weight_bytes, "weight_GBps": round(gb, 1),
                "variant": v, "frac_of_measured_peak": round(gb / probe, 4) if probe else None}
    out["format variants 5120->10240, bf16 (step layout on the streaming and resident "
        "kernels; 3/4-bit groups of 128 on the native layout)"] = fmt
    out["residual add + RMS norm, bf16"] = {
        "4x3840 (decode)": time_norm(torch, binding, synth, 4, 3840),
        "16384x5120 (HBM-bound)": time_norm(torch, binding, synth, 16384, 5120)}
    out["decode attention over a 4-bit group-64 KV cache, bf16"] = {
        "16 heads / 8 KV heads, D=256, N=8192": time_attention(torch, binding, synth, 16, 8, 8192,
                                                               256, 4, 64),
        "16 heads / 8 KV heads, D=256, N=32768": time_attention(torch, binding, synth, 16, 8,
                                                                32768, 256, 4, 64)}
    (p0,) = synth.workload(0)
    us, v = time_workload(torch, binding, p0, 1)
    out["4-bit 512->512, 1 row, f32 (launch-bound)"] = {"us": round(us, 3), "variant": v}
    return out


def main() -> int:
    global ROWS, BITS
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--variant", default="auto",
                    choices=["auto", "gemv", "mfma", "stream", "resident", "slab"])
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the other workloads (4-bit 5120->10240 at 1 row, the MLP trio at "
                         "4 rows, 4-bit 8192->28672 at 128 rows, 4-bit 512->512 at 1 row) and the "
                         "cache-resident numbers")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-probe", action="store_true", help="skip the HBM read probe")
    ap.add_argument("--bits", type=int, default=3, choices=[3, 4],
                    help="3: the measured 3-bit workload; 4: the 4-bit GEMV of the same shape "
                         "(one row, for kernel comparisons at --rows 1)")
    ap.add_argument("--rows", default=",".join(map(str, ROWS)),
                    help="row counts of a step (default 1,9,16,32,64, the measured workload; a "
                         "single row count serves per-row-count kernel traces)")
    ap.add_argument("--wave-timeline", action="store_true",
                    help="print per-wave phase times of the streaming, resident and split slab "
                         "kernels from the timing build (libqmm_stamps.so) and exit")
    ap.add_argument("--counter-summary", nargs="+", metavar="CSV",
                    help="print per-kernel means of rocprofv3 --pmc counter CSVs and exit (no "
                         "GPU needed)")
    ap.add_argument("--timeline-summary", metavar="JSON",
                    help="print the phase tables of a --wave-timeline JSON and exit (no GPU "
                         "needed)")
    ap.add_argument("--trace-summary", metavar="CSV",
                    help="print per-dispatch duration statistics (median, p10, p90) of a "
                         "rocprofv3 --kernel-trace CSV and exit (no GPU needed)")
    ap.add_argument("--traffic-summary", nargs="+", metavar="CSV",
                    help="PROBE_FETCH_CSV ROWS:FETCH_CSV:WRITE_CSV ...: HBM bytes per dispatch "
                         "from rocprofv3 --pmc runs; writes profiles/hbm_traffic.json (no GPU)")
    ap.add_argument("--crossover-only", action="store_true",
                    help="only time the 4-bit 8192 -> 28672 block of 128 rows (cold weights) and "
                         "print its figures")
    ap.add_argument("--probe-only", action="store_true",
                    help="only run the HBM read probe on a 1 GiB buffer five times (a kernel of "
                         "known traffic, used to scale hardware byte counters)")
    args = ap.parse_args()
    if args.counter_summary:
        print(counter_summary(args.counter_summary))
        return 0
    if args.timeline_summary:
        print(timeline_summary(args.timeline_summary))
        return 0
    if args.trace_summary:
        print(trace_summary(args.trace_summary))
        return 0
    if args.traffic_summary:
        runs = []
        for spec in args.traffic_summary[1:]:
            m, fcsv, wcsv = spec.split(":")
            runs.append((int(m), fcsv, wcsv))
        print(traffic_summary(args.traffic_summary[0], runs))
        return 0
    ROWS = tuple(int(v) for v in args.rows.split(","))
    assert all(1 <= m <= 64 for m in ROWS), "row counts of the workload: 1..64"
    BITS = args.bits
    assert BITS == 3 or ROWS == (1,), "the 4-bit workload is the one-row GEMV: --rows 1"
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus > 1 or world > 1:
        print("bench.py runs on one GPU only: this library has no multi-GPU path",
              file=sys.stderr)
        return 2

    import torch
    from bit_quantized_matmul_affine_amd import binding, synth
    from bit_quantized_matmul_affine_amd import build as qbuild

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.wave_timeline:
        binding.LIB_PATH = qbuild.STAMPS_LIB
        print(json.dumps(wave_timeline(torch, binding, synth)), flush=True)
        return 0
    if args.crossover_only:
        print(json.dumps(crossover(torch, binding, synth, reps=1)), flush=True)
        return 0
    if args.probe_only:
        gbps = measure_hbm(torch, binding, gib=1)
        print(json.dumps({"probe_bytes_per_launch": 1 << 30, "launches": 5,
                          "best_GBps": round(gbps, 1)}), flush=True)
        return 0
    log("drawing inputs")
    # 3-bit: the M=64 draw, smaller M use its first rows; 4-bit: the one-row GEMV
    (prob,) = synth.workload(2 if BITS == 3 else 1)
    plan = binding.Plan(BITS, K, N, max(ROWS), "bf16", "bf16")
    lin = binding.QuantizedLinear(prob, max_rows=max(ROWS))
    ring = max(2, -(-RING_BYTES // weight_bytes()))
    log("ring of %d weight copies (%.2f GiB)" % (ring, ring * weight_bytes() / 2**30))
    copies = [(lin.codes.clone(), lin.sb.clone()) for _ in range(ring)]
    del lin
    x = binding.to_device(prob.x)             # [64, K] bf16
    ys = {m: torch.empty(m, N, dtype=torch.bfloat16, device="cuda") for m in ROWS}
    ws = plan.workspace(max(plan.workspace_bytes(m) for m in ROWS), x.device)
    torch.cuda.synchronize()

    probe = None
    if not args.no_probe:
        log("HBM read probe")
        probe = measure_hbm(torch, binding)

    counter = [0]

    def call(m):
        codes, sb = copies[counter[0] % ring]
        counter[0] += 1
        plan.run(x[:m], codes, sb, out=ys[m], variant=args.variant, workspace=ws)

    def capture(fn):
        """Record fn's launches into a HIP graph (no memsets are recorded: the
        kernels re-arm their own tickets)."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        return g

    log("warmup %d steps" % args.warmup)
    for _ in range(args.warmup):
        for m in ROWS:
            call(m)
    torch.cuda.synchronize()

    # The timed steps run as one graph so that host launch overhead does not
    # starve the GPU; each call still reads a different weight copy.
    log("capturing %d steps" % args.steps)
    step_graph = capture(lambda: [call(m) for _ in range(args.steps) for m in ROWS])
    step_graph.replay()
    torch.cuda.synchronize()
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    log("timing %d steps" % args.steps)
    torch.cuda.synchronize()
    t_start.record()
    step_graph.replay()
    t_end.record()
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_step = total_ms / args.steps

    # Per-row-count launch duration: `ring` back-to-back launches of one
    # kernel (one per weight copy) replayed as a graph, HIP events around it.
    per = {}
    reps = 5
    for m in ROWS:
        g = capture(lambda: [call(m) for _ in range(ring)])
        d = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            e1.synchronize()
            d.append(e0.elapsed_time(e1) * 1e3 / ring)
        d.sort()
        mean = sum(d) / len(d)
        per[str(m)] = {
            "us_mean": round(mean, 3), "us_min": round(d[0], 3), "us_max": round(d[-1], 3),
            "weight_GBps": round(weight_bytes() / (mean * 1e-6) / 1e9, 1),
            "algorithmic_GBps": round(algorithmic_bytes(m) / (mean * 1e-6) / 1e9, 1),
            "frac_of_8TBps": round(algorithmic_bytes(m) / (mean * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
            "tflops": round(2.0 * m * N * K / (mean * 1e-6) / 1e12, 2),
            "launch": plan.stats(),
        }
        if probe:
            per[str(m)]["frac_of_measured_peak"] = round(
                weight_bytes() / (mean * 1e-6) / 1e9 / probe, 4)
        del g
    dominant = max(ROWS, key=lambda m: per[str(m)]["us_mean"])
    dom = per[str(dominant)]
    achieved = algorithmic_bytes(dominant) / (dom["us_mean"] * 1e-6) / 1e9
    value = len(ROWS) * weight_bytes() / (ms_step * 1e-3) / 1e9

    extra, warm = None, None
    if not args.no_extra:
        log("cache-resident numbers")
        warm = {}
        for m in ROWS:
            us, _ = time_workload(torch, binding, prob.rows(m), m, cold=False)
            warm[str(m)] = {"us": round(us, 3),
                            "weight_GBps_cache_resident": round(weight_bytes() / (us * 1e-6) / 1e9, 1)}
        log("other workloads")
        extra = other_workloads(torch, binding, synth, probe)

    cpu = None
    if not args.no_cpu:
        log("oracle CPU baseline")
        cpu = cpu_baseline(prob)

    out = {
        "metric": "weight-stream GB/s over the %d-bit 5120->10240 sweep M=%s "
                  "(with us/matmul and %% of HBM peak per M)" % (BITS, ",".join(map(str, ROWS))),
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "%d-bit group-64 affine qmm K=5120 N=10240, M in {%s}, "
                               "bf16 activations/scales/biases, cold weights (%d-copy ring)"
                               % (BITS, ",".join(map(str, ROWS)), ring),
                   "variant": args.variant},
        "per_rows": per,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic(dominant),
                     "kernel": "M=%d (%s)" % (dominant, dom["launch"]["last_variant"]),
                     "bytes_per_launch": algorithmic_bytes(dominant),
                     "us_per_launch": dom["us_mean"]},
        "hbm_read_probe_GBps": round(probe, 1) if probe else None,
        "cache_resident_per_rows": warm,
        "other_workloads": extra,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
