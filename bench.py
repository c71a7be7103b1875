"""Benchmark of the AnchorKV hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = the whole hot path over one batch of synthetic input: the
end-of-prefill compression of every unit (all layers of all sequences) of the
workload, then one decode-attention step over the compressed cache of every
unit.  Inputs are generated on the GPU before the timed region.  Prints one
JSON line.  `value` is sequence tokens compressed (and decoded over) per
second of step time; per-stage times come from HIP events the library records
between its kernels on the bench stream (anchorkv_profile_*).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "compressed tokens/s (prefill compress) + decode-attn HBM GB/s, % of roofline"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_F32_MFMA_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "kv_cache_compression_snapkv_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def stage_work(p, stage):
    """Algorithmic work of one launch of a stage over all units:
    (flops, bytes).  Re-reads, recomputation and precision splits are not
    counted."""
    U, H, G, N, D, A, e = p.units, p.H, p.G, p.N, p.D, p.A, p.elem_bytes
    GQ = G * p.n_obs
    xb = U * H * N * D * e                      # one side's inputs
    qb = U * H * GQ * D * e
    if stage == "assign":                        # N x A x D similarity per side and head
        return 2 * U * H * 2.0 * N * A * D, 2 * xb + 2 * U * H * A * D * e + U * 2 * H * N * 4
    if stage == "obs_stats":                     # Q K^T
        return U * H * 2.0 * N * GQ * D, xb + qb
    if stage == "obs_score":                     # Q K^T for p, P V
        return U * H * 2 * 2.0 * N * GQ * D, 2 * xb + qb + U * H * N * 4
    if stage == "obs_util":                      # Q K^T for p, Q R_K, V O
        return U * H * 3 * 2.0 * N * GQ * D, 2 * xb + qb + U * 2 * H * N * 4
    if stage == "dec_stream":                    # anchors, pointer words, residual records, q, o
        rec = 36 if p.params.codec == 1 else 48
        nrec = p.R_total if p.joint else p.R_K + p.R_V
        return (U * H * N * G * 6.0 + 2 * U * H * G * A * 2.0 * D,
                U * (8 * H * N + rec * nrec + 2 * H * A * D * e) + U * H * G * D * (e + 4))
    return 0.0, 0.0


def decode_bytes(p):
    """Algorithmic bytes of one decode step over all units: the compressed
    cache (anchors, pointer words, residual records, offsets, positions) plus
    q and o."""
    return p.cache_bytes + p.units * p.H * p.G * p.D * (p.elem_bytes + 4)


def roofline(p, stage, ms):
    flops, byts = stage_work(p, stage)
    peak_f = PEAK_BF16_TFLOPS if p.dtype == 1 else PEAK_F32_MFMA_TFLOPS
    t_f = flops / (peak_f * 1e12)
    t_b = byts / (PEAK_HBM_GBS * 1e9)
    s = ms * 1e-3
    if stage.startswith("dec_stream") or t_b >= t_f:
        return {"kernel": stage, "bound": "hbm", "achieved": byts / s / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": (byts / s / 1e9) / PEAK_HBM_GBS, "algorithmic_bytes": byts}
    return {"kernel": stage, "bound": "mfma", "achieved": flops / s / 1e12, "peak": peak_f, "unit": "TFLOP/s",
            "frac": (flops / s / 1e12) / peak_f, "algorithmic_flops": flops}


def measure_tail(akv, w, p, cache, q, o, dws, stream, n_tail, reps=5):
    """Decode over the compressed cache plus an exact tail of n_tail tokens per
    KV head (outside the timed steps): the stream part and the tail part
    (tail kernel + merge) separately, HIP events, median of reps.  The tail
    part reads the tail keys and values once: 2*U*H*n_tail*D*e bytes."""
    import torch
    g = torch.Generator(device=o.device).manual_seed(0xA7C4)
    shape = (w.units, w.kv_heads, n_tail, w.head_dim)
    Kt = torch.randn(shape, generator=g, device=o.device).to(w.torch_dtype)
    Vt = torch.randn(shape, generator=g, device=o.device).to(w.torch_dtype)
    akv.decode_attn_tail(p, cache, q, Kt, Vt, n_tail, o, dws, stream)
    torch.cuda.synchronize()
    akv.profile_enable(True)
    akv.profile_read()
    for _ in range(reps):
        akv.decode_attn_tail(p, cache, q, Kt, Vt, n_tail, o, dws, stream)
    torch.cuda.synchronize()
    st = akv.profile_read()
    akv.profile_enable(False)
    tail_ms = sorted(ms for n, ms in st if n == "dec_tail")[reps // 2]
    stream_ms = sorted(ms for n, ms in st if n == "dec_stream")[reps // 2]
    tb = 2 * w.units * w.kv_heads * n_tail * w.head_dim * p.elem_bytes
    return {"n_tail": n_tail, "stream_us": stream_ms * 1e3, "tail_us": tail_ms * 1e3, "tail_bytes": tb,
            "tail_GB_s": tb / (tail_ms * 1e-3) / 1e9, "tail_hbm_frac": tb / (tail_ms * 1e-3) / 1e9 / PEAK_HBM_GBS}


def measure_one_unit(akv, w, cache, p, q, stream, reps=20):
    """Decode of one unit (one layer of one sequence) per launch: the latency a
    per-layer caller sees (outside the timed steps; HIP events, median).  The
    unit's plan and cache bytes are those of unit 0 of the full cache."""
    import torch
    p1 = akv.plan(1, w.kv_heads, w.q_per_kv, w.n_tokens, w.head_dim, w.n_obs, p.dtype, w.theta, w.window)
    _, _, dws1 = akv.alloc(p1, q.device)
    q1 = q[:1].contiguous()
    o1 = torch.empty(1, w.kv_heads * w.q_per_kv, w.head_dim, dtype=torch.float32, device=q.device)
    c1 = cache[:p1.cache_bytes]
    akv.decode_attn(p1, c1, q1, o1, dws1, stream)
    torch.cuda.synchronize()
    akv.profile_enable(True)
    akv.profile_read()
    for _ in range(reps):
        akv.decode_attn(p1, c1, q1, o1, dws1, stream)
    torch.cuda.synchronize()
    st = sorted(ms for n, ms in akv.profile_read() if n == "dec_stream")
    akv.profile_enable(False)
    return {"units": 1, "us": st[len(st) // 2] * 1e3, "bytes": decode_bytes(p1)}


COMPRESS_STAGES = ["obs_stats", "ml_combine", "obs_score", "o_combine", "select", "assign", "obs_util", "util_fix",
                   "topr", "quant"]


def measure_variant(akv, w, K, V, Q, q, stream, reps=3, **kw):
    """Compress and one decode step of the same inputs under other method
    parameters (kw: codec, pool_kv_jointly, ...), outside the timed steps:
    HIP-event stage times, median over reps of the per-call sums."""
    import torch
    try:
        p = akv.plan(w.units, w.kv_heads, w.q_per_kv, w.n_tokens, w.head_dim, w.n_obs,
                     akv.BF16 if w.dtype == "bf16" else akv.F32, w.theta, w.window, **kw)
    except akv.AnchorKVError as e:   # a variant this workload's shape does not allow
        return {"params": kw, "refused": str(e)}
    cache, ws, dws = akv.alloc(p, K.device)
    o = torch.empty(w.units, w.kv_heads * w.q_per_kv, w.head_dim, dtype=torch.float32, device=K.device)
    akv.compress(p, K, V, Q, cache, ws, stream)
    akv.decode_attn(p, cache, q, o, dws, stream)
    torch.cuda.synchronize()
    akv.profile_enable(True)
    akv.profile_read()
    comp, dec = [], []
    for _ in range(reps):
        akv.compress(p, K, V, Q, cache, ws, stream)
        comp.append(sum(ms for n, ms in akv.profile_read() if n in COMPRESS_STAGES))
        akv.decode_attn(p, cache, q, o, dws, stream)
        dec.append(sum(ms for n, ms in akv.profile_read() if n == "dec_stream"))
    akv.profile_enable(False)
    comp_ms, dec_ms = sorted(comp)[reps // 2], sorted(dec)[reps // 2]
    db = decode_bytes(p)
    _, sb = stage_work(p, "dec_stream")
    del cache, ws, dws
    return {"params": kw, "compress_ms": comp_ms, "decode_us": dec_ms * 1e3, "decode_bytes": db,
            "decode_GB_s": db / (dec_ms * 1e-3) / 1e9, "decode_hbm_frac": sb / (dec_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "residual_records_per_unit": p.R_total if p.joint else p.R_K + p.R_V,
            "compression_ratio": p.compression_ratio}


def cpu_baseline(w, budget_s=20.0):
    """The oracle as it stands, on the host cores, with the BLAS thread pool
    set to every core this process may run on: compress + one decode step of
    a bounded sample, extrapolated to the workload's tokens/s.

    Whole units while they take about budget_s each or less; at shapes where
    one unit takes longer (131072 tokens x 8 heads), one KV head of unit 0
    compressed as a one-head unit plus its decode step, scaled by the heads of
    the workload (the oracle's work is per head: the pooled budget only
    changes the residual count)."""
    import numpy as np
    import threadpoolctl
    import kvsynth
    from oracle import anchorkv_oracle as O
    cores = len(os.sched_getaffinity(0))
    threadpoolctl.threadpool_limits(cores)
    per_head = w.n_tokens * w.kv_heads > 8 * 32768
    n = 0
    t_tot = 0.0
    for u in range(w.units):
        if t_tot >= budget_s or (per_head and n == 1):
            break
        n += 1
        s, l = kvsynth.unit_index(w, u)
        K, V, Q = kvsynth.unit_inputs(w, s, l, device="cpu")
        K64, V64, Q64 = (kvsynth.to_f64(x) for x in (K, V, Q))
        q = kvsynth.to_f64(kvsynth.decode_queries(w, 0, units=1)[0])
        if per_head:
            K64, V64, Q64, q = K64[:1], V64[:1], Q64[:w.q_per_kv], q[:w.q_per_kv]
        t0 = time.perf_counter()
        c = O.compress_unit(K64, V64, Q64, w.q_per_kv, w.n_obs, w.theta, w.window, w.elem_bytes)
        O.decode_unit(c, q)
        t_tot += time.perf_counter() - t0
    per_sample = t_tot / n
    step_s = per_sample * (w.units * w.kv_heads if per_head else w.units)
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), cpu_model)
    except OSError:
        pass
    if per_head:
        sample = (f"1 KV head of unit 0 (compress as a 1-head unit + 1 decode step, float64 NumPy) in "
                  f"{per_sample:.1f} s, extrapolated x{w.units * w.kv_heads} heads (labelled extrapolation)")
    else:
        sample = (f"{n} of {w.units} units (compress + 1 decode step each, float64 NumPy), "
                  f"{per_sample:.2f} s/unit, extrapolated to all units")
    return {"value": w.seqs * w.n_tokens / step_s, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model, "blas_threads": cores, "seconds_per_sample": per_sample,
            "extrapolated_step_s": step_s, "sample": sample}


# ---- HBM traffic from rocprofv3 counters (FETCH_SIZE / WRITE_SIZE, KiB per
# dispatch), scaled by what the same counters read for a copy of known size.
COPY_PROBE_BYTES = 1 << 30


def copy_probe():
    """A plain device-to-device copy of COPY_PROBE_BYTES, three times: the
    calibration workload of the traffic counters."""
    import torch
    src = torch.empty(COPY_PROBE_BYTES, dtype=torch.uint8, device="cuda:0")
    src.fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": COPY_PROBE_BYTES, "repeats": 3}), flush=True)


def kernel_stage(name):
    """Stage of the hot path that a kernel (rocprofv3 kernel name) belongs to."""
    import re
    m = re.search(r"k_obs_pipe<(\d)", name) or re.search(r"k_obs<\d, (\d)", name)
    if m:
        return {0: "obs_stats", 1: "obs_score", 2: "obs_util", 3: "util_fix"}[int(m.group(1))]
    for key, stage in (("k_ml_combine", "ml_combine"), ("k_o_combine", "o_combine"), ("k_select", "select"),
                       ("k_assign", "assign"), ("k_topr", "topr"), ("k_quant", "quant"), ("k_headers", "headers"),
                       ("k_dec_stream", "dec_stream"), ("k_dec_rope", "dec_stream"), ("k_dec_merge", "dec_stream"),
                       ("k_dec_tail", "dec_tail"), ("k_rope_table", "obs_stats"),
                       ("k_zero_u32", "zero")):
        if key in name:
            return stage
    return None


def read_counters(d, counter):
    """[(kernel name, value)] of one counter over all dispatches in a rocprofv3 csv output folder."""
    import csv
    import glob
    out = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter:
                out.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return out


def traffic_summary(workload, fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, commands, path=None):
    """profiles/traffic_<workload>.json (or `path`): scaled HBM bytes per launch of every stage."""
    def copy_kib(d, counter):
        vals = [v for n, v in read_counters(d, counter) if "copyBuffer" in n or "copy" in n.lower()]
        if not vals:
            raise SystemExit(f"no copy kernel in {d}")
        return max(vals)
    cf, cw = copy_kib(copy_fetch_dir, "FETCH_SIZE"), copy_kib(copy_write_dir, "WRITE_SIZE")
    f_scale, w_scale = COPY_PROBE_BYTES / (cf * 1024.0), COPY_PROBE_BYTES / (cw * 1024.0)
    per = {}
    for d, counter, key in ((fetch_dir, "FETCH_SIZE", "fetch"), (write_dir, "WRITE_SIZE", "write")):
        for name, v in read_counters(d, counter):
            st = kernel_stage(name)
            if st is None:
                continue
            e = per.setdefault(st, {"fetch": 0.0, "write": 0.0, "n_fetch": 0, "n_write": 0})
            e[key] += v * 1024.0
            e["n_" + key] += 1
    calls = max(1, per.get("headers", {}).get("n_fetch", 1))
    # one decode call = one k_dec_stream dispatch (plus a merge when split)
    dec_calls = max(1, sum(1 for n, _ in read_counters(fetch_dir, "FETCH_SIZE") if "k_dec_stream" in n))
    stages = {}
    for st, e in per.items():
        n = dec_calls if st == "dec_stream" else (e["n_fetch"] or 1) if st == "dec_tail" else calls
        fb, wb = e["fetch"] * f_scale / n, e["write"] * w_scale / n
        stages[st] = {"fetch_bytes": fb, "write_bytes": wb, "bytes": fb + wb, "dispatches_per_call": e["n_fetch"] / n}
    out = {"workload": workload, "source_hash": kernel_source_hash(), "unit": "bytes per call of the stage",
           "copy_calibration": {"bytes": COPY_PROBE_BYTES, "fetch_counter_bytes": cf * 1024.0,
                                "write_counter_bytes": cw * 1024.0, "fetch_scale": f_scale, "write_scale": w_scale},
           "commands": commands, "stages": stages}
    path = path or os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps({"written": path, "stages": {k: round(v["bytes"] / 1e6, 2) for k, v in stages.items()}}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama70b_128k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode-steps", type=int, default=1, help="decode steps per step (default 1)")
    ap.add_argument("--tail", type=int, default=1024,
                    help="tokens of the exact tail in the separate decode-with-tail measurement (0: skip)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the measurements after the timed steps (decode with a tail, one-unit decode)")
    ap.add_argument("--copy-probe", action="store_true", help="run only the traffic-counter calibration copy")
    ap.add_argument("--traffic-summary", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="write profiles/traffic_<workload>.json from four rocprofv3 --pmc csv folders")
    ap.add_argument("--traffic-command", action="append", default=[], help="command recorded with --traffic-summary")
    args = ap.parse_args()
    if args.traffic_summary:
        traffic_summary(args.workload, *args.traffic_summary, args.traffic_command)
        return
    if args.copy_probe:
        copy_probe()
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)

    import torch
    import kvsynth
    import kv_cache_compression_snapkv_amd as akv

    w = kvsynth.WORKLOADS[args.workload]
    dev = "cuda:0"
    torch.cuda.set_device(0)
    print(f"[bench] workload {w.name}: units={w.units} H={w.kv_heads} G={w.q_per_kv} N={w.n_tokens}", file=sys.stderr,
          flush=True)
    dt = akv.BF16 if w.dtype == "bf16" else akv.F32
    p = akv.plan(w.units, w.kv_heads, w.q_per_kv, w.n_tokens, w.head_dim, w.n_obs, dt, w.theta, w.window)
    K = torch.empty(w.units, w.kv_heads, w.n_tokens, w.head_dim, dtype=w.torch_dtype, device=dev)
    V = torch.empty_like(K)
    Q = torch.empty(w.units, w.kv_heads * w.q_per_kv, w.n_obs, w.head_dim, dtype=w.torch_dtype, device=dev)
    for u in range(w.units):
        s, l = kvsynth.unit_index(w, u)
        k, v, q = kvsynth.unit_inputs(w, s, l, device=dev)
        K[u].copy_(k); V[u].copy_(v); Q[u].copy_(q)
        del k, v, q
    cache, ws, dws = akv.alloc(p, dev)
    qs = [kvsynth.decode_queries(w, i, device=dev).contiguous() for i in range(8)]
    o = torch.empty(w.units, w.kv_heads * w.q_per_kv, w.head_dim, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()

    def step(i):
        akv.compress(p, K, V, Q, cache, ws, stream)
        for j in range(args.decode_steps):
            akv.decode_attn(p, cache, qs[(i + j) % len(qs)], o, dws, stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    print("[bench] warmup done", file=sys.stderr, flush=True)
    akv.profile_enable(True)
    akv.profile_read()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    stages = akv.profile_read()
    akv.profile_enable(False)
    extras = not args.no_extras
    tail_rec = measure_tail(akv, w, p, cache, qs[0], o, dws, stream, args.tail) if extras and args.tail > 0 else None
    unit_rec = measure_one_unit(akv, w, cache, p, qs[0], stream) if extras else None
    # the same inputs under the paper's codec, the joint key/value ranking and
    # pre-RoPE key storage (the keys taken as pre-RoPE; refused where the
    # shape has more than 128 observation queries per KV head)
    variants = [measure_variant(akv, w, K, V, Q, qs[0], stream, **kw)
                for kw in (dict(codec=1), dict(pool_kv_jointly=1), dict(rope=1))] if extras else None
    total_s = t1 - t0
    ms_per_step = total_s * 1e3 / args.steps
    print(f"[bench] timed {args.steps} steps: {ms_per_step:.3f} ms/step", file=sys.stderr, flush=True)

    agg, cnt = {}, {}
    for name, ms in stages:
        agg[name] = agg.get(name, 0.0) + ms
        cnt[name] = cnt.get(name, 0) + 1
    stage_ms = {k: agg[k] / cnt[k] for k in agg}           # average per launch
    comp_stages = COMPRESS_STAGES
    dec_stages = ["dec_stream"]
    compress_ms = sum(stage_ms.get(k, 0.0) for k in comp_stages)
    decode_ms = sum(stage_ms.get(k, 0.0) for k in dec_stages)
    dom = max(comp_stages + dec_stages, key=lambda k: stage_ms.get(k, 0.0) * (1 if k in comp_stages else args.decode_steps))
    rl = roofline(p, dom, stage_ms[dom])
    tf = os.path.join(ROOT, "profiles", f"traffic_{w.name}.json")
    tjson = json.load(open(tf)) if os.path.exists(tf) else None

    def stage_traffic(stage):
        """HBM bytes per launch of a stage from the committed counter summary,
        or None when it is missing or the kernels changed since it was taken."""
        if tjson and tjson.get("source_hash") == kernel_source_hash() and stage in tjson.get("stages", {}):
            return tjson["stages"][stage]["bytes"]
        return None
    rl["traffic"] = stage_traffic(dom)
    dec_b = decode_bytes(p)
    seq_tokens = w.seqs * w.n_tokens
    # compress roofline: algorithmic flops and bytes of the whole pass, each at its peak
    comp_flops = sum(stage_work(p, k)[0] for k in ("assign", "obs_stats", "obs_score", "obs_util")) \
        - 2 * stage_work(p, "obs_stats")[0]                 # Q K^T counted once
    comp_bytes = 2 * p.units * p.H * p.N * p.D * p.elem_bytes + p.cache_bytes
    t_roof = max(comp_flops / (PEAK_BF16_TFLOPS * 1e12), comp_bytes / (PEAK_HBM_GBS * 1e9))
    out = {
        "metric": METRIC,
        "value": seq_tokens / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded clustered keys, N(0,1) values, N(0,I) queries; no dataset)",
        "config": {"workload": w.name, "units": w.units, "seqs": w.seqs, "layers": w.layers, "kv_heads": w.kv_heads,
                   "q_per_kv": w.q_per_kv, "n_tokens": w.n_tokens, "head_dim": w.head_dim, "n_obs": w.n_obs,
                   "theta": w.theta, "window": w.window, "decode_steps_per_step": args.decode_steps,
                   "parallelism": "none (1 GPU)"},
        "compress": {"ms": compress_ms, "tokens_per_s": seq_tokens / (compress_ms * 1e-3),
                     "roofline_ms": t_roof * 1e3, "roofline_frac": t_roof * 1e3 / compress_ms,
                     "anchors": p.A, "residuals_per_side_per_unit": p.R_K,
                     "compression_ratio": p.compression_ratio},
        "decode": {"us": decode_ms * 1e3, "bytes": dec_b, "GB_s": dec_b / (decode_ms * 1e-3) / 1e9,
                   "hbm_frac": dec_b / (decode_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                   "note": "cache fits the 256 MB Infinity Cache" if dec_b < 256e6 else "HBM-resident"},
        "stages_ms": stage_ms,
        "decode_tail": tail_rec,
        "decode_one_unit": unit_rec,
        "variants": variants,
        "roofline": rl,
        # each main stage against its own roofline (the contraction of the
        # assignment also against the bf16 MFMA peak, whatever bounds it)
        # the decode kernel against HBM and the whole compression pass against
        # max(flops at the bf16 MFMA peak, bytes at the HBM peak)
        "decode_roofline": dict(roofline(p, "dec_stream", stage_ms["dec_stream"]), traffic=stage_traffic("dec_stream")),
        "compress_roofline": {"bound": "mfma" if comp_flops / (PEAK_BF16_TFLOPS * 1e12) >= comp_bytes / (PEAK_HBM_GBS * 1e9)
                              else "hbm", "roofline_ms": t_roof * 1e3, "measured_ms": compress_ms,
                              "frac": t_roof * 1e3 / compress_ms, "algorithmic_flops": comp_flops,
                              "algorithmic_bytes": comp_bytes},
        "stage_roofline": {k: {"bound": r["bound"], "frac": r["frac"]}
                           for k in ("obs_stats", "obs_score", "assign", "obs_util", "dec_stream") if k in stage_ms
                           for r in [roofline(p, k, stage_ms[k])]},
        "assign_mfma_frac": (stage_work(p, "assign")[0] / (stage_ms["assign"] * 1e-3)
                             / ((PEAK_BF16_TFLOPS if p.dtype == 1 else PEAK_F32_MFMA_TFLOPS) * 1e12)
                             if "assign" in stage_ms else None),
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle) ...", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
