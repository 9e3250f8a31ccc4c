#!/usr/bin/env python3
"""LSH-attention forward benchmark on one MI355X.

One step is one pass of the whole hot path -- hash -> sort -> chunked
attention -> unsort + round combine -- over one batch of seeded synthetic
input with every tensor already resident in HBM.  Default workload: the
headline shape (batch 1, 8 heads, L = 65,536, d = 64, B = 1,024 buckets,
8 hash rounds, chunk 64, causal, self-masked, bf16 inputs).

Prints one JSON line: tokens/s (batch * L per step, all heads and rounds;
`value` over the whole timed region, plus the median step and its p10-p90
range from HIP events around every step), token-head-rounds/s, the roofline
position of the dominant kernel (per-launch time from HIP events on the
stream the kernels run on), the roofline time of a whole step against the
median step, the same figures for the other LSH configs (tiny, small,
medium, verylong), and the fp64 CPU oracle timed on a bounded sample of the
same workload on this host's cores (with the CPU model, and the small
configs on all cores and on one).

    python bench.py [--steps K] [--warmup W] [--workload long] [--no-cpu-baseline]
                    [--no-other-configs] [--union]
    python bench.py --workload local_long | layer_long
"""
import argparse
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2500.0  # dense
METRIC = "LSH-attention fwd tokens/s (all heads, rounds) at L=64K; % of HBM/MFMA roofline"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def algorithmic(w, union=False):
    """Algorithmic work per launch of each kernel (bytes or flops), for the
    per-round output format the workload uses (fp32 rows, or fp16 rows with a
    per-head scale taken from one extra pass over v)."""
    N = w.token_rounds
    T = w.batch * w.heads * w.seq_len
    d = w.head_dim
    bf16 = w.dtype == "bf16"
    el = 2 if bf16 else 4
    oel = 2 if w.o16 else 4   # per-round output rows: fp16 / fp32
    rot = w.heads * w.n_rounds * (w.n_buckets // 2) * d * el
    out = {
        # x read once, rotations read, bucket ids written; contraction flops
        "hash": {"bytes": T * d * el + rot + 4 * N, "flops": N * d * w.n_buckets},
        # keys read twice, perm and inv_perm written
        "sort": {"bytes": 16 * N},
        # per token-round: x and v rows gathered (predecessor reused), perm and
        # bucket id, output row and lse; fp16 rows: v read once more for the
        # output scale
        "attend": {"bytes": N * (2 * d * el + 8 + oel * d + 4) + (T * d * el if w.o16 else 0),
                   "flops": N * 4 * 2 * 64 * d},
        # per token-round: o row, lse and inv_perm read; per token-head: y row written
        "combine": {"bytes": N * (oel * d + 8) + T * 4 * d},
    }
    if union:
        # round-key table: built from buckets and inv_perm (8 B per token-round
        # read, the keys of rounds 0 .. R-2 per token written: 4, 8 or 16 per
        # token), then gathered with every key row of round r for rounds 0 .. r-1
        R = w.n_rounds
        stride = 4 if R <= 5 else (8 if R <= 9 else 16)
        out["attend"]["bytes"] += 8 * N + 4 * stride * T + 4 * T * (R * (R - 1) // 2)
    return out


def fixed_count_bytes(w):
    """The fixed per-step byte counts every build is compared on (bf16 or fp32
    inputs, fp32 per-round rows, predecessor chunk reused): hash T*2d + 4N
    (bf16), sort 16 N, attention 524 N (780 N for fp32 inputs), combine
    264 N + 256 T."""
    N = w.token_rounds
    T = w.batch * w.heads * w.seq_len
    el = 2 if w.dtype == "bf16" else 4
    return {"hash": T * w.head_dim * el + 4 * N, "sort": 16 * N,
            "attend": N * (2 * w.head_dim * el + 8 + 4 * w.head_dim + 4),
            "combine": N * (4 * w.head_dim + 8) + T * 4 * w.head_dim}


def path_targets(w, per, union=False):
    """The two target branches at this shape: the chunk attention's flops
    against the dense bf16 matrix-core peak (target 0.40), and the bytes of
    sort + attention + combine against HBM peak (target 0.60), the bytes
    counted as this layout moves them and as the fixed counts above."""
    work = algorithmic(w, union)
    fixed = fixed_count_bytes(w)
    t_att = per["attend"] * 1e-3
    t_path = sum(per[n] for n in ("sort", "attend", "combine")) * 1e-3
    mine = sum(work[n]["bytes"] for n in ("sort", "attend", "combine"))
    theirs = sum(fixed[n] for n in ("sort", "attend", "combine"))
    mfma = work["attend"]["flops"] / t_att / (BF16_MFMA_PEAK_TFLOPS * 1e12)
    hbm = mine / t_path / (HBM_PEAK_GBS * 1e9)
    hbm_fixed = theirs / t_path / (HBM_PEAK_GBS * 1e9)
    return {"attend_mfma_frac": round(mfma, 4), "attend_mfma_target": 0.40,
            "path": "sort + attend + combine", "path_us": round(t_path * 1e6, 2),
            "path_bytes": mine, "path_hbm_frac": round(hbm, 4),
            "path_bytes_fixed_counts": theirs, "path_hbm_frac_fixed_counts": round(hbm_fixed, 4),
            "path_hbm_target": 0.60,
            "met": bool(mfma >= 0.40 or hbm >= 0.60)}


def algorithmic_local(w):
    """Local attention, one launch: x and v read once, y and lse written; the
    flops are the score and value products of every query's window."""
    T = w.batch * w.heads * w.seq_len
    d = w.head_dim
    el = 2 if w.dtype == "bf16" else 4
    C = w.seq_len // w.chunk_len
    after = 0 if w.causal else w.look_after
    keys = sum(min(C - 1, c + after) - max(0, c - w.look_before) + 1 for c in range(C)) * w.chunk_len
    return {"bytes": T * (2 * d * el + 4 * d + 4),
            "flops": w.batch * w.heads * w.chunk_len * keys * 4 * d}


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current source of that kernel (else None)."""
    from lsh_sparse_attention_hash_amd.rocprof_summary import source_digest
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    digest = source_digest(kernel)
    pat = re.compile(r"^\|\s*%s\s*\|\s*%s\s*\|\s*([0-9a-f]+)\s*\|\s*([0-9.eE+]+)\s*\|" %
                     (kernel, workload))
    for line in open(path):
        m = pat.match(line)
        if m and m.group(1) == digest:
            return float(m.group(2))
    return None


def measured_kernel_traffic(step, workload, kernels):
    """HBM bytes of a call made of several kernel launches: sum of count x
    (read + written bytes per launch) over {kernel name: count}, from the
    per-kernel table of the committed counter summary, if the step's sources
    are unchanged since it was taken (else None)."""
    if measured_traffic(step, workload) is None:
        return None
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.md")
    found = {}
    for line in open(path):
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) == 3 and cells[0] in kernels:
            found[cells[0]] = (float(cells[1]) + float(cells[2])) * 1e6
    if set(found) != set(kernels):
        return None
    return sum(kernels[k] * found[k] for k in kernels)


def measured_busy(step, workload, kernel=None):
    """Fraction of the matrix cores' cycles busy during a launch, from the
    committed rocprofv3 counter summary, if it was taken on the step's current
    sources (else None): the step's kernel with the most matrix-core work, or
    the named kernel."""
    from lsh_sparse_attention_hash_amd.rocprof_summary import source_digest
    path = os.path.join(ROOT, "profiles", f"mfma_busy_{workload}.md")
    if not os.path.exists(path):
        return None
    rows = [[c.strip() for c in line.strip().strip("|").split("|")] for line in open(path)
            if line.startswith("|")]
    steprow = [r for r in rows if len(r) == 5 and r[0] == step and r[1] == workload]
    if not steprow or steprow[0][2] != source_digest(step):
        return None
    if kernel is None:
        return float(steprow[0][4])
    krow = [r for r in rows if len(r) == 8 and r[0] == kernel]
    return float(krow[0][7]) if krow else None


def cpu_baseline(w, inputs, union=False, small_configs=True):
    """The fp64 oracle on a bounded sample of the workload: every head for the
    shapes up to L = 64K (a few seconds on a many-core host), one head of the
    half-million-token shape.  With `small_configs`, also the full forward of
    the tiny, small and medium configs on all cores and on one core."""
    threads = len(os.sched_getaffinity(0))
    os.environ["OMP_NUM_THREADS"] = str(threads)
    from lsh_sparse_attention_hash_amd import synth
    from oracle import oracle
    oracle.build(force=False)
    oracle.set_threads(threads)
    hs = w.heads if w.seq_len <= 65536 else 1
    qk = synth.to_f64(inputs["qk"][:, :hs], w.dtype)
    v = synth.to_f64(inputs["v"][:, :hs], w.dtype)
    rot = synth.to_f64(inputs["rot"][:hs], w.dtype)
    t0 = time.perf_counter()
    (oracle.forward_union if union else oracle.forward)(qk, v, rot, w.n_buckets, w.n_rounds,
                                                        w.chunk_len, w.causal, w.self_mask)
    dt = time.perf_counter() - t0
    full_est = dt * w.heads / hs
    out = {"value": w.batch * w.seq_len / full_est, "unit": "tokens/s", "cores": threads,
           "cpu_model": cpu_model(), "kind": "oracle", "seconds": round(dt, 3),
            "sample": f"{hs} of {w.heads} heads (batch {w.batch}, L={w.seq_len}, all "
                      f"{w.n_rounds} rounds), full fp64 forward (hash, sort, "
                      f"{'set-union attend' if union else 'attend'}, combine)" +
                      ("" if hs == w.heads else
                                     f"; tokens/s scaled by {w.heads // hs}x to all heads")}
    if not union and small_configs:
        out["small_configs"] = cpu_small_configs(synth)
    return out


def bench_layer(args, binding, torch, synth):
    """One reversible layer: one step is lsh_reversible_forward (qk/v maps,
    the four LSH calls, output map, chunked FFN).  The same calls are then
    timed one by one for the per-kernel roofline."""
    w = synth.LAYER_WORKLOADS[args.workload]
    log(f"[bench] layer workload {w}")
    inp = synth.make_layer_inputs(w)
    lc = binding.make_layer_config(w)
    wd = binding.layer_weights_to_device(inp)
    x1 = torch.from_numpy(inp["x1"]).cuda()
    x2 = torch.from_numpy(inp["x2"]).cuda()
    y1, y2 = torch.empty_like(x1), torch.empty_like(x2)
    layer = binding.Layer(lc, wd)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        layer.forward(x1, x2, y1, y2)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    t0 = time.perf_counter()
    start.record(stream)
    for k in range(args.steps):
        ev[k][0].record(stream)
        layer.forward(x1, x2, y1, y2)
        ev[k][1].record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(end) / args.steps
    log(f"[bench] {args.steps} layer steps: {ms:.4f} ms/step (wall {wall:.3f} s)")

    # the same work call by call
    H, L, b, D, F = w.heads, w.seq_len, w.batch, w.d_model, w.d_ff
    qk = torch.empty((b, H, L, 64), dtype=torch.bfloat16, device="cuda")
    v = torch.empty_like(qk)
    att = binding.Forward(binding.attention_config(lc))
    ffn_ws = torch.empty(max(16, binding.lsh_ffn_workspace_bytes(lc)), dtype=torch.uint8,
                         device="cuda")
    calls = {
        "project_qkv": lambda: binding.lsh_project_qkv(lc, x2, wd["w_qk"], wd["w_v"], qk, v),
        "hash": lambda: att.hash(qk, wd["rot"]),
        "sort": lambda: att.sort(),
        "attend": lambda: att.attend(qk, v),
        "combine": lambda: att.combine(v),
        "project_out": lambda: binding.lsh_project_out(lc, att.y, wd["w_o"], x1, 0, y1),
        "ffn": lambda: binding.lsh_ffn(lc, y1, wd["w_1"], wd["b_1"], wd["w_2"], wd["b_2"], x2, 0,
                                       y2, ffn_ws),
    }
    for f in calls.values():
        f()
    torch.cuda.synchronize()
    per = {}
    for name, f in calls.items():
        a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(args.steps):
            f()
        e.record(stream)
        torch.cuda.synchronize()
        per[name] = a.elapsed_time(e) / args.steps
    if args.copy_calibration:
        copy_calibration(torch)
    M = b * L
    aw = synth.Workload(w.name, b, H, L, 64, w.n_buckets, w.n_rounds, 64, w.causal, w.self_mask,
                        "bf16", w.seed)
    work = algorithmic(aw)
    work["project_qkv"] = {"flops": 2 * M * 2 * D * D, "bytes": M * D * 4 + 2 * D * D * 2 + 2 * M * D * 2}
    work["project_out"] = {"flops": 2 * M * D * D, "bytes": M * D * 4 * 3 + D * D * 2}
    # x and the residual read, the output written (fp32), both weights read,
    # and the bf16 hidden activation of every chunk written and read back
    work["ffn"] = {"flops": 2 * 2 * M * D * F,
                   "bytes": M * D * 4 * 3 + 2 * D * F * 2 + 2 * M * F * 2}
    kernels = {}
    for n, t_ms in per.items():
        t = t_ms * 1e-3
        kb = {"ms": round(t_ms, 5), "algorithmic_bytes": work[n]["bytes"],
              "GBps": round(work[n]["bytes"] / t / 1e9, 1)}
        if "flops" in work[n]:
            kb["algorithmic_flops"] = work[n]["flops"]
            kb["TFLOPs"] = round(work[n]["flops"] / t / 1e12, 2)
        kernels[n] = kb
    # matrix-core busy fraction per launch, from the committed counter summary
    busy_of = {"hash": ("hash", None), "attend": ("attend", None),
               "project_qkv": ("gemm", "lsh::gemm_bf16_kernel<0, 0>"),
               "project_out": ("gemm", "lsh::gemm_bf16_kernel<2, 1>")}
    for n, (st, k) in busy_of.items():
        kernels[n]["mfma_busy"] = measured_busy(st, w.name, k)
    kernels["ffn"]["mfma_busy"] = {k: measured_busy("gemm", w.name, k)
                                   for k in ("lsh::gemm_bf16_kernel<0, 2>",
                                             "lsh::gemm_bf16_kernel<1, 1>")}
    log("[bench] per call ms: " + ", ".join(f"{n} {t:.4f}" for n, t in per.items()))
    gemms = ("project_qkv", "project_out", "ffn")
    dom = max(per, key=lambda n: per[n])
    t = per[dom] * 1e-3
    if dom in gemms or dom == "hash":
        ach = work[dom]["flops"] / t / 1e12
        roof = {"kernel": dom, "bound": "mfma", "achieved": round(ach, 2),
                "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(ach / BF16_MFMA_PEAK_TFLOPS, 4)}
    else:
        ach = work[dom]["bytes"] / t / 1e9
        roof = {"kernel": dom, "bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4)}
    if dom == "ffn":
        chunks = -(-M // (w.ffn_chunk or M))
        roof["traffic"] = measured_kernel_traffic(
            "gemm", w.name, {"lsh::gemm_bf16_kernel<0, 2>": chunks,
                             "lsh::gemm_bf16_kernel<1, 1>": chunks})
    elif dom in gemms:
        k = {"project_qkv": "lsh::gemm_bf16_kernel<0, 0>",
             "project_out": "lsh::gemm_bf16_kernel<2, 1>"}[dom]
        roof["traffic"] = measured_kernel_traffic("gemm", w.name, {k: 1})
    else:
        roof["traffic"] = measured_traffic(dom, w.name)
    return {
        "metric": "reversible LSH layer fwd tokens/s (qk/v maps, LSH attention, output map, "
                  "chunked FFN) at L=64K; % of roofline",
        "value": round(M / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "step_ms": pct([a.elapsed_time(e) for a, e in ev]), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) stream, N(0,1/fan_in) bf16 weights, random rotations)",
        "config": {"workload": w.name, "batch": b, "seq_len": L, "d_model": D, "heads": H,
                   "d_ff": F, "n_buckets": w.n_buckets, "n_rounds": w.n_rounds,
                   "causal": w.causal, "self_mask": w.self_mask, "ffn_chunk": w.ffn_chunk},
        "roofline": roof, "kernels": kernels,
        "gemm_TFLOPs": round(sum(work[n]["flops"] for n in gemms) /
                             (sum(per[n] for n in gemms) * 1e-3) / 1e12, 2),
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline_layer(w, inp, synth),
    }


def cpu_baseline_layer(w, inp, synth):
    """The fp64 oracle of the whole layer forward (dense maps in plain loops,
    the LSH oracle for the attention) over the full workload."""
    threads = len(os.sched_getaffinity(0))
    os.environ["OMP_NUM_THREADS"] = str(threads)
    import numpy as np
    from oracle import layer as olayer
    from oracle import oracle
    oracle.build(force=False)
    oracle.set_threads(threads)
    log("[bench] timing the CPU oracle of the layer")
    wf = {k: synth.to_f64(inp[k], "bf16") for k in ("w_qk", "w_v", "w_o", "rot", "w_1", "w_2")}
    wf.update({k: inp[k].astype(np.float64) for k in ("b_1", "b_2")})
    cfg = dict(n_buckets=w.n_buckets, n_rounds=w.n_rounds, causal=w.causal,
               self_mask=w.self_mask, ffn_chunk=w.ffn_chunk)
    t0 = time.perf_counter()
    olayer.reversible_forward(inp["x1"].astype(np.float64), inp["x2"].astype(np.float64), wf, cfg)
    dt = time.perf_counter() - t0
    return {"value": w.batch * w.seq_len / dt, "unit": "tokens/s", "cores": threads,
            "cpu_model": cpu_model(), "kind": "oracle", "seconds": round(dt, 3),
            "sample": f"the whole layer forward (batch {w.batch}, L={w.seq_len}, d_model "
                      f"{w.d_model}, d_ff {w.d_ff}), fp64"}


def copy_calibration(torch):
    """Plain device copies of known size, after the timed steps: the reference
    that scales the HBM byte counters of a profiled run."""
    nbytes = 512 << 20
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[bench] copy calibration: 3 x {nbytes} B device copies")


def bench_local(args, w, inputs, binding, torch):
    """Local chunked attention: one step is one lsh_local_attend call."""
    qk = binding.to_device(inputs["qk"], w.dtype)
    v = binding.to_device(inputs["v"], w.dtype)
    loc = binding.Local(binding.config_for(w), w.look_before, w.look_after)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        loc.run(qk, v, stream)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for k in range(args.steps):
        ev[k][0].record(stream)
        loc.run(qk, v, stream)
        ev[k][1].record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(end) / args.steps
    per = sum(a.elapsed_time(b) for a, b in ev) / args.steps
    log(f"[bench] {args.steps} steps: {ms:.4f} ms/step (wall {wall:.3f} s); local_attend {per:.4f} ms")
    if args.copy_calibration:
        copy_calibration(torch)
    work = algorithmic_local(w)
    t = per * 1e-3
    ach = work["bytes"] / t / 1e9
    roof = {"kernel": "local_bf16_kernel" if w.dtype == "bf16" else "local_f32_kernel",
            "bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": measured_traffic("local", w.name)}
    result = {
        "metric": "local chunked attention fwd tokens/s (all heads) at L=64K; % of HBM roofline",
        "value": round(w.batch * w.seq_len / (ms * 1e-3), 1),
        "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "step_ms": pct([a.elapsed_time(b) for a, b in ev]),
        "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) inputs)",
        "config": {"workload": w.name, "batch": w.batch, "heads": w.heads, "seq_len": w.seq_len,
                   "head_dim": w.head_dim, "chunk_len": w.chunk_len,
                   "look_before": w.look_before, "look_after": w.look_after,
                   "causal": w.causal, "self_mask": w.self_mask},
        "roofline": roof,
        "kernels": {"local_attend": {"ms": round(per, 5), "algorithmic_bytes": work["bytes"],
                                     "GBps": round(ach, 1), "algorithmic_flops": work["flops"],
                                     "TFLOPs": round(work["flops"] / t / 1e12, 2),
                                     "mfma_busy": measured_busy("local", w.name)}},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample")
        result["cpu_baseline"] = cpu_baseline_local(w, inputs)
        log(f"[bench] cpu baseline: {result['cpu_baseline']}")
    return result


def cpu_baseline_local(w, inputs):
    """The fp64 oracle's local attention over every head of the workload."""
    threads = len(os.sched_getaffinity(0))
    os.environ["OMP_NUM_THREADS"] = str(threads)
    from lsh_sparse_attention_hash_amd import synth
    from oracle import oracle
    oracle.build(force=False)
    oracle.set_threads(threads)
    qk = synth.to_f64(inputs["qk"], w.dtype)
    v = synth.to_f64(inputs["v"], w.dtype)
    t0 = time.perf_counter()
    oracle.local_attend(qk, v, w.chunk_len, w.look_before, w.look_after, w.causal, w.self_mask)
    dt = time.perf_counter() - t0
    return {"value": w.batch * w.seq_len / dt, "unit": "tokens/s", "cores": threads,
            "cpu_model": cpu_model(), "kind": "oracle", "seconds": round(dt, 3),
            "sample": f"all {w.heads} heads (batch {w.batch}, L={w.seq_len}), full fp64 local "
                      f"attention"}


def pct(xs):
    """Median and the p10-p90 range of a list of times (ms)."""
    import numpy as np
    a = np.asarray(xs, dtype=np.float64)
    return {"median": round(float(np.median(a)), 5), "p10": round(float(np.percentile(a, 10)), 5),
            "p90": round(float(np.percentile(a, 90)), 5)}


def time_forward(args, w, inputs, binding, torch, union=False):
    """Warm-up steps, then `args.steps` timed passes of the four calls on one
    stream with HIP events around each pass and each call (recorded on the
    stream the calls are launched on).  Inputs and scratch are allocated
    before the timed region."""
    qk = binding.to_device(inputs["qk"], w.dtype)
    v = binding.to_device(inputs["v"], w.dtype)
    rot = binding.to_device(inputs["rot"], w.dtype)
    f = binding.Forward(binding.config_for(w))
    stream = torch.cuda.current_stream()
    attend = f.attend_union if union else f.attend
    for _ in range(args.warmup):
        f.run(qk, v, rot, union=union)
    torch.cuda.synchronize()
    names = ("hash", "sort", "attend", "combine")
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for k in range(args.steps):
        e = ev[k]
        e[0].record(stream)
        f.hash(qk, rot)
        e[1].record(stream)
        f.sort()
        e[2].record(stream)
        attend(qk, v)
        e[3].record(stream)
        f.combine(v)
        e[4].record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(end) / args.steps
    kt = {n: [ev[k][i].elapsed_time(ev[k][i + 1]) for k in range(args.steps)]
          for i, n in enumerate(names)}
    steps = [ev[k][0].elapsed_time(ev[k][4]) for k in range(args.steps)]
    per = {n: sum(kt[n]) / args.steps for n in names}
    log(f"[bench] {w.name}: {args.steps} steps: {ms:.4f} ms/step (wall {wall:.3f} s); per call "
        "ms: " + ", ".join(f"{n} {per[n]:.4f}" for n in names))
    out = {"ms": ms, "per": per, "step_pct": pct(steps),
           "kernel_pct": {n: pct(kt[n]) for n in names},
           "fallback_rows": int(f.fallback_rows.item()) // (args.warmup + args.steps)}
    del f, qk, v, rot
    torch.cuda.synchronize()
    return out


def roofline_us(w, union=False):
    """Time of one forward at the roofline: each call at the larger of its
    algorithmic bytes at HBM peak and its algorithmic flops at the dense bf16
    MFMA peak (flops counted for the hash only: the attention's intensity sits
    far below the ridge point)."""
    work = algorithmic(w, union)
    t = {n: work[n]["bytes"] / (HBM_PEAK_GBS * 1e9) for n in work}
    t["hash"] = max(t["hash"], work["hash"]["flops"] / (BF16_MFMA_PEAK_TFLOPS * 1e12))
    return {n: round(x * 1e6, 2) for n, x in t.items()}


def forward_summary(w, tm, union=False):
    """Median-based figures of one config: tokens/s and token-head-rounds/s
    over the median step, and the roofline time over the median step."""
    med = tm["step_pct"]["median"] * 1e-3
    roof = roofline_us(w, union)
    t_roof = sum(roof.values())
    return {"tokens_per_s_median": round(w.batch * w.seq_len / med, 1),
            "token_head_rounds_per_s": round(w.token_rounds / med, 1),
            "roofline_us": {**roof, "total": round(t_roof, 2)},
            "frac_of_roofline_time": round(t_roof * 1e-6 / med, 4)}


def other_configs(args, w0, binding, torch, synth):
    """The same protocol on every other LSH-attention config (throughput only;
    their parity is covered by the tests)."""
    res = {}
    for name, w in synth.WORKLOADS.items():
        if name == w0.name or w.is_local:
            continue
        inputs = synth.make_inputs(w)
        tm = time_forward(args, w, inputs, binding, torch)
        del inputs
        res[name] = {"batch": w.batch, "heads": w.heads, "seq_len": w.seq_len,
                     "n_buckets": w.n_buckets, "n_rounds": w.n_rounds, "dtype": w.dtype,
                     "ms_per_step": round(tm["ms"], 5), "step_ms": tm["step_pct"],
                     **forward_summary(w, tm),
                     "kernels_ms": {n: round(x, 5) for n, x in tm["per"].items()},
                     "hash_fallback_rows_per_step": tm["fallback_rows"]}
    return res


def cpu_model():
    """The host CPU's model name, as lscpu prints it (from /proc/cpuinfo)."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_small_configs(synth):
    """The oracle's full forward on the small configs, on every core the
    process may use and on one core."""
    from oracle import oracle
    threads = len(os.sched_getaffinity(0))
    res = {}
    for name in ("tiny", "small", "medium"):
        w = synth.WORKLOADS[name]
        inp = synth.make_inputs(w)
        qk, v, rot = (synth.to_f64(inp[k], w.dtype) for k in ("qk", "v", "rot"))
        row = {}
        for th in (threads, 1):
            oracle.set_threads(th)
            t0 = time.perf_counter()
            oracle.forward(qk, v, rot, w.n_buckets, w.n_rounds, w.chunk_len, w.causal,
                           w.self_mask)
            row["seconds_1_thread" if th == 1 else "seconds"] = round(time.perf_counter() - t0, 4)
        row["tokens_per_s"] = round(w.batch * w.seq_len / row["seconds"], 1)
        res[name] = row
    oracle.set_threads(threads)
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="long")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="time the headline config only (skip tiny/small/medium/verylong)")
    ap.add_argument("--union", action="store_true",
                    help="set reading of the union over rounds (lsh_chunk_attend_union)")
    ap.add_argument("--o-format", default="auto", choices=("auto", "f32", "f16_scaled"),
                    help="per-round output rows between attention and combine (auto: scaled "
                         "fp16 for bf16 inputs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed steps, run plain device copies of known size "
                         "(reference for HBM counter scaling)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(heads would shard across GPUs with no communication); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np  # noqa: F401
    import torch
    from lsh_sparse_attention_hash_amd import build as lib_build
    if not lib_build.is_current():
        log("[bench] liblsh.so is missing or stale: rebuilding")
        lib_build.build()
    from lsh_sparse_attention_hash_amd import binding, synth

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    torch.cuda.set_device(0)
    if args.workload in synth.LAYER_WORKLOADS:
        print(json.dumps(bench_layer(args, binding, torch, synth)), flush=True)
        return
    w = synth.WORKLOADS[args.workload]
    if not w.is_local:
        w = w.replace(o_format=args.o_format)
    log(f"[bench] workload {w}")
    inputs = synth.make_inputs(w)
    if w.is_local:
        print(json.dumps(bench_local(args, w, inputs, binding, torch)), flush=True)
        return
    tm = time_forward(args, w, inputs, binding, torch, args.union)
    ms, per = tm["ms"], tm["per"]
    names = ("hash", "sort", "attend", "combine")
    if args.copy_calibration:
        copy_calibration(torch)

    work = algorithmic(w, args.union)
    fixed = fixed_count_bytes(w)
    kernels = {}
    for n in names:
        t = per[n] * 1e-3
        kb = {"ms": round(per[n], 5), "median_ms": round(tm["kernel_pct"][n]["median"], 5),
              "algorithmic_bytes": work[n]["bytes"], "GBps": round(work[n]["bytes"] / t / 1e9, 1),
              "hbm_frac": round(work[n]["bytes"] / t / 1e9 / HBM_PEAK_GBS, 4),
              "fixed_count_bytes": fixed[n],
              "hbm_frac_fixed_counts": round(fixed[n] / t / 1e9 / HBM_PEAK_GBS, 4)}
        if "flops" in work[n]:
            kb["algorithmic_flops"] = work[n]["flops"]
            kb["TFLOPs"] = round(work[n]["flops"] / t / 1e12, 2)
            kb["mfma_busy"] = measured_busy(n, w.name + ("_union" if args.union else ""))
        kernels[n] = kb
    # the dominant step by time among the single-launch kernels
    dom = max(("hash", "attend", "combine"), key=lambda n: per[n])
    t = per[dom] * 1e-3
    if dom == "hash":
        ach = work["hash"]["flops"] / t / 1e12
        # the epilogue the library picks: keys up to 1,024 directions, else quads
        epi = "KeyEpilogue" if w.n_buckets // 2 <= 1024 else "QuadEpilogue"
        roof = {"kernel": f"hash_bf16_kernel<{epi}>", "bound": "mfma", "achieved": round(ach, 2),
                "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / BF16_MFMA_PEAK_TFLOPS, 4)}
    else:
        ach = work[dom]["bytes"] / t / 1e9
        roof = {"kernel": {"attend": "attend_bf16_kernel", "combine": "combine_kernel"}[dom],
                "bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4)}
    roof["traffic"] = measured_traffic(dom, w.name + ("_union" if args.union else ""))
    # what the HIP events around the call time (one ABI call can launch two
    # kernels; the traffic is that of the same kernels)
    roof["timed"] = {"hash": "lsh_hash: hash_bf16_kernel<...Epilogue> + hash_settle_kernel",
                     "attend": ("lsh_chunk_attend_union: union_keys_kernel + vmax_kernel + "
                                "attend_bf16_kernel" if args.union else
                                "lsh_chunk_attend: vmax_kernel + attend_bf16_kernel"),
                     "combine": "lsh_unsort_combine: combine_kernel"}[dom]

    result = {
        "metric": METRIC if not args.union else
        "LSH-attention fwd tokens/s, set union of rounds (all heads) at L=64K; % of roofline",
        "value": round(w.batch * w.seq_len / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) / Gaussian-mixture inputs, random rotations)",
        "config": {"workload": w.name + ("+union" if args.union else ""), "batch": w.batch,
                   "heads": w.heads, "seq_len": w.seq_len,
                   "head_dim": w.head_dim, "n_buckets": w.n_buckets, "n_rounds": w.n_rounds,
                   "chunk_len": w.chunk_len, "causal": w.causal, "self_mask": w.self_mask,
                   "o_format": "f16_scaled" if w.o16 else "f32",
                   "qk": ("gaussian mixture, %d clusters" % w.n_clusters) if w.n_clusters
                   else "N(0,1)"},
        "step_ms": tm["step_pct"],
        **forward_summary(w, tm, args.union),
        "roofline": roof,
        "targets": path_targets(w, per, args.union),
        "kernels": kernels,
        "hash_fallback_rows_per_step": tm["fallback_rows"],
        "cpu_baseline": None,
    }
    if not args.union and not args.no_other_configs:
        if w.dtype == "bf16":
            # the same shape with the other per-round output format
            wa = w.replace(o_format="f32" if w.o16 else "f16_scaled")
            ta = time_forward(args, wa, inputs, binding, torch)
            result["other_o_format"] = {
                "o_format": "f16_scaled" if wa.o16 else "f32",
                "ms_per_step": round(ta["ms"], 5), "step_ms": ta["step_pct"],
                "value": round(w.batch * w.seq_len / (ta["ms"] * 1e-3), 1),
                "kernels_ms": {n: round(x, 5) for n, x in ta["per"].items()},
                "targets": path_targets(wa, ta["per"])}
        result["other_configs"] = other_configs(args, w, binding, torch, synth)
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample")
        result["cpu_baseline"] = cpu_baseline(w, inputs, args.union)
        log(f"[bench] cpu baseline: {result['cpu_baseline']}")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
