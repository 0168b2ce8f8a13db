"""Benchmark: Engram forward tokens/s on one MI355X, with per-stage roofline fractions.

    python bench.py [--steps K] [--warmup W] [--config 2] [--no-cpu-baseline] [--mxfp8]
                    [--overlap]

A step is one pass of the whole hot path over the batch: the hash for every
layer, then per layer the row gather and the projection, then the gate of
every layer (one pass over the highway when there are several).  The
inputs are resident in HBM before timing starts.  The timed region issues the
same C-ABI calls that engram_forward makes, in its order, on one stream, and
records HIP events between them, so each kernel's average duration comes from
the timed run itself.  For Q2_K tables that is engram_project_q2k (row gather
and projection fused into one kernel); the two-kernel path it replaces
(engram_rows, engram_project) is timed after the steps for comparison, as is
engram_forward itself.  With --mxfp8 (FP8 tables only) the layers carry an
MXFP8 copy of wkv, made once before timing, and the step runs the MXFP8
projection in place of rows -> projection, as engram_forward picks it:
engram_stage_mxfp8 (the raw FP8 rows copied into an MXFP8 activation) then
engram_project_mxfp8_staged (block-scaled matrix cores), or, for up to 64
tokens, engram_project_mxfp8's weight-streaming form.  With --overlap (several layers) the layers after the
first are projected on a second stream beside the first layer's projection
and gate, each later gate waiting for its layer (a comparison schedule).

Prints ONE JSON line: the headline metric, plus `roofline` for the dominant
kernel (the bf16 MFMA projection), `stages` for every kernel, and
`cpu_baseline` (the CPU oracle, timed on a bounded sample).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Engram forward tokens/s at T=8192 (1 GPU); % HBM roofline gather+gate, % MFMA GEMM"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published (no sparsity)
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense fp8 MFMA, published (no sparsity)
Q2K_FUSED_MAX_BYTES = 2147483504   # engram.h: ENGRAM_Q2K_FUSED_MAX_BYTES
MX_MAX_BYTES = 2147483632          # engram.h: ENGRAM_MX_MAX_WEIGHT_BYTES
SKINNY_MAX_TOKENS = 128            # engram_project streams wkv at or below this many tokens
CPU_SAMPLE_TOKENS = 8192       # whole sequences of the workload, up to this many tokens
CPU_MIN_SECONDS = 10.0         # the CPU baseline repeats its sample at least this long
CPU_MAX_PASSES = 100


def profiled_traffic(profile: str) -> int | None:
    """HBM bytes per launch from a committed rocprofv3 summary, or None.

    The summary records the FETCH_SIZE + WRITE_SIZE bytes (copy-calibrated)
    and the sha256 of the kernel's sources (concatenated, in the order
    listed) it was taken on; different sources today mean the number is
    stale, so none is reported.
    """
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", profile)
    try:
        text = open(path).read()
        traffic = int(re.search(r"^traffic_bytes_per_launch: (\d+)$", text, re.M).group(1))
        srcs = re.search(r"^source: (.+)$", text, re.M).group(1).split()
        sha = re.search(r"^source_sha256: ([0-9a-f]+)$", text, re.M).group(1)
        h = hashlib.sha256()
        for src in srcs:
            h.update(open(os.path.join(ROOT, src), "rb").read())
    except (OSError, AttributeError, ValueError):
        return None
    return traffic if h.hexdigest() == sha else None


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def algorithmic(spec, token_mask) -> dict:
    """Bytes (or FLOP) each stage must move per call, from the method's sizes."""
    T, L, cols, hc, dim = spec.T, len(spec.layer_ids), spec.cols, spec.hc, spec.dim
    live = T if token_mask is None else int((token_mask != 0).sum())
    row_bytes = 84 if spec.fmt == "q2k" else 256 + 8
    per_tok_rows = cols * 4 + cols * row_bytes + cols * 256 * 2
    per_live_gate = 2 * hc * dim * 4 + (hc + 1) * dim * 2
    mask_bytes = 0 if token_mask is None else T
    return {
        # all layers' gates in one pass: h read and written once, every kv read
        "gate_pass": live * (2 * hc * dim * 4 + L * (hc + 1) * dim * 2) + mask_bytes,
        "hash": T * 4 + T * L * cols * 4,
        "rows": T * per_tok_rows,                 # per layer
        "project": 2.0 * T * spec.K * spec.N,     # FLOP per layer
        "gate": live * per_live_gate + mask_bytes,  # per layer
        # the MXFP8 staging: ids, then each row's 256 codes + 8 scale bytes read and written
        "stage_mx": T * cols * (4 + 2 * (256 + 8)),
        "rows_per_token": per_tok_rows,
        "gate_per_token": per_live_gate,
    }


def cpu_baseline(wl, mx: bool = False) -> dict:
    """The oracle, as it stands, on the workload's first whole sequences (<= CPU_SAMPLE_TOKENS).

    With mx, the oracle's layers carry its own MXFP8 copy of wkv, made before
    the clock starts (as the GPU's is).
    """
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    s = wl.spec
    cu = [int(c) for c in wl.cu_seqlens]
    n_seq = max(1, max(i for i in range(1, len(cu)) if cu[i] <= CPU_SAMPLE_TOKENS or i == 1))
    n = cu[n_seq]
    sl = slice(0, n)
    opt = lambda a: None if a is None else a[sl]
    layers = [l.as_dict() for l in wl.layers]
    if mx:
        for d in layers:
            d["wkv_mx"] = oracle.quantize_mxfp8(d["wkv"])
    # Whole passes over the sample until CPU_MIN_SECONDS have gone by (a
    # bounded amount of CPU work however small the sample), mean rate.
    passes, t0 = 0, time.perf_counter()
    while True:
        oracle.forward(wl.h[sl], wl.cids[sl], np.array(cu[:n_seq + 1], dtype=np.int32),
                       wl.hash_params, layers, s.eps, s.clamp,
                       s.dot_scale, doc_ids=opt(wl.doc_ids), token_mask=opt(wl.token_mask),
                       lookback=None if wl.lookback is None else wl.lookback[:n_seq],
                       lookback_live=None if wl.lookback_live is None else wl.lookback_live[:n_seq])
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= CPU_MIN_SECONDS or passes >= CPU_MAX_PASSES:
            break
    return {"value": passes * n / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {n} tokens ({n_seq} sequences) of the {s.name} workload, whole "
                      f"forward (hash, rows, {'MXFP8 ' if mx else ''}projection, gate) in "
                      f"float64 numpy; {passes} pass(es), {dt:.1f} s"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # The GPU clock takes ~50 ms of sustained load to settle (the fused
    # projection runs 2.7 ms cold, 1.8 ms warm), so the default warm-up is
    # long enough to cover that at the prefill workload.
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--overlap", action="store_true",
                    help="several layers: project every layer after the first on a second "
                         "stream while the first layer's projection and gate run")
    ap.add_argument("--mxfp8", action="store_true",
                    help="FP8 tables: project the raw rows in MXFP8 against an MXFP8 copy "
                         "of wkv (engram_project_mxfp8)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES (for scaling "
                         "the FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the Engram forward here runs on a single "
              "MI355X with no sharding or collectives (--gpus 1).", file=sys.stderr)
        return 2

    import torch
    if args.calibrate_copy:
        src = torch.ones(args.calibrate_copy, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": args.calibrate_copy}), flush=True)
        return 0
    import workloads
    from workloads.device import to_device
    import __graft_entry__
    __graft_entry__._ensure_built()
    import gram_hash_memory_amd as eg
    log(f"bench: libengram {eg.BUILD_ID}")

    t0 = time.perf_counter()
    wl = workloads.make_workload(args.config)
    s = wl.spec
    log(f"bench: inputs for config {args.config} ({s.name}) built in {time.perf_counter()-t0:.1f} s")
    torch.cuda.set_device(0)
    dw = to_device(wl, "cuda")
    stream = torch.cuda.current_stream()
    L = len(s.layer_ids)
    fmt = eg.ENGRAM_ROWS_Q2K if s.fmt == "q2k" else eg.ENGRAM_ROWS_FP8_E4M3_E8M0
    params = eg.HashParams.from_dict(wl.hash_params)
    tokens = eg.Tokens(dw.cids, dw.cu_seqlens, dw.doc_ids, dw.token_mask, dw.lookback,
                       dw.lookback_live)
    mx = args.mxfp8
    if mx and fmt != eg.ENGRAM_ROWS_FP8_E4M3_E8M0:
        print("--mxfp8 needs a workload with FP8 tables (config 4)", file=sys.stderr)
        return 2
    wmx = []
    if mx:
        # Weight prep, once per weight, outside the timed region.
        for l in dw.layers:
            codes = torch.empty((s.N, s.K), dtype=torch.uint8, device="cuda")
            scl = torch.empty((s.N, s.K // 32), dtype=torch.uint8, device="cuda")
            eg.engram_quantize_mxfp8(l.wkv, s.N, s.K, codes, scl)
            wmx.append((codes, scl))
    layers = [eg.Layer(fmt, l.table, l.scales, l.wkv, l.q_weight, l.k_weight, s.hc, s.dim,
                       s.cols, *(wmx[i] if mx else ())) for i, l in enumerate(dw.layers)]
    h = dw.h
    ids = torch.empty((s.T, L, s.cols), dtype=torch.int32, device="cuda")
    rows = torch.empty((s.T, s.K), dtype=torch.int16, device="cuda")
    kv = torch.empty((s.T, s.N), dtype=torch.int16, device="cuda")
    # --overlap: one kv buffer per layer, layers after the first projected on
    # a second stream (the projection does not depend on h; only the gates
    # are ordered).
    overlap = args.overlap and len(s.layer_ids) > 1
    kvs = [kv] + [torch.empty_like(kv) for _ in range(len(s.layer_ids) - 1)]
    side = torch.cuda.Stream() if overlap else None
    num_rows = [l.table.numel() // (84 if fmt == eg.ENGRAM_ROWS_Q2K else 256) for l in dw.layers]
    # The fused Q2_K rows+projection, as engram_forward picks it: table and
    # columns within its limits, and either more than SKINNY_MAX_TOKENS tokens
    # (256 x 256 tiles) or K quarters of whole table columns (weight streaming).
    fused = (fmt == eg.ENGRAM_ROWS_Q2K and s.cols <= 32 and
             (s.T > SKINNY_MAX_TOKENS or s.cols % 4 == 0) and
             all(n * 84 <= Q2K_FUSED_MAX_BYTES for n in num_rows))
    # MXFP8 as engram_forward runs it: the weight-streaming form for up to 64
    # tokens (cols % 4 == 0, cols <= 64), else the rows staged into an MXFP8
    # activation and the 256 x 256 tiles on it.
    mx_staged = mx and not (s.T <= 64 and s.cols % 4 == 0 and s.cols <= 64) and \
        s.T * s.K <= MX_MAX_BYTES
    if mx_staged:
        a_codes = torch.empty((s.T, s.K), dtype=torch.uint8, device="cuda")
        a_scales = torch.empty((s.T, s.K // 32), dtype=torch.uint8, device="cuda")

    def layer_ids(l):
        return ids.view(-1)[l * s.cols:]

    def rows_call(l):
        dl = dw.layers[l]
        eg.engram_rows(fmt, dl.table, dl.scales, num_rows[l], layer_ids(l), L * s.cols, s.cols,
                       s.T, rows, None, stream)

    def project_call(l, st=None):
        eg.engram_project(rows, dw.layers[l].wkv, kvs[l], s.T, s.K, s.N, st or stream)

    def fused_call(l, st=None):
        dl = dw.layers[l]
        eg.engram_project_q2k(dl.table, num_rows[l], layer_ids(l), L * s.cols, s.cols, dl.wkv,
                              kvs[l], s.T, s.N, None, st or stream)

    def mx_call(l):
        dl = dw.layers[l]
        eg.engram_project_mxfp8(dl.table, dl.scales, num_rows[l], layer_ids(l), L * s.cols,
                                s.cols, wmx[l][0], wmx[l][1], kvs[l], s.T, s.N, None, stream)

    def stage_call(l):
        dl = dw.layers[l]
        eg.engram_stage_mxfp8(dl.table, dl.scales, num_rows[l], layer_ids(l), L * s.cols,
                              s.cols, s.T, a_codes, a_scales, None, stream)

    def mx_staged_call(l):
        eg.engram_project_mxfp8_staged(a_codes, a_scales, s.cols, wmx[l][0], wmx[l][1], kvs[l],
                                       s.T, s.N, stream)

    def gate_pass_call():
        eg.engram_gate_layers(h, kvs, [dl.q_weight for dl in dw.layers],
                              [dl.k_weight for dl in dw.layers], dw.token_mask, s.T, s.hc,
                              s.dim, s.eps, s.clamp, s.dot_scale, stream)

    def gate_call(l):
        dl = dw.layers[l]
        eg.engram_gate(h, kvs[l], dl.q_weight, dl.k_weight, dw.token_mask, s.T, s.hc, s.dim, s.eps,
                       s.clamp, s.dot_scale, stream)

    # One step = the launches engram_forward makes, in its order.
    plan = [("hash", lambda: eg.engram_hash(params, tokens, ids, stream))]
    if overlap:
        # hash -> (side stream: layers 1.. projected) || (layer 0 projected, gated);
        # each later gate waits for its layer's projection.
        ev_hash = torch.cuda.Event()
        ev_kv = [torch.cuda.Event() for _ in range(L)]
        proj = fused_call if fused else None
        if proj is None:
            raise SystemExit("--overlap is built for the fused Q2_K projection")

        def side_projections():
            ev_hash.record(stream)
            side.wait_event(ev_hash)
            for l in range(1, L):
                proj(l, side)
                ev_kv[l].record(side)

        def gate_after(l):
            stream.wait_event(ev_kv[l])
            gate_call(l)
        plan.append(("side_projections", side_projections))
        plan.append(("rows_project", lambda: proj(0)))
        plan.append(("gate", lambda: gate_call(0)))
        for l in range(1, L):
            plan.append(("gate", lambda l=l: gate_after(l)))
    for l in range(L if not overlap else 0):
        if mx_staged:
            plan += [("stage_mx", lambda l=l: stage_call(l)),
                     ("project_mx", lambda l=l: mx_staged_call(l))]
        elif mx:
            plan.append(("rows_project", lambda l=l: mx_call(l)))
        elif fused:
            plan.append(("rows_project", lambda l=l: fused_call(l)))
        else:
            plan += [("rows", lambda l=l: rows_call(l)), ("project", lambda l=l: project_call(l))]
    if not overlap:
        # engram_forward: every projection first, then one gate pass for all layers
        plan.append(("gate", gate_pass_call if L > 1 else (lambda: gate_call(0))))

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        for i, (_, fn) in enumerate(plan):
            fn()
            if ev is not None:
                ev[i + 1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"bench: {args.warmup} warmup steps done; timing {args.steps} steps")

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(plan) + 1)]
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for k in range(args.steps):
        step(events[k])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start

    total, count = {}, {}
    for ev in events:
        for i, (name, _) in enumerate(plan):
            total[name] = total.get(name, 0.0) + ev[i].elapsed_time(ev[i + 1])
            count[name] = count.get(name, 0) + 1
    per_launch_ms = {k: total[k] / count[k] for k in total}

    def time_alone(fn, n):
        """Average ms of n back-to-back launches of fn (outside the timed steps)."""
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    n_ref = max(3, args.steps // 2)
    if fused or mx:
        # The two-kernel path the fused kernel replaces, for comparison (the
        # row gather is also a C-ABI entry point of its own).
        per_launch_ms["rows"] = time_alone(lambda: rows_call(0), n_ref)
        per_launch_ms["project"] = time_alone(lambda: project_call(0), n_ref)
    ws = torch.empty(eg.engram_workspace_bytes(s.T, L, s.cols, s.hc, s.dim), dtype=torch.uint8,
                     device="cuda")
    forward_ms = time_alone(lambda: eg.engram_forward(params, tokens, layers, h, s.hc, s.dim,
                                                      s.eps, s.clamp, s.dot_scale, ws, None,
                                                      stream), n_ref)
    graph_ms = None
    if s.T <= SKINNY_MAX_TOKENS:
        # Decode: the same forward captured once in a HIP graph and replayed
        # (launch overhead is a visible share of a ~0.1 ms step).
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            eg.engram_forward(params, tokens, layers, h, s.hc, s.dim, s.eps, s.clamp,
                              s.dot_scale, ws, None)
        graph_ms = time_alone(graph.replay, n_ref)

    alg = algorithmic(s, wl.token_mask)

    def tflops(ms):
        return alg["project"] / (ms * 1e-3) / 1e12

    def gbs(nbytes, ms):
        return nbytes / (ms * 1e-3) / 1e9

    gate_pass = L > 1 and not overlap
    gate_bytes = alg["gate_pass"] if gate_pass else alg["gate"]
    gg_ms = L * per_launch_ms["rows"] + per_launch_ms["gate"] * (1 if gate_pass or L == 1 else L)
    gg_gbs = gbs(L * alg["rows"] + (gate_bytes if gate_pass or L == 1 else L * alg["gate"]), gg_ms)
    ms_per_step = elapsed * 1e3 / args.steps

    def prof(name):
        # Summaries exist for the prefill (T=8192) and decode (T=64) workloads.
        suffix = {2: "_prefill_T8192.md", 1: "_decode_T64.md", 3: "_two_layer_T4096.md",
                  4: "_fp8_T16384.md"}.get(args.config)
        return profiled_traffic(name + suffix) if suffix else None

    if mx_staged:
        dom_name = "project_mx"
        dom_kernel = "gemm_mx_persistent_kernel<true> (engram_project_mxfp8_staged)"
        dom_prof = "gemm_mx"
    elif mx:
        dom_name, dom_kernel = "rows_project", (
            "gemm_mx_persistent_kernel" if s.cols >= 2 else "gemm_mx_kernel") + \
            " (engram_project_mxfp8)"
        dom_prof = "gemm_mx"
    elif fused:
        dom_name, dom_kernel = "rows_project", (
            "gemm_q2k_persistent_kernel" if s.cols % 2 == 0 else "gemm_q2k_kernel") + \
            " + gemm_q2k_exact_kernel (engram_project_q2k)"
        dom_prof = "gemm_q2k"
    else:
        dom_name, dom_kernel = "project", (
            "gemm_nt_persistent_kernel" if s.K % 128 == 0 else "gemm_nt_kernel") + \
            " (engram_project)"
        dom_prof = "gemm_nt"
    dom_tf = tflops(per_launch_ms[dom_name])
    dom_peak = FP8_PEAK_TFLOPS if mx else BF16_PEAK_TFLOPS
    skinny = s.T <= SKINNY_MAX_TOKENS and not mx
    if skinny:
        # Few tokens: the projection streams wkv once and is bound by HBM.
        # Fused, it reads the tokens' Q2_K blocks and ids instead of bf16 rows.
        if fused:
            dom_kernel = "gemm_skinny_q2k_kernel (engram_project_q2k, T <= 128)"
            dom_bytes = 2.0 * s.N * s.K + s.T * s.cols * (84 + 4) + 2.0 * s.T * s.N
            dom_prof = "gemm_skinny_q2k"
        else:
            dom_kernel = "gemm_skinny_kernel (engram_project, T <= 128)"
            dom_bytes = 2.0 * (s.N * s.K + s.T * s.K + s.T * s.N)
            dom_prof = "gemm_skinny"
        dom_gbs = gbs(dom_bytes, per_launch_ms[dom_name])
        roofline = {"bound": "hbm", "achieved": round(dom_gbs, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(dom_gbs / HBM_PEAK_GBS, 4),
                    "traffic": prof(dom_prof),
                    "bytes_per_launch": dom_bytes}
    else:
        roofline = {"bound": "mfma", "achieved": round(dom_tf, 1), "peak": dom_peak,
                    "unit": "TFLOP/s", "frac": round(dom_tf / dom_peak, 4),
                    "traffic": prof(dom_prof)}
    roofline.update({"kernel": dom_kernel, "per_launch_ms": round(per_launch_ms[dom_name], 4)})
    stages = {
        "hash": {"ms": round(per_launch_ms["hash"], 4), "bound": "alu",
                 "hbm_gbs": round(gbs(alg["hash"], per_launch_ms["hash"]), 1),
                 "traffic": prof("hash")},
    }
    if mx_staged:
        stage_gbs = gbs(alg["stage_mx"], per_launch_ms["stage_mx"])
        stages["stage_mx"] = {
            "ms": round(per_launch_ms["stage_mx"], 4), "bound": "hbm",
            "achieved_gbs": round(stage_gbs, 1), "frac": round(stage_gbs / HBM_PEAK_GBS, 4),
            "bytes_per_launch": alg["stage_mx"], "traffic": prof("stage_mx")}
        stages["project_mx"] = {
            "ms": round(per_launch_ms["project_mx"], 4), "bound": "mfma",
            "achieved_tflops": round(dom_tf, 1), "frac": round(dom_tf / dom_peak, 4),
            "traffic": prof(dom_prof)}
    elif (fused or mx) and skinny:
        stages["rows_project"] = {
            "ms": round(per_launch_ms["rows_project"], 4), "bound": "hbm",
            "achieved_gbs": round(dom_gbs, 1), "frac": round(dom_gbs / HBM_PEAK_GBS, 4),
            "bytes_per_launch": dom_bytes, "traffic": prof(dom_prof)}
    elif fused or mx:
        stages["rows_project"] = {
            "ms": round(per_launch_ms["rows_project"], 4), "bound": "mfma",
            "achieved_tflops": round(dom_tf, 1), "frac": round(dom_tf / dom_peak, 4),
            "traffic": prof(dom_prof)}
    rows_gbs = gbs(alg["rows"], per_launch_ms["rows"])
    proj_tf = tflops(per_launch_ms["project"])
    stages["rows"] = {"ms": round(per_launch_ms["rows"], 4), "bound": "hbm",
                      "achieved_gbs": round(rows_gbs, 1),
                      "frac": round(rows_gbs / HBM_PEAK_GBS, 4),
                      "bytes_per_launch": alg["rows"],
                      "traffic": prof("rows_q2k" if s.fmt == "q2k" else "rows_fp8"),
                      "in_step": not (fused or mx)}
    stages["project"] = {"ms": round(per_launch_ms["project"], 4),
                         "bound": "hbm" if skinny else "mfma",
                         "achieved_tflops": round(proj_tf, 1),
                         "frac": round(proj_tf / BF16_PEAK_TFLOPS, 4),
                         "traffic": prof("gemm_skinny" if skinny else "gemm_nt"),
                         "in_step": not (fused or mx)}
    gate_gbs = gbs(gate_bytes, per_launch_ms["gate"])
    stages["gate"] = {"ms": round(per_launch_ms["gate"], 4), "bound": "hbm",
                      "achieved_gbs": round(gate_gbs, 1),
                      "frac": round(gate_gbs / HBM_PEAK_GBS, 4),
                      "bytes_per_launch": gate_bytes,
                      "layers_per_launch": L if gate_pass else 1,
                      "traffic": prof("gate")}
    gg = {"ms": round(gg_ms, 4), "achieved_gbs": round(gg_gbs, 1),
          "frac": round(gg_gbs / HBM_PEAK_GBS, 4),
          "kernels": "engram_rows + engram_gate" +
                     (" (one gate pass for all layers)" if gate_pass else "")}
    if mx_staged:
        # The step's gather is the MXFP8 staging kernel, HBM-bound like the gate.
        sg_ms = L * per_launch_ms["stage_mx"] + per_launch_ms["gate"] * (
            1 if gate_pass or L == 1 else L)
        sg_bytes = L * alg["stage_mx"] + (gate_bytes if gate_pass or L == 1 else L * alg["gate"])
        stages["gather_plus_gate"] = {
            "in_step": True, "ms": round(sg_ms, 4), "achieved_gbs": round(gbs(sg_bytes, sg_ms), 1),
            "frac": round(gbs(sg_bytes, sg_ms) / HBM_PEAK_GBS, 4),
            "kernels": "engram_stage_mxfp8 + engram_gate"}
        stages["gather_plus_gate_standalone"] = dict(gg, in_step=False)
    elif fused or mx:
        # The step gathers inside the fused projection (MFMA-bound, timed
        # above as rows_project); its only HBM-bound kernel is the gate.
        stages["gather_plus_gate"] = {
            "in_step": "gate", "ms": stages["gate"]["ms"],
            "achieved_gbs": stages["gate"]["achieved_gbs"], "frac": stages["gate"]["frac"],
            "note": "the row gather runs inside the fused projection; the step's "
                    "HBM-bound stage is the gate alone"}
        stages["gather_plus_gate_standalone"] = dict(gg, in_step=False)
    else:
        stages["gather_plus_gate"] = dict(gg, in_step=True)
    stages["engram_forward_ms"] = round(forward_ms, 4)
    if graph_ms is not None:
        stages["engram_forward_graph_replay_ms"] = round(graph_ms, 4)

    result = {
        "metric": METRIC,
        "value": s.T * args.steps / elapsed,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp8" if mx else "bf16",
        "data": "synthetic",
        "config": {"workload": f"{s.name}: T={s.T} ({len(s.seq_lens)}x{s.seq_lens[0]}), "
                               f"{L} layer(s), {s.cols} cols, {s.fmt} table "
                               f"{s.num_rows} rows, dim={s.dim}, hc={s.hc}, "
                               f"{s.id_dist} ids",
                   "T": s.T, "K": s.K, "N": s.N, "row_format": s.fmt,
                   "projection": "mxfp8" if mx else "bf16",
                   "schedule": "two streams: later layers projected beside layer 0"
                               if overlap else "one stream, engram_forward order"},
        "roofline": roofline,
        "stages": stages,
    }
    if not args.no_cpu_baseline:
        log("bench: timing the CPU oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline(wl, mx)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
