"""Benchmark of the Gated DeltaNet token-mixer hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one pass of the hot path over one batch of seeded synthetic input
already resident in HBM: cu_seqlens localisation, causal conv1d + SiLU with
halo, chunked gated delta rule forward (and, for a workload with backward,
the chunk and conv backward).  Default workload: the 131072-token single
sequence with 16 q/k heads and 32 value heads, dk = dv = 128, bfloat16.

Prints one JSON line with throughput (tokens/s), per-call times from HIP
events on the launch stream, the roofline position of the dominant call and
the fp64 CPU oracle timed on a bounded sample of the same workload.
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

METRIC = "tokens/s conv1d+chunk_gated_delta fwd(+bwd), 1 GPU; % bf16 MFMA / HBM peak"
HBM_PEAK = 8.0e12           # B/s, MI355X published
MFMA_PEAK = {"bf16": 2.5e15, "f32": 157.3e12}  # dense FLOP/s, MI355X published
BT = 64


def chunk_fwd_flops_per_token_head(dk, dv, C=BT):
    """Algorithmic FLOP of the chunked forward per token and value head: the
    products of the page's chunk algorithm, triangular ones counted at half.
      kh kh^T, qh kh^T (lower halves)   2 * C*dk
      T (I+L)^-1 (triangular solve)     2*C*C/3
      u = T vb, w = T kb (lower halves) C*dv + C*dk
      w S, qh S                          4*dk*dv
      P v_new (lower half)               C*dv
      kh^T v_new (state update)          2*dk*dv
    = C*(3dk + 2dv) + 2C^2/3 + 6*dk*dv."""
    return C * (3 * dk + 2 * dv) + 2 * C * C / 3 + 6 * dk * dv


def conv_bytes_per_token(C, s):
    return 2 * C * s  # read x, write y


def conv_bwd_bytes_per_token(C, s):
    return 3 * C * s  # read x and dy, write dx


def chunk_fwd_bytes(T, N, Hk, Hv, dk, dv, s):
    """Algorithmic HBM bytes of one chunk forward: read q, k, v, g, beta;
    write o; read h0 and write ht once per sequence."""
    per_tok = 2 * Hk * dk * s + 2 * Hv * dv * s + 8 * Hv
    return T * per_tok + 2 * N * Hv * dk * dv * 4


def chunk_bwd_bytes(T, N, Hk, Hv, dk, dv, s):
    """Algorithmic HBM bytes of one chunk backward: read q, k, v, g, beta and
    dO, write dq, dk, dv, dg and dbeta; read h0 and dht and write dh0 once
    per sequence."""
    per_tok = 4 * Hk * dk * s + 3 * Hv * dv * s + 16 * Hv
    return T * per_tok + 3 * N * Hv * dk * dv * 4


def roof(flops, nbytes, t, act):
    """The call's position under both roofs, and the binding one: at the
    call's algorithmic intensity (FLOP per algorithmic HBM byte) the bound
    is HBM below the ridge (MFMA peak / HBM peak) and MFMA above it; frac is
    the binding roof's time over the measured time."""
    mfma = {"bound": "mfma", "achieved": flops / t / 1e12, "peak": MFMA_PEAK[act] / 1e12,
            "unit": "TFLOP/s", "frac": flops / t / MFMA_PEAK[act]}
    hbm = {"bound": "hbm", "achieved": nbytes / t / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
           "frac": nbytes / t / HBM_PEAK}
    ridge = MFMA_PEAK[act] / HBM_PEAK
    intensity = flops / nbytes
    binding = dict(hbm if intensity < ridge else mfma)
    binding.update({"intensity_flop_per_byte": intensity, "ridge_flop_per_byte": ridge})
    return binding, mfma, hbm


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="long131k_hk16_hv32_d128_bf16")
    ap.add_argument("--cpu-sample-tokens", type=int, default=0,
                    help="tokens of the oracle sample (0: chosen for ~10-30 s)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calls", default="",
                    help="profiling only: comma-separated calls (localize, conv_fwd, chunk_fwd, "
                         "chunk_bwd, conv_bwd) run in the loop, the others once before it; the "
                         "line then reports those calls' times, not the workload's throughput")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path; run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)
    import torch

    from linear_attention_sequence_causal_amd import gdn, workloads

    gdn.load_library()
    spec = workloads.config(args.workload)
    inp = workloads.make(spec)
    dev = "cuda"
    torch.cuda.set_device(0)
    dtype = workloads.ACT_DTYPES[spec.act]
    T, Hk, Hv, dk, dv, K = inp["T"], spec.Hk, spec.Hv, spec.dk, spec.dv, spec.K
    C = spec.C
    x, w = inp["x"].to(dev), inp["w"].to(dev)
    halo = None if inp["halo"] is None else inp["halo"].to(dev)
    g, beta = inp["g"].to(dev), inp["beta"].to(dev)
    h0 = None if inp["h0"] is None else inp["h0"].to(dev)
    cu_glob = torch.tensor(inp["cu_global"], dtype=torch.int32, device=dev)
    total = int(inp["cu_global"][-1])
    do = None if inp["do"] is None else inp["do"].to(dev)
    dht = None if inp["dht"] is None else inp["dht"].to(dev)
    N = inp["cap"]
    stream = torch.cuda.current_stream()

    # preallocated outputs and workspaces: the timed region allocates nothing
    y = torch.empty_like(x)
    o = torch.empty((T, Hv, dv), dtype=dtype, device=dev)
    ht = torch.empty((N, Hv, dk, dv), dtype=torch.float32, device=dev)
    ws_f = torch.empty(max(gdn.chunk_workspace_size(T, N, Hk, Hv, dk, dv, dtype), 1),
                       dtype=torch.uint8, device=dev)
    if spec.world_size == 1 and spec.n_halo:
        meta_fixed = gdn.make_meta(dev, n_halo=spec.n_halo)
    else:
        meta_fixed = None

    local_buf = torch.empty(N + 1, dtype=torch.int32, device=dev)
    meta_buf = torch.empty(gdn.META_BYTES, dtype=torch.uint8, device=dev)
    bwd_out = conv_out = ws_b = ws_cb = saved = None
    if spec.backward:
        bwd_out = (torch.empty_like(x), torch.empty((T, Hv), dtype=torch.float32, device=dev),
                   torch.empty((T, Hv), dtype=torch.float32, device=dev),
                   torch.empty((N, Hv, dk, dv), dtype=torch.float32, device=dev))
        conv_out = (torch.empty_like(x), torch.empty((C, K), dtype=torch.float32, device=dev), None,
                    None if halo is None else torch.empty_like(halo))
        ws_b = torch.empty(max(gdn.chunk_workspace_size(T, N, Hk, Hv, dk, dv, dtype, bwd=True), 1),
                           dtype=torch.uint8, device=dev)
        ws_cb = torch.empty(max(gdn.conv_bwd_workspace_size(T, C, K), 1), dtype=torch.uint8,
                            device=dev)
        # the training pair: the forward keeps the per-chunk states and records
        # for the backward
        saved = torch.empty(max(gdn.chunk_saved_size(T, N, Hk, Hv, dk, dv, dtype), 1),
                            dtype=torch.uint8, device=dev)

    def step(ev=None, only=None):
        # only: the calls run (profiling); the others keep their last outputs
        def mark(i):
            if ev is not None:
                ev[i].record(stream)

        def run(name):
            return only is None or name in only
        mark(0)
        if run("localize"):
            gdn.gdn_localize_cu_seqlens(cu_glob, total, spec.world_size, spec.rank, K,
                                        out=(local_buf, meta_buf))
        local = local_buf
        m = meta_buf if spec.world_size > 1 else meta_fixed
        mark(1)
        if run("conv_fwd"):
            gdn.gdn_conv1d_silu_halo(x, w, local, halo=halo, meta=m, out=y)
        mark(2)
        if run("chunk_fwd"):
            if spec.backward:
                gdn.gdn_chunk_fwd_save(y, g, beta, local, Hk, Hv, dk, dv, h0=h0, out=o, ht_out=ht,
                                       ws=ws_f, saved=saved)
            else:
                gdn.gdn_chunk_fwd(y, g, beta, local, Hk, Hv, dk, dv, h0=h0, out=o, ht_out=ht,
                                  ws=ws_f)
        mark(3)
        if spec.backward:
            if run("chunk_bwd"):
                gdn.gdn_chunk_bwd_saved(y, g, beta, local, Hk, Hv, dk, dv, do, saved, h0=h0,
                                        dht=dht, ws=ws_b, out=bwd_out)
            mark(4)
            if run("conv_bwd"):
                gdn.gdn_conv1d_silu_halo_bwd(x, w, local, bwd_out[0], halo=halo, meta=m,
                                             out=conv_out, ws=ws_cb)
            mark(5)

    names = ["localize", "conv_fwd", "chunk_fwd"] + (["chunk_bwd", "conv_bwd"] if spec.backward else [])
    if args.calls:
        return profile_calls(args, names, step, stream, spec.backward)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(evs[s])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # per call: the median over the timed steps of its HIP-event interval
    per_call = {n: float(np.median([e[i].elapsed_time(e[i + 1]) for e in evs]))
                for i, n in enumerate(names)}
    ms_per_step = elapsed * 1e3 / args.steps
    value = T * args.steps / elapsed

    s_bytes = 2 if dtype == torch.bfloat16 else 4
    flops = chunk_fwd_flops_per_token_head(dk, dv) * T * Hv
    t_chunk = per_call["chunk_fwd"] * 1e-3
    conv_b = conv_bytes_per_token(C, s_bytes) * T + C * K * s_bytes
    t_conv = per_call["conv_fwd"] * 1e-3
    chunk_hbm = chunk_fwd_bytes(T, N, Hk, Hv, dk, dv, s_bytes)
    roofline, fwd_mfma, fwd_hbm = roof(flops, chunk_hbm, t_chunk, spec.act)
    roofline.update({"traffic": measured_traffic("chunk_fwd", spec.name),
                     "kernel": "gdn_chunk_fwd call: plan, prep, replay table, summaries + scan "
                               "for the (sequence, head) pairs that cannot replay, output pass"})
    extra = {
        "chunk_fwd_mfma": fwd_mfma,
        "chunk_fwd_hbm": fwd_hbm,
        "conv_fwd": {"bound": "hbm", "achieved": conv_b / t_conv / 1e9, "peak": HBM_PEAK / 1e9,
                     "unit": "GB/s", "frac": conv_b / t_conv / HBM_PEAK},
    }
    if spec.backward:
        # the backward dominates such a step: its call is the roofline line,
        # the forward's moves to the other entries
        t_bwd = per_call["chunk_bwd"] * 1e-3
        bwd_flops = 2 * flops  # reverse mode of the chunk algorithm: twice the forward's products
        extra["chunk_fwd"] = dict(roofline, kernel="gdn_chunk_fwd_save call (keeps the "
                                  "per-chunk states for the backward)")
        bwd_hbm = chunk_bwd_bytes(T, N, Hk, Hv, dk, dv, s_bytes)
        roofline, bwd_mfma, bwd_hbm_roof = roof(bwd_flops, bwd_hbm, t_bwd, spec.act)
        roofline.update({"traffic": measured_traffic("chunk_bwd", spec.name),
                         "kernel": "gdn_chunk_bwd_saved call: plan, replay table, dS summaries + "
                                   "scan where needed, dS final pass, gradients (per-chunk states "
                                   "saved by the forward)"})
        extra["chunk_bwd_mfma"] = bwd_mfma
        extra["chunk_bwd_hbm"] = bwd_hbm_roof
        t_cbwd = per_call["conv_bwd"] * 1e-3
        cbwd_b = conv_bwd_bytes_per_token(C, s_bytes) * T + C * K * (s_bytes + 4)
        extra["conv_bwd"] = {"bound": "hbm", "achieved": cbwd_b / t_cbwd / 1e9, "peak": HBM_PEAK / 1e9,
                             "unit": "GB/s", "frac": cbwd_b / t_cbwd / HBM_PEAK}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(spec, inp, args.cpu_sample_tokens)

    line = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": spec.act, "data": "synthetic",
        "config": {"workload": spec.name, "tokens": T, "sequences": len(inp["lengths"]),
                   "qk_heads": Hk, "v_heads": Hv, "dk": dk, "dv": dv, "conv_k": K,
                   "passes": "fwd+bwd" if spec.backward else "fwd",
                   "world_size": spec.world_size, "rank": spec.rank},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "per_call_ms": per_call,
        "rooflines_other": extra,
    }
    print(json.dumps(line), flush=True)


def profile_calls(args, names, step, stream, fwd_feeds_bwd):
    """Runs the calls that make the named calls' inputs once, then only the
    named calls, so that a profiler sees those calls' kernels alone (the
    chunk forward is set-up only where its saved states feed the backward)."""
    import torch
    keep = [c.strip() for c in args.calls.split(",") if c.strip()]
    bad = [c for c in keep if c not in names]
    if bad:
        sys.exit("--calls: %s not among %s" % (bad, names))
    first = min(names.index(c) for c in keep)
    setup = {c for c in names[:first] if c != "chunk_fwd" or fwd_feeds_bwd}
    if "conv_bwd" in keep and "chunk_bwd" not in keep:
        setup.add("chunk_bwd")  # dy of the conv backward
    step(only=setup)
    torch.cuda.synchronize()
    times = {c: [] for c in keep}
    for i in range(args.warmup + args.steps):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
        step(ev, only=set(keep))
        torch.cuda.synchronize()
        if i >= args.warmup:
            for j, n in enumerate(names):
                if n in keep:
                    times[n].append(ev[j].elapsed_time(ev[j + 1]))
    print(json.dumps({"profile_only": True, "calls": keep, "steps": args.steps,
                      "warmup": args.warmup,
                      "per_call_ms": {n: float(np.median(t)) for n, t in times.items()}}),
          flush=True)


def measured_traffic(call, workload):
    """HBM bytes per call from the FETCH_SIZE / WRITE_SIZE counters stored
    under profiles/, if they were taken on the kernels built from the current
    sources; else None."""
    path = os.path.join(ROOT, "profiles", "%s_%s_traffic.json" % (call, workload))
    if not os.path.exists(path):
        return None
    from linear_attention_sequence_causal_amd import profiling
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("source_sha256") != profiling.source_digest():
        return None
    return rec["bytes_per_call"]


def cpu_baseline(spec, inp, sample_tokens):
    """The fp64 oracle (conv + token recurrence forward) on the first
    `sample_tokens` tokens of the workload, all heads: tokens/s of the whole
    sample, with each leg (conv, recurrence) timed and its thread count
    reported on its own."""
    from oracle import capi
    T = inp["T"]
    thr = capi.max_threads()
    if sample_tokens <= 0:
        # ~7*dk*dv fp64 FLOP per token and head; aim for ~15 s at ~2.5 GFLOP/s/thread
        per_tok = 7.0 * spec.dk * spec.dv * spec.Hv
        sample_tokens = int(min(T, max(256, 15 * 2.5e9 * min(thr, spec.Hv) / per_tok)))
    n = min(sample_tokens, T)
    x = inp["x"][:n].double().numpy()
    w = inp["w"].double().numpy()
    # the workload's own sequence boundaries within the sample (a shard's
    # tokens start at rank * T of the global batch)
    start = spec.rank * T if spec.world_size > 1 else 0
    cuts = np.clip(np.asarray(inp["cu_global"]) - start, 0, n)
    cu = [0] + sorted({int(c) for c in cuts if 0 < c < n}) + [n]
    # the recurrence runs its (sequence, head) chains in parallel
    rec_threads = min(thr, (len(cu) - 1) * spec.Hv)
    Hk, Hv, dk, dv = spec.Hk, spec.Hv, spec.dk, spec.dv
    t0 = time.perf_counter()
    yv = capi.conv1d_silu(x, w, None, None, 0, cu)
    t1 = time.perf_counter()
    q = yv[:, :Hk * dk].reshape(n, Hk, dk)
    k = yv[:, Hk * dk:2 * Hk * dk].reshape(n, Hk, dk)
    v = yv[:, 2 * Hk * dk:].reshape(n, Hv, dv)
    capi.gdn_fwd(q, k, v, inp["g"][:n].double().numpy(), inp["beta"][:n].double().numpy(), None,
                 cu, dk ** -0.5, nthreads=rec_threads)
    t2 = time.perf_counter()
    dt = t2 - t0
    return {"value": n / dt, "unit": "tokens/s", "cores": max(thr, rec_threads), "kind": "oracle",
            "sample": "first %d tokens of the workload, all %d value heads, conv + gated delta "
                      "rule forward in fp64 (%.1f s)" % (n, Hv, dt),
            "legs": {"conv": {"seconds": t1 - t0, "threads": thr,
                              "tokens_per_s": n / (t1 - t0)},
                     "recurrence": {"seconds": t2 - t1, "threads": rec_threads,
                                    "tokens_per_s": n / (t2 - t1)}},
            "host_cpus": len(os.sched_getaffinity(0))}


if __name__ == "__main__":
    main()
