#!/usr/bin/env python3
"""Benchmark of the QSA hot path on one MI355X.

A step is one QSA layer step for one batch: append the new tokens' K/V and
indexer keys, pool completed blocks, score, select, and attend
(``qsa_forward``).  The default workload is the ragged batched decode at up
to 128K context (32 sequences, contexts ~U[8192, 131072], paged KV), the
configuration the decode tok/s + HBM GB/s metric is quoted on.

Cache memory (256 MB on MI355X) would hold one step's selected KV, so the
steps rotate over several layer copies of the caches (distinct buffers, as
the QSA layers of a model are) and every step's bytes come from HBM.

Printed: ONE JSON line with the throughput, a roofline object for the
dominant kernel (the attention kernel: its algorithmic bytes per launch over
its average launch time, measured with HIP events on the launch stream) and
the CPU oracle's throughput on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "QSA decode tok/s + HBM GB/s at 128K ctx; prefill TFLOP/s (selected blocks)"
HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="ragged_paged_decode_128k_bf16")
    ap.add_argument("--layers", type=int, default=0, help="cache copies to rotate over (0 = auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MB",
                    help="only run a plain device copy of MB megabytes (counter calibration)")
    ap.add_argument("--no-graph", action="store_true",
                    help="decode: skip timing the steps replayed from a HIP graph")
    return ap.parse_args()


def calibrate_copy(mb: int) -> None:
    """A plain device-to-device copy of a known size, 5 times: what the HBM
    counters read for it scales their readings of the QSA kernels."""
    import torch
    n = mb * 1000 * 1000
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": n, "copies": 5}), flush=True)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; the QSA hot path "
                                   "has no multi-GPU leg (it would shard by sequence, KV head "
                                   "or context; none of these is built)",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    from block_sparse_attention_keys_amd import qsa, runner, workloads

    qsa.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    name = args.workload
    if name in BLOCK_BENCH:
        return bench_block(args, name)
    if name == "block_chunked_prefill_32k":
        return bench_block_prefill(args, name)
    sp = workloads.SPECS[name]
    if sp.kind != "decode":
        return bench_prefill(args, name)

    t0 = time.time()
    case = workloads.make_case(name, seed=0)
    log(f"[bench] workload {name}: drawn in {time.time() - t0:.1f}s, ctx "
        f"min/max {min(case.ctx)}/{max(case.ctx)}")

    B, r, k = sp.n_seqs, sp.block_size, sp.k_blocks
    m = sp.q_per_step          # new tokens (queries) per sequence per step
    T = B * m
    Hq, Hkv, D, HI, dI = sp.n_q_heads, sp.n_kv_heads, sp.head_dim, sp.n_idx_heads, sp.idx_dim
    esz = 2  # bf16
    kv_esz = 1 if sp.kv_fp8 else esz  # bytes per cached K/V element

    # Algorithmic bytes of one step (host formula from positions only): every
    # query reads its own selected (or, dense, all) K/V rows.
    def step_bytes(ctx_now):
        kv = idx = 0
        for c in ctx_now:
            for i in range(m):
                n = c + i + 1
                if r > 0:
                    nb = n // r
                    nsel = r * min(k, nb) + (n - r * nb)
                    idx += nb * dI * 4              # pooled keys read by the scorer
                else:
                    nsel = n
                kv += nsel * Hkv * D * kv_esz * 2
        qgo = T * Hq * D * esz * 3 + (T * (HI * dI * esz + HI * 4) if r > 0 else 0)
        new_rows = T * (2 * Hkv * D + (dI if r > 0 else 0)) * esz
        return kv, idx, qgo + new_rows

    kv0, idx0, small0 = step_bytes(case.ctx)
    per_step = kv0 + idx0 + small0
    L = args.layers or max(2, math.ceil(3 * 256e6 / per_step))
    total = args.warmup + args.steps
    per_layer_steps = math.ceil(total / L) + 1
    t0 = time.time()
    dc = runner.DeviceCase(case, device=dev, n_layers=L, extra_steps=per_layer_steps * m)
    log(f"[bench] {L} layer copies on the GPU in {time.time() - t0:.1f}s "
        f"({per_step / 1e6:.1f} MB algorithmic per step)")

    # Per-step inputs, drawn on the GPU with the workload's distributions, resident in HBM.
    gen = torch.Generator(device=dev)
    gen.manual_seed(1)
    bf = torch.bfloat16

    def nrm(shape, scale):
        return (torch.randn(shape, generator=gen, device=dev) * scale).to(bf)

    steps_in = []
    for s in range(total):
        x = {"q": nrm((T, Hq, D), D ** -0.5), "k_new": nrm((T, Hkv, D), D ** -0.5),
             "v_new": nrm((T, Hkv, D), D ** -0.5), "gate": nrm((T, Hq, D), 1.0),
             "qI": None, "kI_new": None, "w": None}
        if r > 0:
            x.update({"qI": nrm((T, HI, dI), dI ** -0.5), "kI_new": nrm((T, dI), dI ** -0.5),
                      "w": torch.rand((T, HI), generator=gen, device=dev)})
        steps_in.append(x)
    batches = [dc.batch_for([c + j * m for c in case.ctx], [m] * B)
               for j in range(per_layer_steps)]
    ws_bytes = max(qsa.qsa_workspace_size(dc.params, bt) for bt in batches)
    ws = torch.zeros((ws_bytes,), dtype=torch.uint8, device=dev)
    outs = [torch.empty((T, Hq, D), dtype=bf, device=dev) for _ in range(total)]
    sels = [torch.empty((T, max(k, 1)), dtype=torch.int32, device=dev) for _ in range(total)]
    nbls = [torch.empty((T,), dtype=torch.int32, device=dev) for _ in range(total)]
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream

    def fwd(s, stream_handle=sh):
        l, j = s % L, s // L
        st, x = dc.layers[l], steps_in[s]
        qsa.qsa_forward(dc.params, batches[j], x["q"], x["k_new"], x["v_new"], x["qI"],
                        x["kI_new"], x["w"], x["gate"], st["k"], st["v"], st.get("kI"),
                        st.get("pooled"), outs[s], sels[s], nbls[s], ws, stream_handle)

    for s in range(args.warmup):
        fwd(s)
    torch.cuda.synchronize(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for s in range(args.warmup, total):
        fwd(s)
    e1.record(stream)
    torch.cuda.synchronize(dev)
    ms_step = e0.elapsed_time(e1) / args.steps
    tok_s = T / (ms_step * 1e-3)
    hbm_gbps = per_step / (ms_step * 1e-3) / 1e9

    # The same timed steps captured into one HIP graph and replayed (replays
    # rewrite the same cache rows with the same values): launch gaps and
    # host launch cost removed.
    graph = None
    if not args.no_graph:
        graph = graph_timing(torch, lambda: [fwd(s, None) for s in range(args.warmup, total)],
                             args.steps, stream)
        if graph is not None:
            graph["value"] = round(T / (graph["ms_per_step"] * 1e-3), 1)
            graph["hbm_GBps_step"] = round(per_step / (graph["ms_per_step"] * 1e-3) / 1e9, 1)

    # Dominant kernel: the attention of each timed step, launched alone on the
    # same stream in the same layer rotation, bracketed by events.
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    for i, s in enumerate(range(args.warmup, total)):
        l, j = s % L, s // L
        st, x = dc.layers[l], steps_in[s]
        ev[i][0].record(stream)
        qsa.qsa_attend(dc.params, batches[j], x["q"], st["k"], st["v"], sels[s], nbls[s],
                       x["gate"], outs[s], ws, sh)
        ev[i][1].record(stream)
    torch.cuda.synchronize(dev)
    attn_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    attn_bytes = kv0 + T * Hq * D * esz * 3
    attn_gbps = attn_bytes / (attn_ms * 1e-3) / 1e9

    res = {
        "metric": METRIC, "value": round(tok_s, 1), "unit": "tok/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": ("synthetic (seeded; " + (f"contexts U[{sp.ctx_lo},{sp.ctx_hi}]" if sp.ctx_hi
                                          else f"context {sp.ctx}") +
                 "; N(0,1)/sqrt(d) q/k/v; decode inputs drawn on the GPU" +
                 ("; K/V cached as E4M3 codes" + (" in the Hadamard basis" if sp.kv_rotate
                                                  else "") if sp.kv_fp8 else "") + ")"),
        "config": {"workload": name, "batch": B, "q_per_step": m, "ctx_min": min(case.ctx),
                   "ctx_max": max(case.ctx), "n_q_heads": Hq, "n_kv_heads": Hkv,
                   "head_dim": D, "block_size": r, "budget": sp.budget,
                   "idx_heads": HI, "idx_dim": dI, "paged": bool(sp.page_size),
                   "kv_cache": ("e4m3" + ("+hadamard" if sp.kv_rotate else "")) if sp.kv_fp8
                   else "bf16", "layer_copies": L},
        "hbm_GBps_step": round(hbm_gbps, 1),
        "hbm_frac_step": round(hbm_gbps / HBM_PEAK_GBPS, 4),
        "graph_replay": graph,
        "step_bytes": {"selected_kv": kv0, "pooled_keys": idx0, "q_gate_out_new_rows": small0},
        "roofline": {"bound": "hbm",
                     "kernel": ("decode attention + split combine as qsa_attend launches them "
                                "(selection given; in qsa_forward the same kernel also selects)"),
                     "achieved": round(attn_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(attn_gbps / HBM_PEAK_GBPS, 4),
                     "avg_launch_us": round(attn_ms * 1e3, 2), "bytes_per_launch": attn_bytes,
                     "traffic": counter_traffic(f"attn_{name}_hbm_counters.txt")},
    }

    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(case, sp, args.cpu_seconds)
    print(json.dumps(res), flush=True)


# The QSA block (projections, norms, RoPE, QSA, o_proj) over a decode workload.
BLOCK_BENCH = {
    "block_ragged_paged_decode_128k": dict(spec="ragged_paged_decode_128k_bf16", d_model=2560,
                                           rotary_dim=64, rope_theta=1e7, idx_rope_dim=64),
}


def bench_block(args, name):
    """One decode step of the QSA block per sequence (qsa_block_forward): a
    step is the whole block for B new tokens.  Hidden states, weights (one
    copy per layer copy of the caches) and the per-step inputs are drawn on
    the GPU; the caches hold the workload's synthetic context, pooled with
    rotated indexer keys.  The roofline object prices the whole step's
    algorithmic bytes (weights, selected K/V, pooled keys) against HBM."""
    import torch
    from block_sparse_attention_keys_amd import qsa, runner, workloads
    cfg = BLOCK_BENCH[name]
    sp = workloads.SPECS[cfg["spec"]]
    dev = torch.device("cuda:0")
    case = workloads.make_case(cfg["spec"], seed=0)
    B, r, k = sp.n_seqs, sp.block_size, sp.k_blocks
    Hq, Hkv, D, HI, dI = sp.n_q_heads, sp.n_kv_heads, sp.head_dim, sp.n_idx_heads, sp.idx_dim
    dm, T = cfg["d_model"], sp.n_seqs
    n_in = workloads.block_n_in(sp)
    w_bytes = (n_in * dm + dm * Hq * D) * 2
    kv = idx = 0
    for c in case.ctx:
        n = c + 1
        nb = n // r
        kv += (r * min(k, nb) + (n - r * nb)) * Hkv * D * 2 * 2
        idx += nb * dI * 4
    per_step = w_bytes + kv + idx + T * dm * 2 * 2
    L = args.layers or max(2, math.ceil(3 * 256e6 / per_step))
    total = args.warmup + args.steps
    per_layer_steps = math.ceil(total / L) + 1
    dc = runner.DeviceCase(case, device=dev, n_layers=L, extra_steps=per_layer_steps,
                           idx_rope=(cfg["idx_rope_dim"], cfg["rope_theta"]))
    bp = qsa.make_block_params(dm, cfg["rotary_dim"], cfg["rope_theta"], 1e-6)
    gen = torch.Generator(device=dev)
    gen.manual_seed(2)
    bf = torch.bfloat16

    def nrm(shape, scale):
        return (torch.randn(shape, generator=gen, device=dev) * scale).to(bf)

    weights = [{"w_in": nrm((n_in, dm), dm ** -0.5), "w_o": nrm((dm, Hq * D), (Hq * D) ** -0.5),
                "qn": nrm((D,), 0.1), "kn": nrm((D,), 0.1)} for _ in range(L)]
    xs = [nrm((T, dm), 1.0) for _ in range(total)]
    batches = [dc.batch_for([c + j for c in case.ctx], [1] * B) for j in range(per_layer_steps)]
    ws_bytes = max(qsa.qsa_block_workspace_size(dc.params, bp, bt) for bt in batches)
    ws = torch.zeros((ws_bytes,), dtype=torch.uint8, device=dev)
    ys = [torch.empty((T, dm), dtype=bf, device=dev) for _ in range(total)]
    sels = [torch.empty((T, k), dtype=torch.int32, device=dev) for _ in range(total)]
    nbls = [torch.empty((T,), dtype=torch.int32, device=dev) for _ in range(total)]
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream

    def fwd(s):
        l, j = s % L, s // L
        st, w = dc.layers[l], weights[l]
        qsa.qsa_block_forward(dc.params, bp, batches[j], xs[s], w["w_in"], w["qn"], w["kn"],
                              w["w_o"], st["k"], st["v"], st["kI"], st["pooled"], ys[s], sels[s],
                              nbls[s], ws, sh)

    for s in range(args.warmup):
        fwd(s)
    torch.cuda.synchronize(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for s in range(args.warmup, total):
        fwd(s)
    e1.record(stream)
    torch.cuda.synchronize(dev)
    ms_step = e0.elapsed_time(e1) / args.steps
    gbps = per_step / (ms_step * 1e-3) / 1e9
    res = {
        "metric": METRIC, "value": round(T / (ms_step * 1e-3), 1), "unit": "tok/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": (f"synthetic (seeded; contexts U[{sp.ctx_lo},{sp.ctx_hi}]; hidden states "
                 "N(0,1), Linear weights N(0,1/fan_in), all drawn on the GPU)"),
        "config": {"workload": name, "batch": B, "d_model": dm, "n_q_heads": Hq,
                   "n_kv_heads": Hkv, "head_dim": D, "block_size": r, "budget": sp.budget,
                   "idx_heads": HI, "idx_dim": dI, "rotary_dim": cfg["rotary_dim"],
                   "idx_rope_dim": cfg["idx_rope_dim"], "ctx_min": min(case.ctx),
                   "ctx_max": max(case.ctx), "paged": True, "layer_copies": L},
        "step_bytes": {"weights": w_bytes, "selected_kv": kv, "pooled_keys": idx,
                       "x_y": T * dm * 4},
        "roofline": {"bound": "hbm", "kernel": "whole block step (qsa_block_forward)",
                     "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4), "avg_launch_us": round(ms_step * 1e3, 2),
                     "bytes_per_launch": per_step, "traffic": None},
    }
    print(json.dumps(res), flush=True)


def bench_block_prefill(args, name):
    """The QSA block over the 32K chunked prefill (d_model 2560): a step is
    every 4096-token chunk through qsa_block_forward, caches filled by the
    block itself.  The roofline prices the step's projection flops plus the
    selected-block attention flops against the bf16 MFMA peak."""
    import torch
    from block_sparse_attention_keys_amd import runner, workloads
    bc = workloads.make_block_case("chunked_prefill_32k_bf16", d_model=2560, chunk=4096,
                                   decode_steps=0)
    sp = bc.spec
    dc = runner.BlockDeviceCase(bc)
    calls = [dc.call_inputs(i) for i in range(len(bc.calls))]
    T = sum(c["T"] for c in calls)
    n_in = workloads.block_n_in(sp)
    proj = 2.0 * T * bc.d_model * (n_in + sp.n_q_heads * sp.head_dim)
    r, k = sp.block_size, sp.k_blocks
    n = np.arange(1, sp.prefill_len + 1)
    nb = n // r
    attn = float((r * np.minimum(k, nb) + (n - r * nb)).sum()) * sp.n_q_heads * 4 * sp.head_dim
    stream = torch.cuda.current_stream()

    def step():
        for c in calls:
            dc.forward(c)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    tflops = (proj + attn) / (ms * 1e-3) / 1e12
    print(json.dumps({
        "metric": METRIC, "value": round(T / (ms * 1e-3), 1), "unit": "tok/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; hidden states N(0,1), Linear weights N(0,1/fan_in))",
        "config": {"workload": name, "tokens": T, "chunk": 4096, "d_model": bc.d_model,
                   "n_q_heads": sp.n_q_heads, "n_kv_heads": sp.n_kv_heads,
                   "head_dim": sp.head_dim, "block_size": r, "budget": sp.budget},
        "gflop_per_step": {"projections": round(proj / 1e9, 1), "selected_attention": round(attn / 1e9, 1)},
        "roofline": {"bound": "mfma", "kernel": "whole block step (qsa_block_forward per chunk)",
                     "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                     "avg_launch_us": round(ms * 1e3 / len(calls), 1),
                     "flops_per_launch": round((proj + attn) / len(calls)), "traffic": None},
    }), flush=True)


def graph_timing(torch, run, steps, stream, replays=3):
    """Capture run() (the timed steps) into one graph and time replays of it
    with events on the replay stream: per-step milliseconds, or None when
    the capture fails."""
    try:
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            run()  # warm the capture stream
        stream.wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run()
        torch.cuda.synchronize()
        g.replay()  # first replay uploads the graph
        torch.cuda.synchronize()
        cur = torch.cuda.current_stream()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(cur)
        for _ in range(replays):
            g.replay()
        b.record(cur)
        torch.cuda.synchronize()
        return {"ms_per_step": round(a.elapsed_time(b) / (replays * steps), 5),
                "replays": replays}
    except Exception as e:  # noqa: BLE001  (reported, not fatal)
        log(f"[bench] graph timing failed: {e}")
        return None


def counter_traffic(summary_name):
    """HBM bytes per attention launch from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE, copy-calibrated), or None when the kernel
    source has changed since the counters were taken."""
    from block_sparse_attention_keys_amd import profiling
    s = profiling.read_summary(os.path.join(ROOT, "profiles", summary_name))
    if not s or s.get("kernel_source_sha256") != profiling.kernel_source_sha256():
        return None
    return int(float(s["traffic_bytes_per_launch"]))


def bench_prefill(args, name):
    """Chunked prefill of one sequence: a step is every chunk call of the
    workload in order (append, pool, score, select, attend per chunk).  The
    value is selected attention FLOP/s (4 D Hq per selected key per token)."""
    import torch
    from block_sparse_attention_keys_amd import qsa, runner, workloads
    sp = workloads.SPECS[name]
    case = workloads.make_case(name, seed=0)
    dc = runner.DeviceCase(case)
    calls = [dc.call_inputs(i) for i in range(len(case.calls))]
    outs = [dc.alloc_outputs(x) for x in calls]
    r, k = sp.block_size, sp.k_blocks
    flops, algo = [], []
    kv_row = sp.n_kv_heads * sp.head_dim * (1 if sp.kv_fp8 else 2)  # bytes per K (or V) row
    for x in calls:
        s0, e0 = x["spans"][0]
        n = np.arange(s0, e0) + 1
        nb = n // r
        nsel = r * np.minimum(k, nb) + (n - r * nb)
        flops.append(float((nsel * sp.n_q_heads * 4 * sp.head_dim).sum()))
        # algorithmic bytes of one qsa_attend launch: q, gate and out; the
        # selections and counts; each K/V row of the prefix once
        T = e0 - s0
        algo.append(3 * T * sp.n_q_heads * sp.head_dim * 2 + T * (k + 1) * 4 + e0 * kv_row * 2)
    total_flops = sum(flops)
    stream = torch.cuda.current_stream()

    def step():
        for x, o in zip(calls, outs):
            dc.forward(x, o)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps
    # dominant kernel: the attention of each chunk call, alone, bracketed by events
    st = dc.layers[0]
    ev = []
    for x, o in zip(calls, outs):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        qsa.qsa_attend(dc.params, x["batch"], x["q"], st["k"], st["v"], o["sel"], o["n_blocks"],
                       x["gate"], o["out"], o["ws"])
        b.record(stream)
        ev.append((a, b))
    torch.cuda.synchronize()
    attn_ms = [a.elapsed_time(b) for a, b in ev]
    attn_tflops = total_flops / (sum(attn_ms) * 1e-3) / 1e12
    res = {
        "metric": METRIC, "value": round(total_flops / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s (selected blocks, whole prefill step)", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": ("synthetic (seeded; N(0,1)/sqrt(d); planted blocks at 1% density" +
                 ("; K/V cached as E4M3 codes in the Hadamard basis" if sp.kv_fp8 else "") + ")"),
        "config": {"workload": name, "tokens": sp.prefill_len, "chunk": sp.chunk,
                   "kv_cache": "e4m3+hadamard" if sp.kv_fp8 else "bf16",
                   "n_q_heads": sp.n_q_heads, "n_kv_heads": sp.n_kv_heads,
                   "head_dim": sp.head_dim, "block_size": r, "budget": sp.budget},
        "selected_gflop_per_step": round(total_flops / 1e9, 2),
        "roofline": {"bound": "mfma", "kernel": ("prefill attention as qsa_attend launches it (key-stationary plan, "
                                "bf16 MFMA attention, merge)"),
                     "achieved": round(attn_tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                     "avg_launch_us": round(float(np.mean(attn_ms)) * 1e3, 1),
                     "flops_per_launch": round(total_flops / len(calls)),
                     "bytes_per_launch": round(sum(algo) / len(calls)),
                     "traffic": counter_traffic(f"attn_{name}_hbm_counters.txt")},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_prefill(case, sp, args.cpu_seconds)
    print(json.dumps(res), flush=True)


def cpu_baseline_prefill(case, sp, seconds):
    """The CPU oracle on query tokens of the last chunk (evenly spaced),
    repeated until about `seconds` of wall time; selected TFLOP/s."""
    import oracle
    from block_sparse_attention_keys_amd import workloads
    orc = oracle.load()
    dims = dict(n_q_heads=sp.n_q_heads, n_kv_heads=sp.n_kv_heads, head_dim=sp.head_dim,
                n_idx_heads=sp.n_idx_heads, idx_dim=sp.idx_dim, block_size=sp.block_size,
                budget=sp.budget, attn_scale=0.0, idx_scale=0.0)
    K, V, kI = (workloads.as_f32(case.k[0]), workloads.as_f32(case.v[0]),
                workloads.as_f32(case.kI[0]))
    n_tok = K.shape[0]
    if sp.kv_fp8:  # the cache as the oracle stores it (outside the timed loop)
        ks_, vs_ = workloads.kv_scales(sp.head_dim, sp.kv_rotate)
        Kc = orc.kv8_encode(K, sp.kv_rotate, float(np.float32(1.0) / np.float32(ks_)))
        Vc = orc.kv8_encode(V, sp.kv_rotate, float(np.float32(1.0) / np.float32(vs_)))
    pos = np.linspace(n_tok - sp.chunk, n_tok - 1, 64).astype(np.int64)
    r, k = sp.block_size, sp.k_blocks
    n = pos + 1
    nb = n // r
    flops = float(((r * np.minimum(k, nb) + n - r * nb) * sp.n_q_heads * 4 * sp.head_dim).sum())
    def timed(budget, n_pos):
        reps = 0
        t0 = time.time()
        while True:
            p = pos[:n_pos]
            if sp.kv_fp8:
                orc.sequence_kv8(dims, Kc, Vc, sp.kv_rotate, ks_, vs_, kI, p, case.q[0][p],
                                 case.qI[0][p], case.w[0][p], case.gate[0][p])
            else:
                orc.sequence(dims, K, V, kI, p, case.q[0][p], case.qI[0][p], case.w[0][p],
                             case.gate[0][p])
            reps += 1
            if time.time() - t0 >= budget:
                break
        return reps, time.time() - t0

    cores = orc.threads()
    reps, dt = timed(seconds, len(pos))
    # single core: the same oracle with one OpenMP thread, on 8 of the queries
    orc.set_threads(1)
    try:
        reps1, dt1 = timed(max(2.0, seconds / 3), 8)
    finally:
        orc.set_threads(cores)
    flops8 = float(((r * np.minimum(k, nb[:8]) + n[:8] - r * nb[:8]) * sp.n_q_heads * 4 *
                    sp.head_dim).sum())
    return {"value": round(reps * flops / dt / 1e12, 5), "unit": "TFLOP/s (selected blocks)",
            "cores": cores, "kind": "oracle",
            "gflops": round(reps * flops / dt / 1e9, 3),
            "sample": f"{reps} x 64 query tokens of the last 4096-token chunk (OpenMP over "
                      f"queries), {dt:.1f}s wall",
            "single_core": {"value": round(reps1 * flops8 / dt1 / 1e12, 6),
                            "gflops": round(reps1 * flops8 / dt1 / 1e9, 4), "cores": 1,
                            "sample": f"{reps1} x 8 of those query tokens, one thread, "
                                      f"{dt1:.1f}s wall"},
            "cpu_model": _cpu_model()}


def cpu_baseline(case, sp, seconds):
    """The CPU oracle on the same step (each sequence's new token), threads
    across sequences; repeated until about `seconds` of wall time."""
    import concurrent.futures as cf
    import oracle
    from block_sparse_attention_keys_amd import workloads

    orc = oracle.load()
    cores = len(os.sched_getaffinity(0))
    dims = dict(n_q_heads=sp.n_q_heads, n_kv_heads=sp.n_kv_heads, head_dim=sp.head_dim,
                n_idx_heads=sp.n_idx_heads, idx_dim=sp.idx_dim, block_size=sp.block_size,
                budget=sp.budget, attn_scale=0.0, idx_scale=0.0)
    B = sp.n_seqs
    f32 = [(workloads.as_f32(case.k[b]), workloads.as_f32(case.v[b]),
            workloads.as_f32(case.kI[b])) for b in range(B)]

    m = sp.q_per_step

    codes = [None] * B
    if sp.kv_fp8:  # the cache as the oracle stores it (outside the timed loop)
        ks, vs = workloads.kv_scales(sp.head_dim, sp.kv_rotate)

        def enc(b):
            K, V, _ = f32[b]
            inv_k = float(np.float32(1.0) / np.float32(ks))
            inv_v = float(np.float32(1.0) / np.float32(vs))
            codes[b] = (orc.kv8_encode(K, sp.kv_rotate, inv_k),
                        orc.kv8_encode(V, sp.kv_rotate, inv_v))

        with cf.ThreadPoolExecutor(max_workers=min(len(os.sched_getaffinity(0)), B)) as ex:
            list(ex.map(enc, range(B)))

    def one(b):
        K, V, kI = f32[b]
        p = case.ctx[b]
        if sp.kv_fp8:
            orc.sequence_kv8(dims, codes[b][0], codes[b][1], sp.kv_rotate, ks, vs, kI,
                             np.arange(p, p + m), case.q[b][:m], case.qI[b][:m],
                             case.w[b][:m], case.gate[b][:m])
            return
        orc.sequence(dims, K, V, kI, np.arange(p, p + m), case.q[b][:m], case.qI[b][:m],
                     case.w[b][:m], case.gate[b][:m])

    def step_bytes_of(b):
        """Algorithmic bytes of sequence b's decode step (selected K/V rows
        at the oracle's fp32 width counted as the cache's element size,
        pooled keys): the same formula as the GPU's step bytes."""
        r_, k_ = sp.block_size, sp.k_blocks
        tot = 0
        for i in range(m):
            n = case.ctx[b] + i + 1
            if r_ > 0:
                nb = n // r_
                nsel = r_ * min(k_, nb) + (n - r_ * nb)
                tot += nb * sp.idx_dim * 4
            else:
                nsel = n
            tot += nsel * sp.n_kv_heads * sp.head_dim * (1 if sp.kv_fp8 else 2) * 2
        return tot

    threads = min(cores, B)
    reps = 0
    t0 = time.time()
    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        while True:
            list(ex.map(one, range(B)))
            reps += 1
            if time.time() - t0 >= seconds:
                break
    dt = time.time() - t0
    # single core: one sequence at a time, one OpenMP thread, the first
    # sequences of the batch
    omp = orc.threads()
    orc.set_threads(1)
    n1, t1 = 0, time.time()
    try:
        while True:
            one(n1 % B)
            n1 += 1
            if time.time() - t1 >= max(2.0, seconds / 3):
                break
    finally:
        orc.set_threads(omp)
    dt1 = time.time() - t1
    byt1 = sum(step_bytes_of(b) for b in range(B)) * (n1 // B) + \
        sum(step_bytes_of(b) for b in range(n1 % B))
    byt = sum(step_bytes_of(b) for b in range(B)) * reps
    return {"value": round(reps * B * m / dt, 2), "unit": "tok/s", "cores": threads,
            "kind": "oracle", "GBps": round(byt / dt / 1e9, 3),
            "sample": f"{reps} x one decode step of all {B} sequences ({m} new token(s) "
                      f"each, the same inputs), threads over sequences, {dt:.1f}s wall",
            "single_core": {"value": round(n1 * m / dt1, 3), "unit": "tok/s", "cores": 1,
                            "GBps": round(byt1 / dt1 / 1e9, 4),
                            "sample": f"{n1} sequences' decode steps one after another, one "
                                      f"thread, {dt1:.1f}s wall"},
            "cpu_model": _cpu_model()}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


if __name__ == "__main__":
    main()
