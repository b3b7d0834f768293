#!/usr/bin/env python3
"""Throughput of 4-bit weight + 4-bit KV-cache greedy generation on one MI355X.

One step = one full generation on the workload: prefill of the 144 prompts (three
micro-batches of 48, each the whole layer stack) followed by 31 decode steps of the
whole batch, i.e. 32 generated tokens per sequence.  Throughput follows the FlexGen
walkthrough, section 5.1: generated tokens / (prompt processing + generation time).

Default workload: OPT-175B shape (96 layers, hidden 12288, 96 heads x 128, FFN
49152, vocab 50272), batch 144, prompt 512, 32 new tokens; weights ~N(0, 0.02)
generated on the device, quantized once with flexq_quantize (load time, not timed).

Prints one JSON line.  `roofline` is measured live: HIP events bracket every prefill
4-bit GEMM launch of the timed steps on the stream they run on.  `cpu_baseline`
times the oracle on a bounded sample of the same workload and extrapolates.

Run length.  A step of the OPT-175B workload is a whole generation (about 20 s on
one MI355X), so --steps and --warmup are upper bounds: after the first warm-up step
the run keeps as many further warm-up steps as fit in a quarter of --budget-s and as
many timed steps as fit in --budget-s (at least one).  The JSON line reports the
counts actually run (`steps`, `warmup`) next to the requested ones.

--graph captures each decode step (one graph per position) in a HIP graph once,
outside the timed region, and replays them inside it; prefill runs eagerly.
"""
from __future__ import annotations

import argparse
import ctypes as C
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP16_TFLOPS = 2500.0   # MI355X dense fp16/bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
PAGES_TOKS_PER_S = 1.12     # OPT-175B, W4+KV4, batch 144, 512/32 (T4 + offloading)
W4_BYTES_PER_ELEM = 0.5625


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="opt175b")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--budget-s", type=float, default=90.0,
                    help="wall-clock seconds the timed steps may take (caps --steps)")
    ap.add_argument("--graph", action="store_true",
                    help="replay the decode steps from HIP graphs captured once")
    return ap.parse_args()


class Hip:
    """The few HIP runtime calls bench needs for events (torch's runtime, already loaded)."""

    def __init__(self):
        self.lib = C.CDLL("libamdhip64.so.7")
        self.lib.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.lib.hipEventDestroy.argtypes = [C.c_void_p]

    def events(self, n):
        arr = (C.c_void_p * n)()
        for i in range(n):
            e = C.c_void_p()
            if self.lib.hipEventCreate(C.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            arr[i] = e
        return arr

    def elapsed_ms(self, a, b):
        ms = C.c_float()
        if self.lib.hipEventElapsedTime(C.byref(ms), C.c_void_p(a), C.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, arr):
        for e in arr:
            self.lib.hipEventDestroy(C.c_void_p(e))


def generate(model, wl, tokens, out, trace_ptr=None, events=None, graphs=None):
    """One step: prefill per micro-batch, then gen-1 decode steps over the whole batch.

    out: int32 [gen][batch]; row i receives the i-th generated token of every sequence
    (decode step i reads row i - 1 and writes row i in place, so nothing is copied).
    events: optional three torch.cuda.Events recorded at start / end of prefill / end.
    graphs: optional HIP graphs of the decode steps (see capture_decode)."""
    mb, S = wl.micro_batch, wl.prompt
    if events:
        events[0].record()
    model._struct.trace = trace_ptr
    for j in range(wl.batch // mb):
        model.prefill(tokens[j * mb:(j + 1) * mb], b0=j * mb, next_out=out[0, j * mb:(j + 1) * mb])
    model._struct.trace = None
    if events:
        events[1].record()
    for i in range(wl.gen - 1):
        if graphs:
            graphs[i].replay()
        else:
            model.decode_step(out[i], S + i, next_out=out[i + 1])
    if events:
        events[2].record()


def capture_decode(model, wl, out):
    """One HIP graph per decode position: step i reads out[i], writes out[i + 1]."""
    import torch
    graphs = []
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(wl.gen - 1):      # eager once, so every kernel is loaded
            model.decode_step(out[i], wl.prompt + i, next_out=out[i + 1])
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for i in range(wl.gen - 1):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            model.decode_step(out[i], wl.prompt + i, next_out=out[i + 1])
        graphs.append(g)
    torch.cuda.synchronize()
    return graphs


def decode_bytes(wl):
    """Algorithmic HBM bytes of the gen-1 decode steps: 4-bit weights, LM head, KV4 reads."""
    h = wl.hidden
    w = wl.layers * 12 * h * h * W4_BYTES_PER_ELEM + wl.vocab * h * W4_BYTES_PER_ELEM
    total = 0.0
    for i in range(wl.gen - 1):
        T = wl.prompt + i + 1
        total += w + wl.layers * wl.batch * T * 2 * h * W4_BYTES_PER_ELEM
    return total


def gemm_source_hash():
    """Hash of the device code the prefill GEMM is built from: common.h and gemm_w4.hip
    up to its small-M kernels (changes to the decode kernels or to host-side planning
    do not invalidate counters taken on the prefill kernel)."""
    csrc = os.path.join(ROOT, "group_wise_bit_flexq_amd", "csrc")
    gemm = open(os.path.join(csrc, "gemm_w4.hip"), "rb").read()
    cut = gemm.find(b"// ------------------------------------------------------------------ small-M kernel")
    body = open(os.path.join(csrc, "common.h"), "rb").read() + (gemm[:cut] if cut >= 0 else gemm)
    return hashlib.sha256(body).hexdigest()[:16]


def traffic_from_profiles(wl):
    """HBM bytes per prefill-GEMM launch from the committed rocprofv3 counter summary,
    or None if it is missing or was taken on a different GEMM source."""
    p = os.path.join(ROOT, "profiles", "gemm_w4_prefill_traffic.json")
    try:
        d = json.load(open(p))
    except (OSError, ValueError):
        return None
    if d.get("gemm_source_sha256_16") != gemm_source_hash() or d.get("workload") != wl.name:
        return None
    return d.get("bytes_per_launch")


def cpu_baseline(wl, seed):
    """Time the oracle on a bounded sample of the workload and extrapolate to a full step.

    Sample (layer-shaped pieces of the workload): the 4-bit linear of one 512-token
    prompt and of one 144-token decode step against 16384 weight rows of width h,
    causal prefill attention of 2 sequences x all heads, and decode attention of 16
    sequences over a cache of prompt + gen/2 positions.  Each piece is scaled by how
    often one full step repeats it (weight rows x tokens for the linears, the LM head
    included; sequences x layers for attention).  LayerNorm and the embedding are
    left out (< 0.1 % of the work).
    """
    from threadpoolctl import threadpool_info

    from group_wise_bit_flexq_amd import synth
    from oracle import flexq_oracle as O

    h, nh, hd, S, B, L, G = wl.hidden, wl.heads, wl.head_dim, wl.prompt, wl.batch, wl.layers, wl.gen
    rows = min(16384, 12 * h)
    codes, params = O.quantize(synth.normal_fp16((rows, h), 0.02, 17).numpy())
    xp = synth.normal_fp16((S, h), 1.0, 18).numpy()
    xd = synth.normal_fp16((B, h), 1.0, 19).numpy()

    def timed(fn):
        t = time.perf_counter()
        fn()
        return time.perf_counter() - t

    t_lin_p = timed(lambda: O.linear_w4(xp, codes, params))
    t_lin_d = timed(lambda: O.linear_w4(xd, codes, params))
    del codes, params
    ns_p = 2
    qkv = synth.normal_fp16((ns_p * S, 3 * h), 1.0, 20).numpy()
    t_att_p = timed(lambda: O.attn_prefill(qkv, ns_p, S, nh, hd))
    del qkv
    T = S + G // 2
    ns_d = 16
    cache = O.KVCache(ns_d, nh, hd, T + 1)
    for b in range(ns_d):
        kvx = synth.normal_fp16((nh, T, hd), 1.0, 21 + b).numpy()
        cache.store(b, 0, kvx, kvx)
    q1 = synth.normal_fp16((ns_d, 3 * h), 1.0, 40).numpy()
    t_att_d = timed(lambda: O.attn_decode(q1, T, cache))
    sample_s = t_lin_p + t_lin_d + t_att_p + t_att_d

    wrows = L * 12 * h                               # weight rows of width h in the layer stack
    full = (t_lin_p * (wrows / rows) * B             # prefill linears, one 512-token prompt each
            + t_lin_d * (wrows / rows) * (G - 1)     # decode linears, M = batch per step
            + t_lin_d * (wl.vocab / rows) * G        # LM head (prefill rows + decode steps)
            + t_att_p * (B / ns_p) * L               # prefill attention
            + t_att_d * (B / ns_d) * L * (G - 1))    # decode attention
    threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    return {
        "value": B * G / full,
        "unit": "tokens/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"{wl.name} shapes: 4-bit linear of {S} prompt tokens and of {B} decode tokens "
                   f"against {rows} weight rows x {h}, prefill attention {ns_p} seqs x {nh} heads "
                   f"(S={S}), decode attention {ns_d} seqs x {nh} heads at T={T}; {sample_s:.1f} s "
                   f"measured on the host, extrapolated to one full step ({full:.3g} s)"),
        "extrapolated": True,
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the path is single-GPU by design).", file=sys.stderr)
        sys.exit(2)
    import torch

    from group_wise_bit_flexq_amd import flexq as F
    from group_wise_bit_flexq_amd import synth, workloads

    wl = workloads.WORKLOADS[args.workload]
    assert wl.full_model and wl.batch % wl.micro_batch == 0
    F.lib()
    hip = Hip()
    log(f"workload {wl}")
    model = workloads.build_model(wl, args.seed, log=log)
    tokens = synth.token_ids(wl.batch, wl.prompt, wl.vocab, synth.sub_seed(args.seed, "tokens"))
    tokens = tokens.cuda()
    out = torch.empty(wl.gen, wl.batch, dtype=torch.int32, device="cuda")
    graphs = None
    if args.graph:
        t = time.perf_counter()
        generate(model, wl, tokens, out)     # fills the caches the captured steps read
        graphs = capture_decode(model, wl, out)
        log(f"captured {len(graphs)} decode-step graphs ({time.perf_counter() - t:.1f}s)")

    # warm-up: the first step measures the step time, the rest fit in budget / 4
    warm, step_s = 0, None
    t_w = time.perf_counter()
    while warm < args.warmup:
        t = time.perf_counter()
        generate(model, wl, tokens, out, graphs=graphs)
        torch.cuda.synchronize()
        step_s = time.perf_counter() - t
        warm += 1
        log(f"warmup {warm}/{args.warmup} done ({step_s:.2f}s)")
        if time.perf_counter() - t_w + step_s > 0.25 * args.budget_s:
            break
    steps = max(1, min(args.steps, int(args.budget_s // step_s))) if step_s else args.steps
    if steps < args.steps:
        log(f"timing {steps} of {args.steps} requested steps ({step_s:.1f}s each, "
            f"budget {args.budget_s:.0f}s)")

    # trace of the prefill linears (events recorded by the library on its stream)
    n_mb = wl.batch // wl.micro_batch
    cap = n_mb * (wl.layers * 4 + 1) * steps
    ev = hip.events(2 * cap)
    kinds = (C.c_int32 * cap)()
    rows = (C.c_int64 * cap)()
    trace = F.TraceStruct(C.cast(ev, C.POINTER(C.c_void_p)), kinds, rows, cap, 0)

    e_pre = [torch.cuda.Event(enable_timing=True) for _ in range(3 * steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    done = 0
    while done < steps:
        generate(model, wl, tokens, out, C.pointer(trace), events=e_pre[3 * done:3 * done + 3],
                 graphs=graphs)
        done += 1
        log(f"step {done}/{steps} enqueued")
        if step_s is None:        # no warm-up: the first timed step sets the count
            torch.cuda.synchronize()
            step_s = time.perf_counter() - t0
            steps = max(1, min(steps, int(args.budget_s // step_s)))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    prefill_ms = sum(e_pre[3 * s].elapsed_time(e_pre[3 * s + 1]) for s in range(steps))
    decode_ms = sum(e_pre[3 * s + 1].elapsed_time(e_pre[3 * s + 2]) for s in range(steps))
    log(f"timed {steps} step(s): wall {wall:.2f}s prefill {prefill_ms / 1e3:.2f}s "
        f"decode {decode_ms / 1e3:.2f}s")

    # dominant kernel: the prefill 4-bit GEMM (every linear of a prefill micro-batch)
    h, f = wl.hidden, wl.ffn
    nk = {0: (3 * h, h), 1: (h, h), 2: (f, h), 3: (h, f), 4: (wl.vocab, h)}
    gemm_ms, gemm_flop, n_launch = 0.0, 0.0, 0
    for i in range(trace.count):
        if kinds[i] == 4:
            continue
        N, K = nk[kinds[i]]
        gemm_ms += hip.elapsed_ms(ev[2 * i], ev[2 * i + 1])
        gemm_flop += 2.0 * rows[i] * N * K
        n_launch += 1
    hip.destroy(ev)
    achieved = gemm_flop / (gemm_ms / 1e3) / 1e12 if gemm_ms > 0 else 0.0
    traffic = traffic_from_profiles(wl)

    gen_tokens = wl.batch * wl.gen * steps
    value = gen_tokens / wall
    dec_gbps = decode_bytes(wl) * steps / (decode_ms / 1e3) / 1e9
    metric = "generated tokens/s, OPT-175B-shape W4+KV4 batch 144; decode HBM GB/s vs peak"
    if wl.name != "opt175b":
        metric = (f"generated tokens/s, {wl.name}-shape W4+KV4 batch {wl.batch}; "
                  "decode HBM GB/s vs peak")
    res = {
        "metric": metric,
        "value": round(value, 3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "steps_requested": args.steps,
        "warmup_requested": args.warmup,
        "budget_s": args.budget_s,
        "ms_per_step": round(wall * 1e3 / steps, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(value / PAGES_TOKS_PER_S, 2) if wl.name == "opt175b" else None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {
            "workload": (f"{wl.name}-shape greedy generation: {wl.layers} layers, hidden {wl.hidden}, "
                         f"{wl.heads} heads x {wl.head_dim}, ffn {wl.ffn}, vocab {wl.vocab}; 4-bit "
                         f"weights and KV cache (group 64, asymmetric); batch {wl.batch} (prefill "
                         f"micro-batches of {wl.micro_batch}), prompt {wl.prompt}, {wl.gen} new tokens"),
            "global_batch": wl.batch,
            "seq_len": wl.prompt,
            "gen_len": wl.gen,
            "parallelism": "single GPU",
            "decode_graphs": bool(graphs),
        },
        "prefill_s": round(prefill_ms / 1e3 / steps, 3),
        "decode_s": round(decode_ms / 1e3 / steps, 3),
        "decode_hbm_gbps": round(dec_gbps, 1),
        "decode_hbm_frac": round(dec_gbps / PEAK_HBM_GBPS, 4),
        "roofline": {
            "kernel": "gemm_w4_big_kernel<2,4,4,2,0> (prefill, 256x256x64 tile, 8 waves)",
            "bound": "mfma",
            "achieved": round(achieved, 1),
            "peak": PEAK_FP16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_FP16_TFLOPS, 4),
            "traffic": traffic,
            "launches": n_launch,
            "avg_launch_ms": round(gemm_ms / max(n_launch, 1), 4),
            "flop_per_launch": gemm_flop / max(n_launch, 1),
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("timing the oracle on a bounded sample ...")
        res["cpu_baseline"] = cpu_baseline(wl, args.seed)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
