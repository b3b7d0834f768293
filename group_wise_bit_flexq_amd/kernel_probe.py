"""Kernel probes at workload shapes, for rocprofv3 kernel traces and counter runs.

    python -m group_wise_bit_flexq_amd.kernel_probe gemm --workload opt175b --reps 2
        the four prefill 4-bit GEMMs of one decoder layer (M = micro-batch x prompt
        rows), launched exactly as the model path launches them;
    python -m group_wise_bit_flexq_amd.kernel_probe gemm_vs_library --workload opt175b --reps 2
        the same four GEMMs beside torch.mm (the vendor library's fp16 GEMM) on the
        dequantized weights, alternated in one process;
    python -m group_wise_bit_flexq_amd.kernel_probe decode --workload opt175b --reps 2
        one decode step's 4-bit GEMMs (M = batch) and decode attention over a cache
        of prompt + gen/2 positions;
    python -m group_wise_bit_flexq_amd.kernel_probe sparse --workload opt175b --reps 10
        decode attention over a filled cache of prompt + gen/2 positions: dense, and
        top-k sparse at sparsity 1, 0.5, 0.25, 0.1 (algorithmic bytes: every K, the
        kept V);
    python -m group_wise_bit_flexq_amd.kernel_probe host_attn --workload opt175b --reps 5 --threads 16
        decode attention on the host CPU over a host-memory cache for one micro-batch of
        sequences (prompt + gen/2 positions), beside the host's multi-threaded read rate;
    python -m group_wise_bit_flexq_amd.kernel_probe host_tier --workload opt30b --reps 3 --threads 16
        the whole OPT-30B-shaped model with its last micro-batch's caches in host memory,
        beside the all-device model: prefill per micro-batch and decode step times;
    python -m group_wise_bit_flexq_amd.kernel_probe prefill_attn --workload opt175b --reps 3
        causal prefill attention of one micro-batch (micro_batch x prompt tokens, all
        heads) with the fused 4-bit KV store;
    python -m group_wise_bit_flexq_amd.kernel_probe quant --reps 3
        the standalone quantizer on a 4 GiB fp16 tensor [524288][4096];
    python -m group_wise_bit_flexq_amd.kernel_probe quant_ex --reps 3
        the general-config quantizer on the same tensor at 3 bits, group 64, asymmetric
        (groups along the rows, and along the columns: group_dim 0);
    python -m group_wise_bit_flexq_amd.kernel_probe stress --reps 3
        decode attention of the KV-compression stress shape (batch 64, 56 heads x 128,
        cache of 2048 + 64 positions);
    python -m group_wise_bit_flexq_amd.kernel_probe pick --workload opt175b --reps 5
        the token choice of one decode step (batch x vocab fp32 logits): greedy, and
        temperature sampling with a stop token;
    python -m group_wise_bit_flexq_amd.kernel_probe mfma --reps 3
        the matrix cores' sustained fp16 rate (v_mfma_f32_32x32x16_f16 streams, two waves
        per SIMD on every CU) with constant, fixed random and changing random operands:
        the ceiling the GEMMs' TFLOP/s are read against;
    python -m group_wise_bit_flexq_amd.kernel_probe copy --mib 1024 --reps 3
        an elementwise device copy of a known size, the reference that scales the
        HBM byte counters (FETCH_SIZE / WRITE_SIZE) of the probes above, and a
        measured HBM rate (read + write) beside the nominal 8 TB/s.
Each prints its per-launch times (HIP events) as one JSON line; --warm S runs the
calls untimed for about S seconds first (the clock of a GPU that was idle ramps up).
"""
from __future__ import annotations

import argparse
import json
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))


WARM_S = 0.0   # set by --warm


def _time(fn, reps):
    """Average time of one call, from `reps` calls launched back to back between two
    events: the host's per-call argument handling overlaps the previous call's kernels,
    as it does in the generation loop, instead of being timed as GPU idle time.  With
    --warm S the calls first run for about S seconds (at most 2000 calls): a GPU that
    has just been idle runs its first milliseconds of work at a lower clock.  Without
    it (the default, used by the counter runs) one untimed call precedes the timed ones."""
    import time

    import torch
    warm_s = WARM_S
    fn()
    torch.cuda.synchronize()
    t0, n = time.perf_counter(), 0
    while time.perf_counter() - t0 < warm_s and n < 2000:
        fn()
        n += 1
        if n % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def gemm(wl, reps, rows):
    import torch

    from group_wise_bit_flexq_amd import flexq as F
    from group_wise_bit_flexq_amd import synth
    h, f = wl.hidden, wl.ffn
    w16 = synth.layer_weights_fp16(h, f, 0, 0, device="cuda")
    L = F.QLayer.from_fp16(w16, wl.heads)
    del w16
    res = {}
    for name, (n, k) in {"wqkv": (3 * h, h), "wo": (h, h), "w1": (f, h), "w2": (h, f)}.items():
        x = synth.normal_fp16((rows, k), 1.0, 1, device="cuda")
        y = torch.empty(rows, n, dtype=torch.float16, device="cuda")
        ws = torch.empty(max(F.linear_ws_bytes(rows, n, k), 16), dtype=torch.uint8, device="cuda")
        ms = _time(lambda: F.linear_w4(x, L.m[name], bias=L.v["b1"] if name == "w1" else None,
                                       out=y, ws=ws), reps)
        res[name] = {"M": rows, "N": n, "K": k, "ms": ms, "tflops": 2 * rows * n * k / ms / 1e9}
        del x, y, ws
    return res


def gemm_vs_library(wl, reps, rows, rounds=3):
    """The prefill GEMMs beside the vendor library's plain fp16 GEMM on the same shapes
    (torch.mm, i.e. hipBLASLt, on the dequantized weights: what the 4-bit GEMM would
    cost if the weights were kept in fp16), alternated in one process."""
    import torch

    from group_wise_bit_flexq_amd import flexq as F
    from group_wise_bit_flexq_amd import synth
    h, f = wl.hidden, wl.ffn
    w16 = synth.layer_weights_fp16(h, f, 0, 0, device="cuda")
    L = F.QLayer.from_fp16(w16, wl.heads)
    shapes = {"wqkv": (3 * h, h), "wo": (h, h), "w1": (f, h), "w2": (h, f)}
    res = {name: {"M": rows, "N": n, "K": k, "w4_ms": [], "fp16_library_ms": []}
           for name, (n, k) in shapes.items()}
    for _ in range(rounds):
        for name, (n, k) in shapes.items():
            x = synth.normal_fp16((rows, k), 1.0, 1, device="cuda")
            y = torch.empty(rows, n, dtype=torch.float16, device="cuda")
            ws = torch.empty(max(F.linear_ws_bytes(rows, n, k), 16), dtype=torch.uint8,
                             device="cuda")
            res[name]["w4_ms"].append(_time(lambda: F.linear_w4(x, L.m[name], out=y, ws=ws), reps))
            wd = F.dequantize(F.quantize(w16[name]))     # [n][k] fp16: the same codes
            res[name]["fp16_library_ms"].append(_time(lambda: torch.mm(x, wd.t(), out=y), reps))
            del x, y, ws, wd
    for name, r in res.items():
        fl = 2.0 * r["M"] * r["N"] * r["K"]
        r["w4_tflops"] = fl / min(r["w4_ms"]) / 1e9
        r["fp16_library_tflops"] = fl / min(r["fp16_library_ms"]) / 1e9
    return res


def decode(wl, reps):
    import torch

    from group_wise_bit_flexq_amd import flexq as F
    res = gemm(wl, reps, wl.batch)
    T = wl.prompt + wl.gen // 2
    kv = F.KV4(wl.batch, wl.heads, wl.head_dim, T + 1)
    qkv = torch.randn(wl.batch, 3 * wl.hidden, device="cuda").half()
    out = torch.empty(wl.batch, wl.hidden, dtype=torch.float16, device="cuda")
    ws = torch.empty(max(F.attn_decode_ws_bytes(wl.batch, wl.heads, wl.head_dim, T), 16),
                     dtype=torch.uint8, device="cuda")
    ms = _time(lambda: F.attn_decode(qkv, T, kv, out=out, ws=ws), reps)
    nbytes = wl.batch * wl.heads * (T + 1) * 2 * wl.head_dim * 0.5625
    res["attn_decode"] = {"T": T + 1, "ms": ms, "gbps": nbytes / ms / 1e6}
    return res


def sparse(wl, reps):
    """Decode attention over a filled cache (random codes, offsets N(0, 0.25), steps
    U(0.01, 0.1)): dense, then top-k at several sparsities."""
    import torch

    from group_wise_bit_flexq_amd import flexq as F
    B, nh, hd = wl.batch, wl.heads, wl.head_dim
    T = wl.prompt + wl.gen // 2
    kv = F.KV4(B, nh, hd, T + 1)
    for c in (kv.k_codes, kv.v_codes):
        c.random_(0, 256)
    for p in (kv.k_params, kv.v_params):
        p[..., 0].normal_(0.0, 0.5)
        p[..., 1].uniform_(0.01, 0.1)
    qkv = torch.randn(B, 3 * wl.hidden, device="cuda").half()
    out = torch.empty(B, wl.hidden, dtype=torch.float16, device="cuda")
    ws = torch.empty(max(F.attn_decode_ws_bytes(B, nh, hd, T), 16), dtype=torch.uint8,
                     device="cuda")
    row = hd * 0.5625                       # bytes of one position's K (or V) in one head
    res = {"T": T + 1}
    ms = _time(lambda: F.attn_decode(qkv, T, kv, out=out, ws=ws), reps)
    res["dense"] = {"ms": ms, "gbps": B * nh * (T + 1) * 2 * row / ms / 1e6}
    for sp in (1.0, 0.5, 0.25, 0.1):
        k = max(1, int(-(-(sp * (T + 1)) // 1)))
        ms = _time(lambda: F.attn_decode_topk(qkv, T, kv, sp, out=out), reps)
        nbytes = B * nh * ((T + 1) + k) * row   # every K, the kept V
        res[f"topk_{sp}"] = {"kept": k, "ms": ms, "gbps": nbytes / ms / 1e6}
    return res


def host_attn(wl, reps, threads):
    """Decode attention on the host CPU over a host-memory cache: the sequences of one
    micro-batch of the workload (prompt + gen/2 positions, random codes), beside the
    host's multi-threaded read rate (a float32 sum over 2 GiB)."""
    import time

    import torch

    from group_wise_bit_flexq_amd import flexq as F
    B, nh, hd = wl.micro_batch, wl.heads, wl.head_dim
    T = wl.prompt + wl.gen // 2
    kv = F.KV4(B, nh, hd, T + 1, device="cpu")
    for c in (kv.k_codes, kv.v_codes):
        c.random_(0, 256)
    for p in (kv.k_params, kv.v_params):
        p[..., 0].normal_(0.0, 0.5)
        p[..., 1].uniform_(0.01, 0.1)
    qkv = torch.randn(B, 3 * wl.hidden).half()
    out = torch.empty(B, wl.hidden, dtype=torch.float16)
    F.host_attn_decode(qkv, T, kv, out=out, threads=threads)
    t0 = time.perf_counter()
    for _ in range(reps):
        F.host_attn_decode(qkv, T, kv, out=out, threads=threads)
    ms = (time.perf_counter() - t0) * 1e3 / reps
    nbytes = B * nh * (T + 1) * 2 * hd * 0.5625
    torch.set_num_threads(threads)
    x = torch.rand(1 << 29)
    x.sum()
    t0 = time.perf_counter()
    for _ in range(reps):
        x.sum()
    read_gbps = x.numel() * 4 * reps / (time.perf_counter() - t0) / 1e9
    return {"B": B, "heads": nh, "T": T + 1, "threads": threads, "ms": ms,
            "gbps": nbytes / ms / 1e6, "host_read_gbps": read_gbps}


def host_tier(wl, reps, threads):
    """Whole-model timing with the last micro-batch's caches in host memory
    (flexq_host_tier) beside the all-device model on the same weights: prefill time of
    a device and of a host micro-batch, and the decode step time."""
    import time

    import torch

    from group_wise_bit_flexq_amd import flexq as F
    from group_wise_bit_flexq_amd import synth
    from group_wise_bit_flexq_amd.workloads import POS_ROWS
    h, f, nh, mb, S = wl.hidden, wl.ffn, wl.heads, wl.micro_batch, wl.prompt
    layers = []
    for l in range(wl.layers):
        w16 = synth.layer_weights_fp16(h, f, 0, l, device="cuda")
        layers.append(F.QLayer.from_fp16(w16, nh, "cuda"))
        del w16
    emb = F.quantize_weight(synth.model_tensor("embed", (wl.vocab, h), 0, "cuda"))
    pos = synth.model_tensor("pos", (POS_ROWS, h), 0, "cuda")
    g = synth.model_tensor("lnf_g", (h,), 0, "cuda")
    b = synth.model_tensor("lnf_b", (h,), 0, "cuda")
    toks = synth.token_ids(wl.batch, S, wl.vocab, 1).cuda()
    res = {"host_rows": mb, "threads": threads}
    for name, hr in (("device", 0), ("host_tier", mb)):
        m = F.QModel(layers, emb, pos, g, b, nh, wl.batch, wl.max_len, mb * S, "cuda",
                     host_rows=hr, host_threads=threads, max_prefill_batch=mb)
        pre = []
        for j in range(wl.batch // mb):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            m.prefill(toks[j * mb:(j + 1) * mb], b0=j * mb)
            torch.cuda.synchronize()
            pre.append((time.perf_counter() - t0) * 1e3)
        cur = torch.zeros(wl.batch, dtype=torch.int32, device="cuda")
        m.decode_step(cur, S)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(reps):
            m.decode_step(cur, S + 1 + i)
        torch.cuda.synchronize()
        res[name] = {"prefill_ms": pre, "decode_step_ms": (time.perf_counter() - t0) * 1e3 / reps}
        del m
        torch.cuda.empty_cache()
    return res


def prefill_attn(wl, reps):
    import torch

    from group_wise_bit_flexq_amd import flexq as F
    from group_wise_bit_flexq_amd import synth
    B, S, nh, hd = wl.micro_batch, wl.prompt, wl.heads, wl.head_dim
    kv = F.KV4(B, nh, hd, S)
    qkv = synth.normal_fp16((B * S, 3 * nh * hd), 1.0, 7, device="cuda")
    out = torch.empty(B * S, nh * hd, dtype=torch.float16, device="cuda")
    ms = _time(lambda: F.attn_prefill(qkv, B, S, kv, out=out), reps)
    flop = B * nh * 2 * (2 * hd * S * (S + 1) / 2)      # QK^T and PV over the causal half
    return {"B": B, "S": S, "heads": nh, "head_dim": hd, "ms": ms, "tflops": flop / ms / 1e9}


def quant(reps):
    import torch

    from group_wise_bit_flexq_amd import flexq as F
    from group_wise_bit_flexq_amd import synth
    from group_wise_bit_flexq_amd.workloads import QUANT_4GIB
    rows, cols = QUANT_4GIB["rows"], QUANT_4GIB["cols"]
    x = synth.normal_fp16((rows, cols), 1.0, 5, device="cuda")
    w = F.Q4.empty(rows, cols)
    ms = _time(lambda: F.quantize(x, out=w), reps)
    nbytes = rows * cols * 2.5625
    return {"elements": rows * cols, "ms": ms, "gbps": nbytes / ms / 1e6}


def quant_ex(reps):
    import torch

    from group_wise_bit_flexq_amd import flexq as F
    from group_wise_bit_flexq_amd import synth
    from group_wise_bit_flexq_amd.workloads import QUANT_4GIB
    rows, cols = QUANT_4GIB["rows"], QUANT_4GIB["cols"]
    x = synth.normal_fp16((rows, cols), 1.0, 5, device="cuda")
    nbytes = rows * cols * (2 + 3 / 8 + 4 / 64)
    res = {}
    for name, gd in (("innermost", -1), ("group_dim0", 0)):
        ms = _time(lambda: F.quantize_ex(x, 3, 64, gd), reps)
        res[name] = {"elements": rows * cols, "ms": ms, "gbps": nbytes / ms / 1e6}
    return res


def stress(reps):
    import torch

    from group_wise_bit_flexq_amd import flexq as F
    from group_wise_bit_flexq_amd.workloads import KV_STRESS as c
    B, nh, hd = c["batch"], c["heads"], c["head_dim"]
    T = c["prompt"] + c["steps"] - 1
    kv = F.KV4(B, nh, hd, T + 1)
    qkv = torch.randn(B, 3 * nh * hd, device="cuda").half()
    out = torch.empty(B, nh * hd, dtype=torch.float16, device="cuda")
    ws = torch.empty(max(F.attn_decode_ws_bytes(B, nh, hd, T), 16), dtype=torch.uint8,
                     device="cuda")
    ms = _time(lambda: F.attn_decode(qkv, T, kv, out=out, ws=ws), reps)
    nbytes = B * nh * (T + 1) * 2 * hd * 0.5625
    return {"T": T + 1, "ms": ms, "gbps": nbytes / ms / 1e6}


def pick(wl, reps):
    import torch

    from group_wise_bit_flexq_amd import flexq as F
    M, N = wl.batch, wl.vocab
    lg = torch.randn(M, N, device="cuda") * 3
    out = torch.empty(M, dtype=torch.int32, device="cuda")
    stopped = torch.zeros(M, dtype=torch.int32, device="cuda")
    res = {}
    for name, gen in (("greedy", None), ("sample_t0.7_stop", F.gen_config(True, 0.7, 1, 2))):
        ms = _time(lambda: F.pick(lg, gen, step=100, stopped=stopped, out=out), reps)
        res[name] = {"M": M, "N": N, "ms": ms, "logit_gbps": M * N * 4 / ms / 1e6}
    return res


def mfma(reps, iters=20000):
    import torch

    from group_wise_bit_flexq_amd import flexq as F
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks = 2 * cus
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    flop = blocks * 4 * iters * 4 * 32768.0          # 4 waves x iters x 4 MFMAs x 32x32x16x2
    res = {"cus": cus, "blocks": blocks, "iters": iters}
    for mode, name in ((0, "constant"), (1, "random_fixed"), (2, "random_changing")):
        ms = _time(lambda: F.probe_mfma(mode, blocks, iters, out=out), reps)
        res[name] = {"ms": ms, "tflops": flop / ms / 1e9}
    return res


def copy(mib, reps):
    import torch
    n = mib * (1 << 20) // 2
    src = torch.randn(n, device="cuda").half()
    dst = torch.empty_like(src)
    ms = _time(lambda: torch.mul(src, 1.0, out=dst), reps)
    return {"bytes_read": 2 * n, "bytes_written": 2 * n, "ms": ms, "gbps": 4 * n / ms / 1e6}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("what", choices=["gemm", "gemm_vs_library", "decode", "sparse", "host_attn", "host_tier",
                                     "prefill_attn", "quant", "quant_ex", "stress", "pick",
                                     "mfma", "copy"])
    ap.add_argument("--threads", type=int, default=16)
    ap.add_argument("--workload", default="opt175b")
    ap.add_argument("--reps", type=int, default=2)
    ap.add_argument("--mib", type=int, default=1024)
    ap.add_argument("--warm", type=float, default=0.0,
                    help="seconds of untimed calls before each timed batch (default: one call)")
    a = ap.parse_args()
    global WARM_S
    WARM_S = max(a.warm, 0.0)
    from group_wise_bit_flexq_amd import flexq as F
    from group_wise_bit_flexq_amd.workloads import WORKLOADS
    F.lib()
    wl = WORKLOADS[a.workload]
    if a.what == "gemm":
        r = gemm(wl, a.reps, wl.micro_batch * wl.prompt)
    elif a.what == "gemm_vs_library":
        r = gemm_vs_library(wl, a.reps, wl.micro_batch * wl.prompt)
    elif a.what == "decode":
        r = decode(wl, a.reps)
    elif a.what == "host_tier":
        r = host_tier(wl, a.reps, a.threads)
    elif a.what == "host_attn":
        r = host_attn(wl, a.reps, a.threads)
    elif a.what == "sparse":
        r = sparse(wl, a.reps)
    elif a.what == "prefill_attn":
        r = prefill_attn(wl, a.reps)
    elif a.what == "quant":
        r = quant(a.reps)
    elif a.what == "quant_ex":
        r = quant_ex(a.reps)
    elif a.what == "stress":
        r = stress(a.reps)
    elif a.what == "pick":
        r = pick(wl, a.reps)
    elif a.what == "mfma":
        r = mfma(a.reps)
    else:
        r = copy(a.mib, a.reps)
    print(json.dumps({"probe": a.what, "workload": a.workload, "results": r}), flush=True)


if __name__ == "__main__":
    main()
