"""Layer-by-layer parity of a whole generation, as the benchmark runs it (GPU side:
record; CPU side: the oracle replays the recorded layers).

The GPU runs the workload's generation exactly as the benchmark does: prefill of
every micro-batch, then the decode steps of the whole batch, greedy.  A tap on the
model copies the hidden state entering the sampled layers (and the output head) at
every call; the rows of the sampled sequences are kept on the host, with the
generated tokens and the logits of the sampled steps.

The oracle then checks, for each sampled layer l and sequence b, teacher-forced:
the layer's prefill on b's recorded input, then every decode step on b's recorded
input at that step, against the recorded input of layer l + 1 (the layer's output).
Layer 0's inputs are also compared bit for bit with the oracle's embedding of the
tokens, and the output head's input with the logits and the greedy tokens.  The
oracle's weights are drawn again from the same per-tensor seeds.

The layer's state is teacher-forced too.  The oracle quantizes its own K and V into
its cache; those entries are compared with the GPU's cache (recorded at the end of
the run), and then replaced by the GPU's, so that each decode step of the oracle
attends over the same 4-bit state as the GPU's did.  The two sides' K and V come from
GEMMs that sum in different orders and may round to fp16 one ulp apart; where such a
value sits on a code boundary the two 4-bit codes differ by one step.  One such code
at a position the softmax weights heavily moves the layer's output by more than the
output tolerance, so the state is forced, and the cache check bounds the codes
instead: every dequantized entry within one quantization step of the oracle's, and
such one-step differences rare.
"""
import numpy as np
import torch

from oracle import flexq_oracle as O
from tests.gpu_helpers import F16, to_np


def say(*a):
    print("[case]", *a, flush=True)


def record(F, wl, layers, seqs, logit_steps, seed=0):
    """Runs the generation of workload wl on the GPU; returns the recorded rows.

    layers: sampled layer indices (their inputs and outputs are recorded);
    seqs: sampled sequences; logit_steps: generated-token indices (0 = the prefill's
    token) whose fp32 logits are recorded."""
    from group_wise_bit_flexq_amd import synth, workloads
    B, S, G, mb = wl.batch, wl.prompt, wl.gen, wl.micro_batch
    seqs = list(seqs)
    say("build", wl.name)
    model = workloads.build_model(wl, seed)
    taps = sorted(set(layers) | {l + 1 for l in layers})
    bufs = dict(zip(taps, model.set_tap(taps, rows=mb * S)))
    tokens = synth.token_ids(B, S, wl.vocab, synth.sub_seed(seed, "tokens")).cuda()
    out = torch.empty(G, B, dtype=torch.int32, device="cuda")
    logits = torch.empty(B, wl.vocab, dtype=torch.float32, device="cuda")
    rec = {"tokens": to_np(tokens), "prefill": {}, "decode": {}, "logits": {}}
    say("prefill", wl.name, B // mb, "micro-batches")
    for j in range(B // mb):
        model.prefill(tokens[j * mb:(j + 1) * mb], b0=j * mb, next_out=out[0, j * mb:(j + 1) * mb],
                      logits=logits[j * mb:(j + 1) * mb] if 0 in logit_steps else None)
        for b in seqs:
            if j * mb <= b < (j + 1) * mb:
                r = (b - j * mb) * S
                rec["prefill"][b] = {t: to_np(bufs[t][r:r + S]) for t in taps}
    if 0 in logit_steps:
        rec["logits"][0] = to_np(logits[seqs])
    for i in range(G - 1):
        model.decode_step(out[i], S + i, next_out=out[i + 1],
                          logits=logits if i + 1 in logit_steps else None)
        rec["decode"][i] = {t: to_np(bufs[t][seqs]) for t in taps}
        if i + 1 in logit_steps:
            rec["logits"][i + 1] = to_np(logits[seqs])
    torch.cuda.synchronize()
    rec["out"] = to_np(out).T.copy()                         # [B][G]
    rec["seqs"] = list(seqs)
    # the 4-bit caches of the sampled layers and sequences after the whole run
    rec["cache"] = {l: {b: {n: to_np(getattr(model.caches[l], n)[b])
                            for n in ("k_codes", "v_codes", "k_params", "v_params")}
                        for b in seqs} for l in layers}
    model.set_tap(None)
    del model, bufs, logits
    torch.cuda.empty_cache()
    return rec


def _ulp(x):
    return np.spacing(np.abs(np.asarray(x, np.float64)).astype(F16)).astype(np.float64)


def r20_close(got, ref, what, x1=None):
    """Layer outputs at the large shapes: relative Frobenius <= 1e-2 and, element-wise,
    |got - ref| <= max(2e-2, 2 ulp_fp16(|ref|)), the residual stream of a deep stack
    growing past the range where 2e-2 is an fp16 ulp.  With x1 (the layer's attention
    half, an fp16 tensor on both sides that the output adds to), the element bound is
    also at least ulp(|x1|) + ulp(|ref|) + 2e-2: one rounding of x1 and one of the
    output may each land on the other neighbour, in their own binades."""
    g = np.asarray(got, np.float64)
    r = np.asarray(ref, np.float64)
    err = np.abs(g - r)
    bound = np.maximum(2e-2, 2 * _ulp(r))
    if x1 is not None:
        bound = np.maximum(bound, _ulp(x1) + _ulp(r) + 2e-2)
    rf = np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30)
    bad = err > bound
    assert not bad.any(), (f"{what}: {bad.sum()} elements beyond the bound; worst "
                           f"{err.max():.3g} at |ref| {np.abs(r).flat[err.argmax()]:.3g}")
    assert rf <= 1e-2, f"{what}: rel-frob {rf:.3g} > 1e-2"
    return err.max(), rf


def oracle_layer(wl, l, seed=0):
    """The oracle's layer l, its weights drawn again from the same seeds (on the device,
    as the GPU model drew them, then copied to the host)."""
    from group_wise_bit_flexq_amd import synth
    w16 = synth.layer_weights_fp16(wl.hidden, wl.ffn, seed, l, device="cuda")
    w = {k: v.cpu().numpy() for k, v in w16.items()}
    del w16
    torch.cuda.empty_cache()
    return O.QLayer(w, wl.heads)


class ForcedCache(O.KVCache):
    """A one-sequence oracle cache whose every store keeps the oracle's own codes for
    inspection (`own`: positions -> (k codes, k params, v codes, v params)) and then
    puts the GPU's entries of those positions in their place."""

    def __init__(self, wl, gpu):
        super().__init__(1, wl.heads, wl.head_dim, wl.max_len)
        self.gpu = gpu
        self.own = []

    def store(self, b, t0, k, v):
        super().store(b, t0, k, v)
        t1 = t0 + k.shape[1]
        self.own.append((t0, t1, self.k_codes[b, :, t0:t1].copy(),
                         self.k_params[b, :, t0:t1].copy(), self.v_codes[b, :, t0:t1].copy(),
                         self.v_params[b, :, t0:t1].copy()))
        for n in ("k_codes", "v_codes", "k_params", "v_params"):
            getattr(self, n)[b, :, t0:t1] = self.gpu[n][:, t0:t1]


def cache_close(own_c, own_p, gpu_c, gpu_p, what):
    """The GPU's 4-bit entries against the oracle's quantization of its own values:
    dequantized, every element within one quantization step (the larger of the two
    sides' steps, plus the difference of the offsets and 15 times that of the steps),
    and elements off by more than half a step rare.  Returns their count."""
    dq_o = O.dequantize_kv(own_c, own_p)
    dq_g = O.dequantize_kv(gpu_c, gpu_p)
    po, pg = own_p.astype(np.float64), gpu_p.astype(np.float64)
    step = np.maximum(po[..., 1], pg[..., 1])
    slack = np.abs(po[..., 0] - pg[..., 0]) + 15 * np.abs(po[..., 1] - pg[..., 1])
    rep = lambda a: np.repeat(a, 64, axis=-1)           # per group -> per element
    d = np.abs(dq_o - dq_g)
    assert (d <= rep(step + slack) * (1 + 2.0**-10)).all(), f"{what}: beyond one step"
    flips = int((d > 0.5 * rep(step)).sum())
    assert flips <= 2e-3 * d.size + 2, f"{what}: {flips} of {d.size} entries a step apart"
    return flips


def check_layer(wl, rec, l, seed=0):
    """Teacher-forced replay of layer l for every recorded sequence (inputs and cache
    state from the GPU's run, the cache checked against the oracle's own codes)."""
    say("oracle layer", l, "of", wl.name)
    L = oracle_layer(wl, l, seed)
    S, G = wl.prompt, wl.gen
    worst, flips, entries = 0.0, 0, 0
    nh, hd = wl.heads, wl.head_dim
    for k, b in enumerate(rec["seqs"]):
        cache = ForcedCache(wl, rec["cache"][l][b])
        # the oracle's layer in its two halves (QLayer.prefill / decode in the same
        # order), keeping the attention half's fp16 output x1 for the bound
        x = rec["prefill"][b][l]
        x1 = L._attn_block(x, lambda qkv: O.attn_prefill(qkv, 1, S, nh, hd, cache, 0))
        y = L._mlp_block(x1)
        e, _ = r20_close(rec["prefill"][b][l + 1], y, f"layer {l} prefill seq {b}", x1)
        worst = max(worst, e)
        for i in range(G - 1):
            xd = rec["decode"][i][l][k:k + 1]
            x1 = L._attn_block(xd, lambda qkv: O.attn_decode(qkv, S + i, cache, 0))
            yd = L._mlp_block(x1)
            e, _ = r20_close(rec["decode"][i][l + 1][k:k + 1], yd,
                             f"layer {l} decode step {i + 1} seq {b}", x1)
            worst = max(worst, e)
        g = rec["cache"][l][b]
        for t0, t1, kc, kp, vc, vp in cache.own:
            for name, c, p, gc, gp in (("K", kc, kp, "k_codes", "k_params"),
                                       ("V", vc, vp, "v_codes", "v_params")):
                flips += cache_close(c, p, g[gc][:, t0:t1], g[gp][:, t0:t1],
                                     f"layer {l} seq {b} {name} positions {t0}..{t1 - 1}")
                entries += c.size * 2
    say(f"layer {l}: worst abs error {worst:.3g} over {len(rec['seqs'])} sequences x "
        f"(prefill + {G - 1} decode steps); cache entries a step apart from the oracle's "
        f"own: {flips} of {entries}")
    return worst


def oracle_head(wl, seed=0):
    from group_wise_bit_flexq_amd import synth
    from group_wise_bit_flexq_amd.workloads import POS_ROWS
    dev = "cuda"
    e = synth.model_tensor("embed", (wl.vocab, wl.hidden), seed, dev).cpu().numpy()
    pos = synth.model_tensor("pos", (POS_ROWS, wl.hidden), seed, dev).cpu().numpy()
    g = synth.model_tensor("lnf_g", (wl.hidden,), seed, dev).cpu().numpy()
    b = synth.model_tensor("lnf_b", (wl.hidden,), seed, dev).cpu().numpy()
    codes, params = O.quantize(e)
    return codes, params, pos, g, b


def check_embedding(wl, rec, head):
    """Layer 0's recorded inputs are the oracle's embedding of the tokens, bit for bit."""
    codes, params, pos, _, _ = head
    S = wl.prompt
    for k, b in enumerate(rec["seqs"]):
        x = O.embed(rec["tokens"][b], np.arange(S), codes, params, pos)
        assert np.array_equal(x.view(np.uint16), rec["prefill"][b][0].view(np.uint16)), b
        for i in range(wl.gen - 1):
            xd = O.embed(rec["out"][b, i:i + 1], np.array([S + i]), codes, params, pos)
            assert np.array_equal(xd.view(np.uint16), rec["decode"][i][0][k:k + 1].view(np.uint16)), \
                (b, i)


def check_head(wl, rec, head):
    """Logits of the recorded steps from the recorded last hidden state (max-abs 2e-2,
    relative Frobenius 1e-2),
    and every greedy token: identical to the oracle's argmax unless the oracle's own top-2
    gap at that step is within twice the measured logit error (a near-tie).  Returns the
    number of near-ties."""
    codes, params, _, g, bln = head
    ew = O.dequantize_weight(codes, params).astype(np.float64)
    S, G, Lh = wl.prompt, wl.gen, wl.layers
    ties, worst = 0, 0.0
    for k, b in enumerate(rec["seqs"]):
        xs = [rec["prefill"][b][Lh][S - 1:S]] + [rec["decode"][i][Lh][k:k + 1] for i in range(G - 1)]
        for i, x in enumerate(xs):
            lg, nx = O.lm_head(x, g, bln, codes, params, ew)
            tok = rec["out"][b, i]
            err = None
            if i in rec["logits"]:
                gl = rec["logits"][i][k:k + 1]
                err, _ = r20_close(gl, lg, f"logits step {i} seq {b}")
                assert err <= 2e-2, f"logits step {i} seq {b}: max-abs {err:.3g}"
                worst = max(worst, err)
                assert tok == int(np.argmax(gl[0])), "GPU token is not its own argmax"
            if tok != nx[0]:
                gap = lg[0].max() - lg[0, tok]
                margin = 2 * (err if err is not None else max(worst, 2e-2))
                assert gap <= margin, (f"step {i} seq {b}: GPU token {tok} vs oracle {nx[0]}, "
                                       f"gap {gap:.3g} > {margin:.3g}")
                ties += 1
    say(f"head: worst logit error {worst:.3g}, near-tie token differences {ties} of "
        f"{len(rec['seqs']) * G}")
    return ties
