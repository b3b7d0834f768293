"""Workload shapes: OPT-shaped decoder stacks and the generation sizes run on them.

The pages measure OPT models at prompt 512 / 32 generated tokens with an effective
batch of 144 = 48 x 3 for the 4-bit weight + KV configuration (FlexGen article,
section 5.1 and the --gpu-batch-size/--num-gpu-batches flags of section 2.3).
Vocabulary 50272 and learned positions with an offset of 2 are the OPT conventions.
"""
from __future__ import annotations

from dataclasses import dataclass

VOCAB = 50272
POS_ROWS = 2050          # 2048 learned positions + the OPT offset of 2
POS_OFFSET = 2


@dataclass(frozen=True)
class Workload:
    name: str
    layers: int
    hidden: int
    heads: int
    ffn: int
    batch: int
    prompt: int
    gen: int                 # generated tokens (1 from prefill + gen-1 decode steps)
    micro_batch: int         # prefill micro-batch (rows of the batch per prefill call)
    full_model: bool = True  # False: lone decoder layer fed with N(0,1) activations
    vocab: int = VOCAB

    @property
    def head_dim(self) -> int:
        return self.hidden // self.heads

    @property
    def max_len(self) -> int:
        # the last decode step writes position prompt + gen - 2; full models also
        # keep one more slot so that the cache covers every generated token
        return self.prompt + self.gen - 1 if self.full_model else self.prompt + self.gen


WORKLOADS = {
    # one OPT-125m-shaped layer, batch 4, prompt 128, then 8 decode steps
    "opt125m-layer": Workload("opt125m-layer", 1, 768, 12, 3072, 4, 128, 8, 4, full_model=False),
    # OPT-1.3B shape, batch 32, prompt 512, 32 generated tokens
    "opt1.3b": Workload("opt1.3b", 24, 2048, 32, 8192, 32, 512, 32, 32),
    # OPT-30B shape, batch 144 = 3 x 48, prompt 512, 32 generated tokens
    "opt30b": Workload("opt30b", 48, 7168, 56, 28672, 144, 512, 32, 48),
    # OPT-175B shape, batch 144 = 3 x 48, prompt 512, 32 generated tokens
    "opt175b": Workload("opt175b", 96, 12288, 96, 49152, 144, 512, 32, 48),
}

# KV-compression stress: OPT-30B attention only, batch 64, prompt 2048, 64 decode steps
KV_STRESS = dict(batch=64, heads=56, head_dim=128, prompt=2048, steps=64,
                 outlier_frac=0.01, outlier_factor=8.0)
# standalone quantize of a 4 GiB fp16 tensor (2^31 elements)
QUANT_4GIB = dict(rows=524288, cols=4096)


def build_model(wl: Workload, seed: int = 0, device="cuda", log=None):
    """The OPT-shaped model of a full-model workload with synthetic weights (every
    tensor drawn on the device from its per-tensor seed, matrices and the embedding
    quantized there): the model the benchmark times and the full-size parity tests
    check.  log: None, or a function taking one status line."""
    import time

    import torch

    from group_wise_bit_flexq_amd import flexq as F
    from group_wise_bit_flexq_amd import synth
    h, f, nh = wl.hidden, wl.ffn, wl.heads
    layers = []
    t0 = time.time()
    for l in range(wl.layers):
        w16 = synth.layer_weights_fp16(h, f, seed, l, device=device)
        layers.append(F.QLayer.from_fp16(w16, nh, device))
        del w16
        if log and ((l + 1) % 16 == 0 or l + 1 == wl.layers):
            torch.cuda.synchronize()
            log(f"built layer {l + 1}/{wl.layers} ({time.time() - t0:.1f}s)")
    emb16 = synth.model_tensor("embed", (wl.vocab, h), seed, device)
    emb = F.quantize_weight(emb16)
    del emb16
    pos = synth.model_tensor("pos", (POS_ROWS, h), seed, device)
    lnf_g = synth.model_tensor("lnf_g", (h,), seed, device)
    lnf_b = synth.model_tensor("lnf_b", (h,), seed, device)
    model = F.QModel(layers, emb, pos, lnf_g, lnf_b, nh, wl.batch, wl.max_len,
                     wl.micro_batch * wl.prompt, device)
    torch.cuda.synchronize()
    if log:
        log(f"model ready: weights {model.weight_bytes() / 1e9:.1f} GB, KV4 "
            f"{sum(c.nbytes() for c in model.caches) / 1e9:.1f} GB, workspace "
            f"{model.workspace.numel() / 1e9:.1f} GB")
    return model
