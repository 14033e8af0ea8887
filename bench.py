"""Decode-attention benchmark on one MI355X.

One step = one decode step of every sequence through all layers: the host
allocator reserves one new slot per sequence and rebuilds the block tables,
they are uploaded, then per layer the new token's K/V are appended (quantized
for an INT8 cache) and the split-context decode runs, in one launch per layer
(pkv_decode_step; --unfused: pkv_append_kv + pkv_decode_attention). Inputs
are seeded synthetic tensors already resident in HBM; the cache is filled
before timing, to lengths at which the first timed step decodes at the
configured context.

Prints one JSON line: tokens/s (one new token per sequence per step), the
decode kernel's KV-read bandwidth against the 8 TB/s HBM peak, and the FP64
CPU oracle timed on a bounded sample of the same workload.

  python bench.py [--config qwen|llama29|llama128|mix16|mix32|long_i8|long_f16]
                  [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
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

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, GB/s

# rocprofv3 FETCH_SIZE + WRITE_SIZE summaries (scaled by a plain-copy reference)
# per workload; used only while the kernel sources they depend on still have
# the hash they record.
TRAFFIC_PROFILES = {"qwen": "profiles/decode_kernel_qwen3_tts_int8.md",
                    "llama29": "profiles/decode_kernel_llama2_7b_29x4096_fp16.md",
                    "llama128": "profiles/decode_kernel_llama2_7b_128x1024_fp16.md",
                    "mix16": "profiles/decode_kernel_mix_bs16_int8.md",
                    "long_i8": "profiles/decode_kernel_long_context_int8.md",
                    "prefill512": "profiles/prefill_kernel_qwen3_tts_chunk512_int8.md",
                    "prefill2k": "profiles/prefill_kernel_qwen3_tts_prompt2048_int8.md"}


# The kernel sources, and those each workload's launches are built from.
KERNEL_SOURCES = ("device.h", "append.hip", "decode.hip", "prefill.hip")
DECODE_SOURCES = ("device.h", "append.hip", "decode.hip")
PREFILL_SOURCES = ("device.h", "prefill.hip")


def workload_sources(config):
    return PREFILL_SOURCES if config.startswith("prefill") else DECODE_SOURCES


def code_hash(text):
    """sha256 of source text with comments and whitespace removed: it changes
    when the code does, not when its comments do."""
    import hashlib
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return hashlib.sha256(" ".join(text.split()).encode()).hexdigest()


def kernels_code_hash(sources=KERNEL_SOURCES):
    """code_hash of the given kernel sources (paged_kv_cache_62_amd/csrc),
    concatenated in that order."""
    return code_hash("\n".join(open(os.path.join(ROOT, "paged_kv_cache_62_amd", "csrc", name),
                                    encoding="utf-8").read() for name in sources))


def measured_traffic(config):
    """HBM bytes per launch from the committed counter summary, or None when
    there is none or the code of the kernels the workload runs changed since
    it was taken."""
    import re
    path = TRAFFIC_PROFILES.get(config)
    if path is None or not os.path.exists(os.path.join(ROOT, path)):
        return None
    text = open(os.path.join(ROOT, path), encoding="utf-8").read()
    t = re.search(r"traffic_bytes_per_launch: (\d+)", text)
    h = re.search(r"kernels_code_sha256: ([0-9a-f]{64})", text)
    if not t or not h or kernels_code_hash(workload_sources(config)) != h.group(1):
        return None
    return int(t.group(1))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (40; serving configs 400)")
    # The HIP runtime's first few dozen asynchronous uploads from pinned
    # memory include a handful that block the host for ~6 ms (measured on
    # MI355X with ROCm 7); 50 untimed steps leave them behind.
    ap.add_argument("--warmup", type=int, default=None, help="untimed steps first (50; serving configs 100)")
    ap.add_argument("--config", default="qwen")
    ap.add_argument("--partition", type=int, default=0, help="partition tokens (0 = automatic)")
    ap.add_argument("--piece-tokens", type=int, default=0,
                    help="prefill configs: context piece tokens, a multiple of 64 (0 = automatic)")
    ap.add_argument("--merge", choices=["auto", "fused", "separate"], default="auto",
                    help="where partitions are merged: automatic, last workgroup, or a second launch")
    ap.add_argument("--unfused", action="store_true",
                    help="append and decode as two launches per layer instead of one pkv_decode_step")
    ap.add_argument("--contraction", choices=["mfma", "valu"], default="mfma",
                    help="decode contractions on the matrix cores, or (with --unfused, for comparison) "
                         "as fp32 FMAs on the vector ALUs")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying a HIP graph")
    ap.add_argument("--kernel-reps", type=int, default=20, help="graph replays for the kernel timing")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only copy a MIB-sized device buffer 3 times (reference for HBM byte counters)")
    ap.add_argument("--calibrate-read", type=float, default=0.0, metavar="MIB",
                    help="only time pkv_stream_read of MIB-sized buffers (rotated past the 256 MB MALL) at "
                         "several grid sizes: the practical HBM read floor for a launch of that many bytes")
    ap.add_argument("--append-timing", action="store_true",
                    help="only time pkv_append_kv calls (prompts and a decode step's single tokens) into "
                         "INT8, seal-on-full INT8 and FP16 layers, bf16 input, 8 KV heads, d 128")
    ap.add_argument("--extra", default="auto",
                    help="comma-separated decode workloads also timed in this run and reported under "
                         "'extra_workloads' (no CPU baseline); 'auto' = llama29,llama128 after the default "
                         "qwen workload, 'none' = no others")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target oracle CPU time")
    return ap.parse_args()


CONFIGS = {
    # Qwen3-TTS talker: 28 layers, 8 KV / 16 query heads, d 128, bs 16, B=4 x 8000, INT8.
    "qwen": dict(layers=28, hq=16, hkv=8, dim=128, bs=16, nblocks=2048, B=4, ctx=8000, kv="i8",
                 q="bf16", kvin="bf16", sigma="per_head", seed=62002, outlier=0.0),
    # the same with FP16 first and last layers, INT8 in between ("轻量级推理引擎实战" §3.2)
    "qwen_mixed": dict(layers=28, hq=16, hkv=8, dim=128, bs=16, nblocks=2048, B=4, ctx=8000, kv="i8",
                       q="bf16", kvin="bf16", sigma="per_head", seed=62002, outlier=0.0, fp16_ends=True),
    # the same with lazy quantization: a sequence's partly filled last block stays FP16
    # and is quantized when full ("轻量级推理引擎实战" §三); append + decode launches
    "qwen_seal": dict(layers=28, hq=16, hkv=8, dim=128, bs=16, nblocks=2048, B=4, ctx=8000, kv="i8",
                      q="bf16", kvin="bf16", sigma="per_head", seed=62002, outlier=0.0, seal=True),
    # Llama-2-7B MHA, FP16 KV: 29 x 4096 (the A100 sizing case) and 128 x 1024.
    "llama29": dict(layers=32, hq=32, hkv=32, dim=128, bs=16, nblocks=8192, B=29, ctx=4096, kv="f16",
                    q="f16", kvin="f16", sigma="unit", seed=62003, outlier=0.0),
    "llama128": dict(layers=32, hq=32, hkv=32, dim=128, bs=16, nblocks=8192, B=128, ctx=1024, kv="f16",
                     q="f16", kvin="f16", sigma="unit", seed=62003, outlier=0.0),
    # continuous-batching mix: shared 200-token prefix + lognormal suffixes, INT8, GQA 32/8.
    "mix16": dict(layers=32, hq=32, hkv=8, dim=128, bs=16, nblocks=15000, B=128, ctx=None, kv="i8",
                  q="bf16", kvin="bf16", sigma="unit", seed=62004, outlier=0.0),
    "mix32": dict(layers=32, hq=32, hkv=8, dim=128, bs=32, nblocks=15000, B=128, ctx=None, kv="i8",
                  q="bf16", kvin="bf16", sigma="unit", seed=62004, outlier=0.0),
    # long context: 8 x 32768, bs 64, one layer timed over two rotating copies.
    "long_i8": dict(layers=2, hq=32, hkv=8, dim=128, bs=64, nblocks=None, B=8, ctx=32768, kv="i8",
                    q="bf16", kvin="bf16", sigma="unit", seed=62005, outlier=0.01, partition=512,
                    rotate=True),
    "long_f16": dict(layers=2, hq=32, hkv=8, dim=128, bs=64, nblocks=None, B=8, ctx=32768, kv="f16",
                     q="bf16", kvin="bf16", sigma="unit", seed=62005, outlier=0.01, partition=512,
                     rotate=True),
}

# Continuous-batching serving ("vLLM核心概念" §3.6 after tuning: max-num-seqs
# 128, max-model-len 1024, a ~200-token system prompt shared by every request,
# average generation 300 tokens; 15000 blocks as in its "used / total" log).
SERVE_CONFIGS = {
    "serve16": dict(layers=32, hq=32, hkv=8, dim=128, bs=16, nblocks=15000, max_batch=128,
                    max_model_len=1024, prefix=200, requests=1024, seed=62006),
    "serve32": dict(layers=32, hq=32, hkv=8, dim=128, bs=32, nblocks=15000, max_batch=128,
                    max_model_len=1024, prefix=200, requests=1024, seed=62006),
}

# Chunked prefill ("轻量级推理引擎实战" §一), Qwen3-TTS talker shape, INT8 KV:
# a 512-query chunk ending at context 8000, and whole 2048-token prompts.
PREFILL_CONFIGS = {
    "prefill512": dict(layers=28, hq=16, hkv=8, dim=128, bs=16, B=4, ctx=8000, chunk=512, seed=62007),
    "prefill2k": dict(layers=28, hq=16, hkv=8, dim=128, bs=16, B=4, ctx=2048, chunk=2048, seed=62008),
}

WORKLOAD_NAMES = {
    "prefill512": ("qwen3-tts-talker chunked prefill: 28 layers, B=4, the last 512 of 8000 cached tokens as "
                   "causal queries, 16q/8kv, d128, bs16, int8 kv"),
    "prefill2k": ("qwen3-tts-talker prefill: 28 layers, B=4 whole 2048-token prompts as causal queries, "
                  "16q/8kv, d128, bs16, int8 kv"),
    "serve16": ("continuous-batching serving: 32 layers, 32q/8kv, d128, bs16, int8 kv; 1024 queued requests, "
                "each a shared 200-token system prompt + lognormal(mean 300) suffix, ended by EOS after "
                "lognormal(mean 300) tokens or at max-model-len 1024; max batch 128; pkv_sched plans each step"),
    "serve32": ("continuous-batching serving: 32 layers, 32q/8kv, d128, bs32, int8 kv; 1024 queued requests, "
                "each a shared 200-token system prompt + lognormal(mean 300) suffix, ended by EOS after "
                "lognormal(mean 300) tokens or at max-model-len 1024; max batch 128; pkv_sched plans each step"),
    "qwen": "qwen3-tts-talker decode: 28 layers, B=4 x 8000 ctx, 16q/8kv, d128, bs16, int8 kv",
    "qwen_mixed": ("qwen3-tts-talker decode: 28 layers, B=4 x 8000 ctx, 16q/8kv, d128, bs16, fp16 kv in the "
                   "first and last layers, int8 kv in the other 26"),
    "qwen_seal": ("qwen3-tts-talker decode: 28 layers, B=4 x 8000 ctx, 16q/8kv, d128, bs16, int8 kv "
                  "quantized when a block fills (fp16 until then)"),
    "llama29": "llama-2-7b decode: 32 layers, B=29 x 4096 ctx, 32q/32kv, d128, bs16, fp16 kv",
    "llama128": "llama-2-7b decode: 32 layers, B=128 x 1024 ctx, 32q/32kv, d128, bs16, fp16 kv",
    "mix16": "continuous-batching mix: 32 layers, 128 seqs, shared 200-token prefix + lognormal suffix, 32q/8kv, bs16, int8 kv",
    "mix32": "continuous-batching mix: 32 layers, 128 seqs, shared 200-token prefix + lognormal suffix, 32q/8kv, bs32, int8 kv",
    "long_i8": "long-context: 1 layer (2 rotating copies), B=8 x 32768, 32q/8kv, d128, bs64, T=512, int8 kv",
    "long_f16": "long-context: 1 layer (2 rotating copies), B=8 x 32768, 32q/8kv, d128, bs64, T=512, fp16 kv",
}


def mix_suffix_lengths(seed, n):
    """round(X), X ~ lognormal(ln 300 - 0.32, 0.8) (mean 300), clamped to [1, 1024]."""
    from paged_kv_cache_62_amd import synth
    z = synth.normal(synth.stream_seed(seed, 4242), n)
    x = np.exp(math.log(300.0) - 0.32 + 0.8 * z)
    return np.clip(np.rint(x), 1, 1024).astype(np.int64)


class Workload:
    def __init__(self, name, steps_total, partition=0, flags=0, fused=True, warmup=0):
        import torch
        from paged_kv_cache_62_amd import pkv, synth
        self.torch, self.pkv = torch, pkv
        c = dict(CONFIGS[name])
        self.c, self.name = c, name
        self.dev = torch.device("cuda")
        self.B, self.L, self.hq, self.hkv, self.dim, self.bs = c["B"], c["layers"], c["hq"], c["hkv"], c["dim"], c["bs"]
        self.kv_code = pkv.PKV_I8 if c["kv"] == "i8" else pkv.PKV_F16
        self.rotate = c.get("rotate", False)
        self.partition = partition or c.get("partition", 0)
        self.flags = flags
        # one pkv_decode_step launch per decoded layer instead of append + decode
        self.fused = fused
        self.scale = 1.0 / math.sqrt(self.dim)
        tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}
        seed = c["seed"]
        # sequence lengths before the timed steps
        if c["ctx"] is None:  # mix: prefix 200 shared by all, then per-sequence suffixes
            self.suffix = mix_suffix_lengths(seed, self.B)
            lens0 = 200 + self.suffix
        else:
            # the first step after `warmup` appends decodes at ctx
            lens0 = np.full(self.B, c["ctx"] - 1 - warmup, dtype=np.int64)
        appends = steps_total  # host_prep() calls: one new slot per sequence each (shared by all layers)
        need = int(sum((int(n) + appends + self.bs - 1) // self.bs for n in lens0)) + 8
        nblocks = c["nblocks"] if c["nblocks"] is not None else need
        if need > nblocks:
            nblocks = need  # headroom for the blocks the timed steps append
        self.nblocks = nblocks
        order = synth.permutation(synth.stream_seed(seed, 1), nblocks)
        # per-layer element types: FP16 for the first and last layers when the
        # configuration asks for it ("轻量级推理引擎实战" §3.2)
        self.layer_kv = ([pkv.PKV_F16] + [self.kv_code] * (self.L - 2) + [pkv.PKV_F16]
                         if c.get("fp16_ends") else [self.kv_code] * self.L)
        self.pool = pkv.Pool(self.L, self.hkv, self.dim, self.bs, nblocks, self.kv_code,
                             layer_kv_dtypes=self.layer_kv if c.get("fp16_ends") else None,
                             seal_on_full=bool(c.get("seal")),
                             initial_free_order=order)
        self.seqs = np.arange(self.B, dtype=np.int64)
        gen = torch.Generator(device=self.dev)
        gen.manual_seed(seed)
        u = synth.uniform(synth.stream_seed(seed, 7777), self.L * 2 * self.hkv)
        sig = (0.5 + 3.5 * u).reshape(self.L, 2, self.hkv) if c["sigma"] == "per_head" else np.ones((self.L, 2, self.hkv))
        self.sig = torch.tensor(sig, dtype=torch.float32, device=self.dev)

        def kv_fill(layer, n):
            out = []
            for kv in range(2):
                x = torch.randn(n, self.hkv, self.dim, generator=gen, device=self.dev)
                x *= self.sig[layer, kv][None, :, None]
                if c["outlier"] > 0:
                    m = torch.rand(x.shape, generator=gen, device=self.dev) < c["outlier"]
                    sgn = torch.where(torch.rand(x.shape, generator=gen, device=self.dev) < 0.5, -20.0, 20.0)
                    x = torch.where(m, sgn, x)
                out.append(x.to(tdt[c["kvin"]]).contiguous())
            return out

        # fill the cache
        if c["ctx"] is None:
            slots = self.pool.allocate(0, 200)
            self._append_all(kv_fill, slots)
            for s in range(1, self.B):
                self.pool.fork(0, s)
            slots = self.pool.append_slots(self.seqs, self.suffix.astype(np.int32))
            self._append_all(kv_fill, slots)
        else:
            for s in range(self.B):
                slots = self.pool.allocate(s, int(lens0[s]))
                self._append_all(kv_fill, slots)
        torch.cuda.synchronize()
        # the batch in pkv_seq_order_longest_first's order (longest context
        # first; equal lengths keep their order): with one partition per
        # sequence each compute unit then gets sequences from every part of
        # the length range
        self.seqs = self.pool.order_longest_first(self.seqs)
        # per-step inputs: one query and one new K/V row per sequence and layer
        self.q = [torch.randn(self.B, self.hq, self.dim, generator=gen, device=self.dev).to(tdt[c["q"]])
                  for _ in range(self.L)]
        self.knew, self.vnew = [], []
        for layer in range(self.L):
            k, v = kv_fill(layer, self.B)
            self.knew.append(k)
            self.vnew.append(v)
        self.max_blocks = max((int(n) + appends + self.bs - 1) // self.bs for n in lens0) + 1
        self.out = torch.empty(self.B, self.hq, self.dim, dtype=torch.float32, device=self.dev)
        self.max_ctx = max_ctx = int(lens0.max()) + appends
        ws = self.pool.workspace_bytes(self.B, self.hq, max_ctx, self.partition)
        self.ws = torch.zeros(max(ws, 256), dtype=torch.uint8, device=self.dev)
        # Per-step uploads: slots int64[B], lengths int32[B] and the block
        # table int32[B][max_blocks], packed in one buffer so a step makes one
        # host-to-device copy; a ring of pinned staging buffers lets the host
        # prepare the next steps while earlier uploads are in flight.
        self.up_bytes = 8 * self.B + 4 * self.B + 4 * self.B * self.max_blocks

        def views(buf):
            B, mb = self.B, self.max_blocks
            return (buf[: 8 * B].view(torch.int64), buf[8 * B: 12 * B].view(torch.int32),
                    buf[12 * B: 12 * B + 4 * B * mb].view(torch.int32).view(B, mb))
        self.ring = []
        for _ in range(4):
            buf = torch.empty(self.up_bytes, dtype=torch.uint8, pin_memory=True)
            sl, ln, tb = views(buf)
            self.ring.append(dict(buf=buf, slots=sl.numpy(), lens=ln.numpy(), table=tb.numpy(),
                                  ev=torch.cuda.Event()))
        self.d_up = torch.empty(self.up_bytes, dtype=torch.uint8, device=self.dev)
        self.d_slots, self.d_lens, self.d_table = views(self.d_up)
        self.ones = np.ones(self.B, dtype=np.int32)
        self.step_i = 0

    def _append_all(self, kv_fill, slots):
        t = self.torch
        d_slots = t.from_numpy(np.ascontiguousarray(slots)).to(self.dev)
        chunk = 65536
        for layer in range(self.L):
            for i in range(0, len(slots), chunk):
                k, v = kv_fill(layer, min(chunk, len(slots) - i))
                self.pool.append_kv(layer, k, v, d_slots[i:i + chunk])

    def kv_read_bytes(self, lens, layer=0):
        """Algorithmic bytes one decode launch reads: K and V payload of the
        valid tokens plus one fp32 scale per (block, head, K|V) for INT8."""
        elem = 1 if self.layer_kv[layer] == self.pkv.PKV_I8 else 2
        if elem == 1 and self.c.get("seal"):  # full blocks INT8 + scales, partly filled ones FP16
            lens = np.asarray(lens, dtype=np.int64)
            full = lens // self.bs
            return int((full * self.bs).sum() * self.hkv * self.dim * 2 + full.sum() * self.hkv * 2 * 4 +
                       (lens - full * self.bs).sum() * self.hkv * self.dim * 2 * 2)
        b = int(lens.sum()) * self.hkv * self.dim * 2 * elem
        if elem == 1:
            b += int(sum((int(n) + self.bs - 1) // self.bs for n in lens)) * self.hkv * 2 * 4
        return b

    def host_prep(self):
        """Host side of a step: one new slot per sequence from the allocator
        and the block tables rebuilt, written into a pinned staging buffer
        and uploaded with one copy."""
        slot = self.ring[self.step_i % len(self.ring)]
        slot["ev"].synchronize()  # the upload that last used this staging buffer is done
        self.pool.append_slots(self.seqs, self.ones, out=slot["slots"])
        self.pool.block_table(self.seqs, self.max_blocks, table=slot["table"], lens=slot["lens"])
        self.d_up.copy_(slot["buf"], non_blocking=True)
        slot["ev"].record()
        self.step_i += 1
        return slot["lens"].copy()

    def device_step(self, layers=None, decode_only=False):
        """Device side of a step: per layer, the new tokens' K/V are appended
        and the layer decoded, in one pkv_decode_step launch (fused) or as
        pkv_append_kv + pkv_decode_attention. decode_only keeps just the
        launches that decode (the fused ones include their append).
        max_context_len is the capacity for the whole run, so the launch
        shapes never change (the kernels read the true lengths)."""
        dec = set(range(self.L) if layers is None else layers)
        for layer in range(self.L):  # every layer receives the new token
            if layer in dec and self.fused:
                self.pool.decode_step(layer, self.q[layer], self.knew[layer], self.vnew[layer], self.d_table,
                                      self.d_lens, self.max_ctx, self.scale, out=self.out, workspace=self.ws,
                                      partition_tokens=self.partition, flags=self.flags)
                continue
            if not decode_only:
                self.pool.append_kv(layer, self.knew[layer], self.vnew[layer], self.d_slots)
            if layer in dec:
                self.pool.decode(layer, self.q[layer], self.d_table, self.d_lens, self.max_ctx,
                                 self.scale, out=self.out, workspace=self.ws,
                                 partition_tokens=self.partition, flags=self.flags)

    def decode_layers(self, step_i):
        """Layers decoded in a step (one rotating copy for the long-context runs)."""
        return range(self.L) if not self.rotate else [step_i % self.L]


def cpu_model() -> str:
    """The host CPU's model name from /proc/cpuinfo (empty if unavailable)."""
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


def cpu_baseline(w: Workload, target_s: float):
    """The FP64 oracle on a bounded sample: layers in order until ~target_s of
    CPU time, over the GPU's cache read back after the timed steps."""
    from oracle import oracle as orc
    from paged_kv_cache_62_amd import synth
    table, lens = w.pool.block_table(w.seqs, w.max_blocks)
    blocks = sorted({int(b) for i in range(w.B) for b in table[i, : (int(lens[i]) + w.bs - 1) // w.bs]})
    threads = max(1, min(16, os.cpu_count() or 1))
    done, elapsed = 0, 0.0
    layers = range(w.L) if not w.rotate else [0]
    last = None
    for layer in layers:
        kvd = orc.I8 if w.pool.layer_kv_dtypes[layer] == w.pkv.PKV_I8 else orc.F16
        dt = np.int8 if kvd == orc.I8 else np.uint16
        codes, scales = w.pool.read_blocks(layer, blocks)
        kc = np.zeros((w.nblocks, w.hkv, w.bs, w.dim), dtype=dt)
        vc = np.zeros_like(kc)
        ks = np.ones((w.nblocks, w.hkv), np.float32)
        vs = np.ones_like(ks)
        kc[blocks], vc[blocks] = codes[:, 0], codes[:, 1]
        if kvd == orc.I8:
            ks[blocks], vs[blocks] = scales[:, 0], scales[:, 1]
        del codes
        q = synth.as_f32(w.q[layer].cpu())
        t0 = time.perf_counter()
        orc.decode_attention(kvd, kc, vc, ks, vs, q, table, lens, w.scale, threads=threads)
        elapsed += time.perf_counter() - t0
        done += 1
        last = (kvd, kc, vc, ks, vs, q)
        if elapsed >= target_s:
            break
    t_layer = elapsed / done
    layers_per_step = 1 if w.rotate else w.L
    value = w.B / (t_layer * layers_per_step)
    # the same oracle on one thread, the last sampled layer once
    t0 = time.perf_counter()
    orc.decode_attention(*last[:6], table, lens, w.scale, threads=1)
    t_one = time.perf_counter() - t0
    return {"value": value, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "value_1thread": w.B / (t_one * layers_per_step), "cpu_model": cpu_model(),
            "sample": (f"FP64 oracle decode of {done} of {layers_per_step} layer(s) per step "
                       f"({t_layer * 1e3:.1f} ms per layer, {threads} threads) over the GPU cache "
                       f"read back after the timed steps; tokens/s = B / (layers x time per layer), "
                       f"extrapolated from the sampled layers")}


def main():
    args = parse()
    serve = args.config in SERVE_CONFIGS
    prefill = args.config in PREFILL_CONFIGS
    if args.steps is None:
        args.steps = 400 if serve else 10 if prefill else 40
    if args.warmup is None:
        args.warmup = 100 if serve else 2 if prefill else 50
    if args.gpus != 1:
        print(json.dumps({"error": "this library runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)
    known = sorted(CONFIGS) + sorted(SERVE_CONFIGS) + sorted(PREFILL_CONFIGS)
    if args.config not in known:
        sys.exit(f"unknown --config {args.config}; choose from {known}")
    import torch
    from paged_kv_cache_62_amd import pkv
    pkv.lib()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.calibrate_copy:
        # A plain device copy of known size: reads and writes exactly
        # calibrate_copy MiB per launch, for scaling FETCH_SIZE / WRITE_SIZE.
        n = args.calibrate_copy << 20
        x = torch.ones(n, dtype=torch.uint8, device="cuda")
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n}), flush=True)
        return
    if args.calibrate_read:
        print(json.dumps(calibrate_read(args.calibrate_read)), flush=True)
        return
    if args.append_timing:
        print(json.dumps(append_timing()), flush=True)
        return
    stream = torch.cuda.Stream()  # graphs are captured on (and replayed to) a side stream
    with torch.cuda.stream(stream):
        res = (run_serve if args.config in SERVE_CONFIGS else
               run_prefill if args.config in PREFILL_CONFIGS else run)(args, stream)
    if not args.no_cpu_baseline:
        print("# cpu baseline (oracle)", file=sys.stderr, flush=True)
        base = prefill_cpu_baseline if args.config in PREFILL_CONFIGS else cpu_baseline
        res["cpu_baseline"] = base(res.pop("_workload"), args.cpu_seconds)
    else:
        res.pop("_workload")
    extra = extra_workloads(args)
    if extra:
        res["extra_workloads"] = {}
        for name in extra:
            # the previous workload's pool is released before the next is built
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
            sub = argparse.Namespace(**{**vars(args), "config": name, "partition": 0})
            with torch.cuda.stream(stream):
                r = run(sub, stream)
            r.pop("_workload")
            res["extra_workloads"][name] = {k: r[k] for k in ("value", "unit", "ms_per_step", "steps", "warmup",
                                                              "dtype", "config", "roofline")}
            print(f"# {name}: {r['value']:.1f} tokens/s, frac {r['roofline']['frac']:.3f}",
                  file=sys.stderr, flush=True)
            del r
    print(json.dumps(res), flush=True)


def append_timing():
    """pkv_append_kv on its own: for each layer kind, block size and call shape
    (tokens per sequence x sequences, each sequence allocated to that length
    and written again every call), 20 calls captured in a HIP graph and
    replayed between two events; per call time. bf16 K/V, 8 KV heads, d 128."""
    import torch
    from paged_kv_cache_62_amd import pkv
    kinds = [("int8", pkv.PKV_I8, False), ("int8_seal", pkv.PKV_I8, True), ("fp16", pkv.PKV_F16, False)]
    shapes = [(4096, 1), (500, 8), (512, 4), (300, 16), (64, 16), (1, 4), (1, 32), (1, 128), (1, 512)]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(62062)
    stream = torch.cuda.Stream()
    rows = []
    for name, kvd, seal in kinds:
        for bs in (16, 32, 64):
            for n, seqs in shapes:
                pool = pkv.Pool(1, 8, 128, bs, 8192, kvd, seal_on_full=seal)
                slots = np.concatenate([pool.allocate(s, n) for s in range(seqs)])
                sl = torch.from_numpy(np.ascontiguousarray(slots)).to("cuda")
                k = torch.randn(n * seqs, 8, 128, generator=gen, device="cuda").to(torch.bfloat16)
                v = torch.randn(n * seqs, 8, 128, generator=gen, device="cuda").to(torch.bfloat16)
                calls = 20
                g = torch.cuda.CUDAGraph()
                with torch.cuda.stream(stream):
                    pool.append_kv(0, k, v, sl, stream)
                    with torch.cuda.graph(g, stream=stream):
                        for _ in range(calls):
                            pool.append_kv(0, k, v, sl, stream)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                with torch.cuda.stream(stream):
                    g.replay()
                    torch.cuda.synchronize()
                    e0.record(stream)
                    for _ in range(5):
                        g.replay()
                    e1.record(stream)
                torch.cuda.synchronize()
                rows.append({"layer": name, "block_size": bs, "tokens_per_seq": n, "seqs": seqs,
                             "avg_call_us": e0.elapsed_time(e1) * 1e3 / (5 * calls)})
                del g
                pool.close()
    return {"append_timing": rows,
            "timing": "HIP events around graph replays of 20 pkv_append_kv calls; bf16 K/V, 8 KV heads, d 128"}


def calibrate_read(mib):
    """pkv_stream_read of buffers of `mib` MiB, enough of them (>= 1 GiB in all)
    that the 256 MB MALL holds none between its reads, one launch per buffer
    in a HIP graph replayed back to back between two events; per launch time
    and rate for 256 to 4096 workgroups."""
    import torch
    from paged_kv_cache_62_amd import pkv
    nbytes = int(round(mib * (1 << 20) / 16)) * 16
    nbuf = max(2, -(-(1 << 30) // nbytes))
    bufs = [torch.full((nbytes,), i, dtype=torch.uint8, device="cuda") for i in range(nbuf)]
    sink = torch.empty(4096 * 256, dtype=torch.int32, device="cuda")
    stream = torch.cuda.Stream()
    rows = []
    for wg in (256, 512, 1024, 2048, 4096):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            for b in bufs:  # once eagerly (first-touch), then captured
                pkv.pkv_stream_read(b, wg, sink, stream)
            with torch.cuda.graph(g, stream=stream):
                for b in bufs:
                    pkv.pkv_stream_read(b, wg, sink, stream)
        reps = max(3, int(2e9 // (nbytes * nbuf)))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):  # replays go to the current stream: the events' stream
            g.replay()
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(reps):
                g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (reps * nbuf)
        rows.append({"workgroups": wg, "avg_launch_us": us, "GBps": nbytes / us / 1e3,
                     "frac": nbytes / us / 1e3 / HBM_PEAK_GBS})
    best = min(rows, key=lambda r: r["avg_launch_us"])
    return {"calibrate_read_bytes": nbytes, "buffers": nbuf, "rows": rows, "best": best,
            "timing": "HIP events around graph replays of one pkv_stream_read per buffer"}


def extra_workloads(args):
    """Decode workloads timed after the main one in the same run: by default
    the two Llama-2-7B shapes ("vLLM核心概念" §3.1 and §3.5) after the default
    Qwen3-TTS-talker workload, so one run measures both shapes the target names."""
    if args.extra == "none":
        return []
    if args.extra == "auto":
        return ["llama29", "llama128"] if args.config == "qwen" else []
    names = [x for x in args.extra.split(",") if x]
    bad = [x for x in names if x not in CONFIGS]
    if bad:
        sys.exit(f"--extra: unknown decode workloads {bad}; choose from {sorted(CONFIGS)}")
    return names


def run(args, stream):
    import torch
    from paged_kv_cache_62_amd import pkv
    print(f"# building workload {args.config}", file=sys.stderr, flush=True)
    merge_flags = {"auto": 0, "fused": pkv.PKV_DECODE_FUSED_MERGE, "separate": pkv.PKV_DECODE_SEPARATE_MERGE}
    if args.contraction == "valu" and not args.unfused:
        sys.exit("--contraction valu times pkv_decode_attention: add --unfused")
    valu_flag = pkv.PKV_DECODE_VALU_CONTRACTION if args.contraction == "valu" else 0
    # Every host_prep() appends one token per sequence: the one before graph
    # capture, the warm-up steps and the timed steps. The workload sizes its
    # lengths and max_context_len for exactly that many, so the first timed
    # step decodes at the configured context and no step exceeds the capacity.
    pre = args.warmup + (0 if args.no_graph else 1)
    w = Workload(args.config, pre + args.steps, args.partition, flags=merge_flags[args.merge] | valu_flag,
                 fused=not args.unfused, warmup=pre)
    graphs = {}
    if not args.no_graph:
        # The device work of a step, captured once as a HIP graph per layer
        # set (all layers, or each rotating copy) and replayed every step.
        w.host_prep()
        for key in sorted({tuple(w.decode_layers(i)) for i in range(max(2, w.L))}):
            w.device_step(key)  # eager once before capture
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                w.device_step(key)
            graphs[key] = g
        torch.cuda.synchronize()

    def run_step():
        i = w.step_i
        lens = w.host_prep()
        if int(lens.max()) > w.max_ctx:  # the decode calls' contract: len <= max_context_len
            raise RuntimeError(f"step {i}: length {int(lens.max())} exceeds max_context_len {w.max_ctx}")
        key = tuple(w.decode_layers(i))
        if graphs:
            graphs[key].replay()
        else:
            w.device_step(key)
        return lens

    for _ in range(args.warmup):
        run_step()
    torch.cuda.synchronize()
    print(f"# warmup done; timing {args.steps} steps", file=sys.stderr, flush=True)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    step_bytes = []
    start.record()
    tokens = 0
    for _ in range(args.steps):
        lens = run_step()
        step_bytes.append(sum(w.kv_read_bytes(lens, l) for l in w.decode_layers(w.step_i - 1)))
        tokens += w.B
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps

    # The decode kernel alone: a graph of the step's decode launches on the
    # same stream, replayed back to back between two events; the cache is in
    # its final state, so each launch reads the current lengths. A fused
    # launch also re-stores the last token, which leaves the cache unchanged
    # (the same rows at the same slots give the same codes and scales).
    layers = list(w.decode_layers(0))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        w.device_step(layers, decode_only=True)
    g.replay()
    torch.cuda.synchronize()
    reps = max(5, int(args.kernel_reps))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    avg_dur_s = e0.elapsed_time(e1) / 1e3 / (reps * len(layers))
    # H1 alone: the step's appends as pkv_append_kv launches (one per decoded
    # layer), timed the same way; storing the last tokens again leaves the
    # cache unchanged.
    ga = torch.cuda.CUDAGraph()
    with torch.cuda.graph(ga, stream=stream):
        for layer in layers:
            w.pool.append_kv(layer, w.knew[layer], w.vnew[layer], w.d_slots)
    ga.replay()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        ga.replay()
    e1.record()
    torch.cuda.synchronize()
    append_us = e0.elapsed_time(e1) * 1e3 / (reps * len(layers))
    _, lens_now = w.pool.block_table(w.seqs, w.max_blocks)
    bytes_launch = float(np.mean([w.kv_read_bytes(lens_now, l) for l in layers]))  # per launch, averaged
    achieved = bytes_launch / avg_dur_s / 1e9
    kv_gbs_step = float(np.sum(step_bytes)) / (total_ms / 1e3) / 1e9
    plan = w.pool.decode_plan(w.B, w.max_ctx, w.partition, w.flags)
    # what a launch moves besides the K/V it reads: q, the fp32 output, the
    # table entries and lengths it reads, the partition partials (written,
    # then read by the merge) and, for a decode step, the new K/V rows read
    qbytes = w.q[layers[0]].element_size()
    used_blocks = int(sum((int(n) + w.bs - 1) // w.bs for n in lens_now))
    nparts = sum((int(n) + plan[0] - 1) // plan[0] for n in lens_now)
    other_bytes = (w.B * w.hq * w.dim * (qbytes + 4) + 4 * used_blocks + 4 * w.B +
                   (2 * nparts * w.hq * (w.dim + 2) * 4 if plan[1] > 1 else 0) +
                   (2 * w.B * w.hkv * w.dim * qbytes if w.fused else 0))
    res = {
        "metric": "decode attn tokens/sec and KV-read HBM GB/s (% of MI355X peak), 1 GPU",
        "value": tokens / (total_ms / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("int8 kv (fp16 first and last layers) / fp32 accumulate" if w.c.get("fp16_ends") else
                  "int8 kv quantized when a block fills (fp16 partly filled blocks) / fp32 accumulate"
                  if w.c.get("seal") else
                  "int8 kv / fp32 accumulate" if w.kv_code == pkv.PKV_I8 else "fp16 kv / fp32 accumulate"),
        "data": "synthetic (seeded), cache filled through pkv_append_kv before timing",
        "config": {"workload": WORKLOAD_NAMES[args.config], "batch": w.B,
                   "layers_per_step": len(layers),
                   "partition_tokens": plan[0], "partitions": plan[1],
                   "merge": "none (one partition)" if plan[1] == 1 else
                            "last workgroup" if plan[2] else "separate launch",
                   "hip_graph": not args.no_graph,
                   "batch_order": "longest context first",
                   "contraction": "vector ALU (comparison)" if valu_flag else "matrix cores",
                   "launches_per_layer": 1 if w.fused else 2,
                   "kv_read_GBps_whole_step": kv_gbs_step,
                   "append_kernel_us": append_us},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic(args.config) if w.fused and not valu_flag else None,
                     "kernel": ("decode_kernel, decode step (new token's append + split-context decode + merge)"
                                if w.fused else "decode_kernel_valu (vector-ALU contractions; "
                                "split-context decode incl. partition merge)" if valu_flag else
                                "decode_kernel (split-context decode incl. partition merge)"),
                     "avg_launch_us": avg_dur_s * 1e6, "bytes_per_launch": bytes_launch,
                     "other_bytes_per_launch": other_bytes,
                     "timing": f"HIP events around {reps} replays of a graph of the {len(layers)} decode launches"},
    }
    res["_workload"] = w
    return res

class _ServeView:
    """What cpu_baseline reads, for the serving loop's last batch."""

    def __init__(self, pool, seqs, max_blocks, c, q, scale):
        import paged_kv_cache_62_amd.pkv as pkv
        self.pkv, self.pool, self.seqs = pkv, pool, seqs
        self.B, self.L, self.bs, self.max_blocks = len(seqs), c["layers"], c["bs"], max_blocks
        self.nblocks, self.hkv, self.dim = c["nblocks"], c["hkv"], c["dim"]
        self.kv_code, self.rotate, self.scale = pkv.PKV_I8, False, scale
        self.q = [q[: len(seqs)]] * self.L


class ServeWorkload:
    """The serving workload SERVE_CONFIGS[name]: all requests queued at the
    start behind a resident shared system prompt; pkv_sched plans every step
    (admissions, block tables, copy-on-write of the shared prompt's partly
    filled block); admitted prompts' K/V are written with pkv_append_kv and
    the batch runs pkv_decode_step per layer; a request ends with EOS after
    its drawn generation length."""

    def __init__(self, name, stream):
        import torch
        from paged_kv_cache_62_amd import pkv, synth
        self.torch = torch
        c = self.c = SERVE_CONFIGS[name]
        self.L, self.hq, self.hkv, self.dim, self.bs = L, hq, hkv, dim, bs = (
            c["layers"], c["hq"], c["hkv"], c["dim"], c["bs"])
        seed, R, self.mb, self.mml = c["seed"], c["requests"], c["max_batch"], c["max_model_len"]
        mb, mml = self.mb, self.mml
        self.stream = stream
        dev = self.dev = torch.device("cuda")
        self.scale = 1.0 / math.sqrt(dim)
        self.nblocks = c["nblocks"]
        order = synth.permutation(synth.stream_seed(seed, 1), c["nblocks"])
        pool = self.pool = pkv.Pool(L, hkv, dim, bs, c["nblocks"], pkv.PKV_I8, initial_free_order=order)
        gen = torch.Generator(device=dev)
        gen.manual_seed(seed)
        # K/V rows written at admission and per decoded token (the values do not
        # change the work; every write still quantizes and stores)
        self.src_rows = 131072
        self.ksrc = torch.randn(self.src_rows, hkv, dim, generator=gen, device=dev).to(torch.bfloat16)
        self.vsrc = torch.randn(self.src_rows, hkv, dim, generator=gen, device=dev).to(torch.bfloat16)
        self.q = torch.randn(mb, hq, dim, generator=gen, device=dev).to(torch.bfloat16)
        self.knew = torch.randn(mb, hkv, dim, generator=gen, device=dev).to(torch.bfloat16)
        self.vnew = torch.randn(mb, hkv, dim, generator=gen, device=dev).to(torch.bfloat16)
        self.prefix_seq = 1 << 40
        slots = pool.allocate(self.prefix_seq, c["prefix"])
        d = torch.from_numpy(slots).to(dev)
        for layer in range(L):
            pool.append_kv(layer, self.ksrc[: len(slots)], self.vsrc[: len(slots)], d)
        self.sched = pkv.Scheduler(pool, mb, mml, reserve_blocks=1, batch_order=pkv.PKV_BATCH_LONGEST_FIRST)
        suffix = np.minimum(mix_suffix_lengths(seed, R), mml - c["prefix"] - 1)
        z = synth.normal(synth.stream_seed(seed, 4343), R)
        self.eos_at = np.maximum(np.rint(np.exp(math.log(300.0) - 0.32 + 0.8 * z)), 1).astype(np.int64)
        for r in range(R):
            self.sched.submit(r, int(c["prefix"] + suffix[r]), mml, self.prefix_seq)
        self.made = np.zeros(R, dtype=np.int64)
        self.maxb = (mml + bs - 1) // bs
        self.d_table = torch.empty(mb * self.maxb, dtype=torch.int32, device=dev)
        self.d_lens = torch.empty(mb, dtype=torch.int32, device=dev)
        self.d_pslots = torch.empty(self.src_rows, dtype=torch.int64, device=dev)
        self.ws = torch.zeros(256, dtype=torch.uint8, device=dev)
        self.out = torch.empty(mb, hq, dim, dtype=torch.float32, device=dev)
        self.counts = dict(generated=0, prefill=0, steps=0)
        self.eos = []
        self.last = {}

    def plan(self):
        """Host side of a step: the scheduler's plan (its copy-on-write copies
        are queued on the stream), uploaded."""
        torch = self.torch
        p = self.sched.step(self.eos, self.stream)
        n, npf = len(p["seqs"]), int(p["prefill_slots"].size)
        if npf:
            assert npf <= self.src_rows
            self.d_pslots[:npf].copy_(torch.from_numpy(p["prefill_slots"]), non_blocking=True)
        if n:
            self.d_table[: n * self.maxb].copy_(torch.from_numpy(p["block_tables"].reshape(-1)), non_blocking=True)
            self.d_lens[:n].copy_(torch.from_numpy(p["context_lens"]), non_blocking=True)
            need = self.pool.workspace_bytes(n, self.hq, p["max_context_len"])
            if need > self.ws.numel():
                self.ws = torch.zeros(need, dtype=torch.uint8, device=self.dev)
        return p

    def table(self, n):
        return self.d_table[: n * self.maxb].view(n, self.maxb)

    def launch(self, p):
        """Device side of a step: admitted prompts' K/V, then per layer the
        batch's decode step; EOS for the requests that reached their length."""
        n, npf = len(p["seqs"]), int(p["prefill_slots"].size)
        for layer in range(self.L):
            if npf:
                self.pool.append_kv(layer, self.ksrc[:npf], self.vsrc[:npf], self.d_pslots[:npf], self.stream)
            if n:
                self.pool.decode_step(layer, self.q[:n], self.knew[:n], self.vnew[:n], self.table(n),
                                      self.d_lens[:n], p["max_context_len"], self.scale, out=self.out[:n],
                                      workspace=self.ws, stream=self.stream)
        ids = p["seqs"]
        self.made[ids] += 1
        self.eos = [int(r) for r in ids[self.made[ids] >= self.eos_at[ids]]]
        self.counts["generated"] += n
        self.counts["prefill"] += npf
        self.counts["steps"] += 1
        self.last.update(p)

    def step(self):
        self.launch(self.plan())


def run_serve(args, stream):
    """The serving loop of ServeWorkload: W untimed steps fill the batch,
    then K steps are timed."""
    import torch
    print(f"# building serving workload {args.config}", file=sys.stderr, flush=True)
    w = ServeWorkload(args.config, stream)
    c, L, hq, hkv, dim, bs = w.c, w.L, w.hq, w.hkv, w.dim, w.bs
    pool, sched, q, knew, vnew, scale, out = w.pool, w.sched, w.q, w.knew, w.vnew, w.scale, w.out
    maxb, counts, last = w.maxb, w.counts, w.last
    one_step = w.step

    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    print(f"# warmup done; timing {args.steps} steps", file=sys.stderr, flush=True)
    st0 = sched.stats()
    counts.update(generated=0, prefill=0, steps=0)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        one_step()
    e1.record(stream)
    torch.cuda.synchronize()
    total_ms = e0.elapsed_time(e1)
    st1 = sched.stats()

    # the decode-step kernel alone, over the last batch (graph of its L launches)
    n, mctx = len(last["seqs"]), last["max_context_len"]
    tab = w.table(n)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for layer in range(L):
            pool.decode_step(layer, q[:n], knew[:n], vnew[:n], tab, w.d_lens[:n], mctx, scale, out=out[:n],
                             workspace=w.ws, stream=stream)
    g.replay()
    torch.cuda.synchronize()
    reps = max(5, int(args.kernel_reps))
    k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    k0.record(stream)
    for _ in range(reps):
        g.replay()
    k1.record(stream)
    torch.cuda.synchronize()
    avg_dur_s = k0.elapsed_time(k1) / 1e3 / (reps * L)
    lens = last["context_lens"].astype(np.int64)
    bytes_launch = float(lens.sum() * hkv * dim * 2 + ((lens + bs - 1) // bs).sum() * hkv * 2 * 4)
    achieved = bytes_launch / avg_dur_s / 1e9
    plan = pool.decode_plan(n, mctx, 0, 0)
    res = {
        "metric": "decode attn tokens/sec and KV-read HBM GB/s (% of MI355X peak), 1 GPU",
        "value": counts["generated"] / (total_ms / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": total_ms / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8 kv / fp32 accumulate",
        "data": "synthetic (seeded request lengths and K/V), queued before timing",
        "config": {
            "workload": WORKLOAD_NAMES[args.config],
            "avg_batch": counts["generated"] / args.steps,
            "prefill_tokens_per_s": counts["prefill"] / (total_ms / 1e3),
            "admitted": st1["admitted"] - st0["admitted"],
            "finished_eos": st1["finished_eos"] - st0["finished_eos"],
            "finished_max_length": st1["finished_max_length"] - st0["finished_max_length"],
            "preempted": st1["preempted"] - st0["preempted"],
            "kv_cache_blocks": f"{st1['used_blocks']} used / {st1['total_blocks']} total",
            "waiting": st1["waiting"],
            "last_batch": {"seqs": n, "max_context_len": mctx, "partition_tokens": plan[0],
                           "partitions": plan[1]},
            "launches_per_layer": "pkv_decode_step, plus pkv_append_kv on steps that admit",
            "batch_order": "longest context first (scheduler option)",
        },
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "decode_kernel, decode step over the last batch",
                     "avg_launch_us": avg_dur_s * 1e6, "bytes_per_launch": bytes_launch,
                     "timing": f"HIP events around {reps} replays of a graph of the {L} decode launches"},
    }
    res["_workload"] = _ServeView(pool, [int(x) for x in last["seqs"]], maxb, c, q, scale)
    res["_workload"].sched = sched  # its requests hold the blocks the baseline reads
    return res


MFMA_FP16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 matrix-core peak


class PrefillWorkload:
    """The chunked-prefill workload PREFILL_CONFIGS[name]: B sequences of ctx
    cached tokens (seeded bf16 K/V appended through pkv_append_kv, every layer)
    and, per layer, queries for the last `chunk` tokens of each sequence.
    `prefill(layer)` is the launch a benchmark step makes per layer."""

    def __init__(self, name, stream=None, piece_tokens=0):
        import torch
        from paged_kv_cache_62_amd import pkv, synth
        c = self.c = PREFILL_CONFIGS[name]
        L, hq, hkv, dim, bs, B, ctx, C = (c[k] for k in ("layers", "hq", "hkv", "dim", "bs", "B", "ctx", "chunk"))
        self.L, self.hq, self.hkv, self.dim, self.bs, self.B, self.ctx, self.C = L, hq, hkv, dim, bs, B, ctx, C
        dev = torch.device("cuda")
        self.stream = stream
        self.scale = 1.0 / math.sqrt(dim)
        self.nblocks = B * ((ctx + bs - 1) // bs) + 8
        order = synth.permutation(synth.stream_seed(c["seed"], 1), self.nblocks)
        self.pool = pkv.Pool(L, hkv, dim, bs, self.nblocks, pkv.PKV_I8, initial_free_order=order)
        gen = torch.Generator(device=dev)
        gen.manual_seed(c["seed"])
        for s in range(B):
            slots = torch.from_numpy(self.pool.allocate(s, ctx)).to(dev)
            for layer in range(L):
                k = torch.randn(ctx, hkv, dim, generator=gen, device=dev).to(torch.bfloat16)
                v = torch.randn(ctx, hkv, dim, generator=gen, device=dev).to(torch.bfloat16)
                self.pool.append_kv(layer, k, v, slots, stream)
        self.max_blocks = (ctx + bs - 1) // bs
        self.table, self.lens = self.pool.block_table(list(range(B)), self.max_blocks)
        self.d_table, self.d_lens = torch.from_numpy(self.table).to(dev), torch.from_numpy(self.lens).to(dev)
        self.qstart = np.arange(B + 1, dtype=np.int32) * C
        self.d_qstart = torch.from_numpy(self.qstart).to(dev)
        self.qs = [torch.randn(B * C, hq, dim, generator=gen, device=dev).to(torch.bfloat16) for _ in range(L)]
        self.q = self.qs[0]  # what the CPU baseline reads
        self.out = torch.empty(B * C, hq, dim, dtype=torch.float32, device=dev)
        # the context split and its workspace, planned once (every layer's
        # launch reuses it in turn on the one stream)
        self.piece_tokens, self.pieces, nb, self.waves = self.pool.prefill_plan(pkv.PKV_BF16, hq, B, C, ctx,
                                                                               piece_tokens, waves=True)
        self.ws = torch.zeros(nb, dtype=torch.uint8, device=dev) if nb > 0 else None

    def prefill(self, layer):
        self.pool.prefill(layer, self.qs[layer], self.d_qstart, self.C, self.d_table, self.d_lens, self.scale,
                          self.ctx, out=self.out, workspace=self.ws, piece_tokens=self.piece_tokens,
                          stream=self.stream)
        return self.out


def prefill_cpu_baseline(w, target_s):
    """The FP64 prefill oracle on a bounded sample: one layer, sequences in
    order until ~target_s of CPU time; tokens/s = query tokens / (layers x time)."""
    from oracle import oracle as orc
    from paged_kv_cache_62_amd import synth
    c = w.c
    threads = max(1, min(16, os.cpu_count() or 1))
    blocks = sorted({int(b) for b in w.table.ravel() if b >= 0})
    codes, scales = w.pool.read_blocks(0, blocks)
    N = int(max(blocks)) + 1
    kc = np.zeros((N, c["hkv"], c["bs"], c["dim"]), np.int8)
    vc = np.zeros_like(kc)
    ks = np.ones((N, c["hkv"]), np.float32)
    vs = np.ones_like(ks)
    kc[blocks], vc[blocks] = codes[:, 0], codes[:, 1]
    ks[blocks], vs[blocks] = scales[:, 0], scales[:, 1]
    q = synth.as_f32(w.q.cpu())
    done_q, elapsed = 0, 0.0
    for s in range(len(w.lens)):
        a, b = int(w.qstart[s]), int(w.qstart[s + 1])
        t0 = time.perf_counter()
        orc.prefill_attention(orc.I8, kc, vc, ks, vs, q[a:b], np.array([0, b - a], np.int32), w.table[s:s + 1],
                              w.lens[s:s + 1], w.scale, threads=threads)
        elapsed += time.perf_counter() - t0
        done_q += b - a
        if elapsed >= target_s:
            break
    return {"value": done_q / (elapsed * c["layers"]), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": (f"FP64 prefill oracle on layer 0 for {done_q} of {int(w.qstart[-1])} query tokens "
                       f"({elapsed:.1f} s, {threads} threads) over the GPU cache read back; tokens/s = query "
                       f"tokens / (layers x time), extrapolated from the sampled layer and sequences")}


def run_prefill(args, stream):
    """Chunked prefill: the cache holds B x ctx tokens (the chunk's K/V
    included); a step is one pkv_prefill_attention per layer over the last
    `chunk` tokens of every sequence, as a HIP graph replayed K times."""
    import torch
    print(f"# building prefill workload {args.config}", file=sys.stderr, flush=True)
    w = PrefillWorkload(args.config, stream, args.piece_tokens)
    c = w.c
    L, hq, dim, B, ctx, C = w.L, w.hq, w.dim, w.B, w.ctx, w.C

    def step():
        for layer in range(L):
            w.prefill(layer)

    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        step()
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    print(f"# warmup done; timing {args.steps} steps", file=sys.stderr, flush=True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    total_ms = e0.elapsed_time(e1)
    avg_dur_s = total_ms / 1e3 / (args.steps * L)
    # algorithmic work per launch: every (query, head, visible token) pair costs
    # 2*d flops for q.k and 2*d for p*v
    pairs = sum(sum(ctx - C + i + 1 for i in range(C)) for _ in range(B)) * hq
    flops = 4.0 * dim * pairs
    achieved = flops / avg_dur_s / 1e12
    res = {
        "metric": "decode attn tokens/sec and KV-read HBM GB/s (% of MI355X peak), 1 GPU",
        "value": B * C * args.steps / (total_ms / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": total_ms / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8 kv, fp16 matrix-core products / fp32 accumulate",
        "data": "synthetic (seeded K/V and queries), cache filled before timing",
        "config": {"workload": WORKLOAD_NAMES[args.config], "batch": B, "query_tokens_per_seq": C,
                   "context": ctx, "layers_per_step": L, "hip_graph": True,
                   "context_pieces": w.pieces, "piece_tokens": w.piece_tokens if w.pieces > 1 else None,
                   "wavefronts_per_workgroup": w.waves},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": MFMA_FP16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / MFMA_FP16_PEAK_TFLOPS, "traffic": measured_traffic(args.config),
                     "kernel": ("prefill_kernel (causal paged attention, fp16 matrix cores"
                                + (", context pieces merged by the last to finish)" if w.pieces > 1 else ")")),
                     "avg_launch_us": avg_dur_s * 1e6, "flops_per_launch": flops,
                     "timing": f"HIP events around {args.steps} replays of a graph of the {L} prefill launches"},
    }
    res["_workload"] = w
    return res


if __name__ == "__main__":
    main()
