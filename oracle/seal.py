"""Oracle of the seal-on-full INT8 cache (lazy quantization).

TEST INFRASTRUCTURE ONLY (tests and the benchmark's checks import it; the
library never does). numpy, written from "轻量级推理引擎实战：KV Cache 量化与连续
批处理的底层优化" §三: its quantizer works on FP16 data (modelled as f32), one
scale per (block, KV head) = max|x| / 127 (1.0 when the head is all zero),
codes round(x / scale) clamped to [-127, 127] -- and its third design note
defers quantization off the hot path. Reading (the page gives no mechanism):
a block stays in FP16 while it is a sequence's partly filled last block and
is quantized once, all of its rows together, when its last row is written.

State per (layer, K|V): FP16 rows [N][Hkv][bs][d] (binary16 bits), INT8
codes [N][Hkv][bs][d] and scales [N][Hkv] (meaningful once a block is full).
"""
from __future__ import annotations

import numpy as np


def f16_bits(x: np.ndarray) -> np.ndarray:
    """binary32 -> binary16, round to nearest even (IEEE)."""
    return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def quantize_block(x: np.ndarray):
    """The page's quantize_block over one (block, head): x [rows][d] binary32.
    Returns (int8 codes [rows][d], binary32 scale). Division is IEEE binary32
    (numpy's float32 divide), rounding half to even (np.rint)."""
    x = np.asarray(x, dtype=np.float32)
    m = np.float32(np.abs(x).max()) if x.size else np.float32(0)
    scale = np.float32(m / np.float32(127.0)) if m > np.float32(1e-6) else np.float32(1.0)
    q = np.clip(np.rint(x / scale), -127, 127).astype(np.int8)
    return q, scale


class SealCache:
    def __init__(self, layers, heads, dim, bs, nblocks):
        self.layers, self.heads, self.dim, self.bs, self.nblocks = layers, heads, dim, bs, nblocks
        shp = (layers, 2, nblocks, heads, bs, dim)
        self.f16 = np.zeros(shp, dtype=np.uint16)
        self.codes = np.zeros(shp, dtype=np.int8)
        self.scales = np.ones((layers, 2, nblocks, heads), dtype=np.float32)

    def append(self, layer, k, v, slots):
        """k, v: [n][heads][dim] binary32 (exact widenings of the inputs), the
        tokens in slot order. Each row is stored in FP16; a block whose last
        row is written is quantized, all rows at once, per (head, K|V)."""
        for i, slot in enumerate(np.asarray(slots, dtype=np.int64)):
            b, r = int(slot) // self.bs, int(slot) % self.bs
            for kv, x in ((0, k), (1, v)):
                self.f16[layer, kv, b, :, r, :] = f16_bits(x[i])
            if r == self.bs - 1:
                self._seal(layer, b)

    def _seal(self, layer, b):
        for kv in range(2):
            for h in range(self.heads):
                x = self.f16[layer, kv, b, h].view(np.float16).astype(np.float32)
                self.codes[layer, kv, b, h], self.scales[layer, kv, b, h] = quantize_block(x)

    def copy_block(self, src, dst, rows):
        """Copy-on-write: the first `rows` rows of every layer, K and V."""
        self.f16[:, :, dst, :, :rows] = self.f16[:, :, src, :, :rows]
        self.codes[:, :, dst] = self.codes[:, :, src]
        self.scales[:, :, dst] = self.scales[:, :, src]

    def values(self, layer, table, lens):
        """float64 keys and values [N][Hkv][bs][d] as decode reads them: the
        dequantized codes of full blocks, the FP16 rows of each sequence's
        partly filled last block. Blocks no sequence reaches stay zero."""
        k = np.zeros((self.nblocks, self.heads, self.bs, self.dim), dtype=np.float64)
        v = np.zeros_like(k)
        for s in range(len(lens)):
            n = int(lens[s])
            for j in range(-(-n // self.bs)):
                b = int(table[s, j])
                rows = min(self.bs, n - j * self.bs)
                for kv, out in ((0, k), (1, v)):
                    if rows == self.bs:
                        out[b] = self.codes[layer, kv, b].astype(np.float64) * \
                            self.scales[layer, kv, b].astype(np.float64)[:, None, None]
                    else:
                        out[b, :, :rows] = self.f16[layer, kv, b, :, :rows].view(np.float16).astype(np.float64)
        return k, v
