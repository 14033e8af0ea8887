"""ctypes binding of the CPU oracle (``pkv_oracle.cpp``).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the library. It shares nothing with the
HIP path but the seeded input arrays that both sides are handed.

Every function here is argument marshalling; the arithmetic lives in the C++
file, where each step cites the page it follows.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pkv_oracle.cpp")
_LIB = os.path.join(_HERE, "liboracle.so")

OK, INVALID, OOM, NO_FREE_BLOCK, UNKNOWN_SEQ, SEQ_EXISTS = 0, -1, -2, -3, -4, -5
F16, I8 = 1, 3  # cache element types (binary16 bits / int8 codes)
VALUES = 0      # decode_attention over float64 key/value numbers (mixed-format caches)


def build(force: bool = True) -> str:
    """Compile the oracle with g++ (IEEE arithmetic: no fast-math, no contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["g++", "-std=c++17", "-O2", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", "-pthread", _SRC, "-o", tmp]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = C.CDLL(_LIB)
        i32, i64, u64, f32, f64, vp = C.c_int32, C.c_int64, C.c_uint64, C.c_float, C.c_double, C.c_void_p
        sig = {
            "orc_kv_bytes": (u64, [u64] * 6),
            "orc_num_blocks": (i64, [i64, i64]),
            "orc_tail_waste": (i64, [i64, i64]),
            "orc_f16_to_f32": (f32, [C.c_uint16]),
            "orc_f32_to_f16": (C.c_uint16, [f32]),
            "orc_bf16_to_f32": (f32, [C.c_uint16]),
            "orc_alloc_create": (vp, [i32, i32, vp]),
            "orc_alloc_destroy": (None, [vp]),
            "orc_alloc_allocate": (C.c_int, [vp, i64, i32, vp]),
            "orc_alloc_append": (C.c_int, [vp, vp, i32, vp, vp]),
            "orc_alloc_fork": (C.c_int, [vp, i64, i64]),
            "orc_alloc_free": (C.c_int, [vp, i64]),
            "orc_alloc_table": (C.c_int, [vp, vp, i32, i32, vp, vp]),
            "orc_alloc_stats": (None, [vp, vp]),
            "orc_alloc_refcount": (i32, [vp, i32]),
            "orc_alloc_free_queue": (i32, [vp, vp]),
            "orc_alloc_take_cows": (i32, [vp, vp, i32]),
            "orc_quant_append": (None, [vp, vp, i32, vp, i32, i32]),
            "orc_cache_create": (vp, [i32, i32, i32, i32, i32, i32]),
            "orc_cache_destroy": (None, [vp]),
            "orc_cache_append": (C.c_int, [vp, i32, vp, vp, vp, i32]),
            "orc_cache_copy_block": (None, [vp, i32, i32, i32]),
            "orc_cache_read_block": (None, [vp, i32, i32, vp, vp]),
            "orc_decode_attention": (C.c_int, [i32, i32, i32, i32, i32, vp, vp, vp, vp, vp,
                                               i32, vp, i32, vp, i32, f64, vp, i32]),
            "orc_prefill_attention": (C.c_int, [i32, i32, i32, i32, i32, vp, vp, vp, vp, vp,
                                                i32, vp, vp, i32, vp, i32, f64, vp, i32]),
            "orc_hardware_threads": (i32, []),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


# ----------------------------------------------------------------- O1, O2
def kv_bytes(L, H, d, s, B, nbytes) -> int:
    return int(lib().orc_kv_bytes(L, H, d, s, B, nbytes))


def num_blocks(length, bs) -> int:
    return int(lib().orc_num_blocks(length, bs))


def tail_waste(length, bs) -> int:
    return int(lib().orc_tail_waste(length, bs))


# ------------------------------------------------------ binary16 / bfloat16
def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32).ravel()
    f = lib().orc_f32_to_f16
    return np.array([f(float(v)) for v in x], dtype=np.uint16)


def f16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    f = lib().orc_f16_to_f32
    return np.array([f(int(v)) for v in np.asarray(h, dtype=np.uint16).ravel()], dtype=np.float32)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    f = lib().orc_bf16_to_f32
    return np.array([f(int(v)) for v in np.asarray(b, dtype=np.uint16).ravel()], dtype=np.float32)


# ------------------------------------------------------------------- O3
class Allocator:
    """The FIFO / refcount / copy-on-write block allocator model."""

    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        self.num_blocks, self.block_size = num_blocks, block_size
        fo = None if free_order is None else np.ascontiguousarray(free_order, dtype=np.int32)
        self._keep = fo
        self.h = lib().orc_alloc_create(num_blocks, block_size, None if fo is None else _p(fo))
        if not self.h:
            raise ValueError("bad allocator arguments")

    def __del__(self):
        if getattr(self, "h", None):
            lib().orc_alloc_destroy(self.h)
            self.h = None

    def allocate(self, seq: int, n_tokens: int):
        slots = np.zeros(max(n_tokens, 1), dtype=np.int64)
        st = lib().orc_alloc_allocate(self.h, seq, n_tokens, _p(slots))
        return st, slots[:n_tokens]

    def append(self, seqs, n_new):
        seqs = np.ascontiguousarray(seqs, dtype=np.int64)
        n_new = np.ascontiguousarray(n_new, dtype=np.int32)
        slots = np.zeros(max(int(n_new.sum()) if len(n_new) else 0, 1), dtype=np.int64)
        st = lib().orc_alloc_append(self.h, _p(seqs), len(seqs), _p(n_new), _p(slots))
        return st, slots[: int(n_new.sum()) if len(n_new) else 0]

    def fork(self, parent: int, child: int) -> int:
        return lib().orc_alloc_fork(self.h, parent, child)

    def free(self, seq: int) -> int:
        return lib().orc_alloc_free(self.h, seq)

    def table(self, seqs, max_blocks: int):
        seqs = np.ascontiguousarray(seqs, dtype=np.int64)
        table = np.zeros((len(seqs), max_blocks), dtype=np.int32)
        lens = np.zeros(len(seqs), dtype=np.int32)
        st = lib().orc_alloc_table(self.h, _p(seqs), len(seqs), max_blocks, _p(table), _p(lens))
        return st, table, lens

    def stats(self) -> dict:
        out = np.zeros(5, dtype=np.int64)
        lib().orc_alloc_stats(self.h, _p(out))
        return dict(free=int(out[0]), used=int(out[1]), shared=int(out[2]),
                    cow=int(out[3]), seqs=int(out[4]))

    def refcount(self, block: int) -> int:
        return int(lib().orc_alloc_refcount(self.h, block))

    def free_queue(self) -> np.ndarray:
        out = np.zeros(self.num_blocks, dtype=np.int32)
        n = lib().orc_alloc_free_queue(self.h, _p(out))
        return out[:n]

    def take_cows(self) -> np.ndarray:
        out = np.zeros((self.num_blocks, 3), dtype=np.int32)
        n = lib().orc_alloc_take_cows(self.h, _p(out), self.num_blocks)
        return out[:n]


# ------------------------------------------------------------------- O4
def quant_append(codes: np.ndarray, scale: float, fill: int, x: np.ndarray):
    """Quantize rows x [rows][dim] into a tile of codes [bs][dim] holding
    `fill` rows already. Returns (new codes, new scale); inputs unchanged."""
    codes = np.ascontiguousarray(codes, dtype=np.int8).copy()
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, dim = x.shape
    assert codes.shape[1] == dim and fill + rows <= codes.shape[0]
    sc = np.array([scale], dtype=np.float32)
    lib().orc_quant_append(_p(codes), _p(sc), fill, _p(x), rows, dim)
    return codes, float(sc[0])


class Cache:
    """The oracle's own paged cache, filled by replaying appends and copies."""

    def __init__(self, layers, heads, dim, bs, nblocks, kv_dtype):
        self.layers, self.heads, self.dim, self.bs, self.nblocks = layers, heads, dim, bs, nblocks
        self.kv_dtype = kv_dtype
        self.h = lib().orc_cache_create(layers, heads, dim, bs, nblocks, kv_dtype)
        if not self.h:
            raise ValueError("bad cache arguments")

    def __del__(self):
        if getattr(self, "h", None):
            lib().orc_cache_destroy(self.h)
            self.h = None

    def append(self, layer, k: np.ndarray, v: np.ndarray, slots: np.ndarray) -> int:
        """k, v: [n][heads][dim] binary32 (exact widenings of the inputs)."""
        k = np.ascontiguousarray(k, dtype=np.float32)
        v = np.ascontiguousarray(v, dtype=np.float32)
        slots = np.ascontiguousarray(slots, dtype=np.int64)
        return lib().orc_cache_append(self.h, layer, _p(k), _p(v), _p(slots), len(slots))

    def copy_block(self, src, dst, rows):
        lib().orc_cache_copy_block(self.h, src, dst, rows)

    def read_block(self, layer, block):
        dt = np.int8 if self.kv_dtype == I8 else np.uint16
        codes = np.zeros((2, self.heads, self.bs, self.dim), dtype=dt)
        scales = np.zeros((2, self.heads), dtype=np.float32)
        lib().orc_cache_read_block(self.h, layer, block, _p(codes), _p(scales))
        return codes, scales

    def layer_arrays(self, layer, blocks=None):
        """Oracle-layout arrays of one layer for decode_attention:
        (k_codes, v_codes [N][H][bs][dim], k_scales, v_scales [N][H])."""
        dt = np.int8 if self.kv_dtype == I8 else np.uint16
        N = self.nblocks
        kc = np.zeros((N, self.heads, self.bs, self.dim), dtype=dt)
        vc = np.zeros_like(kc)
        ks = np.ones((N, self.heads), dtype=np.float32)
        vs = np.ones_like(ks)
        for b in (range(N) if blocks is None else blocks):
            codes, sc = self.read_block(layer, b)
            kc[b], vc[b] = codes[0], codes[1]
            ks[b], vs[b] = sc[0], sc[1]
        return kc, vc, ks, vs


# ------------------------------------------------------------------- O5
def decode_attention(kv_dtype, k_codes, v_codes, k_scales, v_scales, q, table, lens,
                     softmax_scale, threads=0):
    """FP64 paged decode attention over one layer's cache arrays
    (oracle layout [N][Hkv][bs][dim]): int8 codes (I8), binary16 bits (F16),
    or the values themselves as float64 (VALUES). q: [B][Hq][dim] binary32.
    Returns [B][Hq][dim] float64."""
    want = {I8: np.int8, F16: np.uint16, VALUES: np.float64}[kv_dtype]
    k_codes = np.ascontiguousarray(k_codes)
    v_codes = np.ascontiguousarray(v_codes)
    assert k_codes.dtype == want and v_codes.dtype == want
    N, hkv, bs, dim = k_codes.shape
    k_scales = np.ascontiguousarray(k_scales, dtype=np.float32)
    v_scales = np.ascontiguousarray(v_scales, dtype=np.float32)
    q = np.ascontiguousarray(q, dtype=np.float32)
    B, hq, _ = q.shape
    table = np.ascontiguousarray(table, dtype=np.int32)
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    out = np.zeros((B, hq, dim), dtype=np.float64)
    st = lib().orc_decode_attention(kv_dtype, N, hkv, bs, dim, _p(k_codes), _p(v_codes),
                                    _p(k_scales), _p(v_scales), _p(q), hq, _p(table),
                                    table.shape[1], _p(lens), B, float(softmax_scale),
                                    _p(out), threads)
    if st != OK:
        raise ValueError(f"oracle decode_attention rejected its arguments ({st})")
    return out


def prefill_attention(kv_dtype, k_codes, v_codes, k_scales, v_scales, q, query_start, table, lens,
                      softmax_scale, threads=0):
    """FP64 causal attention of each sequence's last q_len cached tokens
    (query_start: [B+1] prefix offsets into q's rows) over its context.
    q: [total][Hq][dim] binary32. Returns [total][Hq][dim] float64."""
    want = {I8: np.int8, F16: np.uint16, VALUES: np.float64}[kv_dtype]
    k_codes = np.ascontiguousarray(k_codes)
    v_codes = np.ascontiguousarray(v_codes)
    assert k_codes.dtype == want and v_codes.dtype == want
    N, hkv, bs, dim = k_codes.shape
    k_scales = np.ascontiguousarray(k_scales, dtype=np.float32)
    v_scales = np.ascontiguousarray(v_scales, dtype=np.float32)
    q = np.ascontiguousarray(q, dtype=np.float32)
    total, hq, _ = q.shape
    qs = np.ascontiguousarray(query_start, dtype=np.int32)
    table = np.ascontiguousarray(table, dtype=np.int32)
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    assert qs[-1] == total
    out = np.zeros((total, hq, dim), dtype=np.float64)
    st = lib().orc_prefill_attention(kv_dtype, N, hkv, bs, dim, _p(k_codes), _p(v_codes), _p(k_scales),
                                     _p(v_scales), _p(q), hq, _p(qs), _p(table), table.shape[1], _p(lens),
                                     len(lens), float(softmax_scale), _p(out), threads)
    if st != OK:
        raise ValueError(f"oracle prefill_attention rejected its arguments ({st})")
    return out


def hardware_threads() -> int:
    return int(lib().orc_hardware_threads())
