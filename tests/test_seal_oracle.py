"""Pins of the seal-on-full oracle (oracle/seal.py) against what the page and
the mathematics fix, independently of its own code. CPU only.

"轻量级推理引擎实战：KV Cache 量化与连续批处理的底层优化" §三: the quantizer takes FP16
data (modelled as f32), one scale per (block, head) = max|x|/127 (1.0 for an
all-zero head), codes round(x/scale) clamped to [-127, 127]; third design
note: quantize off the hot path, read here as "once a block is
full" (until then its rows are FP16)."""
import numpy as np
import pytest

from oracle import oracle as orc
from oracle import seal
from paged_kv_cache_62_amd import synth
from tests.test_oracle_pins import exact_encode


def _rows(seed, n, dim, scale=1.0, outliers=0.0):
    x = synth.normal(synth.stream_seed(seed, 1), n * dim).reshape(n, dim) * scale
    if outliers:
        u = synth.uniform(synth.stream_seed(seed, 2), n * dim).reshape(n, dim)
        x = np.where(u < outliers, 20.0, x)
    return x.astype(np.float32)


@pytest.mark.parametrize("seed", range(6))
def test_quantize_block_is_the_pinned_quantizer_on_fp16_rows(oracle_lib, seed):
    """Sealing = the C++ oracle's quantizer (pinned separately) writing a
    fresh block in one call, applied to the binary16-rounded rows."""
    x = _rows(62000 + seed, 16, 64, scale=[0.5, 1, 4, 1e-3, 30, 1][seed], outliers=0.02 * (seed % 2))
    x16 = x.astype(np.float16).astype(np.float32)
    q, s = seal.quantize_block(x16)
    q_ref, s_ref = orc.quant_append(np.zeros((16, 64), np.int8), 1.0, 0, x16)
    np.testing.assert_array_equal(q, q_ref)
    assert np.float32(s).view(np.uint32) == np.float32(s_ref).view(np.uint32)
    np.testing.assert_array_equal(q, exact_encode(x16, s))


def test_quantize_block_closed_forms():
    q, s = seal.quantize_block(np.full((4, 8), -2.5, np.float32))
    assert s == np.float32(2.5) / np.float32(127) and np.all(q == -127)
    q, s = seal.quantize_block(np.zeros((4, 8), np.float32))
    assert s == 1.0 and np.all(q == 0)
    x = np.zeros((2, 4), np.float32)
    x[1, 2] = 127.0      # scale exactly 1: codes are the rounded values
    x[0, 0] = 2.5        # a tie: rounds to even
    x[0, 1] = -3.5
    q, s = seal.quantize_block(x)
    assert s == 1.0 and q[1, 2] == 127 and q[0, 0] == 2 and q[0, 1] == -4


@pytest.mark.parametrize("bs", [16, 32, 64])
def test_one_token_at_a_time_equals_one_call(bs):
    """A block is FP16 until its last row is written; the sealed codes do not
    depend on how the rows arrived."""
    heads, dim = 2, 64
    a = seal.SealCache(1, heads, dim, bs, 4)
    b = seal.SealCache(1, heads, dim, bs, 4)
    k = _rows(1, bs, heads * dim).reshape(bs, heads, dim)
    v = _rows(2, bs, heads * dim, scale=3.0).reshape(bs, heads, dim)
    blk = 2
    slots = blk * bs + np.arange(bs)
    for t in range(bs):
        a.append(0, k[t:t + 1], v[t:t + 1], slots[t:t + 1])
        if t < bs - 1:  # still FP16: the rows so far, binary16-rounded; codes untouched
            np.testing.assert_array_equal(a.f16[0, 0, blk, :, :t + 1].transpose(1, 0, 2),
                                          k[:t + 1].astype(np.float16).view(np.uint16))
            assert np.all(a.codes[0, :, blk] == 0)
    b.append(0, k, v, slots)
    np.testing.assert_array_equal(a.codes, b.codes)
    np.testing.assert_array_equal(a.scales.view(np.uint32), b.scales.view(np.uint32))
    for h in range(heads):
        q, s = seal.quantize_block(v[:, h].astype(np.float16).astype(np.float32))
        np.testing.assert_array_equal(a.codes[0, 1, blk, h], q)
        assert a.scales[0, 1, blk, h] == s


def test_values_mix_sealed_and_fp16_rows(oracle_lib):
    bs, heads, dim = 16, 1, 64
    c = seal.SealCache(1, heads, dim, bs, 4)
    k = _rows(3, 40, dim).reshape(40, 1, dim)
    table = np.array([[3, 0, 2]], dtype=np.int32)
    slots = np.concatenate([3 * bs + np.arange(16), np.arange(16), 2 * bs + np.arange(8)])
    c.append(0, k, k, slots)
    kv, _ = c.values(0, table, np.array([40]))
    f16 = k.astype(np.float16).astype(np.float64)
    np.testing.assert_array_equal(kv[2, 0, :8], f16[32:, 0])            # partial block: FP16 rows
    q, s = seal.quantize_block(k[:16, 0].astype(np.float16).astype(np.float32))
    np.testing.assert_array_equal(kv[3, 0], q.astype(np.float64) * np.float64(s))
    # the FP64 decode over these values equals the int8 / fp16 decodes where one type holds throughout
    qv = _rows(4, 1, dim).reshape(1, 1, dim)
    t1 = np.array([[3]], np.int32)
    ref = orc.decode_attention(orc.I8, c.codes[0, 0], c.codes[0, 1], c.scales[0, 0], c.scales[0, 1], qv, t1,
                               np.array([16], np.int32), 0.125)
    got = orc.decode_attention(orc.VALUES, kv, kv, None, None, qv, t1, np.array([16], np.int32), 0.125)
    np.testing.assert_array_equal(ref, got)
    t2 = np.array([[2]], np.int32)
    ref = orc.decode_attention(orc.F16, c.f16[0, 0], c.f16[0, 1], np.ones((4, 1)), np.ones((4, 1)), qv, t2,
                               np.array([8], np.int32), 0.125)
    got = orc.decode_attention(orc.VALUES, kv, kv, None, None, qv, t2, np.array([8], np.int32), 0.125)
    np.testing.assert_array_equal(ref, got)


def test_copy_on_write_copies_fp16_rows():
    bs = 16
    c = seal.SealCache(2, 1, 64, bs, 4)
    for layer in range(2):
        k = _rows(10 + layer, 5, 64).reshape(5, 1, 64)
        c.append(layer, k, k, 1 * bs + np.arange(5))
    c.copy_block(1, 3, 5)
    np.testing.assert_array_equal(c.f16[:, :, 3, :, :5], c.f16[:, :, 1, :, :5])
