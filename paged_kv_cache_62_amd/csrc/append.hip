// append.hip -- H1 of libpkv for gfx950: store new tokens' K/V at their slots,
// rounded to binary16, or quantized with the per-(block, KV head) symmetric
// INT8 quantizer of "轻量级推理引擎实战：KV Cache 量化与连续批处理的底层优化" §三
// (also its seal-on-full variant, the section's third design note).

#include "device.h"

namespace pkv {
namespace {

// ---------------------------------------------------------------------------
// H1 (binary16 cache): one thread per (token, head, K|V, 8-element chunk);
// each value rounded to binary16, ties to even.
// ---------------------------------------------------------------------------
// Chunk ch (8 elements) of token i's row of head h, K (kv 0) or V (kv 1),
// into row `row` of block blk.
template <int IN>
__device__ __forceinline__ void append_f16_chunk(const LayerView& lv, int kv, int h, int64_t blk, int row,
                                                 const void* src, int64_t i, int ch) {
  const int D = lv.head_dim;
  const int hkv = lv.num_kv_heads;
  const size_t sbase = ((size_t)i * hkv + h) * D + ch * 8;
  uint16_t hv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e)
    hv[e] = __builtin_bit_cast(uint16_t, (_Float16)load_elem<IN>(src, sbase + e));
  uint16_t* tile = (uint16_t*)(kv ? lv.v_codes : lv.k_codes) +
                   ((size_t)blk * hkv + h) * lv.block_size * D;
  if (kv == 0) {
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = (uint32_t)hv[2 * e] | ((uint32_t)hv[2 * e + 1] << 16);
    *(uint4*)(tile + k_tile_offset(row, ch * 8, D)) = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) tile[v_tile_offset(row, ch * 8 + e, D)] = hv[e];
  }
}

template <int IN>
__global__ __launch_bounds__(256) void append_f16_kernel(const LayerView lv, const void* k,
                                                         const void* v, const int64_t* slots,
                                                         int32_t n) {
  const int hkv = lv.num_kv_heads;
  const int chunks = lv.head_dim / 8;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)n * hkv * 2 * chunks) return;
  const int ch = (int)(idx % chunks);
  int64_t rest = idx / chunks;
  const int h = (int)(rest % hkv);
  rest /= hkv;
  const int kv = (int)(rest & 1);
  const int64_t i = rest >> 1;
  const int64_t slot = slots[i];
  const int64_t blk = slot / lv.block_size;
  const int row = (int)(slot % lv.block_size);
  if (slot < 0 || blk >= lv.num_blocks) return;  // not a slot of this pool
  append_f16_chunk<IN>(lv, kv, h, blk, row, kv ? v : k, i, ch);
}

// ---------------------------------------------------------------------------
// H1 (int8 cache): one wavefront per (run, head, K|V), where a run is the
// maximal group of consecutive tokens that land in one block. Only the
// wavefront of a run's first token works, so every (block, head, K|V) tile
// has a single writer and no atomics are needed.
// ---------------------------------------------------------------------------

// One wavefront appends tokens i .. i+nr-1 (rows of src [token][Hkv][d]) of
// head h, K (kv 0) or V (kv 1), at rows row0 .. row0+nr-1 of block blk:
// grow-only scale, old rows re-encoded when it grows (P5 section 3 plus the
// rule for partly filled blocks). issue() sends every load without waiting
// (the block's old codes, rows < row0, 16 bytes per load; its scale; up to
// kPre new values per lane), so a wavefront can have the K and the V append
// in flight together; finish() does the rest and returns the new scale.
// Old rows of a K tile are its first row0*D bytes; those of a V tile lie in
// its first ceil(row0/16) 16-token sub-tiles, where each byte's token is
// decoded from its offset.
template <int IN>
struct I8Append {
  static constexpr int kMaxChunks = 8;  // per lane: 64 lanes x 8 x 16 bytes covers any tile
  static constexpr int kPre = 2;        // new values held per lane (one row of d <= 128)
  const LayerView* lv;
  int kv, h, row0, nr;
  int64_t i;
  const void* src;
  int8_t* tile;
  float* sp;
  int32_t* qp;
  int old_bytes;
  uint4 oc[kMaxChunks];
  float s_old;
  float pre[kPre];

  __device__ __forceinline__ void issue(const LayerView& lv_, int kv_, int h_, int64_t blk, int row0_, int nr_,
                                        const void* src_, int64_t i_) {
    lv = &lv_; kv = kv_; h = h_; row0 = row0_; nr = nr_; src = src_; i = i_;
    const int lane = threadIdx.x & 63;
    const int hkv = lv_.num_kv_heads, D = lv_.head_dim, ld = __builtin_ctz(D);
    tile = (int8_t*)(kv ? lv_.v_codes : lv_.k_codes) + ((size_t)blk * hkv + h) * lv_.block_size * D;
    sp = (kv ? lv_.v_scales : lv_.k_scales) + (size_t)blk * hkv + h;
    qp = (kv ? lv_.v_qmax : lv_.k_qmax) + (size_t)blk * hkv + h;
    old_bytes = kv ? ((row0 + 15) >> 4) * 16 * D : row0 * D;  // <= 63*128 = 504 chunks
#pragma unroll
    for (int k = 0; k < kMaxChunks; ++k) {
      const int c = lane + 64 * k;
      oc[k] = c * 16 < old_bytes ? *(const uint4*)(tile + (size_t)c * 16) : make_uint4(0u, 0u, 0u, 0u);
    }
    s_old = row0 > 0 ? *sp : 1.f;
    if (nr * D <= 64 * kPre) {
#pragma unroll
      for (int k = 0; k < kPre; ++k) {
        const int e = lane + 64 * k;
        pre[k] = e < nr * D ? load_elem<IN>(src, ((size_t)(i + (e >> ld)) * hkv + h) * D + (e & (D - 1))) : 0.f;
      }
    }
  }

  __device__ __forceinline__ float finish() {
    const int lane = threadIdx.x & 63;
    const int hkv = lv->num_kv_heads, D = lv->head_dim, ld = __builtin_ctz(D);
    const uint32_t bias4 = kv ? 0x80808080u : 0u;  // V codes are stored biased by 128 (code ^ 0x80)
    auto off = [&](int t, int dd) { return kv ? v_tile_offset(t, dd, D) : k_tile_offset(t, dd, D); };
    // Bytes of chunk k that hold rows < row0, as a mask over each of its four
    // words (the same for all four). A K chunk lies in one row. A V chunk
    // lies in one lane's slice of a 16-token sub-tile (d/4 >= 16 bytes):
    // tokens base + byte % 4 with base = 16*sub + 4*tg.
    auto word_mask = [&](int k) -> uint32_t {
      const int c = lane + 64 * k;
      if (c * 16 >= old_bytes) return 0u;
      if (!kv) return ~0u;
      const int byte = c * 16;
      const int sub = byte >> (ld + 4);                     // 16-token sub-tile
      const int L = (byte & ((16 << ld) - 1)) >> (ld - 2);  // lane slice tg*16 + dm
      const int n = min(max(row0 - (sub * 16 + (L >> 4) * 4), 0), 4);  // valid tokens of the word
      return n == 4 ? ~0u : (1u << (8 * n)) - 1u;
    };
    auto new_value = [&](int e) {
      return load_elem<IN>(src, ((size_t)(i + (e >> ld)) * hkv + h) * D + (e & (D - 1)));
    };
    const bool held = nr * D <= 64 * kPre;
    int qm = 0;
#pragma unroll
    for (int k = 0; k < kMaxChunks; ++k) {
      const uint32_t wm = word_mask(k);
      const uint32_t ws[4] = {oc[k].x, oc[k].y, oc[k].z, oc[k].w};
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t x = (ws[w] ^ bias4) & wm;  // signed codes; other rows read as 0
#pragma unroll
        for (int b = 0; b < 4; ++b) qm = max(qm, abs((int)(int8_t)(x >> (8 * b))));
      }
    }
    float mx = 0.f;
    if (held) {
#pragma unroll
      for (int k = 0; k < kPre; ++k) mx = fmaxf(mx, fabsf(pre[k]));
    } else {
      for (int e = lane; e < nr * D; e += 64) mx = fmaxf(mx, fabsf(new_value(e)));
    }
    mx = wave_max(mx);

    float sc;
    int qold = 0;  // largest |code| of the old rows once this append is done
    if (row0 == 0) {
      sc = scale_of(mx);
    } else {
      qm = wave_max_int(qm);
      const float m_old = (float)qm * s_old;
      if (mx <= m_old) {
        sc = s_old;
        qold = qm;
      } else {
        // the max grew: re-encode the old codes from their dequantised values,
        // in the registers they were read into, and store whole chunks back
        // (bytes of rows >= row0 are written back unchanged)
        sc = scale_of(mx);
#pragma unroll
        for (int k = 0; k < kMaxChunks; ++k) {
          const int c = lane + 64 * k;
          if (c * 16 < old_bytes) {
            const uint32_t wm = word_mask(k);
            uint32_t ws[4] = {oc[k].x ^ bias4, oc[k].y ^ bias4, oc[k].z ^ bias4, oc[k].w ^ bias4};
#pragma unroll
            for (int w = 0; w < 4; ++w) {
#pragma unroll
              for (int b = 0; b < 4; ++b) {
                if (wm & (0xFFu << (8 * b))) {
                  const int code = (int)(int8_t)(ws[w] >> (8 * b));
                  const int8_t qn = encode((float)code * s_old, sc);
                  qold = max(qold, abs((int)qn));
                  ws[w] = (ws[w] & ~(0xFFu << (8 * b))) | ((uint32_t)(uint8_t)qn << (8 * b));
                }
              }
            }
            *(uint4*)(tile + (size_t)c * 16) = make_uint4(ws[0] ^ bias4, ws[1] ^ bias4, ws[2] ^ bias4, ws[3] ^ bias4);
          }
        }
        qold = wave_max_int(qold);
      }
    }
    int qnew = 0;  // largest |code| of the new rows
    if (held) {
#pragma unroll
      for (int k = 0; k < kPre; ++k) {
        const int e = lane + 64 * k;
        if (e < nr * D) {
          const int8_t q = encode(pre[k], sc);
          qnew = max(qnew, abs((int)q));
          tile[off(row0 + (e >> ld), e & (D - 1))] = (int8_t)(q ^ (int8_t)bias4);
        }
      }
    } else {
      for (int e = lane; e < nr * D; e += 64) {
        const int8_t q = encode(new_value(e), sc);
        qnew = max(qnew, abs((int)q));
        tile[off(row0 + (e >> ld), e & (D - 1))] = (int8_t)(q ^ (int8_t)bias4);
      }
    }
    qnew = wave_max_int(qnew);
    if (lane == 0) {
      *sp = sc;
      *qp = max(qold, qnew);
    }
    return sc;  // the same in every lane
  }
};

template <int IN>
__global__ __launch_bounds__(256) void append_i8_kernel(const LayerView lv, const void* k,
                                                        const void* v, const int64_t* slots,
                                                        int32_t n) {
  const int lane = threadIdx.x & 63;
  const int64_t wid = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hkv = lv.num_kv_heads;
  if (wid >= (int64_t)n * hkv * 2) return;
  const int h = (int)(wid % hkv);
  const int kv = (int)((wid / hkv) & 1);
  const int64_t i = wid / hkv / 2;
  const int bs = lv.block_size;
  const int lbs = __builtin_ctz(bs);  // block sizes are powers of two

  // The slots of tokens i .. i+63, one per lane, and of token i-1: the run
  // starting at i is the leading lanes whose slot lies in the same block.
  const int64_t sj = i + lane < n ? slots[i + lane] : -1;
  const int64_t slot0 = __builtin_amdgcn_readfirstlane((int)sj) | ((int64_t)__builtin_amdgcn_readfirstlane((int)(sj >> 32)) << 32);
  const int64_t blk = slot0 >> lbs;
  if (slot0 < 0 || blk >= lv.num_blocks) return;  // not a slot of this pool
  if (i > 0 && (slots[i - 1] >> lbs) == blk) return;  // not the first token of its run
  const uint64_t same = __ballot(sj >= 0 && (sj >> lbs) == blk);
  const int run = ~same == 0 ? 64 : __builtin_ctzll(~same);
  const int row0 = (int)(slot0 & (bs - 1));
  const int nr = min(run, bs - row0);  // rows stay inside the tile even for malformed slots
  I8Append<IN> ap;
  ap.issue(lv, kv, h, blk, row0, nr, kv ? v : k, i);
  (void)ap.finish();
}

// ---------------------------------------------------------------------------
// H1 for a seal-on-full INT8 layer (lazy quantization, "轻量级推理引擎实战"
// §三, third design note): one wavefront per (run, head, K|V), runs found as
// above. A run that leaves its block partly filled is stored as binary16
// rows in the block's FP16 staging tile. The run that writes the block's last
// row quantizes the whole block -- its staged rows and the run's own, all as
// binary16 values -- with the section's quantize_block: one scale max|x|/127
// (1.0 for an all-zero head), codes round(x / scale) to even, clamped to
// [-127, 127]; it stores the codes, the scale and the largest |code|.
// ---------------------------------------------------------------------------
template <int IN>
__global__ __launch_bounds__(256) void append_seal_kernel(const LayerView lv, const void* k,
                                                          const void* v, const int64_t* slots,
                                                          int32_t n) {
  const int lane = threadIdx.x & 63;
  const int64_t wid = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hkv = lv.num_kv_heads;
  if (wid >= (int64_t)n * hkv * 2) return;
  const int h = (int)(wid % hkv);
  const int kv = (int)((wid / hkv) & 1);
  const int64_t i = wid / hkv / 2;
  const int bs = lv.block_size;
  const int lbs = __builtin_ctz(bs);
  const int64_t sj = i + lane < n ? slots[i + lane] : -1;
  const int64_t slot0 = __builtin_amdgcn_readfirstlane((int)sj) | ((int64_t)__builtin_amdgcn_readfirstlane((int)(sj >> 32)) << 32);
  const int64_t blk = slot0 >> lbs;
  if (slot0 < 0 || blk >= lv.num_blocks) return;  // not a slot of this pool
  if (i > 0 && (slots[i - 1] >> lbs) == blk) return;  // not the first token of its run
  const uint64_t same = __ballot(sj >= 0 && (sj >> lbs) == blk);
  const int run = ~same == 0 ? 64 : __builtin_ctzll(~same);
  const int row0 = (int)(slot0 & (bs - 1));
  const int nr = min(run, bs - row0);

  const int D = lv.head_dim, ld = __builtin_ctz(D);
  const void* src = kv ? v : k;
  uint16_t* t16 = (uint16_t*)(kv ? lv.tail_v : lv.tail_k) + ((size_t)blk * hkv + h) * bs * D;
  auto off = [&](int t, int dd) { return kv ? v_tile_offset(t, dd, D) : k_tile_offset(t, dd, D); };
  // element e of the run (row e >> ld, dim e % D) as binary16 bits
  auto run_bits = [&](int e) {
    return __builtin_bit_cast(uint16_t, (_Float16)load_elem<IN>(src, ((size_t)(i + (e >> ld)) * hkv + h) * D + (e & (D - 1))));
  };
  if (row0 + nr < bs) {  // the block stays partly filled: stage the rows
    for (int e = lane; e < nr * D; e += 64) t16[off(row0 + (e >> ld), e & (D - 1))] = run_bits(e);
    return;
  }
  // the block is complete: its bs rows as binary16 values, staged or new
  auto value = [&](int e) {  // element e of the block (row e >> ld)
    const int t = e >> ld, dd = e & (D - 1);
    return f16_to_f32(t < row0 ? t16[off(t, dd)] : run_bits(((t - row0) << ld) | dd));
  };
  float mx = 0.f;
  for (int e = lane; e < bs * D; e += 64) mx = fmaxf(mx, fabsf(value(e)));
  mx = wave_max(mx);
  const float sc = scale_of(mx);
  int8_t* tile = (int8_t*)(kv ? lv.v_codes : lv.k_codes) + ((size_t)blk * hkv + h) * bs * D;
  const int8_t bias = kv ? (int8_t)0x80 : 0;  // V codes are stored biased by 128
  int qm = 0;
  for (int e = lane; e < bs * D; e += 64) {
    const int8_t q = encode(value(e), sc);
    qm = max(qm, abs((int)q));
    tile[off(e >> ld, e & (D - 1))] = (int8_t)(q ^ bias);
  }
  qm = wave_max_int(qm);
  if (lane == 0) {
    (kv ? lv.v_scales : lv.k_scales)[(size_t)blk * hkv + h] = sc;
    (kv ? lv.v_qmax : lv.k_qmax)[(size_t)blk * hkv + h] = qm;
  }
}

}  // namespace

hipError_t launch_append(const LayerView& lv, const void* k, const void* v, int in_dtype,
                         const int64_t* slots, int32_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  if (lv.kv_dtype == kF16) {
    const int64_t total = (int64_t)n * lv.num_kv_heads * 2 * (lv.head_dim / 8);
    const dim3 grid((unsigned)((total + 255) / 256));
    switch (in_dtype) {
      case kF32: hipLaunchKernelGGL(append_f16_kernel<kF32>, grid, dim3(256), 0, stream, lv, k, v, slots, n); break;
      case kF16: hipLaunchKernelGGL(append_f16_kernel<kF16>, grid, dim3(256), 0, stream, lv, k, v, slots, n); break;
      case kBF16: hipLaunchKernelGGL(append_f16_kernel<kBF16>, grid, dim3(256), 0, stream, lv, k, v, slots, n); break;
      default: return hipErrorInvalidValue;
    }
  } else if (lv.seal) {
    const int64_t waves = (int64_t)n * lv.num_kv_heads * 2;
    const dim3 grid((unsigned)((waves + 3) / 4));
    switch (in_dtype) {
      case kF32: hipLaunchKernelGGL(append_seal_kernel<kF32>, grid, dim3(256), 0, stream, lv, k, v, slots, n); break;
      case kF16: hipLaunchKernelGGL(append_seal_kernel<kF16>, grid, dim3(256), 0, stream, lv, k, v, slots, n); break;
      case kBF16: hipLaunchKernelGGL(append_seal_kernel<kBF16>, grid, dim3(256), 0, stream, lv, k, v, slots, n); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    const int64_t waves = (int64_t)n * lv.num_kv_heads * 2;
    const dim3 grid((unsigned)((waves + 3) / 4));
    switch (in_dtype) {
      case kF32: hipLaunchKernelGGL(append_i8_kernel<kF32>, grid, dim3(256), 0, stream, lv, k, v, slots, n); break;
      case kF16: hipLaunchKernelGGL(append_i8_kernel<kF16>, grid, dim3(256), 0, stream, lv, k, v, slots, n); break;
      case kBF16: hipLaunchKernelGGL(append_i8_kernel<kBF16>, grid, dim3(256), 0, stream, lv, k, v, slots, n); break;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

}  // namespace pkv
