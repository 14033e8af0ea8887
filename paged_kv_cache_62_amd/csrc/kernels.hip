// kernels.hip -- gfx950 kernels of libpkv.
//
//  H1 append:  store new tokens' K/V at their slots; binary16 rounding, or the
//              per-(block, KV head) symmetric INT8 quantizer of
//              "轻量级推理引擎实战：KV Cache 量化与连续批处理的底层优化" §三.
//  H2 decode:  split-context decode attention ("vLLM核心概念" §3.1: the new
//              query against every cached key/value; §3.2: logical token t in
//              block table[t / bs], row t % bs). One workgroup per (sequence,
//              KV head, context partition) serves all G query heads of the
//              group, so each K/V byte is read from HBM once per step.
//  H3 merge:   log-sum-exp merge of the partitions, done by the last
//              workgroup of each (sequence, KV head) to arrive, or by a
//              separate launch.
//  Decode step: H1 of each sequence's new token folded into H2 (one launch
//              per layer); the INT8 step has a second variant for grids the
//              device cannot hold at once.
//  Prefill:    causal attention of each sequence's newest tokens over its
//              context ("轻量级推理引擎实战" §一), on the same matrix-core
//              contractions with the context staged once per workgroup in LDS.
//
// Both contractions of H2 run on the matrix cores, 16 tokens at a time:
//   S^T[token][col] = K[token][:] . Q^T[:][col]      (A = K rows from HBM)
//   O^T[dim][col]  += V^T[dim][token] . P^T[token][col]
// The output layout of the first product is exactly the B-operand layout of
// the second, so the probabilities never leave their lanes. The 16 columns
// carry the G <= 4 query heads of the group, each split into exact parts:
//  * int8 K: q is rounded to a 22-bit integer (per-head power-of-two scale)
//    and split into three signed 8-bit digits, one column each, so the int8
//    product on the raw codes is exact and the three columns recombine to
//    the fp32 score;
//  * fp16 K: q is scaled by a power of two into fp16 (a second "lo" column
//    carries the rest of an fp32 q);
//  * P goes in as fp16 hi and lo parts in two columns, so the product keeps
//    about 22 bits of each probability.
// Scores are in base 2 (softmax_scale * log2 e folded in) so exp2 is one
// instruction.

#include <hip/hip_runtime.h>

#include <mutex>
#include <type_traits>
#include <utility>

#include "kernels.h"


namespace pkv {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// f(integral_constant<int, 0>) ... f(integral_constant<int, N - 1>), in order: a
// loop whose index is a compile-time constant in every body, so that arrays
// indexed by it stay in registers.
template <class F, int... I>
__device__ __forceinline__ void static_for_seq(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_seq(f, std::make_integer_sequence<int, N>{});
}

constexpr int kWaves = 4;             // wavefronts per decode workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kUnit = 16;             // tokens per unit of work (one MFMA tile of tokens)
constexpr int kRsrcWord3 = 0x00020000; // buffer descriptor word 3 for untyped dword loads (gfx9 family)
// sched_barrier mask: ALU, VALU, SALU and MFMA instructions may be scheduled
// across the barrier; memory instructions may not.
constexpr int kSchedAluOnly = 0x000F;
constexpr int kSlack = 4;              // the running max may trail the true maximum by this much (log2)
// The longest partition is 4 wavefronts x 64 units of 16 tokens, so one lane
// per unit holds a wavefront's bookkeeping.
static_assert(kMaxPartitionTokens == kWaves * 64 * kUnit, "partition bound");
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }
__device__ __forceinline__ float f16_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

template <int DT>
__device__ __forceinline__ float load_elem(const void* p, size_t i) {
  if constexpr (DT == kF32) return ((const float*)p)[i];
  else if constexpr (DT == kF16) return f16_to_f32(((const uint16_t*)p)[i]);
  else return bf16_to_f32(((const uint16_t*)p)[i]);
}

// DPP moves inside a row of 16 lanes; lanes that would read outside the row
// read 0 (bound_ctrl).
constexpr int kQuadXor1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kHalfMirror = 0x141; // lane i <- 7-i within 8
constexpr int kMirror = 0x140;     // lane i <- 15-i within 16
constexpr int kRowShl4 = 0x104;    // lane i <- i+4
constexpr int kRowShl8 = 0x108;    // lane i <- i+8
constexpr int kRowShr8 = 0x118;    // lane i <- i-8

template <int CTRL>
__device__ __forceinline__ int dpp_i(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, true);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(float, dpp_i<CTRL>(__builtin_bit_cast(int, x)));
}

// Maximum over all 64 lanes, returned wave-uniform.
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_f<kQuadXor1>(x));
  x = fmaxf(x, dpp_f<kQuadXor2>(x));
  x = fmaxf(x, dpp_f<kHalfMirror>(x));
  x = fmaxf(x, dpp_f<kMirror>(x));
  const int b = __builtin_bit_cast(int, x);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// Combine the four 16-lane rows holding the same column: lane l with lanes
// l^16, l^32, l^48 (the swaps exchange whole rows between two registers).
__device__ __forceinline__ float max_over_lane_groups(float x) {
  const int b = __builtin_bit_cast(int, x);
  const auto r16 = __builtin_amdgcn_permlane16_swap(b, b, false, false);
  x = fmaxf(__builtin_bit_cast(float, (int)r16[0]), __builtin_bit_cast(float, (int)r16[1]));
  const int c = __builtin_bit_cast(int, x);
  const auto r32 = __builtin_amdgcn_permlane32_swap(c, c, false, false);
  return fmaxf(__builtin_bit_cast(float, (int)r32[0]), __builtin_bit_cast(float, (int)r32[1]));
}
__device__ __forceinline__ float sum_over_lane_groups(float x) {
  const int b = __builtin_bit_cast(int, x);
  const auto r16 = __builtin_amdgcn_permlane16_swap(b, b, false, false);
  x = __builtin_bit_cast(float, (int)r16[0]) + __builtin_bit_cast(float, (int)r16[1]);
  const int c = __builtin_bit_cast(int, x);
  const auto r32 = __builtin_amdgcn_permlane32_swap(c, c, false, false);
  return __builtin_bit_cast(float, (int)r32[0]) + __builtin_bit_cast(float, (int)r32[1]);
}

__device__ __forceinline__ int wave_max_int(int x) {
  for (int off = 32; off >= 1; off >>= 1) x = max(x, __shfl_xor(x, off));
  return x;
}

// A float that is wave-uniform by construction, moved to a scalar register.
__device__ __forceinline__ float uniform_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}

// A pointer the compiler can treat as wave-uniform (it is, by construction,
// wherever this is used): buffer descriptors must live in scalar registers,
// and a value it cannot prove uniform costs a loop over the lanes per load.
__device__ __forceinline__ void* uniform_ptr(const void* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (void*)(((uint64_t)hi << 32) | lo);
}

// INT8 V codes are stored biased (code + 128, i.e. code ^ 0x80). Four of them
// -> four fp16 codes, exactly: each byte becomes the low mantissa byte of
// 1024.0 (0x6400), giving 1152 + code, and 1152 is subtracted. (Leaving the
// 1152 in and removing 1152 * sum(P) after the product would save the two
// subtractions, but the fp32 accumulators would then carry ~1152/|code|
// times the signal and its rounding error.)
__device__ __forceinline__ f16x4 biased_i8x4_to_f16x4(uint32_t u) {
  const uint32_t lo = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);
  const uint32_t hi = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);
  const f16x2 bias = {(_Float16)1152.0f, (_Float16)1152.0f};
  const f16x2 a = __builtin_bit_cast(f16x2, lo) - bias;
  const f16x2 b = __builtin_bit_cast(f16x2, hi) - bias;
  return f16x4{a[0], a[1], b[0], b[1]};
}

// x0, x1 as binary16 pairs hi + lo: hi is x rounded toward zero (one
// conversion instruction, which the compiler cannot fuse with anything, so
// every use sees the same hi) and lo = x - hi rounded to nearest; hi + lo
// carries about 22 significant bits.
__device__ __forceinline__ void split_f16x2(float x0, float x1, f16x2& hi, f16x2& lo) {
  hi = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(x0, x1));
  lo = f16x2{(_Float16)(x0 - (float)hi[0]), (_Float16)(x1 - (float)hi[1])};
}

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
__device__ __forceinline__ float scale_of(float max_abs) {
  return max_abs > 1e-6f ? max_abs / 127.0f : 1.0f;
}
__device__ __forceinline__ int8_t encode(float x, float scale) {
  const float y = x / scale;  // IEEE binary32 division (correctly rounded)
  const float rr = fminf(fmaxf(rintf(y), -127.0f), 127.0f);  // rintf: ties to even
  return (int8_t)(int)rr;
}
// Re-encode the bytes of a word of codes selected by `mask` from scale s_old
// to s_new (the bytes are stored XOR bias4).
__device__ __forceinline__ uint32_t requant_word(uint32_t w, uint32_t mask, float s_old, float s_new,
                                                 uint32_t bias4) {
  uint32_t x = w ^ bias4;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    if (mask & (0xFFu << (8 * b))) {
      const int code = (int)(int8_t)(x >> (8 * b));
      const uint32_t q = (uint32_t)(uint8_t)encode((float)code * s_old, s_new);
      x = (x & ~(0xFFu << (8 * b))) | (q << (8 * b));
    }
  }
  return x ^ bias4;
}

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

// ---------------------------------------------------------------------------
// H2: split-context decode on the matrix cores.
//
// Lane l of a wavefront: n16 = l % 16 (MFMA column / K row), gq = l / 16.
// Per 16-token unit a lane loads NCH 16-byte chunks of K row n16 (bytes
// 16*gq + 64*c) and NCH chunks of the V sub-tile (bytes l*16*NCH + 16*c).
// Each wavefront runs an online softmax over the units dealt to it (units
// u0+w, u0+w+4, ...): per-head running max m and sum l live in the lanes of
// that head's column. The running max is a reference that may trail the true
// maximum by up to kSlack (log2 units): it is raised, and the accumulators
// rescaled, only when some head's score exceeds it by more, so P stays below
// 2^kSlack. The four wavefronts merge through LDS; a single-partition
// sequence writes its output, otherwise the partition's (m, l, o/l) goes to
// the workspace and the last workgroup of the (sequence, KV head) to finish
// merges all partitions.
// ---------------------------------------------------------------------------
template <bool I8, int D, int G, int QT, bool APPEND, bool SEAL, int NB>
__device__ __forceinline__ void decode_body(const DecodeLaunch& a) {
  static_assert(!SEAL || I8, "seal-on-full: INT8 layers");
  constexpr int ESZ = I8 ? 1 : 2;
  constexpr int RB = D * ESZ;       // bytes per K row
  constexpr int NCH = RB / 64;      // 16-byte chunks per lane per unit (K, and V)
  constexpr int NDT = D / 16;       // 16-dim tiles of the PV product
  constexpr int UB = kUnit * RB;    // bytes of one 16-token sub-tile
  constexpr int NCH16 = D / 32;     // 16-byte chunks per lane of an FP16 unit (seal-on-full tail)
  static_assert(NB >= 2 && NB <= 3, "units in flight per wavefront");

  const int lane = threadIdx.x & 63;
  // wave-uniform: lets unit indices, table entries, scales and tile addresses
  // live in scalar registers (scalar loads and ALU) instead of every lane
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n16 = lane & 15;
  const int gq = lane >> 4;
  const int part = blockIdx.x;
  const int g = blockIdx.y;
  const int s = blockIdx.z;

  const int T = a.partition_tokens;
  const int t0 = part * T;
  const int u0 = t0 / kUnit;
  const int maxb = a.max_blocks;
  const int hkv = __builtin_amdgcn_readfirstlane(a.lv.num_kv_heads);
  const int bs = __builtin_amdgcn_readfirstlane(a.lv.block_size);
  const int lupb = __builtin_ctz(bs / kUnit);  // log2 units per block (block sizes are powers of two)
  const int hq = a.num_q_heads;
  const int32_t* table = a.tables + (size_t)s * maxb;
  const uint64_t tile_bytes = (uint64_t)bs * RB;
  const char* kcodes = (const char*)a.lv.k_codes;
  const char* vcodes = (const char*)a.lv.v_codes;
  const int upb = 1 << lupb;
  // Wavefront w takes whole blocks: the partition's blocks w, w+4, w+8, ...
  // (partitions start on a block). Its unit i is unit i % upb of its block
  // i / upb, so every unit of a block is read by one wavefront.
  auto unit_of = [&](int i) { return u0 + ((((i >> lupb) * kWaves + wave) << lupb) | (i & (upb - 1))); };

  // ---- start-up: the sequence length, this wavefront's block-table entries
  // (at most 64) and the query all go out before the first wait, none of their
  // addresses depending on another load. Lane i of a wavefront handles its
  // unit i (i < nu). Table reads are clamped to the row, so a lane past the
  // sequence's end reads a valid (unused) entry.
  auto table_entry = [&](int base) { return table[min(unit_of(base + lane) >> lupb, maxb - 1)]; };
  const int raw_len = a.lens[s];
  int tentry = table_entry(0);
  constexpr int QPT = (G * D + kThreads - 1) / kThreads;  // query elements per thread
  float qe[QPT];
#pragma unroll
  for (int k = 0; k < QPT; ++k) {
    const int e = threadIdx.x + k * kThreads;
    const float v = load_elem<QT>(a.q, ((size_t)s * hq + g * G) * D + min(e, G * D - 1));
    qe[k] = e < G * D ? v : 0.f;
  }

  // Lengths beyond what the table or the grid covers are clamped, so a bad
  // length cannot send a load outside the cache or the workspace. A decode
  // step whose length was clamped appends nothing: its new token (position
  // raw_len - 1) lies outside what this launch covers, and writing it at
  // len - 1 would overwrite a cached row.
  const int len = min(raw_len, min(maxb * bs, a.max_partitions * T));
  const bool step_fits = APPEND && raw_len == len;  // wave-uniform (one length per sequence)
  const int t1 = min(len, t0 + T);  // t0 >= len (nothing to do): nu = 0 below
  const int nparts = (len + T - 1) / T;
  const int u1 = (t1 + kUnit - 1) / kUnit;
  const int nblk_full = max(u1 - u0, 0) >> lupb;  // whole blocks of the partition, and units left over
  const int nrem = max(u1 - u0, 0) & (upb - 1);
  const int nu = (nblk_full > wave ? ((nblk_full - wave + kWaves - 1) / kWaves) << lupb : 0) +
                 (nrem > 0 && (nblk_full & (kWaves - 1)) == wave ? nrem : 0);
  // Seal-on-full cache: a partly filled last block of the sequence is still
  // in FP16 (its staging tiles); the wavefront that holds it reads its units
  // (its last ntail units) after the loop, from there. In a decode step the
  // last block also takes the new token: if that fills it, it is sealed in
  // this launch, and the same wavefront takes the whole block after the loop.
  int ntail = 0;
  if constexpr (SEAL) {
    const int r = len & (bs - 1);
    const int nbl = ((len - 1) >> (lupb + 4)) - (u0 >> lupb);  // the last block within the partition
    // (a partition past the sequence's end, t0 >= len, also has t1 == len
    // but holds none of its blocks)
    if (t0 < len && t1 == len && (nbl & (kWaves - 1)) == wave) {
      if (r > 0) ntail = (r + kUnit - 1) / kUnit;
      else if (step_fits) ntail = bs / kUnit;
    }
  }
  const int nu8 = nu - ntail;  // units read through the ring

  // Lane i keeps unit i's block id, its byte offset in the K (and V) codes
  // of the layer and (int8) its scales; the loop reads them with readlane.
  // Scalar loads would put their latency on the loop's path: they can only
  // be awaited all at once. Lanes past nu hold in-bounds values never used.
  int ublk = 0;
  uint32_t usub_lo = 0, usub_hi = 0;
  float uks = 1.f, uvs = 1.f;
  auto set_blocks = [&](int base, int entry) {
    const int u = unit_of(base + lane);
    ublk = min(max(entry, 0), a.lv.num_blocks - 1);  // in-bounds even for a bad entry
    const uint64_t sub = ((uint64_t)ublk * hkv + g) * tile_bytes + (uint64_t)(u & ((1 << lupb) - 1)) * UB;
    usub_lo = (uint32_t)sub;
    usub_hi = (uint32_t)(sub >> 32);
  };
  auto gather_scales = [&]() {
    if constexpr (I8) {
      uks = a.lv.k_scales[(size_t)ublk * hkv + g];
      uvs = a.lv.v_scales[(size_t)ublk * hkv + g];
    }
  };
  // NB-deep ring of K/V buffers: unit i is requested NB units before use.
  // Every slot of the loop issues its loads, also past the last unit: there
  // the buffer descriptor's size is 0, so the loads return zeros without
  // touching memory. With the same number of loads on every path the
  // compiler's wait counts stay exact; a skipped issue on any path would
  // make each wait drain the whole ring.
  uint4 kb[NB][NCH], vb[NB][NCH];
  auto issue = [&](int i, int n, uint4 (&kd)[NCH], uint4 (&vd)[NCH]) {
    const bool live = i < n;
    const int j = min(i, 63);
    const uint64_t sub = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane(usub_hi, j) << 32) |
                         (uint32_t)__builtin_amdgcn_readlane(usub_lo, j);
    const __amdgpu_buffer_rsrc_t kr =
        __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(kcodes + sub), (short)0, live ? UB : 0, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t vr =
        __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(vcodes + sub), (short)0, live ? UB : 0, kRsrcWord3);
    const int ko = n16 * RB + 16 * gq;
    const int vo = lane * (16 * NCH);
    // The loads of a ring slot always leave in the same order (its K, then
    // its V, then the next slot), in the start-up as in the loop: the wait
    // counts the compiler derives on the paths into the loop then agree. The
    // scheduling barriers let ALU and matrix work move across, not memory
    // operations.
    __builtin_amdgcn_sched_barrier(kSchedAluOnly);
#pragma unroll
    for (int c = 0; c < NCH; ++c)
      kd[c] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(kr, ko + 64 * c, 0, 0));
    __builtin_amdgcn_sched_barrier(kSchedAluOnly);
#pragma unroll
    for (int c = 0; c < NCH; ++c)
      vd[c] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(vr, vo + 16 * c, 0, 0));
    __builtin_amdgcn_sched_barrier(kSchedAluOnly);
  };
  // ---- decode step (APPEND): the sequence's last position, len - 1, is the
  // token this step adds. The one wavefront whose units cover its block (the
  // owner) appends it in registers: the block's units reach it through the
  // ring like any others; when it comes to them it re-encodes their old rows
  // if the block's scale grows, puts the new row in, stores the changed
  // 16-byte chunks back and decodes them from its registers. Nothing is read
  // back after those stores, so the owner streams from the start like every
  // other wavefront. Whether the scale grows is decided before the loop from
  // the new row, the block's scale and the largest |code| of its rows. No
  // other wavefront or workgroup reads that block (it is not shared).
  const int pos = len - 1;
  const int nb_rel = (pos >> (lupb + 4)) - (u0 >> lupb);  // the new token's block within the partition
  const int i_new = (nb_rel >> 2) << lupb;  // owner: its unit index of that block's first unit
  const int row0 = pos & (bs - 1);          // the new token's row in its block
  bool owner = step_fits && !SEAL && pos >= t0 && pos < t1 && (nb_rel & (kWaves - 1)) == wave;  // wave-uniform
  int a_entry = 0;
  constexpr int NPL = D / 64;  // new-row elements per lane: dims lane + 64*k
  float nk[NPL], nv[NPL];
  int a_qk = 0, a_qv = 0;
#pragma unroll
  for (int k = 0; k < NPL; ++k) nk[k] = nv[k] = 0.f;
  if constexpr (APPEND) {
    if (owner) {
      a_entry = __builtin_amdgcn_readlane(tentry, i_new);  // i_new < nu <= 64
      owner = a_entry >= 0 && a_entry < a.lv.num_blocks;  // a bad entry is not written
    }
    if (owner) {
      const size_t rowbase = ((size_t)s * hkv + g) * D;
#pragma unroll
      for (int k = 0; k < NPL; ++k) {
        nk[k] = load_elem<QT>(a.k_new, rowbase + lane + 64 * k);
        nv[k] = load_elem<QT>(a.v_new, rowbase + lane + 64 * k);
      }
      if constexpr (I8) {
        a_qk = a.lv.k_qmax[(size_t)a_entry * hkv + g];
        a_qv = a.lv.v_qmax[(size_t)a_entry * hkv + g];
      }
    }
  }

  set_blocks(0, tentry);
  gather_scales();
#pragma unroll
  for (int b = 0; b < NB; ++b) issue(b, nu8, kb[b], vb[b]);


  // ---- the query as the B operand of the QK product (Q^T: dims x columns),
  // built once per workgroup in LDS. Column n16 carries head hc, part pc:
  // int8 K: pc = digit 0..2 of q rounded to a 22-bit integer; fp16 K: pc = 0
  // hi / 1 lo fp16 part of q scaled into [2^14, 2^15). The exponent is per
  // head, from max |q| over its d dims.
  const int hc = I8 ? (n16 & 3) : (n16 & 7);
  const int pc = I8 ? (n16 >> 2) : (n16 >> 3);
  const bool qcol = hc < G && (I8 ? pc < 3 : (pc == 0 || QT == kF32));
  __shared__ __align__(16) uint32_t sm_qb[NCH * 64 * 4];  // [c][lane][16 bytes]
  __shared__ __align__(16) uint32_t sm_qt[SEAL ? NCH16 * 64 * 4 : 4];  // fp16 form (SEAL)
  if constexpr (SEAL) {  // unused column parts must read as zero
    for (int w = threadIdx.x; w < NCH16 * 64 * 4; w += kThreads) sm_qt[w] = 0u;
  }
  __shared__ int sm_hmax[G];
  if (threadIdx.x < G) sm_hmax[threadIdx.x] = 0;
  __syncthreads();
#pragma unroll
  for (int k = 0; k < QPT; ++k) {
    const int e = threadIdx.x + k * kThreads;
    if (e < G * D) atomicMax(&sm_hmax[e / D], __float_as_int(fabsf(qe[k])));  // |q| >= 0: int order
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < QPT; ++k) {
    const int e = threadIdx.x + k * kThreads;
    if (e >= G * D) break;
    const int h = e / D, dim = e % D;
    int qexp;
    frexpf(__int_as_float(sm_hmax[h]), &qexp);  // max = f * 2^qexp, f in [0.5, 1)
    if constexpr (I8) {
      // q * 2^(22 - qexp) rounded: |qi| < 2^22, so qi + 0x808080 holds the three
      // balanced digits (each in [-128, 127]) as biased bytes, no carries.
      const int qi = (int)rintf(ldexpf(qe[k], 22 - qexp));
      const uint32_t z = (uint32_t)(qi + 0x808080);
      const int c = dim >> 6, gql = (dim >> 4) & 3, j = dim & 15;
      unsigned char* b = (unsigned char*)sm_qb;
#pragma unroll
      for (int d = 0; d < 3; ++d)
        b[((c * 64 + gql * 16 + 4 * d + h) << 4) + j] = (unsigned char)(((z >> (8 * d)) & 255u) ^ 0x80u);
      if constexpr (SEAL) {  // the fp16 form too, for the FP16 tail units
        const float y = ldexpf(qe[k], 15 - qexp);
        const _Float16 hi = (_Float16)y;
        const int c16 = dim >> 5, gql16 = (dim >> 3) & 3, j16 = dim & 7;
        _Float16* bt = (_Float16*)sm_qt;
        bt[((c16 * 64 + gql16 * 16 + h) << 3) + j16] = hi;
        if constexpr (QT == kF32) bt[((c16 * 64 + gql16 * 16 + 8 + h) << 3) + j16] = (_Float16)(y - (float)hi);
      }
    } else {
      const float y = ldexpf(qe[k], 15 - qexp);
      const _Float16 hi = (_Float16)y;
      const int c = dim >> 5, gql = (dim >> 3) & 3, j = dim & 7;
      _Float16* b = (_Float16*)sm_qb;
      b[((c * 64 + gql * 16 + h) << 3) + j] = hi;
      if constexpr (QT == kF32) b[((c * 64 + gql * 16 + 8 + h) << 3) + j] = (_Float16)(y - (float)hi);
    }
  }
  __syncthreads();
  // A partition past the sequence's end leaves only here (its K/V requests
  // had size 0). Any earlier exit would let the compiler move the start-up
  // loads behind the branch, each then waited for before the next.
  if (t0 >= len) return;

  // The owner's decision, and the new row's codes in LDS for the lanes that
  // hold that row in the ring: K codes in dim order, V codes as [dm][dt]
  // (dim = 16*dt + dm), V biased like the stored ones. The largest |code| of
  // the old rows after a re-encode is that of the largest old code: the
  // encoding is odd and non-decreasing.
  __shared__ __align__(16) unsigned char sm_new[2][APPEND ? D * ESZ : 16];
  float sk_new = 1.f, sv_new = 1.f, sk_old = 1.f, sv_old = 1.f;
  bool rq_k = false, rq_v = false;
  int qmax_k = 0, qmax_v = 0;
  if constexpr (APPEND) {
    if (owner) {
      auto put = [&](int kv, int dim, uint32_t code) {
        const int at = kv ? (dim & 15) * NDT + (dim >> 4) : dim;
        if constexpr (I8) sm_new[kv][at] = (unsigned char)code;
        else ((uint16_t*)sm_new[kv])[at] = (uint16_t)code;
      };
      if constexpr (I8) {
        sk_old = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, uks), i_new));
        sv_old = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, uvs), i_new));
        auto decide = [&](int kv, const float (&x)[NPL], float s_old, int q_old, float& s_new, bool& rq) {
          float mx = 0.f;
#pragma unroll
          for (int k = 0; k < NPL; ++k) mx = fmaxf(mx, fabsf(x[k]));
          mx = wave_max(mx);
          int qo = 0;
          if (row0 == 0) {
            s_new = scale_of(mx);
          } else if (mx <= (float)q_old * s_old) {
            s_new = s_old;
            qo = q_old;
          } else {
            s_new = scale_of(mx);
            rq = true;
            qo = encode((float)q_old * s_old, s_new);
          }
          int qn = 0;
#pragma unroll
          for (int k = 0; k < NPL; ++k) {
            const int8_t q = encode(x[k], s_new);
            qn = max(qn, abs((int)q));
            put(kv, lane + 64 * k, (uint8_t)q ^ (kv ? 0x80u : 0u));
          }
          return max(qo, wave_max_int(qn));
        };
        qmax_k = decide(0, nk, sk_old, a_qk, sk_new, rq_k);
        qmax_v = decide(1, nv, sv_old, a_qv, sv_new, rq_v);
      } else {
#pragma unroll
        for (int k = 0; k < NPL; ++k) {
          put(0, lane + 64 * k, __builtin_bit_cast(uint16_t, (_Float16)nk[k]));
          put(1, lane + 64 * k, __builtin_bit_cast(uint16_t, (_Float16)nv[k]));
        }
      }
    }
  }

  int qexp;
  frexpf(__int_as_float(sm_hmax[min(hc, G - 1)]), &qexp);
  const float qconst = ldexpf(a.softmax_scale * kLog2e, (I8 ? qexp - 22 : qexp - 15));
  i32x4 qb[I8 ? NCH : 1];
  f16x8 qh[I8 ? 1 : NCH];
  // SEAL: the fp16 operand for tail units, columns as in the FP16 kernel
  // (hi part of head n16 < 8, lo part of head n16 - 8 for an fp32 query)
  f16x8 qt[SEAL ? NCH16 : 1];
  float qconst_t = 0.f;
  if constexpr (SEAL) {
    const int hc16 = n16 & 7, pc16 = n16 >> 3;
    const bool qcol16 = hc16 < G && (pc16 == 0 || QT == kF32);
    int qexp16;
    frexpf(__int_as_float(sm_hmax[min(hc16, G - 1)]), &qexp16);
    qconst_t = ldexpf(a.softmax_scale * kLog2e, qexp16 - 15);
#pragma unroll
    for (int c = 0; c < NCH16; ++c) {
      uint4 w = *(const uint4*)&sm_qt[(c * 64 + lane) * 4];
      if (!qcol16) w = make_uint4(0u, 0u, 0u, 0u);
      qt[c] = __builtin_bit_cast(f16x8, w);
    }
  }
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    uint4 w = *(const uint4*)&sm_qb[(c * 64 + lane) * 4];
    if (!qcol) w = make_uint4(0u, 0u, 0u, 0u);  // columns with no head part
    if constexpr (I8) qb[c] = __builtin_bit_cast(i32x4, w);
    else qh[c] = __builtin_bit_cast(f16x8, w);
  }

  const bool colv = n16 < G;  // this lane's column is a real head (hi / digit 0)
  // Only the real head columns decide when the running max is raised; the
  // other columns of the S^T tile carry partial digits or nothing and are
  // never read. They may hold any value (even inf or NaN): an MFMA output
  // column depends on its own B column only, and P enters the PV product
  // with its hi part cleared in lanes n16 >= 8.
  const uint64_t colmask = __ballot(colv);
  float m = -INFINITY, l = 0.f;
  // P enters the PV product as p * vscale * 2^(14 - kSlack - ev) with ev the
  // largest binary exponent of any V scale seen so far (wave-uniform), which
  // keeps the fp16 parts below 2^14 and their lo part clear of fp16
  // subnormals; the accumulators are rescaled exactly when ev grows and
  // scaled back by 2^(ev + kSlack - 14) at the end. An fp16 cache has no
  // scale: ev stays 0.
  int ev = I8 ? -1000 : 0;
  f32x4 o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One unit of 16 tokens. TAIL: an FP16 unit in an INT8 kernel (a
  // seal-on-full cache's partly filled last block), scored with the fp16
  // query operand and taken with V scale 1; otherwise the kernel's own type.
  auto process = [&](auto tail, const auto& kr, const auto& vr, float kscale, float vscale, int tok0) {
    constexpr bool TAIL = decltype(tail)::value;
    const int nvalid = t1 - tok0;  // rows of this unit inside the partition

    // S^T = K Q^T: lane holds tokens 4*gq + i of column n16
    float sc[4];
    if constexpr (TAIL) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NCH16; ++c)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, kr[c]), qt[c], acc, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x = acc[i];
        if constexpr (QT == kF32) x += dpp_f<kRowShl8>(x);  // + the lo column
        sc[i] = x * qconst_t;
      }
    } else if constexpr (I8) {
      i32x4 acc = {0, 0, 0, 0};
#pragma unroll
      for (int c = 0; c < NCH; ++c)
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, kr[c]), qb[c], acc, 0, 0, 0);
      const float f = kscale * qconst;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c1 = dpp_i<kRowShl4>(acc[i]);   // digit-1 column of this head
        const int c2 = dpp_i<kRowShl8>(acc[i]);   // digit-2 column
        const int t = acc[i] + (c1 << 8);         // exact, |t| < 2^30
        sc[i] = fmaf((float)c2, 65536.f, (float)t) * f;
      }
    } else {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NCH; ++c)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, kr[c]), qh[c], acc, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x = acc[i];
        if constexpr (QT == kF32) x += dpp_f<kRowShl8>(x);  // + the lo column
        sc[i] = x * qconst;
      }
    }

    if (nvalid < kUnit) {  // the partition's last unit: rows past its end (wave-uniform branch)
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[i] = 4 * gq + i < nvalid ? sc[i] : -INFINITY;
    }
    const float lm = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    int evn = ev;
    if constexpr (I8) {
      int ve;
      frexpf(vscale, &ve);  // vscale < 2^ve
      evn = max(ev, __builtin_amdgcn_readfirstlane(ve));  // uniform: one scale per unit
    }
    // m = -inf before the first unit: every finite score raises it
    if ((__ballot(lm > m + kSlack) & colmask) != 0 || evn > ev) {  // wave-uniform
      const float mn = fmaxf(m, max_over_lane_groups(lm));  // + the column's maximum
      const float alpha = __builtin_amdgcn_exp2f(m - mn);
      l *= alpha;
      // lo columns follow their head: lane n16 >= 8 takes lane n16 - 8's alpha.
      // The DPP result is consumed in every lane (lanes n16 < 8 read 0 from
      // outside the row) so it cannot be moved under a lane mask, where a
      // DPP read from a disabled lane would return 0.
      const float ao = (dpp_f<kRowShr8>(alpha) + (n16 < 8 ? alpha : 0.f)) *
                       ldexpf(1.0f, ev - evn);  // exact power of two
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) o[dt] *= ao;
      m = mn;
      ev = evn;
    }

    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(sc[i] - m);  // < 2^kSlack in head columns
    const float lsum = (p[0] + p[1]) + (p[2] + p[3]);
    l += lsum;
    const float pscale = ldexpf(I8 ? vscale : 1.0f, 14 - kSlack - ev);  // p * pscale < 2^14
    f16x4 ph, pl;
#pragma unroll
    for (int i = 0; i < 4; i += 2) {  // the V scale rides on P
      f16x2 h2, l2;
      split_f16x2(p[i] * pscale, p[i + 1] * pscale, h2, l2);
      ph[i] = h2[0];
      ph[i + 1] = h2[1];
      pl[i] = l2[0];
      pl[i + 1] = l2[1];
    }
    // B operand of PV: column n16 < 8 is the hi part of head n16, column
    // 8 + h the lo part of head h (moved over from lane n16 - 8). hi is
    // cleared in lanes 8..15 and the shifted lo is zero in lanes 0..7
    // (outside the row), so OR-ing the bits merges them.
    uint2 hb = __builtin_bit_cast(uint2, ph);
    hb.x = n16 < 8 ? hb.x : 0u;
    hb.y = n16 < 8 ? hb.y : 0u;
    const uint2 lb = __builtin_bit_cast(uint2, pl);
    const f16x4 pb = __builtin_bit_cast(
        f16x4, make_uint2(hb.x | (uint32_t)dpp_i<kRowShr8>((int)lb.x), hb.y | (uint32_t)dpp_i<kRowShr8>((int)lb.y)));

    constexpr int NV = TAIL ? NCH16 : NCH;
    uint32_t vw[4 * NV];
#pragma unroll
    for (int c = 0; c < NV; ++c) {
      vw[4 * c] = vr[c].x; vw[4 * c + 1] = vr[c].y; vw[4 * c + 2] = vr[c].z; vw[4 * c + 3] = vr[c].w;
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      f16x4 av;
      if constexpr (I8 && !TAIL) {
        av = biased_i8x4_to_f16x4(vw[dt]);
      } else {
        av = __builtin_bit_cast(f16x4, make_uint2(vw[2 * dt], vw[2 * dt + 1]));
        if (nvalid < kUnit) {  // rows past the end may hold any bits (NaN included)
#pragma unroll
          for (int j = 0; j < 4; ++j) av[j] = 4 * gq + j < nvalid ? av[j] : (_Float16)0.0f;
        }
      }
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x16f16(av, pb, o[dt], 0, 0, 0);
    }
  };

  // The owner's unit of the new token's block that starts at block row rb
  // (its unit i): old rows re-encoded if the scale grew, the new row put in,
  // and every 16-byte chunk that changed stored back.
  auto patch = [&](uint4 (&kr)[NCH], uint4 (&vr)[NCH], int rb, int i) {
    const uint64_t sub = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane(usub_hi, i) << 32) |
                         (uint32_t)__builtin_amdgcn_readlane(usub_lo, i);
    char* kt = (char*)a.lv.k_codes + sub + n16 * RB + 16 * gq;
    char* vt = (char*)a.lv.v_codes + sub + lane * (16 * NCH);
    // K: this lane holds row rb + n16, bytes 16*gq + 64*c of it
    const int krow = rb + n16;
    bool kst = false;
    if (krow == row0) {
#pragma unroll
      for (int c = 0; c < NCH; ++c) kr[c] = *(const uint4*)&sm_new[0][16 * gq + 64 * c];
      kst = true;
    } else if (I8 && rq_k && krow < row0) {
#pragma unroll
      for (int c = 0; c < NCH; ++c)
        kr[c] = make_uint4(requant_word(kr[c].x, ~0u, sk_old, sk_new, 0u), requant_word(kr[c].y, ~0u, sk_old, sk_new, 0u),
                           requant_word(kr[c].z, ~0u, sk_old, sk_new, 0u), requant_word(kr[c].w, ~0u, sk_old, sk_new, 0u));
      kst = true;
    }
    if (kst) {
#pragma unroll
      for (int c = 0; c < NCH; ++c) *(uint4*)(kt + 64 * c) = kr[c];
    }
    // V: this lane holds rows rb + 4*gq + ti (ti < 4) of dims 16*dt + n16:
    // element 4*dt + ti of its slice
    const int ti0 = row0 - (rb + 4 * gq);  // the new row's ti, when in [0, 4)
    uint32_t vw[4 * NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      vw[4 * c] = vr[c].x; vw[4 * c + 1] = vr[c].y; vw[4 * c + 2] = vr[c].z; vw[4 * c + 3] = vr[c].w;
    }
    bool vst = false;
    if constexpr (I8) {
      if (rq_v && ti0 > 0) {  // its rows below the new one are old
        const uint32_t m = ti0 >= 4 ? ~0u : (1u << (8 * ti0)) - 1u;
#pragma unroll
        for (int w = 0; w < 4 * NCH; ++w) vw[w] = requant_word(vw[w], m, sv_old, sv_new, 0x80808080u);
        vst = true;
      }
      if (ti0 >= 0 && ti0 < 4) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
          vw[dt] = (vw[dt] & ~(0xFFu << (8 * ti0))) | ((uint32_t)sm_new[1][n16 * NDT + dt] << (8 * ti0));
        vst = true;
      }
    } else {
      if (ti0 >= 0 && ti0 < 4) {
        const int sh = 16 * (ti0 & 1);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const int w = 2 * dt + (ti0 >> 1);
          vw[w] = (vw[w] & ~(0xFFFFu << sh)) | ((uint32_t)((const uint16_t*)sm_new[1])[n16 * NDT + dt] << sh);
        }
        vst = true;
      }
    }
    if (vst) {
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        vr[c] = make_uint4(vw[4 * c], vw[4 * c + 1], vw[4 * c + 2], vw[4 * c + 3]);
        *(uint4*)(vt + 16 * c) = vr[c];
      }
    }
  };

  // Decode step on a seal-on-full layer, by the owner of the sequence's last
  // block, after the loop (its streaming starts with everyone else's; staged
  // before the loop, it started several microseconds late): the block's
  // staged rows and the new token's row (binary16, as pkv_append_kv stages
  // it) go to wave-private LDS. If the new row leaves
  // the block partly filled, it is also staged in memory; if it fills the
  // block, the block is sealed as the append does it (scale = max|x| / 127
  // per K and V, codes, largest |code|).
  constexpr int kMaxBs = 64;
  // (two rows in every variant: the seal-on-full code below is compiled, never run, in the others)
  __shared__ __align__(16) uint16_t sm_tail[2][SEAL && APPEND ? kMaxBs * D : 8];
  float seal_sk = 1.f, seal_sv = 1.f;  // scales of a block sealed in this launch
  const int seal_row = (len - 1) & (bs - 1);  // the new token's row in its block
  auto seal_step_stage = [&]() {
    const int blk = min(max(__builtin_amdgcn_readlane(tentry, nu - 1), 0), a.lv.num_blocks - 1);
    const size_t toff = ((size_t)blk * hkv + g) * bs * D;
    uint16_t* tk = (uint16_t*)a.lv.tail_k + toff;
    uint16_t* tv = (uint16_t*)a.lv.tail_v + toff;
    // the new row first, then rows [0, 16 * ntail) of both tiles (prefixes
    // of the tiles), four 16-byte chunks per lane and tile in flight at once
    const size_t rowbase = ((size_t)s * hkv + g) * D;
    float xk[NPL], xv[NPL];
#pragma unroll
    for (int k = 0; k < NPL; ++k) {
      xk[k] = load_elem<QT>(a.k_new, rowbase + lane + 64 * k);
      xv[k] = load_elem<QT>(a.v_new, rowbase + lane + 64 * k);
    }
    const int nchunk = ntail * kUnit * D * 2 / 16;  // 16-byte chunks per tile
    for (int c0 = 0; c0 < nchunk; c0 += 4 * 64) {
      uint4 ck[4], cv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c = min(c0 + 64 * u + lane, nchunk - 1);
        ck[u] = ((const uint4*)tk)[c];
        cv[u] = ((const uint4*)tv)[c];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c = c0 + 64 * u + lane;
        if (c < nchunk) {
          ((uint4*)sm_tail[0])[c] = ck[u];
          ((uint4*)sm_tail[1])[c] = cv[u];
        }
      }
    }
#pragma unroll
    for (int k = 0; k < NPL; ++k) {
      const int dd = lane + 64 * k;
      const uint16_t hk = __builtin_bit_cast(uint16_t, (_Float16)xk[k]);
      const uint16_t hv = __builtin_bit_cast(uint16_t, (_Float16)xv[k]);
      sm_tail[0][k_tile_offset(seal_row, dd, D)] = hk;
      sm_tail[1][v_tile_offset(seal_row, dd, D)] = hv;
      if (seal_row < bs - 1) {
        tk[k_tile_offset(seal_row, dd, D)] = hk;
        tv[v_tile_offset(seal_row, dd, D)] = hv;
      }
    }
    if (seal_row < bs - 1) return;
    // seal: per K and V, the scale from the block's largest |x|
    float mk = 0.f, mv = 0.f;
    for (int e = lane; e < bs * D; e += 64) {
      mk = fmaxf(mk, fabsf(f16_to_f32(sm_tail[0][e])));
      mv = fmaxf(mv, fabsf(f16_to_f32(sm_tail[1][e])));
    }
    seal_sk = scale_of(wave_max(mk));
    seal_sv = scale_of(wave_max(mv));
    int8_t* ck = (int8_t*)a.lv.k_codes + toff;
    int8_t* cv = (int8_t*)a.lv.v_codes + toff;
    int qk = 0, qv = 0;
    for (int e = lane; e < bs * D; e += 64) {  // element e of each tile, in its layout
      const int8_t xk = encode(f16_to_f32(sm_tail[0][e]), seal_sk);
      const int8_t xv = encode(f16_to_f32(sm_tail[1][e]), seal_sv);
      qk = max(qk, abs((int)xk));
      qv = max(qv, abs((int)xv));
      ck[e] = xk;
      cv[e] = (int8_t)(xv ^ (int8_t)0x80);  // V codes are stored biased by 128
    }
    qk = wave_max_int(qk);
    qv = wave_max_int(qv);
    if (lane == 0) {
      const size_t at = (size_t)blk * hkv + g;
      a.lv.k_scales[at] = seal_sk;
      a.lv.v_scales[at] = seal_sv;
      a.lv.k_qmax[at] = qk;
      a.lv.v_qmax[at] = qv;
    }
  };
  // Decode step on a seal-on-full layer, after the loop: the last block's
  // units, staged in LDS just before, in the order a decode of the
  // appended cache takes them: as FP16, or from the codes of a block sealed
  // in this launch.
  auto seal_step_decode = [&]() {
    if (seal_row < bs - 1) {
      for (int j = 0; j < ntail; ++j) {
        uint4 kr[NCH16], vr[NCH16];
#pragma unroll
        for (int c = 0; c < NCH16; ++c) {
          kr[c] = *(const uint4*)((const char*)sm_tail[0] + (size_t)(kUnit * j + n16) * D * 2 + 16 * gq + 64 * c);
          vr[c] = *(const uint4*)((const char*)sm_tail[1] + (size_t)j * kUnit * D * 2 + lane * (16 * NCH16) + 16 * c);
        }
        process(std::true_type{}, kr, vr, 1.f, 1.f, unit_of(nu8 + j) * kUnit);
      }
      return;
    }
    // the sealed block's units as INT8, in the ring's register layout
    for (int j = 0; j < ntail; ++j) {
      uint4 kd[NCH], vd[NCH];
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        uint32_t kw[4], vw[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          uint32_t x = 0, y = 0;
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const int dk = 16 * gq + 64 * c + 4 * w + b;  // K row kUnit * j + n16, this dim
            const int ve = j * kUnit * D + lane * (16 * NCH) + 16 * c + 4 * w + b;  // V element
            x |= (uint32_t)(uint8_t)encode(f16_to_f32(sm_tail[0][(kUnit * j + n16) * D + dk]), seal_sk) << (8 * b);
            y |= (uint32_t)(uint8_t)(encode(f16_to_f32(sm_tail[1][ve]), seal_sv) ^ (int8_t)0x80) << (8 * b);
          }
          kw[w] = x;
          vw[w] = y;
        }
        kd[c] = make_uint4(kw[0], kw[1], kw[2], kw[3]);
        vd[c] = make_uint4(vw[0], vw[1], vw[2], vw[3]);
      }
      process(std::false_type{}, kd, vd, seal_sk, seal_sv, unit_of(nu8 + j) * kUnit);
    }
  };
  // The scales reach the loop through a register move the compiler cannot
  // see into: it waits once for their loads here, and the loop's readlanes
  // then carry no wait. (Otherwise, where the scales' registers were
  // written along several paths, it kept them pending and drained the ring
  // at every unit.)
  if constexpr (I8) {
    asm volatile("v_mov_b32 %0, %1" : "=v"(uks) : "v"(uks));
    asm volatile("v_mov_b32 %0, %1" : "=v"(uvs) : "v"(uvs));
  }
  // At most 64 units per wavefront (partitions of at most kMaxPartition
  // tokens): lane i's bookkeeping covers every unit. A slot past the last
  // unit still consumes its (zero-size) loads, so that every path through
  // the loop leaves the same loads outstanding and the compiler's wait
  // counts stay exact.
  for (int i0 = 0; i0 < nu8; i0 += NB) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int i = i0 + b;
      if (i < nu8) {
        float ks = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, uks), i));
        float vs = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, uvs), i));
        if constexpr (APPEND) {
          if (owner && i >= i_new) {  // a unit of the new token's block (wave-uniform)
            patch(kb[b], vb[b], (i - i_new) * kUnit, i);
            ks = sk_new;
            vs = sv_new;
          }
        }
        process(std::false_type{}, kb[b], vb[b], ks, vs, unit_of(i) * kUnit);
      } else {
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
          asm volatile("" ::"v"(kb[b][c].x), "v"(kb[b][c].y), "v"(kb[b][c].z), "v"(kb[b][c].w));
          asm volatile("" ::"v"(vb[b][c].x), "v"(vb[b][c].y), "v"(vb[b][c].z), "v"(vb[b][c].w));
        }
      }
      issue(i + NB, nu8, kb[b], vb[b]);
    }
  }

  if constexpr (APPEND && I8 && !SEAL) {  // the new token's block: its scales and largest codes
    if (owner && lane == 0) {
      const size_t at = (size_t)a_entry * hkv + g;
      a.lv.k_scales[at] = sk_new;
      a.lv.v_scales[at] = sv_new;
      a.lv.k_qmax[at] = qmax_k;
      a.lv.v_qmax[at] = qmax_v;
    }
  }

  if constexpr (SEAL && APPEND) {
    if (ntail > 0 && step_fits) {  // wave-uniform
      seal_step_stage();
      seal_step_decode();
    }
  }
  if constexpr (SEAL) {
    if (ntail > 0 && !step_fits) {  // wave-uniform: the FP16 tail, after the INT8 units
      const int blk = min(max(__builtin_amdgcn_readlane(tentry, nu - 1), 0), a.lv.num_blocks - 1);
      const size_t tile16 = (size_t)bs * D * 2;
      const char* tk = (const char*)a.lv.tail_k + ((size_t)blk * hkv + g) * tile16;
      const char* tv = (const char*)a.lv.tail_v + ((size_t)blk * hkv + g) * tile16;
      for (int j = 0; j < ntail; ++j) {
        uint4 kr[NCH16], vr[NCH16];
#pragma unroll
        for (int c = 0; c < NCH16; ++c) {
          kr[c] = *(const uint4*)(tk + (size_t)(kUnit * j + n16) * D * 2 + 16 * gq + 64 * c);
          vr[c] = *(const uint4*)(tv + (size_t)j * kUnit * D * 2 + lane * (16 * NCH16) + 16 * c);
        }
        process(std::true_type{}, kr, vr, 1.f, 1.f, unit_of(nu8 + j) * kUnit);
      }
    }
  }

  // hi + lo columns, back to unit scale; l summed over the four lane groups
  const float oscale = ldexpf(1.0f, ev + kSlack - 14);
  l = sum_over_lane_groups(l);
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) o[dt][i] = (o[dt][i] + dpp_f<kRowShl8>(o[dt][i])) * oscale;

  __shared__ float sm_o[kWaves][G][D];
  __shared__ float sm_m[kWaves][G];
  __shared__ float sm_l[kWaves][G];
  __shared__ int sm_last;
  if (colv) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) sm_o[wave][n16][16 * dt + 4 * gq + i] = o[dt][i];
    if (gq == 0) { sm_m[wave][n16] = m; sm_l[wave][n16] = l; }
  }
  __syncthreads();

  const size_t pmax = a.max_partitions;
  const size_t nrow = (size_t)a.num_seqs * hq * pmax;
  float* ws_m = a.ws;
  float* ws_l = a.ws + nrow;
  float* ws_o = a.ws + 2 * nrow;
  for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
    const int j = idx / D;
    const int dd = idx % D;
    float M = sm_m[0][j];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sm_m[w][j]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float wt = __builtin_amdgcn_exp2f(sm_m[w][j] - M);  // idle wave: exp2(-inf) = 0
      L = fmaf(wt, sm_l[w][j], L);
      O = fmaf(wt, sm_o[w][j][dd], O);
    }
    const int h = g * G + j;
    if (nparts == 1) {
      a.out[((size_t)s * hq + h) * D + dd] = O / L;
    } else {
      // Partials are stored as device-scope atomics (written through to the
      // point of coherence shared by all XCDs), so the workgroup that merges
      // them needs no cache write-back or invalidate, which would cost every
      // workgroup a pass over its XCD's L2.
      const size_t slot = ((size_t)s * hq + h) * pmax + part;
      __hip_atomic_store(&ws_o[slot * D + dd], O / L, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (dd == 0) {
        __hip_atomic_store(&ws_m[slot], M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&ws_l[slot], L, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  if (nparts == 1 || !a.fused_merge) return;

  // ---- last arrival of this (sequence, KV head) merges every partition.
  // Every thread waits until its partial stores have completed before the
  // workgroup barrier; only then does one thread count the arrival.
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  if (threadIdx.x == 0)
    sm_last = __hip_atomic_fetch_add(&a.counters[(size_t)s * hkv + g], 1, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT) == nparts - 1;
  __syncthreads();
  if (!sm_last) return;
  for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
    const int j = idx / D;
    const int dd = idx % D;
    const size_t base = ((size_t)s * hq + g * G + j) * pmax;
    float M = -INFINITY, L = 0.f, O = 0.f;
    for (int p0 = 0; p0 < nparts; p0 += 16) {  // 16 partitions' loads in flight at a time
      float pm[16], pl[16], po[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const bool ok = p0 + k < nparts;
        const size_t r = base + (ok ? p0 + k : 0);
        const float vm = __hip_atomic_load(&ws_m[r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const float vl = __hip_atomic_load(&ws_l[r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const float vo = __hip_atomic_load(&ws_o[r * D + dd], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        pm[k] = ok ? vm : -INFINITY;
        pl[k] = ok ? vl : 0.f;
        po[k] = ok ? vo : 0.f;
      }
      float Mn = M;
#pragma unroll
      for (int k = 0; k < 16; ++k) Mn = fmaxf(Mn, pm[k]);
      const float r = __builtin_amdgcn_exp2f(M - Mn);  // M = -inf on the first chunk: 0
      L *= r;
      O *= r;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const float w = __builtin_amdgcn_exp2f(pm[k] - Mn) * pl[k];
        L += w;
        O = fmaf(w, po[k], O);
      }
      M = Mn;
    }
    a.out[((size_t)s * hq + g * G + j) * D + dd] = O / L;
  }
  if (threadIdx.x == 0)  // ready for the next call
    __hip_atomic_store(&a.counters[(size_t)s * hkv + g], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Both variants fit in 168 registers with their K/V rings: three wavefronts
// (three workgroups) per SIMD pair of registers budget, i.e. 768 resident
// workgroups on 256 CUs.
template <int D, int G, int QT, bool APPEND, bool SEAL = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3, 8)))
void decode_kernel_i8(const DecodeLaunch a) {
  decode_body<true, D, G, QT, APPEND, SEAL, 3>(a);
}
// The INT8 decode step for grids larger than the device holds at once: two
// units in flight per wavefront instead of three, which fits the step in 128
// registers, so four wavefronts share a SIMD (1024 resident workgroups
// instead of 768) with as many units in flight per SIMD. Measured per launch
// against the three-deep kernel: serving batch of 128 at bs 16 31.6 vs
// 36.4 us, 128-sequence mix 32.9 vs 33.7 us, long context 114.4 vs 115.6 us;
// with one workgroup per compute unit (Qwen3-TTS shape) 17.12 vs 17.06 us,
// so that grid keeps the three-deep kernel.
template <int D, int G, int QT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 8)))
void decode_step_kernel_i8_many(const DecodeLaunch a) {
  decode_body<true, D, G, QT, true, false, 2>(a);
}
template <int D, int G, int QT, bool APPEND>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3, 8)))
void decode_kernel_f16(const DecodeLaunch a) {
  decode_body<false, D, G, QT, APPEND, false, 2>(a);
}

// ---------------------------------------------------------------------------
// H3 as its own launch: merge the partitions of each (sequence, query head):
//   M = max_p m_p,  w_p = l_p * 2^(m_p - M),  out = sum_p w_p o_p / sum_p w_p
// where o_p is the partition's normalised output and m_p its base-2 maximum.
// The partials are a few KB per row, so the merge is bound by memory latency:
// one 256-thread workgroup per row takes the partitions CHUNK (16, 32 or 64,
// the least that covers max_partitions) at a time, with every load of a
// chunk in flight at once. Wavefront 0 loads the chunk's m and l (lane =
// partition) and puts the weights in LDS; thread t
// loads dim t % D of partitions t / D, t / D + S, ... (S = 256 / D slices).
// The first chunk's loads leave before the sequence length is known (they
// stay inside the row's max_partitions slots; partitions past the sequence's
// get weight 0). The slices' sums are added through LDS at the end.
// ---------------------------------------------------------------------------
constexpr int kMergeThreads = 256;

template <int D, int CHUNK>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(const DecodeLaunch a) {
  static_assert(CHUNK <= 64, "one partition per lane of wavefront 0");
  constexpr int S = kMergeThreads / D;
  constexpr int NO = CHUNK / S;  // o values per thread and chunk
  const int hq = a.num_q_heads;
  const int s = blockIdx.x / hq;
  const int h = blockIdx.x % hq;
  const int pmax = a.max_partitions;
  const size_t nrow = (size_t)a.num_seqs * hq * pmax;
  const float* ws_m = a.ws;
  const float* ws_l = a.ws + nrow;
  const float* ws_o = a.ws + 2 * nrow;
  const size_t base = ((size_t)s * hq + h) * pmax;
  const int t = threadIdx.x;
  const int dd = t % D;
  const int slice = t / D;
  const int T = a.partition_tokens;
  const int len = min(a.lens[s], min(a.max_blocks * a.lv.block_size, pmax * T));
  const int nparts = (len + T - 1) / T;

  __shared__ float sm_w[CHUNK];
  __shared__ float sm_mn;
  float M = -INFINITY, L = 0.f, O = 0.f;  // L: wavefront 0 only
  for (int c0 = 0; c0 < pmax; c0 += CHUNK) {
    float ov[NO];
#pragma unroll
    for (int k = 0; k < NO; ++k) ov[k] = ws_o[(base + min(c0 + slice + k * S, pmax - 1)) * D + dd];
    float mv = -INFINITY, lv = 0.f;
    if (t < CHUNK) {
      const int p = min(c0 + t, pmax - 1);
      mv = ws_m[base + p];
      lv = ws_l[base + p];
    }
    if (nparts <= 1) return;  // (uniform) one partition: the decode kernel wrote the output
    if (c0 >= nparts) break;  // (uniform) nothing more to merge
    if (t < 64) {  // wavefront 0
      const bool live = t < CHUNK && c0 + t < nparts;
      const float Mn = fmaxf(M, wave_max(live ? mv : -INFINITY));
      const float w = live ? __builtin_amdgcn_exp2f(mv - Mn) * lv : 0.f;
      float ws = w;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) ws += __shfl_xor(ws, off);
      L = L * __builtin_amdgcn_exp2f(M - Mn) + ws;  // M = -inf on the first chunk: 0
      if (t < CHUNK) sm_w[t] = w;
      if (t == 0) sm_mn = Mn;
    }
    __syncthreads();
    const float Mn = sm_mn;
    O *= __builtin_amdgcn_exp2f(M - Mn);
#pragma unroll
    for (int k = 0; k < NO; ++k)  // slots past nparts may hold anything from earlier calls
      O = fmaf(sm_w[slice + k * S], c0 + slice + k * S < nparts ? ov[k] : 0.f, O);
    M = Mn;
    __syncthreads();  // sm_w and sm_mn are rewritten by the next chunk
  }
  __shared__ float sm_o[S][D];
  __shared__ float sm_l;
  sm_o[slice][dd] = O;
  if (t == 0) sm_l = L;
  __syncthreads();
  if (slice != 0) return;
  float Ot = 0.f;
#pragma unroll
  for (int k = 0; k < S; ++k) Ot += sm_o[k][dd];
  a.out[((size_t)s * hq + h) * D + dd] = Ot / sm_l;
}


template <int D>
void launch_merge(const DecodeLaunch& d, int chunk, dim3 grid, hipStream_t stream) {
  if (chunk == 16)
    hipLaunchKernelGGL((merge_kernel<D, 16>), grid, dim3(kMergeThreads), 0, stream, d);
  else if (chunk == 32)
    hipLaunchKernelGGL((merge_kernel<D, 32>), grid, dim3(kMergeThreads), 0, stream, d);
  else
    hipLaunchKernelGGL((merge_kernel<D, 64>), grid, dim3(kMergeThreads), 0, stream, d);
}

template <bool I8, int D, int G, int QT>
void launch_one(const DecodeLaunch& d, hipStream_t stream) {
  const dim3 grid(d.max_partitions, d.lv.num_kv_heads, d.num_seqs);
  const bool step = d.k_new != nullptr;
  if constexpr (I8) {
    if (step && d.lv.seal)
      hipLaunchKernelGGL((decode_kernel_i8<D, G, QT, true, true>), grid, dim3(kThreads), 0, stream, d);
    else if (step && (int64_t)grid.x * grid.y * grid.z > 3LL * device_compute_units())  // more than one round
      hipLaunchKernelGGL((decode_step_kernel_i8_many<D, G, QT>), grid, dim3(kThreads), 0, stream, d);
    else if (step)
      hipLaunchKernelGGL((decode_kernel_i8<D, G, QT, true>), grid, dim3(kThreads), 0, stream, d);
    else if (d.lv.seal)
      hipLaunchKernelGGL((decode_kernel_i8<D, G, QT, false, true>), grid, dim3(kThreads), 0, stream, d);
    else
      hipLaunchKernelGGL((decode_kernel_i8<D, G, QT, false>), grid, dim3(kThreads), 0, stream, d);
  } else {
    if (step)
      hipLaunchKernelGGL((decode_kernel_f16<D, G, QT, true>), grid, dim3(kThreads), 0, stream, d);
    else
      hipLaunchKernelGGL((decode_kernel_f16<D, G, QT, false>), grid, dim3(kThreads), 0, stream, d);
  }
}

template <bool I8, int D, int G>
hipError_t launch_decode_q(const DecodeLaunch& d, hipStream_t stream) {
  switch (d.q_dtype) {
    case kF32: launch_one<I8, D, G, kF32>(d, stream); break;
    case kF16: launch_one<I8, D, G, kF16>(d, stream); break;
    case kBF16: launch_one<I8, D, G, kBF16>(d, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool I8, int D>
hipError_t launch_decode_g(const DecodeLaunch& d, int group, hipStream_t stream) {
  switch (group) {
    case 1: return launch_decode_q<I8, D, 1>(d, stream);
    case 2: return launch_decode_q<I8, D, 2>(d, stream);
    case 4: return launch_decode_q<I8, D, 4>(d, stream);
    default: return hipErrorInvalidValue;
  }
}

// ---------------------------------------------------------------------------
// Chunked prefill ("轻量级推理引擎实战" §一: prefill handles a prompt's tokens in
// parallel): each sequence's last q_len cached tokens are queries; query i
// sits at position p = len - q_len + i and attends to positions 0..p.
//
// A tile is 16 matrix-core columns = 16/G query tokens x the G query heads of
// one KV head. A workgroup takes NW (4 or 8) consecutive tiles of one
// sequence and KV head, one per wavefront, and streams that head's context
// through them in steps of two 16-token units (A, B). Its wavefronts read the
// same units, so the workgroup loads each once: every thread requests 16-byte pieces of a
// step into registers three steps ahead and writes them into a three-slot LDS
// ring as binary16 (INT8 codes convert exactly; the block scales stay factors
// of the scores and of P). Per step and wavefront:
//   S^T[token][col] = K[token][:] . Q^T[:][col]   per unit (fp16 products, fp32 sums)
//   O^T[dim][col]  += V^T[dim][k] . P^T[k][col]   over the step's 32 tokens, P as
//                                                 fp16 hi + lo parts
// Lane (column n16, group gq) holds dims [gq*D/4, (gq+1)*D/4) of its column's
// query and of K row n16; QK product c contracts elements [8c, 8c+8) of every
// lane's range, on both sides. The scores leave QK with lane (n16, gq) holding
// tokens 4gq..4gq+3 of each unit, so the PV products take contraction index
// 8gq + j as token 4gq + j of unit A (j < 4) or 4gq + j - 4 of unit B: P^T
// needs no data movement, and the LDS ring keeps each lane's four V rows of A
// and of B side by side per dim tile. The query is scaled per column by a
// power of two into fp16 (a lo part too for an fp32 query). Scores are in
// base 2; each column keeps a running max that may trail the true maximum by
// up to kSlack and is raised (the accumulators rescaled) only when a score
// exceeds it by more.
//
// The loop is software-pipelined: a wavefront issues the QK products of step
// st + 1 before the softmax of step st, so its vector ALU work overlaps the
// matrix-core queue; the ring holds step st (V), st + 1 (K) and st + 2 (being
// written).
//
// Workgroups are numbered so that the tiles of one (sequence, KV head) pair
// run on one XCD, whose L2 then serves the pair's context to all of them
// (consecutive workgroup ids go to the eight XCDs in turn), and so that on each
// XCD the tiles with the longest context start first.
// ---------------------------------------------------------------------------
template <bool I8, int D, int G, int QT, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 8)))
void prefill_kernel(const PrefillLaunch a) {
  constexpr int NT = 64 * NW;               // threads
  constexpr int TQ = 16 / G;                // query tokens per tile
  constexpr int ESZ = I8 ? 1 : 2;           // bytes per cached element
  constexpr int NK = D / 32;                // 16-byte binary16 pieces of a K row per lane
  constexpr int NDT = D / 16;               // 16-dim tiles of the PV product
  constexpr int QE = D / 4;                 // query, K and V elements per lane
  constexpr int GB = kUnit * D * ESZ;       // cache bytes of a unit's K (or V)
  constexpr int NCH = 2 * GB / 16;          // 16-byte cache pieces per unit, K and V together
  constexpr int SP = 2 * NCH;               // pieces per step
  constexpr int CPS = (SP + NT - 1) / NT;   // pieces per thread per step
  constexpr int PE = 16 / ESZ;              // elements per piece
  constexpr int RP = 2 * D + 16;            // LDS pitch of a binary16 K row (padded against bank conflicts)
  constexpr int VP = 16 * NDT + 16;         // LDS pitch of a lane's V operands
  constexpr int KS = kUnit * RP;            // LDS bytes of a unit's K rows
  constexpr int SS = 2 * KS + 64 * VP;      // LDS bytes of a step: K rows of A, of B, then V
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n16 = lane & 15, gq = lane >> 4;
  const int hq = a.num_q_heads, hkv = a.lv.num_kv_heads, bs = a.lv.block_size;

  // workgroup -> (pair, tile group); XCD x runs ids x, x + 8, ... and takes
  // the x-th contiguous stretch of pair-major, longest-first order
  const int ngroups = ((a.max_query_len + TQ - 1) / TQ + NW - 1) / NW;
  const int nwg = gridDim.x, xcd = blockIdx.x & 7, base = nwg >> 3, rem = nwg & 7;
  const int jo = xcd * base + min(xcd, rem) + (blockIdx.x >> 3);
  const int pair = jo / ngroups, grp = ngroups - 1 - jo % ngroups;
  const int g = pair % hkv, s = pair / hkv;

  const int lupb = __builtin_ctz(bs / kUnit);
  const int qs = a.query_start[s];
  const int ql = min(a.query_start[s + 1] - qs, a.max_query_len);
  const int len = min(a.lens[s], a.max_blocks * bs);
  const int jw = grp * NW * TQ;        // first query of the workgroup's tiles
  if (jw >= ql || ql > len) return;    // the whole workgroup (no barrier passed yet)
  const int j0 = jw + wave * TQ;       // this wavefront's tile (may lie past the chunk)

  // lane column n16: query j0 + n16 / G, head n16 % G. A column past the
  // chunk computes over the whole context (its query is zero) and is not
  // written.
  const int qi = j0 + n16 / G, h = n16 % G;
  const bool colv = qi < ql;
  const int pos = colv ? len - ql + qi : len - 1;  // last position the column sees
  const int pmin = len - ql + j0;                  // the tile's first query position
  const int p_wave = j0 < ql ? len - ql + min(j0 + TQ, ql) - 1 : -1;  // last position the tile sees
  const int nunits = (len - ql + min(jw + NW * TQ, ql) - 1) / kUnit + 1;  // units the workgroup reads
  const int nsteps = (nunits + 1) / 2;
  const int vlim = min(len, nunits * kUnit);       // rows from here on are not staged or not cached

  // ---- query operand (B of QK): D/4 elements per lane, fp16 hi (+ lo)
  f16x8 qh[NK], ql8[QT == kF32 ? NK : 1];
  float qconst;
  {
    float qv[QE];
    const size_t qrow = ((size_t)(qs + (colv ? qi : 0)) * hq + g * G + h) * D + gq * QE;
#pragma unroll
    for (int e = 0; e < QE; ++e) qv[e] = colv ? load_elem<QT>(a.q, qrow + e) : 0.f;
    float qm = 0.f;
#pragma unroll
    for (int e = 0; e < QE; ++e) qm = fmaxf(qm, fabsf(qv[e]));
    qm = max_over_lane_groups(qm);  // the column's max |q|
    int qexp;
    frexpf(qm, &qexp);              // qm < 2^qexp (0 for a zero column)
#pragma unroll
    for (int c = 0; c < NK; ++c) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float y = ldexpf(qv[8 * c + e], 15 - qexp);
        const _Float16 hi = (_Float16)y;
        qh[c][e] = hi;
        if constexpr (QT == kF32) ql8[c][e] = (_Float16)(y - (float)hi);
      }
    }
    qconst = ldexpf(a.softmax_scale * kLog2e, qexp - 15);  // > 0
  }

  // ---- the unit stream. Every request issues the same vector loads (steps
  // past the end reload the last unit), so that the waits for a step's data
  // count precisely and leave the later requests in flight: block-table
  // entries of step x are loaded right after the pieces of step x - 3, and
  // step x's pieces (and INT8 scales) three steps before it is staged.
  const int32_t* table = a.tables + (size_t)s * a.max_blocks;
  const char* kcodes = (const char*)a.lv.k_codes;
  const char* vcodes = (const char*)a.lv.v_codes;
  const uint64_t tile_bytes = (uint64_t)bs * D * ESZ;
  auto table_entry = [&](int x) {  // lane j = 0, 1: the block of unit 2x + j
    const int u = min(2 * x + (lane & 1), nunits - 1);
    return table[u >> lupb];
  };
  auto piece = [&](int c, int& V, int& o) {  // unit and byte of this thread's piece c of a step
    if constexpr (NCH % NT == 0) {  // a thread's pieces of one unit: the unit index is static
      V = NT * c / NCH;
      o = 16 * ((NT * c) % NCH + (int)threadIdx.x);
    } else {
      const int q = min((int)threadIdx.x + NT * c, SP - 1);
      V = q / NCH;
      o = 16 * (q % NCH);
    }
  };
  int tq[3];                 // table entries of the next requests, by step % 3
  i32x4 ring[3][CPS];        // requested steps' pieces, by step % 3
  float rsc[3];              // and their scales: lane 0/1 K scale of unit A/B, lane 2/3 V scale
  auto request = [&](int st, auto r) {  // wave-uniform st; r = st % 3
    const int ba = min(max(__builtin_amdgcn_readlane(tq[r], 0), 0), a.lv.num_blocks - 1);
    const int bb = min(max(__builtin_amdgcn_readlane(tq[r], 1), 0), a.lv.num_blocks - 1);
#pragma unroll
    for (int c = 0; c < CPS; ++c) {
      int V, o;  // piece NT * c + threadIdx.x of the step: unit V, byte o of its K (o < GB) or V
      piece(c, V, o);
      const int u = min(2 * st + V, nunits - 1);
      const uint64_t sub =
          ((uint64_t)(V == 0 ? ba : bb) * hkv + g) * tile_bytes + (uint64_t)(u & ((1 << lupb) - 1)) * GB;
      ring[r][c] = *(const i32x4*)(o < GB ? kcodes + sub + o : vcodes + sub + (o - GB));
    }
    if constexpr (I8) {
      const float* sp = (lane & 2) ? a.lv.v_scales : a.lv.k_scales;
      rsc[r] = sp[(size_t)((lane & 1) ? bb : ba) * hkv + g];
    }
    tq[r] = table_entry(st + 3);
  };
  __shared__ __align__(16) unsigned char lds[3][SS];
  float sks[3][2], svs[3][2];  // scales of the steps in the LDS slots
  auto stage = [&](int st, auto slot) {  // the requested step st -> LDS slot st % 3, as binary16
    static_for<2>([&](auto V) {
      sks[slot][V] = 1.f;
      svs[slot][V] = 1.f;
      if constexpr (I8) {
        if (2 * st + V < nunits) {
          sks[slot][V] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, rsc[slot]), V));
          svs[slot][V] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, rsc[slot]), 2 + V));
        }
      }
    });
#pragma unroll
    for (int c = 0; c < CPS; ++c) {
      if (SP % NT != 0 && (int)threadIdx.x + NT * c >= SP) continue;
      int V, o;
      piece(c, V, o);
      if (2 * st + V >= nunits) continue;  // the last step of an odd count has no unit B
      {
        const bool isk = o < GB;
        const int e = (isk ? o : o - GB) / ESZ;  // first element of the piece within K (V)
        const i32x4 w = ring[slot][c];
        f16x4 x[PE / 4];
        if constexpr (I8) {  // 16 codes -> 16 binary16 values (K signed, V stored biased)
          const uint32_t flip = isk ? 0x80808080u : 0u;
#pragma unroll
          for (int k = 0; k < 4; ++k) x[k] = biased_i8x4_to_f16x4((uint32_t)w[k] ^ flip);
        } else {
          x[0] = __builtin_bit_cast(f16x4, make_uint2(w[0], w[1]));
          x[1] = __builtin_bit_cast(f16x4, make_uint2(w[2], w[3]));
        }
        unsigned char* sl = lds[slot];
        if (isk) {  // K row e / D, elements e % D ..
          unsigned char* dst = sl + V * KS + (e / D) * RP + 2 * (e % D);
#pragma unroll
          for (int k = 0; k < PE / 8; ++k)
            *(f16x8*)(dst + 16 * k) = f16x8{x[2 * k][0], x[2 * k][1], x[2 * k][2], x[2 * k][3],
                                            x[2 * k + 1][0], x[2 * k + 1][1], x[2 * k + 1][2], x[2 * k + 1][3]};
        } else {  // lane e / QE's V elements: four per dim tile, unit A's then unit B's
          unsigned char* dst = sl + 2 * KS + (e / QE) * VP + 4 * (e % QE) + 8 * V;
#pragma unroll
          for (int k = 0; k < PE / 4; ++k) *(f16x4*)(dst + 16 * k) = x[k];
        }
      }
    }
  };

  float m = -INFINITY, l = 0.f;
  // P enters the PV product as p * vscale * 2^(14 - kSlack - ev), ev the
  // largest binary exponent of any V scale so far (uniform): the fp16 hi and
  // lo parts stay below 2^14 and clear of fp16 subnormals however small the
  // scales. The accumulators are rescaled exactly when ev grows and scaled
  // back by 2^(ev + kSlack - 14) at the end. A binary16 cache has no scale:
  // ev stays 0.
  int ev = I8 ? -1000 : 0;
  f32x4 o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // S^T of step st (LDS slot), both units
  auto qk = [&](int st, auto slot, f32x4& sa, f32x4& sb) {
    const unsigned char* sl = lds[slot];
    f16x8 ka[NK], kb[NK];
#pragma unroll
    for (int c = 0; c < NK; ++c) {
      ka[c] = *(const f16x8*)&sl[n16 * RP + gq * (2 * QE) + 16 * c];
      kb[c] = *(const f16x8*)&sl[KS + n16 * RP + gq * (2 * QE) + 16 * c];
    }
    sa = f32x4{0.f, 0.f, 0.f, 0.f};
    sb = sa;
#pragma unroll
    for (int c = 0; c < NK; ++c) {
      sa = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[c], qh[c], sa, 0, 0, 0);
      sb = __builtin_amdgcn_mfma_f32_16x16x32_f16(kb[c], qh[c], sb, 0, 0, 0);
      if constexpr (QT == kF32) {
        sa = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[c], ql8[c], sa, 0, 0, 0);
        sb = __builtin_amdgcn_mfma_f32_16x16x32_f16(kb[c], ql8[c], sb, 0, 0, 0);
      }
    }
  };

  // softmax of step st from its scores, then O += V^T P^T
  auto softmax_pv = [&](int st, auto slot, f32x4 sa, f32x4 sb) {
    const int t0 = st * 2 * kUnit;  // the step's first token
    const unsigned char* vl = &lds[slot][2 * KS + lane * VP];
    f16x8 av[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) av[dt] = *(const f16x8*)&vl[16 * dt];
    const float fa = sks[slot][0] * qconst, fb = sks[slot][1] * qconst;
    if (t0 + 2 * kUnit - 1 > pmin) {  // some column does not see the whole step (wave-uniform)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sa[i] = t0 + 4 * gq + i <= pos ? sa[i] : -INFINITY;
        sb[i] = t0 + kUnit + 4 * gq + i <= pos ? sb[i] : -INFINITY;
      }
    }
    if (t0 + 2 * kUnit > vlim) {  // rows not staged, or past the context, may hold any bits
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          av[dt][j] = t0 + 4 * gq + j < vlim ? av[dt][j] : (_Float16)0.0f;
          av[dt][4 + j] = t0 + kUnit + 4 * gq + j < vlim ? av[dt][4 + j] : (_Float16)0.0f;
        }
    }
    // scales are positive: the max of the raw sums times the scale is the max score
    const float lm = fmaxf(fmaxf(fmaxf(sa[0], sa[1]), fmaxf(sa[2], sa[3])) * fa,
                           fmaxf(fmaxf(sb[0], sb[1]), fmaxf(sb[2], sb[3])) * fb);
    int evn = ev;
    if constexpr (I8) {
      int ea, eb;
      frexpf(svs[slot][0], &ea);  // vscale < 2^ea
      frexpf(svs[slot][1], &eb);
      evn = max(ev, __builtin_amdgcn_readfirstlane(max(ea, eb)));  // one scale per unit
    }
    // m = -inf and ev = -1000 before the first step: both raise it
    if (__ballot(lm > m + kSlack) != 0 || evn > ev) {  // wave-uniform
      const float mn = fmaxf(m, max_over_lane_groups(lm));
      const float alpha = __builtin_amdgcn_exp2f(m - mn);
      l *= alpha;
      const float ao = alpha * ldexpf(1.0f, ev - evn);  // times an exact power of two
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) o[dt] *= ao;
      m = mn;  // finite from the first step on: every column sees token 0
      ev = evn;
    }
    float pa[4], pb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pa[i] = __builtin_amdgcn_exp2f(fmaf(sa[i], fa, -m));  // < 2^kSlack
      pb[i] = __builtin_amdgcn_exp2f(fmaf(sb[i], fb, -m));
    }
    l += ((pa[0] + pa[1]) + (pa[2] + pa[3])) + ((pb[0] + pb[1]) + (pb[2] + pb[3]));
    // P^T (times the scaled V scale) as fp16 hi + lo: contraction index 8gq + j
    const float psa = I8 ? uniform_f(ldexpf(svs[slot][0], 14 - kSlack - ev)) : 1.f;  // p * psa < 2^14
    const float psb = I8 ? uniform_f(ldexpf(svs[slot][1], 14 - kSlack - ev)) : 1.f;
    f16x8 ph, pl;
#pragma unroll
    for (int i = 0; i < 4; i += 2) {
      f16x2 ha, la, hb, lb;
      split_f16x2(I8 ? pa[i] * psa : pa[i], I8 ? pa[i + 1] * psa : pa[i + 1], ha, la);
      split_f16x2(I8 ? pb[i] * psb : pb[i], I8 ? pb[i + 1] * psb : pb[i + 1], hb, lb);
      ph[i] = ha[0];
      ph[i + 1] = ha[1];
      ph[4 + i] = hb[0];
      ph[4 + i + 1] = hb[1];
      pl[i] = la[0];
      pl[i + 1] = la[1];
      pl[4 + i] = lb[0];
      pl[4 + i + 1] = lb[1];
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[dt], ph, o[dt], 0, 0, 0);
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[dt], pl, o[dt], 0, 0, 0);
    }
  };

  auto active = [&](int st) { return st * 2 * kUnit <= p_wave; };  // wave-uniform

  // prologue: steps 0 and 1 staged, 2..4 requested, the scores of step 0
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  tq[0] = table_entry(0);
  tq[1] = table_entry(1);
  tq[2] = table_entry(2);
  request(0, I0{});
  request(1, I1{});
  request(2, I2{});
  stage(0, I0{});
  request(3, I0{});
  if (1 < nsteps) stage(1, I1{});
  request(4, I1{});
  __syncthreads();
  f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = sa;
  if (active(0)) qk(0, I0{}, sa, sb);

  for (int s0 = 0; s0 < nsteps; s0 += 3) {
    // all three iterations run (a step past the end only requests and waits),
    // so every path through the loop issues the same loads
    static_for<3>([&](auto B) {  // step st = s0 + b in LDS slot b
      constexpr int b = decltype(B)::value;
      const int st = s0 + b;
      f32x4 na = {0.f, 0.f, 0.f, 0.f}, nb = na;
      if (st + 1 < nsteps && active(st + 1)) qk(st + 1, std::integral_constant<int, (b + 1) % 3>{}, na, nb);
      if (st < nsteps && active(st)) softmax_pv(st, B, sa, sb);
      if (st + 2 < nsteps) stage(st + 2, std::integral_constant<int, (b + 2) % 3>{});
      request(st + 5, std::integral_constant<int, (b + 2) % 3>{});
      __syncthreads();  // step st + 2 staged; every wavefront is done with slot b
      sa = na;
      sb = nb;
    });
  }
  l = sum_over_lane_groups(l);
  if (colv) {
    float* dst = a.out + ((size_t)(qs + qi) * hq + g * G + h) * D;
    const float inv = ldexpf(1.0f, I8 ? ev + kSlack - 14 : 0) / l;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[16 * dt + 4 * gq + i] = o[dt][i] * inv;
  }
}

template <bool I8, int D, int G, int NW>
hipError_t launch_prefill_w(const PrefillLaunch& p, hipStream_t stream) {
  const int ngroups = ((p.max_query_len + 16 / G - 1) / (16 / G) + NW - 1) / NW;
  const int64_t nwg = (int64_t)ngroups * p.lv.num_kv_heads * p.num_seqs;
  if (nwg * 64 * NW >= (int64_t{1} << 32)) return hipErrorInvalidConfiguration;  // grid size in threads
  const dim3 grid((unsigned)nwg), block(64 * NW);
  switch (p.q_dtype) {
    case kF32: hipLaunchKernelGGL((prefill_kernel<I8, D, G, kF32, NW>), grid, block, 0, stream, p); break;
    case kF16: hipLaunchKernelGGL((prefill_kernel<I8, D, G, kF16, NW>), grid, block, 0, stream, p); break;
    case kBF16: hipLaunchKernelGGL((prefill_kernel<I8, D, G, kBF16, NW>), grid, block, 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Eight tiles per workgroup halve the loads and conversions per tile, but
// leave more wavefronts idle where causal tiles of one workgroup see
// different lengths; they are taken when four-tile workgroups would give the
// device at most two per compute unit, i.e. few tiles over a long context.
template <bool I8, int D, int G>
hipError_t launch_prefill_q(const PrefillLaunch& p, hipStream_t stream) {
  const int64_t tiles = (p.max_query_len + 16 / G - 1) / (16 / G);
  const int64_t wg4 = (tiles + 3) / 4 * p.lv.num_kv_heads * p.num_seqs;
  return wg4 <= 2 * (int64_t)device_compute_units() ? launch_prefill_w<I8, D, G, 8>(p, stream)
                                          : launch_prefill_w<I8, D, G, 4>(p, stream);
}

template <bool I8, int D>
hipError_t launch_prefill_g(const PrefillLaunch& p, int group, hipStream_t stream) {
  switch (group) {
    case 1: return launch_prefill_q<I8, D, 1>(p, stream);
    case 2: return launch_prefill_q<I8, D, 2>(p, stream);
    case 4: return launch_prefill_q<I8, D, 4>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// Decode workspace owned by the library (arrival counters, then partition
// partials, as in a caller's workspace), for pkv_decode_step_noalloc. In host
// code `scratch` names a host-side stand-in, not device memory: host code
// uses only the address hipGetSymbolAddress gives for the current device.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch[64];  // per device: the array's device address, once found
}  // namespace

hipError_t scratch_setup() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev]) return hipSuccess;
  void* ptr = nullptr;
  e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  // the arrival counters must start at zero (every call leaves them so)
  e = hipMemset(ptr, 0, kScratchBytes);
  if (e != hipSuccess) return e;
  g_scratch[dev] = ptr;
  return hipSuccess;
}

void* scratch_ptr(int device) {
  if (device < 0 || device >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  return g_scratch[device];
}

hipError_t launch_decode(const DecodeLaunch& d, hipStream_t stream) {
  const int group = d.num_q_heads / d.lv.num_kv_heads;
  const bool i8 = d.lv.kv_dtype == kI8;
  hipError_t e;
  if (d.lv.head_dim == 128)
    e = i8 ? launch_decode_g<true, 128>(d, group, stream) : launch_decode_g<false, 128>(d, group, stream);
  else
    e = i8 ? launch_decode_g<true, 64>(d, group, stream) : launch_decode_g<false, 64>(d, group, stream);
  if (e != hipSuccess || d.max_partitions <= 1 || d.fused_merge) return e;
  const dim3 grid((unsigned)(d.num_seqs * d.num_q_heads));
  const int chunk = d.max_partitions <= 16 ? 16 : d.max_partitions <= 32 ? 32 : 64;
  if (d.lv.head_dim == 128)
    launch_merge<128>(d, chunk, grid, stream);
  else
    launch_merge<64>(d, chunk, grid, stream);
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillLaunch& p, hipStream_t stream) {
  if (p.num_seqs <= 0 || p.max_query_len <= 0) return hipSuccess;
  const int group = p.num_q_heads / p.lv.num_kv_heads;
  const bool i8 = p.lv.kv_dtype == kI8;
  if (p.lv.head_dim == 128)
    return i8 ? launch_prefill_g<true, 128>(p, group, stream) : launch_prefill_g<false, 128>(p, group, stream);
  return i8 ? launch_prefill_g<true, 64>(p, group, stream) : launch_prefill_g<false, 64>(p, group, stream);
}

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
