// append.hip -- H1 of libpkv for gfx950: store new tokens' K/V at their slots,
// rounded to binary16, or quantized with the per-(block, KV head) symmetric
// INT8 quantizer of "轻量级推理引擎实战：KV Cache 量化与连续批处理的底层优化" §三
// (also its seal-on-full variant, the section's third design note).

#include "device.h"

namespace pkv {
namespace {

// ---------------------------------------------------------------------------
// H1 (binary16 cache): one thread per (token, head, K|V, 8-element chunk);
// each value rounded to binary16, ties to even. The token index is the
// fastest, so the four lanes of a quad hold four consecutive tokens of one
// chunk. 16-bit input is read with one 16-byte load per thread when K/V are
// 16-byte aligned. A K chunk is one 16-byte store. When a quad's four slots
// are the rows 4m .. 4m+3 of one block (a prompt's tokens), the V values of
// one dim for the four tokens are adjacent in the tile (its token index
// 4tg + ti is fastest): the quad exchanges its values with DPP broadcasts and
// each lane stores two dims as 8-byte words. Otherwise each lane stores its
// token's V values two bytes at a time.
// ---------------------------------------------------------------------------
template <int P>  // value of lane P of the quad, in all four lanes
__device__ __forceinline__ uint32_t quad_bcast(uint32_t x) {
  return (uint32_t)dpp_i<P | (P << 2) | (P << 4) | (P << 6)>((int)x);
}

template <int IN>
__global__ __launch_bounds__(256) void append_f16_kernel(const LayerView lv, const void* k,
                                                         const void* v, const int64_t* slots,
                                                         int32_t n, int vec) {
  const int hkv = lv.num_kv_heads, D = lv.head_dim;
  const int lc = __builtin_ctz(D / 8);          // chunks per row: a power of two
  const int lbs = __builtin_ctz(lv.block_size);  // block sizes are powers of two
  const int64_t groups = ((int64_t)n + 3) / 4;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= ((groups * hkv * 2) << (lc + 2))) return;  // whole quads leave together
  const int ti = (int)(idx & 3);
  const int ch = (int)((idx >> 2) & ((1 << lc) - 1));
  const uint32_t rest = (uint32_t)(idx >> (lc + 2));  // (group, K|V, head) < 2^32, checked on the host
  const int h = (int)(rest % (uint32_t)hkv);
  const int kv = (int)((rest / (uint32_t)hkv) & 1);
  const int64_t i = (int64_t)(rest / (uint32_t)hkv >> 1) * 4 + ti;
  const void* src = kv ? v : k;
  const int64_t slot = i < n ? slots[i] : -1;
  const bool ok = slot >= 0 && (slot >> lbs) < lv.num_blocks;  // a slot of this pool
  const size_t e0 = ((size_t)i * hkv + h) * D + ch * 8;
  float x[8] = {};
  if (ok) {
    if (vec && IN != kF32) {
      const uint4 r = *((const uint4*)src + e0 / 8);
      const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[2 * j] = IN == kF16 ? f16_to_f32(w[j] & 0xFFFFu) : bf16_to_f32(w[j] & 0xFFFFu);
        x[2 * j + 1] = IN == kF16 ? f16_to_f32(w[j] >> 16) : bf16_to_f32(w[j] >> 16);
      }
    } else if (vec) {
      const uint4 r0 = *((const uint4*)src + e0 / 4), r1 = *((const uint4*)src + e0 / 4 + 1);
      const uint32_t w[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = __uint_as_float(w[j]);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = load_elem<IN>(src, e0 + j);
    }
  }
  uint32_t d[4];  // the chunk as binary16 pairs: dims 2j (low half), 2j + 1
#pragma unroll
  for (int j = 0; j < 4; ++j)
    d[j] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x[2 * j]) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x[2 * j + 1]) << 16);
  const int row = (int)(slot & (lv.block_size - 1));
  uint16_t* tile = (uint16_t*)(kv ? lv.v_codes : lv.k_codes) + (((size_t)(slot >> lbs) * hkv + h) << lbs) * D;
  if (kv == 0) {
    if (ok) *(uint4*)(tile + k_tile_offset(row, ch * 8, D)) = make_uint4(d[0], d[1], d[2], d[3]);
    return;
  }
  // rows 4m .. 4m+3 of one block in lanes 0..3 of the quad (block sizes are multiples of 4)
  const uint32_t lo0 = quad_bcast<0>((uint32_t)slot), hi0 = quad_bcast<0>((uint32_t)(slot >> 32));
  const int64_t base = (int64_t)(((uint64_t)hi0 << 32) | lo0);
  const int mine = ok && slot == base + ti && (base & 3) == 0;
  const int all = mine & (int)quad_bcast<0>((uint32_t)mine) & (int)quad_bcast<1>((uint32_t)mine) &
                  (int)quad_bcast<2>((uint32_t)mine) & (int)quad_bcast<3>((uint32_t)mine);
  if (all) {
    // lane ti stores dims 2 ti and 2 ti + 1 of the four tokens
    uint32_t b[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t v0 = quad_bcast<0>(d[j]), v1 = quad_bcast<1>(d[j]), v2 = quad_bcast<2>(d[j]),
                     v3 = quad_bcast<3>(d[j]);
      if (j == ti) {
        b[0] = (v0 & 0xFFFFu) | (v1 << 16);
        b[1] = (v2 & 0xFFFFu) | (v3 << 16);
        b[2] = (v0 >> 16) | (v1 & 0xFFFF0000u);
        b[3] = (v2 >> 16) | (v3 & 0xFFFF0000u);
      }
    }
    *(uint2*)(tile + v_tile_offset(row - ti, ch * 8 + 2 * ti, D)) = make_uint2(b[0], b[1]);
    *(uint2*)(tile + v_tile_offset(row - ti, ch * 8 + 2 * ti + 1, D)) = make_uint2(b[2], b[3]);
  } else if (ok) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      tile[v_tile_offset(row, ch * 8 + 2 * j, D)] = (uint16_t)(d[j] & 0xFFFFu);
      tile[v_tile_offset(row, ch * 8 + 2 * j + 1, D)] = (uint16_t)(d[j] >> 16);
    }
  }
}

// ---------------------------------------------------------------------------
// H1 (int8 cache): a run is the maximal group of consecutive tokens that
// land in one block. Workgroups of (window of 64 tokens, split, K|V, head)
// find the runs that start in their window and deal them to their
// wavefronts; a wavefront appends its runs one after another, single-token
// runs four at a time. Every (block, head, K|V) tile has a single writer, so
// no atomics are needed.
// ---------------------------------------------------------------------------

// One wavefront appends tokens i .. i+nr-1 (rows of src [token][Hkv][d]) of
// head h, K (kv 0) or V (kv 1), at rows row0 .. row0+nr-1 of block blk:
// grow-only scale, old rows re-encoded when it grows (the §三 quantizer named
// at the top of this file, plus the rule for partly filled blocks). issue()
// sends its loads without waiting
// (the block's scale and the largest |code| of its old rows; up to kPre new
// values per lane); finish() does the rest and returns the new scale. The old
// codes are read only when the max grows, 16 bytes per load and kOcBatch
// loads per lane at a time. Old rows of a K tile are its first row0*D bytes;
// those of a V tile lie in its first ceil(row0/16) 16-token sub-tiles, where
// each byte's token is decoded from its offset.
template <int IN>
struct I8Append {
  static constexpr int kOcBatch = 2;  // old-code chunks per lane in flight (a tile is at most 8 per lane)
  static constexpr int kPre = 2;      // new values held per lane (one row of d <= 128)
  const LayerView* lv;
  int kv, h, row0, nr;
  int64_t i;
  const void* src;
  int8_t* tile;
  float* sp;
  int32_t* qp;
  int old_bytes;
  float s_old;
  int q_old;
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
    s_old = row0 > 0 ? *sp : 1.f;
    q_old = row0 > 0 ? *qp : 0;
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
      // the old rows' largest |code| is kept beside the scale, so the old
      // codes are read only when the max grows
      const float m_old = (float)q_old * s_old;
      if (mx <= m_old) {
        sc = s_old;
        qold = q_old;
      } else {
        // the max grew: re-encode the old codes from their dequantised values
        // and store whole chunks back (bytes of rows >= row0 are written back
        // unchanged)
        sc = scale_of(mx);
        for (int k0 = 0; k0 * 1024 < old_bytes; k0 += kOcBatch) {  // kOcBatch chunks per lane at a time
          uint4 oc[kOcBatch];
#pragma unroll
          for (int u = 0; u < kOcBatch; ++u) {
            const int c = lane + 64 * (k0 + u);
            oc[u] = c * 16 < old_bytes ? *(const uint4*)(tile + (size_t)c * 16) : make_uint4(0u, 0u, 0u, 0u);
          }
#pragma unroll
          for (int u = 0; u < kOcBatch; ++u) {
            const int c = lane + 64 * (k0 + u);
            if (c * 16 < old_bytes) {
              const uint32_t wm = word_mask(k0 + u);
              uint32_t ws[4] = {oc[u].x ^ bias4, oc[u].y ^ bias4, oc[u].z ^ bias4, oc[u].w ^ bias4};
#pragma unroll
              for (int w = 0; w < 4; ++w) {
#pragma unroll 1
                for (int b = 0; b < 4; ++b) {  // rolled: this path runs only when a scale grows
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

// A run of several tokens with 16-byte aligned K/V (a prompt's runs): one
// wavefront reads its nr x D new values with 16-byte loads, a row's chunks in
// consecutive lanes, keeping the first four loads per lane in registers for
// the encode pass (runs of up to 16 x 128 bf16 values fit; longer ones are
// read again from L2). The scale follows I8Append: max|x| / 127 for a fresh
// block; kept when the block's old max (its stored largest |code| times its
// scale) covers the new values. When it does not, nothing is written and the
// call returns false: the old codes must be re-encoded, which I8Append does.
// K codes go straight to their row-major places. V codes of a run from row 0
// that fills whole 16-token sub-tiles are gathered in the wavefront's LDS
// stage in tile order and stored as 16-byte chunks; other V codes are stored
// byte by byte.
constexpr int kStageBytes = 64 * 128;  // the largest tile: bs 64 x d 128 codes

template <int IN, bool WHOLE, bool F16R = false>  // WHOLE: row0 == 0 and nr a multiple of 16;
                                                  // F16R: values rounded to binary16 first (sealing)
__device__ __forceinline__ bool append_i8_vec(const LayerView& lv, int kv, int h, int64_t blk, int row0, int nr,
                                              const void* src, int64_t i, uint8_t* stage) {
  constexpr int EPV = IN == kF32 ? 4 : 8;  // elements per 16-byte load
  constexpr int G = 4;                     // loads per lane in flight
  const int lane = threadIdx.x & 63;
  const int hkv = lv.num_kv_heads, D = lv.head_dim, ld = __builtin_ctz(D);
  const size_t at = (size_t)blk * hkv + h;
  float* sp = (kv ? lv.v_scales : lv.k_scales) + at;
  int32_t* qp = (kv ? lv.v_qmax : lv.k_qmax) + at;
  if constexpr (WHOLE) row0 = 0;
  const int nvec = nr * D / EPV;      // a multiple of 8 (d >= 64); of 64 for WHOLE
  const int per = (nvec + 63) >> 6;  // loads per lane, the last one masked
  auto addr = [&](int q) {  // vector q of the run: row (q*EPV) / D, dims (q*EPV) % D ..
    const int e = q * EPV;
    return (const uint4*)src + ((((size_t)(i + (e >> ld)) * hkv + h) << ld) + (e & (D - 1))) / EPV;
  };
  auto in_run = [&](int q) { return q < nvec; };
  auto load = [&](int q) { return in_run(q) ? *addr(q) : make_uint4(0u, 0u, 0u, 0u); };
  auto unpack = [&](const uint4& r, float* x) {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (IN == kF32) {
        x[j] = __uint_as_float(w[j]);
      } else if constexpr (IN == kF16) {
        x[2 * j] = f16_to_f32(w[j] & 0xFFFFu);
        x[2 * j + 1] = f16_to_f32(w[j] >> 16);
      } else {
        x[2 * j] = bf16_to_f32(w[j] & 0xFFFFu);
        x[2 * j + 1] = bf16_to_f32(w[j] >> 16);
      }
    }
    if constexpr (F16R) {
#pragma unroll
      for (int j = 0; j < EPV; ++j) x[j] = (float)(_Float16)x[j];
    }
  };
  auto absmax = [&](const uint4& r, float m) {
    float x[EPV];
    unpack(r, x);
#pragma unroll
    for (int j = 0; j < EPV; ++j) m = fmaxf(m, fabsf(x[j]));
    return m;
  };
  uint4 r0[G];
#pragma unroll
  for (int u = 0; u < G; ++u) r0[u] = load(u * 64 + lane);
  float s_old = 1.f;
  int q_old = 0;
  if (!WHOLE && row0 > 0) {
    s_old = *sp;
    q_old = *qp;
  }
  float mx = 0.f;
  for (int g = G; g < per; g += G) {
    uint4 r[G];
#pragma unroll
    for (int u = 0; u < G; ++u) r[u] = load((g + u) * 64 + lane);
#pragma unroll
    for (int u = 0; u < G; ++u) mx = absmax(r[u], mx);
  }
#pragma unroll
  for (int u = 0; u < G; ++u) mx = absmax(r0[u], mx);  // zero padding leaves the max unchanged
  mx = uniform_f(wave_max(mx));
  if (!WHOLE && row0 > 0 && mx > (float)q_old * s_old) return false;  // the max grows
  const float sc = row0 == 0 ? scale_of(mx) : s_old;

  int8_t* tile = (int8_t*)(kv ? lv.v_codes : lv.k_codes) + at * lv.block_size * D;
  const bool staged = WHOLE && kv;
  int qm = 0;
  if (staged) {  // the stage may still be read by this wavefront's previous run
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  auto encode_vec = [&](const uint4& r, int q) {
    float x[EPV];
    unpack(r, x);
    const int e = q * EPV, t = row0 + (e >> ld), d0 = e & (D - 1);
    uint32_t w[EPV / 4] = {};
#pragma unroll
    for (int j = 0; j < EPV; ++j) {
      const int8_t c = encode(x[j], sc);
      qm = max(qm, abs((int)c));
      if (kv) {
        // V byte (t, d0 + j): consecutive dims are d/4 bytes apart in a lane slice
        const int64_t o = v_tile_offset(t, d0, D) + j * (D >> 2);
        const uint8_t b = (uint8_t)(c ^ (int8_t)0x80);
        if constexpr (WHOLE) stage[o] = b;
        else tile[o] = (int8_t)b;
      } else {
        w[j >> 2] |= (uint32_t)(uint8_t)c << (8 * (j & 3));
      }
    }
    if (!kv) {
      if constexpr (EPV == 8) *(uint2*)(tile + k_tile_offset(t, d0, D)) = make_uint2(w[0], w[1]);
      else *(uint32_t*)(tile + k_tile_offset(t, d0, D)) = w[0];
    }
  };
  for (int g = 0; g < per; g += G) {  // the held first group, then groups read again
    uint4 r[G];
    if (g == 0) {
#pragma unroll
      for (int u = 0; u < G; ++u) r[u] = r0[u];
    } else {
#pragma unroll
      for (int u = 0; u < G; ++u) r[u] = load((g + u) * 64 + lane);
    }
#pragma unroll
    for (int u = 0; u < G; ++u)
      if (g + u < per && (WHOLE || in_run((g + u) * 64 + lane))) encode_vec(r[u], (g + u) * 64 + lane);
  }
  if (staged) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    for (int c = lane; c < (nr * D) >> 4; c += 64) *(uint4*)(tile + 16 * c) = *(const uint4*)(stage + 16 * c);
  }
  qm = wave_max_int(qm);
  if (lane == 0) {
    *sp = sc;
    *qp = row0 == 0 ? qm : max(q_old, qm);
  }
  return true;
}

// The runs of a call -- maximal groups of consecutive tokens whose slots lie
// in one block -- that start among tokens [base, base + 64), each as its
// first token i, its block, first row and length. The window's positions are
// dealt in equal stretches to the 4 * splits wavefronts of its `splits`
// workgroups (wavefront w of split s takes stretch 4 s + w), and a wavefront
// appends the runs that start in its stretch: one run per 16 positions for a
// prompt in 16-token blocks, four single-token runs per wavefront when
// splits is 4. A token whose slot is not in the pool starts no run; a run
// stops at the end of its block and is at most 64 tokens long (the slots of
// base .. base + 127 cover every run that starts in the window).
constexpr int64_t kAppendGroups = 512;      // workgroups a launch aims for before splitting stops
constexpr int64_t kAppendMaxGrid = 1 << 22;  // workgroups per launch (grids stay far below 2^32 threads)

struct Run {
  int64_t i, blk;
  int row0, nr;
};

struct WindowRuns {
  int64_t sa, sb, base;
  int lbs, bs;
  uint64_t starts;  // window positions that start a run
  uint64_t mine;    // those that start this wavefront's runs

  __device__ __forceinline__ void init(const LayerView& lv, const int64_t* slots, int32_t n, int64_t base_,
                                       int split, int splits) {
    const int lane = threadIdx.x & 63;
    const int wave = split * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // of 4 * splits
    const int ways = 4 * splits;
    base = base_;
    bs = lv.block_size;
    lbs = __builtin_ctz(bs);  // block sizes are powers of two
    sa = base + lane < n ? slots[base + lane] : -1;
    sb = base + 64 + lane < n ? slots[base + 64 + lane] : -1;
    const int64_t sprev = base > 0 ? slots[base - 1] : -1;
    // lane j: the slot of the token before base + j
    const int64_t up = ((int64_t)__shfl_up((int)(sa >> 32), 1) << 32) | (uint32_t)__shfl_up((int)sa, 1);
    const int64_t pa = lane == 0 ? sprev : up;
    const bool in_pool = sa >= 0 && (sa >> lbs) < lv.num_blocks;
    starts = __ballot(in_pool && (base + lane == 0 || (pa >> lbs) != (sa >> lbs)));
    const int per = 64 / ways;  // window positions per wavefront (ways is a power of two)
    mine = starts & (((uint64_t(1) << per) - 1) << (wave * per));  // per <= 16
  }

  // The next of this wavefront's runs, in token order; false when none is left.
  __device__ __forceinline__ bool next(Run& run) {
    if (mine == 0) return false;
    const int j = __builtin_ctzll(mine);
    mine &= mine - 1;
    at(j, run);
    return true;
  }

  // The run that starts at window position j (a bit of starts).
  __device__ __forceinline__ void at(int j, Run& run) const {
    const int64_t slot0 = ((int64_t)__builtin_amdgcn_readlane((int)(sa >> 32), j) << 32) |
                          (uint32_t)__builtin_amdgcn_readlane((int)sa, j);
    const int64_t blk = slot0 >> lbs;
    // tokens base + j, base + j + 1, ... while their slots stay in blk
    const uint64_t ma = __ballot(sa >= 0 && (sa >> lbs) == blk);
    const uint64_t mb = __ballot(sb >= 0 && (sb >> lbs) == blk);
    const uint64_t from = j == 0 ? ma : (ma >> j) | (mb << (64 - j));
    const int len = ~from == 0 ? 64 : __builtin_ctzll(~from);
    run.i = base + j;
    run.blk = blk;
    run.row0 = (int)(slot0 & (bs - 1));
    run.nr = min(len, bs - run.row0);  // rows stay inside the tile even for malformed slots
  }

  // Starts with no other start in the 31 positions after them in the window:
  // the only ones whose runs can be 32 tokens or longer.
  __device__ __forceinline__ uint64_t long_candidates() const {
    uint64_t y = starts >> 1;  // OR of starts >> 1 .. 31, spread by doubling
    y |= y >> 1;
    y |= y >> 2;
    y |= y >> 4;
    y |= y >> 8;
    y |= y >> 15;
    return starts & ~y;
  }
};

// A run from row 0 of at least 32 tokens, a multiple of 16 (a prompt's full
// 64-token blocks, or 32 or 48 rows of one), by a team of `size` wavefronts of the workgroup
// (four, or two when two such runs of 32 tokens go side by side), wavefronts
// first .. first + size - 1: each takes an equal share of the run's 16-byte
// vectors (whole rows: a share holds nr/size >= 8 rows), the maxima meet in
// LDS, and the V codes are gathered in the team's stage tile, which its
// threads store as 16-byte chunks. Scale and codes as in append_i8_vec.
// Every thread of the workgroup makes one such call (two barriers), for its
// team's run. K/V must be 16-byte aligned; a share is at most kMaxPer loads
// per lane (size 4 for 64-token runs).
template <int IN>
__device__ __forceinline__ void append_i8_coop(const LayerView& lv, int kv, int h, const Run& run, const void* src,
                                               int first, int size, uint8_t* stage, float* red, int* redq) {
  constexpr int EPV = IN == kF32 ? 4 : 8;  // elements per 16-byte load
  constexpr int kMaxPer = IN == kF32 ? 8 : 4;  // loads per lane for a 64 x 128 tile over four wavefronts
  const int lane = threadIdx.x & 63, w = (threadIdx.x >> 6) - first;  // rank in the team
  const int hkv = lv.num_kv_heads, D = lv.head_dim, ld = __builtin_ctz(D);
  const int nr = run.nr;
  const int64_t i = run.i;
  const int qw = nr * D / EPV / size;  // vectors per wavefront (a multiple of 32), at most kMaxPer * 64
  auto addr = [&](int q) {  // vector q of the run: row (q*EPV) / D, dims (q*EPV) % D ..
    const int e = q * EPV;
    return (const uint4*)src + ((((size_t)(i + (e >> ld)) * hkv + h) << ld) + (e & (D - 1))) / EPV;
  };
  auto unpack = [&](const uint4& r, float* x) {
    const uint32_t u32[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (IN == kF32) {
        x[j] = __uint_as_float(u32[j]);
      } else if constexpr (IN == kF16) {
        x[2 * j] = f16_to_f32(u32[j] & 0xFFFFu);
        x[2 * j + 1] = f16_to_f32(u32[j] >> 16);
      } else {
        x[2 * j] = bf16_to_f32(u32[j] & 0xFFFFu);
        x[2 * j + 1] = bf16_to_f32(u32[j] >> 16);
      }
    }
  };
  uint4 r[kMaxPer];
#pragma unroll
  for (int u = 0; u < kMaxPer; ++u)
    r[u] = u * 64 + lane < qw ? *addr(w * qw + u * 64 + lane) : make_uint4(0u, 0u, 0u, 0u);
  float mx = 0.f;
#pragma unroll
  for (int u = 0; u < kMaxPer; ++u) {
    float x[EPV];
    unpack(r[u], x);
#pragma unroll
    for (int j = 0; j < EPV; ++j) mx = fmaxf(mx, fabsf(x[j]));
  }
  mx = wave_max(mx);
  if (lane == 0) red[first + w] = mx;
  __syncthreads();
  float m_all = red[first];
  for (int t = 1; t < size; ++t) m_all = fmaxf(m_all, red[first + t]);
  const float sc = uniform_f(scale_of(m_all));
  const size_t at = (size_t)run.blk * hkv + h;
  int8_t* tile = (int8_t*)(kv ? lv.v_codes : lv.k_codes) + at * lv.block_size * D;
  int qm = 0;
#pragma unroll
  for (int u = 0; u < kMaxPer; ++u) {
    if (u * 64 + lane < qw) {
      float x[EPV];
      unpack(r[u], x);
      const int e = (w * qw + u * 64 + lane) * EPV, t = e >> ld, d0 = e & (D - 1);
      uint32_t wd[EPV / 4] = {};
#pragma unroll
      for (int j = 0; j < EPV; ++j) {
        const int8_t c = encode(x[j], sc);
        qm = max(qm, abs((int)c));
        if (kv) stage[v_tile_offset(t, d0, D) + j * (D >> 2)] = (uint8_t)(c ^ (int8_t)0x80);
        else wd[j >> 2] |= (uint32_t)(uint8_t)c << (8 * (j & 3));
      }
      if (!kv) {
        if constexpr (EPV == 8) *(uint2*)(tile + k_tile_offset(t, d0, D)) = make_uint2(wd[0], wd[1]);
        else *(uint32_t*)(tile + k_tile_offset(t, d0, D)) = wd[0];
      }
    }
  }
  qm = wave_max_int(qm);
  if (lane == 0) redq[first + w] = qm;
  __syncthreads();
  const int tid = w * 64 + lane;  // thread rank in the team
  if (kv)
    for (int c = tid; c < (nr * D) >> 4; c += 64 * size) *(uint4*)(tile + 16 * c) = *(const uint4*)(stage + 16 * c);
  if (tid == 0) {
    int q_all = redq[first];
    for (int t = 1; t < size; ++t) q_all = max(q_all, redq[first + t]);
    (kv ? lv.v_scales : lv.k_scales)[at] = sc;
    (kv ? lv.v_qmax : lv.k_qmax)[at] = q_all;
  }
}

// Maximum over each 16-lane row of the wavefront, in every lane of the row.
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp_f<kQuadXor1>(x));
  x = fmaxf(x, dpp_f<kQuadXor2>(x));
  x = fmaxf(x, dpp_f<kHalfMirror>(x));
  return fmaxf(x, dpp_f<kMirror>(x));
}
__device__ __forceinline__ int row16_max_int(int x) {  // x >= 0
  x = max(x, dpp_i<kQuadXor1>(x));
  x = max(x, dpp_i<kQuadXor2>(x));
  x = max(x, dpp_i<kHalfMirror>(x));
  return max(x, dpp_i<kMirror>(x));
}

// Up to four single-token runs q0 .. q{cnt-1} at once (a decode step's new
// tokens), one per 16-lane row of the wavefront: each lane holds d/16 values
// of its run's row. The rule is I8Append's; a run whose max grows past the
// block's old max (which needs its old codes re-encoded) is not written here:
// its bit is set in the returned mask and I8Append does it whole.
template <int IN>
__device__ __forceinline__ unsigned append_i8_rows(const LayerView& lv, int kv, int h, const Run& q0, const Run& q1,
                                                   const Run& q2, const Run& q3, int cnt, const void* src, int vec) {
  constexpr int kMaxE = 8;  // d / 16 for d <= 128
  const int lane = threadIdx.x & 63, g = lane >> 4;
  const int hkv = lv.num_kv_heads, D = lv.head_dim, E = D >> 4;
  const int64_t i = g == 0 ? q0.i : g == 1 ? q1.i : g == 2 ? q2.i : q3.i;
  const int64_t blk = g == 0 ? q0.blk : g == 1 ? q1.blk : g == 2 ? q2.blk : q3.blk;
  const int row0 = g == 0 ? q0.row0 : g == 1 ? q1.row0 : g == 2 ? q2.row0 : q3.row0;
  const bool act = g < cnt;
  const size_t at = (size_t)blk * hkv + h;
  float* sp = (kv ? lv.v_scales : lv.k_scales) + at;
  int32_t* qp = (kv ? lv.v_qmax : lv.k_qmax) + at;
  const float s_old = act && row0 > 0 ? *sp : 1.f;
  const int q_old = act && row0 > 0 ? *qp : 0;
  const int d0 = (lane & 15) * E;
  float x[kMaxE] = {};
  const size_t e0 = ((size_t)i * hkv + h) * D + d0;
  if (act && vec && IN != kF32 && E == 8) {  // the lane's 8 values in one 16-byte load
    const uint4 r = *((const uint4*)src + e0 / 8);
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = IN == kF16 ? f16_to_f32(w[j] & 0xFFFFu) : bf16_to_f32(w[j] & 0xFFFFu);
      x[2 * j + 1] = IN == kF16 ? f16_to_f32(w[j] >> 16) : bf16_to_f32(w[j] >> 16);
    }
  } else if (act) {
#pragma unroll
    for (int e = 0; e < kMaxE; ++e)
      if (e < E) x[e] = load_elem<IN>(src, e0 + e);
  }
  float mx = 0.f;
#pragma unroll
  for (int e = 0; e < kMaxE; ++e) mx = fmaxf(mx, fabsf(x[e]));
  mx = row16_max(mx);
  const bool grow = act && row0 > 0 && mx > (float)q_old * s_old;
  const uint64_t gb = __ballot(grow);
  const unsigned grows = (unsigned)((gb & 1u) | ((gb >> 15) & 2u) | ((gb >> 30) & 4u) | ((gb >> 45) & 8u));
  if (act && !grow) {
    const float sc = row0 == 0 ? scale_of(mx) : s_old;
    int8_t* tile = (int8_t*)(kv ? lv.v_codes : lv.k_codes) + at * lv.block_size * D;
    uint32_t w[kMaxE / 4] = {};
    int qn = 0;
#pragma unroll
    for (int e = 0; e < kMaxE; ++e) {
      if (e < E) {
        const int8_t c = encode(x[e], sc);
        qn = max(qn, abs((int)c));
        if (kv) {
          // V byte (row0, d0 + e): consecutive dims are d/4 bytes apart in a lane slice
          tile[v_tile_offset(row0, d0, D) + e * (D >> 2)] = (int8_t)(c ^ (int8_t)0x80);
        } else {
          w[e >> 2] |= (uint32_t)(uint8_t)c << (8 * (e & 3));
        }
      }
    }
    if (!kv) {
      if (E == 8) *(uint2*)(tile + k_tile_offset(row0, d0, D)) = make_uint2(w[0], w[1]);
      else *(uint32_t*)(tile + k_tile_offset(row0, d0, D)) = w[0];
    }
    qn = row16_max_int(qn);
    if ((lane & 15) == 0) {
      *sp = sc;
      *qp = row0 == 0 ? qn : max(q_old, qn);
    }
  }
  return grows;
}

template <int IN>
__global__ __launch_bounds__(256, 4) void append_i8_kernel(const LayerView lv, const void* k,
                                                        const void* v, const int64_t* slots,
                                                        int32_t n, int64_t w0, int splits, int vec) {
  // workgroup: (window w0 + .. of 64 tokens, split, K|V, head)
  __shared__ __align__(16) uint8_t stage[4][kStageBytes];
  const int hkv = lv.num_kv_heads;
  const int h = (int)(blockIdx.x % hkv);
  const int kv = (int)((blockIdx.x / hkv) & 1);
  const int split = (int)((blockIdx.x / hkv / 2) % splits);
  const int64_t base = (w0 + (int64_t)(blockIdx.x / hkv / 2 / splits)) * 64;
  __shared__ float red[4];
  __shared__ int redq[4];
  WindowRuns wr;
  wr.init(lv, slots, n, base, split, splits);
  const void* src = kv ? v : k;
  if (vec && lv.block_size == 64) {
    // In 64-token blocks, whole runs of 32 or more tokens from row 0 (at most
    // two start in a window): the window's k-th such run goes to split
    // k % splits, where the workgroup's four wavefronts take it together; two
    // runs of 32 tokens in one workgroup go side by side, two wavefronts each.
    // Every wavefront finds the same runs, so all take the same barriers.
    // (In 32-token blocks the runs of a window already keep two wavefronts
    // busy, and working them jointly measured slower on a serving workload.)
    uint64_t coop = 0;
    int k_long = 0, mine_n = 0;
    Run r0, r1;
    for (uint64_t m = wr.long_candidates(); m != 0; m &= m - 1) {
      const int j = __builtin_ctzll(m);
      Run r;
      wr.at(j, r);
      if (r.row0 == 0 && (r.nr & 15) == 0 && r.nr >= 32) {
        coop |= uint64_t(1) << j;
        if (k_long % splits == split) {
          if (mine_n == 0) r0 = r;
          else r1 = r;
          ++mine_n;
        }
        ++k_long;
      }
    }
    uint8_t* st = &stage[0][0];
    const int w = threadIdx.x >> 6;
    const bool pair = mine_n == 2 && r0.nr == 32 && r1.nr == 32;  // side by side, two wavefronts each
    for (int c = 0; c < (pair ? 1 : mine_n); ++c) {
      const bool second = pair ? w >= 2 : c == 1;
      append_i8_coop<IN>(lv, kv, h, second ? r1 : r0, src, pair ? (w & 2) : 0, pair ? 2 : 4,
                         pair && second ? st + 2 * kStageBytes : st, red, redq);
    }
    if (coop != 0) {
      wr.mine &= ~coop;
      __syncthreads();  // the stage is read to its end before any wavefront writes its own part again
    }
  }
  Run a;
  bool have = wr.next(a);
  while (have) {
    // runs for the general path (I8Append), as a mask over q0 .. q3
    Run q0 = a, q1 = a, q2 = a, q3 = a;
    unsigned general;
    if (vec && a.nr > 1) {
      const bool done = a.row0 == 0 && (a.nr & 15) == 0
                            ? append_i8_vec<IN, true>(lv, kv, h, a.blk, 0, a.nr, src, a.i, stage[threadIdx.x >> 6])
                            : append_i8_vec<IN, false>(lv, kv, h, a.blk, a.row0, a.nr, src, a.i, nullptr);
      general = done ? 0u : 1u;  // the block's max grows: old codes re-encoded
      have = wr.next(a);
    } else if (a.nr == 1) {  // up to four consecutive single-token runs together
      int cnt = 1;
      have = wr.next(a);
      if (have && a.nr == 1) {
        q1 = a;
        cnt = 2;
        have = wr.next(a);
        if (have && a.nr == 1) {
          q2 = a;
          cnt = 3;
          have = wr.next(a);
          if (have && a.nr == 1) {
            q3 = a;
            cnt = 4;
            have = wr.next(a);
          }
        }
      }
      general = append_i8_rows<IN>(lv, kv, h, q0, q1, q2, q3, cnt, src, vec);  // those whose max grows
    } else {
      general = 1u;  // unaligned K/V
      have = wr.next(a);
    }
    for (unsigned m = general; m != 0; m &= m - 1) {
      const int g = __builtin_ctz(m);
      const Run r = g == 0 ? q0 : g == 1 ? q1 : g == 2 ? q2 : q3;
      I8Append<IN> p;
      p.issue(lv, kv, h, r.blk, r.row0, r.nr, src, r.i);
      (void)p.finish();
    }
  }
}

// ---------------------------------------------------------------------------
// H1 for a seal-on-full INT8 layer (lazy quantization, "轻量级推理引擎实战"
// §三, third design note): runs found and dealt to wavefronts as above, one
// run at a time per wavefront. A run that leaves its block partly filled is
// stored as binary16 rows in the block's FP16 staging tile. The run that
// writes the block's last row quantizes the whole block -- its staged rows and
// the run's own, all as binary16 values -- with the section's quantize_block:
// one scale max|x|/127 (1.0 for an all-zero head), codes round(x / scale) to
// even, clamped to [-127, 127]; it stores the codes, the scale and the largest
// |code|. A run that fills a whole block from row 0 (a prompt's full blocks)
// has no staged rows: it takes the 16-byte-load path of the INT8 append with
// its values rounded to binary16 first, which is the same arithmetic.
// ---------------------------------------------------------------------------
template <int IN>
__global__ __launch_bounds__(256) void append_seal_kernel(const LayerView lv, const void* k,
                                                          const void* v, const int64_t* slots,
                                                          int32_t n, int64_t w0, int splits, int vec) {
  // workgroup: (window w0 + .. of 64 tokens, split, K|V, head)
  const int lane = threadIdx.x & 63;
  const int hkv = lv.num_kv_heads;
  const int h = (int)(blockIdx.x % hkv);
  const int kv = (int)((blockIdx.x / hkv) & 1);
  const int split = (int)((blockIdx.x / hkv / 2) % splits);
  const int64_t base = (w0 + (int64_t)(blockIdx.x / hkv / 2 / splits)) * 64;
  const int bs = lv.block_size;
  __shared__ __align__(16) uint8_t stage[4][kStageBytes];
  WindowRuns wr;
  wr.init(lv, slots, n, base, split, splits);
  for (Run r; wr.next(r);) {
    const int64_t i = r.i, blk = r.blk;
    const int row0 = r.row0, nr = r.nr;
    const int D = lv.head_dim, ld = __builtin_ctz(D);
    const void* src = kv ? v : k;
    if (vec && row0 == 0 && nr == bs) {  // a whole block from row 0: no staged rows
      (void)append_i8_vec<IN, true, true>(lv, kv, h, blk, 0, nr, src, i, stage[threadIdx.x >> 6]);
      continue;
    }
    uint16_t* t16 = (uint16_t*)(kv ? lv.tail_v : lv.tail_k) + ((size_t)blk * hkv + h) * bs * D;
    auto off = [&](int t, int dd) { return kv ? v_tile_offset(t, dd, D) : k_tile_offset(t, dd, D); };
    // element e of the run (row e >> ld, dim e % D) as binary16 bits
    auto run_bits = [&](int e) {
      return __builtin_bit_cast(uint16_t, (_Float16)load_elem<IN>(src, ((size_t)(i + (e >> ld)) * hkv + h) * D + (e & (D - 1))));
    };
    if (row0 + nr < bs) {  // the block stays partly filled: stage the rows
      for (int e = lane; e < nr * D; e += 64) t16[off(row0 + (e >> ld), e & (D - 1))] = run_bits(e);
      continue;
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
}

}  // namespace

hipError_t launch_append(const LayerView& lv, const void* k, const void* v, int in_dtype,
                         const int64_t* slots, int32_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int vec = (((uintptr_t)k | (uintptr_t)v) & 15) == 0;  // 16-byte loads
  if (lv.kv_dtype == kF16) {
    const int64_t units = ((int64_t)n + 3) / 4 * lv.num_kv_heads * 2;  // (group of 4 tokens, K|V, head)
    if (units >> 32) return hipErrorInvalidValue;  // more than any device holds
    const int64_t total = units * (lv.head_dim / 8) * 4;
    const dim3 grid((unsigned)((total + 255) / 256));
    switch (in_dtype) {
      case kF32: hipLaunchKernelGGL(append_f16_kernel<kF32>, grid, dim3(256), 0, stream, lv, k, v, slots, n, vec); break;
      case kF16: hipLaunchKernelGGL(append_f16_kernel<kF16>, grid, dim3(256), 0, stream, lv, k, v, slots, n, vec); break;
      case kBF16: hipLaunchKernelGGL(append_f16_kernel<kBF16>, grid, dim3(256), 0, stream, lv, k, v, slots, n, vec); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    // A window's runs are dealt to the 4 wavefronts of `splits` workgroups:
    // few windows (a decode step's single tokens) get up to 16 wavefronts,
    // four runs each; many windows one workgroup each.
    const int64_t windows = ((int64_t)n + 63) / 64;
    const int64_t per_window = 2 * (int64_t)lv.num_kv_heads;
    int splits = 1;  // 1, 2 or 4
    while (splits < 4 && 2 * splits * windows * per_window <= kAppendGroups) splits *= 2;
    const int64_t chunk = std::max<int64_t>(1, kAppendMaxGrid / (splits * per_window));
    for (int64_t w0 = 0; w0 < windows; w0 += chunk) {
      const dim3 grid((unsigned)(std::min(chunk, windows - w0) * splits * per_window));
      if (lv.seal) {
        switch (in_dtype) {
          case kF32: hipLaunchKernelGGL(append_seal_kernel<kF32>, grid, dim3(256), 0, stream, lv, k, v, slots, n, w0, splits, vec); break;
          case kF16: hipLaunchKernelGGL(append_seal_kernel<kF16>, grid, dim3(256), 0, stream, lv, k, v, slots, n, w0, splits, vec); break;
          case kBF16: hipLaunchKernelGGL(append_seal_kernel<kBF16>, grid, dim3(256), 0, stream, lv, k, v, slots, n, w0, splits, vec); break;
          default: return hipErrorInvalidValue;
        }
      } else {
        switch (in_dtype) {
          case kF32: hipLaunchKernelGGL(append_i8_kernel<kF32>, grid, dim3(256), 0, stream, lv, k, v, slots, n, w0, splits, vec); break;
          case kF16: hipLaunchKernelGGL(append_i8_kernel<kF16>, grid, dim3(256), 0, stream, lv, k, v, slots, n, w0, splits, vec); break;
          case kBF16: hipLaunchKernelGGL(append_i8_kernel<kBF16>, grid, dim3(256), 0, stream, lv, k, v, slots, n, w0, splits, vec); break;
          default: return hipErrorInvalidValue;
        }
      }
    }
  }
  return hipGetLastError();
}

}  // namespace pkv
