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
//  H3 merge:   log-sum-exp merge of the partition partials.
//
// Cache layout per layer and per K/V: codes [N][Hkv][bs][d] -- each
// (block, head) tile is bs*d contiguous elements, so a 16-row slice of a tile
// is one contiguous 2 KB (int8, d=128) or 4 KB (fp16) run that a wavefront
// reads with 16-byte loads, 8 or 4 rows per load instruction.

#include <hip/hip_runtime.h>

#include "kernels.h"

namespace pkv {
namespace {

constexpr int kWaves = 4;             // wavefronts per decode workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kUnit = 16;             // tokens per unit of work (16-row tile slice)
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

// Cross-lane moves inside a row of 16 lanes (DPP). bound_ctrl: lanes that
// would read outside the row read 0 (none of the patterns below do).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                               0xF, 0xF, true));
}
constexpr int kQuadXor1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kHalfMirror = 0x141; // lane i <-> 7-i within 8
constexpr int kMirror = 0x140;     // lane i <-> 15-i within 16

// Sum over the LPT consecutive lanes that hold one token row (LPT = 4, 8, 16):
// after the quad steps every lane holds its quad's sum; the mirror steps pair
// lanes from different quads / halves, so every lane ends with the group sum.
template <int LPT>
__device__ __forceinline__ float row_group_sum(float x) {
  x += dpp<kQuadXor1>(x);
  x += dpp<kQuadXor2>(x);
  if constexpr (LPT >= 8) x += dpp<kHalfMirror>(x);
  if constexpr (LPT >= 16) x += dpp<kMirror>(x);
  return x;
}

// Maximum over all 64 lanes, returned wave-uniform.
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp<kQuadXor1>(x));
  x = fmaxf(x, dpp<kQuadXor2>(x));
  x = fmaxf(x, dpp<kHalfMirror>(x));
  x = fmaxf(x, dpp<kMirror>(x));
  const int b = __builtin_bit_cast(int, x);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

__device__ __forceinline__ int wave_max_int(int x) {
  for (int off = 32; off >= 1; off >>= 1) x = max(x, __shfl_xor(x, off));
  return x;
}

// 16 int8 codes -> fp32 (sign-extending byte conversions).
__device__ __forceinline__ void cvt_i8x16(const uint4 raw, float* f) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int b = 0; b < 4; ++b) f[4 * i + b] = (float)(int8_t)(w[i] >> (8 * b));
}

// 8 binary16 values -> fp32.
__device__ __forceinline__ void cvt_f16x8(const uint4 raw, float* f) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = f16_to_f32(w[i] & 0xffffu);
    f[2 * i + 1] = f16_to_f32(w[i] >> 16);
  }
}

// ---------------------------------------------------------------------------
// H2: split-context decode.
//
// Lane layout inside a wavefront: a token row of d elements is read by LPT
// lanes with one 16-byte load each (EPL elements per load); the wavefront
// covers TPI = 64 / LPT rows per load instruction and NLD loads per 16-token
// unit. Lane (r, c) = (lane / LPT, lane % LPT) owns dims [c*EPL, c*EPL+EPL)
// of rows r, r+TPI, ... of each unit.
//
// Each wavefront runs an online softmax over the units it is dealt (units
// u0+w, u0+w+4, ...): per unit it forms the G scores of every row (a dot
// product of EPL terms per lane, summed over the row's LPT lanes with DPP),
// takes the unit maximum across the wavefront, rescales its running (m, l, o)
// only when that maximum grows, then accumulates p * v. Scores are kept in
// base 2 (softmax_scale * log2 e folded into q) so exp2 is one instruction.
// The four wavefronts' states are merged through LDS at the end; a sequence
// that fits in one partition writes its output directly, otherwise the
// partition's (m, l, o/l) goes to the workspace for the merge kernel.
// ---------------------------------------------------------------------------
template <bool I8, int D, int G, int QT>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(const DecodeLaunch a) {
  constexpr int ESZ = I8 ? 1 : 2;
  constexpr int EPL = 16 / ESZ;
  constexpr int LPT = D / EPL;
  constexpr int TPI = 64 / LPT;
  constexpr int NLD = kUnit / TPI;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane / LPT;
  const int c = lane % LPT;
  const int part = blockIdx.x;
  const int g = blockIdx.y;
  const int s = blockIdx.z;

  const int T = a.partition_tokens;
  // Lengths beyond what the table or the grid covers are clamped, so a bad
  // length cannot send a load outside the cache or the workspace.
  const int len = min(a.lens[s], min(a.max_blocks * a.lv.block_size, a.max_partitions * T));
  const int t0 = part * T;
  if (t0 >= len) return;
  const int t1 = min(len, t0 + T);
  const int nparts = (len + T - 1) / T;
  const int u0 = t0 / kUnit;
  const int u1 = (t1 + kUnit - 1) / kUnit;
  const int hkv = a.lv.num_kv_heads;
  const int bs = a.lv.block_size;
  const int upb = bs / kUnit;
  const int hq = a.num_q_heads;
  const int32_t* table = a.tables + (size_t)s * a.max_blocks;
  const size_t tile_bytes = (size_t)bs * D * ESZ;
  const char* kcodes = (const char*)a.lv.k_codes;
  const char* vcodes = (const char*)a.lv.v_codes;

  // Query slice of every head of the group, pre-scaled into base 2.
  float qr[G][EPL];
  const float qscale = a.softmax_scale * kLog2e;
#pragma unroll
  for (int j = 0; j < G; ++j)
#pragma unroll
    for (int e = 0; e < EPL; ++e)
      qr[j][e] = load_elem<QT>(a.q, ((size_t)s * hq + g * G + j) * D + c * EPL + e) * qscale;

  float m[G], l[G], o[G][EPL];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    m[j] = -INFINITY;
    l[j] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[j][e] = 0.f;
  }

  const size_t row_off = ((size_t)r * D + c * EPL) * ESZ;
  uint4 kr[NLD], vr[NLD];
  float ksc = 1.f, vsc = 1.f;
  auto load_unit = [&](int u) {
    const int blk = min(max(table[u / upb], 0), a.lv.num_blocks - 1);  // in-bounds even for a bad entry
    const size_t tile = ((size_t)blk * hkv + g) * tile_bytes + (size_t)(u % upb) * kUnit * D * ESZ;
    const char* kp = kcodes + tile + row_off;
    const char* vp = vcodes + tile + row_off;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      kr[i] = *(const uint4*)(kp + (size_t)i * TPI * D * ESZ);
      vr[i] = *(const uint4*)(vp + (size_t)i * TPI * D * ESZ);
    }
    if constexpr (I8) {
      ksc = a.lv.k_scales[(size_t)blk * hkv + g];
      vsc = a.lv.v_scales[(size_t)blk * hkv + g];
    }
  };

  int u = u0 + wave;
  if (u < u1) load_unit(u);
  for (; u < u1; u += kWaves) {
    uint4 kc[NLD], vc[NLD];
#pragma unroll
    for (int i = 0; i < NLD; ++i) { kc[i] = kr[i]; vc[i] = vr[i]; }
    const float kscale = ksc, vscale = vsc;
    const int tok0 = u * kUnit;
    if (u + kWaves < u1) load_unit(u + kWaves);  // prefetch the next unit
    const bool partial = tok0 + kUnit > t1;

    float sc[NLD][G];
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      float kf[EPL];
      if constexpr (I8) cvt_i8x16(kc[i], kf); else cvt_f16x8(kc[i], kf);
#pragma unroll
      for (int j = 0; j < G; ++j) {
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc = fmaf(qr[j][e], kf[e], acc);
        acc = row_group_sum<LPT>(acc);
        sc[i][j] = I8 ? acc * kscale : acc;
      }
    }
    if (partial) {
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        const bool valid = tok0 + i * TPI + r < t1;
#pragma unroll
        for (int j = 0; j < G; ++j) sc[i][j] = valid ? sc[i][j] : -INFINITY;
      }
    }
#pragma unroll
    for (int j = 0; j < G; ++j) {
      float cm = sc[0][j];
#pragma unroll
      for (int i = 1; i < NLD; ++i) cm = fmaxf(cm, sc[i][j]);
      cm = wave_max(cm);
      if (cm > m[j]) {  // wave-uniform
        const float alpha = __builtin_amdgcn_exp2f(m[j] - cm);
        l[j] *= alpha;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[j][e] *= alpha;
        m[j] = cm;
      }
    }
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      float vf[EPL];
      if constexpr (I8) cvt_i8x16(vc[i], vf); else cvt_f16x8(vc[i], vf);
      if (partial && tok0 + i * TPI + r >= t1) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) vf[e] = 0.f;  // rows past the end may hold any bits
      }
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const float pj = __builtin_amdgcn_exp2f(sc[i][j] - m[j]);
        l[j] += pj;
        const float pv = I8 ? pj * vscale : pj;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[j][e] = fmaf(pv, vf[e], o[j][e]);
      }
    }
  }

  // Sum l and o over the token slots (lanes with equal c).
#pragma unroll
  for (int off = LPT; off < 64; off <<= 1) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      l[j] += __shfl_xor(l[j], off);
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[j][e] += __shfl_xor(o[j][e], off);
    }
  }

  __shared__ float sm_o[kWaves][G][D];
  __shared__ float sm_m[kWaves][G];
  __shared__ float sm_l[kWaves][G];
  if (r == 0) {
#pragma unroll
    for (int j = 0; j < G; ++j)
#pragma unroll
      for (int e = 0; e < EPL; ++e) sm_o[wave][j][c * EPL + e] = o[j][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int j = 0; j < G; ++j) { sm_m[wave][j] = m[j]; sm_l[wave][j] = l[j]; }
  }
  __syncthreads();

  const size_t pmax = a.max_partitions;
  for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
    const int j = idx / D;
    const int dd = idx % D;
    float M = sm_m[0][j];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sm_m[w][j]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float wt = __builtin_amdgcn_exp2f(sm_m[w][j] - M);  // empty wave: exp2(-inf) = 0
      L = fmaf(wt, sm_l[w][j], L);
      O = fmaf(wt, sm_o[w][j][dd], O);
    }
    const int h = g * G + j;
    if (nparts == 1) {
      a.out[((size_t)s * hq + h) * D + dd] = O / L;
    } else {
      const size_t slot = ((size_t)s * hq + h) * pmax + part;
      const size_t nrow = (size_t)a.num_seqs * hq * pmax;
      float* ws_m = a.ws;
      float* ws_l = a.ws + nrow;
      float* ws_o = a.ws + 2 * nrow;
      ws_o[slot * D + dd] = O / L;
      if (dd == 0) { ws_m[slot] = M; ws_l[slot] = L; }
    }
  }
}

// ---------------------------------------------------------------------------
// H3: merge the partitions of each (sequence, query head):
//   M = max_p m_p,  w_p = l_p * 2^(m_p - M),  out = sum_p w_p o_p / sum_p w_p
// where o_p is the partition's normalised output and m_p its base-2 maximum.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(D) void merge_kernel(const DecodeLaunch a) {
  const int hq = a.num_q_heads;
  const int s = blockIdx.x / hq;
  const int h = blockIdx.x % hq;
  const int T = a.partition_tokens;
  const int len = min(a.lens[s], min(a.max_blocks * a.lv.block_size, a.max_partitions * T));
  const int nparts = (len + T - 1) / T;
  if (nparts <= 1) return;
  const size_t pmax = a.max_partitions;
  const size_t nrow = (size_t)a.num_seqs * hq * pmax;
  const float* ws_m = a.ws;
  const float* ws_l = a.ws + nrow;
  const float* ws_o = a.ws + 2 * nrow;
  const size_t base = ((size_t)s * hq + h) * pmax;
  float M = -INFINITY;
  for (int p = 0; p < nparts; ++p) M = fmaxf(M, ws_m[base + p]);
  float L = 0.f, O = 0.f;
  for (int p = 0; p < nparts; ++p) {
    const float w = __builtin_amdgcn_exp2f(ws_m[base + p] - M) * ws_l[base + p];
    L += w;
    O = fmaf(w, ws_o[(base + p) * D + threadIdx.x], O);
  }
  a.out[((size_t)s * hq + h) * D + threadIdx.x] = O / L;
}

// ---------------------------------------------------------------------------
// H1 (binary16 cache): one thread per (token, head, K|V, 8-element chunk);
// each value rounded to binary16, ties to even.
// ---------------------------------------------------------------------------
template <int IN>
__global__ __launch_bounds__(256) void append_f16_kernel(const LayerView lv, const void* k,
                                                         const void* v, const int64_t* slots,
                                                         int32_t n) {
  const int D = lv.head_dim;
  const int hkv = lv.num_kv_heads;
  const int chunks = D / 8;
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
  const int64_t row = slot % lv.block_size;
  if (slot < 0 || blk >= lv.num_blocks) return;  // not a slot of this pool
  const void* src = kv ? v : k;
  const size_t sbase = ((size_t)i * hkv + h) * D + ch * 8;
  uint32_t packed[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const _Float16 lo = (_Float16)load_elem<IN>(src, sbase + 2 * e);
    const _Float16 hi = (_Float16)load_elem<IN>(src, sbase + 2 * e + 1);
    packed[e] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
                ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
  }
  uint16_t* dst = (uint16_t*)(kv ? lv.v_codes : lv.k_codes) +
                  (((size_t)blk * hkv + h) * lv.block_size + row) * D + ch * 8;
  *(uint4*)dst = make_uint4(packed[0], packed[1], packed[2], packed[3]);
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

template <int IN>
__global__ __launch_bounds__(256) void append_i8_kernel(const LayerView lv, const void* k,
                                                        const void* v, const int64_t* slots,
                                                        int32_t n) {
  const int lane = threadIdx.x & 63;
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int hkv = lv.num_kv_heads;
  if (wid >= (int64_t)n * hkv * 2) return;
  const int h = (int)(wid % hkv);
  const int kv = (int)((wid / hkv) & 1);
  const int64_t i = wid / hkv / 2;
  const int bs = lv.block_size;
  const int D = lv.head_dim;
  const int64_t slot0 = slots[i];
  const int64_t blk = slot0 / bs;
  if (slot0 < 0 || blk >= lv.num_blocks) return;  // not a slot of this pool
  if (i > 0 && slots[i - 1] / bs == blk) return;  // not the first token of its run
  int nr = 1;
  while (i + nr < n && slots[i + nr] / bs == blk) ++nr;
  const int row0 = (int)(slot0 % bs);
  nr = min(nr, bs - row0);  // rows stay inside the tile even for malformed slots

  const void* src = kv ? v : k;
  float mx = 0.f;
  for (int e = lane; e < nr * D; e += 64) {
    const int rr = e / D, dd = e % D;
    mx = fmaxf(mx, fabsf(load_elem<IN>(src, ((size_t)(i + rr) * hkv + h) * D + dd)));
  }
  mx = wave_max(mx);

  int8_t* tile = (int8_t*)(kv ? lv.v_codes : lv.k_codes) + ((size_t)blk * hkv + h) * bs * D;
  float* sp = (kv ? lv.v_scales : lv.k_scales) + (size_t)blk * hkv + h;
  float sc;
  if (row0 == 0) {
    sc = scale_of(mx);
  } else {
    int qm = 0;
    for (int e = lane; e < row0 * D; e += 64) qm = max(qm, abs((int)tile[e]));
    qm = wave_max_int(qm);
    const float s_old = *sp;
    const float m_old = (float)qm * s_old;
    if (mx <= m_old) {
      sc = s_old;
    } else {
      sc = scale_of(mx);
      for (int e = lane; e < row0 * D; e += 64) tile[e] = encode((float)tile[e] * s_old, sc);
    }
  }
  for (int e = lane; e < nr * D; e += 64) {
    const int rr = e / D, dd = e % D;
    tile[(size_t)row0 * D + e] = encode(load_elem<IN>(src, ((size_t)(i + rr) * hkv + h) * D + dd), sc);
  }
  if (lane == 0) *sp = sc;
}

template <bool I8, int D, int G>
hipError_t launch_decode_q(const DecodeLaunch& d, hipStream_t stream) {
  const dim3 grid(d.max_partitions, d.lv.num_kv_heads, d.num_seqs);
  switch (d.q_dtype) {
    case kF32: hipLaunchKernelGGL((decode_split_kernel<I8, D, G, kF32>), grid, dim3(kThreads), 0, stream, d); break;
    case kF16: hipLaunchKernelGGL((decode_split_kernel<I8, D, G, kF16>), grid, dim3(kThreads), 0, stream, d); break;
    case kBF16: hipLaunchKernelGGL((decode_split_kernel<I8, D, G, kBF16>), grid, dim3(kThreads), 0, stream, d); break;
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

}  // namespace

bool decode_supported(int head_dim, int group) {
  return (head_dim == 64 || head_dim == 128) && (group == 1 || group == 2 || group == 4);
}

size_t decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                              int32_t max_partitions) {
  if (max_partitions <= 1) return 0;
  const size_t rows = (size_t)num_seqs * num_q_heads * max_partitions;
  return rows * (2 + (size_t)head_dim) * sizeof(float);
}

hipError_t launch_decode(const DecodeLaunch& d, hipStream_t stream) {
  const int group = d.num_q_heads / d.lv.num_kv_heads;
  const bool i8 = d.lv.kv_dtype == kI8;
  hipError_t e;
  if (d.lv.head_dim == 128)
    e = i8 ? launch_decode_g<true, 128>(d, group, stream) : launch_decode_g<false, 128>(d, group, stream);
  else
    e = i8 ? launch_decode_g<true, 64>(d, group, stream) : launch_decode_g<false, 64>(d, group, stream);
  if (e != hipSuccess || d.max_partitions <= 1) return e;
  const dim3 grid((unsigned)(d.num_seqs * d.num_q_heads));
  if (d.lv.head_dim == 128)
    hipLaunchKernelGGL(merge_kernel<128>, grid, dim3(128), 0, stream, d);
  else
    hipLaunchKernelGGL(merge_kernel<64>, grid, dim3(64), 0, stream, d);
  return hipGetLastError();
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
