// prefill.hip -- chunked prefill attention of libpkv for gfx950: causal
// attention of each sequence's newest tokens over its paged context
// ("轻量级推理引擎实战" §一), on the matrix-core contractions of decode, with
// the context staged once per workgroup in LDS.

#include "device.h"

namespace pkv {
namespace {

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

hipError_t launch_prefill(const PrefillLaunch& p, hipStream_t stream) {
  if (p.num_seqs <= 0 || p.max_query_len <= 0) return hipSuccess;
  const int group = p.num_q_heads / p.lv.num_kv_heads;
  const bool i8 = p.lv.kv_dtype == kI8;
  if (p.lv.head_dim == 128)
    return i8 ? launch_prefill_g<true, 128>(p, group, stream) : launch_prefill_g<false, 128>(p, group, stream);
  return i8 ? launch_prefill_g<true, 64>(p, group, stream) : launch_prefill_g<false, 64>(p, group, stream);
}

}  // namespace pkv
