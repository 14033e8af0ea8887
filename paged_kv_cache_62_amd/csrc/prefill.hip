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
// one KV head. A workgroup of NW wavefronts (four; eight where the context is
// cut into pieces, so that twice the tiles share each staged step) takes
// NW * NTW consecutive tiles of one sequence and KV head, NTW per wavefront,
// and streams a range of that head's context (the whole of what its queries
// see, or one piece of it) through them in steps of two 16-token units (A, B).
// Its wavefronts read the same units, so the workgroup loads each once: each
// staging thread (all of them, or the first half with eight wavefronts and an
// INT8 cache) requests the same 16-byte piece of both units of a step (of K or
// of V, alike across its wavefront, so each request is a scalar buffer
// descriptor and a fixed per-lane offset) into registers three steps ahead,
// and writes the pair into a three-slot LDS ring as binary16 (INT8 codes
// convert exactly; the block
// scales stay factors of the scores and of P). Per step and wavefront, for
// each of its tiles (the K and V operands read from LDS once for all of them):
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
// exceeds it by more. The running max starts at a finite floor, so a column
// that sees no token of the workgroup's range keeps zero weights.
//
// The loop is software-pipelined. Step st first stages step st + 2 into the
// slot step st - 1 last read, then issues the QK products of step st + 1,
// then the softmax and PV products of step st, and reads the V operands of
// step st + 1 last; one barrier per step. The ring holds step st (V read a
// step early), st + 1 (K) and st + 2 (being written).
//
// Context pieces: with few query tiles over a long context, the context is
// cut into pieces of piece_tokens (a multiple of 64) and each (tile group,
// piece) is a workgroup. Each writes, per (query, head), its partial (m, l,
// o/l) -- m the base-2 running max, l the sum of weights relative to it --
// and counts its arrival; the last piece of a tile group to finish combines
// the group's pieces (log-sum-exp) and writes the output. With one piece the
// workgroup writes the output itself.
//
// Workgroups are numbered so that each XCD takes a contiguous stretch of the
// (sequence, KV head, piece) units' tile groups (consecutive workgroup ids go
// to the eight XCDs in turn), whose L2 then serves those context ranges to
// all of them. With one piece it runs them longest context first across its
// units: list scheduling in that order keeps its compute units busy to the
// end, where unit after unit left the long tile groups of the last units to
// run alone.
// ---------------------------------------------------------------------------
constexpr float kMaxFloor = -1e30f;  // running max before any visible token (finite: no inf - inf)

// The order in which a workgroup's lanes take the 16-byte pieces of a unit's
// K (V): piece = the lane's index q with bits 2 and up permuted (kd[cfg][i],
// vd[cfg][i] is where bit 2 + i goes). Four consecutive lanes keep 64 contiguous bytes;
// the LDS addresses the staging writes then reach from 8 (16) consecutive
// lanes fall in distinct banks of 32 (64) banks of 4 bytes, for the row
// pitches and V operand layout of prefill_kernel (checked exhaustively for
// each of the four configurations when the orders were chosen).
template <bool I8, int D>
__device__ __forceinline__ int piece_order(int q, bool k) {
  constexpr int n = (I8 ? D : 2 * D) == 64 ? 4 : (I8 ? D : 2 * D) == 128 ? 5 : 6;  // bits above the low two
  constexpr int kd[4][6] = {{2, 5, 3, 4, 0, 0}, {3, 2, 4, 5, 6, 0}, {2, 6, 3, 4, 5, 0}, {2, 3, 4, 5, 6, 7}};
  constexpr int vd[4][6] = {{2, 3, 4, 5, 0, 0}, {2, 4, 3, 5, 6, 0}, {3, 4, 2, 5, 6, 0}, {2, 5, 3, 4, 6, 7}};
  constexpr int cfg = I8 ? (D == 64 ? 0 : 1) : (D == 64 ? 2 : 3);
  int p = q & 3;
#pragma unroll
  for (int i = 0; i < n; ++i) p |= ((q >> (2 + i)) & 1) << (k ? kd[cfg][i] : vd[cfg][i]);
  return p;
}

template <bool I8, int D, int G, int QT, int NTW, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 8)))
void prefill_kernel(const PrefillLaunch a) {
  constexpr int NT = 64 * NW;               // threads
  constexpr int TQ = 16 / G;                // query tokens per tile
  constexpr int WQ = NW * NTW * TQ;         // query tokens per workgroup
  constexpr int ESZ = I8 ? 1 : 2;           // bytes per cached element
  constexpr int NK = D / 32;                // 16-byte binary16 pieces of a K row per lane
  constexpr int NDT = D / 16;               // 16-dim tiles of the PV product
  constexpr int QE = D / 4;                 // query, K and V elements per lane
  constexpr int GB = kUnit * D * ESZ;       // cache bytes of a unit's K (or V)
  constexpr int HP = GB / 16;               // 16-byte pieces of a unit's K (or V)
  // A thread stages pairs: the same piece of units A and B, of K or of V
  static_assert(HP % 64 == 0, "a wavefront's pairs lie in K or in V");
  constexpr int PPT = (2 * HP + NT - 1) / NT;  // pairs per thread per step (some threads idle at PPT = 1)
  constexpr int PE = 16 / ESZ;              // elements per piece
  constexpr int RP = 2 * D + 16;            // LDS pitch of a binary16 K row (padded against bank conflicts)
  constexpr int VP = 16 * NDT + 16;         // LDS pitch of a lane's V operands
  constexpr int KS = kUnit * RP;            // LDS bytes of a unit's K rows
  constexpr int SS = 2 * KS + 64 * VP;      // LDS bytes of a step: K rows of A, of B, then V
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n16 = lane & 15, gq = lane >> 4;
  const int hq = a.num_q_heads, hkv = a.lv.num_kv_heads, bs = a.lv.block_size;

  // workgroup -> (pair, piece, tile group). Work item jo = unit * ngroups + r
  // is tile group ngroups - 1 - r (r = 0 the one with the longest context) of
  // unit (pair, piece). XCD x runs ids x, x + 8, ... and takes the x-th
  // contiguous stretch of items, so its units' context stays in its L2. With
  // one piece (a grid that may take several rounds) it runs them in the order
  // r = 0, 1, ... across those units, longest first: the k-th id of the XCD
  // is the k-th item of the stretch in that order. A context cut into pieces
  // (planned only for grids that fit at once) runs unit after unit instead,
  // which measured faster there.
  const int ngroups = (a.max_query_len + WQ - 1) / WQ;
  const int npc = a.pieces;
  const int nwg = gridDim.x, xcd = blockIdx.x & 7, base = nwg >> 3, rem = nwg & 7;
  const int jstart = xcd * base + min(xcd, rem), jend = jstart + base + (xcd < rem ? 1 : 0);
  int k = blockIdx.x >> 3, r = 0, unit = 0;
  if (npc > 1) {
    unit = (jstart + k) / ngroups;
    r = (jstart + k) % ngroups;
  } else {
    for (; r < ngroups; ++r) {  // the units holding item r in [jstart, jend): [lo, hi)
      const int lo = (jstart - r + ngroups - 1) / ngroups, hi = (jend - r + ngroups - 1) / ngroups;
      if (k < hi - lo) {
        unit = lo + k;
        break;
      }
      k -= hi - lo;
    }
  }
  const int pair = unit / npc, piece = unit % npc, grp = ngroups - 1 - r;
  const int g = pair % hkv, s = pair / hkv;

  const int lupb = __builtin_ctz(bs / kUnit);
  const int qs = a.query_start[s];
  const int ql = min(a.query_start[s + 1] - qs, a.max_query_len);
  const int len = min(a.lens[s], a.max_blocks * bs);
  const int jw = grp * WQ;             // first query of the workgroup's tiles
  if (jw >= ql || ql > len) return;    // the whole workgroup (no barrier passed yet)
  const int plast = len - ql + min(jw + WQ, ql) - 1;  // last position the workgroup's queries see
  const int c0 = piece * a.piece_tokens;              // its context range: tokens [c0, cend)
  if (c0 > plast) return;              // a piece past what its queries see (no partial is read)
  // the last piece takes the rest of the context (also past max_context_len)
  const int cend = piece == npc - 1 ? plast + 1 : min(c0 + a.piece_tokens, plast + 1);
  const int u0 = c0 / kUnit;                          // c0 is a multiple of 64
  const int nun = (cend - c0 + kUnit - 1) / kUnit;    // units the workgroup reads
  const int nsteps = (nun + 1) / 2;
  const int vlim = min(len, c0 + nun * kUnit);        // rows from here on are not staged or not cached

  // lane column n16 of tile t: query j0[t] + n16 / G, head n16 % G. A column
  // past the chunk computes over the whole range (its query is zero) and is
  // not written. Every wavefront runs every step of the workgroup's range
  // (masking covers what its columns do not see), so that no branch splits
  // a step's matrix-core and vector work.
  const int h = n16 % G;
  int qi[NTW], pos[NTW], pmin[NTW];  // pmin grows with t
  bool colv[NTW];
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    const int j0 = jw + (wave * NTW + t) * TQ;
    qi[t] = j0 + n16 / G;
    colv[t] = qi[t] < ql;
    pos[t] = colv[t] ? len - ql + qi[t] : len - 1;   // last position the column sees
    pmin[t] = len - ql + j0;                         // the tile's first query position
  }

  // ---- query operands (B of QK): D/4 elements per lane and tile, fp16 hi (+ lo)
  f16x8 qh[NTW][NK], ql8[NTW][QT == kF32 ? NK : 1];
  float qconst[NTW];
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    float qv[QE];
    const size_t qrow = ((size_t)(qs + (colv[t] ? qi[t] : 0)) * hq + g * G + h) * D + gq * QE;
#pragma unroll
    for (int e = 0; e < QE; ++e) {
      const float x = load_elem<QT>(a.q, qrow + e);  // row qs (valid) for a column past the chunk
      qv[e] = colv[t] ? x : 0.f;
    }
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
        qh[t][c][e] = hi;
        if constexpr (QT == kF32) ql8[t][c][e] = (_Float16)(y - (float)hi);
      }
    }
    qconst[t] = ldexpf(a.softmax_scale * kLog2e, qexp - 15);  // > 0
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
  auto table_entry = [&](int x) {  // lane j = 0, 1: the block of unit 2x + j of the range
    const int u = u0 + min(2 * x + (lane & 1), nun - 1);
    return table[u >> lupb];
  };
  // Pair c of a thread: piece q of K (shK[c]) or of V, byte shO[c] of each
  // unit's K (V), the same every step; shA[c] false for a thread without a
  // pair c. Pieces are taken in an order (a permutation of the piece index
  // that keeps four lanes on 64 contiguous bytes) under which the LDS
  // writes of 8 (16) consecutive lanes fall in distinct banks of 32 (64).
  int shO[PPT];
  bool shK[PPT], shA[PPT];
#pragma unroll
  for (int c = 0; c < PPT; ++c) {
    const int pr = (int)threadIdx.x + NT * c;
    const bool k = pr < HP;
    const int q = pr % HP;
    shA[c] = __builtin_amdgcn_readfirstlane(pr < 2 * HP ? 1 : 0) != 0;
    shK[c] = __builtin_amdgcn_readfirstlane(k ? 1 : 0) != 0;
    shO[c] = 16 * piece_order<I8, D>(q, k);
  }
  int tq[3];                    // table entries of the next requests, by step % 3
  i32x4 ring[3][PPT][2];        // requested steps' pieces, by step % 3, pair and unit
  float rsc[3];                 // and their scales: lane 0/1 K scale of unit A/B, lane 2/3 V scale
  auto request = [&](int st, auto r) {  // wave-uniform st; r = st % 3
    const int ba = min(max(__builtin_amdgcn_readlane(tq[r], 0), 0), a.lv.num_blocks - 1);
    const int bb = min(max(__builtin_amdgcn_readlane(tq[r], 1), 0), a.lv.num_blocks - 1);
    const int umask = (1 << lupb) - 1;
    const uint64_t sub[2] = {
        ((uint64_t)ba * hkv + g) * tile_bytes + (uint64_t)((u0 + min(2 * st, nun - 1)) & umask) * GB,
        ((uint64_t)bb * hkv + g) * tile_bytes + (uint64_t)((u0 + min(2 * st + 1, nun - 1)) & umask) * GB};
#pragma unroll
    for (int c = 0; c < PPT; ++c) {
      if (!shA[c]) continue;
#pragma unroll
      for (int V = 0; V < 2; ++V) {
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            uniform_ptr((shK[c] ? kcodes : vcodes) + sub[V]), (short)0, GB, kRsrcWord3);
        ring[r][c][V] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, shO[c], 0, 0));
      }
    }
    if constexpr (I8) {
      const float* sp = (lane & 2) ? a.lv.v_scales : a.lv.k_scales;
      rsc[r] = sp[(size_t)((lane & 1) ? bb : ba) * hkv + g];
    }
    tq[r] = table_entry(st + 3);
  };
  __shared__ __align__(16) unsigned char lds[3][SS];
  // Per LDS slot and unit (uniform): the K scale; log2 and reciprocal of the
  // V scale; the larger binary exponent of the two V scales. Derived when
  // the step is staged, off the path of the step that uses them.
  float sks[3][2], lsv[3][2], isv[3][2];
  int esv[3];
  // The requested step st -> LDS slot st % 3, as binary16. Without a unit B
  // (the last step of an odd count) the pieces of the last unit stand in
  // for it: finite values, behind the causal mask and the V row limit.
  auto stage = [&](int st, auto slot) {
    esv[slot] = -1000;
    static_for<2>([&](auto V) {
      sks[slot][V] = 1.f;
      lsv[slot][V] = 0.f;
      isv[slot][V] = 1.f;
      if constexpr (I8) {
        if (2 * st + V < nun) {
          const float vs = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, rsc[slot]), 2 + V));
          sks[slot][V] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, rsc[slot]), V));
          lsv[slot][V] = uniform_f(__builtin_amdgcn_logf(vs));
          isv[slot][V] = uniform_f(__builtin_amdgcn_rcpf(vs));
          int e;
          frexpf(vs, &e);  // vs < 2^e
          esv[slot] = max(esv[slot], __builtin_amdgcn_readfirstlane(e));
        }
      }
    });
#pragma unroll
    for (int c = 0; c < PPT; ++c) {
      if (!shA[c]) continue;
      const bool isk = shK[c];
      const int e = shO[c] / ESZ;  // first element of the piece within K (V)
      // four elements of piece V of the pair, as binary16 (INT8: K signed,
      // V stored biased)
      auto four = [&](int V, int k) {
        const uint32_t w = (uint32_t)ring[slot][c][V][k];
        if constexpr (I8) return biased_i8x4_to_f16x4(w ^ (isk ? 0x80808080u : 0u));
        else return __builtin_bit_cast(f16x4, make_uint2(ring[slot][c][V][2 * (k & 1)], ring[slot][c][V][2 * (k & 1) + 1]));
      };
      unsigned char* sl = lds[slot];
      if (isk) {  // K row e / D of each unit, elements e % D ..
#pragma unroll
        for (int V = 0; V < 2; ++V) {
          unsigned char* dst = sl + V * KS + (e / D) * RP + 2 * (e % D);
#pragma unroll
          for (int k = 0; k < PE / 8; ++k) {
            const f16x4 x0 = four(V, 2 * k), x1 = four(V, 2 * k + 1);
            *(f16x8*)(dst + 16 * k) = f16x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
          }
        }
      } else {  // lane e / QE's V elements: per dim tile four rows of unit A, then four of B
        unsigned char* dst = sl + 2 * KS + (e / QE) * VP + 4 * (e % QE);
#pragma unroll
        for (int k = 0; k < PE / 4; ++k) {
          const f16x4 xa = four(0, k), xb = four(1, k);
          *(f16x8*)(dst + 16 * k) = f16x8{xa[0], xa[1], xa[2], xa[3], xb[0], xb[1], xb[2], xb[3]};
        }
      }
    }
  };

  float m[NTW], l[NTW];
  // P enters the PV product as P' = p * vscale * 2^(14 - kSlack - ev), ev
  // the largest binary exponent of any V scale so far (uniform), computed
  // as one exponential, 2^(s f - m + log2(vscale) + 14 - kSlack - ev): its
  // fp16 hi and lo parts stay below 2^14 and clear of fp16 subnormals
  // however small the scales. The accumulators are rescaled exactly when ev
  // grows and scaled back by 2^(ev + kSlack - 14) at the end. A binary16
  // cache has no scale: P' = p.
  int ev = I8 ? -1000 : 0;
  f32x4 o[NTW][NDT];
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    m[t] = kMaxFloor;
    l[t] = 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[t][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // S^T of the step in an LDS slot, both units, every tile
  auto qk = [&](auto slot, f32x4 (&sa)[NTW], f32x4 (&sb)[NTW]) {
    const unsigned char* sl = lds[slot];
    f16x8 ka[NK], kb[NK];
#pragma unroll
    for (int c = 0; c < NK; ++c) {
      ka[c] = *(const f16x8*)&sl[n16 * RP + gq * (2 * QE) + 16 * c];
      kb[c] = *(const f16x8*)&sl[KS + n16 * RP + gq * (2 * QE) + 16 * c];
    }
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
#pragma unroll
      for (int c = 0; c < NK; ++c) {
        sa[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[c], qh[t][c], c == 0 ? zero : sa[t], 0, 0, 0);
        sb[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kb[c], qh[t][c], c == 0 ? zero : sb[t], 0, 0, 0);
        if constexpr (QT == kF32) {
          sa[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[c], ql8[t][c], sa[t], 0, 0, 0);
          sb[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kb[c], ql8[t][c], sb[t], 0, 0, 0);
        }
      }
    }
  };

  // V operands of the step in an LDS slot
  auto read_v = [&](auto slot, f16x8 (&av)[NDT]) {
    const unsigned char* vl = &lds[slot][2 * KS + lane * VP];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) av[dt] = *(const f16x8*)&vl[16 * dt];
  };

  // Step st (LDS slot): softmax from its scores sa, sb and V operands vv;
  // the next step's scores (LDS slot nslot, possibly past the range: then
  // unused) into sa, sb and its V operands into vv (that slot was staged
  // before the last barrier); O += V^T P^T, every tile.
  auto step = [&](int st, auto slot, auto nslot, f32x4 (&sa)[NTW], f32x4 (&sb)[NTW], f16x8 (&vv)[NDT]) {
    const int t0 = c0 + st * 2 * kUnit;  // the step's first token
    f16x8 av[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) av[dt] = vv[dt];
    if (t0 + 2 * kUnit > vlim) {  // rows not staged, or past the context, may hold any bits
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          av[dt][j] = t0 + 4 * gq + j < vlim ? av[dt][j] : (_Float16)0.0f;
          av[dt][4 + j] = t0 + kUnit + 4 * gq + j < vlim ? av[dt][4 + j] : (_Float16)0.0f;
        }
    }
    f32x4 sc[NTW], sd[NTW];  // this step's scores; sa, sb take the next step's
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      sc[t] = sa[t];
      sd[t] = sb[t];
    }
    // first, so that the matrix cores work through what follows; at raised
    // priority, so that the other wavefront of the SIMD, at its exponentials,
    // does not hold back their issue (s_setprio around the PV products
    // instead measured slower)
    __builtin_amdgcn_s_setprio(1);
    qk(nslot, sa, sb);
    __builtin_amdgcn_s_setprio(0);
    const int evn = I8 ? max(ev, esv[slot]) : ev;
    // some column does not see the whole step (wave-uniform; the first tile
    // has the earliest queries, so it decides for all)
    if (t0 + 2 * kUnit - 1 > pmin[0]) {
#pragma unroll
      for (int t = 0; t < NTW; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sc[t][i] = t0 + 4 * gq + i <= pos[t] ? sc[t][i] : -INFINITY;
          sd[t][i] = t0 + kUnit + 4 * gq + i <= pos[t] ? sd[t][i] : -INFINITY;
        }
    }
    float fa[NTW], fb[NTW];
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      fa[t] = sks[slot][0] * qconst[t];
      fb[t] = sks[slot][1] * qconst[t];
    }
    // log2 of each unit's P' / p (uniform) and the exponent arguments
    // s f - m + log2(P' / p), at the current m and ev
    float la = 0.f, lb = 0.f, xa[NTW][4], xb[NTW][4];
    auto arguments = [&]() {
      if constexpr (I8) {
        la = lsv[slot][0] + (float)(14 - kSlack - ev);
        lb = lsv[slot][1] + (float)(14 - kSlack - ev);
      }
#pragma unroll
      for (int t = 0; t < NTW; ++t) {
        const float ca = la - m[t], cb = lb - m[t];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          xa[t][i] = fmaf(sc[t][i], fa[t], ca);
          xb[t][i] = fmaf(sd[t][i], fb[t], cb);
        }
      }
    };
    arguments();
    // raise the running max when a score exceeds it by more than kSlack (its
    // argument, less log2(P' / p), above kSlack) or a V scale has a larger
    // exponent
    bool raise = evn > ev;
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      const float mx = fmaxf(fmaxf(fmaxf(xa[t][0], xa[t][1]), fmaxf(xa[t][2], xa[t][3])) - la,
                             fmaxf(fmaxf(xb[t][0], xb[t][1]), fmaxf(xb[t][2], xb[t][3])) - lb);
      raise = raise || __ballot(mx > kSlack) != 0;  // wave-uniform
    }
    // the first step with a visible token raises it (m starts at a finite floor)
    if (raise) {
#pragma unroll
      for (int t = 0; t < NTW; ++t) {
        // the step's maximum score from the raw sums (scales are positive)
        const float lm = fmaxf(fmaxf(fmaxf(sc[t][0], sc[t][1]), fmaxf(sc[t][2], sc[t][3])) * fa[t],
                               fmaxf(fmaxf(sd[t][0], sd[t][1]), fmaxf(sd[t][2], sd[t][3])) * fb[t]);
        const float mn = fmaxf(m[t], max_over_lane_groups(lm));
        const float alpha = __builtin_amdgcn_exp2f(m[t] - mn);
        l[t] *= alpha;
        const float ao = alpha * ldexpf(1.0f, ev - evn);  // times an exact power of two
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[t][dt] *= ao;
        m[t] = mn;
      }
      ev = evn;
      arguments();
    }
    // p / P' for l (uniform)
    float ia = 1.f, ib = 1.f;
    if constexpr (I8) {
      ia = ldexpf(isv[slot][0], ev + kSlack - 14);
      ib = ldexpf(isv[slot][1], ev + kSlack - 14);
    }
    const f16x2 m0 = {(_Float16)-1.0f, (_Float16)0.0f}, m1 = {(_Float16)0.0f, (_Float16)-1.0f};
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      float pa[4], pb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pa[i] = __builtin_amdgcn_exp2f(xa[t][i]);  // < 2^14
        pb[i] = __builtin_amdgcn_exp2f(xb[t][i]);
      }
      const float sA = (pa[0] + pa[1]) + (pa[2] + pa[3]), sB = (pb[0] + pb[1]) + (pb[2] + pb[3]);
      l[t] += I8 ? fmaf(sA, ia, sB * ib) : sA + sB;
      // P'^T as fp16 hi + lo, contraction index 8gq + j: hi is P' rounded
      // toward zero; P' - hi is exact in binary32 (a dot product with -1
      // takes it in one instruction) and is rounded to nearest into lo
      f16x8 ph, pl;
#pragma unroll
      for (int i = 0; i < 4; i += 2) {
        const f16x2 ha = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(pa[i], pa[i + 1]));
        const f16x2 hb = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(pb[i], pb[i + 1]));
        ph[i] = ha[0];
        ph[i + 1] = ha[1];
        ph[4 + i] = hb[0];
        ph[4 + i + 1] = hb[1];
        pl[i] = (_Float16)__builtin_amdgcn_fdot2(ha, m0, pa[i], false);
        pl[i + 1] = (_Float16)__builtin_amdgcn_fdot2(ha, m1, pa[i + 1], false);
        pl[4 + i] = (_Float16)__builtin_amdgcn_fdot2(hb, m0, pb[i], false);
        pl[4 + i + 1] = (_Float16)__builtin_amdgcn_fdot2(hb, m1, pb[i + 1], false);
      }
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        o[t][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[dt], ph, o[t][dt], 0, 0, 0);
        o[t][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[dt], pl, o[t][dt], 0, 0, 0);
      }
    }
    read_v(nslot, vv);
  };

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
  f32x4 sa[NTW], sb[NTW];
  f16x8 vv[NDT];
  qk(I0{}, sa, sb);
  read_v(I0{}, vv);

  for (int s0 = 0; s0 < nsteps; s0 += 3) {
    // all three iterations run (a step past the end only requests and waits),
    // so every path through the loop issues the same loads
    static_for<3>([&](auto B) {  // step st = s0 + b in LDS slot b
      constexpr int b = decltype(B)::value;
      const int st = s0 + b;
      // slot (b + 2) % 3 was last read in step st - 1: stage into it first,
      // so that the writes complete while the step computes
      if (st + 2 < nsteps) stage(st + 2, std::integral_constant<int, (b + 2) % 3>{});
      if (st < nsteps) step(st, B, std::integral_constant<int, (b + 1) % 3>{}, sa, sb, vv);
      request(st + 5, std::integral_constant<int, (b + 2) % 3>{});
      __syncthreads();  // step st + 2 staged; every wavefront is done with slot b
    });
  }

  // The output, or this piece's partial (m, l, o/l) and, in the last piece of
  // the tile group to finish, the merge of all its pieces. The tile group runs
  // the pieces that start at or before plast; a piece holds l = 0 (and m at
  // the floor) for a column that sees none of its tokens, which weighs nothing
  // in the merge.
  const float oscale = ldexpf(1.0f, I8 ? ev + kSlack - 14 : 0);
  const int nvis = min(plast / a.piece_tokens + 1, npc);
  float lt[NTW];
#pragma unroll
  for (int t = 0; t < NTW; ++t) lt[t] = sum_over_lane_groups(l[t]);
  if (nvis == 1) {
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      if (!colv[t]) continue;
      float* dst = a.out + ((size_t)(qs + qi[t]) * hq + g * G + h) * D;
      const float inv = oscale / lt[t];
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[16 * dt + 4 * gq + i] = o[t][dt][i] * inv;
    }
    return;
  }
  // Partials, piece-major: slot (piece, sequence, query, head). They are
  // written through to the point of coherence of all XCDs (device scope: the
  // o/l vectors as 16-byte stores with the SC1 cache-policy bit, m and l as
  // atomic stores), so the workgroup that merges them needs no cache
  // write-back or invalidate. Lane (n16, gq) holds dims 16 dt + 4 gq .. + 3 of
  // its column: four lanes write 64 contiguous bytes of a row.
  constexpr int kScopeDevice = 16;  // cache-policy operand of buffer instructions: SC1
  const size_t nrow = (size_t)a.num_seqs * a.max_query_len * hq;  // slots per piece
  float* ws_m = a.ws;
  float* ws_l = a.ws + nrow * npc;
  float* ws_o = a.ws + 2 * nrow * npc;
  const int col = (n16 / G) * hq + h;  // the lane's slot past its tile's first
  const uint32_t lane_off = (uint32_t)(col * D + 4 * gq) * 4;
  // tile t's first slot of piece c (the same in every lane)
  auto tile_slot = [&](int t, int c) {
    return (size_t)c * nrow + ((size_t)s * a.max_query_len + qi[t] - n16 / G) * hq + g * G;
  };
  auto o_rsrc = [&](int t, int c) {
    return __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(ws_o + tile_slot(t, c) * D), (short)0, 0x7fffffff,
                                             kRsrcWord3);
  };
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    if (!colv[t]) continue;
    const float inv = lt[t] > 0.f ? oscale / lt[t] : 0.f;
    const auto rs = o_rsrc(t, piece);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, o[t][dt] * inv), rs, lane_off + 64 * dt, 0,
                                             kScopeDevice);
    if (gq == 0) {
      const size_t slot = tile_slot(t, piece) + col;
      __hip_atomic_store(&ws_m[slot], m[t], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&ws_l[slot], lt[t], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  // Every thread's stores complete before the barrier; then one thread counts
  // the arrival, and the workgroup that brings the count to nvis merges.
  __shared__ int sm_last;
  int32_t* counter = a.counters + ((size_t)s * hkv + g) * ngroups + grp;
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  if (threadIdx.x == 0)
    sm_last = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == nvis - 1;
  __syncthreads();
  if (!sm_last) return;
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    if (!colv[t]) continue;
    const float inv = lt[t] > 0.f ? oscale / lt[t] : 0.f;
    // pieces in order, each folded in against the running maximum M:
    //   M' = max(M, m_c),  L' = L 2^(M - M') + l_c 2^(m_c - M'),  O' likewise with l_c (o/l)_c
    float M = kMaxFloor, L = 0.f;
    f32x4 O[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) O[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int c = 0; c < nvis; ++c) {
      float mc, lc;
      f32x4 oc[NDT];
      if (c == piece) {
        mc = m[t];
        lc = lt[t];
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) oc[dt] = o[t][dt] * inv;
      } else {
        const size_t slot = tile_slot(t, c) + col;
        mc = __hip_atomic_load(&ws_m[slot], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        lc = __hip_atomic_load(&ws_l[slot], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const auto rs = o_rsrc(t, c);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
          oc[dt] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, lane_off + 64 * dt, 0,
                                                                                   kScopeDevice));
      }
      const float Mn = fmaxf(M, mc);
      const float rs = __builtin_amdgcn_exp2f(M - Mn);
      const float w = lc * __builtin_amdgcn_exp2f(mc - Mn);
      L = fmaf(L, rs, w);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) O[dt][i] = fmaf(w, oc[dt][i], O[dt][i] * rs);
      M = Mn;
    }
    float* dst = a.out + ((size_t)(qs + qi[t]) * hq + g * G + h) * D;
    const float rl = 1.0f / L;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[16 * dt + 4 * gq + i] = O[dt][i] * rl;
  }
  if (threadIdx.x == 0)  // ready for the next call
    __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <bool I8, int D, int G, int QT, int NTW, int NW>
hipError_t launch_prefill_t(const PrefillLaunch& p, hipStream_t stream) {
  constexpr int WQ = NW * NTW * (16 / G);
  const int64_t ngroups = (p.max_query_len + WQ - 1) / WQ;
  const int64_t nwg = ngroups * p.pieces * p.lv.num_kv_heads * p.num_seqs;
  if (nwg * 64 * NW >= (int64_t{1} << 32)) return hipErrorInvalidConfiguration;  // grid size in threads
  if (p.pieces > 1 && ngroups * p.lv.num_kv_heads * p.num_seqs > kMergeCounters)  // one counter per tile group
    return hipErrorInvalidValue;
  hipLaunchKernelGGL((prefill_kernel<I8, D, G, QT, NTW, NW>), dim3((unsigned)nwg), dim3(64 * NW), 0, stream, p);
  return hipGetLastError();
}

template <bool I8, int D, int G, int QT, int NTW>
hipError_t launch_prefill_w(const PrefillLaunch& p, hipStream_t stream) {
  switch (p.waves) {
    case kPrefillWaves: return launch_prefill_t<I8, D, G, QT, NTW, kPrefillWaves>(p, stream);
    case kPrefillWavesLong: return launch_prefill_t<I8, D, G, QT, NTW, kPrefillWavesLong>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

// Tiles per wavefront: two share each K and V operand read from LDS, except
// where their registers would not fit two wavefronts per SIMD: an fp32 query
// (its lo parts) and a binary16 cache at head_dim 128 (its staging pieces).
template <bool I8, int D, int G>
hipError_t launch_prefill_q(const PrefillLaunch& p, hipStream_t stream) {
  constexpr int NTW = I8 || D == 64 ? 2 : 1;
  switch (p.q_dtype) {
    case kF32: return launch_prefill_w<I8, D, G, kF32, 1>(p, stream);
    case kF16: return launch_prefill_w<I8, D, G, kF16, NTW>(p, stream);
    case kBF16: return launch_prefill_w<I8, D, G, kBF16, NTW>(p, stream);
    default: return hipErrorInvalidValue;
  }
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
