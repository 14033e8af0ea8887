// decode.hip -- decode kernels of libpkv for gfx950.
//
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

#include "device.h"

#include <mutex>

namespace pkv {
namespace {

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
template <bool I8, int D, int G, int QT, bool APPEND, bool SEAL, int NB, bool VALU = false>
__device__ __forceinline__ void decode_body(const DecodeLaunch& a) {
  static_assert(!SEAL || I8, "seal-on-full: INT8 layers");
  static_assert(!VALU || (!APPEND && !SEAL && D == 128 && G <= 2), "vector-ALU contraction: plain decode");
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
  // INT8 V enters the PV product as 1152 + code (two byte permutes per four
  // codes, exact in fp16); lb = sum of p * pscale over the INT8 units, kept
  // in the accumulators' scale, so that 1152 * lb is taken off once at the
  // end. The accumulators then carry 1152 times sum(P) besides the signal:
  // their fp32 rounding adds ~2^-24 * 1152 * sqrt(units) code units (about
  // 1e-4 after the V scale, far inside the attention tolerance).
  float lb = 0.f;
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

  // ---- VALU: the same decode with both contractions on the vector ALUs in
  // fp32, for comparison with the matrix-core form (same loads, ring,
  // bookkeeping and merge). Lane (n16, gq) holds this lane's D/4 dims of K
  // row n16 (the ring's layout) and the query of every head over those dims;
  // the scores are summed over the four lane groups, so every lane of row gq
  // holds token n16's score. For P.V, lane (tg = gq, dm = n16) holds tokens
  // 4 tg + ti of dims 16 dt + dm (the ring's V layout) and fetches their
  // probabilities from lanes 16 tg + 4 tg + ti. INT8 codes are read as
  // unsigned bytes (code + 128) with the 128 taken off through sum(q) and
  // sum(p * vscale). Per head: the running max (wave-uniform, raised by more
  // than kSlack only), this lane's share of the sum, its dims' output.
  constexpr int EPC = 16 / ESZ;  // elements per 16-byte chunk
  float qv[VALU ? G : 1][VALU ? D / 4 : 1];
  float qsum[VALU ? G : 1];
  float vm[VALU ? G : 1], vl[VALU ? G : 1], vps[VALU ? G : 1];
  float vo[VALU ? G : 1][VALU ? NDT : 1];
  if constexpr (VALU) {
    const float qscale = a.softmax_scale * kLog2e;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float qs = 0.f;
#pragma unroll
      for (int c = 0; c < NCH; ++c)
#pragma unroll
        for (int j = 0; j < EPC; ++j) {
          const int e = (16 * gq + 64 * c) / ESZ + j;
          qv[h][c * EPC + j] = load_elem<QT>(a.q, ((size_t)s * hq + g * G + h) * D + e) * qscale;
          qs += qv[h][c * EPC + j];
        }
      qsum[h] = sum_over_lane_groups(qs);
      vm[h] = -INFINITY;
      vl[h] = 0.f;
      vps[h] = 0.f;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) vo[h][dt] = 0.f;
    }
  }
  auto row_sum = [](float x) {  // sum over the 16 lanes of each row, in every lane of the row
    x += dpp_f<kQuadXor1>(x);
    x += dpp_f<kQuadXor2>(x);
    x += dpp_f<kHalfMirror>(x);
    return x + dpp_f<kMirror>(x);
  };
  auto row_max = [](float x) {
    x = fmaxf(x, dpp_f<kQuadXor1>(x));
    x = fmaxf(x, dpp_f<kQuadXor2>(x));
    x = fmaxf(x, dpp_f<kHalfMirror>(x));
    return fmaxf(x, dpp_f<kMirror>(x));
  };

  // One unit of 16 tokens. TAIL: an FP16 unit in an INT8 kernel (a
  // seal-on-full cache's partly filled last block), scored with the fp16
  // query operand and taken with V scale 1; otherwise the kernel's own type.
  auto process = [&](auto tail, const auto& kr, const auto& vr, float kscale, float vscale, int tok0) {
    constexpr bool TAIL = decltype(tail)::value;
    const int nvalid = t1 - tok0;  // rows of this unit inside the partition
    if constexpr (VALU) {
      float sk[G];
#pragma unroll
      for (int h = 0; h < G; ++h) sk[h] = 0.f;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const uint32_t w[4] = {kr[c].x, kr[c].y, kr[c].z, kr[c].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
#pragma unroll
          for (int b = 0; b < 4 / ESZ; ++b) {
            float x;
            if constexpr (I8) x = (float)(((w[k] ^ 0x80808080u) >> (8 * b)) & 0xFFu);  // code + 128
            else x = f16_to_f32((w[k] >> (16 * b)) & 0xFFFFu);
#pragma unroll
            for (int h = 0; h < G; ++h) sk[h] = fmaf(qv[h][c * EPC + k * (4 / ESZ) + b], x, sk[h]);
          }
        }
      }
      float pt[G][4];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float sc = sum_over_lane_groups(sk[h]);
        if constexpr (I8) sc = (sc - 128.f * qsum[h]) * kscale;
        if (n16 >= nvalid) sc = -INFINITY;  // rows past the partition's end
        const float um = uniform_f(row_max(sc));  // finite: every unit has a valid row
        if (um > vm[h] + kSlack) {  // wave-uniform
          const float alpha = __builtin_amdgcn_exp2f(vm[h] - um);
          vl[h] *= alpha;
          vps[h] *= alpha;
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) vo[h][dt] *= alpha;
          vm[h] = um;
        }
        const float p = __builtin_amdgcn_exp2f(sc - vm[h]);
        vl[h] += p;
        const float pv = I8 ? p * vscale : p;
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) pt[h][ti] = __shfl(pv, 20 * gq + ti);  // lane 16 gq + 4 gq + ti
        if constexpr (I8) vps[h] += (pt[h][0] + pt[h][1]) + (pt[h][2] + pt[h][3]);
      }
      uint32_t vw[4 * NCH];
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        vw[4 * c] = vr[c].x; vw[4 * c + 1] = vr[c].y; vw[4 * c + 2] = vr[c].z; vw[4 * c + 3] = vr[c].w;
      }
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
          float x;
          if constexpr (I8) {  // word dt: tokens 4 gq + 0..3 of dim 16 dt + n16 (code + 128)
            x = (float)((vw[dt] >> (8 * ti)) & 0xFFu);
          } else {
            x = f16_to_f32((vw[2 * dt + (ti >> 1)] >> (16 * (ti & 1))) & 0xFFFFu);
            if (4 * gq + ti >= nvalid) x = 0.f;  // rows past the end may hold any bits
          }
#pragma unroll
          for (int h = 0; h < G; ++h) vo[h][dt] = fmaf(pt[h][ti], x, vo[h][dt]);
        }
      }
      return;
    }

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
      if constexpr (I8) lb *= ao;  // (lanes n16 < 8: alpha * 2^(ev - evn))
      m = mn;
      ev = evn;
    }

    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(sc[i] - m);  // < 2^kSlack in head columns
    const float lsum = (p[0] + p[1]) + (p[2] + p[3]);
    l += lsum;
    const float pscale = ldexpf(I8 ? vscale : 1.0f, 14 - kSlack - ev);  // p * pscale < 2^14
    if constexpr (I8 && !TAIL) lb = fmaf(lsum, pscale, lb);
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
        av = biased_i8x4_to_f16x4_plus1152(vw[dt]);
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

  __shared__ float sm_o[kWaves][G][D];
  __shared__ float sm_m[kWaves][G];
  __shared__ float sm_l[kWaves][G];
  __shared__ int sm_last;
  if constexpr (VALU) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float lt = row_sum(vl[h]);  // a row holds each of the wave's tokens once
      const float bias = I8 ? 128.f * sum_over_lane_groups(vps[h]) : 0.f;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const float od = sum_over_lane_groups(vo[h][dt]) - bias;
        if (gq == 0) sm_o[wave][h][16 * dt + n16] = od;
      }
      if (lane == 0) { sm_m[wave][h] = vm[h]; sm_l[wave][h] = lt; }
    }
  }

  // hi + lo columns, back to unit scale; l summed over the four lane groups
  const float oscale = ldexpf(1.0f, ev + kSlack - 14);
  l = sum_over_lane_groups(l);
  const float bias = I8 ? 1152.f * sum_over_lane_groups(lb) : 0.f;  // the INT8 V offset, whole column
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) o[dt][i] = (o[dt][i] + dpp_f<kRowShl8>(o[dt][i]) - bias) * oscale;

  if (colv && !VALU) {
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
// Plain decode with both contractions on the vector ALUs (fp32 FMAs) instead
// of the matrix cores, kept to compare the two forms; same ring depths. The
// query of both heads over a lane's dims takes 64 more registers, so this
// variant is allowed two wavefronts per SIMD (up to 256 registers) and does
// not spill.
template <bool I8, int D, int G, int QT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 8)))
void decode_kernel_valu(const DecodeLaunch a) {
  decode_body<I8, D, G, QT, false, false, I8 ? 3 : 2, true>(a);
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
  if constexpr (D == 128 && G <= 2) {
    if (d.valu_contraction) {  // plain decode only (the host checks the rest)
      hipLaunchKernelGGL((decode_kernel_valu<I8, D, G, QT>), grid, dim3(kThreads), 0, stream, d);
      return;
    }
  }
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

}  // namespace

// A plain streaming read (measurement): each thread reads 16-byte pieces i,
// i + S, i + 2S, ... (S = all threads of the grid), four loads in flight,
// and folds them into one word it stores, so the loads cannot be dropped.
// Consecutive threads read consecutive pieces, so every workgroup streams
// whole 4 KB runs, as the decode kernels' units are.
__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* __restrict__ buf, size_t n16,
                                                          uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = buf[i], b = buf[i + stride], c = buf[i + 2 * stride], d = buf[i + 3 * stride];
    acc ^= (a.x ^ a.y ^ a.z ^ a.w) ^ (b.x ^ b.y ^ b.z ^ b.w) ^ (c.x ^ c.y ^ c.z ^ c.w) ^ (d.x ^ d.y ^ d.z ^ d.w);
  }
  for (; i < n16; i += stride) {
    const uint4 a = buf[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  sink[(size_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

hipError_t launch_stream_read(const void* buf, size_t bytes, int32_t workgroups, uint32_t* sink,
                              hipStream_t stream) {
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)workgroups), dim3(256), 0, stream,
                     (const uint4*)buf, bytes / 16, sink);
  return hipGetLastError();
}

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

}  // namespace pkv
