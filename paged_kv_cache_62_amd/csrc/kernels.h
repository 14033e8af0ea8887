// kernels.h -- launch interface between the host library (pool.cpp) and the
// gfx950 kernels (append.hip, decode.hip, prefill.hip). Internal to libpkv.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

// Element type codes, same values as pkv_dtype in pkv.h.
enum : int { kF32 = 0, kF16 = 1, kBF16 = 2, kI8 = 3 };

// Tile layouts. A (block, KV head) tile holds bs tokens x d elements.
//  K: row-major, element (t, dim) at t*d + dim, so a token row is contiguous
//     and a 16-token slice is the A operand of the QK matrix-core product
//     read straight from memory.
//  V: split into 16-token sub-tiles; inside one, token t = 4*tg + ti and
//     dim = 16*dt + dm sit at ((tg*16 + dm) * (d/16) + dt) * 4 + ti, so lane
//     tg*16 + dm of a wavefront reads d/4 contiguous elements holding, for
//     every 16-dim tile dt, the 4 tokens that make up its A operand of the
//     PV product (16 dims x 16 tokens). INT8 V codes are stored biased by
//     128 (code ^ 0x80), which the decode kernel turns into fp16 with byte
//     permutes alone.
__host__ __device__ inline int64_t k_tile_offset(int t, int dim, int d) {
  return (int64_t)t * d + dim;
}
__host__ __device__ inline int64_t v_tile_offset(int t, int dim, int d) {
  const int sub = t >> 4, tt = t & 15;
  const int tg = tt >> 2, ti = tt & 3, dm = dim & 15, dt = dim >> 4;
  return (int64_t)sub * 16 * d + ((int64_t)(tg * 16 + dm) * (d / 16) + dt) * 4 + ti;
}

// One layer's view of the cache. Codes are [N][Hkv][tile] per K and V;
// scales [N][Hkv] per K and V (int8 only), and beside each scale the largest
// |code| among the rows written so far (0 for a block of zero codes). The
// append kernels keep it up to date; the decode step uses it to decide, with
// no pass over the old codes, whether a new row grows the block's scale.
struct LayerView {
  void* k_codes;
  void* v_codes;
  float* k_scales;
  float* v_scales;
  int32_t* k_qmax;
  int32_t* v_qmax;
  // Seal-on-full INT8 layer (seal != 0): FP16 staging tiles [N][Hkv][tile]
  // per K and V, laid out as an FP16 cache's. A block's rows stay there
  // while it is a sequence's partly filled last block; the append that
  // writes its last row quantizes the whole block into the INT8 tile.
  void* tail_k;
  void* tail_v;
  int32_t seal;
  int32_t num_blocks, num_kv_heads, head_dim, block_size, kv_dtype;
};

hipError_t launch_append(const LayerView& lv, const void* k, const void* v, int in_dtype,
                         const int64_t* slots, int32_t n_tokens, hipStream_t stream);

struct DecodeLaunch {
  LayerView lv;
  const void* q;
  int q_dtype;
  int32_t num_q_heads;
  const int32_t* tables;
  int32_t max_blocks;
  const int32_t* lens;
  int32_t num_seqs;
  int32_t partition_tokens;  // multiple of block_size (and of 16)
  int32_t max_partitions;    // ceil(max_context_len / partition_tokens)
  float softmax_scale;
  float* out;
  int32_t* counters;         // [num_seqs][Hkv] arrival counters (zero between calls)
  float* ws;                 // partials m, l [num_seqs][Hq][P], o [num_seqs][Hq][P][d]
  int32_t fused_merge;       // 1: the last workgroup of a (seq, KV head) merges
  int32_t valu_contraction;  // 1: both contractions on the vector ALUs (comparison variant:
                             // plain decode, head_dim 128, 1 or 2 query heads per KV head)
  // Decode step: the new token of each sequence (position len-1), rows of
  // [num_seqs][Hkv][d] in q's dtype, written into the cache before it is
  // read. Null for plain decode.
  const void* k_new;
  const void* v_new;
};

// Chunked prefill: the last q_len = query_start[s+1] - query_start[s] of
// each sequence's lens[s] cached tokens are queries, attending causally.
struct PrefillLaunch {
  LayerView lv;
  const void* q;              // [total][Hq][d] of q_dtype
  int q_dtype;
  int32_t num_q_heads;
  const int32_t* query_start; // [num_seqs + 1]
  int32_t max_query_len;
  const int32_t* tables;
  int32_t max_blocks;
  const int32_t* lens;
  int32_t num_seqs;
  float softmax_scale;
  float* out;                 // [total][Hq][d] fp32
  // Context split: pieces of piece_tokens (a multiple of 64; the last piece
  // takes the rest), each (query tile group, piece) one workgroup; with
  // pieces > 1 their partials go to ws and the last piece of each tile group
  // to finish merges them.
  int32_t pieces;
  int32_t piece_tokens;
  int32_t waves;              // wavefronts per workgroup: kPrefillWaves or kPrefillWavesLong
  int32_t* counters;          // [num_seqs][Hkv][tile groups] arrival counters (zero between calls)
  float* ws;                  // partials m, l [num_seqs][max_query_len][Hq][pieces], then o (x head_dim)
};

hipError_t launch_prefill(const PrefillLaunch& p, hipStream_t stream);

// Wavefronts of a prefill workgroup, and the query tokens a four-wavefront
// workgroup takes for planning: two 16-column tiles per wavefront (one for an
// fp32 query), a tile being 16 / group query tokens. (A binary16 cache at
// head_dim 128 runs one tile per wavefront; the plan does not depend on the
// layer.) Launches whose context the automatic plan cuts into pieces, or
// whose four-wavefront grid would take two or more rounds (at two workgroups
// per compute unit), run eight wavefronts per workgroup instead: twice the
// query tiles share each staged step of the context, in half as many
// workgroups (one per compute unit at two wavefronts per SIMD); the piece
// count comes out the same.
constexpr int kPrefillWaves = 4;
constexpr int kPrefillWavesLong = 8;
constexpr int prefill_query_tokens_per_workgroup(int group, int q_dtype) {
  return kPrefillWaves * (q_dtype == kF32 ? 1 : 2) * (16 / group);
}

// The context split of a prefill launch: piece_tokens (0: automatic, else a
// multiple of 64) -> the piece size used, the number of pieces and the
// wavefronts per workgroup. The automatic split cuts the context only when
// the query tiles alone give fewer than two four-wavefront workgroups per
// compute unit (cus of them), and keeps pieces of at least 1024 tokens. The
// launch runs kPrefillWavesLong wavefronts per workgroup when the
// four-wavefront workgroups of a sequence and KV head come in an even number
// (so the larger ones leave no more query slots idle) and either the
// automatic split cuts (whatever piece_tokens is) or those workgroups make
// two or more rounds of two per compute unit.
void prefill_plan(int32_t cus, int32_t num_seqs, int32_t num_kv_heads, int32_t group, int q_dtype,
                  int32_t max_query_len, int32_t max_context_len, int32_t piece_tokens, int32_t* piece_out,
                  int32_t* pieces_out, int32_t* waves_out);
// Query tile groups per (sequence, KV head) of any prefill launch: at most
// this many (at least one 16 / group query-token tile per wavefront).
constexpr int32_t prefill_tile_groups_bound(int32_t max_query_len, int32_t group) {
  return (max_query_len + kPrefillWaves * (16 / group) - 1) / (kPrefillWaves * (16 / group));
}
// Workspace bytes of a launch with this many pieces (0 for one piece): the
// counter prefix, then the partials.
size_t prefill_workspace_bytes(int32_t num_seqs, int32_t max_query_len, int32_t num_q_heads, int32_t head_dim,
                               int32_t pieces);

// Arrival counters of the merges that the last workgroup to finish does: the
// first kMergeCounterBytes of every decode or prefill workspace, whatever the
// call's sizes, so that no call's partials land on counters a later call
// reads (every call leaves the counters it used at zero).
constexpr size_t kMergeCounterBytes = size_t{64} << 10;
constexpr int64_t kMergeCounters = int64_t(kMergeCounterBytes / sizeof(int32_t));

// Longest decode partition (tokens) the kernels take.
constexpr int32_t kMaxPartitionTokens = 4096;

// True if the kernels cover this head_dim / group size.
bool decode_supported(int head_dim, int group);

// Compute units of the current HIP device (a partitioned GPU exposes fewer;
// 256 if the device cannot be asked), queried once per device.
int device_compute_units();

hipError_t launch_decode(const DecodeLaunch& d, hipStream_t stream);

// Workspace: the counter prefix, then the partials (0 bytes for one partition).
size_t decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t max_partitions);

// Measurement: a plain streaming read of `bytes` (a multiple of 16) with
// `workgroups` 256-thread workgroups; sink holds workgroups * 256 words.
hipError_t launch_stream_read(const void* buf, size_t bytes, int32_t workgroups, uint32_t* sink,
                              hipStream_t stream);

// The library's own decode workspace for callers that cannot allocate: a
// device array of kScratchBytes on every GPU the library runs on, zero-filled
// once. scratch_setup() finds its address on the current device (once per
// device; call it with that device current); scratch_ptr() returns it, or
// null before set-up. Calls that use it on one GPU share it.
constexpr size_t kScratchBytes = size_t{16} << 20;
hipError_t scratch_setup();
void* scratch_ptr(int device);

}  // namespace pkv
