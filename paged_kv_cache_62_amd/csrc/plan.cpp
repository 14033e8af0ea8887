// plan.cpp -- host-side sizes and device facts the decode launches are
// planned with (workspace layout, supported shapes, compute units). Shared
// by the host library (pool.cpp) and the kernel launchers (*.hip);
// host code only.

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <atomic>

#include "kernels.h"

namespace pkv {

int device_compute_units() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

bool decode_supported(int head_dim, int group) {
  return (head_dim == 64 || head_dim == 128) && (group == 1 || group == 2 || group == 4);
}

size_t decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t max_partitions) {
  if (max_partitions <= 1) return 0;
  const size_t rows = (size_t)num_seqs * num_q_heads * max_partitions;
  return kMergeCounterBytes + rows * (2 + (size_t)head_dim) * sizeof(float);
}

void prefill_plan(int32_t cus, int32_t num_seqs, int32_t num_kv_heads, int32_t group, int q_dtype,
                  int32_t max_query_len, int32_t max_context_len, int32_t piece_tokens, int32_t* piece_out,
                  int32_t* pieces_out, int32_t* waves_out) {
  constexpr int32_t kMinPiece = 1024;
  const int32_t ctx = max_context_len > 0 ? max_context_len : 1;
  const int32_t wq = prefill_query_tokens_per_workgroup(group, q_dtype);
  const int32_t groups = (max_query_len + wq - 1) / wq;  // of four-wavefront workgroups
  const int64_t items = (int64_t)groups * num_kv_heads * num_seqs;
  const int64_t want = 2 * (int64_t)cus;
  int64_t na = items >= want || items <= 0 ? 1 : (want + items - 1) / items;
  na = std::min<int64_t>(na, std::max(1, ctx / kMinPiece));
  const int32_t t = piece_tokens > 0 ? piece_tokens : (int32_t)((((int64_t)ctx + na - 1) / na + 63) / 64 * 64);
  const int32_t n = (int32_t)(((int64_t)ctx + t - 1) / t);
  *piece_out = n > 1 ? t : std::max(t, ((ctx + 63) / 64) * 64);
  *pieces_out = n;
  // eight wavefronts only where they leave no more query slots idle than four,
  // and where their grid still has a workgroup for every compute unit
  // through its rounds: a cut context, or two or more rounds of four
  const bool many = items >= 4 * (int64_t)cus;
  *waves_out = groups % 2 == 0 && (na > 1 || many) ? kPrefillWavesLong : kPrefillWaves;
}

size_t prefill_workspace_bytes(int32_t num_seqs, int32_t max_query_len, int32_t num_q_heads, int32_t head_dim,
                               int32_t pieces) {
  if (pieces <= 1) return 0;
  const size_t slots = (size_t)num_seqs * max_query_len * num_q_heads * pieces;
  return kMergeCounterBytes + slots * (2 + (size_t)head_dim) * sizeof(float);
}

}  // namespace pkv
