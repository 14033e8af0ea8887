// kernels.h -- launch interface between the host library (pool.cpp) and the
// gfx950 kernels (kernels.hip). Internal to libpkv.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

// Element type codes, same values as pkv_dtype in pkv.h.
enum : int { kF32 = 0, kF16 = 1, kBF16 = 2, kI8 = 3 };

// One layer's view of the cache. Codes are [N][Hkv][bs][d] per K and V;
// scales [N][Hkv] per K and V (int8 only).
struct LayerView {
  void* k_codes;
  void* v_codes;
  float* k_scales;
  float* v_scales;
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
  float* ws;                 // partials; may be null when max_partitions == 1
};

// True if the kernels cover this head_dim / group size.
bool decode_supported(int head_dim, int group);

hipError_t launch_decode(const DecodeLaunch& d, hipStream_t stream);

// Bytes of workspace for the partials (m, l, o/l).
size_t decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                              int32_t max_partitions);

}  // namespace pkv
