// host.h -- host-side helpers shared by the translation units of libpkv
// (pool.cpp defines them). Internal to the library.
#pragma once

#include <stdint.h>

#include "../../include/pkv.h"

namespace pkv {

// Set the per-thread message pkv_last_error() returns.
void set_last_error(const char* msg);

// Tokens per block of a pool.
int32_t pool_block_size(const pkv_pool* pool);

// Blocks in a pool's free queue (O(1)).
int64_t pool_free_blocks(const pkv_pool* pool);

}  // namespace pkv
