// pool.cpp -- host side of libpkv: the block pool, its allocator and the C ABI.
//
// Allocator ("连续批处理与KV缓存" §4.2): the free blocks form one FIFO queue,
// kept here as a fixed ring of N entries -- allocation takes from the front,
// freeing appends to the back, O(1) per block and no fragmentation. Each
// sequence owns its block table (logical -> physical, "vLLM核心概念" §3.2)
// and a length; each block carries a reference count so forked sequences
// can share a prefix, and the first write into a shared, partly filled
// block copies it first (copy-on-write, same section).
//
// Device memory (one arena): codes [L][2][N][Hkv][bs][d], each layer in its
// own element type (one for all, or per layer: "轻量级推理引擎实战" §3.2 keeps
// the first and last layers in FP16), followed, when any layer is INT8, by
// per-(block, head) metadata [L][2][2][N][Hkv] of 4-byte words: for each layer
// and K|V, the fp32 scales, then the largest |code| of each (block, head)
// among its written rows (int32).

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <unordered_map>
#include <vector>

#include "../../include/pkv.h"
#include "host.h"
#include "kernels.h"

namespace {

thread_local std::string g_last_error;

pkv_status fail(pkv_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

pkv_status ok() {
  g_last_error.clear();
  return PKV_OK;
}

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

size_t elem_bytes(pkv_dtype t) { return t == PKV_I8 ? 1 : 2; }

struct Seq {
  std::vector<int32_t> blocks;
  int64_t len = 0;
};

}  // namespace

struct pkv_pool {
  pkv_pool_config cfg{};
  // FIFO free queue as a ring buffer: entries [head, head + count) mod N.
  std::vector<int32_t> ring;
  int64_t head = 0, count = 0;
  std::vector<int32_t> refcount;
  int64_t shared = 0;                   // blocks with reference count > 1
  std::unordered_map<int64_t, Seq> seqs;
  int64_t cow_total = 0;
  int32_t cus = 256;                    // compute units of the pool's device (planning)
  // device side
  int device = -1;
  char* arena = nullptr;
  bool owns_arena = false;
  size_t tile_elems = 0;               // bs * d
  std::vector<pkv_dtype> ldt;           // element type of each layer
  std::vector<size_t> layer_off;        // byte offset of each layer's K slice (V follows)
  size_t codes_bytes = 0;               // all layers
  float* scales = nullptr;              // metadata [L][2][scale | qmax][N][Hkv] (int8 layers)
  char* tails = nullptr;                // seal_on_full: FP16 staging [INT8 layers][2][N][Hkv][tile]
  std::vector<int32_t> tail_index;      // seal_on_full: each layer's index among the INT8 layers, or -1
  size_t tail_slice = 0;                // bytes of one (INT8 layer, K|V) staging slice

  // one (layer, K|V) slice of codes: N*Hkv*bs*d*elem
  size_t slice_bytes(int32_t layer) const {
    return (size_t)cfg.num_blocks * cfg.num_kv_heads * tile_elems * elem_bytes(ldt[layer]);
  }

  int32_t pop_front() {
    const int32_t b = ring[head];
    head = (head + 1) % cfg.num_blocks;
    --count;
    refcount[b] = 1;
    return b;
  }
  void push_back(int32_t b) {
    ring[(head + count) % cfg.num_blocks] = b;
    ++count;
  }
  // The k-th block the next pops will return (k < count), without popping.
  int32_t peek(int64_t k) const { return ring[(head + k) % cfg.num_blocks]; }
  void add_ref(int32_t b) {
    if (++refcount[b] == 2) ++shared;
  }
  // One reference less; a block reaching zero goes to the back of the queue.
  void drop_ref(int32_t b) {
    const int32_t r = --refcount[b];
    if (r == 1) --shared;
    if (r == 0) push_back(b);
  }
  pkv::LayerView layer_view(int32_t layer) const {
    pkv::LayerView lv{};
    lv.k_codes = arena + layer_off[layer];
    lv.v_codes = arena + layer_off[layer] + slice_bytes(layer);
    const size_t sc_slice = (size_t)cfg.num_blocks * cfg.num_kv_heads;
    lv.k_scales = scales ? scales + (size_t)(4 * layer) * sc_slice : nullptr;
    lv.k_qmax = scales ? (int32_t*)(scales + (size_t)(4 * layer + 1) * sc_slice) : nullptr;
    lv.v_scales = scales ? scales + (size_t)(4 * layer + 2) * sc_slice : nullptr;
    lv.v_qmax = scales ? (int32_t*)(scales + (size_t)(4 * layer + 3) * sc_slice) : nullptr;
    lv.num_blocks = cfg.num_blocks;
    lv.num_kv_heads = cfg.num_kv_heads;
    lv.head_dim = cfg.head_dim;
    lv.block_size = cfg.block_size;
    lv.kv_dtype = ldt[layer];
    if (tails && tail_index[layer] >= 0) {
      lv.seal = 1;
      lv.tail_k = tails + (size_t)(2 * tail_index[layer]) * tail_slice;
      lv.tail_v = tails + (size_t)(2 * tail_index[layer] + 1) * tail_slice;
    }
    return lv;
  }
};

namespace {

pkv_status check_config(const pkv_pool_config* c) {
  if (!c) return fail(PKV_ERR_INVALID_ARG, "config is NULL");
  if (c->num_layers < 1 || c->num_kv_heads < 1 || c->num_blocks < 1)
    return fail(PKV_ERR_INVALID_ARG, "num_layers, num_kv_heads and num_blocks must be >= 1");
  if (c->kv_dtype != PKV_F16 && c->kv_dtype != PKV_I8)
    return fail(PKV_ERR_INVALID_ARG, "kv_dtype must be PKV_F16 or PKV_I8");
  if (c->layer_kv_dtype)
    for (int32_t l = 0; l < c->num_layers; ++l)
      if (c->layer_kv_dtype[l] != PKV_F16 && c->layer_kv_dtype[l] != PKV_I8)
        return fail(PKV_ERR_INVALID_ARG, "layer_kv_dtype[%d] must be PKV_F16 or PKV_I8", l);
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, "head_dim %d: supported are 64 and 128", c->head_dim);
  if (c->block_size != 16 && c->block_size != 32 && c->block_size != 64)
    return fail(PKV_ERR_UNSUPPORTED, "block_size %d: supported are 16, 32 and 64", c->block_size);
  return PKV_OK;
}

pkv_dtype layer_dtype(const pkv_pool_config* c, int32_t layer) {
  return c->layer_kv_dtype ? (pkv_dtype)c->layer_kv_dtype[layer] : c->kv_dtype;
}

size_t required_bytes(const pkv_pool_config* c) {
  const size_t elems = (size_t)c->num_blocks * c->num_kv_heads * c->block_size * c->head_dim;
  size_t codes = 0;
  bool any_i8 = false;
  for (int32_t l = 0; l < c->num_layers; ++l) {
    codes += 2 * elems * elem_bytes(layer_dtype(c, l));
    any_i8 = any_i8 || layer_dtype(c, l) == PKV_I8;
  }
  size_t total = round_up(codes, 256);
  if (any_i8)
    total += round_up((size_t)c->num_layers * 4 * c->num_blocks * c->num_kv_heads * sizeof(float), 256);
  if (c->seal_on_full) {  // FP16 staging tiles for every INT8 layer
    int32_t n_i8 = 0;
    for (int32_t l = 0; l < c->num_layers; ++l) n_i8 += layer_dtype(c, l) == PKV_I8;
    total += round_up(2 * (size_t)n_i8 * elems * 2, 256);
  }
  return total;
}

pkv_status hip_fail(hipError_t e, const char* what) {
  return fail(PKV_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

int64_t nblocks_for(int64_t len, int64_t bs) { return (len + bs - 1) / bs; }

}  // namespace

// Copy-on-write of one block into another, on `stream`: whole (block, head)
// tiles of every layer and K/V, one 2-D copy per run of layers of one element
// type (one row per (layer, K|V) slice); the FP16 staging tiles of a
// seal-on-full pool the same way; then the scales and largest codes, one row
// per (layer, K|V, scale|qmax).
static hipError_t copy_block_async(pkv_pool* pool, int32_t old, int32_t fresh, hipStream_t st) {
  hipError_t e = hipSuccess;
  const int32_t L = pool->cfg.num_layers;
  for (int32_t l0 = 0; l0 < L && e == hipSuccess;) {
    int32_t l1 = l0 + 1;
    while (l1 < L && pool->ldt[l1] == pool->ldt[l0]) ++l1;
    const size_t tile_bytes = (size_t)pool->cfg.num_kv_heads * pool->tile_elems * elem_bytes(pool->ldt[l0]);
    char* base = pool->arena + pool->layer_off[l0];
    e = hipMemcpy2DAsync(base + (size_t)fresh * tile_bytes, pool->slice_bytes(l0),
                         base + (size_t)old * tile_bytes, pool->slice_bytes(l0), tile_bytes,
                         2 * (size_t)(l1 - l0), hipMemcpyDeviceToDevice, st);
    l0 = l1;
  }
  if (e == hipSuccess && pool->tails) {  // staged FP16 rows: one slice per (INT8 layer, K|V)
    int32_t n_i8 = 0;
    for (int32_t l = 0; l < L; ++l) n_i8 += pool->tail_index[l] >= 0;
    const size_t t16 = (size_t)pool->cfg.num_kv_heads * pool->tile_elems * 2;
    e = hipMemcpy2DAsync(pool->tails + (size_t)fresh * t16, pool->tail_slice,
                         pool->tails + (size_t)old * t16, pool->tail_slice, t16, 2 * (size_t)n_i8,
                         hipMemcpyDeviceToDevice, st);
  }
  if (e == hipSuccess && pool->scales) {
    const size_t sc_row = (size_t)pool->cfg.num_kv_heads * sizeof(float);
    const size_t sc_pitch = (size_t)pool->cfg.num_blocks * sc_row;
    e = hipMemcpy2DAsync((char*)pool->scales + (size_t)fresh * sc_row, sc_pitch,
                         (char*)pool->scales + (size_t)old * sc_row, sc_pitch, sc_row,
                         4 * (size_t)L, hipMemcpyDeviceToDevice, st);
  }
  return e;
}

namespace pkv {
void set_last_error(const char* msg) { g_last_error = msg ? msg : ""; }
int32_t pool_block_size(const pkv_pool* pool) { return pool->cfg.block_size; }
int64_t pool_free_blocks(const pkv_pool* pool) { return pool->count; }
}  // namespace pkv

extern "C" {

size_t pkv_pool_required_bytes(const pkv_pool_config* cfg) {
  if (check_config(cfg) != PKV_OK) return 0;
  return required_bytes(cfg);
}

pkv_status pkv_pool_create(const pkv_pool_config* cfg, pkv_pool** out) {
  if (!out) return fail(PKV_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  pkv_status st = check_config(cfg);
  if (st != PKV_OK) return st;
  const int32_t N = cfg->num_blocks;
  std::vector<int32_t> order(N);
  if (cfg->initial_free_order) {
    std::vector<char> seen(N, 0);
    for (int32_t i = 0; i < N; ++i) {
      const int32_t b = cfg->initial_free_order[i];
      if (b < 0 || b >= N || seen[b])
        return fail(PKV_ERR_INVALID_ARG, "initial_free_order is not a permutation of [0, %d)", N);
      seen[b] = 1;
      order[i] = b;
    }
  } else {
    for (int32_t i = 0; i < N; ++i) order[i] = i;
  }
  const size_t need = required_bytes(cfg);
  if (!cfg->host_only && cfg->device_arena && cfg->arena_bytes < need)
    return fail(PKV_ERR_INVALID_ARG, "device_arena holds %zu bytes, the pool needs %zu",
                cfg->arena_bytes, need);

  auto* p = new pkv_pool;
  p->cfg = *cfg;
  p->cfg.initial_free_order = nullptr;  // copied below, not retained
  p->ring = order;
  p->head = 0;
  p->count = N;
  p->refcount.assign(N, 0);
  p->cfg.layer_kv_dtype = nullptr;      // copied below, not retained
  p->tile_elems = (size_t)cfg->block_size * cfg->head_dim;
  bool any_i8 = false;
  for (int32_t l = 0; l < cfg->num_layers; ++l) {
    p->ldt.push_back(layer_dtype(cfg, l));
    any_i8 = any_i8 || p->ldt[l] == PKV_I8;
    p->layer_off.push_back(p->codes_bytes);
    p->codes_bytes += 2 * p->slice_bytes(l);
  }
  if (!cfg->host_only) {
    hipError_t e = hipGetDevice(&p->device);
    if (e != hipSuccess) { delete p; return hip_fail(e, "hipGetDevice"); }
    p->cus = pkv::device_compute_units();
    // the library's decode scratch on this device (pkv_decode_step_noalloc)
    e = pkv::scratch_setup();
    if (e != hipSuccess) { delete p; return hip_fail(e, "decode scratch set-up"); }
    if (cfg->device_arena) {
      p->arena = (char*)cfg->device_arena;
    } else {
      e = hipMalloc((void**)&p->arena, need);
      if (e != hipSuccess) { delete p; return hip_fail(e, "hipMalloc(pool arena)"); }
      p->owns_arena = true;
    }
    size_t at = round_up(p->codes_bytes, 256);
    if (any_i8) {
      p->scales = (float*)(p->arena + at);
      at += round_up((size_t)cfg->num_layers * 4 * N * cfg->num_kv_heads * sizeof(float), 256);
    }
    if (cfg->seal_on_full && any_i8) {
      p->tails = p->arena + at;
      p->tail_slice = (size_t)N * cfg->num_kv_heads * p->tile_elems * 2;
      int32_t k = 0;
      for (int32_t l = 0; l < cfg->num_layers; ++l) p->tail_index.push_back(p->ldt[l] == PKV_I8 ? k++ : -1);
    }
  }
  *out = p;
  return ok();
}

void pkv_pool_destroy(pkv_pool* pool) {
  if (!pool) return;
  if (pool->owns_arena && pool->arena) (void)hipFree(pool->arena);
  delete pool;
}

pkv_status pkv_seq_allocate(pkv_pool* pool, int64_t seq, int32_t n_tokens, int64_t* slots_out) {
  if (!pool) return fail(PKV_ERR_INVALID_ARG, "pool is NULL");
  if (n_tokens < 0) return fail(PKV_ERR_INVALID_ARG, "n_tokens %d < 0", n_tokens);
  if (pool->seqs.count(seq)) return fail(PKV_ERR_SEQ_EXISTS, "sequence %lld already exists", (long long)seq);
  const int64_t bs = pool->cfg.block_size;
  const int64_t need = nblocks_for(n_tokens, bs);
  if (need > pool->count)
    return fail(PKV_ERR_OOM, "sequence %lld needs %lld blocks, %lld free", (long long)seq,
                (long long)need, (long long)pool->count);
  Seq s;
  s.blocks.reserve(need);
  for (int64_t j = 0; j < need; ++j) s.blocks.push_back(pool->pop_front());
  s.len = n_tokens;
  if (slots_out)
    for (int64_t t = 0; t < n_tokens; ++t) slots_out[t] = (int64_t)s.blocks[t / bs] * bs + t % bs;
  pool->seqs.emplace(seq, std::move(s));
  return ok();
}

pkv_status pkv_seq_append_slots(pkv_pool* pool, const int64_t* seqs, int32_t n_seqs,
                                const int32_t* n_new, int64_t* slots_out, void* stream) {
  if (!pool) return fail(PKV_ERR_INVALID_ARG, "pool is NULL");
  if (n_seqs < 0 || (n_seqs > 0 && (!seqs || !n_new)))
    return fail(PKV_ERR_INVALID_ARG, "bad sequence list");
  const int64_t bs = pool->cfg.block_size;
  // Validate, and count the blocks the whole call will take (new blocks plus
  // copy-on-write targets), tracking reference counts that earlier sequences
  // of this call release by copying.
  std::vector<Seq*> ss(n_seqs);
  std::unordered_map<int64_t, int> seen;
  for (int32_t i = 0; i < n_seqs; ++i) {
    if (n_new[i] < 0) return fail(PKV_ERR_INVALID_ARG, "n_new[%d] = %d < 0", i, n_new[i]);
    if (!seen.emplace(seqs[i], i).second)
      return fail(PKV_ERR_INVALID_ARG, "sequence %lld listed twice", (long long)seqs[i]);
    auto it = pool->seqs.find(seqs[i]);
    if (it == pool->seqs.end())
      return fail(PKV_ERR_UNKNOWN_SEQ, "unknown sequence %lld", (long long)seqs[i]);
    ss[i] = &it->second;
  }
  // The call's pops, in order, are the queue's first `need` entries: plan
  // the copy-on-write targets (tracking reference counts that earlier
  // sequences of this call release by copying) and count the blocks.
  struct Cow { int32_t old, fresh; };
  std::vector<Cow> cows;
  int64_t need = 0;
  std::unordered_map<int32_t, int32_t> released;
  for (int32_t i = 0; i < n_seqs; ++i) {
    if (n_new[i] == 0) continue;
    const Seq& s = *ss[i];
    const int64_t have = (int64_t)s.blocks.size();
    if (s.len % bs != 0) {  // first new token lands in the partly filled last block
      const int32_t b = s.blocks[have - 1];
      if (pool->refcount[b] - released[b] > 1) {
        if (need < pool->count) cows.push_back({b, pool->peek(need)});
        ++need;
        ++released[b];
      }
    }
    need += nblocks_for(s.len + n_new[i], bs) - have;
  }
  if (need > pool->count)
    return fail(PKV_ERR_NO_FREE_BLOCK, "append needs %lld blocks, %lld free", (long long)need,
                (long long)pool->count);

  // The copies go out before anything changes: if one cannot be enqueued the
  // call fails with the pool as it was (the targets are still free blocks).
  if (pool->arena)
    for (const Cow& c : cows) {
      const hipError_t e = copy_block_async(pool, c.old, c.fresh, (hipStream_t)stream);
      if (e != hipSuccess) return hip_fail(e, "copy-on-write copy");
    }

  int64_t o = 0;
  for (int32_t i = 0; i < n_seqs; ++i) {
    Seq& s = *ss[i];
    if (n_new[i] == 0) continue;
    if (s.len % bs != 0) {
      const int64_t j = (int64_t)s.blocks.size() - 1;
      const int32_t old = s.blocks[j];
      if (pool->refcount[old] > 1) {  // a planned copy: pops come in the planned order
        const int32_t fresh = pool->pop_front();
        pool->drop_ref(old);  // stays referenced (it was shared)
        s.blocks[j] = fresh;
        pool->cow_total += 1;
      }
    }
    for (int64_t t = s.len; t < s.len + n_new[i]; ++t) {
      if (t / bs == (int64_t)s.blocks.size()) s.blocks.push_back(pool->pop_front());
      if (slots_out) slots_out[o] = (int64_t)s.blocks[t / bs] * bs + t % bs;
      ++o;
    }
    s.len += n_new[i];
  }
  return ok();
}

pkv_status pkv_seq_fork(pkv_pool* pool, int64_t parent, int64_t child) {
  if (!pool) return fail(PKV_ERR_INVALID_ARG, "pool is NULL");
  auto it = pool->seqs.find(parent);
  if (it == pool->seqs.end()) return fail(PKV_ERR_UNKNOWN_SEQ, "unknown parent %lld", (long long)parent);
  if (pool->seqs.count(child)) return fail(PKV_ERR_SEQ_EXISTS, "sequence %lld already exists", (long long)child);
  Seq c = it->second;
  for (int32_t b : c.blocks) pool->add_ref(b);
  pool->seqs.emplace(child, std::move(c));
  return ok();
}

pkv_status pkv_seq_free(pkv_pool* pool, int64_t seq) {
  if (!pool) return fail(PKV_ERR_INVALID_ARG, "pool is NULL");
  auto it = pool->seqs.find(seq);
  if (it == pool->seqs.end()) return ok();
  for (int32_t b : it->second.blocks) pool->drop_ref(b);
  pool->seqs.erase(it);
  return ok();
}

pkv_status pkv_seq_block_table(const pkv_pool* pool, const int64_t* seqs, int32_t n,
                               int32_t max_blocks, int32_t* table_out, int32_t* lens_out) {
  if (!pool) return fail(PKV_ERR_INVALID_ARG, "pool is NULL");
  if (n < 0 || max_blocks < 0 || (n > 0 && (!seqs || !table_out || !lens_out)))
    return fail(PKV_ERR_INVALID_ARG, "bad arguments");
  std::vector<const Seq*> ss(n);
  for (int32_t i = 0; i < n; ++i) {
    auto it = pool->seqs.find(seqs[i]);
    if (it == pool->seqs.end()) return fail(PKV_ERR_UNKNOWN_SEQ, "unknown sequence %lld", (long long)seqs[i]);
    if ((int64_t)it->second.blocks.size() > max_blocks)
      return fail(PKV_ERR_INVALID_ARG, "sequence %lld holds %zu blocks > max_blocks %d",
                  (long long)seqs[i], it->second.blocks.size(), max_blocks);
    ss[i] = &it->second;
  }
  for (int32_t i = 0; i < n; ++i) {
    int32_t* row = table_out + (size_t)i * max_blocks;
    const auto& b = ss[i]->blocks;
    std::copy(b.begin(), b.end(), row);
    std::fill(row + b.size(), row + max_blocks, -1);
    lens_out[i] = (int32_t)ss[i]->len;
  }
  return ok();
}

pkv_status pkv_seq_length(const pkv_pool* pool, int64_t seq, int64_t* len_out) {
  if (!pool || !len_out) return fail(PKV_ERR_INVALID_ARG, "NULL argument");
  auto it = pool->seqs.find(seq);
  if (it == pool->seqs.end()) return fail(PKV_ERR_UNKNOWN_SEQ, "unknown sequence %lld", (long long)seq);
  *len_out = it->second.len;
  return ok();
}

pkv_status pkv_seq_order_longest_first(const pkv_pool* pool, const int64_t* seqs, int32_t n, int64_t* seqs_out) {
  if (!pool) return fail(PKV_ERR_INVALID_ARG, "pool is NULL");
  if (n < 0 || (n > 0 && (!seqs || !seqs_out))) return fail(PKV_ERR_INVALID_ARG, "bad arguments");
  std::vector<std::pair<int64_t, int64_t>> by_len(n);  // (length, id), in the given order
  for (int32_t i = 0; i < n; ++i) {
    auto it = pool->seqs.find(seqs[i]);
    if (it == pool->seqs.end()) return fail(PKV_ERR_UNKNOWN_SEQ, "unknown sequence %lld", (long long)seqs[i]);
    by_len[i] = {it->second.len, seqs[i]};
  }
  std::stable_sort(by_len.begin(), by_len.end(),
                   [](const std::pair<int64_t, int64_t>& x, const std::pair<int64_t, int64_t>& y) {
                     return x.first > y.first;
                   });
  for (int32_t i = 0; i < n; ++i) seqs_out[i] = by_len[i].second;
  return ok();
}

pkv_status pkv_pool_stats(const pkv_pool* pool, pkv_stats* out) {
  if (!pool || !out) return fail(PKV_ERR_INVALID_ARG, "NULL argument");
  // every block is either in the free queue or referenced (conservation)
  out->free_blocks = pool->count;
  out->used_blocks = pool->cfg.num_blocks - pool->count;
  out->shared_blocks = pool->shared;
  out->cow_copies = pool->cow_total;
  out->num_seqs = (int64_t)pool->seqs.size();
  out->total_blocks = pool->cfg.num_blocks;
  return ok();
}

pkv_status pkv_pool_free_queue(const pkv_pool* pool, int32_t* out, int32_t cap, int32_t* n_out) {
  if (!pool || !out || !n_out) return fail(PKV_ERR_INVALID_ARG, "NULL argument");
  if (cap < pool->count) return fail(PKV_ERR_INVALID_ARG, "cap %d < %lld queued", cap, (long long)pool->count);
  for (int64_t i = 0; i < pool->count; ++i) out[i] = pool->ring[(pool->head + i) % pool->cfg.num_blocks];
  *n_out = (int32_t)pool->count;
  return ok();
}

pkv_status pkv_append_kv(pkv_pool* pool, int32_t layer, const void* k, const void* v,
                         pkv_dtype in_dtype, const int64_t* slot_mapping, int32_t n_tokens,
                         void* stream) {
  if (!pool) return fail(PKV_ERR_INVALID_ARG, "pool is NULL");
  if (!pool->arena) return fail(PKV_ERR_UNSUPPORTED, "host-only pool has no device cache");
  if (layer < 0 || layer >= pool->cfg.num_layers)
    return fail(PKV_ERR_INVALID_ARG, "layer %d outside [0, %d)", layer, pool->cfg.num_layers);
  if (in_dtype != PKV_F32 && in_dtype != PKV_F16 && in_dtype != PKV_BF16)
    return fail(PKV_ERR_INVALID_ARG, "input dtype must be F32, F16 or BF16");
  if (n_tokens < 0) return fail(PKV_ERR_INVALID_ARG, "n_tokens %d < 0", n_tokens);
  if (n_tokens == 0) return ok();
  if (!k || !v || !slot_mapping) return fail(PKV_ERR_INVALID_ARG, "NULL k, v or slot_mapping");
  hipError_t e = pkv::launch_append(pool->layer_view(layer), k, v, in_dtype, slot_mapping,
                                    n_tokens, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "append launch");
  return ok();
}

// Decode workgroups the device holds at once: three per compute unit (the
// compute units of the pool's device, asked at creation; 256 for a host-only
// pool).
static int64_t resident_workgroups(const pkv_pool* pool) { return 3LL * pool->cus; }

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

static int32_t auto_partition(const pkv_pool* pool, int32_t num_seqs, int32_t max_context_len) {
  const pkv_pool_config& c = pool->cfg;
  const int64_t pairs = (int64_t)num_seqs * c.num_kv_heads;
  const int64_t cus = pool->cus;
  // Every compute unit has a (sequence, KV head) and contexts are short: one
  // partition per sequence, nothing to merge. Splitting would add the
  // partials' stores, the merge and more workgroup start-ups; measured with
  // INT8 GQA 32/8 decode steps (one partition vs the best split): 32 x 1024
  // tokens 17.5 vs 22.0 us, 64 x 1024 28.5 vs 37.5 us, 96 x 2000 74.6 vs
  // 81.9 us, 128 sequences of 200..1270 tokens 30.7 vs 38.9 us.
  if (pairs >= cus && max_context_len <= 2048) {
    int32_t T = c.block_size;
    while (T < max_context_len) T *= 2;
    return T;
  }
  // About 256 KiB of K and V per workgroup amortises its start-up and its
  // share of the merge: 1024 tokens of INT8 or 512 of FP16 at head_dim 128.
  // (A pool with per-layer types plans by its kv_dtype, so one workspace
  // size serves every layer.)
  const int64_t token_bytes = 2LL * c.head_dim * (c.kv_dtype == PKV_I8 ? 1 : 2);
  int32_t T = 128;
  while (T < 2048 && (int64_t)T * 2 * token_bytes <= 262144) T *= 2;
  // With several rounds of workgroups the longest one sets the tail: longer
  // partitions than 512 tokens only for long contexts.
  if (T > 512 && pairs * ceil_div(max_context_len, T) > resident_workgroups(pool) &&
      max_context_len < 8 * T)
    T = 512;
  // At least one workgroup per compute unit.
  while (T > 128 && pairs * ceil_div(max_context_len, T) < cus) T /= 2;
  if (T < c.block_size) T = c.block_size;
  // A last partition of at most a quarter of T is folded into the others:
  // one partition fewer, all a little longer (T rounded up to the block
  // size). Its workgroups would pay a whole start-up for a few tokens;
  // Llama-2-7B 29 x 4141 (FP16): 9 x 512 tokens 351.5 us per launch, 8 x 528
  // 344.2 us.
  // (Kept only if the block-size rounding leaves no new short last partition.)
  const int64_t P = ceil_div(max_context_len, T);
  if (P >= 2 && max_context_len - (P - 1) * T <= T / 4) {
    const int64_t T2 = ceil_div(ceil_div(max_context_len, P - 1), c.block_size) * c.block_size;
    const int64_t P2 = ceil_div(max_context_len, T2);
    if (T2 <= pkv::kMaxPartitionTokens && max_context_len - (P2 - 1) * T2 > T2 / 4) T = (int32_t)T2;
  }
  return T;
}

// Automatic merge: in the last workgroup of each (sequence, KV head) when the
// whole grid is resident at once; otherwise workgroups waiting on the arrival
// count would hold slots the next ones need, and a second launch is cheaper.
static int32_t plan_fused_merge(const pkv_pool* pool, int32_t num_seqs, int32_t P, int32_t flags) {
  if (flags & PKV_DECODE_FUSED_MERGE) return 1;
  if (flags & PKV_DECODE_SEPARATE_MERGE) return 0;
  const int64_t pairs = (int64_t)num_seqs * pool->cfg.num_kv_heads;
  return pairs <= pkv::kMergeCounters && pairs * P <= resident_workgroups(pool) ? 1 : 0;
}

// A fused merge counts arrivals in the workspace's counter prefix: one
// counter per (sequence, KV head).
static_assert(PKV_MERGE_COUNTER_BYTES == pkv::kMergeCounterBytes, "counter prefix of pkv.h and the kernels");

static pkv_status check_fused_counters(const pkv_pool* pool, int32_t num_seqs, int32_t P, int32_t fused) {
  if (fused && P > 1 && (int64_t)num_seqs * pool->cfg.num_kv_heads > pkv::kMergeCounters)
    return fail(PKV_ERR_UNSUPPORTED, "PKV_DECODE_FUSED_MERGE over %lld (sequence, KV head) pairs; at most %lld",
                (long long)num_seqs * pool->cfg.num_kv_heads, (long long)pkv::kMergeCounters);
  return ok();
}

static bool valid_flags(int32_t flags) {
  return !(flags & ~(PKV_DECODE_SEPARATE_MERGE | PKV_DECODE_FUSED_MERGE | PKV_DECODE_VALU_CONTRACTION)) &&
         !((flags & PKV_DECODE_SEPARATE_MERGE) && (flags & PKV_DECODE_FUSED_MERGE));
}

pkv_status pkv_decode_plan(const pkv_pool* pool, int32_t num_seqs, int32_t max_context_len,
                           int32_t partition_tokens, int32_t flags, int32_t* partition_out,
                           int32_t* partitions_out, int32_t* fused_merge_out) {
  if (!pool) return fail(PKV_ERR_INVALID_ARG, "pool is NULL");
  if (num_seqs < 1 || max_context_len < 1)
    return fail(PKV_ERR_INVALID_ARG, "num_seqs %d and max_context_len %d must be >= 1", num_seqs,
                max_context_len);
  if (partition_tokens < 0 || (partition_tokens > 0 && partition_tokens % pool->cfg.block_size != 0) ||
      partition_tokens > pkv::kMaxPartitionTokens)
    return fail(PKV_ERR_INVALID_ARG, "partition_tokens %d is not a multiple of block_size %d in [0, %d]",
                partition_tokens, pool->cfg.block_size, pkv::kMaxPartitionTokens);
  if (!valid_flags(flags)) return fail(PKV_ERR_INVALID_ARG, "invalid flags 0x%x", flags);
  const int32_t T = partition_tokens > 0 ? partition_tokens : auto_partition(pool, num_seqs, max_context_len);
  const int32_t P = (max_context_len + T - 1) / T;
  if (partition_out) *partition_out = T;
  if (partitions_out) *partitions_out = P;
  const int32_t fused = plan_fused_merge(pool, num_seqs, P, flags);
  const pkv_status st = check_fused_counters(pool, num_seqs, P, fused);
  if (st != PKV_OK) return st;
  if (fused_merge_out) *fused_merge_out = fused;
  return ok();
}

int32_t pkv_decode_auto_partition(const pkv_pool* pool, int32_t num_seqs, int32_t num_q_heads,
                                  int32_t max_context_len) {
  (void)num_q_heads;
  if (!pool || num_seqs < 1 || max_context_len < 1) return 0;
  return auto_partition(pool, num_seqs, max_context_len);
}

size_t pkv_decode_workspace_bytes(const pkv_pool* pool, int32_t num_seqs, int32_t num_q_heads,
                                  int32_t max_context_len, int32_t partition_tokens) {
  if (!pool || num_seqs < 1 || num_q_heads < 1 || max_context_len < 1) return 0;
  const int32_t T = partition_tokens > 0 ? partition_tokens : auto_partition(pool, num_seqs, max_context_len);
  const int32_t P = (max_context_len + T - 1) / T;
  return pkv::decode_workspace_bytes(num_seqs, num_q_heads, pool->cfg.num_kv_heads, pool->cfg.head_dim, P);
}

// Shared by pkv_decode_attention and pkv_decode_step (k_new, v_new non-null).
static pkv_status decode_launch(pkv_pool* pool, int32_t layer, const void* q, pkv_dtype q_dtype,
                                int32_t num_q_heads, const void* k_new, const void* v_new,
                                const int32_t* block_tables, int32_t max_blocks_per_seq,
                                const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
                                float softmax_scale, int32_t partition_tokens, int32_t flags, float* out,
                                void* workspace, size_t workspace_bytes, void* stream) {
  if (!pool) return fail(PKV_ERR_INVALID_ARG, "pool is NULL");
  if (!valid_flags(flags)) return fail(PKV_ERR_INVALID_ARG, "invalid flags 0x%x", flags);
  if (!pool->arena) return fail(PKV_ERR_UNSUPPORTED, "host-only pool has no device cache");
  const pkv_pool_config& c = pool->cfg;
  if (layer < 0 || layer >= c.num_layers)
    return fail(PKV_ERR_INVALID_ARG, "layer %d outside [0, %d)", layer, c.num_layers);
  if (q_dtype != PKV_F32 && q_dtype != PKV_F16 && q_dtype != PKV_BF16)
    return fail(PKV_ERR_INVALID_ARG, "q dtype must be F32, F16 or BF16");
  if (num_q_heads < 1 || num_q_heads % c.num_kv_heads != 0)
    return fail(PKV_ERR_INVALID_ARG, "num_q_heads %d is not a multiple of num_kv_heads %d",
                num_q_heads, c.num_kv_heads);
  const int32_t group = num_q_heads / c.num_kv_heads;
  if (!pkv::decode_supported(c.head_dim, group))
    return fail(PKV_ERR_UNSUPPORTED, "query heads per KV head %d: supported are 1, 2 and 4", group);
  if (num_seqs < 0) return fail(PKV_ERR_INVALID_ARG, "num_seqs %d < 0", num_seqs);
  if (num_seqs == 0) return ok();
  if (max_blocks_per_seq < 1) return fail(PKV_ERR_INVALID_ARG, "max_blocks_per_seq must be >= 1");
  if (max_context_len < 1 || (int64_t)max_context_len > (int64_t)max_blocks_per_seq * c.block_size)
    return fail(PKV_ERR_INVALID_ARG, "max_context_len %d outside [1, max_blocks_per_seq*bs = %lld]",
                max_context_len, (long long)max_blocks_per_seq * c.block_size);
  if (partition_tokens < 0 || (partition_tokens > 0 && partition_tokens % c.block_size != 0) ||
      partition_tokens > pkv::kMaxPartitionTokens)
    return fail(PKV_ERR_INVALID_ARG, "partition_tokens %d is not a multiple of block_size %d in [0, %d]",
                partition_tokens, c.block_size, pkv::kMaxPartitionTokens);
  if (!q || !block_tables || !context_lens || !out)
    return fail(PKV_ERR_INVALID_ARG, "NULL q, block_tables, context_lens or out");
  const int32_t T = partition_tokens > 0 ? partition_tokens : auto_partition(pool, num_seqs, max_context_len);
  const int32_t P = (max_context_len + T - 1) / T;
  const size_t need = pkv::decode_workspace_bytes(num_seqs, num_q_heads, c.num_kv_heads, c.head_dim, P);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(PKV_ERR_INVALID_ARG, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
  if (P > 65535) return fail(PKV_ERR_UNSUPPORTED, "%d partitions exceed the grid limit", P);
  const bool valu = (flags & PKV_DECODE_VALU_CONTRACTION) != 0;
  if (valu && (k_new || c.head_dim != 128 || group > 2 || (pool->tails && pool->tail_index[layer] >= 0)))
    return fail(PKV_ERR_UNSUPPORTED,
                "PKV_DECODE_VALU_CONTRACTION: plain decode of a head_dim 128 layer (not seal_on_full) with "
                "1 or 2 query heads per KV head");

  pkv::DecodeLaunch d{};
  d.lv = pool->layer_view(layer);
  d.q = q;
  d.q_dtype = q_dtype;
  d.num_q_heads = num_q_heads;
  d.tables = block_tables;
  d.max_blocks = max_blocks_per_seq;
  d.lens = context_lens;
  d.num_seqs = num_seqs;
  d.partition_tokens = T;
  d.max_partitions = P;
  d.softmax_scale = softmax_scale;
  d.out = out;
  d.counters = (int32_t*)workspace;
  d.ws = need > 0 ? (float*)((char*)workspace + pkv::kMergeCounterBytes) : nullptr;
  d.fused_merge = plan_fused_merge(pool, num_seqs, P, flags);
  const pkv_status fst = check_fused_counters(pool, num_seqs, P, d.fused_merge);
  if (fst != PKV_OK) return fst;
  d.valu_contraction = valu ? 1 : 0;
  d.k_new = k_new;
  d.v_new = v_new;
  hipError_t e = pkv::launch_decode(d, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return ok();
}

pkv_status pkv_decode_attention(pkv_pool* pool, int32_t layer, const void* q, pkv_dtype q_dtype,
                                int32_t num_q_heads, const int32_t* block_tables,
                                int32_t max_blocks_per_seq, const int32_t* context_lens,
                                int32_t num_seqs, int32_t max_context_len, float softmax_scale,
                                int32_t partition_tokens, int32_t flags, float* out, void* workspace,
                                size_t workspace_bytes, void* stream) {
  return decode_launch(pool, layer, q, q_dtype, num_q_heads, nullptr, nullptr, block_tables,
                       max_blocks_per_seq, context_lens, num_seqs, max_context_len, softmax_scale,
                       partition_tokens, flags, out, workspace, workspace_bytes, stream);
}

pkv_status pkv_decode_step(pkv_pool* pool, int32_t layer, const void* q, const void* k_new,
                           const void* v_new, pkv_dtype dtype, int32_t num_q_heads,
                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
                           float softmax_scale, int32_t partition_tokens, int32_t flags, float* out,
                           void* workspace, size_t workspace_bytes, void* stream) {
  if (num_seqs > 0 && (!k_new || !v_new)) return fail(PKV_ERR_INVALID_ARG, "NULL k_new or v_new");
  return decode_launch(pool, layer, q, dtype, num_q_heads, k_new, v_new, block_tables,
                       max_blocks_per_seq, context_lens, num_seqs, max_context_len, softmax_scale,
                       partition_tokens, flags, out, workspace, workspace_bytes, stream);
}

pkv_status pkv_decode_step_noalloc(pkv_pool* pool, int32_t layer, const void* q, const void* k_new,
                                   const void* v_new, pkv_dtype dtype, int32_t num_q_heads,
                                   const int32_t* block_tables, int32_t max_blocks_per_seq,
                                   const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
                                   float softmax_scale, int32_t partition_tokens, int32_t flags, float* out,
                                   void* stream) {
  if (!pool) return fail(PKV_ERR_INVALID_ARG, "pool is NULL");
  if (!pool->arena) return fail(PKV_ERR_UNSUPPORTED, "host-only pool has no device cache");
  if (num_q_heads < 1 || max_context_len < 1 || num_seqs < 0)
    return fail(PKV_ERR_INVALID_ARG, "num_q_heads %d, max_context_len %d, num_seqs %d", num_q_heads,
                max_context_len, num_seqs);
  if (num_seqs == 0) return ok();
  if (partition_tokens < 0 || (partition_tokens > 0 && partition_tokens % pool->cfg.block_size != 0) ||
      partition_tokens > pkv::kMaxPartitionTokens)
    return fail(PKV_ERR_INVALID_ARG, "partition_tokens %d is not a multiple of block_size %d in [0, %d]",
                partition_tokens, pool->cfg.block_size, pkv::kMaxPartitionTokens);
  const int32_t T = partition_tokens > 0 ? partition_tokens : auto_partition(pool, num_seqs, max_context_len);
  const int32_t P = (max_context_len + T - 1) / T;
  const size_t need = pkv::decode_workspace_bytes(num_seqs, num_q_heads, pool->cfg.num_kv_heads,
                                                  pool->cfg.head_dim, P);
  if (need > pkv::kScratchBytes)
    return fail(PKV_ERR_INVALID_ARG,
                "pkv_decode_step_noalloc: these sizes need %zu bytes of workspace, the library's scratch holds %zu",
                need, pkv::kScratchBytes);
  void* ws = pkv::scratch_ptr(pool->device);
  if (!ws) return fail(PKV_ERR_DEVICE, "decode scratch of device %d is not set up", pool->device);
  if (num_seqs > 0 && (!k_new || !v_new)) return fail(PKV_ERR_INVALID_ARG, "NULL k_new or v_new");
  return decode_launch(pool, layer, q, dtype, num_q_heads, k_new, v_new, block_tables, max_blocks_per_seq,
                       context_lens, num_seqs, max_context_len, softmax_scale, partition_tokens, flags, out,
                       ws, pkv::kScratchBytes, stream);
}

// Checks shared by the prefill plan and the launch: group size, head_dim,
// query dtype, sizes and piece size.
static pkv_status prefill_check(const pkv_pool* pool, pkv_dtype q_dtype, int32_t num_q_heads, int32_t num_seqs,
                                int32_t max_query_len, int32_t max_context_len, int32_t piece_tokens) {
  if (!pool) return fail(PKV_ERR_INVALID_ARG, "pool is NULL");
  const pkv_pool_config& c = pool->cfg;
  if (q_dtype != PKV_F32 && q_dtype != PKV_F16 && q_dtype != PKV_BF16)
    return fail(PKV_ERR_INVALID_ARG, "q_dtype must be F32, F16 or BF16");
  if (num_q_heads < 1 || num_q_heads % c.num_kv_heads != 0)
    return fail(PKV_ERR_INVALID_ARG, "num_q_heads %d is not a multiple of num_kv_heads %d", num_q_heads,
                c.num_kv_heads);
  if (!pkv::decode_supported(c.head_dim, num_q_heads / c.num_kv_heads))
    return fail(PKV_ERR_UNSUPPORTED, "head_dim %d with %d query heads per KV head", c.head_dim,
                num_q_heads / c.num_kv_heads);
  if (num_seqs < 0 || max_query_len < 0 || max_context_len < 0)
    return fail(PKV_ERR_INVALID_ARG, "num_seqs %d, max_query_len %d, max_context_len %d", num_seqs,
                max_query_len, max_context_len);
  if (num_seqs > 0 && (max_query_len < 1 || max_context_len < max_query_len))
    return fail(PKV_ERR_INVALID_ARG, "max_query_len %d must be in [1, max_context_len %d]", max_query_len,
                max_context_len);
  if (piece_tokens < 0 || piece_tokens % 64 != 0)
    return fail(PKV_ERR_INVALID_ARG, "piece_tokens %d is not a non-negative multiple of 64", piece_tokens);
  return ok();
}

// A split context counts arrivals in the workspace's counter prefix: one
// counter per (sequence, KV head, query tile group).
static pkv_status check_prefill_counters(const pkv_pool* pool, int32_t num_q_heads, int32_t num_seqs,
                                         int32_t max_query_len, int32_t pieces) {
  const int32_t hkv = pool->cfg.num_kv_heads;
  const int64_t n = (int64_t)num_seqs * hkv * pkv::prefill_tile_groups_bound(max_query_len, num_q_heads / hkv);
  if (pieces > 1 && n > pkv::kMergeCounters)
    return fail(PKV_ERR_UNSUPPORTED, "context pieces over %lld (sequence, KV head, query tile group) triples; at most %lld",
                (long long)n, (long long)pkv::kMergeCounters);
  return ok();
}

pkv_status pkv_prefill_plan(const pkv_pool* pool, pkv_dtype q_dtype, int32_t num_q_heads, int32_t num_seqs,
                            int32_t max_query_len, int32_t max_context_len, int32_t piece_tokens,
                            int32_t* piece_tokens_out, int32_t* pieces_out, size_t* workspace_bytes_out,
                            int32_t* waves_out) {
  const pkv_status st =
      prefill_check(pool, q_dtype, num_q_heads, num_seqs, max_query_len, max_context_len, piece_tokens);
  if (st != PKV_OK) return st;
  if (num_seqs < 1) return fail(PKV_ERR_INVALID_ARG, "num_seqs %d must be >= 1", num_seqs);
  const pkv_pool_config& c = pool->cfg;
  int32_t T = 0, n = 0, w = 0;
  pkv::prefill_plan(pool->cus, num_seqs, c.num_kv_heads, num_q_heads / c.num_kv_heads, q_dtype, max_query_len,
                    max_context_len, piece_tokens, &T, &n, &w);
  const pkv_status cst = check_prefill_counters(pool, num_q_heads, num_seqs, max_query_len, n);
  if (cst != PKV_OK) return cst;
  if (piece_tokens_out) *piece_tokens_out = T;
  if (pieces_out) *pieces_out = n;
  if (waves_out) *waves_out = w;
  if (workspace_bytes_out)
    *workspace_bytes_out = pkv::prefill_workspace_bytes(num_seqs, max_query_len, num_q_heads, c.head_dim, n);
  return ok();
}

pkv_status pkv_prefill_attention(pkv_pool* pool, int32_t layer, const void* q, pkv_dtype q_dtype,
                                 int32_t num_q_heads, const int32_t* query_start, int32_t max_query_len,
                                 const int32_t* block_tables, int32_t max_blocks_per_seq,
                                 const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
                                 float softmax_scale, int32_t piece_tokens, float* out, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  const pkv_status st =
      prefill_check(pool, q_dtype, num_q_heads, num_seqs, max_query_len, max_context_len, piece_tokens);
  if (st != PKV_OK) return st;
  if (!pool->arena) return fail(PKV_ERR_UNSUPPORTED, "host-only pool has no device cache");
  const pkv_pool_config& c = pool->cfg;
  if (layer < 0 || layer >= c.num_layers)
    return fail(PKV_ERR_INVALID_ARG, "layer %d outside [0, %d)", layer, c.num_layers);
  if (pool->tails && pool->tail_index[layer] >= 0)
    return fail(PKV_ERR_UNSUPPORTED, "pkv_prefill_attention: layer %d quantizes on seal", layer);
  if (max_blocks_per_seq < 1)
    return fail(PKV_ERR_INVALID_ARG, "max_blocks_per_seq %d must be >= 1", max_blocks_per_seq);
  if (num_seqs == 0) return ok();
  if (!q || !query_start || !block_tables || !context_lens || !out)
    return fail(PKV_ERR_INVALID_ARG, "NULL q, query_start, block_tables, context_lens or out");
  int32_t T = 0, n = 0, w = 0;
  pkv::prefill_plan(pool->cus, num_seqs, c.num_kv_heads, num_q_heads / c.num_kv_heads, q_dtype, max_query_len,
                    max_context_len, piece_tokens, &T, &n, &w);
  const pkv_status cst = check_prefill_counters(pool, num_q_heads, num_seqs, max_query_len, n);
  if (cst != PKV_OK) return cst;
  const size_t need = pkv::prefill_workspace_bytes(num_seqs, max_query_len, num_q_heads, c.head_dim, n);
  if (need > 0 && (!workspace || workspace_bytes < need || (uintptr_t)workspace % 16 != 0))
    return fail(PKV_ERR_INVALID_ARG, "workspace of %zu bytes at %p, %zu bytes (16-byte aligned) needed",
                workspace_bytes, workspace, need);
  pkv::PrefillLaunch p{};
  p.lv = pool->layer_view(layer);
  p.q = q;
  p.q_dtype = q_dtype;
  p.num_q_heads = num_q_heads;
  p.query_start = query_start;
  p.max_query_len = max_query_len;
  p.tables = block_tables;
  p.max_blocks = max_blocks_per_seq;
  p.lens = context_lens;
  p.num_seqs = num_seqs;
  p.softmax_scale = softmax_scale;
  p.out = out;
  p.pieces = n;
  p.piece_tokens = T;
  p.waves = w;
  if (n > 1) {
    p.counters = (int32_t*)workspace;
    p.ws = (float*)((char*)workspace + pkv::kMergeCounterBytes);
  }
  hipError_t e = pkv::launch_prefill(p, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "prefill launch");
  return ok();
}

pkv_status pkv_read_blocks(const pkv_pool* pool, int32_t layer, const int32_t* blocks, int32_t n,
                           void* codes_out, float* scales_out) {
  if (!pool) return fail(PKV_ERR_INVALID_ARG, "pool is NULL");
  if (!pool->arena) return fail(PKV_ERR_UNSUPPORTED, "host-only pool has no device cache");
  const pkv_pool_config& c = pool->cfg;
  if (layer < 0 || layer >= c.num_layers)
    return fail(PKV_ERR_INVALID_ARG, "layer %d outside [0, %d)", layer, c.num_layers);
  if (n < 0 || (n > 0 && (!blocks || !codes_out))) return fail(PKV_ERR_INVALID_ARG, "bad arguments");
  for (int32_t i = 0; i < n; ++i)
    if (blocks[i] < 0 || blocks[i] >= c.num_blocks)
      return fail(PKV_ERR_INVALID_ARG, "block %d outside [0, %d)", blocks[i], c.num_blocks);
  hipError_t e = hipDeviceSynchronize();
  if (e != hipSuccess) return hip_fail(e, "synchronize before read-back");
  const bool i8 = pool->ldt[layer] == PKV_I8;
  const size_t esz = elem_bytes(pool->ldt[layer]);
  const size_t tile_bytes = (size_t)c.num_kv_heads * pool->tile_elems * esz;
  const pkv::LayerView lv = pool->layer_view(layer);
  std::vector<char> raw(tile_bytes);
  for (int32_t i = 0; i < n; ++i) {
    for (int kv = 0; kv < 2; ++kv) {
      const char* src = (const char*)(kv ? lv.v_codes : lv.k_codes) + (size_t)blocks[i] * tile_bytes;
      char* dst = (char*)codes_out + ((size_t)i * 2 + kv) * tile_bytes;
      e = hipMemcpy(kv ? raw.data() : dst, src, tile_bytes, hipMemcpyDeviceToHost);
      if (e != hipSuccess) return hip_fail(e, "read-back of codes");
      if (kv) {  // V tiles are stored in matrix-core order: put them back in [token][dim]
        const size_t te = pool->tile_elems;
        for (int32_t hd = 0; hd < c.num_kv_heads; ++hd)
          for (int32_t t = 0; t < c.block_size; ++t)
            for (int32_t d = 0; d < c.head_dim; ++d)
              std::memcpy(dst + (hd * te + (size_t)t * c.head_dim + d) * esz,
                          raw.data() + (hd * te + pkv::v_tile_offset(t, d, c.head_dim)) * esz, esz);
        if (i8)  // int8 V codes are stored biased by 128
          for (size_t b = 0; b < tile_bytes; ++b) dst[b] = (char)(dst[b] ^ 0x80);
      }
      if (scales_out && i8) {
        const float* ssrc = (kv ? lv.v_scales : lv.k_scales) + (size_t)blocks[i] * c.num_kv_heads;
        e = hipMemcpy(scales_out + ((size_t)i * 2 + kv) * c.num_kv_heads, ssrc,
                      c.num_kv_heads * sizeof(float), hipMemcpyDeviceToHost);
        if (e != hipSuccess) return hip_fail(e, "read-back of scales");
      }
    }
  }
  return ok();
}

pkv_status pkv_read_tail_blocks(const pkv_pool* pool, int32_t layer, const int32_t* blocks, int32_t n,
                                uint16_t* f16_out) {
  if (!pool) return fail(PKV_ERR_INVALID_ARG, "pool is NULL");
  if (!pool->arena) return fail(PKV_ERR_UNSUPPORTED, "host-only pool has no device cache");
  const pkv_pool_config& c = pool->cfg;
  if (layer < 0 || layer >= c.num_layers)
    return fail(PKV_ERR_INVALID_ARG, "layer %d outside [0, %d)", layer, c.num_layers);
  if (!pool->tails || pool->tail_index[layer] < 0)
    return fail(PKV_ERR_UNSUPPORTED, "layer %d has no FP16 staging tiles", layer);
  if (n < 0 || (n > 0 && (!blocks || !f16_out))) return fail(PKV_ERR_INVALID_ARG, "bad arguments");
  for (int32_t i = 0; i < n; ++i)
    if (blocks[i] < 0 || blocks[i] >= c.num_blocks)
      return fail(PKV_ERR_INVALID_ARG, "block %d outside [0, %d)", blocks[i], c.num_blocks);
  hipError_t e = hipDeviceSynchronize();
  if (e != hipSuccess) return hip_fail(e, "synchronize before read-back");
  const pkv::LayerView lv = pool->layer_view(layer);
  const size_t te = pool->tile_elems;
  const size_t tile = (size_t)c.num_kv_heads * te;  // elements of one block's K (or V) tiles
  std::vector<uint16_t> raw(tile);
  for (int32_t i = 0; i < n; ++i) {
    for (int kv = 0; kv < 2; ++kv) {
      const uint16_t* src = (const uint16_t*)(kv ? lv.tail_v : lv.tail_k) + (size_t)blocks[i] * tile;
      uint16_t* dst = f16_out + ((size_t)i * 2 + kv) * tile;
      e = hipMemcpy(raw.data(), src, tile * 2, hipMemcpyDeviceToHost);
      if (e != hipSuccess) return hip_fail(e, "read-back of staging tiles");
      for (int32_t hd = 0; hd < c.num_kv_heads; ++hd)
        for (int32_t t = 0; t < c.block_size; ++t)
          for (int32_t d = 0; d < c.head_dim; ++d)
            dst[hd * te + (size_t)t * c.head_dim + d] =
                raw[hd * te + (kv ? pkv::v_tile_offset(t, d, c.head_dim) : pkv::k_tile_offset(t, d, c.head_dim))];
    }
  }
  return ok();
}

pkv_status pkv_stream_read(const void* buf, size_t bytes, int32_t workgroups, uint32_t* sink, void* stream) {
  if (!buf || !sink) return fail(PKV_ERR_INVALID_ARG, "NULL buffer or sink");
  if (bytes == 0 || bytes % 16 != 0 || (uintptr_t)buf % 16 != 0)
    return fail(PKV_ERR_INVALID_ARG, "bytes %zu must be a positive multiple of 16 and buf 16-byte aligned", bytes);
  if (workgroups < 1 || workgroups > 65535)
    return fail(PKV_ERR_INVALID_ARG, "workgroups %d outside [1, 65535]", workgroups);
  const hipError_t e = pkv::launch_stream_read(buf, bytes, workgroups, sink, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "stream-read launch");
  return ok();
}

uint64_t pkv_kv_bytes(uint64_t layers, uint64_t heads, uint64_t head_dim, uint64_t tokens,
                      uint64_t seqs, uint64_t bytes) {
  return 2ull * layers * heads * head_dim * tokens * seqs * bytes;
}

const char* pkv_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
