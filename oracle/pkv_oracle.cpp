// pkv_oracle.cpp -- plain, slow, CPU-only reference for paged-KV decode attention.
//
// TEST INFRASTRUCTURE ONLY. Nothing in the product path may include, link or
// call this file: only the test suite, the smoke check and the benchmark's
// CPU-baseline leg use it. It shares no code, header, table or helper with the
// HIP library; the two meet only in the seeded input arrays both are given.
//
// Sources (page title, section):
//  [P1] "无 vLLM 环境下的 Paged-KV 与连续批处理调度" -- §1.1 fixed buckets,
//       §1.2 block count / tail waste, §2 KV-bytes formula.
//  [P2] "vLLM核心概念：PagedAttention、Continuous Batching、KV Cache等原理" --
//       §3.1 KV-bytes formula and the 512 KB/token example, decode = new Q
//       against cached K/V; §3.2 blocks, block table, copy-on-write sharing.
//  [P4] "连续批处理与KV缓存" -- §4.2 free-block queue and the
//       PagedKVCacheManager allocate / free / append_block pseudo-code.
//  [P5] "轻量级推理引擎实战：KV Cache 量化与连续批处理的底层优化" -- §2.1
//       block layout and shared prefixes; §三 KVCacheQuantizer (per-head
//       symmetric INT8, scale = max|x|/127, zero heads get scale 1.0).
//
// Readings where the pages leave a point open are marked READING below.
// Everything floating point in the attention is FP64; the quantizer is FP32
// because its results must be reproduced bit for bit.
//
// Build: g++ -std=c++17 -O2 -ffp-contract=off -fPIC -shared -pthread
//        (no -ffast-math: the quantizer depends on IEEE division and rounding)

#include <algorithm>
#include <cfenv>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <deque>
#include <map>
#include <thread>
#include <vector>

extern "C" {

// Status codes. These mirror the meaning of the library's codes but are
// defined here separately on purpose.
enum {
  ORC_OK = 0,
  ORC_INVALID = -1,
  ORC_OOM = -2,
  ORC_NO_FREE_BLOCK = -3,
  ORC_UNKNOWN_SEQ = -4,
  ORC_SEQ_EXISTS = -5,
};

// ---------------------------------------------------------------------------
// O1. KV-cache size: 2 (K and V) x layers x heads x head_dim x tokens x
// sequences x bytes per element  ([P1] §2 formula; [P2] §3.1 formula).
// ---------------------------------------------------------------------------
uint64_t orc_kv_bytes(uint64_t layers, uint64_t heads, uint64_t head_dim,
                      uint64_t tokens, uint64_t seqs, uint64_t bytes) {
  return 2ull * layers * heads * head_dim * tokens * seqs * bytes;
}

// ---------------------------------------------------------------------------
// O2. Block arithmetic ([P1] §1.2): a sequence of length len uses
// ceil(len / bs) blocks; only the last block can be partly empty.
// ---------------------------------------------------------------------------
int64_t orc_num_blocks(int64_t len, int64_t bs) { return (len + bs - 1) / bs; }
int64_t orc_tail_waste(int64_t len, int64_t bs) {
  return orc_num_blocks(len, bs) * bs - len;
}

// ---------------------------------------------------------------------------
// IEEE-754 binary16 / bfloat16 helpers, written from the format definitions.
// binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits.
// bfloat16: the top 16 bits of a binary32.
// ---------------------------------------------------------------------------
static uint32_t f32_bits(float x) { uint32_t u; std::memcpy(&u, &x, 4); return u; }
static float bits_f32(uint32_t u) { float x; std::memcpy(&x, &u, 4); return x; }

float orc_f16_to_f32(uint16_t h) {
  const uint32_t sign = (uint32_t)(h >> 15) << 31;
  const int exp = (h >> 10) & 0x1f;
  const uint32_t frac = h & 0x3ff;
  if (exp == 0x1f) return bits_f32(sign | 0x7f800000u | (frac << 13));  // inf/nan
  if (exp == 0) {
    // zero or subnormal: value = frac * 2^-24, exact in binary32
    float v = (float)frac * std::ldexp(1.0f, -24);
    return (h >> 15) ? -v : v;
  }
  return bits_f32(sign | (uint32_t)(exp - 15 + 127) << 23 | (frac << 13));
}

// Round a binary32 to the nearest binary16, ties to even. Overflow goes to
// +-inf; values below half the smallest subnormal go to +-0.
uint16_t orc_f32_to_f16(float x) {
  const uint32_t u = f32_bits(x);
  const uint16_t sign = (uint16_t)((u >> 16) & 0x8000);
  const uint32_t absu = u & 0x7fffffffu;
  if (absu >= 0x7f800000u) {  // inf or nan
    if (absu == 0x7f800000u) return sign | 0x7c00;
    return sign | 0x7e00;  // quiet nan
  }
  const double a = std::fabs((double)x);  // exact copy of |x|
  // Work in units of the binary16 quantum for the binade of a.
  int e;  // a = m * 2^e with m in [0.5, 1)
  std::frexp(a, &e);
  int unbiased = e - 1;        // a in [2^unbiased, 2^(unbiased+1))
  if (unbiased < -14) unbiased = -14;  // subnormal range shares the 2^-24 quantum
  const double quantum = std::ldexp(1.0, unbiased - 10);
  const double scaled = a / quantum;  // exact: power-of-two division
  double r = std::floor(scaled);
  const double rem = scaled - r;
  if (rem > 0.5 || (rem == 0.5 && std::fmod(r, 2.0) != 0.0)) r += 1.0;
  const double v = r * quantum;  // rounded magnitude, exact
  if (v >= 65536.0) return sign | 0x7c00;  // 65520 and above round to inf
  // Encode v.
  if (v < std::ldexp(1.0, -14)) {  // subnormal (or zero)
    return sign | (uint16_t)(v / std::ldexp(1.0, -24));
  }
  int ev;
  double mv = std::frexp(v, &ev);  // v = mv * 2^ev, mv in [0.5,1)
  const int biased = ev - 1 + 15;
  const uint16_t frac = (uint16_t)((mv * 2.0 - 1.0) * 1024.0);
  return sign | (uint16_t)(biased << 10) | frac;
}

float orc_bf16_to_f32(uint16_t b) { return bits_f32((uint32_t)b << 16); }

// ---------------------------------------------------------------------------
// O3. Block allocator model ([P4] §4.2 PagedKVCacheManager; [P2] §3.2 CoW).
//  * a FIFO queue of free block ids: allocation pops from the front,
//    freeing appends to the back, both O(1) per block;
//  * each sequence owns an ordered list of blocks (its block table) and a
//    length in tokens;
//  * each block has a reference count: forked sequences share blocks.
// READING: allocate on an existing id is rejected (the pseudo-code would
// silently overwrite the entry and leak its blocks); freeing an unknown id
// is a no-op (the pseudo-code's pop(request_id, [])); an append that cannot
// be served reports "no free block" and changes nothing (the pseudo-code's
// "return False, needs to wait"); copy-on-write happens on the first write
// into a partly filled block whose reference count is above one.
// ---------------------------------------------------------------------------
struct OrcSeq {
  std::vector<int32_t> blocks;
  int64_t len = 0;
};

struct OrcCow {
  int32_t src, dst, rows;  // copy rows [0, rows) of src into dst (all layers, K and V)
};

struct OrcAlloc {
  int32_t num_blocks = 0, block_size = 0;
  std::deque<int32_t> free_q;
  std::vector<int32_t> refcount;
  std::map<int64_t, OrcSeq> seqs;
  std::vector<OrcCow> cow_log;  // copies requested since the last drain
  int64_t cow_total = 0;
};

void* orc_alloc_create(int32_t num_blocks, int32_t block_size,
                       const int32_t* free_order) {
  if (num_blocks <= 0 || block_size <= 0) return nullptr;
  auto* a = new OrcAlloc;
  a->num_blocks = num_blocks;
  a->block_size = block_size;
  a->refcount.assign(num_blocks, 0);
  for (int32_t i = 0; i < num_blocks; ++i)
    a->free_q.push_back(free_order ? free_order[i] : i);
  return a;
}

void orc_alloc_destroy(void* h) { delete (OrcAlloc*)h; }

static int32_t orc_pop_front(OrcAlloc* a) {
  int32_t b = a->free_q.front();
  a->free_q.pop_front();
  a->refcount[b] = 1;
  return b;
}

// allocate(seq, n_tokens): ceil(n/bs) blocks from the front of the queue.
int orc_alloc_allocate(void* h, int64_t seq, int32_t n_tokens, int64_t* slots) {
  auto* a = (OrcAlloc*)h;
  if (n_tokens < 0) return ORC_INVALID;
  if (a->seqs.count(seq)) return ORC_SEQ_EXISTS;
  const int64_t need = orc_num_blocks(n_tokens, a->block_size);
  if ((int64_t)a->free_q.size() < need) return ORC_OOM;
  OrcSeq s;
  for (int64_t j = 0; j < need; ++j) s.blocks.push_back(orc_pop_front(a));
  s.len = n_tokens;
  for (int64_t p = 0; p < n_tokens; ++p)
    if (slots) slots[p] = (int64_t)s.blocks[p / a->block_size] * a->block_size + p % a->block_size;
  a->seqs[seq] = s;
  return ORC_OK;
}

// append: for each sequence in argument order, each new position in order.
int orc_alloc_append(void* h, const int64_t* seq_ids, int32_t n_seqs,
                     const int32_t* n_new, int64_t* slots) {
  auto* a = (OrcAlloc*)h;
  const int64_t bs = a->block_size;
  // validation and a dry run that counts the blocks the call needs
  std::map<int32_t, int32_t> rc_delta;
  int64_t pops = 0;
  for (int32_t i = 0; i < n_seqs; ++i) {
    if (n_new[i] < 0) return ORC_INVALID;
    for (int32_t k = 0; k < i; ++k)
      if (seq_ids[k] == seq_ids[i]) return ORC_INVALID;
    auto it = a->seqs.find(seq_ids[i]);
    if (it == a->seqs.end()) return ORC_UNKNOWN_SEQ;
  }
  for (int32_t i = 0; i < n_seqs; ++i) {
    const OrcSeq& s = a->seqs[seq_ids[i]];
    int64_t nblk = (int64_t)s.blocks.size();
    for (int64_t p = s.len; p < s.len + n_new[i]; ++p) {
      const int64_t j = p / bs;
      if (j == nblk) { ++pops; ++nblk; continue; }
      if (p == s.len && p % bs != 0) {
        const int32_t b = s.blocks[j];
        if (a->refcount[b] + rc_delta[b] > 1) { ++pops; --rc_delta[b]; }
      }
    }
  }
  if (pops > (int64_t)a->free_q.size()) return ORC_NO_FREE_BLOCK;
  // the real pass
  int64_t out = 0;
  for (int32_t i = 0; i < n_seqs; ++i) {
    OrcSeq& s = a->seqs[seq_ids[i]];
    for (int64_t p = s.len; p < s.len + n_new[i]; ++p) {
      const int64_t j = p / bs;
      if (j == (int64_t)s.blocks.size()) {
        s.blocks.push_back(orc_pop_front(a));
      } else if (p % bs != 0 && a->refcount[s.blocks[j]] > 1) {
        const int32_t old = s.blocks[j];
        const int32_t fresh = orc_pop_front(a);
        a->refcount[old] -= 1;
        s.blocks[j] = fresh;
        a->cow_log.push_back({old, fresh, (int32_t)(p % bs)});
        a->cow_total += 1;
      }
      if (slots) slots[out] = (int64_t)s.blocks[j] * bs + p % bs;
      ++out;
    }
    s.len += n_new[i];
  }
  return ORC_OK;
}

int orc_alloc_fork(void* h, int64_t parent, int64_t child) {
  auto* a = (OrcAlloc*)h;
  auto it = a->seqs.find(parent);
  if (it == a->seqs.end()) return ORC_UNKNOWN_SEQ;
  if (a->seqs.count(child)) return ORC_SEQ_EXISTS;
  OrcSeq c = it->second;
  for (int32_t b : c.blocks) a->refcount[b] += 1;
  a->seqs[child] = c;
  return ORC_OK;
}

int orc_alloc_free(void* h, int64_t seq) {
  auto* a = (OrcAlloc*)h;
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) return ORC_OK;
  for (int32_t b : it->second.blocks) {
    a->refcount[b] -= 1;
    if (a->refcount[b] == 0) a->free_q.push_back(b);
  }
  a->seqs.erase(it);
  return ORC_OK;
}

int orc_alloc_table(void* h, const int64_t* seq_ids, int32_t n, int32_t max_blocks,
                    int32_t* table, int32_t* lens) {
  auto* a = (OrcAlloc*)h;
  for (int32_t i = 0; i < n; ++i) {
    auto it = a->seqs.find(seq_ids[i]);
    if (it == a->seqs.end()) return ORC_UNKNOWN_SEQ;
    if ((int64_t)it->second.blocks.size() > max_blocks) return ORC_INVALID;
  }
  for (int32_t i = 0; i < n; ++i) {
    const OrcSeq& s = a->seqs[seq_ids[i]];
    for (int32_t j = 0; j < max_blocks; ++j)
      table[(int64_t)i * max_blocks + j] = j < (int32_t)s.blocks.size() ? s.blocks[j] : -1;
    lens[i] = (int32_t)s.len;
  }
  return ORC_OK;
}

// out: [0] free blocks, [1] blocks with refcount > 0, [2] blocks with
// refcount > 1, [3] copy-on-write copies so far, [4] live sequences.
void orc_alloc_stats(void* h, int64_t* out) {
  auto* a = (OrcAlloc*)h;
  int64_t used = 0, shared = 0;
  for (int32_t r : a->refcount) { used += r > 0; shared += r > 1; }
  out[0] = (int64_t)a->free_q.size();
  out[1] = used;
  out[2] = shared;
  out[3] = a->cow_total;
  out[4] = (int64_t)a->seqs.size();
}

int32_t orc_alloc_refcount(void* h, int32_t block) { return ((OrcAlloc*)h)->refcount[block]; }

// Copy the free queue, front first. Returns its length.
int32_t orc_alloc_free_queue(void* h, int32_t* out) {
  auto* a = (OrcAlloc*)h;
  int32_t i = 0;
  for (int32_t b : a->free_q) out[i++] = b;
  return i;
}

// Drain the copy-on-write requests made since the last call: triples
// (src, dst, rows). Returns how many there were.
int32_t orc_alloc_take_cows(void* h, int32_t* out, int32_t cap) {
  auto* a = (OrcAlloc*)h;
  int32_t n = (int32_t)a->cow_log.size();
  if (n > cap) return -1;
  for (int32_t i = 0; i < n; ++i) {
    out[3 * i] = a->cow_log[i].src;
    out[3 * i + 1] = a->cow_log[i].dst;
    out[3 * i + 2] = a->cow_log[i].rows;
  }
  a->cow_log.clear();
  return n;
}

// ---------------------------------------------------------------------------
// O4. Symmetric INT8 quantizer, one scale per (block, KV head), separately
// for K and V and for every layer ([P5] §三 KVCacheQuantizer::quantize_block).
//   scale = max|x| / 127 when max|x| > 1e-6, else 1.0;
//   code  = clamp(round(x / scale), -127, 127), round half to even;
//   x_hat = code * scale.
// READING: the comparison lost in the page's text is ">" (all-zero heads get
// 1.0); the page's comment divides by the scale, which is what is done here;
// rounding is half-to-even. When tokens land in a block that already holds
// f > 0 tokens (the pages are silent), the scale only grows: if the new
// values' max |x| does not exceed fl(max|code_old| * scale_old) the old scale
// and codes stay and the new rows are encoded with it; otherwise the scale is
// recomputed from the new max and the old codes are re-encoded from their
// dequantized values. With f == 0 this is exactly the page's quantize_block.
// ---------------------------------------------------------------------------
static float orc_scale_of(float max_abs) { return (max_abs > 1e-6f) ? max_abs / 127.0f : 1.0f; }

static int8_t orc_encode(float x, float scale) {
  const float y = x / scale;          // IEEE binary32 division, round to nearest
  float r = std::nearbyint(y);        // FE_TONEAREST: ties to even
  if (r > 127.0f) r = 127.0f;
  if (r < -127.0f) r = -127.0f;
  return (int8_t)r;
}

// Quantize `rows` new rows (each of `dim` binary32 values, row stride `dim`)
// into a block whose first `fill` rows already hold codes with scale *scale.
// codes points at row 0 of the (block, head) tile, row stride `dim`.
void orc_quant_append(int8_t* codes, float* scale, int32_t fill, const float* x,
                      int32_t rows, int32_t dim) {
  float m_new = 0.0f;
  for (int32_t i = 0; i < rows * dim; ++i) m_new = std::max(m_new, std::fabs(x[i]));
  float s;
  if (fill == 0) {
    s = orc_scale_of(m_new);
  } else {
    int32_t qmax = 0;
    for (int32_t i = 0; i < fill * dim; ++i) qmax = std::max(qmax, std::abs((int32_t)codes[i]));
    const float s_old = *scale;
    const float m_old = (float)qmax * s_old;
    if (m_new <= m_old) {
      s = s_old;
    } else {
      s = orc_scale_of(m_new);
      for (int32_t i = 0; i < fill * dim; ++i) {
        const float deq = (float)codes[i] * s_old;
        codes[i] = orc_encode(deq, s);
      }
    }
  }
  for (int32_t i = 0; i < rows * dim; ++i) codes[fill * dim + i] = orc_encode(x[i], s);
  *scale = s;
}

// ---------------------------------------------------------------------------
// Cache model: the oracle's own copy of the paged cache, filled by replaying
// the same append calls and copy-on-write copies as the library sees.
// Layout (oracle-private): codes[layer][kv][block][head][row][dim];
// scales[layer][kv][block][head]. kv_dtype 1 = binary16 bits, 3 = int8.
// ---------------------------------------------------------------------------
struct OrcCache {
  int32_t layers, heads, dim, bs, nblocks, dtype;
  std::vector<int8_t> q;      // int8 codes
  std::vector<uint16_t> h;    // binary16 bits
  std::vector<float> scale;
  size_t tile() const { return (size_t)bs * dim; }
  size_t tile_index(int l, int kv, int b, int hd) const {
    return (((size_t)l * 2 + kv) * nblocks + b) * heads + hd;
  }
};

void* orc_cache_create(int32_t layers, int32_t heads, int32_t dim, int32_t bs,
                       int32_t nblocks, int32_t dtype) {
  if (dtype != 1 && dtype != 3) return nullptr;
  auto* c = new OrcCache{layers, heads, dim, bs, nblocks, dtype, {}, {}, {}};
  const size_t n = (size_t)layers * 2 * nblocks * heads * bs * dim;
  if (dtype == 3) c->q.assign(n, 0); else c->h.assign(n, 0);
  c->scale.assign((size_t)layers * 2 * nblocks * heads, 1.0f);
  return c;
}

void orc_cache_destroy(void* p) { delete (OrcCache*)p; }

// Append n tokens to one layer. k, v: binary32 values [n][heads][dim] (inputs
// in bf16/fp16 are widened exactly by the caller). slots[i] = block*bs + row.
// Consecutive tokens that fall in the same block form one append into that
// block, starting at row slots[first] % bs; their rows must be consecutive.
// A slot outside [0, nblocks*bs), a same-block neighbour whose row is not
// the next one, or a block that comes back after another block's tokens is
// rejected before anything is written.
int orc_cache_append(void* p, int32_t layer, const float* k, const float* v,
                     const int64_t* slots, int32_t n) {
  auto* c = (OrcCache*)p;
  const int64_t bs = c->bs;
  std::vector<char> done(c->nblocks, 0);  // blocks whose run has ended
  for (int32_t i = 0; i < n; ++i) {
    if (slots[i] < 0 || slots[i] >= (int64_t)c->nblocks * bs) return ORC_INVALID;
    const int64_t blk = slots[i] / bs;
    if (i > 0 && blk == slots[i - 1] / bs) {
      if (slots[i] != slots[i - 1] + 1) return ORC_INVALID;
    } else {
      if (done[blk]) return ORC_INVALID;
      if (i > 0) done[slots[i - 1] / bs] = 1;
    }
  }
  for (int32_t i = 0; i < n;) {
    const int64_t blk = slots[i] / bs;
    const int32_t row0 = (int32_t)(slots[i] % bs);
    int32_t j = i + 1;
    while (j < n && slots[j] / bs == blk) ++j;
    const int32_t rows = j - i;
    for (int kv = 0; kv < 2; ++kv) {
      const float* src = kv == 0 ? k : v;
      for (int32_t hd = 0; hd < c->heads; ++hd) {
        // gather this head's rows into a contiguous [rows][dim] buffer
        std::vector<float> x((size_t)rows * c->dim);
        for (int32_t r = 0; r < rows; ++r)
          for (int32_t d = 0; d < c->dim; ++d)
            x[(size_t)r * c->dim + d] = src[((size_t)(i + r) * c->heads + hd) * c->dim + d];
        const size_t t = c->tile_index(layer, kv, (int)blk, hd);
        if (c->dtype == 3) {
          orc_quant_append(&c->q[t * c->tile()], &c->scale[t], row0, x.data(), rows, c->dim);
        } else {
          for (int32_t r = 0; r < rows; ++r)
            for (int32_t d = 0; d < c->dim; ++d)
              c->h[t * c->tile() + (size_t)(row0 + r) * c->dim + d] =
                  orc_f32_to_f16(x[(size_t)r * c->dim + d]);
        }
      }
    }
    i = j;
  }
  return ORC_OK;
}

// Copy-on-write: rows [0, rows) and the scale of every (layer, kv, head).
void orc_cache_copy_block(void* p, int32_t src, int32_t dst, int32_t rows) {
  auto* c = (OrcCache*)p;
  for (int l = 0; l < c->layers; ++l)
    for (int kv = 0; kv < 2; ++kv)
      for (int hd = 0; hd < c->heads; ++hd) {
        const size_t ts = c->tile_index(l, kv, src, hd), td = c->tile_index(l, kv, dst, hd);
        const size_t n = (size_t)rows * c->dim;
        if (c->dtype == 3)
          std::copy_n(&c->q[ts * c->tile()], n, &c->q[td * c->tile()]);
        else
          std::copy_n(&c->h[ts * c->tile()], n, &c->h[td * c->tile()]);
        c->scale[td] = c->scale[ts];
      }
}

// Canonical export of one (layer, block): codes [kv][head][row][dim] (int8 or
// binary16 bits), scales [kv][head].
void orc_cache_read_block(void* p, int32_t layer, int32_t block, void* codes_out,
                          float* scales_out) {
  auto* c = (OrcCache*)p;
  for (int kv = 0; kv < 2; ++kv)
    for (int hd = 0; hd < c->heads; ++hd) {
      const size_t t = c->tile_index(layer, kv, block, hd);
      const size_t o = ((size_t)kv * c->heads + hd) * c->tile();
      if (c->dtype == 3)
        std::copy_n(&c->q[t * c->tile()], c->tile(), (int8_t*)codes_out + o);
      else
        std::copy_n(&c->h[t * c->tile()], c->tile(), (uint16_t*)codes_out + o);
      scales_out[kv * c->heads + hd] = c->scale[t];
    }
}

// ---------------------------------------------------------------------------
// O5. Decode attention, FP64 ([P2] §3.1: the new token's query against every
// cached key and value; [P2] §3.2 / [P5] §2.1: logical token t of a sequence
// lives in block table[t / bs], row t % bs).
// READING: standard scaled dot-product softmax attention; query head h reads
// KV head h / G with G = Hq / Hkv (contiguous groups); the context length
// counts every token to attend to, including the one just appended.
//
// Cache arrays for ONE layer: k_codes, v_codes [nblocks][Hkv][bs][dim]
// (int8 when kv_dtype == 3, binary16 bits when 1, or the key/value numbers
// themselves as binary64 when 0 -- for caches whose blocks mix formats);
// k_scales, v_scales [nblocks][Hkv] (read only for int8). q: binary32
// [B][Hq][dim] (exact widening of the caller's query). out: [B][Hq][dim] FP64.
// ---------------------------------------------------------------------------
struct OrcAttnArgs {
  int32_t kv_dtype, nblocks, hkv, bs, dim;
  const void* k_codes; const void* v_codes;
  const float* k_scales; const float* v_scales;
  const float* q; int32_t hq;
  const int32_t* table; int32_t max_blocks; const int32_t* lens;
  int32_t nseq; double softmax_scale; double* out;
};

static double orc_dequant(const OrcAttnArgs& a, const void* codes, const float* scales,
                          int32_t block, int32_t head, int32_t row, int32_t d) {
  const size_t idx = (((size_t)block * a.hkv + head) * a.bs + row) * a.dim + d;
  if (a.kv_dtype == 3)
    return (double)((const int8_t*)codes)[idx] * (double)scales[(size_t)block * a.hkv + head];
  if (a.kv_dtype == 0) return ((const double*)codes)[idx];
  return (double)orc_f16_to_f32(((const uint16_t*)codes)[idx]);
}

static void orc_attend_one(const OrcAttnArgs& a, int32_t s, int32_t h) {
  const int32_t group = a.hq / a.hkv;
  const int32_t g = h / group;
  const int32_t len = a.lens[s];
  std::vector<double> score(len);
  const float* q = a.q + ((size_t)s * a.hq + h) * a.dim;
  for (int32_t t = 0; t < len; ++t) {
    const int32_t blk = a.table[(size_t)s * a.max_blocks + t / a.bs];
    const int32_t row = t % a.bs;
    double dot = 0.0;
    for (int32_t d = 0; d < a.dim; ++d)
      dot += (double)q[d] * orc_dequant(a, a.k_codes, a.k_scales, blk, g, row, d);
    score[t] = a.softmax_scale * dot;
  }
  double m = -INFINITY;
  for (double x : score) m = std::max(m, x);
  std::vector<double> acc(a.dim, 0.0);
  double denom = 0.0;
  for (int32_t t = 0; t < len; ++t) {
    const double w = std::exp(score[t] - m);
    denom += w;
    const int32_t blk = a.table[(size_t)s * a.max_blocks + t / a.bs];
    const int32_t row = t % a.bs;
    for (int32_t d = 0; d < a.dim; ++d)
      acc[d] += w * orc_dequant(a, a.v_codes, a.v_scales, blk, g, row, d);
  }
  double* o = a.out + ((size_t)s * a.hq + h) * a.dim;
  for (int32_t d = 0; d < a.dim; ++d) o[d] = acc[d] / denom;
}

// Returns ORC_INVALID on bad arguments (len 0, len past the table, a table
// entry outside the pool, Hq not a multiple of Hkv). threads <= 0: all cores.
int orc_decode_attention(int32_t kv_dtype, int32_t nblocks, int32_t hkv, int32_t bs,
                         int32_t dim, const void* k_codes, const void* v_codes,
                         const float* k_scales, const float* v_scales, const float* q,
                         int32_t hq, const int32_t* table, int32_t max_blocks,
                         const int32_t* lens, int32_t nseq, double softmax_scale,
                         double* out, int32_t threads) {
  if (hkv <= 0 || hq % hkv != 0 || bs <= 0 || dim <= 0) return ORC_INVALID;
  for (int32_t s = 0; s < nseq; ++s) {
    if (lens[s] < 1 || lens[s] > (int64_t)max_blocks * bs) return ORC_INVALID;
    for (int32_t j = 0; j < orc_num_blocks(lens[s], bs); ++j) {
      const int32_t b = table[(size_t)s * max_blocks + j];
      if (b < 0 || b >= nblocks) return ORC_INVALID;
    }
  }
  OrcAttnArgs a{kv_dtype, nblocks, hkv, bs, dim, k_codes, v_codes, k_scales, v_scales,
                q, hq, table, max_blocks, lens, nseq, softmax_scale, out};
  const int64_t tasks = (int64_t)nseq * hq;
  int32_t nt = threads > 0 ? threads : (int32_t)std::max(1u, std::thread::hardware_concurrency());
  if (nt > tasks) nt = (int32_t)std::max<int64_t>(1, tasks);
  std::vector<std::thread> pool;
  for (int32_t w = 0; w < nt; ++w)
    pool.emplace_back([&, w]() {
      for (int64_t i = w; i < tasks; i += nt) orc_attend_one(a, (int32_t)(i / hq), (int32_t)(i % hq));
    });
  for (auto& th : pool) th.join();
  return ORC_OK;
}

// ---------------------------------------------------------------------------
// Chunked prefill attention, FP64 ("轻量级推理引擎实战" §一: prefill handles the
// prompt's tokens in parallel; the decode rule above, applied to every new
// token at once). For sequence s the last qlen[s] = qstart[s+1] - qstart[s] of
// its lens[s] cached tokens are queries: query i sits at position
// p = lens[s] - qlen[s] + i and attends to positions 0..p (causal).
// READING: the same scaled dot-product softmax as decode, one query at a time.
// q: binary32 [total][Hq][dim]; out: FP64 [total][Hq][dim].
// ---------------------------------------------------------------------------
int orc_prefill_attention(int32_t kv_dtype, int32_t nblocks, int32_t hkv, int32_t bs, int32_t dim,
                          const void* k_codes, const void* v_codes, const float* k_scales,
                          const float* v_scales, const float* q, int32_t hq, const int32_t* qstart,
                          const int32_t* table, int32_t max_blocks, const int32_t* lens, int32_t nseq,
                          double softmax_scale, double* out, int32_t threads) {
  if (hkv <= 0 || hq % hkv != 0 || bs <= 0 || dim <= 0 || qstart[0] != 0) return ORC_INVALID;
  int64_t total = 0;
  for (int32_t s = 0; s < nseq; ++s) {
    const int32_t ql = qstart[s + 1] - qstart[s];
    if (ql < 1 || ql > lens[s] || lens[s] > (int64_t)max_blocks * bs) return ORC_INVALID;
    for (int32_t j = 0; j < orc_num_blocks(lens[s], bs); ++j) {
      const int32_t b = table[(size_t)s * max_blocks + j];
      if (b < 0 || b >= nblocks) return ORC_INVALID;
    }
    total += ql;
  }
  // Query row r of sequence s is the decode of a sequence whose context ends
  // at its position: run the decode rule with that length, one row at a time.
  std::vector<int32_t> row_seq(total), row_len(total);
  for (int32_t s = 0; s < nseq; ++s)
    for (int32_t r = qstart[s]; r < qstart[s + 1]; ++r) {
      row_seq[r] = s;
      row_len[r] = lens[s] - (qstart[s + 1] - qstart[s]) + (r - qstart[s]) + 1;
    }
  const int64_t tasks = total * hq;
  int32_t nt = threads > 0 ? threads : (int32_t)std::max(1u, std::thread::hardware_concurrency());
  if (nt > tasks) nt = (int32_t)std::max<int64_t>(1, tasks);
  std::vector<std::thread> pool;
  for (int32_t w = 0; w < nt; ++w)
    pool.emplace_back([&, w]() {
      for (int64_t i = w; i < tasks; i += nt) {
        const int64_t r = i / hq;
        const int32_t h = (int32_t)(i % hq);
        const int32_t s = row_seq[r];
        // one sequence's view: its table row, this query's length, its query row
        OrcAttnArgs a{kv_dtype, nblocks, hkv, bs, dim, k_codes, v_codes, k_scales, v_scales,
                      q + (size_t)r * hq * dim, hq, table + (size_t)s * max_blocks, max_blocks,
                      &row_len[r], 1, softmax_scale, out + (size_t)r * hq * dim};
        orc_attend_one(a, 0, h);
      }
    });
  for (auto& th : pool) th.join();
  return ORC_OK;
}

int32_t orc_hardware_threads(void) { return (int32_t)std::thread::hardware_concurrency(); }

}  // extern "C"
