// Host-side KV block manager ("vLLM 学习笔记 01", sections 1.4, 1.5, 2.2):
// the free-block queue, reference counts, the prefix cache keyed by a hash
// chain, and slot allocation.  It produces the block tables and slot
// mappings that paged_kv_write and paged_attention consume.  The policies the
// pages leave open are stated in include/paged_block_manager.h.
//
// Every operation is O(1) per block it touches: the free queue is an
// intrusive doubly linked list over block ids (taking from the head,
// returning to the tail and removing a cached block that a request reuses
// are constant time), and the cache is a hash map from a block's chained
// hash to its id.
#include "../../include/paged_block_manager.h"

#include <algorithm>
#include <cstring>
#include <string>
#include <unordered_map>
#include <vector>

namespace {

constexpr int kBlockTokens = 16;

thread_local std::string g_bm_error;

int bm_fail(int code, const std::string& msg) {
  g_bm_error = msg;
  return code;
}

// FNV-1a, 64-bit (Fowler, Noll and Vo): for each byte, xor it in, then
// multiply by the FNV prime.
constexpr uint64_t kFnvOffset = 0xcbf29ce484222325ull;
constexpr uint64_t kFnvPrime = 0x100000001b3ull;

uint64_t fnv_bytes(uint64_t h, uint64_t v, int nbytes) {
  for (int i = 0; i < nbytes; ++i) {
    h ^= (v >> (8 * i)) & 0xffu;
    h *= kFnvPrime;
  }
  return h;
}

// Key of a full block: its parent's hash (0 for the first block), the
// request's salt and its 16 tokens, each little-endian.
uint64_t block_hash(uint64_t parent, int64_t salt, const int32_t* tokens) {
  uint64_t h = kFnvOffset;
  h = fnv_bytes(h, parent, 8);
  h = fnv_bytes(h, (uint64_t)salt, 8);
  for (int i = 0; i < kBlockTokens; ++i) h = fnv_bytes(h, (uint32_t)tokens[i], 4);
  return h;
}

struct Block {
  int32_t ref = 0;
  int32_t prev = -1, next = -1;   // free-queue neighbours
  bool in_free = false;
  bool cached = false;            // registered in the cache under `hash`
  uint64_t hash = 0, parent = 0;
  int64_t salt = 0;
  int32_t tokens[kBlockTokens] = {};
};

struct Request {
  int64_t salt = 0;
  std::vector<int32_t> tokens;    // known tokens
  std::vector<int32_t> table;     // block ids
  int32_t computed = 0;           // leading tokens that have slots
  int32_t hashed = 0;             // leading full blocks in (or matched from) the cache
  uint64_t last_hash = 0;         // hash of block hashed - 1, 0 before the first
};

}  // namespace

struct paged_bm {
  bool caching = true;
  std::vector<Block> blocks;
  int32_t head = -1, tail = -1;
  int64_t nfree = 0;
  std::unordered_map<uint64_t, int32_t> cache;
  std::unordered_map<int64_t, Request> reqs;

  void push_back(int32_t id) {
    Block& b = blocks[id];
    b.prev = tail;
    b.next = -1;
    if (tail >= 0) blocks[tail].next = id; else head = id;
    tail = id;
    b.in_free = true;
    ++nfree;
  }

  void unlink(int32_t id) {
    Block& b = blocks[id];
    if (b.prev >= 0) blocks[b.prev].next = b.next; else head = b.next;
    if (b.next >= 0) blocks[b.next].prev = b.prev; else tail = b.prev;
    b.prev = b.next = -1;
    b.in_free = false;
    --nfree;
  }

  // A block from the free queue's head for new content: its cache entry goes.
  int32_t take_fresh() {
    const int32_t id = head;
    unlink(id);
    Block& b = blocks[id];
    if (b.cached) {
      auto it = cache.find(b.hash);
      if (it != cache.end() && it->second == id) cache.erase(it);
      b.cached = false;
    }
    b.ref = 1;
    return id;
  }

  // The longest cached chain of full blocks of r's known tokens, at most
  // (known - 1) / 16 blocks.
  void match_prefix(const Request& r, std::vector<int32_t>& ids, uint64_t& last) const {
    ids.clear();
    last = 0;
    if (!caching || r.tokens.empty()) return;
    const int32_t max_blocks = ((int32_t)r.tokens.size() - 1) / kBlockTokens;
    uint64_t parent = 0;
    for (int32_t b = 0; b < max_blocks; ++b) {
      const int32_t* toks = r.tokens.data() + (size_t)b * kBlockTokens;
      const uint64_t h = block_hash(parent, r.salt, toks);
      auto it = cache.find(h);
      if (it == cache.end()) break;
      const Block& blk = blocks[it->second];
      if (!blk.cached || blk.parent != parent || blk.salt != r.salt ||
          std::memcmp(blk.tokens, toks, sizeof(blk.tokens)) != 0)
        break;
      ids.push_back(it->second);
      parent = h;
    }
    last = parent;
  }

  // Registers r's blocks that are full and not yet hashed.
  void cache_full_blocks(Request& r) {
    while ((int64_t)(r.hashed + 1) * kBlockTokens <= r.computed) {
      const int32_t b = r.hashed;
      const int32_t* toks = r.tokens.data() + (size_t)b * kBlockTokens;
      const uint64_t h = block_hash(r.last_hash, r.salt, toks);
      const int32_t id = r.table[b];
      Block& blk = blocks[id];
      if (!blk.cached && cache.find(h) == cache.end()) {
        cache.emplace(h, id);
        blk.cached = true;
        blk.hash = h;
        blk.parent = r.last_hash;
        blk.salt = r.salt;
        std::memcpy(blk.tokens, toks, sizeof(blk.tokens));
      }
      r.last_hash = h;
      ++r.hashed;
    }
  }
};

namespace {

Request* find_req(paged_bm* bm, int64_t req) {
  auto it = bm->reqs.find(req);
  return it == bm->reqs.end() ? nullptr : &it->second;
}

const Request* find_req(const paged_bm* bm, int64_t req) {
  auto it = bm->reqs.find(req);
  return it == bm->reqs.end() ? nullptr : &it->second;
}

int unknown(int64_t req) {
  return bm_fail(PAGED_BM_EINVAL, "unknown request id " + std::to_string(req));
}

}  // namespace

extern "C" {

paged_bm* paged_bm_create(int64_t num_blocks, int32_t enable_prefix_caching) {
  if (num_blocks < 1 || num_blocks >= (int64_t(1) << 31) / kBlockTokens) {
    bm_fail(PAGED_BM_EINVAL, "num_blocks must be in [1, 2^31 / 16)");
    return nullptr;
  }
  paged_bm* bm = new paged_bm();
  bm->caching = enable_prefix_caching != 0;
  bm->blocks.resize((size_t)num_blocks);
  for (int32_t i = 0; i < (int32_t)num_blocks; ++i) bm->push_back(i);
  return bm;
}

void paged_bm_destroy(paged_bm* bm) { delete bm; }

int paged_bm_add_request(paged_bm* bm, int64_t req, const int32_t* tokens, int32_t n,
                         int64_t salt) {
  if (!bm || !tokens || n < 1) return bm_fail(PAGED_BM_EINVAL, "add_request: null pointer or n < 1");
  if (bm->reqs.count(req)) return bm_fail(PAGED_BM_EINVAL, "request id " + std::to_string(req) + " exists");
  Request& r = bm->reqs[req];
  r.salt = salt;
  r.tokens.assign(tokens, tokens + n);
  return PAGED_BM_OK;
}

int paged_bm_append_tokens(paged_bm* bm, int64_t req, const int32_t* tokens, int32_t n) {
  if (!bm || n < 0 || (n > 0 && !tokens)) return bm_fail(PAGED_BM_EINVAL, "append_tokens: bad arguments");
  Request* r = find_req(bm, req);
  if (!r) return unknown(req);
  r->tokens.insert(r->tokens.end(), tokens, tokens + n);
  return PAGED_BM_OK;
}

int paged_bm_num_cached_tokens(const paged_bm* bm, int64_t req, int32_t* num_cached) {
  if (!bm || !num_cached) return bm_fail(PAGED_BM_EINVAL, "num_cached_tokens: null pointer");
  const Request* r = find_req(bm, req);
  if (!r) return unknown(req);
  if (r->table.empty() && r->computed == 0) {
    std::vector<int32_t> ids;
    uint64_t last = 0;
    bm->match_prefix(*r, ids, last);
    *num_cached = (int32_t)ids.size() * kBlockTokens;
  } else {
    *num_cached = r->computed;
  }
  return PAGED_BM_OK;
}

int paged_bm_allocate_slots(paged_bm* bm, int64_t req, int32_t num_new, int32_t* slots) {
  if (!bm || num_new < 0) return bm_fail(PAGED_BM_EINVAL, "allocate_slots: bad arguments");
  Request* r = find_req(bm, req);
  if (!r) return unknown(req);
  std::vector<int32_t> hits;
  uint64_t last = 0;
  const bool first = r->table.empty() && r->computed == 0;
  if (first) bm->match_prefix(*r, hits, last);
  const int64_t computed = first ? (int64_t)hits.size() * kBlockTokens : r->computed;
  const int64_t end = computed + num_new;
  if (end > (int64_t)r->tokens.size())
    return bm_fail(PAGED_BM_EINVAL, "allocate_slots: computed + num_new exceeds the known tokens");
  const int64_t have = (int64_t)r->table.size() + (int64_t)hits.size();
  const int64_t need = std::max<int64_t>(0, (end + kBlockTokens - 1) / kBlockTokens - have);
  int64_t hits_free = 0;
  for (int32_t id : hits) hits_free += bm->blocks[id].in_free ? 1 : 0;
  if (need > bm->nfree - hits_free)
    return bm_fail(PAGED_BM_ENOSPACE, "allocate_slots: " + std::to_string(need) +
                                          " blocks needed, " + std::to_string(bm->nfree - hits_free) +
                                          " free");
  for (int32_t id : hits) {
    Block& b = bm->blocks[id];
    if (b.in_free) bm->unlink(id);
    ++b.ref;
    r->table.push_back(id);
  }
  if (first) {
    r->computed = (int32_t)computed;
    r->hashed = (int32_t)hits.size();
    r->last_hash = last;
  }
  for (int64_t i = 0; i < need; ++i) r->table.push_back(bm->take_fresh());
  if (slots) {
    for (int64_t p = computed; p < end; ++p)
      slots[p - computed] = r->table[(size_t)(p / kBlockTokens)] * kBlockTokens + (int32_t)(p % kBlockTokens);
  }
  r->computed = (int32_t)end;
  if (bm->caching) bm->cache_full_blocks(*r);
  return PAGED_BM_OK;
}

int paged_bm_free_request(paged_bm* bm, int64_t req) {
  if (!bm) return bm_fail(PAGED_BM_EINVAL, "free_request: null manager");
  auto it = bm->reqs.find(req);
  if (it == bm->reqs.end()) return unknown(req);
  const std::vector<int32_t>& table = it->second.table;
  for (size_t i = table.size(); i-- > 0;) {
    Block& b = bm->blocks[table[i]];
    if (--b.ref == 0) bm->push_back(table[i]);
  }
  bm->reqs.erase(it);
  return PAGED_BM_OK;
}

int paged_bm_block_table(const paged_bm* bm, int64_t req, int32_t* table, int32_t max_entries,
                         int32_t* num_entries) {
  if (!bm || !num_entries || max_entries < 0 || (max_entries > 0 && !table))
    return bm_fail(PAGED_BM_EINVAL, "block_table: bad arguments");
  const Request* r = find_req(bm, req);
  if (!r) return unknown(req);
  const int32_t n = (int32_t)r->table.size();
  for (int32_t i = 0; i < std::min(n, max_entries); ++i) table[i] = r->table[i];
  *num_entries = n;
  return PAGED_BM_OK;
}

int paged_bm_step_metadata(const paged_bm* bm, const int64_t* reqs, const int32_t* num_new,
                           int32_t num_seqs, int32_t width, int32_t* block_tables,
                           int32_t* cu_seqlens_q, int32_t* seq_lens, int32_t* slot_mapping) {
  if (!bm || num_seqs < 0 || width < 1 || !cu_seqlens_q ||
      (num_seqs > 0 && (!reqs || !num_new || !block_tables || !seq_lens || !slot_mapping)))
    return bm_fail(PAGED_BM_EINVAL, "step_metadata: bad arguments");
  cu_seqlens_q[0] = 0;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const Request* r = find_req(bm, reqs[s]);
    if (!r) return unknown(reqs[s]);
    const int32_t L = r->computed;
    const int32_t n = num_new[s];
    if (n < 0 || n > L) return bm_fail(PAGED_BM_EINVAL, "step_metadata: num_new outside [0, L]");
    if ((int64_t)r->table.size() > width)
      return bm_fail(PAGED_BM_EINVAL, "step_metadata: a block table is wider than width");
    int32_t* row = block_tables + (size_t)s * width;
    for (int32_t i = 0; i < width; ++i) row[i] = i < (int32_t)r->table.size() ? r->table[i] : -1;
    seq_lens[s] = L;
    cu_seqlens_q[s + 1] = cu_seqlens_q[s] + n;
    int32_t* out = slot_mapping + cu_seqlens_q[s];
    for (int32_t p = L - n; p < L; ++p)
      out[p - (L - n)] = r->table[p / kBlockTokens] * kBlockTokens + p % kBlockTokens;
  }
  return PAGED_BM_OK;
}

int64_t paged_bm_num_free_blocks(const paged_bm* bm) { return bm ? bm->nfree : -1; }

int64_t paged_bm_num_cached_blocks(const paged_bm* bm) { return bm ? (int64_t)bm->cache.size() : -1; }

int32_t paged_bm_ref_count(const paged_bm* bm, int64_t block) {
  if (!bm || block < 0 || block >= (int64_t)bm->blocks.size()) return -1;
  return bm->blocks[(size_t)block].ref;
}

int64_t paged_bm_free_queue(const paged_bm* bm, int32_t* ids, int64_t max_ids) {
  if (!bm) return -1;
  int64_t n = 0;
  for (int32_t id = bm->head; id >= 0; id = bm->blocks[id].next, ++n)
    if (ids && n < max_ids) ids[n] = id;
  return n;
}

const char* paged_bm_last_error(void) { return g_bm_error.c_str(); }

}  // extern "C"
