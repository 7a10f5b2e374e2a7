// Host-side paged KV block manager: the bookkeeping that produces the block
// tables and slot mappings the attention kernels consume.
//
// What it does (MiniLLM Runtime: "Features" - block allocation, release,
// reuse, reference counting, prefix-cache lookup with shared ownership;
// mini_engine "Features": a block gets its hash the moment it is full; miniserve
// "Architecture" - KVCacheManager with chained hashes, refcounts and an LRU
// free list - and its request-state diagram and "Engine" flowchart):
//
// * Pages are reference counted.  Free pages sit in an LRU list: new pages
//   are taken from its front, pages whose count drops to zero go to its tail
//   in block-table order.
// * A page that fills is registered under the chained hash of its token
//   prefix (hash of the previous block's hash and this block's tokens).  A
//   freed page keeps its registration, so a later request with the same
//   prefix reclaims it, until the page is taken for new content.
// * find_cached_prefix walks the prompt block by block and stops at the first
//   miss, and always leaves at least one token to compute.  A hit is checked
//   against the stored tokens and the parent's hash, so a hash collision is
//   a miss, never a wrong page.
// * Admission (prefix lookup + first allocation) and allocation are all or
//   nothing.
//
// Every operation is O(tokens touched): the free list is intrusive (prev/next
// arrays), the prefix map an open hash table keyed by the 64-bit chain hash.

#include "pka.h"

#include <cstdint>
#include <cstring>
#include <new>
#include <unordered_map>
#include <vector>

namespace {

// 64-bit chained block hash: splitmix64-style mixing over the parent hash and
// the block's token ids.
uint64_t mix64(uint64_t x) {
  x ^= x >> 30;
  x *= 0xbf58476d1ce4e5b9ull;
  x ^= x >> 27;
  x *= 0x94d049bb133111ebull;
  x ^= x >> 31;
  return x;
}

uint64_t chain_hash(uint64_t parent, const int32_t* toks, int n) {
  uint64_t h = mix64(parent ^ 0x9e3779b97f4a7c15ull);
  for (int i = 0; i < n; ++i) h = mix64(h ^ (uint64_t)(uint32_t)toks[i] ^ ((uint64_t)i << 32));
  return h;
}

constexpr uint64_t kRootHash = 0x6a09e667f3bcc908ull;

struct Request {
  std::vector<int32_t> tokens;
  std::vector<int32_t> blocks;
  int32_t computed = 0;
  int32_t hashed = 0;       // leading full blocks whose chain hash is known
  uint64_t tail = kRootHash;  // chain hash of block hashed - 1 (root before any)
};

}  // namespace

struct pka_block_manager {
  int32_t N, B;
  std::vector<int32_t> refcount;
  std::vector<int32_t> prev, next;  // intrusive LRU free list; -1 = none
  std::vector<uint8_t> in_free;
  int32_t head = -1, tail = -1, nfree = 0;
  // Registration of a page: its chain hash, its parent's chain hash and its
  // tokens (to confirm hits).
  std::vector<uint8_t> registered;
  std::vector<uint64_t> page_hash, page_parent;
  std::vector<int32_t> page_tokens;  // N * B
  std::unordered_map<uint64_t, int32_t> hash_to_page;
  std::unordered_map<int64_t, Request> reqs;

  pka_block_manager(int32_t n, int32_t b)
      : N(n), B(b), refcount(n, 0), prev(n, -1), next(n, -1), in_free(n, 0), registered(n, 0), page_hash(n, 0),
        page_parent(n, 0), page_tokens((size_t)n * b, 0) {
    for (int32_t i = 0; i < n; ++i) push_tail(i);
  }

  void push_tail(int32_t b) {
    prev[b] = tail;
    next[b] = -1;
    if (tail >= 0) next[tail] = b;
    else head = b;
    tail = b;
    in_free[b] = 1;
    ++nfree;
  }
  void unlink(int32_t b) {
    if (prev[b] >= 0) next[prev[b]] = next[b];
    else head = next[b];
    if (next[b] >= 0) prev[next[b]] = prev[b];
    else tail = prev[b];
    prev[b] = next[b] = -1;
    in_free[b] = 0;
    --nfree;
  }
  int32_t pop_new() {  // LRU front; the page's old content (and registration) is gone
    const int32_t b = head;
    unlink(b);
    if (registered[b]) {
      auto it = hash_to_page.find(page_hash[b]);
      if (it != hash_to_page.end() && it->second == b) hash_to_page.erase(it);
      registered[b] = 0;
    }
    refcount[b] = 1;
    return b;
  }
  int32_t blocks_for(int64_t ntok) const { return (int32_t)((ntok + B - 1) / B); }

  // Pages of the request's cached whole-block prefix (at least one token left).
  void find_prefix(const Request& r, std::vector<int32_t>* hits) const {
    hits->clear();
    uint64_t parent = kRootHash;
    const int32_t nb = (int32_t)(r.tokens.size() / B);
    for (int32_t j = 0; j < nb; ++j) {
      const int32_t* t = r.tokens.data() + (size_t)j * B;
      const uint64_t h = chain_hash(parent, t, B);
      auto it = hash_to_page.find(h);
      if (it == hash_to_page.end()) break;
      const int32_t p = it->second;
      if (page_parent[p] != parent || std::memcmp(&page_tokens[(size_t)p * B], t, sizeof(int32_t) * B) != 0) break;
      hits->push_back(p);
      parent = h;
    }
    if (!hits->empty() && (int64_t)hits->size() * B >= (int64_t)r.tokens.size()) hits->pop_back();
  }

  // Register the blocks the request's computed tokens have filled, continuing
  // the request's hash chain from its last hashed block.
  void register_filled(Request& r) {
    const int32_t full = r.computed / B;
    for (int32_t j = r.hashed; j < full; ++j) {
      const int32_t* t = r.tokens.data() + (size_t)j * B;
      const uint64_t h = chain_hash(r.tail, t, B);
      const int32_t p = r.blocks[j];
      if (!registered[p] && hash_to_page.find(h) == hash_to_page.end()) {
        hash_to_page.emplace(h, p);
        registered[p] = 1;
        page_hash[p] = h;
        page_parent[p] = r.tail;
        std::memcpy(&page_tokens[(size_t)p * B], t, sizeof(int32_t) * B);
      }
      r.tail = h;
    }
    if (full > r.hashed) r.hashed = full;
  }
};

extern "C" {

pka_block_manager* pka_bm_create(int32_t num_blocks, int32_t block_size) {
  if (num_blocks <= 0 || block_size <= 0) return nullptr;
  return new (std::nothrow) pka_block_manager(num_blocks, block_size);
}

void pka_bm_destroy(pka_block_manager* m) { delete m; }

int32_t pka_bm_num_free(const pka_block_manager* m) { return m ? m->nfree : -1; }

int32_t pka_bm_refcount(const pka_block_manager* m, int32_t block) {
  if (!m || block < 0 || block >= m->N) return -1;
  return m->refcount[block];
}

int32_t pka_bm_add_request(pka_block_manager* m, int64_t req_id, const int32_t* tokens, int32_t num_tokens) {
  if (!m || num_tokens < 0 || (num_tokens > 0 && !tokens)) return PKA_ERR_NULL;
  if (m->reqs.count(req_id)) return PKA_ERR_SHAPE;
  Request r;
  r.tokens.assign(tokens, tokens + num_tokens);
  m->reqs.emplace(req_id, std::move(r));
  return PKA_OK;
}

int32_t pka_bm_append_token(pka_block_manager* m, int64_t req_id, int32_t token) {
  if (!m) return PKA_ERR_NULL;
  auto it = m->reqs.find(req_id);
  if (it == m->reqs.end()) return PKA_ERR_SHAPE;
  it->second.tokens.push_back(token);
  return PKA_OK;
}

int32_t pka_bm_find_cached_prefix(const pka_block_manager* m, int64_t req_id, int32_t* blocks, int32_t max_blocks) {
  if (!m) return -PKA_ERR_NULL;
  auto it = m->reqs.find(req_id);
  if (it == m->reqs.end()) return -PKA_ERR_SHAPE;
  std::vector<int32_t> hits;
  m->find_prefix(it->second, &hits);
  if ((int32_t)hits.size() > max_blocks || (!hits.empty() && !blocks)) return -PKA_ERR_SHAPE;
  for (size_t i = 0; i < hits.size(); ++i) blocks[i] = hits[i];
  return (int32_t)hits.size();
}

int32_t pka_bm_admit(pka_block_manager* m, int64_t req_id, int32_t first_chunk, int32_t* num_cached_tokens) {
  if (!m || !num_cached_tokens) return -PKA_ERR_NULL;
  auto it = m->reqs.find(req_id);
  if (it == m->reqs.end() || first_chunk < 0) return -PKA_ERR_SHAPE;
  Request& r = it->second;
  if (!r.blocks.empty()) return -PKA_ERR_SHAPE;
  std::vector<int32_t> hits;
  m->find_prefix(r, &hits);
  const int32_t cached = (int32_t)hits.size() * m->B;
  int32_t reclaimed = 0;
  for (int32_t p : hits) reclaimed += m->refcount[p] == 0;
  const int32_t need = m->blocks_for((int64_t)cached + first_chunk) - (int32_t)hits.size();
  if (need > m->nfree - reclaimed) return 0;
  for (int32_t p : hits) {
    if (m->refcount[p] == 0) m->unlink(p);
    ++m->refcount[p];
  }
  r.blocks = hits;
  r.computed = cached;
  r.hashed = (int32_t)hits.size();
  r.tail = hits.empty() ? kRootHash : m->page_hash[hits.back()];
  for (int32_t i = 0; i < need; ++i) r.blocks.push_back(m->pop_new());
  *num_cached_tokens = cached;
  return 1;
}

int32_t pka_bm_allocate(pka_block_manager* m, int64_t req_id, int32_t num_new_tokens) {
  if (!m) return -PKA_ERR_NULL;
  auto it = m->reqs.find(req_id);
  if (it == m->reqs.end() || num_new_tokens < 0) return -PKA_ERR_SHAPE;
  Request& r = it->second;
  const int32_t need = m->blocks_for((int64_t)r.computed + num_new_tokens) - (int32_t)r.blocks.size();
  if (need > m->nfree) return 0;
  for (int32_t i = 0; i < need; ++i) r.blocks.push_back(m->pop_new());
  return 1;
}

int32_t pka_bm_commit(pka_block_manager* m, int64_t req_id, int32_t num_tokens) {
  if (!m) return PKA_ERR_NULL;
  auto it = m->reqs.find(req_id);
  if (it == m->reqs.end() || num_tokens < 0) return PKA_ERR_SHAPE;
  Request& r = it->second;
  const int64_t c = (int64_t)r.computed + num_tokens;
  if (c > (int64_t)r.tokens.size() || c > (int64_t)r.blocks.size() * m->B) return PKA_ERR_SHAPE;
  r.computed = (int32_t)c;
  m->register_filled(r);
  return PKA_OK;
}

int32_t pka_bm_free_request(pka_block_manager* m, int64_t req_id, int32_t keep_request) {
  if (!m) return PKA_ERR_NULL;
  auto it = m->reqs.find(req_id);
  if (it == m->reqs.end()) return PKA_ERR_SHAPE;
  Request& r = it->second;
  for (int32_t p : r.blocks)
    if (--m->refcount[p] == 0) m->push_tail(p);
  r.blocks.clear();
  r.computed = 0;
  r.hashed = 0;
  r.tail = kRootHash;
  if (!keep_request) m->reqs.erase(it);
  return PKA_OK;
}

int32_t pka_bm_block_table(const pka_block_manager* m, int64_t req_id, int32_t* out, int32_t max_blocks) {
  if (!m) return -PKA_ERR_NULL;
  auto it = m->reqs.find(req_id);
  if (it == m->reqs.end()) return -PKA_ERR_SHAPE;
  const auto& b = it->second.blocks;
  if ((int32_t)b.size() > max_blocks || (!b.empty() && !out)) return -PKA_ERR_SHAPE;
  for (size_t i = 0; i < b.size(); ++i) out[i] = b[i];
  return (int32_t)b.size();
}

int32_t pka_bm_slot_mapping(const pka_block_manager* m, int64_t req_id, int32_t start, int32_t num_tokens,
                            int64_t* out) {
  if (!m || (num_tokens > 0 && !out)) return PKA_ERR_NULL;
  auto it = m->reqs.find(req_id);
  if (it == m->reqs.end() || start < 0 || num_tokens < 0) return PKA_ERR_SHAPE;
  const auto& b = it->second.blocks;
  if ((int64_t)start + num_tokens > (int64_t)b.size() * m->B) return PKA_ERR_SHAPE;
  for (int32_t i = 0; i < num_tokens; ++i) {
    const int32_t p = start + i;
    out[i] = (int64_t)b[p / m->B] * m->B + p % m->B;
  }
  return PKA_OK;
}

int32_t pka_bm_decode_step(pka_block_manager* m, int32_t num_reqs, const int64_t* req_ids, const int32_t* tokens,
                           int64_t* slots, int32_t* ok) {
  if (!m || num_reqs < 0 || (num_reqs > 0 && (!req_ids || !tokens || !slots || !ok))) return -PKA_ERR_NULL;
  int32_t done = 0;
  for (int32_t i = 0; i < num_reqs; ++i) {
    auto it = m->reqs.find(req_ids[i]);
    if (it == m->reqs.end()) return -PKA_ERR_SHAPE;
    Request& r = it->second;
    r.tokens.push_back(tokens[i]);
    const int32_t need = m->blocks_for((int64_t)r.computed + 1) - (int32_t)r.blocks.size();
    if (need > m->nfree) {
      ok[i] = 0;
      slots[i] = -1;
      continue;
    }
    for (int32_t k = 0; k < need; ++k) r.blocks.push_back(m->pop_new());
    const int32_t p = r.computed;
    slots[i] = (int64_t)r.blocks[p / m->B] * m->B + p % m->B;
    r.computed = p + 1;
    m->register_filled(r);
    ok[i] = 1;
    ++done;
  }
  return done;
}

int32_t pka_bm_num_computed(const pka_block_manager* m, int64_t req_id) {
  if (!m) return -PKA_ERR_NULL;
  auto it = m->reqs.find(req_id);
  if (it == m->reqs.end()) return -PKA_ERR_SHAPE;
  return it->second.computed;
}

}  // extern "C"
