// Host-memory prefix cache of conversation KV between turns: the control
// plane (which token prefixes are cached, in which host slots, what to evict).
//
// What it follows (9c1h.cn news page on Character.AI's inference tricks,
// section 秘訣2; explinks.com "Character.AI 的最佳实践", sections 有状态缓存
// and LRU 缓存结构): attention KV of each conversation's prefix and
// generated messages is kept in host memory between turns; the cached KV is
// organised as a tree with least-recently-used eviction, indexed by a
// rolling hash of the prefix tokens; a new request retrieves the longest
// matching cached prefix, and partially matching messages still hit.
//
// Readings (the pages give no more detail): the unit is a block of
// block_size tokens; a block is identified by the rolling hash of the WHOLE
// token prefix up to its end, so equal hashes mean equal prefixes (checked:
// the block's own tokens and its parent are compared, so a hash collision can
// never return wrong KV). The longest match is the longest chain of cached
// blocks from the start; a partial match reuses every full block it covers.
// Eviction takes the least recently used LEAF (a block no cached block
// extends), so every cached block's prefix stays fully cached; a lookup or an
// insert counts as a use of every block on its chain, oldest first.
//
// Pure host C++ (no HIP calls): the copies are done by the kernels of
// kv_transfer.hip.
#include <cstdint>
#include <cstring>
#include <new>
#include <set>
#include <unordered_map>
#include <utility>
#include <vector>

#include "../../include/mqa_int8.h"

namespace {

// Rolling hash of token prefixes, modulo the Mersenne prime 2^61 - 1:
// h(t_0..t_i) = h(t_0..t_{i-1}) * kBase + (t_i + 1).
constexpr uint64_t kMod = (uint64_t(1) << 61) - 1;
constexpr uint64_t kBase = 0x1c8e31cdcb35b6d5ull % kMod;

uint64_t mulmod(uint64_t a, uint64_t b) {
  const unsigned __int128 p = (unsigned __int128)a * b;
  uint64_t r = (uint64_t)(p & kMod) + (uint64_t)(p >> 61);
  r = (r & kMod) + (r >> 61);
  return r >= kMod ? r - kMod : r;
}
uint64_t roll(uint64_t h, int32_t token) {
  uint64_t r = mulmod(h, kBase) + ((uint64_t)(uint32_t)token + 1);
  return r >= kMod ? r - kMod : r;
}

struct Node {
  uint64_t hash;             // rolling hash of the prefix ending with this block
  int64_t parent;            // node index, -1 for a first block
  int64_t slot;              // host slot holding the block's KV
  int32_t children = 0;
  uint64_t last_use = 0;     // logical clock
  std::vector<int32_t> tokens;
};

}  // namespace

struct mqa_prefix_cache {
  int32_t block_size;
  int64_t capacity;
  std::vector<Node> nodes;          // index = node id; free ids recycled
  std::vector<int64_t> free_ids;
  std::vector<int64_t> free_slots;
  std::unordered_multimap<uint64_t, int64_t> by_hash;
  std::set<std::pair<uint64_t, int64_t>> leaves;  // (last_use, node) of childless nodes
  std::vector<char> live;
  uint64_t clock = 0;
  mqa_prefix_cache_stats stats{};

  bool is_live(int64_t id) const { return id >= 0 && id < (int64_t)live.size() && live[id]; }

  // Node extending `parent` with block tokens tok[0..bs), or -1.
  int64_t find(uint64_t h, int64_t parent, const int32_t* tok) const {
    auto range = by_hash.equal_range(h);
    for (auto it = range.first; it != range.second; ++it) {
      const Node& n = nodes[it->second];
      if (n.parent == parent && std::memcmp(n.tokens.data(), tok, sizeof(int32_t) * block_size) == 0)
        return it->second;
    }
    return -1;
  }

  void touch(int64_t id) {
    Node& n = nodes[id];
    if (n.children == 0) leaves.erase({n.last_use, id});
    n.last_use = ++clock;
    if (n.children == 0) leaves.insert({n.last_use, id});
  }

  void evict_one() {
    const auto it = leaves.begin();
    const int64_t id = it->second;
    leaves.erase(it);
    Node& n = nodes[id];
    auto range = by_hash.equal_range(n.hash);
    for (auto h = range.first; h != range.second; ++h)
      if (h->second == id) {
        by_hash.erase(h);
        break;
      }
    free_slots.push_back(n.slot);
    if (n.parent >= 0) {
      Node& p = nodes[n.parent];
      if (--p.children == 0) leaves.insert({p.last_use, n.parent});
    }
    live[id] = 0;
    n.tokens.clear();
    free_ids.push_back(id);
    ++stats.evicted_blocks;
  }

  int64_t add(uint64_t h, int64_t parent, const int32_t* tok, int64_t slot) {
    int64_t id;
    if (!free_ids.empty()) {
      id = free_ids.back();
      free_ids.pop_back();
    } else {
      id = (int64_t)nodes.size();
      nodes.emplace_back();
      live.push_back(0);
    }
    Node& n = nodes[id];
    n.hash = h;
    n.parent = parent;
    n.slot = slot;
    n.children = 0;
    n.tokens.assign(tok, tok + block_size);
    n.last_use = ++clock;
    live[id] = 1;
    by_hash.emplace(h, id);
    if (parent >= 0) {
      Node& p = nodes[parent];
      if (p.children++ == 0) leaves.erase({p.last_use, parent});
    }
    leaves.insert({n.last_use, id});
    return id;
  }
};

extern "C" {

int mqa_prefix_cache_create(int32_t block_size, int64_t capacity_blocks, mqa_prefix_cache** out) {
  if (!out) return MQA_ERR_NULL;
  *out = nullptr;
  if (block_size <= 0 || capacity_blocks <= 0 || capacity_blocks > ((int64_t)1 << 40)) return MQA_ERR_SHAPE;
  mqa_prefix_cache* c = new (std::nothrow) mqa_prefix_cache();
  if (!c) return MQA_ERR_SHAPE;
  c->block_size = block_size;
  c->capacity = capacity_blocks;
  c->free_slots.reserve((size_t)capacity_blocks);
  for (int64_t s = capacity_blocks - 1; s >= 0; --s) c->free_slots.push_back(s);
  c->stats.capacity_blocks = capacity_blocks;
  *out = c;
  return MQA_OK;
}

void mqa_prefix_cache_destroy(mqa_prefix_cache* c) { delete c; }

int mqa_prefix_cache_match(mqa_prefix_cache* c, const int32_t* tokens, int64_t n_tokens, int64_t* matched_tokens,
                           int64_t* slots) {
  if (!c || !matched_tokens || (n_tokens > 0 && !tokens)) return MQA_ERR_NULL;
  if (n_tokens < 0) return MQA_ERR_SHAPE;
  const int32_t bs = c->block_size;
  const int64_t nb = n_tokens / bs;
  uint64_t h = 0;
  int64_t parent = -1, k = 0;
  std::vector<int64_t> chain;
  for (; k < nb; ++k) {
    for (int32_t i = 0; i < bs; ++i) h = roll(h, tokens[k * bs + i]);
    const int64_t id = c->find(h, parent, tokens + k * bs);
    if (id < 0) break;
    chain.push_back(id);
    parent = id;
  }
  for (size_t i = 0; i < chain.size(); ++i) {
    c->touch(chain[i]);
    if (slots) slots[i] = c->nodes[chain[i]].slot;
  }
  *matched_tokens = k * bs;
  c->stats.lookups += 1;
  c->stats.lookup_tokens += n_tokens;
  c->stats.matched_tokens += k * bs;
  return MQA_OK;
}

int mqa_prefix_cache_insert(mqa_prefix_cache* c, const int32_t* tokens, int64_t n_tokens, int64_t* slots,
                            int64_t* first_new_block, int64_t* n_blocks) {
  if (!c || !slots || !first_new_block || !n_blocks || (n_tokens > 0 && !tokens)) return MQA_ERR_NULL;
  if (n_tokens < 0) return MQA_ERR_SHAPE;
  const int32_t bs = c->block_size;
  const int64_t nb = n_tokens / bs;
  uint64_t h = 0;
  int64_t parent = -1, k = 0;
  std::vector<int64_t> chain;
  std::vector<uint64_t> hashes;
  for (; k < nb; ++k) {
    for (int32_t i = 0; i < bs; ++i) h = roll(h, tokens[k * bs + i]);
    const int64_t id = c->find(h, parent, tokens + k * bs);
    if (id < 0) break;
    chain.push_back(id);
    parent = id;
  }
  // the cached part is used (and so protected from the evictions below)
  for (int64_t id : chain) c->touch(id);
  for (size_t i = 0; i < chain.size(); ++i) slots[i] = c->nodes[chain[i]].slot;
  *first_new_block = k;
  // the rest is added block by block; a block that cannot get a slot (the
  // whole cache is this chain) ends the insert
  int64_t done = k;
  for (; done < nb; ++done) {
    // the search above stopped at block k with its tokens already hashed
    if (done > k)
      for (int32_t i = 0; i < bs; ++i) h = roll(h, tokens[done * bs + i]);
    if (c->free_slots.empty()) {
      // a leaf that is not on this chain (the chain's last block is a leaf
      // but the most recently used; stop rather than evict the chain itself)
      if (c->leaves.empty()) break;
      const int64_t victim = c->leaves.begin()->second;
      if (victim == parent) break;
      c->evict_one();
    }
    const int64_t slot = c->free_slots.back();
    c->free_slots.pop_back();
    parent = c->add(h, parent, tokens + done * bs, slot);
    slots[done] = slot;
    c->stats.inserted_blocks += 1;
  }
  *n_blocks = done;
  c->stats.used_blocks = c->capacity - (int64_t)c->free_slots.size();
  return MQA_OK;
}

int mqa_prefix_cache_get_stats(const mqa_prefix_cache* c, mqa_prefix_cache_stats* out) {
  if (!c || !out) return MQA_ERR_NULL;
  *out = c->stats;
  out->used_blocks = c->capacity - (int64_t)c->free_slots.size();
  return MQA_OK;
}

}  // extern "C"
