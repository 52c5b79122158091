// Host block manager: free list, reference counts, fork and copy-on-write,
// and automatic prefix caching.
//
// Follows "理解 vLLM PagedAttention" sections 三 (blocks taken from one global
// pool, appended as a sequence grows, returned when it ends, shared by pointing
// logical blocks of several sequences at one physical block), 四 (allocation on
// demand; waste confined to the last block) and 六 (sharing with copy-on-write
// on divergence; reuse of computed blocks for a repeated prefix, with an index,
// lifecycle and eviction), "vLLM 核心概念" sections "按需分配", "内存共享" and
// 前缀缓存, and "PagedAttention 实战" section "Prefix Caching" with its fifth
// step (eviction, tenant isolation, invalidation on a model change).
// The policies the pages leave open are stated in pa.h next to the pa_bm_*
// declarations.  Pure host code: no device calls.
//
// Prefix index.  A full block is identified by its whole token prefix.  Each
// distinct prefix that has been committed is a node of a trie keyed by
// (parent node id, the block's 16 token ids); the parent of a first block is a
// per-tenant root id -(tenant + 1).  The nodes live in the hash map itself, so
// one probe per block resolves a lookup.  A node holds the block indexed for
// that prefix (or -1) and stays alive while something pins it: its indexed
// block, a child node, or a live sequence whose committed tokens end on it.
// So a prefix keeps its identity while anything below it is still indexed, and
// a lookup compares keys exactly (no hash collision can alias two prefixes).
// Evictable blocks (indexed, refcount 0) sit on an intrusive LRU list in
// release order.

#include <algorithm>
#include <cstring>
#include <new>
#include <string>
#include <unordered_map>
#include <vector>

#include "pa_internal.h"

namespace {

thread_local std::string g_last_error;

constexpr int kBs = PA_BLOCK_SIZE;

struct PrefixNode;

struct Seq {
  std::vector<int32_t> table;  // logical block j -> physical block
  int64_t len = 0;             // tokens stored
  // prefix caching
  int64_t tenant = 0;
  int64_t committed = 0;       // tokens whose ids are known (a prefix of len)
  PrefixNode* node = nullptr;  // trie node of the committed full blocks (none: root)
  int32_t pend[kBs] = {};      // ids committed into the current partial block
};

struct PrefixKey {
  int64_t parent;
  int32_t tok[kBs];
  bool operator==(const PrefixKey& o) const {
    return parent == o.parent && std::memcmp(tok, o.tok, sizeof tok) == 0;
  }
};

struct PrefixKeyHash {
  size_t operator()(const PrefixKey& k) const {
    uint64_t h = static_cast<uint64_t>(k.parent) * 0x9E3779B97F4A7C15ull;
    for (int i = 0; i < kBs; ++i) {
      h ^= static_cast<uint32_t>(k.tok[i]);
      h *= 0xBF58476D1CE4E5B9ull;
      h ^= h >> 29;
    }
    return static_cast<size_t>(h);
  }
};

struct PrefixNode {
  int64_t id = 0;                 // unique, never reused: the key of the children
  PrefixNode* parent = nullptr;   // nullptr for a first block
  const PrefixKey* key = nullptr; // this node's key inside the map
  int32_t block = -1;             // block indexed for this prefix, or -1
  int32_t pins = 0;               // indexed block + child nodes + sequences ending here
};

int64_t root_id(int64_t tenant) { return -(tenant + 1); }

}  // namespace

struct pa_bm {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::vector<int32_t> free_stack;  // top = back()
  std::vector<int32_t> ref;
  std::unordered_map<int64_t, Seq> seqs;
  std::unordered_map<int32_t, int32_t> scratch_drop;  // reused by batch planning
  int64_t n_shared = 0;             // blocks with refcount > 1

  // prefix caching (off until pa_bm_enable_prefix_cache)
  bool prefix_on = false;
  std::unordered_map<PrefixKey, PrefixNode, PrefixKeyHash> index;  // the trie's nodes
  int64_t next_node = 0;
  std::vector<PrefixNode*> block_node;  // node a block is indexed under, or nullptr
  std::vector<int32_t> lru_prev, lru_next;
  int32_t lru_head = -1, lru_tail = -1;
  int64_t n_evictable = 0, n_indexed = 0;
  int64_t requests = 0, query_blocks = 0, hit_blocks = 0, evictions = 0;

  // host tier for swapping (off until pa_bm_enable_swap)
  int32_t num_host = 0;
  std::vector<int32_t> host_free;   // top = back()
  std::vector<int32_t> host_ref;
  std::unordered_map<int64_t, Seq> swapped;   // tables hold host blocks
  std::vector<int32_t> map_scratch;           // per-call block map, -1 when unused

  int64_t available() const { return static_cast<int64_t>(free_stack.size()) + n_evictable; }

  void lru_unlink(int32_t b) {
    const int32_t p = lru_prev[b], n = lru_next[b];
    (p >= 0 ? lru_next[p] : lru_head) = n;
    (n >= 0 ? lru_prev[n] : lru_tail) = p;
    lru_prev[b] = lru_next[b] = -1;
    --n_evictable;
  }
  void lru_push(int32_t b) {
    lru_prev[b] = lru_tail;
    lru_next[b] = -1;
    (lru_tail >= 0 ? lru_next[lru_tail] : lru_head) = b;
    lru_tail = b;
    ++n_evictable;
  }
  static void pin(PrefixNode* n) {
    if (n) ++n->pins;
  }
  // Drops one pin; a node left with none leaves the trie and unpins its parent.
  void unpin(PrefixNode* n) {
    while (n && --n->pins == 0) {
      PrefixNode* parent = n->parent;
      const PrefixKey key = *n->key;   // a copy: erasing frees the original
      index.erase(key);
      n = parent;
    }
  }
  void unindex(int32_t b) {
    PrefixNode* n = block_node[b];
    block_node[b] = nullptr;
    n->block = -1;
    --n_indexed;
    unpin(n);
  }
  // A block whose last reference went away.
  void release(int32_t b) {
    if (prefix_on && block_node[b])
      lru_push(b);
    else
      free_stack.push_back(b);
  }
  static int64_t parent_id(const Seq& s) { return s.node ? s.node->id : root_id(s.tenant); }
  // The 16 committed ids of s's newest full block are in s.pend: index it.
  void index_full_block(Seq& s) {
    const int32_t blk = s.table[s.committed / kBs - 1];
    PrefixKey key;
    key.parent = parent_id(s);
    std::memcpy(key.tok, s.pend, sizeof key.tok);
    auto ins = index.try_emplace(key);
    PrefixNode& nd = ins.first->second;
    if (ins.second) {
      nd.id = next_node++;
      nd.parent = s.node;
      nd.key = &ins.first->first;
      pin(s.node);                    // the new child pins its parent
    }
    if (nd.block < 0 && !block_node[blk]) {
      nd.block = blk;
      block_node[blk] = &nd;
      ++nd.pins;
      ++n_indexed;
    }
    pin(&nd);
    unpin(s.node);
    s.node = &nd;
  }
  // A new sequence on the longest indexed prefix of tokens[0..n) (full blocks, at
  // most (n - 1) / 16); arguments already checked.  Returns its cached tokens.
  int32_t add_cached(int64_t seq_id, int64_t tenant, const int32_t* tokens, int32_t n) {
    Seq& s = seqs[seq_id];
    s.tenant = tenant;
    PrefixNode* node = nullptr;
    const int32_t most = n > 0 ? (n - 1) / kBs : 0;   // one prompt token stays to compute
    int32_t hits = 0;
    PrefixKey key;
    s.table.reserve((n + kBs - 1) / kBs);
    for (; hits < most; ++hits) {
      key.parent = node ? node->id : root_id(tenant);
      std::memcpy(key.tok, tokens + static_cast<int64_t>(hits) * kBs, sizeof key.tok);
      auto it = index.find(key);
      if (it == index.end() || it->second.block < 0) break;
      const int32_t blk = it->second.block;
      if (ref[blk] == 0) lru_unlink(blk);
      ref_inc(blk);
      s.table.push_back(blk);
      node = &it->second;
    }
    s.len = s.committed = static_cast<int64_t>(hits) * kBs;
    s.node = node;
    pin(node);
    requests += 1;
    query_blocks += most;
    hit_blocks += hits;
    return hits * kBs;
  }
  void commit_one(Seq& s, int32_t token) {
    s.pend[s.committed % kBs] = token;
    ++s.committed;
    if (s.committed % kBs == 0) index_full_block(s);
  }

  void ref_inc(int32_t b) {
    if (++ref[b] == 2) ++n_shared;
  }
  // returns the new count
  int32_t ref_dec(int32_t b) {
    if (ref[b]-- == 2) --n_shared;
    return ref[b];
  }

  Seq* find(int64_t id) {
    auto it = seqs.find(id);
    return it == seqs.end() ? nullptr : &it->second;
  }
  const Seq* find(int64_t id) const {
    auto it = seqs.find(id);
    return it == seqs.end() ? nullptr : &it->second;
  }
  // The next block to hand out (the caller has checked available()): the free
  // stack first, then the evictable block released longest ago.
  int32_t pop_free() {
    int32_t b;
    if (!free_stack.empty()) {
      b = free_stack.back();
      free_stack.pop_back();
    } else {
      b = lru_head;
      lru_unlink(b);
      unindex(b);
      ++evictions;
    }
    ref[b] = 1;
    return b;
  }
  // One append whose block needs were already checked against the free list.
  int64_t append_one(Seq& s, int32_t* cow_src, int32_t* cow_dst) {
    const int32_t off = static_cast<int32_t>(s.len % block_size);
    int32_t blk;
    *cow_src = -1;
    *cow_dst = -1;
    if (off == 0) {
      blk = pop_free();
      s.table.push_back(blk);
    } else {
      const int32_t last = s.table.back();
      if (ref[last] > 1) {
        blk = pop_free();
        ref_dec(last);
        s.table.back() = blk;
        *cow_src = last;
        *cow_dst = blk;
      } else {
        blk = last;
      }
    }
    s.len += 1;
    return static_cast<int64_t>(blk) * block_size + off;
  }
};

namespace pa {

pa_status fail(pa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

void clear_error() { g_last_error.clear(); }

}  // namespace pa

extern "C" {

const char* pa_last_error(void) { return g_last_error.c_str(); }

const char* pa_status_string(pa_status s) {
  switch (s) {
    case PA_OK: return "PA_OK";
    case PA_ERR_INVALID_ARG: return "PA_ERR_INVALID_ARG";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED";
    case PA_ERR_OUT_OF_BLOCKS: return "PA_ERR_OUT_OF_BLOCKS";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE";
    case PA_ERR_HIP: return "PA_ERR_HIP";
    case PA_ERR_NOT_FOUND: return "PA_ERR_NOT_FOUND";
  }
  return "PA_ERR_UNKNOWN";
}

pa_status pa_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                       pa_bm** out) {
  if (!out) return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_create: out is NULL");
  *out = nullptr;
  if (num_blocks <= 0) return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_create: num_blocks %d", num_blocks);
  if (block_size != PA_BLOCK_SIZE && block_size != 2 * PA_BLOCK_SIZE)
    return pa::fail(PA_ERR_UNSUPPORTED, "pa_bm_create: block_size %d (16 or 32)", block_size);
  pa_bm* bm = new (std::nothrow) pa_bm;
  if (!bm) return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_create: out of host memory");
  bm->num_blocks = num_blocks;
  bm->block_size = block_size;
  bm->ref.assign(num_blocks, 0);
  bm->free_stack.resize(num_blocks);
  if (free_order) {
    std::vector<char> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      const int32_t b = free_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete bm;
        return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_create: free_order is not a permutation (entry %d = %d)", i, b);
      }
      seen[b] = 1;
      bm->free_stack[num_blocks - 1 - i] = b;  // free_order[0] on top
    }
  } else {
    for (int32_t i = 0; i < num_blocks; ++i) bm->free_stack[num_blocks - 1 - i] = i;
  }
  *out = bm;
  return PA_OK;
}

void pa_bm_destroy(pa_bm* bm) { delete bm; }

pa_status pa_bm_add_seq(pa_bm* bm, int64_t seq_id) {
  if (!bm) return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_add_seq: bm is NULL");
  if (bm->find(seq_id) || bm->swapped.count(seq_id))
    return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_add_seq: sequence %lld exists", (long long)seq_id);
  bm->seqs.emplace(seq_id, Seq{});
  return PA_OK;
}

pa_status pa_bm_append_batch(pa_bm* bm, int32_t n, const int64_t* seq_ids, int64_t* slots,
                             int32_t* cow_pairs, int32_t cow_cap, int32_t* n_cow) {
  if (!bm || n < 0 || (n > 0 && (!seq_ids || !slots)) || !n_cow)
    return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_append_batch: bad arguments");
  if (cow_cap < n || (n > 0 && !cow_pairs))
    return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_append_batch: cow_cap %d < n %d", cow_cap, n);
  *n_cow = 0;
  std::vector<Seq*> ptr(n);
  for (int32_t i = 0; i < n; ++i) {
    ptr[i] = bm->find(seq_ids[i]);
    if (!ptr[i]) return pa::fail(PA_ERR_NOT_FOUND, "pa_bm_append_batch: no sequence %lld", (long long)seq_ids[i]);
  }
  // distinct ids
  {
    std::vector<int64_t> ids(seq_ids, seq_ids + n);
    std::sort(ids.begin(), ids.end());
    if (std::adjacent_find(ids.begin(), ids.end()) != ids.end())
      return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_append_batch: a sequence appears twice");
  }
  // plan: count blocks taken, with the reference drops earlier copies make
  auto& drop = bm->scratch_drop;
  drop.clear();
  int64_t need = 0;
  for (int32_t i = 0; i < n; ++i) {
    const Seq& s = *ptr[i];
    if (s.len % bm->block_size == 0) {
      ++need;
    } else {
      const int32_t last = s.table.back();
      auto it = drop.find(last);
      const int32_t pending = it == drop.end() ? 0 : it->second;
      if (bm->ref[last] - pending > 1) {
        ++need;
        drop[last] = pending + 1;
      }
    }
  }
  if (need > bm->available())
    return pa::fail(PA_ERR_OUT_OF_BLOCKS, "pa_bm_append_batch: needs %lld blocks, %lld available",
                    (long long)need, (long long)bm->available());
  int32_t nc = 0;
  for (int32_t i = 0; i < n; ++i) {
    int32_t src, dst;
    slots[i] = bm->append_one(*ptr[i], &src, &dst);
    if (src >= 0) {
      cow_pairs[2 * nc] = src;
      cow_pairs[2 * nc + 1] = dst;
      ++nc;
    }
  }
  *n_cow = nc;
  return PA_OK;
}

pa_status pa_bm_append(pa_bm* bm, int64_t seq_id, int64_t* slot, int32_t* cow_src,
                       int32_t* cow_dst) {
  if (!slot || !cow_src || !cow_dst) return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_append: NULL output");
  int32_t pair[2] = {-1, -1};
  int32_t nc = 0;
  pa_status st = pa_bm_append_batch(bm, 1, &seq_id, slot, pair, 1, &nc);
  if (st != PA_OK) return st;
  *cow_src = nc ? pair[0] : -1;
  *cow_dst = nc ? pair[1] : -1;
  return PA_OK;
}

pa_status pa_bm_append_tokens(pa_bm* bm, int64_t seq_id, int32_t count, int64_t* slots,
                              int32_t* cow_pairs, int32_t cow_cap, int32_t* n_cow) {
  if (!bm || count < 0 || (count > 0 && !slots) || !n_cow)
    return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_append_tokens: bad arguments");
  if (cow_cap < count || (count > 0 && !cow_pairs))
    return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_append_tokens: cow_cap %d < count %d", cow_cap, count);
  *n_cow = 0;
  Seq* s = bm->find(seq_id);
  if (!s) return pa::fail(PA_ERR_NOT_FOUND, "pa_bm_append_tokens: no sequence %lld", (long long)seq_id);
  if (count == 0) return PA_OK;
  // blocks taken: a copy of a shared partial last block (first token only),
  // plus one block per block boundary crossed
  const int64_t len = s->len;
  const int64_t bs = bm->block_size;
  int64_t need = 0;
  if (len % bs != 0 && bm->ref[s->table.back()] > 1) need += 1;
  const int64_t first_new_block = (len + bs - 1) / bs;       // blocks held now
  const int64_t blocks_after = (len + count + bs - 1) / bs;
  need += blocks_after - first_new_block;
  if (need > bm->available())
    return pa::fail(PA_ERR_OUT_OF_BLOCKS, "pa_bm_append_tokens: needs %lld blocks, %lld available",
                    (long long)need, (long long)bm->available());
  int32_t nc = 0;
  for (int32_t i = 0; i < count; ++i) {
    int32_t src, dst;
    slots[i] = bm->append_one(*s, &src, &dst);
    if (src >= 0) {
      cow_pairs[2 * nc] = src;
      cow_pairs[2 * nc + 1] = dst;
      ++nc;
    }
  }
  *n_cow = nc;
  return PA_OK;
}

pa_status pa_bm_fork(pa_bm* bm, int64_t parent, int64_t child) {
  if (!bm) return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_fork: bm is NULL");
  const Seq* p = bm->find(parent);
  if (!p) return pa::fail(PA_ERR_NOT_FOUND, "pa_bm_fork: no resident sequence %lld", (long long)parent);
  if (bm->find(child) || bm->swapped.count(child))
    return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_fork: sequence %lld exists", (long long)child);
  Seq c = *p;
  for (int32_t b : c.table) bm->ref_inc(b);
  bm->pin(c.node);
  bm->seqs.emplace(child, std::move(c));
  return PA_OK;
}

pa_status pa_bm_free_seq(pa_bm* bm, int64_t seq_id) {
  if (!bm) return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_free_seq: bm is NULL");
  auto sw = bm->swapped.find(seq_id);
  if (sw != bm->swapped.end()) {            // a swapped-out sequence holds host blocks
    const std::vector<int32_t>& t = sw->second.table;
    for (auto r = t.rbegin(); r != t.rend(); ++r)
      if (--bm->host_ref[*r] == 0) bm->host_free.push_back(*r);
    bm->unpin(sw->second.node);
    bm->swapped.erase(sw);
    return PA_OK;
  }
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return pa::fail(PA_ERR_NOT_FOUND, "pa_bm_free_seq: no sequence %lld", (long long)seq_id);
  const std::vector<int32_t>& t = it->second.table;
  for (auto r = t.rbegin(); r != t.rend(); ++r) {
    if (bm->ref_dec(*r) == 0) bm->release(*r);
  }
  bm->unpin(it->second.node);
  bm->seqs.erase(it);
  return PA_OK;
}

pa_status pa_bm_seq_len(const pa_bm* bm, int64_t seq_id, int64_t* len) {
  if (!bm || !len) return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_seq_len: NULL argument");
  const Seq* s = bm->find(seq_id);
  if (!s) {
    auto sw = bm->swapped.find(seq_id);
    if (sw != bm->swapped.end()) s = &sw->second;
  }
  if (!s) return pa::fail(PA_ERR_NOT_FOUND, "pa_bm_seq_len: no sequence %lld", (long long)seq_id);
  *len = s->len;
  return PA_OK;
}

pa_status pa_bm_block_table(const pa_bm* bm, int64_t seq_id, int32_t* out, int32_t cap,
                            int32_t* n) {
  if (!bm || !n || cap < 0 || (cap > 0 && !out))
    return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_block_table: bad arguments");
  const Seq* s = bm->find(seq_id);
  if (!s) return pa::fail(PA_ERR_NOT_FOUND, "pa_bm_block_table: no sequence %lld", (long long)seq_id);
  const int32_t m = static_cast<int32_t>(s->table.size());
  std::copy_n(s->table.begin(), std::min(m, cap), out);   // (memcpy of nothing from NULL is UB)
  *n = m;
  return PA_OK;
}

pa_status pa_bm_pack(const pa_bm* bm, int32_t n, const int64_t* seq_ids, int32_t* tables,
                     int32_t max_blocks, int32_t* ctx_lens) {
  if (!bm || n < 0 || max_blocks <= 0 || (n > 0 && (!seq_ids || !tables || !ctx_lens)))
    return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_pack: bad arguments");
  // tables are written in the pool's 16-token tiles: block b of a 32-token manager
  // is tiles 2 b and 2 b + 1
  const int32_t f = bm->block_size / PA_BLOCK_SIZE;
  for (int32_t i = 0; i < n; ++i) {
    const Seq* s = bm->find(seq_ids[i]);
    if (!s) return pa::fail(PA_ERR_NOT_FOUND, "pa_bm_pack: no sequence %lld", (long long)seq_ids[i]);
    const int64_t m = static_cast<int64_t>(s->table.size()) * f;
    if (m > max_blocks || s->len > INT32_MAX)
      return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_pack: sequence %lld holds %lld tiles > %d",
                      (long long)seq_ids[i], (long long)m, max_blocks);
  }
  for (int32_t i = 0; i < n; ++i) {
    const Seq* s = bm->find(seq_ids[i]);
    int32_t* row = tables + static_cast<int64_t>(i) * max_blocks;
    const int32_t m = static_cast<int32_t>(s->table.size());
    if (f == 1) {
      std::copy_n(s->table.begin(), m, row);
    } else {
      for (int32_t j = 0; j < m; ++j)
        for (int32_t t = 0; t < f; ++t) row[j * f + t] = s->table[j] * f + t;
    }
    std::fill(row + m * f, row + max_blocks, -1);
    ctx_lens[i] = static_cast<int32_t>(s->len);
  }
  return PA_OK;
}

pa_status pa_bm_step(pa_bm* bm, int32_t n, const int64_t* seq_ids, int64_t* slots,
                     int32_t* cow_pairs, int32_t cow_cap, int32_t* n_cow, int32_t* tables,
                     int32_t max_blocks, int32_t* ctx_lens, int32_t* max_ctx) {
  if (!bm || n < 0 || max_blocks <= 0 || !n_cow || !max_ctx ||
      (n > 0 && (!seq_ids || !slots || !tables || !ctx_lens)))
    return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_step: bad arguments");
  *n_cow = 0;
  *max_ctx = 0;
  // the packing must hold every table after its append, checked before anything changes
  for (int32_t i = 0; i < n; ++i) {
    const Seq* s = bm->find(seq_ids[i]);
    if (!s) return pa::fail(PA_ERR_NOT_FOUND, "pa_bm_step: no sequence %lld", (long long)seq_ids[i]);
    const int64_t tiles_after =
        (s->len + bm->block_size) / bm->block_size * (bm->block_size / PA_BLOCK_SIZE);
    if (tiles_after > max_blocks || s->len + 1 > INT32_MAX)
      return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_step: sequence %lld needs %lld tiles > %d",
                      (long long)seq_ids[i], (long long)tiles_after, max_blocks);
  }
  pa_status st = pa_bm_append_batch(bm, n, seq_ids, slots, cow_pairs, cow_cap, n_cow);
  if (st != PA_OK) return st;
  st = pa_bm_pack(bm, n, seq_ids, tables, max_blocks, ctx_lens);
  if (st != PA_OK) return st;   // not reached: checked above
  int32_t m = 0;
  for (int32_t i = 0; i < n; ++i) m = std::max(m, ctx_lens[i]);
  *max_ctx = m;
  return PA_OK;
}

pa_status pa_bm_tile_pairs(const pa_bm* bm, const int32_t* pairs, int32_t n, int32_t* tile_pairs,
                           int32_t cap, int32_t* n_tiles) {
  if (!bm || n < 0 || (n > 0 && (!pairs || !tile_pairs)) || !n_tiles)
    return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_tile_pairs: bad arguments");
  const int32_t f = bm->block_size / PA_BLOCK_SIZE;        // tiles per manager block
  if (static_cast<int64_t>(n) * f > cap)
    return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_tile_pairs: %d pairs need %lld tile pairs, cap %d", n,
                    static_cast<long long>(n) * f, cap);
  // last pair first, so expanding in place never overwrites a pair not yet read
  for (int32_t i = n - 1; i >= 0; --i) {
    const int32_t src = pairs[2 * i], dst = pairs[2 * i + 1];
    for (int32_t j = f - 1; j >= 0; --j) {
      tile_pairs[2 * (f * i + j)] = f * src + j;
      tile_pairs[2 * (f * i + j) + 1] = f * dst + j;
    }
  }
  *n_tiles = n * f;
  return PA_OK;
}

}  // extern "C"

namespace pa {
int64_t bm_shared_blocks(const pa_bm* bm) { return bm->n_shared; }
int32_t bm_tiles_per_block(const pa_bm* bm) { return bm->block_size / PA_BLOCK_SIZE; }
}  // namespace pa

extern "C" {

pa_status pa_bm_refcount(const pa_bm* bm, int32_t block, int32_t* out) {
  if (!bm || !out || block < 0 || block >= bm->num_blocks)
    return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_refcount: bad arguments");
  *out = bm->ref[block];
  return PA_OK;
}

pa_status pa_bm_free_list(const pa_bm* bm, int32_t* out, int32_t cap, int32_t* n) {
  if (!bm || !n || cap < 0 || (cap > 0 && !out))
    return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_free_list: bad arguments");
  const int32_t m = static_cast<int32_t>(bm->free_stack.size());
  const int32_t k = std::min(m, cap);
  for (int32_t i = 0; i < k; ++i) out[i] = bm->free_stack[m - 1 - i];
  *n = m;
  return PA_OK;
}

pa_status pa_bm_stats_get(const pa_bm* bm, pa_bm_stats* out) {
  if (!bm || !out) return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_stats_get: NULL argument");
  std::vector<int32_t> occupied(bm->num_blocks, 0);
  const int64_t bs = bm->block_size;
  for (const auto& kv : bm->seqs) {
    const Seq& s = kv.second;
    for (size_t j = 0; j < s.table.size(); ++j) {
      const int64_t fill = std::min<int64_t>(bs, s.len - static_cast<int64_t>(j) * bs);
      int32_t& o = occupied[s.table[j]];
      o = std::max<int32_t>(o, static_cast<int32_t>(fill));
    }
  }
  int64_t used = 0, occ = 0;
  for (int32_t b = 0; b < bm->num_blocks; ++b) {
    used += bm->ref[b] > 0;
    occ += occupied[b];
  }
  const int64_t shared = bm->n_shared;   // kept up to date by every reference change
  out->num_blocks = bm->num_blocks;
  out->free_blocks = static_cast<int64_t>(bm->free_stack.size());
  out->used_blocks = used;
  out->shared_blocks = shared;
  out->allocated_slots = used * bs;
  out->occupied_slots = occ;
  out->waste = used ? 1.0 - static_cast<double>(occ) / static_cast<double>(used * bs) : 0.0;
  return PA_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Automatic prefix caching
// ---------------------------------------------------------------------------
extern "C" {

pa_status pa_bm_enable_prefix_cache(pa_bm* bm) {
  if (!bm) return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_enable_prefix_cache: bm is NULL");
  if (bm->prefix_on) return PA_OK;
  if (bm->block_size != PA_BLOCK_SIZE)
    return pa::fail(PA_ERR_UNSUPPORTED, "pa_bm_enable_prefix_cache: block_size %d (only 16)",
                    bm->block_size);
  if (!bm->seqs.empty())
    return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_enable_prefix_cache: %zu sequences are live",
                    bm->seqs.size());
  bm->block_node.assign(bm->num_blocks, nullptr);
  bm->lru_prev.assign(bm->num_blocks, -1);
  bm->lru_next.assign(bm->num_blocks, -1);
  bm->prefix_on = true;
  return PA_OK;
}

pa_status pa_bm_add_seq_cached(pa_bm* bm, int64_t seq_id, int64_t tenant, const int32_t* tokens,
                               int32_t n, int32_t* cached_tokens) {
  if (!bm || !cached_tokens || n < 0 || (n > 0 && !tokens) || tenant < 0 || tenant == INT64_MAX)
    return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_add_seq_cached: bad arguments");
  *cached_tokens = 0;
  if (!bm->prefix_on)
    return pa::fail(PA_ERR_UNSUPPORTED, "pa_bm_add_seq_cached: prefix caching is off");
  if (bm->find(seq_id) || bm->swapped.count(seq_id))
    return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_add_seq_cached: sequence %lld exists", (long long)seq_id);
  *cached_tokens = bm->add_cached(seq_id, tenant, tokens, n);
  return PA_OK;
}

pa_status pa_bm_admit_batch(pa_bm* bm, int32_t n, const int64_t* seq_ids, const int64_t* tenants,
                            const int32_t* tokens, const int64_t* offsets, int32_t* cached,
                            int64_t* slots, int64_t slot_cap, int32_t* admitted) {
  if (!bm || n < 0 || !admitted || (n > 0 && (!seq_ids || !offsets || !cached || !slots)))
    return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_admit_batch: bad arguments");
  *admitted = 0;
  if (!bm->prefix_on)
    return pa::fail(PA_ERR_UNSUPPORTED, "pa_bm_admit_batch: prefix caching is off");
  if (n == 0) return PA_OK;
  if (offsets[0] < 0 || (offsets[n] > offsets[0] && !tokens))
    return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_admit_batch: bad offsets or tokens");
  for (int32_t i = 0; i < n; ++i) {
    const int64_t len = offsets[i + 1] - offsets[i];
    if (len < 0 || len > INT32_MAX)
      return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_admit_batch: prompt %d has %lld tokens", i, (long long)len);
    if (tenants && (tenants[i] < 0 || tenants[i] == INT64_MAX))
      return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_admit_batch: tenant %lld", (long long)tenants[i]);
    if (bm->find(seq_ids[i]) || bm->swapped.count(seq_ids[i]))
      return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_admit_batch: sequence %lld exists", (long long)seq_ids[i]);
  }
  if (slot_cap < offsets[n] - offsets[0])
    return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_admit_batch: slot_cap %lld < %lld prompt tokens",
                    (long long)slot_cap, (long long)(offsets[n] - offsets[0]));
  {
    std::vector<int64_t> ids(seq_ids, seq_ids + n);
    std::sort(ids.begin(), ids.end());
    if (std::adjacent_find(ids.begin(), ids.end()) != ids.end())
      return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_admit_batch: a sequence appears twice");
  }
  int64_t pos = 0;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t* p = tokens + offsets[i];
    const int32_t len = static_cast<int32_t>(offsets[i + 1] - offsets[i]);
    const int32_t c = bm->add_cached(seq_ids[i], tenants ? tenants[i] : 0, p, len);
    Seq& s = bm->seqs.find(seq_ids[i])->second;
    // the sequence holds c/16 full blocks: every further block is new
    const int64_t need = (static_cast<int64_t>(len) + kBs - 1) / kBs - c / kBs;
    if (need > bm->available()) {
      pa_bm_free_seq(bm, seq_ids[i]);
      return pa::fail(PA_ERR_OUT_OF_BLOCKS, "pa_bm_admit_batch: request %d needs %lld blocks, "
                      "%lld available", i, (long long)need, (long long)bm->available());
    }
    int32_t src, dst;
    for (int32_t t = c; t < len; ++t) slots[pos++] = bm->append_one(s, &src, &dst);
    for (int32_t t = c; t < len; ++t) bm->commit_one(s, p[t]);
    cached[i] = c;
    *admitted = i + 1;
  }
  return PA_OK;
}

pa_status pa_bm_commit_tokens(pa_bm* bm, int64_t seq_id, const int32_t* tokens, int32_t count) {
  if (!bm || count < 0 || (count > 0 && !tokens))
    return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_commit_tokens: bad arguments");
  if (!bm->prefix_on)
    return pa::fail(PA_ERR_UNSUPPORTED, "pa_bm_commit_tokens: prefix caching is off");
  Seq* s = bm->find(seq_id);
  if (!s) return pa::fail(PA_ERR_NOT_FOUND, "pa_bm_commit_tokens: no sequence %lld", (long long)seq_id);
  if (s->committed + count > s->len)
    return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_commit_tokens: %d ids for %lld uncommitted tokens",
                    count, (long long)(s->len - s->committed));
  for (int32_t i = 0; i < count; ++i) bm->commit_one(*s, tokens[i]);
  return PA_OK;
}

pa_status pa_bm_commit_batch(pa_bm* bm, int32_t n, const int64_t* seq_ids, const int32_t* tokens) {
  if (!bm || n < 0 || (n > 0 && (!seq_ids || !tokens)))
    return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_commit_batch: bad arguments");
  if (!bm->prefix_on)
    return pa::fail(PA_ERR_UNSUPPORTED, "pa_bm_commit_batch: prefix caching is off");
  std::vector<Seq*> ptr(n);
  for (int32_t i = 0; i < n; ++i) {
    ptr[i] = bm->find(seq_ids[i]);
    if (!ptr[i]) return pa::fail(PA_ERR_NOT_FOUND, "pa_bm_commit_batch: no sequence %lld", (long long)seq_ids[i]);
    if (ptr[i]->committed >= ptr[i]->len)
      return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_commit_batch: sequence %lld has no uncommitted token",
                      (long long)seq_ids[i]);
  }
  {
    std::vector<int64_t> ids(seq_ids, seq_ids + n);
    std::sort(ids.begin(), ids.end());
    if (std::adjacent_find(ids.begin(), ids.end()) != ids.end())
      return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_commit_batch: a sequence appears twice");
  }
  for (int32_t i = 0; i < n; ++i) bm->commit_one(*ptr[i], tokens[i]);
  return PA_OK;
}

pa_status pa_bm_prefix_cache_reset(pa_bm* bm) {
  if (!bm) return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_prefix_cache_reset: bm is NULL");
  if (!bm->prefix_on)
    return pa::fail(PA_ERR_UNSUPPORTED, "pa_bm_prefix_cache_reset: prefix caching is off");
  while (bm->lru_head >= 0) {                 // oldest release first onto the free stack
    const int32_t b = bm->lru_head;
    bm->lru_unlink(b);
    bm->unindex(b);
    bm->free_stack.push_back(b);
  }
  for (int32_t b = 0; b < bm->num_blocks; ++b)
    if (bm->block_node[b]) bm->unindex(b);
  return PA_OK;
}

pa_status pa_bm_prefix_stats_get(const pa_bm* bm, pa_bm_prefix_stats* out) {
  if (!bm || !out) return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_prefix_stats_get: NULL argument");
  out->requests = bm->requests;
  out->query_blocks = bm->query_blocks;
  out->hit_blocks = bm->hit_blocks;
  out->cached_blocks = bm->n_indexed;
  out->evictable_blocks = bm->n_evictable;
  out->evictions = bm->evictions;
  return PA_OK;
}

pa_status pa_bm_evictable_list(const pa_bm* bm, int32_t* out, int32_t cap, int32_t* n) {
  if (!bm || !n || cap < 0 || (cap > 0 && !out))
    return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_evictable_list: bad arguments");
  int32_t k = 0;
  if (bm->prefix_on)
    for (int32_t b = bm->lru_head; b >= 0; b = bm->lru_next[b], ++k)
      if (k < cap) out[k] = b;
  *n = k;
  return PA_OK;
}

pa_status pa_bm_cached_list(const pa_bm* bm, int32_t* out, int32_t cap, int32_t* n) {
  if (!bm || !n || cap < 0 || (cap > 0 && !out))
    return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_cached_list: bad arguments");
  int32_t k = 0;
  if (bm->prefix_on)
    for (int32_t b = 0; b < bm->num_blocks; ++b)
      if (bm->block_node[b]) {
        if (k < cap) out[k] = b;
        ++k;
      }
  *n = k;
  return PA_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Swapping between the device pool and a host tier
// ---------------------------------------------------------------------------
namespace {

// Distinct blocks of the tables, in order of first appearance; map[b] receives
// its position.  Returns the count.
int32_t distinct_blocks(const std::vector<const std::vector<int32_t>*>& tables,
                        std::vector<int32_t>& map, std::vector<int32_t>& order) {
  order.clear();
  for (const auto* t : tables)
    for (int32_t b : *t)
      if (map[b] < 0) {
        map[b] = static_cast<int32_t>(order.size());
        order.push_back(b);
      }
  return static_cast<int32_t>(order.size());
}

pa_status check_list(int32_t n, const int64_t* ids, const char* fn) {
  std::vector<int64_t> v(ids, ids + n);
  std::sort(v.begin(), v.end());
  if (std::adjacent_find(v.begin(), v.end()) != v.end())
    return pa::fail(PA_ERR_INVALID_ARG, "%s: a sequence appears twice", fn);
  return PA_OK;
}

}  // namespace

extern "C" {

pa_status pa_bm_enable_swap(pa_bm* bm, int32_t num_host_blocks, const int32_t* host_free_order) {
  if (!bm || num_host_blocks <= 0)
    return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_enable_swap: bad arguments");
  if (bm->num_host > 0) return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_enable_swap: already on");
  if (bm->block_size != PA_BLOCK_SIZE)
    return pa::fail(PA_ERR_UNSUPPORTED, "pa_bm_enable_swap: block_size %d (only 16)", bm->block_size);
  std::vector<int32_t> stack(num_host_blocks);
  if (host_free_order) {
    std::vector<char> seen(num_host_blocks, 0);
    for (int32_t i = 0; i < num_host_blocks; ++i) {
      const int32_t b = host_free_order[i];
      if (b < 0 || b >= num_host_blocks || seen[b])
        return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_enable_swap: host_free_order is not a permutation");
      seen[b] = 1;
      stack[num_host_blocks - 1 - i] = b;
    }
  } else {
    for (int32_t i = 0; i < num_host_blocks; ++i) stack[num_host_blocks - 1 - i] = i;
  }
  bm->num_host = num_host_blocks;
  bm->host_free = std::move(stack);
  bm->host_ref.assign(num_host_blocks, 0);
  bm->map_scratch.assign(std::max(bm->num_blocks, num_host_blocks), -1);
  return PA_OK;
}

pa_status pa_bm_swap_out(pa_bm* bm, int32_t n, const int64_t* seq_ids, int32_t* pairs,
                         int32_t pair_cap, int32_t* n_pairs) {
  const char* fn = "pa_bm_swap_out";
  if (!bm || n < 0 || !n_pairs || (n > 0 && (!seq_ids || !pairs)))
    return pa::fail(PA_ERR_INVALID_ARG, "%s: bad arguments", fn);
  *n_pairs = 0;
  if (bm->num_host == 0) return pa::fail(PA_ERR_UNSUPPORTED, "%s: swapping is off", fn);
  if (n == 0) return PA_OK;
  pa_status st = check_list(n, seq_ids, fn);
  if (st != PA_OK) return st;
  std::vector<Seq*> ptr(n);
  std::vector<const std::vector<int32_t>*> tables(n);
  for (int32_t i = 0; i < n; ++i) {
    ptr[i] = bm->find(seq_ids[i]);
    if (!ptr[i]) return pa::fail(PA_ERR_NOT_FOUND, "%s: no resident sequence %lld", fn, (long long)seq_ids[i]);
    tables[i] = &ptr[i]->table;
  }
  std::vector<int32_t>& map = bm->map_scratch;
  std::vector<int32_t> order;
  const int32_t k = distinct_blocks(tables, map, order);
  auto reset = [&] { for (int32_t b : order) map[b] = -1; };
  if (k > pair_cap) {
    reset();
    return pa::fail(PA_ERR_INVALID_ARG, "%s: %d pairs, pair_cap %d", fn, k, pair_cap);
  }
  if (k > static_cast<int32_t>(bm->host_free.size())) {
    reset();
    return pa::fail(PA_ERR_OUT_OF_BLOCKS, "%s: needs %d host blocks, %zu free", fn, k,
                    bm->host_free.size());
  }
  std::vector<int32_t> host_of(k);
  for (int32_t i = 0; i < k; ++i) {
    host_of[i] = bm->host_free.back();
    bm->host_free.pop_back();
    pairs[2 * i] = order[i];
    pairs[2 * i + 1] = host_of[i];
  }
  std::vector<std::vector<int32_t>> dev_tables(n);
  for (int32_t i = 0; i < n; ++i) {
    Seq& s = *ptr[i];
    dev_tables[i] = s.table;
    for (int32_t& b : s.table) {
      b = host_of[map[b]];
      ++bm->host_ref[b];
    }
    bm->swapped.emplace(seq_ids[i], std::move(s));
    bm->seqs.erase(seq_ids[i]);
  }
  reset();
  // the listed sequences drop their device references, last logical block first
  for (int32_t i = 0; i < n; ++i)
    for (auto r = dev_tables[i].rbegin(); r != dev_tables[i].rend(); ++r)
      if (bm->ref_dec(*r) == 0) bm->release(*r);
  *n_pairs = k;
  return PA_OK;
}

pa_status pa_bm_swap_in(pa_bm* bm, int32_t n, const int64_t* seq_ids, int32_t* pairs,
                        int32_t pair_cap, int32_t* n_pairs) {
  const char* fn = "pa_bm_swap_in";
  if (!bm || n < 0 || !n_pairs || (n > 0 && (!seq_ids || !pairs)))
    return pa::fail(PA_ERR_INVALID_ARG, "%s: bad arguments", fn);
  *n_pairs = 0;
  if (bm->num_host == 0) return pa::fail(PA_ERR_UNSUPPORTED, "%s: swapping is off", fn);
  if (n == 0) return PA_OK;
  pa_status st = check_list(n, seq_ids, fn);
  if (st != PA_OK) return st;
  std::vector<Seq*> ptr(n);
  std::vector<const std::vector<int32_t>*> tables(n);
  for (int32_t i = 0; i < n; ++i) {
    auto it = bm->swapped.find(seq_ids[i]);
    if (it == bm->swapped.end())
      return pa::fail(PA_ERR_NOT_FOUND, "%s: no swapped-out sequence %lld", fn, (long long)seq_ids[i]);
    ptr[i] = &it->second;
    tables[i] = &ptr[i]->table;
  }
  std::vector<int32_t>& map = bm->map_scratch;
  std::vector<int32_t> order;
  const int32_t k = distinct_blocks(tables, map, order);
  auto reset = [&] { for (int32_t b : order) map[b] = -1; };
  if (k > pair_cap) {
    reset();
    return pa::fail(PA_ERR_INVALID_ARG, "%s: %d pairs, pair_cap %d", fn, k, pair_cap);
  }
  if (k > bm->available()) {
    reset();
    return pa::fail(PA_ERR_OUT_OF_BLOCKS, "%s: needs %d blocks, %lld available", fn, k,
                    (long long)bm->available());
  }
  std::vector<int32_t> dev_of(k);
  for (int32_t i = 0; i < k; ++i) {
    dev_of[i] = bm->pop_free();
    bm->ref[dev_of[i]] = 0;            // counted again per reference below
    pairs[2 * i] = order[i];
    pairs[2 * i + 1] = dev_of[i];
  }
  std::vector<std::vector<int32_t>> host_tables(n);
  for (int32_t i = 0; i < n; ++i) {
    Seq& s = *ptr[i];
    host_tables[i] = s.table;
    for (int32_t& b : s.table) {
      b = dev_of[map[b]];
      bm->ref_inc(b);
    }
    bm->seqs.emplace(seq_ids[i], std::move(s));
    bm->swapped.erase(seq_ids[i]);
  }
  reset();
  for (int32_t i = 0; i < n; ++i)
    for (auto r = host_tables[i].rbegin(); r != host_tables[i].rend(); ++r)
      if (--bm->host_ref[*r] == 0) bm->host_free.push_back(*r);
  *n_pairs = k;
  return PA_OK;
}

pa_status pa_bm_is_swapped(const pa_bm* bm, int64_t seq_id, int32_t* out) {
  if (!bm || !out) return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_is_swapped: NULL argument");
  if (bm->swapped.count(seq_id)) {
    *out = 1;
  } else if (bm->find(seq_id)) {
    *out = 0;
  } else {
    return pa::fail(PA_ERR_NOT_FOUND, "pa_bm_is_swapped: no sequence %lld", (long long)seq_id);
  }
  return PA_OK;
}

pa_status pa_bm_host_table(const pa_bm* bm, int64_t seq_id, int32_t* out, int32_t cap, int32_t* n) {
  if (!bm || !n || cap < 0 || (cap > 0 && !out))
    return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_host_table: bad arguments");
  auto it = bm->swapped.find(seq_id);
  if (it == bm->swapped.end())
    return pa::fail(PA_ERR_NOT_FOUND, "pa_bm_host_table: no swapped-out sequence %lld", (long long)seq_id);
  const std::vector<int32_t>& t = it->second.table;
  const int32_t m = static_cast<int32_t>(t.size());
  std::copy_n(t.begin(), std::min(m, cap), out);
  *n = m;
  return PA_OK;
}

pa_status pa_bm_host_refcount(const pa_bm* bm, int32_t block, int32_t* out) {
  if (!bm || !out || block < 0 || block >= bm->num_host)
    return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_host_refcount: bad arguments");
  *out = bm->host_ref[block];
  return PA_OK;
}

pa_status pa_bm_host_free_list(const pa_bm* bm, int32_t* out, int32_t cap, int32_t* n) {
  if (!bm || !n || cap < 0 || (cap > 0 && !out))
    return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_host_free_list: bad arguments");
  const int32_t m = static_cast<int32_t>(bm->host_free.size());
  const int32_t k = std::min(m, cap);
  for (int32_t i = 0; i < k; ++i) out[i] = bm->host_free[m - 1 - i];
  *n = m;
  return PA_OK;
}

}  // extern "C"
