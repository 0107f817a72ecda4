// Host-side radix tree over token ids with the KV-pool slot allocator, and the
// decode work planners.
//
// The tree follows the RadixAttention description in the SGLang summary
// (unite.ai), section "SGLang: programming model": KV kept in a radix tree used
// for matching, inserting and evicting; every edge carries a token sequence;
// the nine-step example inserts new turns as nodes and splits a node when two
// sessions (or few-shot queries) share only part of it.  Reuse requires an
// exactly identical prefix ("Prompt Caching" glossary, opening paragraph).
//
// Plain C++17; no HIP.  Every public call validates first and mutates after,
// so a failing call leaves the tree and the allocator unchanged.
#include <algorithm>
#include <cstring>
#include <deque>
#include <new>
#include <queue>
#include <system_error>
#include <tuple>
#include <thread>
#include <unordered_map>
#include <vector>

#include "rc_internal.h"

using rc::fail;

namespace {

struct Node {
  int32_t parent = -1;
  int64_t start = 0;  // absolute position of the edge's first token
  std::vector<int32_t> tok, slot;
  std::unordered_map<int32_t, int32_t> kids;  // first token of child edge -> child
  int64_t last_use = 0;
  int32_t lock = 0;     // locks whose pinned path runs through this node
  uint32_t gen = 0;     // bumped when the node is evicted: stale lock handles are refused
  bool alive = true;
};

// Pages of a paged tree as symbols: every distinct run of page_size token ids
// held by the tree gets a number, so the tree stores, matches and shares whole
// pages exactly as it handles single tokens in an unpaged tree (its "slots"
// are then page ids).  A symbol lives while some tree edge holds it: refs
// counts those edge positions, and a symbol whose count drops to zero (its
// last holder evicted) is removed and its number reused.
struct PageDict {
  int32_t ps = 1;
  std::vector<int32_t> arena;                 // tokens of symbol s at [s * ps, (s + 1) * ps)
  std::unordered_map<uint64_t, int32_t> head;  // hash -> most recent symbol with that hash
  std::vector<int32_t> next;                  // older symbol with the same hash, or -1
  std::vector<int32_t> refs;                  // tree edge positions holding the symbol
  std::vector<int32_t> spare;                 // numbers of removed symbols
  int64_t live = 0;

  // four independent multiply-xor chains over the page, then one mix; lookups
  // compare the tokens themselves, so the hash only spreads the buckets
  uint64_t hash(const int32_t* t) const {
    constexpr uint64_t K = 0x9E3779B97F4A7C15ull;
    uint64_t a = 1, b = 2, c = 3, d = 4;
    int32_t i = 0;
    for (; i + 4 <= ps; i += 4) {
      a = (a ^ (uint32_t)t[i]) * K;
      b = (b ^ (uint32_t)t[i + 1]) * K;
      c = (c ^ (uint32_t)t[i + 2]) * K;
      d = (d ^ (uint32_t)t[i + 3]) * K;
    }
    for (; i < ps; ++i) a = (a ^ (uint32_t)t[i]) * K;
    uint64_t h = a ^ (b << 16 | b >> 48) ^ (c << 32 | c >> 32) ^ (d << 48 | d >> 16);
    return (h ^ (h >> 29)) * K;
  }
  bool same(int32_t s, const int32_t* t) const {
    return std::memcmp(arena.data() + (int64_t)s * ps, t, (size_t)ps * sizeof(int32_t)) == 0;
  }
  // the page's symbol, or -1 if the tree holds no such page (read only: safe on several threads)
  int32_t find(const int32_t* t) const {
    auto it = head.find(hash(t));
    if (it == head.end()) return -1;
    for (int32_t s = it->second; s >= 0; s = next[s])
      if (same(s, t)) return s;
    return -1;
  }
  // the page's symbol, added (with no holders yet) if new; *fresh says which
  int32_t intern(const int32_t* t, bool* fresh) {
    int32_t s = find(t);
    *fresh = s < 0;
    if (s >= 0) return s;
    // every allocation first, so that a failure changes nothing
    const bool reuse = !spare.empty();
    if (!reuse) {
      grow(arena, arena.size() + ps);
      grow(next, next.size() + 1);
      grow(refs, refs.size() + 1);
      grow(spare, next.size() + 1);
    }
    s = reuse ? spare.back() : (int32_t)next.size();
    auto [it, added] = head.try_emplace(hash(t), s);
    const int32_t older = added ? -1 : it->second;
    it->second = s;
    if (reuse) {
      spare.pop_back();
      std::memcpy(arena.data() + (int64_t)s * ps, t, (size_t)ps * sizeof(int32_t));
      next[s] = older;
      refs[s] = 0;
    } else {
      arena.insert(arena.end(), t, t + ps);
      next.push_back(older);
      refs.push_back(0);
    }
    ++live;
    return s;
  }
  // capacity for at least `need` elements, growing geometrically
  static void grow(std::vector<int32_t>& v, size_t need) {
    if (v.capacity() < need) v.reserve(std::max(need, 2 * v.capacity()));
  }
  void remove(int32_t s) {
    auto it = head.find(hash(arena.data() + (int64_t)s * ps));
    if (it->second == s) {
      if (next[s] < 0)
        head.erase(it);
      else
        it->second = next[s];
    } else {
      int32_t p = it->second;
      while (next[p] != s) p = next[p];
      next[p] = next[s];
    }
    next[s] = -1;
    spare.push_back(s);  // capacity reserved when s was added
    --live;
  }
  void acquire(int32_t s) { ++refs[s]; }
  void release(int32_t s) {
    if (--refs[s] == 0) remove(s);
  }
};

}  // namespace

struct rc_radix {
  std::vector<Node> nodes;  // nodes[0] is the root; its edge is empty
  std::vector<int32_t> dead_ids;
  std::deque<int32_t> free_q;
  std::vector<uint8_t> is_free;  // slot is in free_q
  std::vector<uint8_t> in_tree;  // slot is owned by a tree node
  int64_t pool = 0;
  int64_t clock = 0;
  int32_t page = 1;  // tokens per page; > 1: the tree's units are pages (symbols of PageDict)
  PageDict dict;
  rc_radix_stats st{};
};

namespace {

// Walk tokens[0..n) down the tree; visit(node, k) for each edge entered with k
// matched tokens (k >= 1).  Returns the matched length.
template <class F>
int64_t walk(const rc_radix& t, const int32_t* tok, int64_t n, F&& visit) {
  int32_t cur = 0;
  int64_t pos = 0;
  while (pos < n) {
    auto it = t.nodes[cur].kids.find(tok[pos]);
    if (it == t.nodes[cur].kids.end()) break;
    const Node& c = t.nodes[it->second];
    const int64_t len = (int64_t)c.tok.size();
    const int64_t lim = std::min(len, n - pos);
    // whole-edge matches are the common case: compare with memcmp first
    const int64_t k = std::memcmp(c.tok.data(), tok + pos, (size_t)lim * sizeof(int32_t)) == 0
                          ? lim
                          : std::mismatch(c.tok.data(), c.tok.data() + lim, tok + pos).first - c.tok.data();
    visit(it->second, k);
    pos += k;
    if (k < len) break;
    cur = it->second;
  }
  return pos;
}

int32_t new_node(rc_radix& t) {
  if (!t.dead_ids.empty()) {
    int32_t id = t.dead_ids.back();
    t.dead_ids.pop_back();
    const uint32_t g = t.nodes[id].gen;
    t.nodes[id] = Node();
    t.nodes[id].gen = g;
    return id;
  }
  t.nodes.emplace_back();
  return (int32_t)t.nodes.size() - 1;
}

// Split node c so that its first k tokens become a new parent node.  Returns the new node.
int32_t split(rc_radix& t, int32_t c, int64_t k) {
  int32_t u = new_node(t);  // may reallocate: index only from here on
  Node& cn = t.nodes[c];
  Node& un = t.nodes[u];
  un.parent = cn.parent;
  un.start = cn.start;
  un.tok.assign(cn.tok.begin(), cn.tok.begin() + k);
  un.slot.assign(cn.slot.begin(), cn.slot.begin() + k);
  un.last_use = cn.last_use;
  un.lock = cn.lock;
  cn.tok.erase(cn.tok.begin(), cn.tok.begin() + k);
  cn.slot.erase(cn.slot.begin(), cn.slot.begin() + k);
  cn.start += k;
  cn.parent = u;
  un.kids[cn.tok[0]] = c;
  t.nodes[un.parent].kids[un.tok[0]] = u;
  t.st.splits++;
  t.st.nodes++;
  return u;
}

bool slot_ok(const rc_radix& t, int32_t s) { return s >= 0 && s < t.pool; }

// A batch of token lists in CSR form: request b owns tokens[tok_off[b] ..
// tok_off[b+1]); with tok_len only its first tok_len[b] tokens are used.
rc_status check_lens(int32_t batch, const int64_t* tok_off, const int64_t* tok_len) {
  for (int32_t b = 0; b < batch; ++b) {
    if (tok_off[b] < 0 || tok_off[b + 1] < tok_off[b]) return fail(RC_ERR_ARG, "tok_off not non-decreasing at %d", b);
    if (tok_len && (tok_len[b] < 0 || tok_len[b] > tok_off[b + 1] - tok_off[b]))
      return fail(RC_ERR_ARG, "tok_len[%d] = %lld outside [0, %lld]", b, (long long)tok_len[b], (long long)(tok_off[b + 1] - tok_off[b]));
  }
  return RC_OK;
}

// Do two requests of the batch name the same table row?
bool rows_repeat(int32_t batch, const int32_t* rows) {
  std::vector<int32_t> v(rows, rows + batch);
  std::sort(v.begin(), v.end());
  return std::adjacent_find(v.begin(), v.end()) != v.end();
}

// A batch in the tree's units: the tokens themselves (unpaged tree), or page
// symbols (paged tree; see units_of).
struct Units {
  const int32_t* data = nullptr;  // request b's units start at data + off[b]
  const int64_t* off = nullptr;
  std::vector<int64_t> n;         // and number n[b]
  std::vector<int32_t> sym;       // storage of a paged batch
  std::vector<int64_t> own_off;
  std::vector<int32_t> created;   // symbols this conversion added to the dictionary
  int64_t len(int32_t b) const { return n[b]; }
  const int32_t* at(int32_t b) const { return data + off[b]; }
};

// f(b) for b in [0, n), on several host threads when the batch holds enough
// tokens to pay for them (f must only read shared state, or write to b's own
// outputs).  Requests are dealt in interleaved order so that long and short
// ones mix across threads.
template <class F>
void for_requests(int32_t n, int64_t tokens, F&& f) {
  constexpr int64_t kTokensPerThread = 1 << 19;
  const unsigned hw = std::max(1u, std::thread::hardware_concurrency());
  const int32_t nt = (int32_t)std::min<int64_t>({(int64_t)hw, 8, (int64_t)n, tokens / kTokensPerThread});
  if (nt <= 1) {
    for (int32_t b = 0; b < n; ++b) f(b);
    return;
  }
  std::vector<std::thread> pool;
  try {
    for (int32_t i = 1; i < nt; ++i)
      pool.emplace_back([&, i] {
        for (int32_t b = i; b < n; b += nt) f(b);
      });
  } catch (const std::system_error&) {  // no threads to spare: the caller's thread does the rest
  }
  const int32_t started = (int32_t)pool.size() + 1;
  for (int32_t i = started; i < nt; ++i)
    for (int32_t b = i; b < n; b += nt) f(b);
  for (int32_t b = 0; b < n; b += nt) f(b);
  for (auto& th : pool) th.join();
}

// The symbols of the stored prefix of a request's n whole pages, appended to
// out; returns their number.  It follows the tree as walk() does, but looks a
// page up in the dictionary only to pick the child edge at a node and
// compares the rest of an edge page by page with the dictionary's copies.
int64_t stored_pages(const rc_radix& t, const int32_t* tok, int64_t n, std::vector<int32_t>& out);

// A batch in the tree's units, request b cut to its first len(b) tokens.
// Unpaged: the tokens themselves.  Paged: the symbols of the request's whole
// pages as far as the tree stores them (a lookup needs no more: the stored
// prefix is all that a walk can match); with create, the remaining whole
// pages follow, added to the dictionary where new (listed in created).
template <class LenF>
Units units_of(rc_radix& t, int32_t batch, const int32_t* tokens, const int64_t* tok_off, LenF&& len, bool create) {
  Units u;
  u.n.resize(batch);
  if (t.page == 1) {
    for (int32_t b = 0; b < batch; ++b) u.n[b] = len(b);
    u.data = tokens;
    u.off = tok_off;
    return u;
  }
  const int64_t ps = t.page;
  std::vector<std::vector<int32_t>> per(batch);
  int64_t total = 0;
  for (int32_t b = 0; b < batch; ++b) {
    per[b].reserve((size_t)(len(b) / ps));  // no allocation on the worker threads
    total += len(b);
  }
  if (!create) {
    for_requests(batch, total, [&](int32_t b) {
      if (len(b) >= ps) stored_pages(t, tokens + tok_off[b], len(b) / ps, per[b]);
    });
  } else {
    for (int32_t b = 0; b < batch; ++b) {
      const int64_t np = len(b) / ps;
      if (np == 0) continue;
      const int32_t* src = tokens + tok_off[b];
      for (int64_t i = stored_pages(t, src, np, per[b]); i < np; ++i) {
        bool fresh = false;
        const int32_t s = t.dict.intern(src + i * ps, &fresh);
        if (fresh) u.created.push_back(s);
        per[b].push_back(s);
      }
    }
  }
  u.own_off.assign(batch + 1, 0);
  for (int32_t b = 0; b < batch; ++b) u.own_off[b + 1] = u.own_off[b] + (int64_t)per[b].size();
  u.sym.resize((size_t)u.own_off[batch]);
  for (int32_t b = 0; b < batch; ++b) {
    std::copy(per[b].begin(), per[b].end(), u.sym.begin() + u.own_off[b]);
    u.n[b] = (int64_t)per[b].size();
  }
  u.data = u.sym.data();
  u.off = u.own_off.data();
  return u;
}

int64_t stored_pages(const rc_radix& t, const int32_t* tok, int64_t n, std::vector<int32_t>& out) {
  const int64_t ps = t.page;
  int32_t cur = 0;
  int64_t pos = 0;
  while (pos < n) {
    const int32_t s = t.dict.find(tok + pos * ps);
    if (s < 0) break;
    auto it = t.nodes[cur].kids.find(s);
    if (it == t.nodes[cur].kids.end()) break;
    const Node& c = t.nodes[it->second];
    const int64_t len = (int64_t)c.tok.size();
    const int64_t lim = std::min(len, n - pos);
    out.push_back(s);
    int64_t k = 1;
    while (k < lim && t.dict.same(c.tok[k], tok + (pos + k) * ps)) out.push_back(c.tok[k++]);
    pos += k;
    if (k < len) break;
    cur = it->second;
  }
  return pos;
}

// Locks.  A lock pins the path from the root to one node (the deepest node
// holding a locked token): that node and its ancestors count the lock and are
// not evicted while it is held.  When a pinned edge is split later, both parts
// keep the count (split copies it to the new upper part), so the pinned token
// positions never change.  A handle is the node id in the low 32 bits and the
// node's generation above them; 0 pins nothing.
int64_t handle_of(const rc_radix& t, int32_t id) {
  return id == 0 ? 0 : (int64_t)(((uint64_t)t.nodes[id].gen << 32) | (uint32_t)id);
}

void pin(rc_radix& t, int32_t id, int32_t delta) {
  for (; id > 0; id = t.nodes[id].parent) t.nodes[id].lock += delta;
}

bool evictable(const rc_radix& t, int32_t id) {
  const Node& nd = t.nodes[id];
  return id > 0 && nd.alive && nd.kids.empty() && nd.lock == 0;
}

// LRU eviction (SGLang summary, RadixAttention bullet and steps 5, 8 and 9 of
// the nine-step example: the least recently used nodes go when memory runs
// short): repeatedly remove the unpinned leaf with the oldest last use (ties:
// the lower first slot), returning its slots, in position order, to the back
// of the free list; a parent left without children becomes a candidate.
// Stops once `want` slots are freed or nothing is evictable.  Returns the
// number freed (whole edges, so possibly more than `want`).
int64_t evict_lru(rc_radix& t, int64_t want) {
  using Key = std::tuple<int64_t, int32_t, int32_t>;  // last use, first slot, node
  std::priority_queue<Key, std::vector<Key>, std::greater<Key>> heap;
  auto key = [&](int32_t id) { return Key(t.nodes[id].last_use, t.nodes[id].slot[0], id); };
  int64_t got = 0;
  if (want <= 0) return 0;
  for (int32_t id = 1; id < (int32_t)t.nodes.size(); ++id)
    if (evictable(t, id)) heap.push(key(id));
  while (got < want && !heap.empty()) {
    const int32_t id = std::get<2>(heap.top());
    heap.pop();
    Node& nd = t.nodes[id];
    const int32_t par = nd.parent;
    const int64_t len = (int64_t)nd.tok.size();
    t.nodes[par].kids.erase(nd.tok[0]);
    if (t.page > 1)
      for (int32_t s : nd.tok) t.dict.release(s);
    for (int32_t s : nd.slot) {
      t.in_tree[s] = 0;
      t.is_free[s] = 1;
      t.free_q.push_back(s);
    }
    got += len;
    t.st.evicted_tokens += len;
    t.st.evicted_nodes++;
    t.st.cached_tokens -= len;
    t.st.nodes--;
    nd.alive = false;
    nd.gen++;
    std::vector<int32_t>().swap(nd.tok);
    std::vector<int32_t>().swap(nd.slot);
    nd.kids.clear();
    t.dead_ids.push_back(id);
    if (evictable(t, par)) heap.push(key(par));
  }
  return got;
}

}  // namespace

extern "C" {

rc_status rc_radix_create(int64_t pool_slots, const int32_t* free_order, rc_radix** out) {
  if (!out) return fail(RC_ERR_ARG, "out is NULL");
  if (pool_slots < 0 || pool_slots > INT32_MAX) return fail(RC_ERR_RANGE, "pool_slots %lld out of range", (long long)pool_slots);
  rc_radix* t = nullptr;
  try {
    t = new rc_radix();
    t->pool = pool_slots;
    t->is_free.assign(pool_slots, 0);
    t->in_tree.assign(pool_slots, 0);
    if (free_order) {
      for (int64_t i = 0; i < pool_slots; ++i) {
        int32_t s = free_order[i];
        if (s < 0 || s >= pool_slots || t->is_free[s]) {
          delete t;
          return fail(RC_ERR_ARG, "free_order is not a permutation of [0, %lld) (entry %lld = %d)", (long long)pool_slots, (long long)i, s);
        }
        t->is_free[s] = 1;
        t->free_q.push_back(s);
      }
    } else {
      for (int64_t i = 0; i < pool_slots; ++i) {
        t->is_free[i] = 1;
        t->free_q.push_back((int32_t)i);
      }
    }
    t->nodes.emplace_back();  // root
    t->st.pool_slots = pool_slots;
  } catch (const std::bad_alloc&) {
    delete t;
    return fail(RC_ERR_NOMEM, "host allocation failed");
  }
  *out = t;
  return RC_OK;
}

rc_status rc_radix_create_paged(int64_t n_pages, int32_t page_size, const int32_t* free_order, rc_radix** out) {
  if (page_size < 1 || page_size > 1024 || (page_size & (page_size - 1)))
    return fail(RC_ERR_ARG, "page_size %d is not a power of two up to 1024", page_size);
  rc_status st = rc_radix_create(n_pages, free_order, out);
  if (st != RC_OK) return st;
  (*out)->page = page_size;
  (*out)->dict.ps = page_size;
  return RC_OK;
}

void rc_radix_destroy(rc_radix* tree) { delete tree; }

rc_status rc_radix_match(rc_radix* t, const int32_t* tokens, int64_t n, int32_t* out_slots, int64_t* matched) {
  if (!t || !matched || n < 0 || (n > 0 && !tokens)) return fail(RC_ERR_ARG, "bad argument to rc_radix_match");
  const int64_t off[2] = {0, n};
  const Units u = units_of(*t, 1, tokens, off, [&](int32_t) { return n; }, false);
  std::vector<int32_t> touched;
  int64_t w = 0;
  const int64_t cap = n > 0 ? (n - 1) / t->page : 0;  // at least one token is computed
  walk(*t, u.at(0), u.len(0), [&](int32_t id, int64_t k) {
    touched.push_back(id);
    const Node& c = t->nodes[id];
    for (int64_t i = 0; i < k && w < cap; ++i, ++w)
      if (out_slots) out_slots[w] = c.slot[i];
  });
  *matched = w * t->page;
  int64_t now = ++t->clock;
  for (int32_t id : touched) t->nodes[id].last_use = now;
  t->st.matches++;
  t->st.matched_tokens += w;
  return RC_OK;
}

rc_status rc_radix_alloc(rc_radix* t, int64_t n, int32_t* out_slots) {
  if (!t || n < 0 || (n > 0 && !out_slots)) return fail(RC_ERR_ARG, "bad argument to rc_radix_alloc");
  if (n > (int64_t)t->free_q.size())
    return fail(RC_ERR_NOMEM, "need %lld slots, %zu free", (long long)n, t->free_q.size());
  for (int64_t i = 0; i < n; ++i) {
    int32_t s = t->free_q.front();
    t->free_q.pop_front();
    t->is_free[s] = 0;
    out_slots[i] = s;
  }
  return RC_OK;
}

rc_status rc_radix_free(rc_radix* t, const int32_t* slots, int64_t n) {
  if (!t || n < 0 || (n > 0 && !slots)) return fail(RC_ERR_ARG, "bad argument to rc_radix_free");
  std::vector<uint8_t> seen;
  for (int64_t i = 0; i < n; ++i) {
    int32_t s = slots[i];
    if (!slot_ok(*t, s)) return fail(RC_ERR_ARG, "slot %d out of range", s);
    if (t->is_free[s]) return fail(RC_ERR_ARG, "slot %d is already free", s);
    if (t->in_tree[s]) return fail(RC_ERR_ARG, "slot %d is held by the tree", s);
  }
  // repeated entries
  {
    std::vector<int32_t> v(slots, slots + n);
    std::sort(v.begin(), v.end());
    if (std::adjacent_find(v.begin(), v.end()) != v.end()) return fail(RC_ERR_ARG, "repeated slot in free list");
  }
  for (int64_t i = 0; i < n; ++i) {
    t->is_free[slots[i]] = 1;
    t->free_q.push_back(slots[i]);
  }
  return RC_OK;
}

// Insert n units (tokens, or page symbols) with their slots (or page ids).
static rc_status insert_units(rc_radix* t, const int32_t* tokens, int32_t* slots, int64_t n, int64_t* n_new) {
  // pass 1 (read only): how much is stored already, and validate every slot
  std::vector<int32_t> stored;
  const int64_t m = walk(*t, tokens, n, [&](int32_t id, int64_t k) {
    const Node& c = t->nodes[id];
    stored.insert(stored.end(), c.slot.begin(), c.slot.begin() + k);
  });
  {
    std::vector<int32_t> mine;
    for (int64_t i = 0; i < n; ++i) {
      int32_t s = slots[i];
      if (!slot_ok(*t, s)) return fail(RC_ERR_ARG, "slot %d (position %lld) out of range", s, (long long)i);
      if (i < m && s == stored[i]) continue;  // the caller already uses the stored slot
      if (t->is_free[s]) return fail(RC_ERR_ARG, "slot %d (position %lld) is free, not allocated", s, (long long)i);
      if (t->in_tree[s]) return fail(RC_ERR_ARG, "slot %d (position %lld) already belongs to the tree", s, (long long)i);
      mine.push_back(s);
    }
    std::sort(mine.begin(), mine.end());
    if (std::adjacent_find(mine.begin(), mine.end()) != mine.end()) return fail(RC_ERR_ARG, "repeated slot in insert");
  }
  try {
    // pass 2: mutate
    int32_t cur = 0;
    int64_t pos = 0;
    const int64_t now = ++t->clock;
    while (pos < n) {
      auto it = t->nodes[cur].kids.find(tokens[pos]);
      if (it == t->nodes[cur].kids.end()) {
        int32_t id = new_node(*t);
        Node& nn = t->nodes[id];
        nn.parent = cur;
        nn.start = pos;
        nn.tok.assign(tokens + pos, tokens + n);
        nn.slot.assign(slots + pos, slots + n);
        nn.last_use = now;
        for (int64_t i = pos; i < n; ++i) t->in_tree[slots[i]] = 1;
        if (t->page > 1)
          for (int64_t i = pos; i < n; ++i) t->dict.acquire(tokens[i]);
        t->nodes[cur].kids[tokens[pos]] = id;
        t->st.nodes++;
        t->st.cached_tokens += n - pos;
        t->st.inserted_tokens += n - pos;
        pos = n;
        break;
      }
      int32_t c = it->second;
      const int64_t len = (int64_t)t->nodes[c].tok.size();
      const int64_t lim = std::min(len, n - pos);
      int64_t k = 0;
      while (k < lim && t->nodes[c].tok[k] == tokens[pos + k]) ++k;
      for (int64_t i = 0; i < k; ++i) {
        int32_t have = t->nodes[c].slot[i];
        if (slots[pos + i] != have) {
          t->is_free[slots[pos + i]] = 1;
          t->free_q.push_back(slots[pos + i]);
          t->st.duplicate_slots++;
          slots[pos + i] = have;
        }
      }
      pos += k;
      if (k < len) {
        if (pos < n) {
          // the walk used the upper part only; the lower part keeps its time
          int32_t u = split(*t, c, k);
          t->nodes[u].last_use = now;
          cur = u;
          continue;  // next lookup adds the new leaf under u
        }
        t->nodes[c].last_use = now;
        break;  // the sequence ends inside this edge: nothing new to store
      }
      t->nodes[c].last_use = now;
      cur = c;
    }
    if (n_new) *n_new = n - m;
  } catch (const std::bad_alloc&) {
    return fail(RC_ERR_INTERNAL, "host allocation failed during insert (tree may be inconsistent)");
  }
  return RC_OK;
}

rc_status rc_radix_insert(rc_radix* t, const int32_t* tokens, int32_t* slots, int64_t n, int64_t* n_new) {
  if (!t || n < 0 || (n > 0 && (!tokens || !slots))) return fail(RC_ERR_ARG, "bad argument to rc_radix_insert");
  if (t->page == 1) return insert_units(t, tokens, slots, n, n_new);
  try {
    const int64_t off[2] = {0, n};
    const Units u = units_of(*t, 1, tokens, off, [&](int32_t) { return n; }, true);  // whole pages only
    rc_status st = insert_units(t, u.at(0), slots, u.len(0), n_new);
    for (int32_t s : u.created)  // pages a failed insert did not store
      if (t->dict.refs[s] == 0) t->dict.remove(s);
    return st;
  } catch (const std::bad_alloc&) {
    return fail(RC_ERR_NOMEM, "host allocation failed");
  }
}

rc_status rc_radix_insert_rows(rc_radix* t, int32_t batch, const int32_t* tokens, const int64_t* tok_off,
                               const int64_t* tok_len, const int32_t* rows, int32_t* table, int32_t table_rows,
                               int64_t stride, int32_t* changed) {
  if (!t || batch < 0 || stride <= 0) return fail(RC_ERR_ARG, "bad argument to rc_radix_insert_rows");
  if (batch > 0 && (!tok_off || !rows || !table)) return fail(RC_ERR_ARG, "NULL array in rc_radix_insert_rows");
  if (rc_status st = check_lens(batch, tok_off, tok_len); st != RC_OK) return st;
  auto len_of = [&](int32_t b) { return tok_len ? tok_len[b] : tok_off[b + 1] - tok_off[b]; };
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t n = len_of(b);
    if (rows[b] < 0 || rows[b] >= table_rows) return fail(RC_ERR_RANGE, "row %d of request %d outside [0, %d)", rows[b], b, table_rows);
    if (n / t->page > stride) return fail(RC_ERR_RANGE, "request %d has %lld tokens, stride is %lld", b, (long long)n, (long long)stride);
  }
  std::vector<int32_t> before;
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t n = len_of(b), ne = n / t->page;  // table entries inserted: one per token, or per whole page
    int32_t* row = table + (int64_t)rows[b] * stride;
    if (changed) before.assign(row, row + ne);
    rc_status st = rc_radix_insert(t, tokens + tok_off[b], row, n, nullptr);
    if (st != RC_OK) return st;
    if (changed) changed[b] = !std::equal(before.begin(), before.end(), row);
  }
  return RC_OK;
}

rc_status rc_radix_emit_rows(rc_radix* t, int32_t batch, const int32_t* tokens, const int64_t* tok_off,
                             int32_t reserve, const int32_t* rows, int32_t* table, int32_t table_rows,
                             int64_t stride, int32_t* prefix_lens, int32_t* extend_lens, int32_t flags,
                             int64_t* handles, int64_t* first_changed, int64_t* row_entries, int32_t* new_slots) {
  if (!t || batch < 0 || reserve < 0 || stride <= 0 || table_rows < 0) return fail(RC_ERR_ARG, "bad argument to rc_radix_emit_rows");
  if (batch > 0 && (!tok_off || !rows || !table || !prefix_lens || !extend_lens)) return fail(RC_ERR_ARG, "NULL array in rc_radix_emit_rows");
  if (flags & ~(RC_EMIT_EVICT | RC_EMIT_FULL_MATCH)) return fail(RC_ERR_ARG, "unknown emit_rows flags 0x%x", (unsigned)flags);
  if (rc_status st = check_lens(batch, tok_off, nullptr); st != RC_OK) return st;
  const bool evict = flags & RC_EMIT_EVICT;
  // In units of the tree: tokens, or pages.  Request b gets entries for its
  // n + reserve tokens (ceil((n + reserve) / page) pages); at most (n - 1) /
  // page units of its prefix are reused, so at least one token is computed
  // (with RC_EMIT_FULL_MATCH all n / page whole units of it).
  const int64_t pg = t->page;
  const bool full = flags & RC_EMIT_FULL_MATCH;
  auto entries = [&](int32_t b) { return (tok_off[b + 1] - tok_off[b] + reserve + pg - 1) / pg; };
  auto cap_of = [&](int32_t b) {
    const int64_t n = tok_off[b + 1] - tok_off[b];
    return full ? n / pg : (n > 0 ? (n - 1) / pg : 0);
  };
  // pass 1 (read only): matched length and the edges entered, per request
  struct Visit { int32_t node; int64_t k; };
  std::vector<int64_t> P(batch);
  std::vector<std::vector<Visit>> visits(batch);
  int64_t need = 0;
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t n = tok_off[b + 1] - tok_off[b];
    if (n > 0 && !tokens) return fail(RC_ERR_ARG, "tokens is NULL");
    if (rows[b] < 0 || rows[b] >= table_rows) return fail(RC_ERR_RANGE, "row %d of request %d outside [0, %d)", rows[b], b, table_rows);
    if (entries(b) > stride) return fail(RC_ERR_RANGE, "request %d needs %lld table entries, stride is %lld", b, (long long)entries(b), (long long)stride);
  }
  const Units u = units_of(*t, batch, tokens, tok_off, [&](int32_t b) { return tok_off[b + 1] - tok_off[b]; }, false);
  const int64_t total = batch > 0 ? tok_off[batch] - tok_off[0] : 0;
  for_requests(batch, total, [&](int32_t b) {
    const int64_t m = walk(*t, u.at(b), u.len(b), [&](int32_t id, int64_t k) { visits[b].push_back({id, k}); });
    P[b] = std::min(m, cap_of(b));
  });
  for (int32_t b = 0; b < batch; ++b) need += entries(b) - P[b];
  if (rows_repeat(batch, rows)) return fail(RC_ERR_ARG, "two requests of the batch share a table row");
  const int64_t free0 = (int64_t)t->free_q.size();
  if (need > free0 && !evict)
    return fail(RC_ERR_NOMEM, "batch needs %lld slots, %zu free", (long long)need, t->free_q.size());
  // pin the matched prefixes: for the caller (handles), and while evicting,
  // so that eviction never takes what the batch has matched
  const bool pinning = handles || need > free0;
  std::vector<int32_t> end(batch, 0);
  if (pinning)
    for (int32_t b = 0; b < batch; ++b) {
      int64_t w = 0;
      for (const Visit& v : visits[b]) {
        if (w >= P[b]) break;
        end[b] = v.node;
        w += v.k;
      }
      pin(*t, end[b], +1);
    }
  const int64_t now = ++t->clock;
  for (int32_t b = 0; b < batch; ++b)
    for (const Visit& v : visits[b]) t->nodes[v.node].last_use = now;
  if (need > free0) {
    try {
      evict_lru(*t, need - free0);
    } catch (const std::bad_alloc&) {
      for (int32_t b = 0; b < batch; ++b) pin(*t, end[b], -1);
      return fail(RC_ERR_INTERNAL, "host allocation failed during eviction");
    }
    if (need > (int64_t)t->free_q.size()) {
      for (int32_t b = 0; b < batch; ++b) pin(*t, end[b], -1);
      return fail(RC_ERR_NOMEM, "batch needs %lld slots, %zu free after eviction", (long long)need, t->free_q.size());
    }
  }
  // pass 2: allocate in request order, then copy the matched prefixes' slots
  // (first_changed: the first entry whose value changes, per request)
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t n = tok_off[b + 1] - tok_off[b];
    int32_t* row = table + (int64_t)rows[b] * stride;
    int64_t fc = entries(b);
    for (int64_t i = P[b]; i < entries(b); ++i) {
      int32_t s = t->free_q.front();
      t->free_q.pop_front();
      t->is_free[s] = 0;
      if (row[i] != s && fc == entries(b)) fc = i;
      row[i] = s;
    }
    if (first_changed) first_changed[b] = fc;
    if (row_entries) row_entries[b] = entries(b);
    prefix_lens[b] = (int32_t)(P[b] * pg);
    extend_lens[b] = (int32_t)(n - P[b] * pg);
    t->st.matches++;
    t->st.matched_tokens += P[b];
  }
  for_requests(batch, total, [&](int32_t b) {
    int32_t* row = table + (int64_t)rows[b] * stride;
    int64_t w = 0;
    for (const Visit& v : visits[b]) {
      if (w >= P[b]) break;
      const Node& c = t->nodes[v.node];
      const int64_t k = std::min(v.k, P[b] - w);
      if (first_changed && w < first_changed[b] &&
          std::memcmp(row + w, c.slot.data(), (size_t)k * sizeof(int32_t)) != 0)
        first_changed[b] = std::min(first_changed[b],
                                    w + (std::mismatch(row + w, row + w + k, c.slot.data()).first - (row + w)));
      std::memcpy(row + w, c.slot.data(), (size_t)k * sizeof(int32_t));
      w += k;
    }
  });
  for (int32_t b = 0; b < batch; ++b) {
    if (handles)
      handles[b] = handle_of(*t, end[b]);
    else if (pinning)
      pin(*t, end[b], -1);
  }
  // pool slots of the new tokens, request after request: position p of a row
  // is slot row[p] (unpaged) or row[p / page] * page + p % page
  if (new_slots) {
    int64_t o = 0;
    for (int32_t b = 0; b < batch; ++b) {
      const int32_t* row = table + (int64_t)rows[b] * stride;
      for (int64_t p = prefix_lens[b]; p < prefix_lens[b] + extend_lens[b]; ++p)
        new_slots[o++] = (int32_t)((int64_t)row[p / pg] * pg + p % pg);
    }
  }
  return RC_OK;
}

rc_status rc_radix_free_rows(rc_radix* t, int32_t batch, const int32_t* rows, const int32_t* table, int32_t table_rows,
                             int64_t stride, const int64_t* keep_lens, const int64_t* row_entries) {
  if (!t || batch < 0 || stride <= 0 || table_rows < 0) return fail(RC_ERR_ARG, "bad argument to rc_radix_free_rows");
  if (batch > 0 && (!rows || !table || !keep_lens || !row_entries)) return fail(RC_ERR_ARG, "NULL array in rc_radix_free_rows");
  // units [keep / page, entries) of each row: the request's own positions
  // from its first position not kept (a partly kept page is not in the tree)
  std::vector<int32_t> units;
  for (int32_t b = 0; b < batch; ++b) {
    if (rows[b] < 0 || rows[b] >= table_rows) return fail(RC_ERR_RANGE, "row %d of request %d outside [0, %d)", rows[b], b, table_rows);
    if (keep_lens[b] < 0 || row_entries[b] < 0 || row_entries[b] > stride)
      return fail(RC_ERR_RANGE, "request %d: kept %lld tokens, %lld row entries (stride %lld)", b, (long long)keep_lens[b],
                  (long long)row_entries[b], (long long)stride);
    const int32_t* row = table + (int64_t)rows[b] * stride;
    for (int64_t i = keep_lens[b] / t->page; i < row_entries[b]; ++i) units.push_back(row[i]);
  }
  return rc_radix_free(t, units.data(), (int64_t)units.size());
}

rc_status rc_decode_steps(const int32_t* table, int32_t table_rows, int64_t stride, int32_t page_size, int32_t batch,
                          const int32_t* rows, const int64_t* row_entries, const int32_t* base_lens, int32_t n_steps,
                          int32_t* slots, int32_t* seq_lens) {
  if (batch < 0 || n_steps < 0 || stride <= 0 || table_rows < 0) return fail(RC_ERR_ARG, "bad argument to rc_decode_steps");
  if (page_size < 1 || page_size > 1024 || (page_size & (page_size - 1)))
    return fail(RC_ERR_SHAPE, "page_size %d is not a power of two up to 1024", page_size);
  if (batch > 0 && n_steps > 0 && (!table || !base_lens || !slots || !seq_lens)) return fail(RC_ERR_ARG, "NULL array in rc_decode_steps");
  for (int32_t b = 0; b < batch && n_steps > 0; ++b) {
    const int32_t r = rows ? rows[b] : b;
    if (r < 0 || r >= table_rows) return fail(RC_ERR_RANGE, "row %d of request %d outside [0, %d)", r, b, table_rows);
    const int64_t ent = row_entries ? row_entries[b] : stride;
    if (base_lens[b] < 0 || ent > stride || (int64_t)base_lens[b] + n_steps > ent * page_size)
      return fail(RC_ERR_RANGE, "request %d: decode positions [%d, %lld) past its %lld row entries", b, base_lens[b],
                  (long long)base_lens[b] + n_steps, (long long)ent);
    const int32_t* row = table + (int64_t)r * stride;
    for (int32_t s = 0; s < n_steps; ++s) {
      const int64_t p = (int64_t)base_lens[b] + s;
      if (row[p / page_size] < 0) return fail(RC_ERR_RANGE, "request %d: position %lld of row %d holds no slot", b, (long long)p, r);
    }
  }
  for (int32_t b = 0; b < batch; ++b) {
    const int32_t* row = table + (int64_t)(rows ? rows[b] : b) * stride;
    for (int32_t s = 0; s < n_steps; ++s) {
      const int64_t p = (int64_t)base_lens[b] + s;  // the token of step s sits at position p ...
      slots[(int64_t)s * batch + b] = (int32_t)((int64_t)row[p / page_size] * page_size + p % page_size);
      seq_lens[(int64_t)s * batch + b] = (int32_t)(p + 1);  // ... and attends over positions [0, p]
    }
  }
  return RC_OK;
}

rc_status rc_radix_fork(rc_radix* t, const int32_t* tokens, const int32_t* parent_slots, int64_t n, int32_t n_children,
                        const int32_t* child_rows, int32_t* table, int32_t table_rows, int64_t stride) {
  if (!t || n < 0 || n_children < 0 || stride <= 0) return fail(RC_ERR_ARG, "bad argument to rc_radix_fork");
  const int64_t ne = n / t->page;  // table entries shared: one per token, or per whole page
  if (ne > stride) return fail(RC_ERR_RANGE, "prefix of %lld tokens exceeds stride %lld", (long long)n, (long long)stride);
  if (n_children > 0 && (!child_rows || !table)) return fail(RC_ERR_ARG, "NULL child rows or table");
  for (int32_t c = 0; c < n_children; ++c)
    if (child_rows[c] < 0 || child_rows[c] >= table_rows) return fail(RC_ERR_RANGE, "child row %d outside [0, %d)", child_rows[c], table_rows);
  std::vector<int32_t> s(parent_slots, parent_slots + ne);
  rc_status st = rc_radix_insert(t, tokens, s.data(), n, nullptr);
  if (st != RC_OK) return st;
  for (int32_t c = 0; c < n_children; ++c) std::copy(s.begin(), s.end(), table + (int64_t)child_rows[c] * stride);
  return RC_OK;
}

rc_status rc_radix_lock(rc_radix* t, int32_t batch, const int32_t* tokens, const int64_t* tok_off,
                        const int64_t* tok_len, int64_t* handles, int64_t* locked) {
  if (!t || batch < 0) return fail(RC_ERR_ARG, "bad argument to rc_radix_lock");
  if (batch > 0 && (!tok_off || !handles)) return fail(RC_ERR_ARG, "NULL array in rc_radix_lock");
  if (rc_status st = check_lens(batch, tok_off, tok_len); st != RC_OK) return st;
  auto len_of = [&](int32_t b) { return tok_len ? tok_len[b] : tok_off[b + 1] - tok_off[b]; };
  int64_t total = 0;
  for (int32_t b = 0; b < batch; ++b) {
    if (len_of(b) > 0 && !tokens) return fail(RC_ERR_ARG, "tokens is NULL");
    total += len_of(b);
  }
  std::vector<int32_t> end(batch, 0);
  std::vector<int64_t> m(batch, 0);
  const Units u = units_of(*t, batch, tokens, tok_off, len_of, false);
  for_requests(batch, total, [&](int32_t b) {
    int32_t last = 0;
    m[b] = walk(*t, u.at(b), u.len(b), [&](int32_t id, int64_t) { last = id; });
    end[b] = last;
  });
  for (int32_t b = 0; b < batch; ++b) {
    pin(*t, end[b], +1);
    handles[b] = handle_of(*t, end[b]);
    if (locked) locked[b] = m[b] * t->page;
  }
  return RC_OK;
}

rc_status rc_radix_unlock(rc_radix* t, const int64_t* handles, int32_t n) {
  if (!t || n < 0 || (n > 0 && !handles)) return fail(RC_ERR_ARG, "bad argument to rc_radix_unlock");
  // validate every handle and that the counts it releases are held, then release
  std::unordered_map<int32_t, int32_t> dec;
  for (int32_t i = 0; i < n; ++i) {
    const int64_t h = handles[i];
    if (h == 0) continue;
    const int64_t id = (int64_t)(uint32_t)((uint64_t)h & 0xffffffffu);
    const uint32_t gen = (uint32_t)((uint64_t)h >> 32);
    if (id <= 0 || id >= (int64_t)t->nodes.size() || !t->nodes[id].alive || t->nodes[id].gen != gen)
      return fail(RC_ERR_ARG, "handle %d (0x%llx) is not a held lock", i, (unsigned long long)h);
    for (int32_t x = (int32_t)id; x > 0; x = t->nodes[x].parent) dec[x]++;
  }
  for (const auto& [x, c] : dec)
    if (t->nodes[x].lock < c) return fail(RC_ERR_ARG, "more unlocks than locks on a node");
  for (const auto& [x, c] : dec) t->nodes[x].lock -= c;
  return RC_OK;
}

rc_status rc_radix_evict(rc_radix* t, int64_t n_slots, int64_t* freed) {
  if (!t) return fail(RC_ERR_ARG, "bad argument to rc_radix_evict");
  int64_t got = 0;
  try {
    got = evict_lru(*t, n_slots);
  } catch (const std::bad_alloc&) {
    return fail(RC_ERR_INTERNAL, "host allocation failed during eviction");
  }
  if (freed) *freed = got;
  return RC_OK;
}

rc_status rc_radix_stats_get(const rc_radix* t, rc_radix_stats* out) {
  if (!t || !out) return fail(RC_ERR_ARG, "NULL argument");
  *out = t->st;
  out->free_slots = (int64_t)t->free_q.size();
  out->page_symbols = t->dict.live;
  out->locked_tokens = 0;
  for (size_t id = 1; id < t->nodes.size(); ++id)
    if (t->nodes[id].alive && t->nodes[id].lock > 0) out->locked_tokens += (int64_t)t->nodes[id].tok.size();
  return RC_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Decode planners.
//
// A work item is a range of positions read through one table row, computed
// for every member request.  Ranges shared by several requests come from tree
// nodes; all requests passing through a node read its slots, so the item loads
// that KV once per step for all of them.
// ---------------------------------------------------------------------------
namespace {

struct Range {
  int64_t begin, end;
  std::vector<int32_t> members;
  bool own = false;  // the positions of its one member alone (its items carry RC_PLAN_ITEM_OWN)
};

struct PlanBuilder {
  int32_t batch, group, chunk, max_m;
  const int32_t* rows;
  std::vector<Range> ranges;
  std::vector<std::vector<int32_t>> path;  // per request: range ids in order
  std::vector<int32_t> item_rows;          // built items, 8 ints each
  std::vector<int32_t> members;
  std::vector<int32_t> nsplit;
  int32_t shared_items = 0;
  int32_t narrow_begin = 0;
  int32_t narrow_first = 0;
  int64_t unique_pos = 0;

  int32_t row_of(int32_t b) const { return rows ? rows[b] : b; }

  // A range of n positions is cut into the fewest near-equal pieces of at
  // most chunk + chunk/8 positions, so a context a few tokens longer than
  // the chunk leaves no tiny last item: every item pays a fixed start-up cost.
  int64_t piece_len(int64_t n) const {
    if (n <= 0) return 1;
    const int64_t cap = (int64_t)chunk + chunk / 8;
    const int64_t k = (n + cap - 1) / cap;
    return (n + k - 1) / k;
  }

  void build() {
    nsplit.assign(batch, 0);
    // split index of each range: chunks of the ranges before it on any member's path
    std::vector<int32_t> first_split(ranges.size(), -1);
    for (int32_t b = 0; b < batch; ++b) {
      int32_t acc = 0;
      for (int32_t r : path[b]) {
        if (first_split[r] < 0) first_split[r] = acc;
        const int64_t len = ranges[r].end - ranges[r].begin;
        const int64_t pl = piece_len(len);
        acc += (int32_t)(len > 0 ? (len + pl - 1) / pl : 0);
      }
      nsplit[b] = acc;
    }
    // items, longest member lists first (more columns = more compute per item)
    std::vector<int32_t> order(ranges.size());
    for (size_t i = 0; i < order.size(); ++i) order[i] = (int32_t)i;
    std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
      return ranges[a].members.size() > ranges[b].members.size();
    });
    // wide items (members*group > 16) first, then narrow ones; within each
    // class the longest running first (wide: members x positions, narrow:
    // positions), so the last workgroups to start are the short ones
    struct Item { int64_t cost; int32_t v[RC_PLAN_ITEM]; int32_t range, first; };
    std::vector<Item> wide, narrow;
    for (int32_t r : order) {
      const Range& R = ranges[r];
      if (R.end <= R.begin) continue;
      int32_t sp = first_split[r];
      const int64_t pl = piece_len(R.end - R.begin);
      for (int64_t p = R.begin; p < R.end; p += pl, ++sp) {
        const int64_t pe = std::min<int64_t>(p + pl, R.end);
        for (size_t g0 = 0; g0 < R.members.size(); g0 += max_m) {
          const size_t cnt = std::min<size_t>(max_m, R.members.size() - g0);
          const bool is_narrow = (int64_t)cnt * group <= 16;
          // a narrow item's time is its range (one wave streams it; its columns
          // fit one tile whatever their number), a wide item's grows with its members
          const Item it{is_narrow ? pe - p : (int64_t)cnt * (pe - p),
                        {row_of(R.members[g0]), (int32_t)p, (int32_t)pe, sp, 0, (int32_t)cnt, R.own ? RC_PLAN_ITEM_OWN : 0, 0},
                        r, (int32_t)g0};
          (is_narrow ? narrow : wide).push_back(it);
          if (R.members.size() > 1) shared_items++;
        }
      }
    }
    auto by_cost = [](const Item& x, const Item& y) { return x.cost > y.cost; };
    std::stable_sort(wide.begin(), wide.end(), by_cost);
    std::stable_sort(narrow.begin(), narrow.end(), by_cost);
    narrow_begin = (int32_t)wide.size();
    // Which class the launch deals out first: the one holding the item that
    // takes longest, so that no long item starts late.  A narrow item is one
    // wave per kv head and streams its range at roughly half the rate of a
    // wide item's workgroup (four waves, eight in a cascade extend), so its
    // length counts double.
    int64_t long_wide = 0, long_narrow = 0;
    for (const Item& it : wide) long_wide = std::max<int64_t>(long_wide, it.v[2] - it.v[1]);
    for (const Item& it : narrow) long_narrow = std::max<int64_t>(long_narrow, it.v[2] - it.v[1]);
    narrow_first = 2 * long_narrow > long_wide;
    item_rows.reserve((wide.size() + narrow.size()) * RC_PLAN_ITEM);
    for (auto* list : {&wide, &narrow})
      for (Item& it : *list) {
        it.v[4] = (int32_t)members.size();
        const auto& mem = ranges[it.range].members;
        members.insert(members.end(), mem.begin() + it.first, mem.begin() + it.first + it.v[5]);
        item_rows.insert(item_rows.end(), it.v, it.v + RC_PLAN_ITEM);
      }
    for (int32_t r : order)
      if (ranges[r].end > ranges[r].begin) unique_pos += ranges[r].end - ranges[r].begin;
  }

  rc_status emit(int32_t* plan, int64_t cap, rc_plan_info* info, int64_t logical) {
    const int32_t n_items = (int32_t)(item_rows.size() / RC_PLAN_ITEM);
    int32_t max_splits = 0;
    for (int32_t v : nsplit) max_splits = std::max(max_splits, v);
    const int64_t need = RC_PLAN_HEADER + (int64_t)item_rows.size() + (int64_t)members.size() + batch;
    info->n_items = n_items;
    info->n_members = (int32_t)members.size();
    info->max_splits = max_splits;
    info->batch = batch;
    info->group = group;
    info->chunk = chunk;
    info->max_cols = max_m * group;
    info->shared_items = shared_items;
    info->narrow_begin = narrow_begin;
    info->narrow_first = narrow_first;
    info->plan_ints = need;
    info->unique_positions = unique_pos;
    info->logical_positions = logical;
    if (!plan || cap < need) return fail(RC_ERR_RANGE, "plan needs %lld int32, capacity %lld", (long long)need, (long long)cap);
    int32_t hdr[RC_PLAN_HEADER] = {(int32_t)RC_PLAN_MAGIC, n_items, (int32_t)members.size(), max_splits, batch, group, chunk, max_m * group};
    int32_t* w = plan;
    w = std::copy(hdr, hdr + RC_PLAN_HEADER, w);
    w = std::copy(item_rows.begin(), item_rows.end(), w);
    w = std::copy(members.begin(), members.end(), w);
    std::copy(nsplit.begin(), nsplit.end(), w);
    return RC_OK;
  }
};

rc_status plan_args(int32_t batch, const int32_t* max_seq, int32_t group, int32_t chunk, rc_plan_info* info) {
  if (batch < 0 || !info || (batch > 0 && !max_seq)) return fail(RC_ERR_ARG, "bad planner argument");
  if (group < 1 || group > 128) return fail(RC_ERR_SHAPE, "group %d outside [1, 128]", group);
  if (chunk < 1) return fail(RC_ERR_ARG, "chunk must be positive");
  for (int32_t b = 0; b < batch; ++b)
    if (max_seq[b] < 1) return fail(RC_ERR_RANGE, "max_seq_lens[%d] = %d < 1", b, max_seq[b]);
  return RC_OK;
}

}  // namespace

extern "C" rc_status rc_plan_decode_unshared(int32_t batch, const int32_t* rows, const int32_t* max_seq, int32_t group,
                                             int32_t chunk, int32_t* plan, int64_t cap, rc_plan_info* info) {
  rc_status st = plan_args(batch, max_seq, group, chunk, info);
  if (st != RC_OK) return st;
  PlanBuilder pb{batch, group, chunk, std::max(1, RC_DECODE_COLS / group), rows, {}, {}, {}, {}, {}};
  pb.path.resize(batch);
  int64_t logical = 0;
  for (int32_t b = 0; b < batch; ++b) {
    pb.ranges.push_back(Range{0, max_seq[b], {b}, true});
    pb.path[b].push_back((int32_t)pb.ranges.size() - 1);
    logical += max_seq[b];
  }
  pb.build();
  return pb.emit(plan, cap, info, logical);
}

namespace {

struct Visit {
  int32_t node;
  int64_t end;  // absolute position just past the part of the node walked
};

// Shared plan for n_mem members.  Member m walks the tree like request
// req_of[m] did (walks / walked per request), reads its context through table
// row rows_of[m] and has max_seq[m] positions.  Every node range is one item
// whose members are all members passing through it; positions past the last
// shared range up to max_seq[m] are the member's own range.
rc_status plan_from_walks(const rc_radix* t, int32_t n_mem, const std::vector<int32_t>& req_of,
                          const std::vector<std::vector<Visit>>& walks, const std::vector<int64_t>& walked,
                          const std::vector<int32_t>& rows_of, const int32_t* max_seq, int32_t group, int32_t chunk,
                          int32_t max_cols, int32_t* plan, int64_t cap, rc_plan_info* info) {
  std::unordered_map<int32_t, std::vector<std::pair<int64_t, int32_t>>> by_node;  // node -> (end, member)
  for (int32_t m = 0; m < n_mem; ++m) {
    const int32_t r = req_of[m];
    if (max_seq[m] < walked[r]) return fail(RC_ERR_RANGE, "max_seq_lens[%d] = %d shorter than its cached prefix %lld", m, max_seq[m], (long long)walked[r]);
    for (const Visit& v : walks[r]) by_node[v.node].push_back({v.end, m});
  }
  PlanBuilder pb{n_mem, group, chunk, std::max(1, max_cols / group), rows_of.data(), {}, {}, {}, {}, {}};
  pb.path.resize(n_mem);
  // node -> list of (sub-range id, sub-range end); members of a sub-range reach at least its end
  std::unordered_map<int32_t, std::vector<std::pair<int32_t, int64_t>>> subs;
  for (auto& kv : by_node) {
    auto v = kv.second;
    std::sort(v.begin(), v.end());
    int64_t prev = t->nodes[kv.first].start * t->page;
    size_t i = 0;
    auto& out = subs[kv.first];
    while (i < v.size()) {
      const int64_t e = v[i].first;
      if (e > prev) {
        Range R{prev, e, {}};
        for (size_t j = i; j < v.size(); ++j) R.members.push_back(v[j].second);
        std::sort(R.members.begin(), R.members.end());
        pb.ranges.push_back(std::move(R));
        out.push_back({(int32_t)pb.ranges.size() - 1, e});
        prev = e;
      }
      while (i < v.size() && v[i].first == e) ++i;
    }
  }
  const size_t n_node_ranges = pb.ranges.size();
  int64_t logical = 0;
  for (int32_t m = 0; m < n_mem; ++m) {
    logical += max_seq[m];
    // shared part of the path, then everything this member alone reads as one range
    int64_t own_begin = 0;
    bool own = false;
    for (const Visit& v : walks[req_of[m]]) {
      for (auto& sr : subs[v.node]) {
        if (sr.second > v.end) break;
        const Range& R = pb.ranges[sr.first];
        if (R.members.size() > 1) {
          pb.path[m].push_back(sr.first);
          own_begin = R.end;
        } else {
          own = true;
          break;
        }
      }
      if (own) break;
    }
    if (max_seq[m] > own_begin) {
      pb.ranges.push_back(Range{own_begin, max_seq[m], {m}, true});
      pb.path[m].push_back((int32_t)pb.ranges.size() - 1);
    }
  }
  // drop the single-member node ranges: each member's own range covers them
  for (size_t r = 0; r < n_node_ranges; ++r)
    if (pb.ranges[r].members.size() == 1) pb.ranges[r].end = pb.ranges[r].begin;
  pb.build();
  return pb.emit(plan, cap, info, logical);
}

// Walk request b's first len(b) tokens through the tree (several threads
// for large batches).
// Positions are in tokens: a paged tree walks whole pages, page tokens each.
template <class LenF>
void walk_requests(const rc_radix* t, int32_t batch, const int32_t* tokens, const int64_t* tok_off, LenF&& len,
                   std::vector<std::vector<Visit>>& walks, std::vector<int64_t>& walked) {
  walks.assign(batch, {});
  walked.assign(batch, 0);
  int64_t total = 0;
  for (int32_t b = 0; b < batch; ++b) total += len(b);
  const Units u = units_of(const_cast<rc_radix&>(*t), batch, tokens, tok_off, len, false);  // reads only
  const int64_t pg = t->page;
  for_requests(batch, total, [&](int32_t b) {
    walked[b] = pg * walk(*t, u.at(b), u.len(b), [&](int32_t id, int64_t k) {
      walks[b].push_back({id, (t->nodes[id].start + k) * pg});
    });
  });
}

}  // namespace

extern "C" rc_status rc_radix_plan_decode(rc_radix* t, int32_t batch, const int32_t* tokens, const int64_t* tok_off,
                                          const int64_t* tok_len, const int32_t* rows, const int32_t* max_seq,
                                          int32_t group, int32_t chunk, int32_t* plan, int64_t cap,
                                          rc_plan_info* info) {
  if (!t) return fail(RC_ERR_ARG, "tree is NULL");
  rc_status st = plan_args(batch, max_seq, group, chunk, info);
  if (st != RC_OK) return st;
  if (batch > 0 && !tok_off) return fail(RC_ERR_ARG, "tok_off is NULL");
  if ((st = check_lens(batch, tok_off, tok_len)) != RC_OK) return st;
  auto len = [&](int32_t b) { return tok_len ? tok_len[b] : tok_off[b + 1] - tok_off[b]; };
  for (int32_t b = 0; b < batch; ++b)
    if (len(b) > 0 && !tokens) return fail(RC_ERR_ARG, "tokens is NULL");
  std::vector<std::vector<Visit>> walks;
  std::vector<int64_t> walked;
  walk_requests(t, batch, tokens, tok_off, len, walks, walked);
  std::vector<int32_t> req_of(batch), rows_of(batch);
  for (int32_t b = 0; b < batch; ++b) {
    req_of[b] = b;
    rows_of[b] = rows ? rows[b] : b;
  }
  return plan_from_walks(t, batch, req_of, walks, walked, rows_of, max_seq, group, chunk, RC_DECODE_COLS, plan, cap,
                         info);
}

extern "C" rc_status rc_radix_plan_extend(rc_radix* t, int32_t batch, const int32_t* tokens, const int64_t* tok_off,
                                          const int32_t* prefix_lens, const int32_t* extend_lens, const int32_t* rows,
                                          int32_t group, int32_t chunk, int32_t* plan, int64_t cap,
                                          rc_plan_info* info, int32_t* seq_lens) {
  if (!t || !info) return fail(RC_ERR_ARG, "tree or info is NULL");
  if (batch < 0) return fail(RC_ERR_ARG, "batch < 0");
  if (batch > 0 && (!tok_off || !prefix_lens || !extend_lens)) return fail(RC_ERR_ARG, "NULL array in rc_radix_plan_extend");
  rc_status st = check_lens(batch, tok_off, nullptr);
  if (st != RC_OK) return st;
  int64_t n_tok = 0;
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t n = tok_off[b + 1] - tok_off[b];
    if (prefix_lens[b] < 0 || extend_lens[b] < 0 || (int64_t)prefix_lens[b] + extend_lens[b] > n)
      return fail(RC_ERR_RANGE, "request %d: prefix %d + extend %d exceed its %lld tokens", b, prefix_lens[b], extend_lens[b], (long long)n);
    if (prefix_lens[b] > 0 && !tokens) return fail(RC_ERR_ARG, "tokens is NULL");
    n_tok += extend_lens[b];
  }
  if (n_tok > INT32_MAX) return fail(RC_ERR_RANGE, "%lld new tokens", (long long)n_tok);
  // members: the new tokens in batch order; token i of request b sees
  // positions [0, prefix_lens[b] + i]
  std::vector<int32_t> req_of((size_t)n_tok), rows_of((size_t)n_tok), max_seq((size_t)n_tok);
  int64_t m = 0;
  for (int32_t b = 0; b < batch; ++b)
    for (int32_t i = 0; i < extend_lens[b]; ++i, ++m) {
      req_of[m] = b;
      rows_of[m] = rows ? rows[b] : b;
      max_seq[m] = prefix_lens[b] + i + 1;
    }
  st = plan_args((int32_t)n_tok, max_seq.data(), group, chunk, info);
  if (st != RC_OK) return st;
  std::vector<std::vector<Visit>> walks;
  std::vector<int64_t> walked;
  walk_requests(t, batch, tokens, tok_off, [&](int32_t b) { return (int64_t)prefix_lens[b]; }, walks, walked);
  st = plan_from_walks(t, (int32_t)n_tok, req_of, walks, walked, rows_of, max_seq.data(), group, chunk,
                       RC_EXTEND_SHARED_COLS, plan, cap, info);
  if (st == RC_OK && seq_lens) std::copy(max_seq.begin(), max_seq.end(), seq_lens);
  return st;
}
