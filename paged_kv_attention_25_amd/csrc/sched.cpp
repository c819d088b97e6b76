// Host-side producer of the paged attention calls' metadata: page allocator,
// prefix cache (radix tree or none) and chunked-prefill / decode batch builder.
//
// The pool is one store every request allocates pages from ("Mini-SGLang deployment
// guide", section 6.2; "miniSGLang intro blog", section 1.2); the cache manager
// shares prefixes through a radix tree or shares nothing (deployment guide, section
// 6.5); prompts are prefilled in chunks under a per-pass token budget (deployment
// guide, section 6.1). The behaviour the pages leave open is stated in pka_sched.h.
//
// Radix tree. A node holds a run of whole pages: its tokens (a multiple of P) and
// their page ids. Children are keyed by the tokens of their first page. Every page
// of a node carries the node's last-use stamp and lock count: a match or insertion
// that ends inside a node first splits it there, so the pages one operation covers
// are always whole nodes. A split makes a new node for the head and keeps the
// original object as the tail, so a live request's locked chain (recorded as its
// deepest node) stays valid across later splits. Evictable nodes (no children, no
// lock) sit in a set ordered by stamp; eviction takes the last page of the first.
#include <algorithm>
#include <cstring>
#include <map>
#include <memory>
#include <new>
#include <set>
#include <tuple>
#include <unordered_map>
#include <vector>

#include "pka_sched.h"

namespace {

using Tokens = std::vector<int32_t>;

struct Node {
  Tokens key;                  // tokens of the node's pages, pages.size() * P of them
  std::vector<int32_t> pages;  // page ids
  Node* parent = nullptr;
  std::map<Tokens, Node*> children;  // by the tokens of the child's first page
  int64_t stamp = 0;
  int32_t lock = 0;
  uint64_t id = 0;
  bool listed = false;  // in the evictable set
};

enum class State { kWaiting, kPrefilling, kRunning };

struct Request {
  int64_t id = 0;
  Tokens tokens;         // prompt, then every pushed token
  int32_t n_prompt = 0;
  int32_t cached = 0;    // tokens whose K/V the scheduler counts as stored
  int32_t matched_pages = 0;  // leading pages owned by the cache (locked)
  Node* chain = nullptr;      // deepest node of the locked chain
  std::vector<int32_t> pages;
  State state = State::kWaiting;
  bool pending = false;  // running: has an input token for the next decode
  uint64_t run_order = 0;
};

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

class RadixTree {
 public:
  explicit RadixTree(int32_t page_size) : P_(page_size) { root_.lock = 1; }
  ~RadixTree() { free_subtree(&root_); }
  RadixTree(const RadixTree&) = delete;
  RadixTree& operator=(const RadixTree&) = delete;

  int64_t cached_pages() const { return cached_pages_; }
  int64_t locked_pages() const { return locked_pages_; }

  // Longest cached prefix of tokens[0 .. limit_pages*P) in whole pages. Stamps and
  // locks the matched chain; returns its deepest node (nullptr when nothing matched)
  // and appends the matched page ids.
  Node* match_and_lock(const int32_t* tokens, int64_t limit_pages, int64_t now,
                       std::vector<int32_t>* pages) {
    Node* cur = &root_;
    int64_t pi = 0;
    while (pi < limit_pages) {
      auto it = cur->children.find(page_tokens(tokens, pi));
      if (it == cur->children.end()) break;
      Node* n = it->second;
      const int64_t np = common_pages(n, tokens, pi, limit_pages - pi);
      const bool whole = np == (int64_t)n->pages.size();
      if (!whole) n = split(n, np);
      pages->insert(pages->end(), n->pages.begin(), n->pages.end());
      pi += np;
      cur = n;
      if (!whole) break;
    }
    if (cur == &root_) return nullptr;
    stamp_chain(cur, now);
    for (Node* n = cur; n != &root_; n = n->parent) {
      unlist(n);
      if (n->lock++ == 0) locked_pages_ += (int64_t)n->pages.size();
    }
    return cur;
  }

  void unlock(Node* chain) {
    for (Node* n = chain; n != nullptr && n != &root_; n = n->parent) {
      if (--n->lock == 0) locked_pages_ -= (int64_t)n->pages.size();
      relist(n);
    }
  }

  // Insert the first n_pages whole pages of tokens, whose K/V sit in req_pages.
  // Positions already cached keep the cache's page; the request's page there is
  // reported in *dup (unless it is that same page). Returns how many of the
  // request's pages the cache took over.
  int64_t insert(const int32_t* tokens, int64_t n_pages, const std::vector<int32_t>& req_pages,
                 int64_t now, std::vector<int32_t>* dup) {
    Node* cur = &root_;
    int64_t pi = 0;
    int64_t taken = 0;
    while (pi < n_pages) {
      Tokens first = page_tokens(tokens, pi);
      auto it = cur->children.find(first);
      if (it == cur->children.end()) {
        Node* c = new Node;
        c->key.assign(tokens + pi * P_, tokens + n_pages * P_);
        c->pages.assign(req_pages.begin() + pi, req_pages.begin() + n_pages);
        c->parent = cur;
        c->stamp = now;
        c->id = next_id_++;
        unlist(cur);
        cur->children.emplace(std::move(first), c);
        taken += n_pages - pi;
        cached_pages_ += n_pages - pi;
        pi = n_pages;
        cur = c;
        break;
      }
      Node* n = it->second;
      const int64_t np = common_pages(n, tokens, pi, n_pages - pi);
      if (np < (int64_t)n->pages.size()) n = split(n, np);
      for (int64_t k = 0; k < np; ++k)
        if (req_pages[pi + k] != n->pages[k]) dup->push_back(req_pages[pi + k]);
      pi += np;
      cur = n;
    }
    if (cur != &root_) stamp_chain(cur, now);
    return taken;
  }

  // Evict the least recently used unlocked leaf page; -1 when there is none.
  int32_t evict_one() {
    if (evictable_.empty()) return -1;
    Node* n = std::get<2>(*evictable_.begin());
    unlist(n);
    const int32_t page = n->pages.back();
    n->pages.pop_back();
    --cached_pages_;
    if (n->pages.empty()) {
      Node* parent = n->parent;
      Tokens first(n->key.begin(), n->key.begin() + P_);
      parent->children.erase(first);
      delete n;
      relist(parent);
    } else {
      n->key.resize(n->pages.size() * (size_t)P_);
      relist(n);
    }
    return page;
  }

 private:
  Tokens page_tokens(const int32_t* tokens, int64_t page) const {
    return Tokens(tokens + page * P_, tokens + (page + 1) * P_);
  }

  // Number of leading pages of n equal to tokens' pages pi, pi+1, ... (at most max_pages).
  int64_t common_pages(const Node* n, const int32_t* tokens, int64_t pi, int64_t max_pages) const {
    const int64_t lim = std::min<int64_t>((int64_t)n->pages.size(), max_pages);
    int64_t k = 0;
    while (k < lim && std::memcmp(n->key.data() + k * P_, tokens + (pi + k) * P_,
                                  sizeof(int32_t) * (size_t)P_) == 0)
      ++k;
    return k;
  }

  // Split n after its first np pages (0 < np < size): a new head node takes them and
  // n keeps the rest, below the head. Returns the head.
  Node* split(Node* n, int64_t np) {
    unlist(n);
    Node* h = new Node;
    h->key.assign(n->key.begin(), n->key.begin() + np * P_);
    h->pages.assign(n->pages.begin(), n->pages.begin() + np);
    h->parent = n->parent;
    h->stamp = n->stamp;
    h->lock = n->lock;
    h->id = next_id_++;
    n->key.erase(n->key.begin(), n->key.begin() + np * P_);
    n->pages.erase(n->pages.begin(), n->pages.begin() + np);
    h->parent->children[Tokens(h->key.begin(), h->key.begin() + P_)] = h;
    h->children.emplace(Tokens(n->key.begin(), n->key.begin() + P_), n);
    n->parent = h;
    relist(n);
    return h;
  }

  void stamp_chain(Node* deepest, int64_t now) {
    for (Node* n = deepest; n != &root_; n = n->parent) {
      unlist(n);
      n->stamp = now;
      relist(n);
    }
  }

  void unlist(Node* n) {
    if (!n->listed) return;
    evictable_.erase(std::make_tuple(n->stamp, n->id, n));
    n->listed = false;
  }
  void relist(Node* n) {
    if (n->listed || n == &root_ || n->lock != 0 || !n->children.empty() || n->pages.empty())
      return;
    evictable_.insert(std::make_tuple(n->stamp, n->id, n));
    n->listed = true;
  }

  void free_subtree(Node* n) {
    for (auto& kv : n->children) {
      free_subtree(kv.second);
      delete kv.second;
    }
    n->children.clear();
  }

  int32_t P_;
  Node root_;
  uint64_t next_id_ = 1;
  int64_t cached_pages_ = 0;
  int64_t locked_pages_ = 0;
  std::set<std::tuple<int64_t, uint64_t, Node*>> evictable_;
};

}  // namespace

struct pka_sched {
  pka_sched(int32_t page_size, int64_t num_pages, int32_t policy, int32_t max_prefill)
      : P(page_size), radix(policy == PKA_CACHE_RADIX), max_prefill_tokens(max_prefill),
        tree(page_size) {
    free_list.reserve((size_t)num_pages);
    for (int64_t p = num_pages - 1; p >= 0; --p) free_list.push_back((int32_t)p);
  }

  int32_t P;
  bool radix;
  int32_t max_prefill_tokens;
  RadixTree tree;
  std::vector<int32_t> free_list;  // popped from the back: pages 0, 1, 2, ... first
  int64_t clock = 0;
  int64_t private_pages = 0;
  int64_t evicted = 0;
  uint64_t next_run_order = 0;
  std::unordered_map<int64_t, std::unique_ptr<Request>> reqs;
  std::vector<Request*> queue;             // waiting and prefilling, first come first
  std::map<uint64_t, Request*> running;    // by the order their prompts completed

  int32_t alloc_page() {
    if (!free_list.empty()) {
      const int32_t p = free_list.back();
      free_list.pop_back();
      return p;
    }
    if (!radix) return -1;
    const int32_t p = tree.evict_one();
    if (p >= 0) ++evicted;
    return p;
  }

  void admit(Request* r) {
    ++clock;
    if (radix) {
      const int64_t limit_pages = (r->n_prompt - 1) / P;
      r->chain = tree.match_and_lock(r->tokens.data(), limit_pages, clock, &r->pages);
      r->matched_pages = (int32_t)r->pages.size();
      r->cached = r->matched_pages * P;
    }
    r->state = State::kPrefilling;
  }

  // Write row b of a batch from request r with `extend` new tokens at positions
  // r->cached .. r->cached + extend - 1, whose out_loc entries start at t0.
  void emit(pka_batch* out, int32_t b, const Request* r, int32_t extend, int32_t t0) {
    const int32_t seq = r->cached + extend;
    out->req_ids[b] = r->id;
    out->seq_lens[b] = seq;
    out->prefix_lens[b] = r->cached;
    out->extend_lens[b] = extend;
    out->cu_extend[b] = t0;
    int32_t* row = out->page_table + (int64_t)b * out->table_width;
    const int32_t used = (int32_t)ceil_div(seq, P);
    std::copy(r->pages.begin(), r->pages.begin() + used, row);
    for (int32_t i = 0; i < extend; ++i) {
      const int32_t pos = r->cached + i;
      out->out_loc[t0 + i] = r->pages[pos / P] * P + pos % P;
    }
    out->max_extend = std::max(out->max_extend, extend);
    out->max_seq_len = std::max(out->max_seq_len, seq);
  }
};

namespace {

int check_batch(const pka_batch* out) {
  if (out == nullptr) return PKA_E_NULLPTR;
  if (out->max_batch < 0 || out->table_width < 1 || out->max_tokens < 0) return PKA_E_SHAPE;
  if (out->max_batch > 0 && (out->req_ids == nullptr || out->page_table == nullptr ||
                             out->seq_lens == nullptr || out->prefix_lens == nullptr ||
                             out->extend_lens == nullptr))
    return PKA_E_NULLPTR;
  if (out->cu_extend == nullptr || (out->max_tokens > 0 && out->out_loc == nullptr))
    return PKA_E_NULLPTR;
  return PKA_OK;
}

// Every entry point runs inside this: no C++ exception crosses the C ABI.
template <class F>
int guarded(F&& f) {
  try {
    return f();
  } catch (...) {
    return PKA_E_NOMEM;
  }
}

void reset_batch(pka_batch* out) {
  out->batch = 0;
  out->num_tokens = 0;
  out->max_extend = 0;
  out->max_seq_len = 0;
  out->cu_extend[0] = 0;
}

}  // namespace

extern "C" {

int pka_sched_create(int32_t page_size, int64_t num_pages, int32_t cache_policy,
                     int32_t max_prefill_tokens, pka_sched** out) {
  return guarded([&]() -> int {
    if (out == nullptr) return PKA_E_NULLPTR;
    *out = nullptr;
    if (page_size < 1 || num_pages < 1 || max_prefill_tokens < 1 ||
        num_pages * (int64_t)page_size > INT32_MAX ||
        (cache_policy != PKA_CACHE_NAIVE && cache_policy != PKA_CACHE_RADIX))
      return PKA_E_SHAPE;
    *out = new (std::nothrow) pka_sched(page_size, num_pages, cache_policy, max_prefill_tokens);
    return *out ? PKA_OK : PKA_E_SHAPE;
  });
}

void pka_sched_destroy(pka_sched* s) { delete s; }

int pka_sched_add_request(pka_sched* s, int64_t req_id, const int32_t* tokens, int32_t n) {
  return guarded([&]() -> int {
    if (s == nullptr || tokens == nullptr) return PKA_E_NULLPTR;
    if (n < 1) return PKA_E_SHAPE;
    if (s->reqs.count(req_id)) return PKA_E_STATE;
    auto r = std::make_unique<Request>();
    r->id = req_id;
    r->tokens.assign(tokens, tokens + n);
    r->n_prompt = n;
    s->queue.push_back(r.get());
    s->reqs.emplace(req_id, std::move(r));
    return PKA_OK;
  });
}

int pka_sched_prefill_batch(pka_sched* s, pka_batch* out) {
  return guarded([&]() -> int {
    if (s == nullptr) return PKA_E_NULLPTR;
    const int st = check_batch(out);
    if (st != PKA_OK) return st;
    for (const Request* r : s->queue)
      if (ceil_div(r->n_prompt, s->P) > out->table_width) return PKA_E_CAPACITY;
    reset_batch(out);
    const int32_t budget = std::min(s->max_prefill_tokens, out->max_tokens);
    int32_t rows = 0, tokens = 0;
    size_t qi = 0;
    while (qi < s->queue.size() && rows < out->max_batch && tokens < budget) {
      Request* r = s->queue[qi];
      if (r->state == State::kWaiting) s->admit(r);
      const int32_t want = std::min(r->n_prompt - r->cached, budget - tokens);
      const int64_t need_pages = ceil_div((int64_t)r->cached + want, s->P);
      while ((int64_t)r->pages.size() < need_pages) {
        const int32_t p = s->alloc_page();
        if (p < 0) break;
        r->pages.push_back(p);
        ++s->private_pages;
      }
      const int32_t extend = std::min<int32_t>(want, (int32_t)r->pages.size() * s->P - r->cached);
      if (extend <= 0) break;  // no page for it: it and everything behind it wait
      s->emit(out, rows, r, extend, tokens);
      r->cached += extend;
      tokens += extend;
      ++rows;
      if (r->cached == r->n_prompt) {
        r->state = State::kRunning;
        r->run_order = s->next_run_order++;
        s->running.emplace(r->run_order, r);
        s->queue.erase(s->queue.begin() + (std::ptrdiff_t)qi);
      } else {
        ++qi;
      }
      if (extend < want) break;  // the pool ran out
    }
    out->batch = rows;
    out->num_tokens = tokens;
    out->cu_extend[rows] = tokens;
    return PKA_OK;
  });
}

int pka_sched_push_token(pka_sched* s, int64_t req_id, int32_t token) {
  return guarded([&]() -> int {
    if (s == nullptr) return PKA_E_NULLPTR;
    auto it = s->reqs.find(req_id);
    if (it == s->reqs.end()) return PKA_E_STATE;
    Request* r = it->second.get();
    if (r->state != State::kRunning || r->pending) return PKA_E_STATE;
    r->tokens.push_back(token);
    r->pending = true;
    return PKA_OK;
  });
}

int pka_sched_push_tokens(pka_sched* s, const int64_t* req_ids, const int32_t* tokens,
                          int32_t n) {
  return guarded([&]() -> int {
    if (s == nullptr) return PKA_E_NULLPTR;
    if (n < 0) return PKA_E_SHAPE;
    if (n > 0 && (req_ids == nullptr || tokens == nullptr)) return PKA_E_NULLPTR;
    // Mark each request pending as it is checked (a second occurrence then fails the
    // check); on any failure the marks made so far are undone.
    std::vector<Request*> rs((size_t)n);
    for (int32_t i = 0; i < n; ++i) {
      auto it = s->reqs.find(req_ids[i]);
      Request* r = it == s->reqs.end() ? nullptr : it->second.get();
      if (r == nullptr || r->state != State::kRunning || r->pending) {
        for (int32_t k = 0; k < i; ++k) rs[(size_t)k]->pending = false;
        return PKA_E_STATE;
      }
      r->pending = true;
      rs[(size_t)i] = r;
    }
    for (int32_t i = 0; i < n; ++i) rs[(size_t)i]->tokens.push_back(tokens[i]);
    return PKA_OK;
  });
}

int pka_sched_decode_batch(pka_sched* s, pka_batch* out) {
  return guarded([&]() -> int {
    if (s == nullptr) return PKA_E_NULLPTR;
    const int st = check_batch(out);
    if (st != PKA_OK) return st;
    for (const auto& kv : s->running) {
      const Request* r = kv.second;
      if (r->pending && ceil_div((int64_t)r->cached + 1, s->P) > out->table_width)
        return PKA_E_CAPACITY;
    }
    reset_batch(out);
    int32_t rows = 0;
    for (auto& kv : s->running) {
      if (rows == out->max_batch || rows == out->max_tokens) break;
      Request* r = kv.second;
      if (!r->pending) continue;
      const int32_t pos = r->cached;
      if (pos / s->P >= (int32_t)r->pages.size()) {
        const int32_t p = s->alloc_page();
        if (p < 0) continue;  // waits for a page
        r->pages.push_back(p);
        ++s->private_pages;
      }
      s->emit(out, rows, r, 1, rows);
      r->cached += 1;
      r->pending = false;
      ++rows;
    }
    out->batch = rows;
    out->num_tokens = rows;
    out->cu_extend[rows] = rows;
    return PKA_OK;
  });
}

int pka_sched_finish(pka_sched* s, int64_t req_id) {
  return guarded([&]() -> int {
    if (s == nullptr) return PKA_E_NULLPTR;
    auto it = s->reqs.find(req_id);
    if (it == s->reqs.end()) return PKA_E_STATE;
    Request* r = it->second.get();
    if (r->state == State::kRunning) {
      s->running.erase(r->run_order);
    } else {
      s->queue.erase(std::find(s->queue.begin(), s->queue.end(), r));
    }
    if (r->state != State::kWaiting) {
      ++s->clock;
      const int64_t n_private = (int64_t)r->pages.size() - r->matched_pages;
      std::vector<int32_t> to_free;
      int64_t full = 0;
      if (s->radix) {
        full = r->cached / s->P;
        s->tree.insert(r->tokens.data(), full, r->pages, s->clock, &to_free);
        s->tree.unlock(r->chain);
      }
      for (int64_t k = std::max<int64_t>(full, r->matched_pages); k < (int64_t)r->pages.size(); ++k)
        to_free.push_back(r->pages[k]);
      s->private_pages -= n_private;
      s->free_list.insert(s->free_list.end(), to_free.begin(), to_free.end());
    }
    s->reqs.erase(it);
    return PKA_OK;
  });
}

int pka_sched_request_pages(const pka_sched* s, int64_t req_id, int32_t* pages, int32_t cap,
                            int32_t* n_pages, int32_t* cached) {
  return guarded([&]() -> int {
    if (s == nullptr || n_pages == nullptr || cached == nullptr) return PKA_E_NULLPTR;
    auto it = s->reqs.find(req_id);
    if (it == s->reqs.end()) return PKA_E_STATE;
    const Request* r = it->second.get();
    if ((int64_t)r->pages.size() > cap) return PKA_E_CAPACITY;
    if (!r->pages.empty() && pages == nullptr) return PKA_E_NULLPTR;
    std::copy(r->pages.begin(), r->pages.end(), pages);
    *n_pages = (int32_t)r->pages.size();
    *cached = r->cached;
    return PKA_OK;
  });
}

int pka_sched_get_stats(const pka_sched* s, pka_sched_stats* out) {
  return guarded([&]() -> int {
    if (s == nullptr || out == nullptr) return PKA_E_NULLPTR;
    std::memset(out, 0, sizeof(*out));
    out->free_pages = (int64_t)s->free_list.size();
    out->cached_pages = s->tree.cached_pages();
    out->locked_pages = s->tree.locked_pages();
    out->private_pages = s->private_pages;
    out->evicted_pages = s->evicted;
    for (const Request* r : s->queue) {
      if (r->state == State::kWaiting)
        ++out->waiting;
      else
        ++out->prefilling;
    }
    out->running = (int32_t)s->running.size();
    return PKA_OK;
  });
}

}  // extern "C"
