// Randomised stress of the host-side metadata producer (csrc/sched.cpp) through its C
// ABI, built and run by tests/test_sched_sanitizers.py with AddressSanitizer and
// UndefinedBehaviorSanitizer (host code only). Streams of requests sharing prompt
// prefixes go through admission, chunked prefill, token pushes, decode batches and
// retirement on small and large pools, with both cache policies and several page sizes,
// so that pool exhaustion, eviction and partial chunks all occur. Every batch is checked
// against what the batch contract promises: consistent lengths and prefix sums, page ids
// inside the pool, and new-token slots equal to the slots of their positions through
// the batch's own page table, distinct within the batch. Prints SCHED_STRESS_OK and
// exits 0 when every check held; any sanitizer report aborts the run.
#include <cstdio>
#include <cstdlib>
#include <random>
#include <set>
#include <vector>

#include "pka_sched.h"

namespace {

int failures = 0;

void fail(const char* what, long a, long b) {
  std::fprintf(stderr, "check failed: %s (%ld, %ld)\n", what, a, b);
  if (++failures > 20) std::exit(1);
}

struct Buffers {
  std::vector<int64_t> req_ids;
  std::vector<int32_t> page_table, seq_lens, prefix_lens, extend_lens, cu_extend, out_loc;
  pka_batch b{};
  Buffers(int max_batch, int width, int max_tokens)
      : req_ids(max_batch), page_table((size_t)max_batch * width), seq_lens(max_batch),
        prefix_lens(max_batch), extend_lens(max_batch), cu_extend(max_batch + 1),
        out_loc(max_tokens > 0 ? max_tokens : 1) {
    b.max_batch = max_batch;
    b.table_width = width;
    b.max_tokens = max_tokens;
    b.req_ids = req_ids.data();
    b.page_table = page_table.data();
    b.seq_lens = seq_lens.data();
    b.prefix_lens = prefix_lens.data();
    b.extend_lens = extend_lens.data();
    b.cu_extend = cu_extend.data();
    b.out_loc = out_loc.data();
  }
};

void check_batch(const pka_batch& b, int page_size, int64_t num_pages, bool decode) {
  if (b.batch < 0 || b.batch > b.max_batch) fail("batch count", b.batch, b.max_batch);
  if (b.num_tokens < 0 || b.num_tokens > b.max_tokens) fail("token count", b.num_tokens, b.max_tokens);
  if (b.cu_extend[0] != 0) fail("cu_extend[0]", b.cu_extend[0], 0);
  std::set<int32_t> slots;
  int32_t max_e = 0, max_s = 0;
  for (int r = 0; r < b.batch; ++r) {
    const int32_t e = b.extend_lens[r], p = b.prefix_lens[r], L = b.seq_lens[r];
    if (e < 1) fail("extend >= 1", r, e);
    if (decode && e != 1) fail("decode extend", r, e);
    if (p < 0 || L != p + e) fail("seq = prefix + extend", r, L);
    if (b.cu_extend[r + 1] != b.cu_extend[r] + e) fail("cu_extend", r, b.cu_extend[r + 1]);
    if ((L + page_size - 1) / page_size > b.table_width) fail("row width", r, L);
    max_e = e > max_e ? e : max_e;
    max_s = L > max_s ? L : max_s;
    const int32_t* row = b.page_table + (size_t)r * b.table_width;
    for (int k = 0; k < (L + page_size - 1) / page_size; ++k)
      if (row[k] < 0 || row[k] >= num_pages) fail("page id in pool", r, row[k]);
    for (int32_t j = p; j < L; ++j) {
      const int32_t t = b.cu_extend[r] + (j - p);
      const int32_t want = row[j / page_size] * page_size + j % page_size;
      if (b.out_loc[t] != want) fail("out_loc = slot of the position", t, b.out_loc[t]);
      if (!slots.insert(b.out_loc[t]).second) fail("out_loc distinct", t, b.out_loc[t]);
    }
  }
  if (b.cu_extend[b.batch] != b.num_tokens) fail("cu_extend total", b.cu_extend[b.batch], b.num_tokens);
  if (b.batch > 0 && (b.max_extend != max_e || b.max_seq_len != max_s))
    fail("max extend / seq", b.max_extend, b.max_seq_len);
}

void run(int page_size, int64_t num_pages, int policy, int chunk, unsigned seed, int ops) {
  pka_sched* s = nullptr;
  if (pka_sched_create(page_size, num_pages, policy, chunk, &s) != PKA_OK || !s) {
    fail("create", page_size, num_pages);
    return;
  }
  std::mt19937 rng(seed);
  auto uni = [&](int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); };
  const int width = 2048 / page_size + 2;
  Buffers pre(16, width, chunk), dec(64, width, 64);
  std::vector<int32_t> system_prompt(200);
  for (auto& t : system_prompt) t = uni(0, 50);
  std::vector<int64_t> live;
  int64_t next_id = 1;
  for (int op = 0; op < ops; ++op) {
    const int what = uni(0, 9);
    if (what <= 2 && live.size() < 80) {
      // a prompt that often starts with the shared system prompt (radix hits)
      const int n = uni(1, 600);
      std::vector<int32_t> toks(n);
      const int shared = uni(0, 1) ? std::min(n, uni(0, 200)) : 0;
      for (int i = 0; i < n; ++i) toks[i] = i < shared ? system_prompt[i] : uni(0, 50);
      const int st = pka_sched_add_request(s, next_id, toks.data(), n);
      if (st != PKA_OK) fail("add", st, next_id);
      live.push_back(next_id++);
    } else if (what <= 4) {
      const int st = pka_sched_prefill_batch(s, &pre.b);
      if (st == PKA_OK) check_batch(pre.b, page_size, num_pages, false);
      else if (st != PKA_E_CAPACITY) fail("prefill batch", st, 0);
    } else if (what <= 6) {
      // next tokens for every running request without one
      std::vector<int64_t> ids;
      std::vector<int32_t> toks;
      for (int64_t id : live) {
        if (pka_sched_push_token(s, id, uni(0, 50)) == PKA_OK) ids.push_back(id);
      }
      const int st = pka_sched_decode_batch(s, &dec.b);
      if (st == PKA_OK) check_batch(dec.b, page_size, num_pages, true);
      else if (st != PKA_E_CAPACITY) fail("decode batch", st, 0);
      (void)toks;
    } else if (what == 7 && !live.empty()) {
      const size_t k = (size_t)uni(0, (int)live.size() - 1);
      const int st = pka_sched_finish(s, live[k]);
      if (st != PKA_OK) fail("finish", st, live[k]);
      live.erase(live.begin() + (long)k);
    } else if (what == 8 && !live.empty()) {
      std::vector<int32_t> pages(width + 8);
      int32_t n = 0, cached = 0;
      const int64_t id = live[(size_t)uni(0, (int)live.size() - 1)];
      const int st = pka_sched_request_pages(s, id, pages.data(), (int32_t)pages.size(), &n, &cached);
      if (st == PKA_OK) {
        if (n < 0 || n > (int32_t)pages.size() || cached < 0) fail("request pages", n, cached);
        for (int i = 0; i < n; ++i)
          if (pages[i] < 0 || pages[i] >= num_pages) fail("request page id", i, pages[i]);
      } else if (st != PKA_E_CAPACITY) {
        fail("request pages status", st, id);
      }
    } else {
      pka_sched_stats st{};
      if (pka_sched_get_stats(s, &st) != PKA_OK) fail("stats", 0, 0);
      const int64_t total = st.free_pages + st.cached_pages + st.private_pages;
      if (total != num_pages) fail("pages accounted", total, num_pages);
    }
  }
  // wrong-state and bad-argument paths
  if (pka_sched_finish(s, -12345) != PKA_E_STATE) fail("finish unknown", 0, 0);
  if (pka_sched_push_token(s, -12345, 1) != PKA_E_STATE) fail("push unknown", 0, 0);
  for (int64_t id : live) pka_sched_finish(s, id);
  pka_sched_destroy(s);
}

}  // namespace

int main() {
  unsigned seed = 1;
  for (int policy : {PKA_CACHE_NAIVE, PKA_CACHE_RADIX})
    for (int page_size : {1, 4, 16})
      for (int64_t pages : {(int64_t)(1024 / page_size), (int64_t)(65536 / page_size)})
        run(page_size, pages, policy, policy == PKA_CACHE_RADIX ? 512 : 300, seed++, 3000);
  if (failures) {
    std::fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  std::printf("SCHED_STRESS_OK\n");
  return 0;
}
