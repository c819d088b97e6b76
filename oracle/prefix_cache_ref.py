"""Prefix cache, page pool and batch builder, written out plainly (CPU, pure Python).

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix: one pool every request allocates from, in pages of page_size
tokens [deployment guide (dpshk.com), section 6.2 "Page Size"; miniSGLang intro
blog (0539edu.com), section 1.2, KV cache module: a pool and a manager]; a cache
manager that either shares prefixes across requests through a radix tree or
shares nothing (naive) [deployment guide, section 6.5 "Radix Cache"]; prompts
prefilled in chunks under a per-pass token budget [deployment guide, section 6.1
"Chunked Prefill"].

The pages give no algorithm, so this follows these READINGS (the same ones the
library's header states):

* A cached page is identified by the whole token prefix it ends: the key of the
  k-th page of a sequence is tuple(tokens[:k*P]). The cache is the set of such
  keys; it is closed under taking shorter page-aligned prefixes, which is what a
  radix tree over pages holds. This model has no tree and no page ids: page ids
  are not unique (any free page will do), so only the page COUNTS are modelled.
* Match on admission: the largest k with every key tuple(tokens[:j*P]), j <= k,
  cached and k*P <= prompt_len - 1. The matched keys get the current clock value as
  their last use and one more lock each.
* Allocation of one page: a free page if there is one, else (radix) evict the
  unlocked leaf key (no cached key one page longer extends it) with the oldest last
  use; with none, the allocation fails.
* Finish: every whole page of the tokens whose K/V are stored is inserted (an
  already-cached key is only re-stamped); the request's pages that did not become
  cached pages are freed; the matched keys are unlocked. Admissions and finishes
  each advance the clock by one.
* Prefill batch: the queue in arrival order (requests part-way through their
  prompt are ahead of new ones, as they arrived earlier); each gets
  min(rest of prompt, rest of budget) tokens, cut down to what the pages it can
  get hold; the first request that gets no token ends the batch, and so does one
  that got fewer than it wanted.
* Decode batch: running requests with a pending token in the order their prompts
  completed; one that needs a page and cannot get one is skipped this time.
"""
from __future__ import annotations


class PrefixCacheRef:
    def __init__(self, page_size: int, num_pages: int, policy: str, max_prefill_tokens: int):
        assert policy in ("naive", "radix")
        self.P = page_size
        self.num_pages = num_pages
        self.radix = policy == "radix"
        self.max_prefill_tokens = max_prefill_tokens
        self.free = num_pages
        self.cache = {}      # key tuple -> [last_use, locks]
        self.clock = 0
        self.evicted = 0
        self.reqs = {}       # id -> dict
        self.queue = []      # ids, arrival order (waiting and prefilling)
        self.running = []    # ids, order of prompt completion

    # --- pages -------------------------------------------------------------------

    def _is_leaf(self, key) -> bool:
        n = len(key) + self.P
        return not any(len(k) == n and k[:len(key)] == key for k in self.cache)

    def _alloc(self) -> bool:
        if self.free > 0:
            self.free -= 1
            return True
        if not self.radix:
            return False
        cands = [k for k, (_, locks) in self.cache.items() if locks == 0 and self._is_leaf(k)]
        if not cands:
            return False
        victim = min(cands, key=lambda k: self.cache[k][0])
        del self.cache[victim]
        self.evicted += 1
        return True

    # --- requests ----------------------------------------------------------------

    def add_request(self, rid, tokens):
        assert rid not in self.reqs and len(tokens) >= 1
        self.reqs[rid] = dict(tokens=list(tokens), n_prompt=len(tokens), cached=0, pages=0,
                              matched=[], state="waiting", pending=False)
        self.queue.append(rid)

    def _admit(self, r):
        self.clock += 1
        if self.radix:
            P = self.P
            k = 0
            while (k + 1) * P <= r["n_prompt"] - 1 and tuple(r["tokens"][:(k + 1) * P]) in self.cache:
                k += 1
            r["matched"] = [tuple(r["tokens"][:j * P]) for j in range(1, k + 1)]
            for key in r["matched"]:
                self.cache[key][0] = self.clock
                self.cache[key][1] += 1
            r["pages"] = k
            r["cached"] = k * P
        r["state"] = "prefilling"

    def prefill_batch(self, max_batch: int, max_tokens: int):
        """Rows (req_id, prefix_len, extend_len) of the next prefill batch."""
        rows = []
        budget = min(self.max_prefill_tokens, max_tokens)
        used = 0
        i = 0
        while i < len(self.queue) and len(rows) < max_batch and used < budget:
            rid = self.queue[i]
            r = self.reqs[rid]
            if r["state"] == "waiting":
                self._admit(r)
            want = min(r["n_prompt"] - r["cached"], budget - used)
            need = -(-(r["cached"] + want) // self.P)
            while r["pages"] < need and self._alloc():
                r["pages"] += 1
            extend = min(want, r["pages"] * self.P - r["cached"])
            if extend <= 0:
                break
            rows.append((rid, r["cached"], extend))
            r["cached"] += extend
            used += extend
            if r["cached"] == r["n_prompt"]:
                r["state"] = "running"
                self.running.append(rid)
                self.queue.pop(i)
            else:
                i += 1
            if extend < want:
                break
        return rows

    def push_token(self, rid, token):
        r = self.reqs[rid]
        assert r["state"] == "running" and not r["pending"]
        r["tokens"].append(token)
        r["pending"] = True

    def decode_batch(self, max_batch: int, max_tokens: int):
        """Rows (req_id, prefix_len, 1) of the next decode batch."""
        rows = []
        for rid in self.running:
            if len(rows) == max_batch or len(rows) == max_tokens:
                break
            r = self.reqs[rid]
            if not r["pending"]:
                continue
            if r["cached"] // self.P >= r["pages"]:
                if not self._alloc():
                    continue
                r["pages"] += 1
            rows.append((rid, r["cached"], 1))
            r["cached"] += 1
            r["pending"] = False
        return rows

    def finish(self, rid):
        r = self.reqs.pop(rid)
        if r["state"] == "running":
            self.running.remove(rid)
        else:
            self.queue.remove(rid)
        if r["state"] == "waiting":
            return
        self.clock += 1
        private = r["pages"] - len(r["matched"])
        taken = 0
        if self.radix:
            for j in range(1, r["cached"] // self.P + 1):
                key = tuple(r["tokens"][:j * self.P])
                if key in self.cache:
                    self.cache[key][0] = self.clock
                else:
                    self.cache[key] = [self.clock, 0]
                    taken += 1
            for key in r["matched"]:
                self.cache[key][1] -= 1
        self.free += private - taken

    def stats(self) -> dict:
        locked = sum(1 for _, locks in self.cache.values() if locks > 0)
        private = sum(r["pages"] - len(r["matched"]) for r in self.reqs.values())
        return dict(free_pages=self.free, cached_pages=len(self.cache), locked_pages=locked,
                    private_pages=private, evicted_pages=self.evicted,
                    waiting=sum(1 for q in self.queue if self.reqs[q]["state"] == "waiting"),
                    prefilling=sum(1 for q in self.queue if self.reqs[q]["state"] == "prefilling"),
                    running=len(self.running))


def longest_cached_prefix_bruteforce(tokens, history, page_size: int) -> int:
    """Closed form of the match when nothing was ever evicted: the longest common
    prefix, in whole pages and capped at len(tokens) - 1, between `tokens` and any
    stored token sequence in `history` (each the stored part of a finished request)."""
    best = 0
    cap = (len(tokens) - 1) // page_size * page_size
    for seq in history:
        full = len(seq) // page_size * page_size
        n = 0
        while n < min(cap, full) and tokens[n] == seq[n]:
            n += 1
        best = max(best, n // page_size * page_size)
    return best
