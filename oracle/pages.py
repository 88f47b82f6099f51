"""Plain Python model of the host page allocator (the C++ one in the library), for the tests.

TEST INFRASTRUCTURE ONLY: it shares no code with the library.  Everything is a dict or a list,
with the rules stated once, so that a reader can check it by eye:

* a page's reference count is the number of sequences listing it plus one if the prefix cache
  holds it; count 0 means free; the lowest free id is taken first;
* forking copies the page list and the length, adding one reference per page;
* growing a sequence by n tokens: if its last page is partly filled and shared, that page is
  replaced by a fresh one (reported as a copy (old, fresh)); then fresh pages cover the new
  length; with too few free pages nothing changes (an error);
* the prefix cache is a tree keyed by (parent node, the page's token ids); insert adds missing
  nodes with a cache reference to the sequence's page; lookup follows equal keys from the root;
  eviction removes least recently used leaves whose page only the cache holds.

(CacheIR page, "Current Capabilities": shared page allocator accounting across forked request
sessions; TorchInferno page, "Runtime Scaffolds": runtime.paged, runtime.prefix radix prefix tree,
runtime.prefix_cache lookup.)
"""
from __future__ import annotations


class OutOfPages(Exception):
    pass


class PageModel:
    def __init__(self, num_pages: int, page_size: int):
        self.ps = page_size
        self.refs = [0] * num_pages
        self.seqs = {}              # id -> [pages, length]
        self.free_ids = []          # released sequence ids, reused last-in first-out
        self.next_id = 0
        self.nodes = []             # [parent, tokens tuple, page, last_use, children, alive]
        self.index = {}             # (parent, tokens) -> node
        self.clock = 0

    # pages
    def free_count(self):
        return sum(1 for r in self.refs if r == 0)

    def _take(self):
        for p, r in enumerate(self.refs):
            if r == 0:
                self.refs[p] = 1
                return p
        raise OutOfPages

    # sequences
    def _new_seq(self):
        if self.free_ids:
            sid = self.free_ids.pop()
        else:
            sid = self.next_id
            self.next_id += 1
        self.seqs[sid] = [[], 0]
        return sid

    def create(self):
        return self._new_seq()

    def fork(self, src):
        pages, length = self.seqs[src]
        sid = self._new_seq()
        self.seqs[sid] = [list(pages), length]
        for p in pages:
            self.refs[p] += 1
        return sid

    def release(self, sid):
        for p in self.seqs.pop(sid)[0]:
            self.refs[p] -= 1
        self.free_ids.append(sid)

    def reserve(self, sid, n):
        pages, length = self.seqs[sid]
        new_len = length + n
        need = -(-new_len // self.ps)
        cow = n > 0 and length % self.ps != 0 and self.refs[pages[-1]] > 1
        if (need - len(pages)) + (1 if cow else 0) > self.free_count():
            raise OutOfPages
        copies = []
        if cow:
            old = pages[-1]
            fresh = self._take()
            self.refs[old] -= 1
            pages[-1] = fresh
            copies.append((old, fresh))
        while len(pages) < need:
            pages.append(self._take())
        self.seqs[sid][1] = new_len
        return copies

    def table(self, sid):
        return list(self.seqs[sid][0])

    def length(self, sid):
        return self.seqs[sid][1]

    # prefix cache
    def prefix_insert(self, sid, tokens):
        pages = self.seqs[sid][0]
        self.clock += 1
        parent = -1
        for i in range(len(tokens) // self.ps):
            key = (parent, tuple(tokens[i * self.ps:(i + 1) * self.ps]))
            node = self.index.get(key)
            if node is None:
                node = len(self.nodes)
                self.nodes.append([parent, key[1], pages[i], self.clock, 0, True])
                if parent >= 0:
                    self.nodes[parent][4] += 1
                self.index[key] = node
                self.refs[pages[i]] += 1
            else:
                self.nodes[node][3] = self.clock
            parent = node

    def create_with_prefix(self, tokens):
        sid = self._new_seq()
        self.clock += 1
        parent, pages = -1, []
        for i in range(len(tokens) // self.ps):
            node = self.index.get((parent, tuple(tokens[i * self.ps:(i + 1) * self.ps])))
            if node is None:
                break
            self.nodes[node][3] = self.clock
            pages.append(self.nodes[node][2])
            self.refs[self.nodes[node][2]] += 1
            parent = node
        self.seqs[sid] = [pages, len(pages) * self.ps]
        return sid, len(pages) * self.ps

    def evict(self, max_pages):
        done = 0
        while done < max_pages:
            cands = [n for n, x in enumerate(self.nodes)
                     if x[5] and x[4] == 0 and self.refs[x[2]] == 1]
            if not cands:
                break
            best = min(cands, key=lambda n: (self.nodes[n][3], n))
            x = self.nodes[best]
            del self.index[(x[0], x[1])]
            if x[0] >= 0:
                self.nodes[x[0]][4] -= 1
            self.refs[x[2]] -= 1
            x[5] = False
            done += 1
        return done
