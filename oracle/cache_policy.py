"""Plain Python model of the paged KV pool manager (test infrastructure).

The reference that the native manager (lazyattn_cache_*) is checked against,
operation by operation.  It follows the pages, with the readings below where
they are silent:

* [KVF] "PagedAttention": the cache is made of 16-token blocks; a table maps
  a sequence's logical positions to physical blocks.
* [KVF] "Exercícios" 3: a list of free blocks; a finished sequence's blocks go
  back to the pool.
* [LA] "Declaração do Problema", "Metodologia": a position-aware cache reuses
  a document only at the position it was encoded for (another placement needs
  another copy); the position-agnostic cache stores the document by content
  once and reuses it at any position.  Prefix caching reuses a document only
  when everything before it matches too.

Readings (the pages give no allocator details nor an eviction policy):

* Free blocks form a stack; the pool starts as [0, 1, 2, ...] from the top, a
  request takes blocks from the top in order, and freed blocks are pushed
  back so that the lowest of them is on top again.
* Eviction happens only when a request needs more blocks than are free, and
  takes cached documents that no live request references, in the order their
  last reference was dropped (least recently used first).
* Within one request, cached documents are referenced first; then the missing
  ones are allocated in request order (a document missing twice in one
  request is allocated once); then the prompt.  A request that cannot be
  placed changes nothing.
* A document's length is part of its identity (it is stored once, by
  content): naming a cached document, or one named earlier in the same
  request, with another length is an argument error, and changes nothing.
* Frame starts (the table word's high 16 bits) are the document's placement
  position (the running sum of the lengths before it) and, for the prompt,
  the first position after the documents; every position must be < 65536.
"""

BLOCK = 16
MAX_POSITION = 65535
AGNOSTIC, AWARE, PREFIX = 0, 1, 2


class NoSpace(Exception):
    pass


class BadPosition(Exception):
    pass


class BadArgument(Exception):
    pass


class CachePolicyModel:
    def __init__(self, num_blocks, mode):
        assert 1 <= num_blocks <= 65536 and mode in (AGNOSTIC, AWARE, PREFIX)
        self.num_blocks = num_blocks
        self.mode = mode
        self.free = list(range(num_blocks - 1, -1, -1))   # top of the stack = end of the list
        self.docs = {}        # key -> {"blocks": [...], "refs": int}
        self.unreferenced = []  # keys with refs == 0, oldest first
        self.requests = {}
        self.next_id = 0
        self.counts = dict(requests=0, doc_hits=0, doc_misses=0, tokens_hit=0, tokens_missed=0,
                           evicted=0)

    def key(self, ids, i, pos):
        if self.mode == AGNOSTIC:
            return (ids[i],)
        if self.mode == AWARE:
            return (ids[i], pos)
        return tuple(ids[: i + 1])

    def _take(self, k):
        d = self.docs[k]
        if d["refs"] == 0:
            self.unreferenced.remove(k)
        d["refs"] += 1

    def _room(self, n):
        while len(self.free) < n:
            k = self.unreferenced.pop(0)
            blocks = self.docs.pop(k)["blocks"]
            self.free.extend(reversed(blocks))
            self.counts["evicted"] += 1

    def _alloc(self, n):
        return [self.free.pop() for _ in range(n)]

    def acquire(self, ids, lens, prompt_len, max_blocks):
        ids, lens = list(ids), list(lens)
        for L in lens:
            assert L > 0 and L % BLOCK == 0
        pos, p = [], 0
        for L in lens:
            if p > MAX_POSITION:
                raise BadPosition()
            pos.append(p)
            p += L
        if prompt_len > 0 and p > MAX_POSITION:
            raise BadPosition()
        if p + prompt_len > MAX_POSITION + 1:
            raise BadPosition()
        keys = [self.key(ids, i, pos[i]) for i in range(len(ids))]
        prompt_nb = -(-prompt_len // BLOCK)
        if sum(L // BLOCK for L in lens) + prompt_nb > max_blocks:
            raise NoSpace()
        named = {}
        for k, L in zip(keys, lens):
            nb = L // BLOCK
            if k in self.docs and len(self.docs[k]["blocks"]) != nb:
                raise BadArgument()
            if named.setdefault(k, nb) != nb:
                raise BadArgument()
        # will it fit?  blocks to allocate against free + evictable-but-not-hit
        hit = {k for k in keys if k in self.docs}
        new, need = set(), prompt_nb
        for k, L in zip(keys, lens):
            if k not in self.docs and k not in new:
                new.add(k)
                need += L // BLOCK
        avail = len(self.free) + sum(len(self.docs[k]["blocks"]) for k in self.unreferenced
                                     if k not in hit)
        if need > avail:
            raise NoSpace()
        miss = [0] * len(ids)
        placed = [False] * len(ids)
        for i, k in enumerate(keys):
            if k in self.docs:
                self._take(k)
                placed[i] = True
        for i, k in enumerate(keys):
            if placed[i]:
                continue
            if k in self.docs:
                self._take(k)
                continue
            nb = lens[i] // BLOCK
            self._room(nb)
            self.docs[k] = {"blocks": self._alloc(nb), "refs": 1}
            miss[i] = 1
        self._room(prompt_nb)
        prompt = self._alloc(prompt_nb)
        row = []
        for i, k in enumerate(keys):
            row += [b | (pos[i] << 16) for b in self.docs[k]["blocks"]]
            if miss[i]:
                self.counts["doc_misses"] += 1
                self.counts["tokens_missed"] += lens[i]
            else:
                self.counts["doc_hits"] += 1
                self.counts["tokens_hit"] += lens[i]
        row += [b | (p << 16) for b in prompt]
        self.counts["requests"] += 1
        rid = self.next_id
        self.next_id += 1
        self.requests[rid] = (keys, prompt)
        return row, miss, rid

    def release(self, rid):
        keys, prompt = self.requests.pop(rid)
        for k in keys:
            d = self.docs[k]
            d["refs"] -= 1
            if d["refs"] == 0:
                self.unreferenced.append(k)
        self.free.extend(reversed(prompt))

    def stats(self):
        s = dict(self.counts)
        s["free_blocks"] = len(self.free)
        s["doc_blocks"] = sum(len(d["blocks"]) for d in self.docs.values())
        s["prompt_blocks"] = sum(len(p) for _, p in self.requests.values())
        s["cached_docs"] = len(self.docs)
        return s
