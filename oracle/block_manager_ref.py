"""Plain Python model of the Block Manager (test infrastructure only).

MapFlow organises its cache of compressed attention state with a Block
Manager that indexes it by prefix hashes, each key carrying the information of
all preceding context (paper page montaan.com/papers/2610.14688, "Practical
Implementation Details"; article aitest123.com/news/zaoi86, third section,
second component).  This model states the index's behaviour in the plainest
code: dictionaries, a sorted free list and a linear search for the least
recently used row.  The library's manager must agree with it call for call
(statuses, returned rows and pages, statistics).

Readings (the pages give no index layout, hash function, page policy or
eviction rule; these are the plainest choices):
  * block row I of a sender layer depends on tokens 0 .. (I+1)B-1 only, so it
    is keyed by (layer, h_{I+1}) with the chained prefix hash
        h_0 = seed,  h_{c+1} = FNV-1a-64(h_c as 8 LE bytes ++ chunk tokens as 4 LE bytes each);
  * only full chunks are cached;
  * an entry keeps its parent hash and chunk tokens, and a lookup compares
    both, so a collision can only make a row look absent;
  * pages are handed out smallest index first; rows held by a lookup are
    never evicted; otherwise the least recently used row goes first (a lookup
    or an insert that meets a row counts as a use); an insert that cannot get
    its pages even by evicting every unheld row fails without evicting any.
"""
from __future__ import annotations

FNV_OFFSET = 14695981039346656037
FNV_PRIME = 1099511628211
MASK = (1 << 64) - 1

OK, INVALID, CAPACITY = 0, 1, 3


def fnv1a64(data: bytes, h: int = FNV_OFFSET) -> int:
    """FNV-1a, 64 bits: for each byte, xor it in, then multiply by the prime."""
    for b in data:
        h ^= b
        h = (h * FNV_PRIME) & MASK
    return h


def chain(parent: int, chunk) -> int:
    data = int(parent).to_bytes(8, "little")
    for t in chunk:
        data += (int(t) & 0xFFFFFFFF).to_bytes(4, "little")
    return fnv1a64(data)


def prefix_hashes(tokens, B: int, seed: int = 0) -> list:
    out, h = [], seed
    for c in range(len(tokens) // B):
        h = chain(h, tokens[c * B:(c + 1) * B])
        out.append(h)
    return out


class BlockManagerRef:
    def __init__(self, B: int, n_layers: int, n_pages: int, seed: int = 0):
        self.B, self.n_layers, self.seed = B, n_layers, seed
        self.rows = {}                       # (layer, h) -> entry dict
        self.free = list(range(n_pages))     # kept sorted
        self.clock = 0
        self.hits = self.misses = self.evictions = self.inserted = 0

    # -- helpers ---------------------------------------------------------------
    def _use(self, e):
        self.clock += 1
        e["stamp"] = self.clock

    def _evict_one(self) -> bool:
        cands = [(e["stamp"], k) for k, e in self.rows.items() if e["refs"] == 0]
        if not cands:
            return False
        _, k = min(cands)
        self.free.extend(self.rows.pop(k)["pages"])
        self.free.sort()
        self.evictions += 1
        return True

    def _take_page(self) -> int:
        return self.free.pop(0)

    def _find(self, layer, parent, chunk):
        e = self.rows.get((layer, chain(parent, chunk)))
        if e is None or e["parent"] != parent or e["tokens"] != tuple(int(t) for t in chunk):
            return None
        return e

    # -- operations --------------------------------------------------------------
    def lookup(self, layer, tokens, max_rows, cap):
        """(status, n_rows, row_ptr, cols, pages)"""
        if not 0 <= layer < self.n_layers or max_rows < 0 or cap < 0:
            return INVALID, 0, [0], [], []
        chunks = min(len(tokens) // self.B, max_rows)
        hit, h = [], self.seed
        for c in range(chunks):
            chunk = tokens[c * self.B:(c + 1) * self.B]
            e = self._find(layer, h, chunk)
            if e is None:
                break
            hit.append(e)
            h = chain(h, chunk)
        if sum(len(e["cols"]) for e in hit) > cap:
            return CAPACITY, len(hit), [0], [], []
        row_ptr, cols, pages = [0], [], []
        for e in hit:
            cols += e["cols"]
            pages += e["pages"]
            row_ptr.append(len(cols))
            self._use(e)
            e["refs"] += 1
        self.hits += len(hit)
        self.misses += chunks - len(hit)
        return OK, len(hit), row_ptr, cols, pages

    def release(self, layer, tokens, n_rows):
        if not 0 <= layer < self.n_layers or n_rows < 0 or n_rows * self.B > len(tokens):
            return INVALID
        es, h = [], self.seed
        for c in range(n_rows):
            chunk = tokens[c * self.B:(c + 1) * self.B]
            e = self.rows.get((layer, chain(h, chunk)))
            if e is None or e["refs"] <= 0:
                return INVALID
            es.append(e)
            h = chain(h, chunk)
        for e in es:
            e["refs"] -= 1
        return OK

    def insert(self, layer, tokens, row0, row_ptr, cols):
        """(status, pages_out)"""
        n_rows = len(row_ptr) - 1
        if not 0 <= layer < self.n_layers or row0 < 0 or n_rows < 0 or \
                (row0 + n_rows) * self.B > len(tokens) or row_ptr[0] != 0:
            return INVALID, None
        for i in range(n_rows):
            if row_ptr[i + 1] < row_ptr[i]:
                return INVALID, None
            rc = cols[row_ptr[i]:row_ptr[i + 1]]
            if any(c < 0 or c > row0 + i for c in rc) or any(b <= a for a, b in zip(rc, rc[1:])):
                return INVALID, None
        hs = [self.seed]
        for c in range(row0 + n_rows):
            hs.append(chain(hs[-1], tokens[c * self.B:(c + 1) * self.B]))
        fresh, need, existing = [], 0, []
        for i in range(n_rows):
            e = self.rows.get((layer, hs[row0 + i + 1]))
            fresh.append(e is None)
            if e is None:
                need += row_ptr[i + 1] - row_ptr[i]
            else:
                existing.append(e)
        for e in existing:                    # used again now, and held while room is made
            self._use(e)
            e["refs"] += 1
        evictable = sum(len(e["pages"]) for e in self.rows.values() if e["refs"] == 0)
        ok = len(self.free) + evictable >= need     # otherwise evict nothing
        while ok and len(self.free) < need:
            self._evict_one()
        for e in existing:
            e["refs"] -= 1
        if not ok:
            return CAPACITY, None
        out = [-1] * row_ptr[-1]
        for i in range(n_rows):
            if not fresh[i]:
                continue
            c = row0 + i
            pages = []
            for k in range(row_ptr[i], row_ptr[i + 1]):
                out[k] = self._take_page()
                pages.append(out[k])
            self.clock += 1
            self.rows[(layer, hs[c + 1])] = dict(
                parent=hs[c], tokens=tuple(int(t) for t in tokens[c * self.B:(c + 1) * self.B]),
                cols=list(cols[row_ptr[i]:row_ptr[i + 1]]), pages=pages, refs=0, stamp=self.clock)
            self.inserted += 1
        return OK, out

    def stats(self) -> dict:
        return dict(free_pages=len(self.free), cached_rows=len(self.rows),
                    held_rows=sum(e["refs"] > 0 for e in self.rows.values()),
                    hits=self.hits, misses=self.misses, evictions=self.evictions,
                    inserted=self.inserted)
