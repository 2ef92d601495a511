"""Oracle of the host prefix index: the two-stage lookup by brute force.

TEST INFRASTRUCTURE ONLY (same rule as the rest of ``oracle/``): only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may import it;
the product path never does, and the two share no code.

Page "Cache de préfixe hybride KDA–MLA" (mkdocs.reaper.mx):
- "Le fonctionnement du prefill": a page is registered under its last complete
  hash block, and that end advances as the page fills; the KDA state is
  persisted at the last hash-aligned position a pass processed.
- "La recherche en deux étages": MLA matches whole physical pages, then the
  hash-block ends inside the first missing page; KDA needs a checkpoint at the
  candidate boundary in every group; the hit is the longest boundary passing
  both.
- "La cohérence sous ordonnancement concurrent": hits are pinned; entries
  registered in the current step are not matched until marked ready; a
  checkpoint is evicted from every group at once.

The library identifies a prefix by chained hashes; this model identifies it
by the token prefix itself (tuples compared element by element), so it
certifies what the hashes are meant to certify.  Readings shared with the
library: first registration wins; a page holds one key (its current end); a
boundary may equal the request length.
"""
from __future__ import annotations


class OracleError(Exception):
    def __init__(self, kind: str):
        super().__init__(kind)
        self.kind = kind  # "pinned" | "not_found" | "alias"


class PrefixIndexModel:
    def __init__(self, hash_block: int, physical_block: int, num_groups: int):
        assert physical_block % hash_block == 0
        self.hb, self.pb, self.groups = hash_block, physical_block, num_groups
        self.pages = {}       # page -> {"prefix": tuple, "step": s, "ready": bool}
        self.ckpts = {}       # prefix tuple -> {"pages": [..], "step", "ready", "durable", "pins"}
        self.page_pins = {}   # page -> count
        self.pins = {}        # handle -> (pages, prefix)
        self.next_pin = 1

    # -- registration -------------------------------------------------------
    def _holder(self, prefix):
        for page, e in self.pages.items():
            if e["prefix"] == prefix:
                return page
        return None

    def register_pages(self, tokens, pages, step):
        tokens = tuple(int(t) for t in tokens)
        n = len(tokens)
        assert len(pages) == -(-n // self.pb)
        full = n // self.hb * self.hb
        taken = []
        for i, page in enumerate(pages):
            end = min((i + 1) * self.pb, full)
            if end <= i * self.pb:
                taken.append(0)
                continue
            prefix = tokens[:end]
            holder = self._holder(prefix)
            if holder is not None:
                taken.append(1 if holder == page else 0)
                continue
            self.pages[page] = {"prefix": prefix, "step": step, "ready": False}
            taken.append(1)
        return taken

    def register_ckpt(self, tokens, pos, group, page, durable, step):
        assert pos > 0 and pos % self.hb == 0
        prefix = tuple(int(t) for t in tokens[:pos])
        for other, c in self.ckpts.items():
            if other != prefix and c["pages"][group] == page:
                raise OracleError("alias")
        c = self.ckpts.setdefault(prefix, {"pages": [-1] * self.groups, "step": step,
                                           "ready": False, "durable": False, "pins": 0})
        if c["pages"][group] >= 0:
            taken = c["pages"][group] == page
        else:
            c["pages"][group] = page
            c["step"] = max(c["step"], step)
            c["ready"] = False
            taken = True
        c["durable"] = c["durable"] or bool(durable)
        return taken

    def mark_ready(self, step):
        for e in self.pages.values():
            if e["step"] <= step:
                e["ready"] = True
        for c in self.ckpts.values():
            if c["step"] <= step:
                c["ready"] = True

    # -- lookup -------------------------------------------------------------
    def _served(self, tokens, end):
        """A ready page registered with exactly the prefix tokens[0:end]."""
        prefix = tuple(tokens[:end])
        for page, e in self.pages.items():
            if e["ready"] and e["prefix"] == prefix:
                return page
        return None

    def mla_match(self, tokens):
        """(matched tokens, pages) of the MLA stage."""
        n = len(tokens)
        full = n // self.hb * self.hb
        pages, i = [], 0
        while True:
            pend = (i + 1) * self.pb
            if pend <= full:
                p = self._served(tokens, pend)
                if p is not None:
                    pages.append(p)
                    i += 1
                    continue
            for e in range(min(pend - self.hb, full), i * self.pb, -self.hb):
                p = self._served(tokens, e)
                if p is not None:
                    pages.append(p)
                    return e, pages
            return i * self.pb, pages

    def _ckpt_ready(self, tokens, b):
        c = self.ckpts.get(tuple(tokens[:b]))
        return c if c is not None and c["ready"] and min(c["pages"]) >= 0 else None

    def lookup(self, tokens, pin=False):
        tokens = tuple(int(t) for t in tokens)
        mla, pages = self.mla_match(tokens)
        boundary, ck = 0, None
        for b in range(mla, 0, -self.hb):
            c = self._ckpt_ready(tokens, b)
            if c is not None:
                boundary, ck = b, c
                break
        np_ = -(-boundary // self.pb)
        out = {"boundary": boundary, "mla_tokens": mla, "pages": pages[:np_],
               "ckpt_pages": list(ck["pages"]) if ck else [-1] * self.groups, "pin_handle": 0}
        if pin and ck is not None:
            h = self.next_pin
            self.next_pin += 1
            for p in out["pages"]:
                self.page_pins[p] = self.page_pins.get(p, 0) + 1
            ck["pins"] += 1
            self.pins[h] = (list(out["pages"]), tuple(tokens[:boundary]))
            out["pin_handle"] = h
        return out

    def release(self, handle):
        if handle not in self.pins:
            raise OracleError("not_found")
        pages, prefix = self.pins.pop(handle)
        for p in pages:
            self.page_pins[p] -= 1
            if self.page_pins[p] == 0:
                del self.page_pins[p]
        if prefix in self.ckpts:
            self.ckpts[prefix]["pins"] -= 1

    # -- eviction -----------------------------------------------------------
    def evict_page(self, page):
        if page not in self.pages:
            raise OracleError("not_found")
        if self.page_pins.get(page, 0) > 0:
            raise OracleError("pinned")
        del self.pages[page]

    def evict_ckpt(self, group, page):
        for prefix, c in self.ckpts.items():
            if c["pages"][group] == page:
                if c["pins"] > 0:
                    raise OracleError("pinned")
                del self.ckpts[prefix]
                return list(c["pages"])
        raise OracleError("not_found")

    def stats(self):
        return len(self.pages), len(self.ckpts), len(self.pins)


def ckpt_plan(start, length, hash_block):
    """Last multiple of hash_block in (start, start+length], or -1."""
    best = -1
    for p in range(start + 1, start + length + 1):
        if p % hash_block == 0:
            best = p
    return best


def longest_certified_boundary(model: PrefixIndexModel, tokens):
    """Independent restatement of the hit, for pins: the largest b (multiple of
    the hash block, b <= n) such that

    (1) MLA covers tokens[0:b]: with R the set of lengths L for which a ready
        page is registered under exactly tokens[0:L], every whole physical page
        before the one holding token b-1 ends in R (k * pb in R for
        k = 1 .. i, i = (b-1) // pb), and some hash-block end e in R lies in
        page i at or after b (b <= e <= min((i+1) * pb, full), full = the
        request's last hash-block end);
    (2) a complete ready checkpoint holds exactly tokens[0:b].

    Computed from the registered entries directly (R by scanning every page
    entry; candidates by scanning every checkpoint), sharing no code with the
    model's lookup walk."""
    tokens = tuple(int(t) for t in tokens)
    n = len(tokens)
    hb, pb = model.hb, model.pb
    full = n // hb * hb
    R = set()
    for e in model.pages.values():
        L = len(e["prefix"])
        if e["ready"] and 0 < L <= n and tokens[:L] == e["prefix"]:
            R.add(L)

    def covered(b):
        i = (b - 1) // pb
        if any(k * pb not in R for k in range(1, i + 1)):
            return False
        top = min((i + 1) * pb, full)
        return any(e in R for e in range(b, top + 1) if e % hb == 0)

    best = 0
    for prefix, c in model.ckpts.items():
        b = len(prefix)
        if (c["ready"] and min(c["pages"]) >= 0 and 0 < b <= n and b % hb == 0
                and tokens[:b] == prefix and b > best and covered(b)):
            best = b
    return best
