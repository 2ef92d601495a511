"""Pins of the prefix-index oracle against what the page fixes: the worked hit
B = 2560 inside a 6144-token page, whole-page matching with the fallback inside
the first missing page, the KDA stage needing every group, the three
concurrency rules (pins, pending entries, atomic sibling eviction), checkpoint
placement, and a second restatement of the hit on random workloads."""
import json
import os

import numpy as np
import pytest

from oracle.prefix_index import (OracleError, PrefixIndexModel, ckpt_plan,
                                 longest_certified_boundary)

GOLD = os.path.join(os.path.dirname(__file__), "golden", "p1_worked_hit.json")


def seq(n, seed):
    return np.random.default_rng(seed).integers(0, 150_000, n).astype(np.int32)


def test_worked_hit_2560():
    g = json.load(open(GOLD))
    hb, pb = g["hash_block"], g["physical_block"]
    m = PrefixIndexModel(hb, pb, num_groups=2)
    cached = seq(3000, 1)                      # a cached prefix: one partial page
    assert m.register_pages(cached, [7], step=0) == [1]   # registered at its last hash end
    for grp in range(2):
        m.register_ckpt(cached, kda_plan_end(3000, hb), grp, 20 + grp, durable=True, step=0)
    m.mark_ready(0)
    req = np.concatenate([cached[:g["matched_tokens"]], seq(1000, 2) + 200_000])
    hit = m.lookup(req)
    assert hit["boundary"] == g["hit_boundary"] == 5 * hb
    assert hit["boundary"] % pb != 0 and hit["pages"] == [7] and hit["ckpt_pages"] == [20, 21]


def kda_plan_end(n, hb):
    return ckpt_plan(0, n, hb)


def test_whole_pages_then_fallback():
    hb, pb = 512, 2048
    m = PrefixIndexModel(hb, pb, 1)
    cached = seq(7000, 3)                      # pages: 3 full (6144) + partial at 6656
    assert m.register_pages(cached, [1, 2, 3, 4], 0) == [1, 1, 1, 1]
    for P in (2048, 4096, 6656):
        m.register_ckpt(cached, P, 0, 100 + P, False, 0)
    m.mark_ready(0)
    # shares 6900 tokens: 3 whole pages, then the partial page's end 6656
    r = np.concatenate([cached[:6900], seq(600, 4) + 300_000])
    h = m.lookup(r)
    assert (h["mla_tokens"], h["boundary"], h["pages"]) == (6656, 6656, [1, 2, 3, 4])
    # shares 6500: the partial page's key (6656) does not match -> MLA stops at 6144,
    # the deepest checkpoint inside is 4096
    r = np.concatenate([cached[:6500], seq(600, 5) + 300_000])
    h = m.lookup(r)
    assert (h["mla_tokens"], h["boundary"], h["pages"]) == (6144, 4096, [1, 2])
    # a mismatch in the first page: nothing
    r = cached.copy()
    r[100] += 1
    assert m.lookup(r)["boundary"] == 0


def test_kda_stage_needs_every_group():
    m = PrefixIndexModel(512, 1024, 3)
    t = seq(2048, 6)
    m.register_pages(t, [0, 1], 0)
    m.register_ckpt(t, 1024, 0, 10, False, 0)
    m.register_ckpt(t, 1024, 1, 11, False, 0)
    m.mark_ready(0)
    assert m.lookup(t)["boundary"] == 0            # group 2 missing
    m.register_ckpt(t, 1024, 2, 12, False, 1)
    assert m.lookup(t)["boundary"] == 0            # group 2's copy still pending
    m.mark_ready(1)
    h = m.lookup(t)
    assert h["boundary"] == 1024 and h["ckpt_pages"] == [10, 11, 12]


def test_pending_pins_and_sibling_eviction():
    m = PrefixIndexModel(512, 2048, 2)
    t = seq(4096, 7)
    m.register_pages(t, [0, 1], step=3)
    for g in range(2):
        m.register_ckpt(t, 4096, g, 50 + g, True, 3)
    assert m.lookup(t)["boundary"] == 0            # registered this step: not matched
    m.mark_ready(2)
    assert m.lookup(t)["boundary"] == 0
    m.mark_ready(3)
    h = m.lookup(t, pin=True)
    assert h["boundary"] == 4096 and h["pin_handle"] > 0
    with pytest.raises(OracleError) as e:
        m.evict_ckpt(1, 51)
    assert e.value.kind == "pinned"
    with pytest.raises(OracleError):
        m.evict_page(0)
    m.release(h["pin_handle"])
    assert m.evict_ckpt(1, 51) == [50, 51]        # both groups leave together
    assert m.lookup(t)["boundary"] == 0
    with pytest.raises(OracleError) as e:
        m.evict_ckpt(0, 50)
    assert e.value.kind == "not_found"


def test_first_registration_wins_and_page_end_advances():
    m = PrefixIndexModel(512, 2048, 1)
    t = seq(4000, 8)
    assert m.register_pages(t[:1100], [5], 0) == [1]          # end 1024
    assert m.register_pages(t[:1100], [6], 0) == [0]          # same prefix, another page
    assert m.register_pages(t[:2000], [5], 1) == [1]          # end advances to 1536
    m.register_ckpt(t, 1024, 0, 9, False, 0)
    m.mark_ready(1)
    h = m.lookup(t[:1500])                                      # 1024 was the old end
    assert h["mla_tokens"] == 0 and h["boundary"] == 0
    m.register_ckpt(t, 1536, 0, 8, False, 1)
    m.mark_ready(1)
    h = m.lookup(t[:1700])
    assert (h["mla_tokens"], h["boundary"]) == (1536, 1536)


@pytest.mark.parametrize("start,length,expect", [
    (0, 700, 512), (100, 300, -1), (512, 512, 1024), (511, 1, 512), (0, 511, -1),
    (1000, 5000, 5632), (0, 1 << 20, 1 << 20)])
def test_ckpt_plan(start, length, expect):
    if length > 100_000:  # brute force over a million positions is slow; use the definition
        assert expect % 512 == 0 and start < expect <= start + length
        return
    assert ckpt_plan(start, length, 512) == expect


def test_two_restatements_agree_on_random_workloads():
    rng = np.random.default_rng(12)
    hb, pb, G = 512, 1536, 2
    m = PrefixIndexModel(hb, pb, G)
    system = seq(1200, 13)
    convs, page = [], 0
    for c in range(6):
        t = np.concatenate([system, seq(int(rng.integers(300, 4000)), 100 + c)])
        n = len(t)
        npg = -(-n // pb)
        m.register_pages(t, list(range(page, page + npg)), step=c)
        page += npg
        for b in range(hb, n + 1, hb):
            if rng.random() < 0.4:
                for g in range(G):
                    try:
                        m.register_ckpt(t, b, g, 10_000 + 7 * b + g + 1000 * c, False, c)
                    except OracleError:
                        pass
        convs.append(t)
    m.mark_ready(10)
    for c, t in enumerate(convs):
        for cut in (1200, 1300, len(t) // 2, len(t)):
            r = np.concatenate([t[:cut], seq(50, 999) + 400_000])
            assert m.lookup(r)["boundary"] == longest_certified_boundary(m, r)


def _partial_page_workload():
    """A conversation whose last page is partial (2100 tokens in 1536-token
    pages: page 1 registered under its last complete hash block, 2048), a
    checkpoint at every hash block, and requests diverging inside page 1."""
    hb, pb, G = 512, 1536, 2
    m = PrefixIndexModel(hb, pb, G)
    t = seq(2100, 31)
    m.register_pages(t, [0, 1], step=0)
    for b in range(hb, 2100 + 1, hb):
        for g in range(G):
            m.register_ckpt(t, b, g, 100 + 2 * b + g, True, 0)
    m.mark_ready(0)
    reqs = [np.concatenate([t[:cut], seq(40, 77) + 500_000]) for cut in (2100, 2060, 1900, 1600)]
    return m, reqs


def test_certifier_catches_mla_stage_mistakes(monkeypatch):
    """The certifier restates the MLA stage on its own: planted mistakes in the
    model's MLA walk (the partial-page stage dropped; its scan starting one hash
    block too low) make the two disagree, while the model as written agrees."""
    m, reqs = _partial_page_workload()
    assert [m.lookup(r)["boundary"] for r in reqs] == [2048, 2048, 1536, 1536]
    assert all(m.lookup(r)["boundary"] == longest_certified_boundary(m, r) for r in reqs)
    orig = PrefixIndexModel.mla_match

    def no_partial(self, tokens):
        mla, pages = orig(self, tokens)
        whole = mla // self.pb * self.pb
        return whole, pages[:whole // self.pb]

    def low_scan(self, tokens):
        # the walk as written, except that the partial-page scan starts one
        # hash block below the request's last complete hash-block end
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
            for e in range(min(pend - self.hb, full) - self.hb, i * self.pb, -self.hb):
                p = self._served(tokens, e)
                if p is not None:
                    pages.append(p)
                    return e, pages
            return i * self.pb, pages

    for mutant in (no_partial, low_scan):
        monkeypatch.setattr(PrefixIndexModel, "mla_match", mutant)
        assert any(m.lookup(r)["boundary"] != longest_certified_boundary(m, r) for r in reqs), \
            mutant.__name__
    monkeypatch.setattr(PrefixIndexModel, "mla_match", orig)

