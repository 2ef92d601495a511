// kda_index.cpp -- host prefix index: chained hash-block hashes, MLA page
// entries whose registered end advances, KDA checkpoints held in every cache
// group or in none, the two-stage lookup, pins, and the pending state of
// entries whose copies have not completed.
//
// Page "Cache de préfixe hybride KDA–MLA" (mkdocs.reaper.mx), sections
// "Le fonctionnement du prefill", "La recherche en deux étages",
// "La cohérence sous ordonnancement concurrent" and "Vérification de
// compréhension" (chained hashing).  The library's readings where the page is
// silent are listed in include/kda_index.h.
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <unordered_map>
#include <vector>

#include "../../include/kda_index.h"

namespace kda {
void host_set_error(const char* msg);
void host_clear_error();
}  // namespace kda

namespace {

kda_status fail(kda_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  kda::host_set_error(buf);
  return st;
}

kda_status ok() {
  kda::host_clear_error();
  return KDA_OK;
}

// ---- XXH64, from the xxHash specification (64-bit variant) -----------------
constexpr uint64_t kP1 = 0x9E3779B185EBCA87ULL;
constexpr uint64_t kP2 = 0xC2B2AE3D27D4EB4FULL;
constexpr uint64_t kP3 = 0x165667B19E3779F9ULL;
constexpr uint64_t kP4 = 0x85EBCA77C2B2AE63ULL;
constexpr uint64_t kP5 = 0x27D4EB2F165667C5ULL;

inline uint64_t rotl(uint64_t x, int r) { return (x << r) | (x >> (64 - r)); }
inline uint64_t rd64(const uint8_t* p) {  // little-endian host
  uint64_t v;
  std::memcpy(&v, p, 8);
  return v;
}
inline uint32_t rd32(const uint8_t* p) {
  uint32_t v;
  std::memcpy(&v, p, 4);
  return v;
}
inline uint64_t lane_round(uint64_t acc, uint64_t lane) {
  acc += lane * kP2;
  acc = rotl(acc, 31);
  return acc * kP1;
}
inline uint64_t merge_round(uint64_t acc, uint64_t v) {
  acc ^= lane_round(0, v);
  return acc * kP1 + kP4;
}

uint64_t xxh64(const uint8_t* p, size_t len, uint64_t seed) {
  const uint8_t* const end = p + len;
  uint64_t h;
  if (len >= 32) {
    uint64_t v1 = seed + kP1 + kP2, v2 = seed + kP2, v3 = seed, v4 = seed - kP1;
    const uint8_t* const limit = end - 32;
    do {  // four accumulators over 32-byte stripes
      v1 = lane_round(v1, rd64(p));
      v2 = lane_round(v2, rd64(p + 8));
      v3 = lane_round(v3, rd64(p + 16));
      v4 = lane_round(v4, rd64(p + 24));
      p += 32;
    } while (p <= limit);
    h = rotl(v1, 1) + rotl(v2, 7) + rotl(v3, 12) + rotl(v4, 18);
    h = merge_round(h, v1);
    h = merge_round(h, v2);
    h = merge_round(h, v3);
    h = merge_round(h, v4);
  } else {
    h = seed + kP5;
  }
  h += static_cast<uint64_t>(len);
  while (p + 8 <= end) {  // remaining 8-byte words, then a 4-byte word, then bytes
    h ^= lane_round(0, rd64(p));
    h = rotl(h, 27) * kP1 + kP4;
    p += 8;
  }
  if (p + 4 <= end) {
    h ^= static_cast<uint64_t>(rd32(p)) * kP1;
    h = rotl(h, 23) * kP2 + kP3;
    p += 4;
  }
  while (p < end) {
    h ^= static_cast<uint64_t>(*p) * kP5;
    h = rotl(h, 11) * kP1;
    ++p;
  }
  h ^= h >> 33;  // avalanche
  h *= kP2;
  h ^= h >> 29;
  h *= kP3;
  h ^= h >> 32;
  return h;
}

// chained hashes at every complete hash-block end of tokens[0..n)
void chain(const int32_t* tokens, int64_t n, int32_t hb, uint64_t seed, std::vector<uint64_t>& out) {
  const int64_t nb = n / hb;
  out.resize(nb);
  uint64_t h = seed;
  for (int64_t j = 0; j < nb; ++j) {
    h = xxh64(reinterpret_cast<const uint8_t*>(tokens + j * hb), (size_t)hb * sizeof(int32_t), h);
    out[j] = h;
  }
}

struct PageEntry {
  int32_t page;
  int64_t end;   // tokens of the prefix the page's key certifies
  int64_t step;  // scheduling step of the registration
  bool ready;
};

struct Ckpt {
  int64_t pos;
  int64_t step;  // latest registration step over the groups
  bool ready;
  bool durable;
  int32_t present;  // groups whose slot is filled
  int32_t pins;
  std::vector<int32_t> pages;  // per group, -1 = not yet registered
};

struct Pin {
  std::vector<int32_t> pages;
  uint64_t ckpt_key;
};

inline uint64_t slot_key(int32_t group, int32_t page) {
  return (static_cast<uint64_t>(static_cast<uint32_t>(group)) << 32) | static_cast<uint32_t>(page);
}

}  // namespace

struct kda_index {
  int32_t hb, pb, groups;
  uint64_t seed;
  std::mutex mu;
  std::unordered_map<uint64_t, PageEntry> mla;      // chained hash at the page's end -> page
  std::unordered_map<int32_t, uint64_t> page_key;   // page -> its current key
  std::unordered_map<int32_t, int32_t> page_pins;   // page -> pin count
  std::unordered_map<uint64_t, Ckpt> ckpts;         // chained hash at B -> checkpoint
  std::unordered_map<uint64_t, uint64_t> ckpt_slot; // (group, page) -> checkpoint key
  std::unordered_map<int64_t, Pin> pins;
  int64_t next_pin = 1;
  std::vector<uint64_t> pending_pages, pending_ckpts;
  std::vector<uint64_t> scratch;  // chained hashes of the current call
};

extern "C" {

uint64_t kda_xxh64(const void* data, int64_t len, uint64_t seed) {
  if (len < 0 || (len > 0 && !data)) return 0;
  return xxh64(static_cast<const uint8_t*>(data), (size_t)len, seed);
}

int64_t kda_chain_hashes(const int32_t* tokens, int64_t n, int32_t hash_block, uint64_t seed,
                         uint64_t* out, int64_t max_out) {
  if (hash_block <= 0 || n < 0 || max_out < 0 || (n >= hash_block && !tokens) ||
      (max_out > 0 && !out))
    return -1;
  const int64_t nb = std::min<int64_t>(n / hash_block, max_out);
  uint64_t h = seed;
  for (int64_t j = 0; j < nb; ++j) {
    h = xxh64(reinterpret_cast<const uint8_t*>(tokens + j * hash_block),
              (size_t)hash_block * sizeof(int32_t), h);
    out[j] = h;
  }
  return nb;
}

int64_t kda_ckpt_plan(int64_t start, int64_t len, int32_t hash_block) {
  if (hash_block <= 0 || start < 0 || len <= 0) return -1;
  const int64_t p = (start + len) / hash_block * hash_block;
  return p > start ? p : -1;
}

kda_index* kda_index_create(int32_t hash_block, int32_t physical_block, int32_t num_groups,
                            uint64_t namespace_seed) {
  if (hash_block <= 0 || physical_block <= 0 || physical_block % hash_block != 0 ||
      num_groups < 1 || num_groups > 64) {
    fail(KDA_ERR_SHAPE, "kda_index_create: need hash_block > 0, physical_block a multiple of it, "
                        "1 <= num_groups <= 64");
    return nullptr;
  }
  kda_index* idx = new kda_index();
  idx->hb = hash_block;
  idx->pb = physical_block;
  idx->groups = num_groups;
  idx->seed = namespace_seed;
  ok();
  return idx;
}

void kda_index_destroy(kda_index* idx) { delete idx; }

kda_status kda_index_register_pages(kda_index* idx, const int32_t* tokens, int64_t n,
                                    const int32_t* pages, int32_t num_pages, int64_t step,
                                    int32_t* taken) {
  if (!idx) return fail(KDA_ERR_NULL, "kda_index_register_pages: index is NULL");
  if (n < 0) return fail(KDA_ERR_SHAPE, "kda_index_register_pages: n < 0");
  if (n > 0 && !tokens) return fail(KDA_ERR_NULL, "kda_index_register_pages: tokens are NULL");
  const int64_t need = (n + idx->pb - 1) / idx->pb;
  if (num_pages != need)
    return fail(KDA_ERR_SHAPE, "kda_index_register_pages: %d pages given, %lld tokens need %lld",
                num_pages, (long long)n, (long long)need);
  if (num_pages > 0 && !pages) return fail(KDA_ERR_NULL, "kda_index_register_pages: pages are NULL");
  for (int32_t i = 0; i < num_pages; ++i) {
    if (pages[i] < 0) return fail(KDA_ERR_PAGE_RANGE, "kda_index_register_pages: page %d < 0", pages[i]);
    for (int32_t j = 0; j < i; ++j)
      if (pages[j] == pages[i])
        return fail(KDA_ERR_PAGE_ALIAS, "kda_index_register_pages: page %d listed twice", pages[i]);
  }
  std::lock_guard<std::mutex> lock(idx->mu);
  chain(tokens, n, idx->hb, idx->seed, idx->scratch);
  const int64_t full = (n / idx->hb) * idx->hb;  // end of the last complete hash block
  for (int32_t i = 0; i < num_pages; ++i) {
    const int64_t end = std::min<int64_t>((int64_t)(i + 1) * idx->pb, full);
    int32_t t = 0;
    if (end > (int64_t)i * idx->pb) {
      const uint64_t key = idx->scratch[end / idx->hb - 1];
      auto it = idx->mla.find(key);
      if (it != idx->mla.end()) {
        t = (it->second.page == pages[i] && it->second.end == end) ? 1 : 0;  // first one wins
      } else {
        auto pk = idx->page_key.find(pages[i]);
        if (pk != idx->page_key.end()) {  // the page's registered end advances
          auto old = idx->mla.find(pk->second);
          if (old != idx->mla.end() && old->second.page == pages[i]) idx->mla.erase(old);
        }
        idx->mla[key] = PageEntry{pages[i], end, step, false};
        idx->page_key[pages[i]] = key;
        idx->pending_pages.push_back(key);
        t = 1;
      }
    }
    if (taken) taken[i] = t;
  }
  return ok();
}

kda_status kda_index_register_ckpt(kda_index* idx, const int32_t* tokens, int64_t pos,
                                   int32_t group, int32_t page, int32_t durable, int64_t step,
                                   int32_t* taken) {
  if (!idx) return fail(KDA_ERR_NULL, "kda_index_register_ckpt: index is NULL");
  if (!tokens) return fail(KDA_ERR_NULL, "kda_index_register_ckpt: tokens are NULL");
  if (pos <= 0 || pos % idx->hb != 0)
    return fail(KDA_ERR_CKPT_ALIGN, "kda_index_register_ckpt: position %lld is not a positive multiple of %d",
                (long long)pos, idx->hb);
  if (group < 0 || group >= idx->groups)
    return fail(KDA_ERR_SHAPE, "kda_index_register_ckpt: group %d outside [0, %d)", group, idx->groups);
  if (page < 0) return fail(KDA_ERR_PAGE_RANGE, "kda_index_register_ckpt: page %d < 0", page);
  std::lock_guard<std::mutex> lock(idx->mu);
  chain(tokens, pos, idx->hb, idx->seed, idx->scratch);
  const uint64_t key = idx->scratch.back();
  auto slot = idx->ckpt_slot.find(slot_key(group, page));
  if (slot != idx->ckpt_slot.end() && slot->second != key)
    return fail(KDA_ERR_PAGE_ALIAS, "kda_index_register_ckpt: group %d page %d holds another checkpoint",
                group, page);
  auto it = idx->ckpts.find(key);
  if (it == idx->ckpts.end()) {
    Ckpt c;
    c.pos = pos;
    c.step = step;
    c.ready = false;
    c.durable = false;
    c.present = 0;
    c.pins = 0;
    c.pages.assign(idx->groups, -1);
    it = idx->ckpts.emplace(key, std::move(c)).first;
  }
  Ckpt& c = it->second;
  int32_t t;
  if (c.pages[group] >= 0) {
    t = c.pages[group] == page ? 1 : 0;
  } else {
    c.pages[group] = page;
    c.present += 1;
    c.step = std::max(c.step, step);
    c.ready = false;  // the new group's copy is pending
    idx->ckpt_slot[slot_key(group, page)] = key;
    idx->pending_ckpts.push_back(key);
    t = 1;
  }
  if (durable) c.durable = true;
  if (taken) *taken = t;
  return ok();
}

kda_status kda_index_mark_ready(kda_index* idx, int64_t step) {
  if (!idx) return fail(KDA_ERR_NULL, "kda_index_mark_ready: index is NULL");
  std::lock_guard<std::mutex> lock(idx->mu);
  std::vector<uint64_t> keep;
  for (uint64_t key : idx->pending_pages) {
    auto it = idx->mla.find(key);
    if (it == idx->mla.end() || it->second.ready) continue;
    if (it->second.step <= step) it->second.ready = true;
    else keep.push_back(key);
  }
  idx->pending_pages.swap(keep);
  keep.clear();
  for (uint64_t key : idx->pending_ckpts) {
    auto it = idx->ckpts.find(key);
    if (it == idx->ckpts.end() || it->second.ready) continue;
    if (it->second.step <= step) it->second.ready = true;
    else keep.push_back(key);
  }
  idx->pending_ckpts.swap(keep);
  return ok();
}

kda_status kda_index_lookup(kda_index* idx, const int32_t* tokens, int64_t n, int32_t pin,
                            int32_t* pages_out, int32_t max_pages, int32_t* ckpt_pages_out,
                            kda_hit* hit) {
  if (!idx || !hit) return fail(KDA_ERR_NULL, "kda_index_lookup: index or hit is NULL");
  if (n < 0) return fail(KDA_ERR_SHAPE, "kda_index_lookup: n < 0");
  if (n > 0 && !tokens) return fail(KDA_ERR_NULL, "kda_index_lookup: tokens are NULL");
  if (max_pages < 0 || (max_pages > 0 && !pages_out))
    return fail(KDA_ERR_NULL, "kda_index_lookup: pages_out is NULL");
  std::lock_guard<std::mutex> lock(idx->mu);
  const int32_t hb = idx->hb, pb = idx->pb;
  chain(tokens, n, hb, idx->seed, idx->scratch);
  const std::vector<uint64_t>& H = idx->scratch;  // H[j] = hash after j+1 blocks
  const int64_t full = (n / hb) * hb;
  auto served = [&](int64_t end) -> const PageEntry* {  // a ready page registered with exactly this end
    auto it = idx->mla.find(H[end / hb - 1]);
    return (it != idx->mla.end() && it->second.ready && it->second.end == end) ? &it->second : nullptr;
  };
  // MLA stage: whole pages, then the hash-block ends inside the first missing one
  std::vector<int32_t> pg;
  int64_t mla_tokens = 0;
  for (int64_t i = 0;; ++i) {
    const int64_t pend = (i + 1) * (int64_t)pb;
    if (pend <= full) {
      if (const PageEntry* e = served(pend)) {
        pg.push_back(e->page);
        mla_tokens = pend;
        continue;
      }
    }
    for (int64_t e = std::min(pend - hb, full); e > i * (int64_t)pb; e -= hb) {
      if (const PageEntry* pe = served(e)) {
        pg.push_back(pe->page);
        mla_tokens = e;
        break;
      }
    }
    break;
  }
  // KDA stage: the longest boundary within the MLA match held by every group
  int64_t B = 0;
  Ckpt* hitc = nullptr;
  uint64_t hit_key = 0;
  for (int64_t b = mla_tokens; b >= hb; b -= hb) {
    auto it = idx->ckpts.find(H[b / hb - 1]);
    if (it != idx->ckpts.end() && it->second.ready && it->second.present == idx->groups) {
      B = b;
      hitc = &it->second;
      hit_key = it->first;
      break;
    }
  }
  const int64_t np = (B + pb - 1) / pb;
  if (np > max_pages)
    return fail(KDA_ERR_SHAPE, "kda_index_lookup: the hit needs %lld pages, max_pages = %d",
                (long long)np, max_pages);
  for (int64_t i = 0; i < np; ++i) pages_out[i] = pg[i];
  if (ckpt_pages_out)
    for (int32_t g = 0; g < idx->groups; ++g) ckpt_pages_out[g] = hitc ? hitc->pages[g] : -1;
  hit->boundary = B;
  hit->mla_tokens = mla_tokens;
  hit->num_pages = (int32_t)np;
  hit->pad = 0;
  hit->pin_handle = 0;
  if (pin && hitc) {
    Pin p;
    p.pages.assign(pg.begin(), pg.begin() + np);
    p.ckpt_key = hit_key;
    for (int32_t q : p.pages) idx->page_pins[q] += 1;
    hitc->pins += 1;
    const int64_t h = idx->next_pin++;
    idx->pins.emplace(h, std::move(p));
    hit->pin_handle = h;
  }
  return ok();
}

kda_status kda_index_release(kda_index* idx, int64_t pin_handle) {
  if (!idx) return fail(KDA_ERR_NULL, "kda_index_release: index is NULL");
  std::lock_guard<std::mutex> lock(idx->mu);
  auto it = idx->pins.find(pin_handle);
  if (it == idx->pins.end())
    return fail(KDA_ERR_NOT_FOUND, "kda_index_release: no pin %lld", (long long)pin_handle);
  for (int32_t q : it->second.pages) {
    auto pp = idx->page_pins.find(q);
    if (pp != idx->page_pins.end() && --pp->second == 0) idx->page_pins.erase(pp);
  }
  auto c = idx->ckpts.find(it->second.ckpt_key);
  if (c != idx->ckpts.end()) c->second.pins -= 1;
  idx->pins.erase(it);
  return ok();
}

kda_status kda_index_evict_page(kda_index* idx, int32_t page) {
  if (!idx) return fail(KDA_ERR_NULL, "kda_index_evict_page: index is NULL");
  std::lock_guard<std::mutex> lock(idx->mu);
  auto pk = idx->page_key.find(page);
  if (pk == idx->page_key.end())
    return fail(KDA_ERR_NOT_FOUND, "kda_index_evict_page: page %d holds no key", page);
  if (idx->page_pins.count(page))
    return fail(KDA_ERR_PINNED, "kda_index_evict_page: page %d is pinned", page);
  auto it = idx->mla.find(pk->second);
  if (it != idx->mla.end() && it->second.page == page) idx->mla.erase(it);
  idx->page_key.erase(pk);
  return ok();
}

kda_status kda_index_evict_ckpt(kda_index* idx, int32_t group, int32_t page,
                                int32_t* freed_pages) {
  if (!idx) return fail(KDA_ERR_NULL, "kda_index_evict_ckpt: index is NULL");
  std::lock_guard<std::mutex> lock(idx->mu);
  auto slot = idx->ckpt_slot.find(slot_key(group, page));
  if (slot == idx->ckpt_slot.end())
    return fail(KDA_ERR_NOT_FOUND, "kda_index_evict_ckpt: no checkpoint in group %d page %d", group, page);
  auto it = idx->ckpts.find(slot->second);
  if (it == idx->ckpts.end()) {  // cannot happen: slots are erased with their checkpoint
    idx->ckpt_slot.erase(slot);
    return fail(KDA_ERR_NOT_FOUND, "kda_index_evict_ckpt: stale slot");
  }
  if (it->second.pins > 0)
    return fail(KDA_ERR_PINNED, "kda_index_evict_ckpt: checkpoint at %lld is pinned",
                (long long)it->second.pos);
  for (int32_t g = 0; g < idx->groups; ++g) {  // every group at once
    const int32_t q = it->second.pages[g];
    if (freed_pages) freed_pages[g] = q;
    if (q >= 0) idx->ckpt_slot.erase(slot_key(g, q));
  }
  idx->ckpts.erase(it);
  return ok();
}

kda_status kda_index_stats(const kda_index* idx, int64_t* mla_entries, int64_t* ckpts,
                           int64_t* pins) {
  if (!idx) return fail(KDA_ERR_NULL, "kda_index_stats: index is NULL");
  kda_index* m = const_cast<kda_index*>(idx);
  std::lock_guard<std::mutex> lock(m->mu);
  if (mla_entries) *mla_entries = (int64_t)idx->mla.size();
  if (ckpts) *ckpts = (int64_t)idx->ckpts.size();
  if (pins) *pins = (int64_t)idx->pins.size();
  return ok();
}

}  // extern "C"
