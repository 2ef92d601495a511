/*
 * kda_index.h -- host-side prefix index of libkda: where a hybrid KDA-MLA
 * request may resume (the hit boundary B), which cached pages serve it, and
 * where its recurrent-state checkpoints go.  Pure host code (no GPU call).
 *
 * Passages this interface implements, page "Cache de préfixe hybride KDA–MLA"
 * (mkdocs.reaper.mx, kimi-k3 infrastructure chapter 08):
 *
 *  [HASH]  "Vérification de compréhension" and "Le fonctionnement du prefill":
 *          prefix hashes are chained -- the hash of hash block n covers block
 *          n-1's hash, so equal hashes at block n certify equal prefixes up to
 *          there; hash blocks are 512 tokens inside coarser physical pages.
 *  [MLA]   "Le fonctionnement du prefill": a partially filled page is
 *          registered under the chained hash of its last complete hash block,
 *          and that registered end advances as the page fills.
 *  [KDA]   same section: after a forward pass the recurrent state is persisted
 *          at the last hash-aligned position processed; intermediate
 *          checkpoints made obsolete by progress are recycled, those at
 *          conversation-turn boundaries are kept.
 *  [TWO]   "La recherche en deux étages": the MLA stage matches whole physical
 *          pages by chained hash and, at the first missing page, falls back to
 *          the hash-block ends inside it; the KDA stage needs a checkpoint at
 *          the candidate boundary in every KDA cache group; the hit is the
 *          longest boundary that passes both (a multiple of the hash block,
 *          not of the physical page).
 *  [SAFE]  "La cohérence sous ordonnancement concurrent": (1) hit entries are
 *          pinned in every group before anything is allocated, so they cannot
 *          be evicted; (2) entries registered in the current scheduling step
 *          are not matched until their copies have completed; (3) evicting a
 *          checkpoint in one group invalidates its siblings in all groups at
 *          once -- a checkpoint is reachable in every group or in none.
 *
 * Readings where the page is silent (the library's choices):
 *  - Hash: XXH64 (the published xxHash 64-bit algorithm) of the block's
 *    token ids as little-endian int32, seeded with the previous block's
 *    chained hash; the hash before block 1 is the index's namespace seed (one
 *    per model version / tokenizer, so foreign entries never match).
 *  - A page holds physical_block tokens; a page is registered under one key
 *    only (its current end); a full page's end is its last token.
 *  - MLA fallback: inside the first page whose full-page key is missing, the
 *    longest hash-block end whose key names a page registered with exactly
 *    that end (ends before it are not searched further).
 *  - A boundary B <= n is returned; B = n means nothing is left to prefill
 *    (callers that need one token of output cap n themselves).
 *  - First registration wins: a key already held by another page or
 *    checkpoint is left as it is and the call reports the page as not taken.
 *
 * Ownership and threading: the index owns its host memory; token and page
 * arrays are read during the call only.  Every call takes the index's lock, so
 * one index may be shared by threads.  All calls return kda_status (kda.h);
 * kda_last_error() has the text.
 */
#ifndef KDA_INDEX_H
#define KDA_INDEX_H

#include <stdint.h>

#include "kda.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct kda_index kda_index;

/* XXH64 of `len` bytes with `seed` (exported for tests of the chain). */
uint64_t kda_xxh64(const void* data, int64_t len, uint64_t seed);

/* Chained hashes of tokens[0..n): out[j] = hash after j+1 complete hash
 * blocks, j < min(n / hash_block, max_out).  Returns the count written, or
 * -1 on bad arguments. */
int64_t kda_chain_hashes(const int32_t* tokens, int64_t n, int32_t hash_block, uint64_t seed,
                         uint64_t* out, int64_t max_out);

/* Checkpoint placement [KDA]: the last multiple of hash_block in
 * (start, start + len], or -1 if there is none. */
int64_t kda_ckpt_plan(int64_t start, int64_t len, int32_t hash_block);

/* hash_block > 0; physical_block a positive multiple of hash_block;
 * 1 <= num_groups <= 64 KDA cache groups.  NULL on bad arguments. */
kda_index* kda_index_create(int32_t hash_block, int32_t physical_block, int32_t num_groups,
                            uint64_t namespace_seed);
void kda_index_destroy(kda_index* idx);

/*
 * [MLA] Register the pages holding the KV of tokens[0..n): pages[i] holds
 * tokens [i*P, min((i+1)*P, n)), i < ceil(n / P), P = physical_block.  Page i
 * is keyed by the chained hash at its end: (i+1)*P if full, else the last
 * hash-block end inside it (pages with no complete hash block are skipped).  A
 * page registered before under a shorter end moves to the new key.  Entries
 * are pending until kda_index_mark_ready(step' >= step).  taken[i] (optional,
 * [num_pages]) = 1 if page i now holds its key, 0 if another page does (or
 * page i was skipped).  Errors: KDA_ERR_NULL, KDA_ERR_SHAPE (num_pages does
 * not match n), KDA_ERR_PAGE_RANGE (negative page id), KDA_ERR_PAGE_ALIAS (a
 * page listed twice).
 */
kda_status kda_index_register_pages(kda_index* idx, const int32_t* tokens, int64_t n,
                                    const int32_t* pages, int32_t num_pages, int64_t step,
                                    int32_t* taken);

/*
 * [KDA] Register group `group`'s checkpoint page of the state after
 * tokens[0..pos) (pos a positive multiple of hash_block).  A checkpoint is
 * visible to lookups only once every group has registered its page and the
 * step is marked ready.  durable = 1 marks a conversation-turn boundary
 * (kept); 0 an intermediate checkpoint (the caller recycles it with
 * kda_index_evict_ckpt when the request moves on).  *taken (optional) = 0 if
 * that group's slot was already filled by another page.  Errors: KDA_ERR_NULL,
 * KDA_ERR_CKPT_ALIGN, KDA_ERR_SHAPE (group), KDA_ERR_PAGE_RANGE,
 * KDA_ERR_PAGE_ALIAS (the group's page already holds another checkpoint).
 */
kda_status kda_index_register_ckpt(kda_index* idx, const int32_t* tokens, int64_t pos,
                                   int32_t group, int32_t page, int32_t durable, int64_t step,
                                   int32_t* taken);

/* [SAFE 2] Entries registered at steps <= step have finished their copies. */
kda_status kda_index_mark_ready(kda_index* idx, int64_t step);

typedef struct {
  int64_t boundary;   /* hit B: multiple of hash_block, 0 = miss              */
  int64_t mla_tokens; /* tokens matched by the MLA stage (>= boundary)        */
  int32_t num_pages;  /* MLA pages covering [0, boundary), in pages_out       */
  int32_t pad;
  int64_t pin_handle; /* > 0 when the call pinned its hit, else 0             */
} kda_hit;

/*
 * [TWO] Longest boundary B <= n served by both stages.  pages_out
 * [max_pages] receives the pages covering [0, B); ckpt_pages_out
 * [num_groups] (optional) the checkpoint page of every group at B (-1 on a
 * miss).  pin = 1 pins those pages and the checkpoint [SAFE 1] until
 * kda_index_release(hit->pin_handle).  Errors: KDA_ERR_NULL, KDA_ERR_SHAPE
 * (max_pages too small for the hit; nothing is pinned then).
 */
kda_status kda_index_lookup(kda_index* idx, const int32_t* tokens, int64_t n, int32_t pin,
                            int32_t* pages_out, int32_t max_pages, int32_t* ckpt_pages_out,
                            kda_hit* hit);
kda_status kda_index_release(kda_index* idx, int64_t pin_handle);

/* Remove a page's MLA entry.  KDA_ERR_PINNED while pinned, KDA_ERR_NOT_FOUND
 * if the page holds no key. */
kda_status kda_index_evict_page(kda_index* idx, int32_t page);

/*
 * [SAFE 3] Evict the checkpoint whose group `group` slot is `page`: the whole
 * checkpoint leaves the index in every group at once, and freed_pages
 * [num_groups] (optional) receives each group's page (-1 where a group had
 * none) for the caller to reuse.  KDA_ERR_PINNED while pinned,
 * KDA_ERR_NOT_FOUND if no checkpoint holds that page.
 */
kda_status kda_index_evict_ckpt(kda_index* idx, int32_t group, int32_t page,
                                int32_t* freed_pages);

/* Counts: MLA entries, checkpoints (complete or not), live pin handles. */
kda_status kda_index_stats(const kda_index* idx, int64_t* mla_entries, int64_t* ckpts,
                           int64_t* pins);

#ifdef __cplusplus
}
#endif
#endif
