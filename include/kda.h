/*
 * kda.h -- C ABI of libkda: the KDA gated delta-rule recurrence on one
 * MI355X (gfx950), with sparse state checkpoints over a paged state pool.
 *
 * Passages this interface implements (pages cited by title and section):
 *
 *  [ARCH]  "Kimi K3 -- Lesson 01 - Architecture map" (gentlecold.top),
 *          section "两种 Attention，两种状态": per head a state S in
 *          R^(d_k x d_v); each token decays S by a channel-wise forget gate
 *          Diag(alpha_t), writes (k_t, v_t) by the delta rule with beta_t, and
 *          reads o_t = S_t^T q_t; prefill is chunk-parallel with the state
 *          carried from chunk to chunk, decode is a single-token update.
 *  [AFF]   "KIMI K3 경량 복제에서 본 KDA의 AI 인프라 과제" (acpost.vercel.app),
 *          sections 1.1/1.3 (per-token affine map S_t = M_t S_{t-1} + b_t; a
 *          segment collapses to one affine map, associative, not commutative)
 *          and 2.1 (decode reads a fixed-size state, not the history).
 *  [CKPT]  "Cache de préfixe hybride KDA–MLA" (mkdocs.reaper.mx), sections
 *          "La solution" (recurrent-state checkpoints only at a sparse subset
 *          of 512-token hash-block ends), "Le fonctionnement du prefill"
 *          (after a forward pass the kernel persists the state at the last
 *          hash-aligned position it processed; checkpoints are read-only: a hit
 *          copies one into the request's private state, new checkpoints go to
 *          fresh slots) and "La recherche en deux étages" (hits are multiples
 *          of the hash block).
 *  [PAGE]  same page, section "La mise en page unifiée": states live in a pool
 *          of pages of one fixed byte size; inside a page the states of all
 *          heads are stored contiguously, head after head.
 *  [INT8]  "KIMI K3 경량 복제에서 본 KDA의 AI 인프라 과제" (acpost.vercel.app),
 *          sections 5.3 (Compressed Checkpoint: cached recurrent states may be
 *          held as int8 with per-channel parameters; a hit dequantises once
 *          into a fresh active slot and decoding continues at full precision)
 *          and 6.6.2 (Int8CheckpointStore: one scale per d_k index from the
 *          max-abs over d_v, symmetric quantisation).
 *
 * Recurrence (decay first, then the delta-rule write, then the read):
 *     S' = Diag(exp(g_t)) S_{t-1};  u = v_t - S'^T k_t;
 *     S_t = S' + beta_t k_t u^T;    o_t = S_t^T q_t.
 * The gate is passed as g = log(alpha).
 *
 * Conventions shared by every entry point
 *  - Device pointers are HIP device memory owned by the caller; host pointers
 *    are read before the call returns.  The library keeps no pointer past a
 *    call and allocates no device memory.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *    is complete once that stream has synchronised.  Calls on one stream run
 *    in call order, so a restore completes before a later prefill or decode on
 *    the same stream reads the restored page.
 *  - All arguments are validated before anything is enqueued; a non-KDA_OK
 *    status means nothing was enqueued, except KDA_ERR_HIP (a launch failed
 *    after validation; earlier launches of the same call may have run).
 *  - kda_last_error() returns a thread-local description of the last failure.
 *  - No exception or abort crosses this interface.
 *  - Floating-point reductions use no atomics: repeated calls on the same
 *    inputs give bitwise-identical results.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KDA_OK = 0,
  KDA_ERR_NULL = 1,        /* a required pointer is NULL                          */
  KDA_ERR_SHAPE = 2,       /* unsupported head dims, counts, chunk or hash sizes  */
  KDA_ERR_DTYPE = 3,       /* unknown dtype code                                  */
  KDA_ERR_PAGE_RANGE = 4,  /* a page index is outside [0, num_pages)              */
  KDA_ERR_PAGE_ALIAS = 5,  /* a destination page repeats or is also read          */
  KDA_ERR_CKPT_ALIGN = 6,  /* checkpoint position not a multiple of hash_block    */
  KDA_ERR_CKPT_RANGE = 7,  /* checkpoint outside (start, start+len] or unordered  */
  KDA_ERR_SEQ = 8,         /* bad cu_seqlens / start_pos                          */
  KDA_ERR_WORKSPACE = 9,   /* workspace NULL, misaligned or too small             */
  KDA_ERR_HIP = 10,        /* a HIP launch or runtime call failed                 */
  KDA_ERR_POOL = 11,       /* invalid pool descriptor                             */
  KDA_ERR_PINNED = 12,     /* prefix index: eviction of an entry a lookup pinned   */
  KDA_ERR_NOT_FOUND = 13   /* prefix index: no entry for that page / pin handle    */
} kda_status;

/* Element-type code of tensors and pools: an int32_t, so that a caller may
 * pass any value and get KDA_ERR_DTYPE for an unknown one (a C++ enum object
 * may not hold values outside its enumerators). */
typedef int32_t kda_dtype;
enum { KDA_F32 = 0, KDA_BF16 = 1 };

/*
 * Paged state pool [PAGE].  `base` is device memory of num_pages * page_bytes
 * bytes.  Page p, head h holds one fp32 state S[d_k][d_v], row-major (row =
 * key channel), at byte offset
 *     p * page_bytes + h * d_k * d_v * 4
 * Bytes past num_heads * d_k * d_v * 4 in a page are padding that no entry
 * point reads or writes.  Requirements (kda_pool_check): base and page_bytes
 * multiples of 256, page_bytes >= num_heads * d_k * d_v * 4, num_pages >= 1,
 * num_heads >= 1, d_k == d_v in {64, 128}.  The pool is owned by the caller.
 */
typedef struct {
  void* base;
  int64_t page_bytes;
  int32_t num_pages;
  int32_t num_heads;
  int32_t d_k;
  int32_t d_v;
} kda_pool;

/* Library version, (major << 16) | minor. */
int32_t kda_version(void);

/* Thread-local text of the last non-KDA_OK status on this thread ("" if none). */
const char* kda_last_error(void);

/* Validates a pool descriptor (no device access).  [PAGE] */
kda_status kda_pool_check(const kda_pool* pool);

/* Byte offset of (page, head) inside the pool, or -1 if the descriptor is
 * invalid or page/head is out of range.  [PAGE] */
int64_t kda_state_offset(const kda_pool* pool, int32_t page, int32_t head);

/*
 * Device workspace bytes kda_prefill_chunked prefers for a call with these
 * sizes (total_tokens = cu_seqlens[num_seqs], num_ckpts = ckpt_cu[num_seqs]).
 * Returns 0 for invalid arguments.  The workspace holds the call's metadata
 * tables, two carried states (H heads each) and one window of the call: the
 * per-(chunk, head) intermediates of the chunk form for up to
 * max(1, 2048 / H) consecutive 64-token chunks (about 135 MB at H = 32,
 * d = 128, bf16), whatever the length of the call.  It must be 256-byte
 * aligned and is free for reuse once the stream passes the call.
 */
size_t kda_prefill_workspace_bytes(const kda_pool* pool, int64_t total_tokens, int32_t num_seqs,
                                   int32_t num_ckpts, kda_dtype in_dtype);

/*
 * The smallest workspace kda_prefill_chunked accepts for num_seqs sequences
 * and num_ckpts checkpoints, of any length: windows of one chunk.  Any size
 * from this one up is accepted; the call uses the largest window (up to the
 * preferred one) that fits, so a smaller workspace means more launches,
 * never different results.  Returns 0 for invalid arguments.
 */
size_t kda_prefill_workspace_min_bytes(const kda_pool* pool, int32_t num_seqs, int32_t num_ckpts,
                                       kda_dtype in_dtype);

/*
 * Chunk-parallel prefill of a packed batch of sequences [ARCH][AFF], with the
 * state carried between 64-token chunks and sparse checkpoint stores [CKPT].
 *
 * Device tensors (token-major, all with `in_dtype`):
 *   q, k, g : [total_tokens, H, d_k]   (g = log alpha, one gate per key channel)
 *   v       : [total_tokens, H, d_v]
 *   beta    : [total_tokens, H]
 *   o       : [total_tokens, H, d_v] written in `out_dtype`
 *   q, k, v, g and o 16-byte aligned (KDA_ERR_SHAPE otherwise); o must not
 *   overlap an input.
 * Host metadata (read before return):
 *   cu_seqlens     [num_seqs+1]  int64, cu_seqlens[0] == 0, non-decreasing;
 *                  sequence s owns rows [cu_seqlens[s], cu_seqlens[s+1]).
 *   start_pos      [num_seqs]    int64 or NULL (all 0): absolute position of the
 *                  sequence's first token; a multiple of chunk_size in [0, 2^62].  A
 *                  resume at boundary B passes start_pos = B and the restored
 *                  page as state_in_page.
 *   state_in_page  [num_seqs]    int32 or NULL: page holding S before the first
 *                  token; -1 (or NULL) = zero state.
 *   state_out_page [num_seqs]    int32 or NULL: page receiving S after the last
 *                  token; -1 (or NULL) = not stored.  May equal the same
 *                  sequence's state_in_page (in-place update).
 *   ckpt_cu        [num_seqs+1]  int32 CSR offsets into ckpt_pos/ckpt_page, or
 *                  NULL for no checkpoints.
 *   ckpt_pos       absolute positions P: multiple of hash_block, strictly
 *                  increasing per sequence, start < P <= start+len.  The
 *                  checkpoint at P is the state after P tokens.
 *   ckpt_page      destination page of each checkpoint (a fresh page).
 * chunk_size must be 64; hash_block a positive multiple of 64 (512 in the
 * pages).  workspace must hold at least kda_prefill_workspace_min_bytes(...)
 * bytes (KDA_ERR_WORKSPACE otherwise).
 * Windows: the call runs in windows of consecutive chunks of the packed batch
 * (prep of the window's chunks, then the scan of the sequences owning them); a
 * sequence cut by a window edge carries its fp32 state across unchanged, so
 * the results are bit-identical for every workspace size.
 * Destination pages (state_out_page, ckpt_page) must be distinct and must not
 * be any state_in_page, apart from the in-place case above (KDA_ERR_PAGE_ALIAS).
 *
 * Numerics: bf16 inputs run the chunk products on bf16 MFMA with fp32
 * accumulation and an fp32 carried state; fp32 inputs run them in fp32.
 * Domain: with G the within-chunk prefix sum of g (g <= 0), the chunk form
 * uses exp(G) and exp(G_C - G) (at most 1) for the state-side operands and
 * exp(+-(G - G_31)) for the intra-chunk Gram products (G_31: the prefix
 * through the chunk's 32nd token).  It needs |G_i - G_31| < 87 in every
 * channel, token i and chunk, so that every factor is a normal fp32 number:
 * any gate sum over half a chunk above -87 (a mean log alpha above -2.7 per
 * token suffices).  Past it, results lose accuracy or become non-finite.
 * Tuning: the environment variable KDA_SCAN_SLAB=1 or 2 forces 16- or
 * 32-column state slabs in the scan (by default 32 when that still gives every
 * CU a workgroup); results are bit-identical either way.
 */
kda_status kda_prefill_chunked(const kda_pool* pool, const void* q, const void* k, const void* v,
                               const void* g, const void* beta, kda_dtype in_dtype, void* o,
                               kda_dtype out_dtype, int32_t num_seqs, const int64_t* cu_seqlens,
                               const int64_t* start_pos, const int32_t* state_in_page,
                               const int32_t* state_out_page, const int32_t* ckpt_cu,
                               const int64_t* ckpt_pos, const int32_t* ckpt_page,
                               int32_t chunk_size, int32_t hash_block, void* workspace,
                               size_t workspace_bytes, void* stream);

/* Size of the static device scratch behind kda_prefill_chunked_noalloc. */
#define KDA_PREFILL_SCRATCH_BYTES (64u << 20)

/*
 * kda_prefill_chunked without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops that
 * must not allocate, harnesses that forbid allocation).  Arguments, results,
 * validation and errors are those of kda_prefill_chunked; the workspace is a
 * static device array of KDA_PREFILL_SCRATCH_BYTES (64 MiB) that the library
 * holds on every GPU it runs on until the process ends.  The call allocates
 * nothing: the array's device address is resolved once per device (on the
 * first call on that device, which must be the current one).  Any length is
 * accepted (the call runs in windows that fit the array; results are
 * bit-identical to kda_prefill_chunked); a call whose tables and one window
 * of one chunk do not fit, i.e. kda_prefill_workspace_min_bytes(...) >
 * KDA_PREFILL_SCRATCH_BYTES, is rejected with KDA_ERR_WORKSPACE before
 * anything is enqueued.  Every call on one GPU uses the same array, and each
 * call writes every scratch byte it reads, so nothing needs clearing between
 * calls; calls that overlap on one GPU (different streams, or host threads
 * without ordering) race on the array and must be serialised by the caller.
 */
kda_status kda_prefill_chunked_noalloc(const kda_pool* pool, const void* q, const void* k,
                                       const void* v, const void* g, const void* beta,
                                       kda_dtype in_dtype, void* o, kda_dtype out_dtype,
                                       int32_t num_seqs, const int64_t* cu_seqlens,
                                       const int64_t* start_pos, const int32_t* state_in_page,
                                       const int32_t* state_out_page, const int32_t* ckpt_cu,
                                       const int64_t* ckpt_pos, const int32_t* ckpt_page,
                                       int32_t chunk_size, int32_t hash_block, void* stream);

/*
 * One decode step for n requests [ARCH][AFF 2.1]: for each request r and head
 * h, read S from page_in[r], apply one token (q, k, v, g, beta of row r), write
 * S to page_out[r] and o.  The state is read and written exactly once.
 *   q, k, g : [n, H, d_k]; v : [n, H, d_v]; beta : [n, H]  (in_dtype, device)
 *   o       : [n, H, d_v] (out_dtype, device)
 *   page_in, page_out : [n] int32 DEVICE arrays (so a step needs no host sync).
 * page_out[r] == page_in[r] updates in place.  The caller guarantees that the
 * page_out entries are distinct and that no page_out[r] equals page_in[r'] for
 * r' != r.  Device-side: a request whose page index is outside [0, num_pages)
 * touches no state and gets NaN outputs.  With the environment variable
 * KDA_VALIDATE=1 the page tables are copied to the host and checked first
 * (this synchronises the stream).
 */
kda_status kda_decode_step(const kda_pool* pool, const void* q, const void* k, const void* v,
                           const void* g, const void* beta, kda_dtype in_dtype, void* o,
                           kda_dtype out_dtype, int32_t n, const int32_t* page_in,
                           const int32_t* page_out, void* stream);

/*
 * Speculative verification [ARCH][AFF 2.1]: apply `tokens` (1..64) consecutive
 * tokens to each of n requests in one launch, keeping every intermediate
 * state so that rejected draft tokens can be rolled back (page "KIMI K3 경량
 * 복제에서 본 KDA의 AI 인프라 과제", sections 6.4 and 6.5: the kernel
 * dispatcher has a target-verify path next to decode and prefill, and one KDA
 * run carries the recurrent state together with the indices of the verify
 * step's intermediate states).  Token t of request r is input row r*tokens + t:
 *   q, k, g : [n*tokens, H, d_k]; v : [n*tokens, H, d_v]; beta : [n*tokens, H]
 *   o       : [n*tokens, H, d_v]
 *   page_in : [n] int32 DEVICE array, the state before the first token;
 *   page_out: [n*tokens] int32 DEVICE array, page_out[r*tokens + t] receives the
 *             state after token t (so accepting a tokens of request r means
 *             continuing from page_out[r*tokens + a - 1]).
 * The state is read once and stays on chip from token to token; outputs equal
 * those of `tokens` consecutive kda_decode_step calls bit for bit.  page_out
 * entries must be distinct and none may equal another request's page_in (one
 * of a request's own outputs may equal its page_in).  Device-side: a request
 * with any page index outside [0, num_pages) touches no state and gets NaN
 * outputs for all its tokens; KDA_VALIDATE=1 checks the tables on the host.
 * kda_decode_step is the case tokens = 1.
 */
kda_status kda_decode_verify(const kda_pool* pool, const void* q, const void* k, const void* v,
                             const void* g, const void* beta, kda_dtype in_dtype, void* o,
                             kda_dtype out_dtype, int32_t n, int32_t tokens, const int32_t* page_in,
                             const int32_t* page_out, void* stream);

/*
 * Checkpoint write [CKPT]: copy the state bytes (num_heads * d_k * d_v * 4) of
 * page src_active[i] to page dst_ckpt[i], i < n.  Host index arrays.  Pages in
 * range; destinations distinct and never a source of the same call.
 */
kda_status kda_checkpoint_write(const kda_pool* pool, const int32_t* src_active,
                                const int32_t* dst_ckpt, int32_t n, void* stream);

/*
 * Checkpoint restore [CKPT]: copy checkpoint page src_ckpt[i] into the
 * request's private active page dst_active[i] (copy-on-write: the checkpoint
 * itself is never modified).  Same rules as kda_checkpoint_write.
 */
kda_status kda_checkpoint_restore(const kda_pool* pool, const int32_t* src_ckpt,
                                  const int32_t* dst_active, int32_t n, void* stream);

/*
 * Compressed (int8) checkpoints [INT8].  A compressed page of `qpool` holds,
 * for each head h at byte offset h * kda_ckpt_int8_head_bytes(d_k, d_v):
 *     int8_t q[d_k][d_v]   (row i is the d_k index, as in the fp32 state)
 *     float  scale[d_k]
 * with, per d_k row i (fp32 arithmetic, IEEE division):
 *     scale_i = max_j |S_ij| / 127
 *     q_ij    = clamp(round_half_even(S_ij / scale_i), -127, 127), 0 if scale_i == 0
 * and restore writes S~_ij = q_ij * scale_i (fp32).  The pages fix neither the
 * rounding nor the clamp; this is the reading taken.  |S~_ij - S_ij| <=
 * scale_i / 2.  States must be finite.
 * qpool: same num_heads, d_k, d_v as pool; page_bytes >= num_heads *
 * kda_ckpt_int8_head_bytes(d_k, d_v); its byte range must not overlap pool's.
 * Host index arrays of n entries; pages in range; destinations distinct.
 * Errors: KDA_ERR_NULL, KDA_ERR_SHAPE (pools disagree), KDA_ERR_POOL (qpool
 * too small / misaligned), KDA_ERR_PAGE_RANGE, KDA_ERR_PAGE_ALIAS (duplicate
 * destination or overlapping pools), KDA_ERR_HIP.
 */
int64_t kda_ckpt_int8_head_bytes(int32_t d_k, int32_t d_v);

/* Quantise active pages pool[src_active[i]] into compressed pages qpool[dst_qckpt[i]]. */
kda_status kda_checkpoint_write_int8(const kda_pool* pool, const int32_t* src_active,
                                     const kda_pool* qpool, const int32_t* dst_qckpt, int32_t n,
                                     void* stream);

/* Dequantise compressed pages qpool[src_qckpt[i]] into fp32 active pages
 * pool[dst_active[i]] (copy-on-write restore: the compressed page is not modified). */
kda_status kda_checkpoint_restore_int8(const kda_pool* qpool, const int32_t* src_qckpt,
                                       const kda_pool* pool, const int32_t* dst_active, int32_t n,
                                       void* stream);

/*
 * Short causal convolution with a checkpointed window state [CONV]: page
 * "KIMI K3 경량 복제에서 본 KDA의 AI 인프라 과제" (acpost.vercel.app), sections
 * 1.1, 6.5, 6.6.3 and 8.2.3/8.2.4: before the recurrence, q, k and v each pass through a
 * short causal convolution whose state is the window of the most recent inputs;
 * that window is checkpointed with the recurrent state at the same boundary,
 * kept at full precision, and a restore must bring it back too.  The pages fix
 * neither the width nor an activation; this library takes a width W in {2, 3, 4}
 * and no activation:
 *     y[t][c] = sum_{j < W} w[c][j] * x[t - (W-1) + j][c]
 * with x at positions before a sequence's start taken from its state page
 * (zeros when there is none).  Call it once per tensor (q, k, v).
 *
 * Conv-state pool: page p holds the W-1 most recent inputs, token-major
 * ([W-1][channels], row i = the input at position P-(W-1)+i), in `dtype` (the
 * input dtype).  page_bytes >= (W-1) * channels * elem, multiple of 256.
 */
typedef struct {
  void* base;          /* device memory, 256-byte aligned */
  int64_t page_bytes;
  int32_t num_pages;
  int32_t channels;    /* C: channels per token, e.g. H * d for one of q, k, v */
  int32_t width;       /* W in {2, 3, 4} */
  int32_t dtype;       /* kda_dtype of x and of the stored window */
} kda_conv_pool;

/* Workspace bytes (per-call metadata tables) of kda_short_conv. */
int64_t kda_conv_workspace_bytes(int32_t num_seqs, int32_t num_ckpts);

/*
 * x : [T, C] (cpool->dtype, device), w : [C][W] fp32 (device), y : [T, C]
 * (out_dtype, device; may not alias x).  Sequences as in kda_prefill_chunked:
 * cu_seqlens [num_seqs+1] int64 host; start_pos [num_seqs] host or NULL (any
 * value in [0, 2^62]); state_in_page / state_out_page [num_seqs] int32 host or
 * NULL (-1 = zero window / not written); checkpoints (ckpt_cu, ckpt_pos,
 * ckpt_page, host) at multiples of hash_block inside (start, start+len] receive
 * the window of the hash_block-aligned position, written in the same pass.  An
 * empty sequence with an output page copies its input window.  Output pages
 * and checkpoint pages are distinct and are never input pages of the call.
 * Errors: KDA_ERR_NULL, KDA_ERR_SHAPE, KDA_ERR_DTYPE, KDA_ERR_POOL, KDA_ERR_SEQ,
 * KDA_ERR_PAGE_RANGE, KDA_ERR_PAGE_ALIAS, KDA_ERR_CKPT_ALIGN, KDA_ERR_CKPT_RANGE,
 * KDA_ERR_WORKSPACE, KDA_ERR_HIP.
 */
kda_status kda_short_conv(const kda_conv_pool* cpool, const void* x, const float* w, void* y,
                          kda_dtype out_dtype, int32_t num_seqs, const int64_t* cu_seqlens,
                          const int64_t* start_pos, const int32_t* state_in_page,
                          const int32_t* state_out_page, const int32_t* ckpt_cu,
                          const int64_t* ckpt_pos, const int32_t* ckpt_page, int32_t hash_block,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode-step convolution update: one token for each of n requests.  Request
 * r reads its window (the W-1 most recent inputs, as kda_short_conv stores
 * them) from page page_in[r], computes y row r from it and x row r, and
 * writes the next window (the last W-2 window rows, then x row r) to page
 * page_out[r].  Same arithmetic as kda_short_conv, so equal inputs give equal
 * bits (page "KIMI K3 경량 복제에서 본 KDA의 AI 인프라 과제", sections 6.4
 * and 8.2.3: in decode the convolution state is updated one token at a time
 * next to the recurrent state).
 *   x : [n, C] (cpool->dtype, device); w : [C][W] fp32 (device);
 *   y : [n, C] (out_dtype, device; may not alias x)
 *   page_in, page_out : [n] int32 DEVICE arrays (no host synchronisation per
 *   step).  page_out[r] == page_in[r] updates in place.  The caller
 *   guarantees that the page_out entries are distinct and that no page_out[r]
 *   equals page_in[r'] for r' != r.  Device-side: a request whose page index
 *   is outside [0, num_pages) touches no page and gets NaN outputs.  With the
 *   environment variable KDA_VALIDATE=1 the page tables are copied to the
 *   host and checked first (this synchronises the stream).  A checkpoint of
 *   the window at a hash-block boundary is the page_out of the token that
 *   ends there.
 * Errors: KDA_ERR_NULL, KDA_ERR_SHAPE, KDA_ERR_DTYPE, KDA_ERR_POOL,
 * KDA_ERR_PAGE_RANGE / KDA_ERR_PAGE_ALIAS (KDA_VALIDATE=1 only), KDA_ERR_HIP.
 */
kda_status kda_short_conv_update(const kda_conv_pool* cpool, const void* x, const float* w, void* y,
                                 kda_dtype out_dtype, int32_t n, const int32_t* page_in,
                                 const int32_t* page_out, void* stream);

/*
 * Optional per-kernel timing (tracing aid).  When enabled, every kernel the
 * library launches is bracketed by a pair of HIP events on its own stream;
 * kda_profile_read synchronises those events and returns, per kernel name, the
 * launch count and the summed duration in milliseconds since the last reset.
 */
typedef struct {
  char name[48];
  int64_t launches;
  double total_ms;
} kda_kernel_stat;

kda_status kda_profile_enable(int32_t on);
int32_t kda_profile_read(kda_kernel_stat* out, int32_t max_entries, int32_t reset);

#ifdef __cplusplus
}
#endif
#endif /* KDA_H_ */
