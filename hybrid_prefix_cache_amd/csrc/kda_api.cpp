// kda_api.cpp -- host side of libkda: argument validation, per-call metadata
// tables, launches, error reporting and optional per-kernel timing.
//
// Every entry point validates all of its arguments before enqueueing anything
// (all-or-nothing), so a rejected call leaves the device untouched.  The
// library allocates no device memory: per-call tables travel in kernel
// arguments into the caller's workspace, and decode page tables are the
// caller's device arrays.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <numeric>
#include <string>
#include <unordered_set>
#include <vector>

#include "../../include/kda.h"
#include "kda_launch.h"
#include "kda_plan.h"


using namespace kda;

namespace {

thread_local std::string g_err;

kda_status fail(kda_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

kda_status ok() {
  g_err.clear();
  return KDA_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Largest accepted start position: positions plus a sequence length (at most
// 2^30) and a hash block stay far from int64 overflow.
constexpr int64_t kMaxStartPos = (int64_t)1 << 62;

// ---- optional per-kernel timing ------------------------------------------
struct TimedLaunch {
  const char* name;
  hipEvent_t ev0, ev1;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<TimedLaunch> g_prof_pending;
std::vector<kda_kernel_stat> g_prof_stats;
std::vector<hipEvent_t> g_event_pool;

hipEvent_t take_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Brackets one launch with events when timing is enabled.
class Launch {
 public:
  Launch(const char* name, hipStream_t st) : name_(name), st_(st) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (!g_prof_on) return;
    ev0_ = take_event();
    ev1_ = take_event();
    if (ev0_ && ev1_) hipEventRecord(ev0_, st_);
  }
  ~Launch() {
    if (!ev0_ || !ev1_) return;
    hipEventRecord(ev1_, st_);
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof_pending.push_back({name_, ev0_, ev1_});
  }

 private:
  const char* name_;
  hipStream_t st_;
  hipEvent_t ev0_ = nullptr, ev1_ = nullptr;
};

kda_status hip_fail(hipError_t e, const char* what) {
  return fail(KDA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

kda_status check_pool(const kda_pool* p) {
  if (!p) return fail(KDA_ERR_NULL, "pool descriptor is NULL");
  if (!p->base) return fail(KDA_ERR_POOL, "pool base is NULL");
  if (!aligned(p->base, 256)) return fail(KDA_ERR_POOL, "pool base must be 256-byte aligned");
  if (p->num_pages < 1 || p->num_heads < 1)
    return fail(KDA_ERR_POOL, "pool needs num_pages >= 1 and num_heads >= 1");
  if (p->d_k != p->d_v || (p->d_k != 64 && p->d_k != 128))
    return fail(KDA_ERR_SHAPE, "d_k == d_v in {64, 128} required (got %d, %d)", p->d_k, p->d_v);
  const int64_t need = (int64_t)p->num_heads * p->d_k * p->d_v * 4;
  if (p->page_bytes < need || p->page_bytes % 256 != 0)
    return fail(KDA_ERR_POOL, "page_bytes %lld must be a multiple of 256 and >= %lld",
                (long long)p->page_bytes, (long long)need);
  return KDA_OK;
}

bool valid_dtype(int d) { return d == KDA_F32 || d == KDA_BF16; }

int64_t state_bytes(const kda_pool* p) { return (int64_t)p->num_heads * p->d_k * p->d_v * 4; }

// Metadata region sizes inside the prefill workspace.
struct MetaLayout {
  int64_t seq_off, order_off, ckpt_off, inter_off;
};
MetaLayout meta_layout(int32_t num_seqs, int32_t num_ckpts) {
  MetaLayout m;
  m.seq_off = 0;
  m.order_off = align256((int64_t)num_seqs * (int64_t)sizeof(SeqEntry));
  m.ckpt_off = m.order_off + align256((int64_t)num_seqs * 4);
  m.inter_off = m.ckpt_off + align256((int64_t)num_ckpts * (int64_t)sizeof(CkptEntry));
  return m;
}

kda_status ship_metadata(uint8_t* ws, const std::vector<uint8_t>& blob, hipStream_t st) {
  for (size_t off = 0; off < blob.size(); off += kMetaChunkBytes) {
    MetaFillArgs a;
    std::memset(&a, 0, sizeof(a));
    const size_t n = std::min<size_t>(kMetaChunkBytes, blob.size() - off);
    a.dst = ws + off;
    a.nwords = (uint32_t)(n / 4);
    std::memcpy(a.words, blob.data() + off, n);
    Launch L("kda_meta_fill", st);
    hipError_t e = launch_meta_fill(a, st);
    if (e != hipSuccess) return hip_fail(e, "metadata fill launch");
  }
  return KDA_OK;
}

}  // namespace

namespace kda {
// error text shared with the host-only translation units (the prefix index)
void host_set_error(const char* msg) { g_err = msg; }
void host_clear_error() { g_err.clear(); }
}  // namespace kda

extern "C" {

int32_t kda_version(void) { return (1 << 16) | 0; }

const char* kda_last_error(void) { return g_err.c_str(); }

kda_status kda_pool_check(const kda_pool* pool) {
  kda_status s = check_pool(pool);
  return s == KDA_OK ? ok() : s;
}

int64_t kda_state_offset(const kda_pool* pool, int32_t page, int32_t head) {
  if (check_pool(pool) != KDA_OK) return -1;
  if (page < 0 || page >= pool->num_pages || head < 0 || head >= pool->num_heads) return -1;
  return (int64_t)page * pool->page_bytes + (int64_t)head * pool->d_k * pool->d_v * 4;
}

size_t kda_prefill_workspace_bytes(const kda_pool* pool, int64_t total_tokens, int32_t num_seqs,
                                   int32_t num_ckpts, kda_dtype in_dtype) {
  if (check_pool(pool) != KDA_OK || !valid_dtype(in_dtype) || total_tokens < 0 || num_seqs < 0 ||
      num_ckpts < 0)
    return 0;
  const int H = pool->num_heads, D = pool->d_k;
  const PrefillLayout m = prefill_layout(num_seqs, num_ckpts, H, D);
  const int64_t max_chunks = (total_tokens + 63) / 64 + num_seqs;
  const int64_t wc = std::min<int64_t>(default_window_chunks(H), std::max<int64_t>(max_chunks, 1));
  return (size_t)(m.inter_off + wc * H * inter_block_bytes(D, in_dtype == KDA_BF16 ? 2 : 4));
}

size_t kda_prefill_workspace_min_bytes(const kda_pool* pool, int32_t num_seqs, int32_t num_ckpts,
                                       kda_dtype in_dtype) {
  if (check_pool(pool) != KDA_OK || !valid_dtype(in_dtype) || num_seqs < 0 || num_ckpts < 0) return 0;
  const int H = pool->num_heads, D = pool->d_k;
  const PrefillLayout m = prefill_layout(num_seqs, num_ckpts, H, D);
  return (size_t)(m.inter_off + (int64_t)H * inter_block_bytes(D, in_dtype == KDA_BF16 ? 2 : 4));
}

}  // extern "C"

// The chunked prefill.  With `scratch` set, `workspace` is ignored: once the
// call has passed validation, scratch() supplies the workspace (the library's
// static device array, workspace_bytes long) and a call that does not fit it
// is rejected as such.
kda_status kda::prefill_impl(const kda_pool* pool, const void* q, const void* k, const void* v,
                             const void* g, const void* beta, kda_dtype in_dtype, void* o,
                             kda_dtype out_dtype, int32_t num_seqs, const int64_t* cu_seqlens,
                             const int64_t* start_pos, const int32_t* state_in_page,
                             const int32_t* state_out_page, const int32_t* ckpt_cu,
                             const int64_t* ckpt_pos, const int32_t* ckpt_page, int32_t chunk_size,
                             int32_t hash_block, void* workspace, size_t workspace_bytes,
                             kda_status (*scratch)(void**), void* stream) {
  kda_status s = check_pool(pool);
  if (s != KDA_OK) return s;
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype))
    return fail(KDA_ERR_DTYPE, "unknown dtype code (in %d, out %d)", (int)in_dtype, (int)out_dtype);
  if (chunk_size != 64) return fail(KDA_ERR_SHAPE, "chunk_size must be 64 (got %d)", chunk_size);
  if (hash_block <= 0 || hash_block % 64 != 0)
    return fail(KDA_ERR_SHAPE, "hash_block must be a positive multiple of 64 (got %d)", hash_block);
  if (num_seqs < 0) return fail(KDA_ERR_SEQ, "num_seqs < 0");
  if (num_seqs == 0) return ok();
  if (!cu_seqlens) return fail(KDA_ERR_NULL, "cu_seqlens is NULL");
  if (cu_seqlens[0] != 0) return fail(KDA_ERR_SEQ, "cu_seqlens[0] must be 0");
  const int D = pool->d_k, H = pool->num_heads, P = pool->num_pages;
  int64_t total_chunks = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    const int64_t len = cu_seqlens[i + 1] - cu_seqlens[i];
    if (len < 0) return fail(KDA_ERR_SEQ, "cu_seqlens decreases at %d", i);
    if (len > (int64_t)1 << 30) return fail(KDA_ERR_SEQ, "sequence %d longer than 2^30", i);
    const int64_t sp = start_pos ? start_pos[i] : 0;
    if (sp < 0 || sp % 64 != 0 || sp > kMaxStartPos)
      return fail(KDA_ERR_SEQ, "start_pos[%d] = %lld must be a multiple of 64 in [0, 2^62]", i,
                  (long long)sp);
    total_chunks += (len + 63) / 64;
  }
  const int64_t total_tokens = cu_seqlens[num_seqs];
  if (total_chunks > (int64_t)1 << 30) return fail(KDA_ERR_SEQ, "too many chunks");
  if (total_tokens > 0 && (!q || !k || !v || !g || !beta || !o))
    return fail(KDA_ERR_NULL, "q, k, v, g, beta and o must be non-NULL");
  for (const void* p : {q, k, v, g, static_cast<const void*>(o)})
    if (p && !aligned(p, 16)) return fail(KDA_ERR_SHAPE, "q, k, v, g, o must be 16-byte aligned");
  const int32_t num_ckpts = ckpt_cu ? ckpt_cu[num_seqs] : 0;
  if (ckpt_cu) {
    if (ckpt_cu[0] != 0) return fail(KDA_ERR_CKPT_RANGE, "ckpt_cu[0] must be 0");
    if (num_ckpts > 0 && (!ckpt_pos || !ckpt_page))
      return fail(KDA_ERR_NULL, "ckpt_pos / ckpt_page are NULL");
  }
  // pages, checkpoints, aliasing
  std::unordered_set<int32_t> reads, writes;
  for (int32_t i = 0; i < num_seqs; ++i) {
    const int32_t pi = state_in_page ? state_in_page[i] : -1;
    const int32_t po = state_out_page ? state_out_page[i] : -1;
    if (pi < -1 || pi >= P) return fail(KDA_ERR_PAGE_RANGE, "state_in_page[%d] = %d", i, pi);
    if (po < -1 || po >= P) return fail(KDA_ERR_PAGE_RANGE, "state_out_page[%d] = %d", i, po);
    if (pi >= 0) reads.insert(pi);
  }
  for (int32_t i = 0; i < num_seqs; ++i) {
    const int32_t pi = state_in_page ? state_in_page[i] : -1;
    const int32_t po = state_out_page ? state_out_page[i] : -1;
    if (po >= 0) {
      if (!writes.insert(po).second)
        return fail(KDA_ERR_PAGE_ALIAS, "destination page %d written twice", po);
      if (reads.count(po) && po != pi)
        return fail(KDA_ERR_PAGE_ALIAS, "state_out_page[%d] = %d is another sequence's input", i, po);
      if (po == pi) {
        for (int32_t j = 0; j < num_seqs; ++j)
          if (j != i && state_in_page && state_in_page[j] == po)
            return fail(KDA_ERR_PAGE_ALIAS, "in-place page %d is also read by sequence %d", po, j);
      }
    }
    if (!ckpt_cu) continue;
    if (ckpt_cu[i + 1] < ckpt_cu[i]) return fail(KDA_ERR_CKPT_RANGE, "ckpt_cu decreases at %d", i);
    const int64_t st = start_pos ? start_pos[i] : 0;
    const int64_t len = cu_seqlens[i + 1] - cu_seqlens[i];
    for (int32_t m = ckpt_cu[i]; m < ckpt_cu[i + 1]; ++m) {
      const int64_t pos = ckpt_pos[m];
      if (pos % hash_block != 0)
        return fail(KDA_ERR_CKPT_ALIGN, "checkpoint %d at %lld is not a multiple of %d", m,
                    (long long)pos, hash_block);
      if (pos <= st || pos > st + len || (m > ckpt_cu[i] && pos <= ckpt_pos[m - 1]))
        return fail(KDA_ERR_CKPT_RANGE, "checkpoint %d at %lld outside (%lld, %lld] or unordered", m,
                    (long long)pos, (long long)st, (long long)(st + len));
      const int32_t pg = ckpt_page[m];
      if (pg < 0 || pg >= P) return fail(KDA_ERR_PAGE_RANGE, "ckpt_page[%d] = %d", m, pg);
      if (reads.count(pg)) return fail(KDA_ERR_PAGE_ALIAS, "checkpoint page %d is also read", pg);
      if (!writes.insert(pg).second)
        return fail(KDA_ERR_PAGE_ALIAS, "destination page %d written twice", pg);
    }
  }
  const bool bf = in_dtype == KDA_BF16;
  const PrefillLayout ml = prefill_layout(num_seqs, num_ckpts, H, D);
  const int64_t blk = inter_block_bytes(D, bf ? 2 : 4);
  if ((int64_t)num_seqs * H > (int64_t)1 << 28) return fail(KDA_ERR_SHAPE, "too many (seq, head) pairs");
  // the kernels address one 64-token chunk of q/k/v/g with 32-bit offsets
  if ((int64_t)H * D > (int64_t)1 << 24) return fail(KDA_ERR_SHAPE, "num_heads * d_k above 2^24");
  const int32_t wc = fit_window_chunks(ml, H, blk, total_chunks, (int64_t)workspace_bytes);
  if (wc < 1) {
    const long long least = (long long)(ml.inter_off + (int64_t)H * blk);
    if (scratch)
      return fail(KDA_ERR_WORKSPACE,
                  "the call needs %lld bytes of workspace, above the static scratch of %zu bytes "
                  "(fewer sequences, checkpoints or heads per call)", least, workspace_bytes);
    return fail(KDA_ERR_WORKSPACE, "workspace too small: %zu < %lld bytes", workspace_bytes, least);
  }
  if (scratch) {
    s = scratch(&workspace);
    if (s != KDA_OK) return s;
  }
  if (!workspace) return fail(KDA_ERR_WORKSPACE, "workspace is NULL");
  if (!aligned(workspace, 256)) return fail(KDA_ERR_WORKSPACE, "workspace must be 256-byte aligned");

  // ---- metadata tables ------------------------------------------------------
  std::vector<uint8_t> blob((size_t)ml.carry_off, 0);
  SeqEntry* seqs = reinterpret_cast<SeqEntry*>(blob.data() + ml.seq_off);
  int32_t cb = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    SeqEntry& e = seqs[i];
    e.row_begin = cu_seqlens[i];
    e.start_pos = start_pos ? start_pos[i] : 0;
    e.len = (int32_t)(cu_seqlens[i + 1] - cu_seqlens[i]);
    e.chunk_begin = cb;
    cb += (e.len + 63) / 64;
    e.state_in = state_in_page ? state_in_page[i] : -1;
    e.state_out = state_out_page ? state_out_page[i] : -1;
    e.ckpt_begin = ckpt_cu ? ckpt_cu[i] : 0;
    e.ckpt_end = ckpt_cu ? ckpt_cu[i + 1] : 0;
  }
  CkptEntry* ck = reinterpret_cast<CkptEntry*>(blob.data() + ml.ckpt_off);
  for (int32_t m = 0; m < num_ckpts; ++m) {
    ck[m].pos = ckpt_pos[m];
    ck[m].page = ckpt_page[m];
    ck[m].pad = 0;
  }
  const std::vector<Window> wins = plan_windows(seqs, num_seqs, total_chunks, wc);

  // ---- launches --------------------------------------------------------------
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  // small tables travel inside the kernel arguments (no fill launch); larger
  // ones are shipped once, and each window's order table before its scan
  const bool inl = num_seqs <= kInlineSeqs && num_ckpts <= kInlineCkpts;
  if (!inl) {
    s = ship_metadata(ws, blob, st);
    if (s != KDA_OK) return s;
  }
  InlineSeqs iseq;
  InlineCkpts ick;
  std::memset(&iseq, 0, sizeof(iseq));
  std::memset(&ick, 0, sizeof(ick));
  if (inl) {
    std::memcpy(iseq.e, seqs, sizeof(SeqEntry) * num_seqs);
    std::memcpy(ick.e, ck, sizeof(CkptEntry) * num_ckpts);
  }
  uint8_t* inter = ws + ml.inter_off;
  float* carry[2] = {reinterpret_cast<float*>(ws + ml.carry_off),
                     reinterpret_cast<float*>(ws + ml.carry_off) + (int64_t)H * D * D};
  for (size_t w = 0; w < wins.size(); ++w) {
    const Window& win = wins[w];
    if (win.nch > 0) {
      PrepArgs pa{q, k, g, beta, reinterpret_cast<const SeqEntry*>(ws + ml.seq_off), num_seqs, H,
                  inter, blk, inl ? 1 : 0, win.c0, iseq};
      Launch L("kda_prefill_prep", st);
      hipError_t e = launch_prep(D, bf, pa, win.nch, st);
      if (e != hipSuccess) return hip_fail(e, "prep launch");
    }
    if (win.seqs.empty()) continue;
    const int32_t nw = (int32_t)win.seqs.size();
    if (inl) {
      std::memcpy(iseq.order, win.seqs.data(), sizeof(int32_t) * nw);
    } else {
      std::vector<uint8_t> ob((size_t)nw * 4);
      std::memcpy(ob.data(), win.seqs.data(), ob.size());
      s = ship_metadata(ws + ml.order_off, ob, st);
      if (s != KDA_OK) return s;
    }
    ScanArgs sa{v, o, out_dtype == KDA_BF16, H,
                reinterpret_cast<const SeqEntry*>(ws + ml.seq_off),
                reinterpret_cast<const int32_t*>(ws + ml.order_off),
                reinterpret_cast<const CkptEntry*>(ws + ml.ckpt_off), nw * H, win.c0, win.nch, 0,
                inter, blk, static_cast<uint8_t*>(pool->base), pool->page_bytes,
                carry[w & 1], carry[(w + 1) & 1], inl ? 1 : 0, 0, iseq, ick};
    Launch L("kda_prefill_scan", st);
    hipError_t e = launch_scan(D, bf, sa, st);
    if (e != hipSuccess) return hip_fail(e, "scan launch");
  }
  return ok();
}

extern "C" {

kda_status kda_prefill_chunked(const kda_pool* pool, const void* q, const void* k, const void* v,
                               const void* g, const void* beta, kda_dtype in_dtype, void* o,
                               kda_dtype out_dtype, int32_t num_seqs, const int64_t* cu_seqlens,
                               const int64_t* start_pos, const int32_t* state_in_page,
                               const int32_t* state_out_page, const int32_t* ckpt_cu,
                               const int64_t* ckpt_pos, const int32_t* ckpt_page,
                               int32_t chunk_size, int32_t hash_block, void* workspace,
                               size_t workspace_bytes, void* stream) {
  return prefill_impl(pool, q, k, v, g, beta, in_dtype, o, out_dtype, num_seqs, cu_seqlens,
                      start_pos, state_in_page, state_out_page, ckpt_cu, ckpt_pos, ckpt_page,
                      chunk_size, hash_block, workspace, workspace_bytes, nullptr, stream);
}

static kda_status decode_impl(const char* what, const kda_pool* pool, const void* q, const void* k,
                              const void* v, const void* g, const void* beta, kda_dtype in_dtype,
                              void* o, kda_dtype out_dtype, int32_t n, int32_t K,
                              const int32_t* page_in, const int32_t* page_out, void* stream) {
  kda_status s = check_pool(pool);
  if (s != KDA_OK) return s;
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype))
    return fail(KDA_ERR_DTYPE, "%s: unknown dtype code (in %d, out %d)", what, (int)in_dtype,
                (int)out_dtype);
  if (n < 0) return fail(KDA_ERR_SHAPE, "%s: n < 0", what);
  if (K < 1 || K > kMaxVerifyTokens)
    return fail(KDA_ERR_SHAPE, "%s: tokens per request %d outside [1, %d]", what, K, kMaxVerifyTokens);
  if (n == 0) return ok();
  if (!q || !k || !v || !g || !beta || !o || !page_in || !page_out)
    return fail(KDA_ERR_NULL, "%s: q, k, v, g, beta, o, page_in and page_out must be non-NULL", what);
  if ((int64_t)n * K * pool->num_heads > (int64_t)1 << 30)
    return fail(KDA_ERR_SHAPE, "%s: n * K * H too large", what);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const char* val = std::getenv("KDA_VALIDATE");
  if (val && val[0] == '1') {
    const int64_t nout = (int64_t)n * K;
    std::vector<int32_t> pin(n), pout(nout);
    hipError_t e = hipMemcpyAsync(pin.data(), page_in, n * 4, hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipMemcpyAsync(pout.data(), page_out, nout * 4, hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_fail(e, "page table read-back");
    std::unordered_set<int32_t> outs;
    for (int32_t r = 0; r < n; ++r)
      if (pin[r] < 0 || pin[r] >= pool->num_pages)
        return fail(KDA_ERR_PAGE_RANGE, "%s: request %d: page_in %d out of range", what, r, pin[r]);
    for (int64_t i = 0; i < nout; ++i) {
      if (pout[i] < 0 || pout[i] >= pool->num_pages)
        return fail(KDA_ERR_PAGE_RANGE, "%s: page_out[%lld] = %d out of range", what, (long long)i, pout[i]);
      if (!outs.insert(pout[i]).second)
        return fail(KDA_ERR_PAGE_ALIAS, "%s: page_out %d repeats", what, pout[i]);
    }
    for (int32_t r = 0; r < n; ++r)
      for (int64_t i = 0; i < nout; ++i)
        if (pout[i] == pin[r] && i / K != r)
          return fail(KDA_ERR_PAGE_ALIAS, "%s: page_in[%d] = %d is another request's output", what, r,
                      pin[r]);
  }
  DecodeArgs a{q, k, v, g, beta, o, page_in, page_out, static_cast<uint8_t*>(pool->base),
               pool->page_bytes, pool->num_pages, pool->num_heads, out_dtype == KDA_BF16, n, K};
  Launch L(K == 1 ? "kda_decode_step" : "kda_decode_verify", st);
  hipError_t e = launch_decode(pool->d_k, in_dtype == KDA_BF16, a, st);
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return ok();
}

kda_status kda_decode_step(const kda_pool* pool, const void* q, const void* k, const void* v,
                           const void* g, const void* beta, kda_dtype in_dtype, void* o,
                           kda_dtype out_dtype, int32_t n, const int32_t* page_in,
                           const int32_t* page_out, void* stream) {
  return decode_impl("kda_decode_step", pool, q, k, v, g, beta, in_dtype, o, out_dtype, n, 1, page_in,
                     page_out, stream);
}

kda_status kda_decode_verify(const kda_pool* pool, const void* q, const void* k, const void* v,
                             const void* g, const void* beta, kda_dtype in_dtype, void* o,
                             kda_dtype out_dtype, int32_t n, int32_t tokens, const int32_t* page_in,
                             const int32_t* page_out, void* stream) {
  return decode_impl("kda_decode_verify", pool, q, k, v, g, beta, in_dtype, o, out_dtype, n, tokens,
                     page_in, page_out, stream);
}

static kda_status copy_pages(const char* what, const kda_pool* pool, const int32_t* src,
                             const int32_t* dst, int32_t n, void* stream) {
  kda_status s = check_pool(pool);
  if (s != KDA_OK) return s;
  if (n < 0) return fail(KDA_ERR_SHAPE, "%s: n < 0", what);
  if (n == 0) return ok();
  if (!src || !dst) return fail(KDA_ERR_NULL, "%s: page arrays are NULL", what);
  std::unordered_set<int32_t> srcs, dsts;
  for (int32_t i = 0; i < n; ++i) {
    if (src[i] < 0 || src[i] >= pool->num_pages || dst[i] < 0 || dst[i] >= pool->num_pages)
      return fail(KDA_ERR_PAGE_RANGE, "%s: pair %d (%d -> %d) out of range", what, i, src[i], dst[i]);
    srcs.insert(src[i]);
    if (!dsts.insert(dst[i]).second)
      return fail(KDA_ERR_PAGE_ALIAS, "%s: destination page %d repeats", what, dst[i]);
  }
  for (int32_t i = 0; i < n; ++i)
    if (srcs.count(dst[i]))
      return fail(KDA_ERR_PAGE_ALIAS, "%s: destination page %d is also a source", what, dst[i]);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int64_t sb = state_bytes(pool);
  for (int32_t b = 0; b < n; b += kCopyPairsPerLaunch) {
    CopyArgs a;
    a.pool = static_cast<uint8_t*>(pool->base);
    a.page_bytes = pool->page_bytes;
    a.state_bytes = sb;
    a.pieces = (int32_t)((sb + kPieceBytes - 1) / kPieceBytes);
    a.npairs = std::min(kCopyPairsPerLaunch, n - b);
    for (int32_t i = 0; i < a.npairs; ++i) {
      a.src[i] = src[b + i];
      a.dst[i] = dst[b + i];
    }
    Launch L("kda_page_copy", st);
    hipError_t e = launch_copy(a, st);
    if (e != hipSuccess) return hip_fail(e, "copy launch");
  }
  return ok();
}

kda_status kda_checkpoint_write(const kda_pool* pool, const int32_t* src_active,
                                const int32_t* dst_ckpt, int32_t n, void* stream) {
  return copy_pages("kda_checkpoint_write", pool, src_active, dst_ckpt, n, stream);
}

kda_status kda_checkpoint_restore(const kda_pool* pool, const int32_t* src_ckpt,
                                  const int32_t* dst_active, int32_t n, void* stream) {
  return copy_pages("kda_checkpoint_restore", pool, src_ckpt, dst_active, n, stream);
}

// ---- short causal convolution --------------------------------------------------

int64_t kda_conv_workspace_bytes(int32_t num_seqs, int32_t num_ckpts) {
  if (num_seqs < 0 || num_ckpts < 0) return -1;
  return meta_layout(num_seqs, num_ckpts).inter_off;
}

static kda_status check_conv_pool(const kda_conv_pool* p) {
  if (!p) return fail(KDA_ERR_NULL, "kda_short_conv: conv pool descriptor is NULL");
  if (!p->base) return fail(KDA_ERR_POOL, "kda_short_conv: conv pool base is NULL");
  if (!aligned(p->base, 256)) return fail(KDA_ERR_POOL, "kda_short_conv: conv pool base must be 256-byte aligned");
  if (p->num_pages < 1) return fail(KDA_ERR_POOL, "kda_short_conv: conv pool needs num_pages >= 1");
  if (p->width < 2 || p->width > 4) return fail(KDA_ERR_SHAPE, "kda_short_conv: width %d not in {2, 3, 4}", p->width);
  if (!valid_dtype(p->dtype)) return fail(KDA_ERR_DTYPE, "kda_short_conv: unknown dtype code %d", p->dtype);
  const int vec = p->dtype == KDA_BF16 ? 8 : 4;
  if (p->channels < vec || p->channels % vec != 0 || p->channels > (1 << 24))
    return fail(KDA_ERR_SHAPE, "kda_short_conv: channels %d must be a positive multiple of %d", p->channels, vec);
  const int64_t need = (int64_t)(p->width - 1) * p->channels * (p->dtype == KDA_BF16 ? 2 : 4);
  if (p->page_bytes < need || p->page_bytes % 256 != 0)
    return fail(KDA_ERR_POOL, "kda_short_conv: page_bytes %lld must be a multiple of 256 and >= %lld",
                (long long)p->page_bytes, (long long)need);
  return KDA_OK;
}

kda_status kda_short_conv(const kda_conv_pool* cpool, const void* x, const float* w, void* y,
                          kda_dtype out_dtype, int32_t num_seqs, const int64_t* cu_seqlens,
                          const int64_t* start_pos, const int32_t* state_in_page,
                          const int32_t* state_out_page, const int32_t* ckpt_cu,
                          const int64_t* ckpt_pos, const int32_t* ckpt_page, int32_t hash_block,
                          void* workspace, size_t workspace_bytes, void* stream) {
  const char* what = "kda_short_conv";
  kda_status s = check_conv_pool(cpool);
  if (s != KDA_OK) return s;
  if (!valid_dtype(out_dtype)) return fail(KDA_ERR_DTYPE, "%s: unknown out dtype %d", what, (int)out_dtype);
  if (hash_block <= 0 || hash_block % 64 != 0)
    return fail(KDA_ERR_SHAPE, "%s: hash_block must be a positive multiple of 64 (got %d)", what, hash_block);
  if (num_seqs < 0) return fail(KDA_ERR_SEQ, "%s: num_seqs < 0", what);
  if (num_seqs == 0) return ok();
  if (!cu_seqlens) return fail(KDA_ERR_NULL, "%s: cu_seqlens is NULL", what);
  if (cu_seqlens[0] != 0) return fail(KDA_ERR_SEQ, "%s: cu_seqlens[0] must be 0", what);
  const int32_t P = cpool->num_pages;
  int64_t total_chunks = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    const int64_t len = cu_seqlens[i + 1] - cu_seqlens[i];
    if (len < 0) return fail(KDA_ERR_SEQ, "%s: cu_seqlens decreases at %d", what, i);
    if (len > (int64_t)1 << 30) return fail(KDA_ERR_SEQ, "%s: sequence %d longer than 2^30", what, i);
    const int64_t sp = start_pos ? start_pos[i] : 0;
    if (sp < 0 || sp > kMaxStartPos) return fail(KDA_ERR_SEQ, "%s: start_pos[%d] outside [0, 2^62]", what, i);
    const int32_t po = state_out_page ? state_out_page[i] : -1;
    total_chunks += len > 0 ? (len + 63) / 64 : (po >= 0 ? 1 : 0);
  }
  if (total_chunks > (int64_t)1 << 28) return fail(KDA_ERR_SEQ, "%s: too many tokens", what);
  const int64_t total_tokens = cu_seqlens[num_seqs];
  if (total_tokens > 0 && (!x || !y)) return fail(KDA_ERR_NULL, "%s: x and y must be non-NULL", what);
  if (!w) return fail(KDA_ERR_NULL, "%s: weights are NULL", what);
  for (const void* p : {x, static_cast<const void*>(y), static_cast<const void*>(w)})
    if (p && !aligned(p, 16)) return fail(KDA_ERR_SHAPE, "%s: x, y, w must be 16-byte aligned", what);
  if (x && x == y) return fail(KDA_ERR_SHAPE, "%s: y may not alias x", what);
  const int32_t num_ckpts = ckpt_cu ? ckpt_cu[num_seqs] : 0;
  if (ckpt_cu) {
    if (ckpt_cu[0] != 0) return fail(KDA_ERR_CKPT_RANGE, "%s: ckpt_cu[0] must be 0", what);
    if (num_ckpts > 0 && (!ckpt_pos || !ckpt_page)) return fail(KDA_ERR_NULL, "%s: ckpt_pos / ckpt_page are NULL", what);
  }
  std::unordered_set<int32_t> reads, writes;
  for (int32_t i = 0; i < num_seqs; ++i) {
    const int32_t pi = state_in_page ? state_in_page[i] : -1;
    const int32_t po = state_out_page ? state_out_page[i] : -1;
    if (pi < -1 || pi >= P) return fail(KDA_ERR_PAGE_RANGE, "%s: state_in_page[%d] = %d", what, i, pi);
    if (po < -1 || po >= P) return fail(KDA_ERR_PAGE_RANGE, "%s: state_out_page[%d] = %d", what, i, po);
    if (pi >= 0) reads.insert(pi);
  }
  for (int32_t i = 0; i < num_seqs; ++i) {
    const int32_t po = state_out_page ? state_out_page[i] : -1;
    if (po >= 0) {
      if (reads.count(po)) return fail(KDA_ERR_PAGE_ALIAS, "%s: output page %d is also an input page", what, po);
      if (!writes.insert(po).second) return fail(KDA_ERR_PAGE_ALIAS, "%s: page %d written twice", what, po);
    }
    if (!ckpt_cu) continue;
    if (ckpt_cu[i + 1] < ckpt_cu[i]) return fail(KDA_ERR_CKPT_RANGE, "%s: ckpt_cu decreases at %d", what, i);
    const int64_t st = start_pos ? start_pos[i] : 0;
    const int64_t len = cu_seqlens[i + 1] - cu_seqlens[i];
    for (int32_t m = ckpt_cu[i]; m < ckpt_cu[i + 1]; ++m) {
      const int64_t pos = ckpt_pos[m];
      if (pos % hash_block != 0)
        return fail(KDA_ERR_CKPT_ALIGN, "%s: checkpoint %d at %lld is not a multiple of %d", what, m,
                    (long long)pos, hash_block);
      if (pos <= st || pos > st + len || (m > ckpt_cu[i] && pos <= ckpt_pos[m - 1]))
        return fail(KDA_ERR_CKPT_RANGE, "%s: checkpoint %d at %lld outside (%lld, %lld] or unordered", what,
                    m, (long long)pos, (long long)st, (long long)(st + len));
      const int32_t pg = ckpt_page[m];
      if (pg < 0 || pg >= P) return fail(KDA_ERR_PAGE_RANGE, "%s: ckpt_page[%d] = %d", what, m, pg);
      if (reads.count(pg)) return fail(KDA_ERR_PAGE_ALIAS, "%s: checkpoint page %d is also an input page", what, pg);
      if (!writes.insert(pg).second) return fail(KDA_ERR_PAGE_ALIAS, "%s: page %d written twice", what, pg);
    }
  }
  const MetaLayout ml = meta_layout(num_seqs, num_ckpts);
  if (!workspace) return fail(KDA_ERR_WORKSPACE, "%s: workspace is NULL", what);
  if (!aligned(workspace, 256)) return fail(KDA_ERR_WORKSPACE, "%s: workspace must be 256-byte aligned", what);
  if ((int64_t)workspace_bytes < ml.inter_off)
    return fail(KDA_ERR_WORKSPACE, "%s: workspace too small: %zu < %lld bytes", what, workspace_bytes,
                (long long)ml.inter_off);
  if (total_chunks == 0) return ok();

  std::vector<uint8_t> blob((size_t)ml.inter_off, 0);
  SeqEntry* seqs = reinterpret_cast<SeqEntry*>(blob.data() + ml.seq_off);
  int32_t cb = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    SeqEntry& e = seqs[i];
    e.row_begin = cu_seqlens[i];
    e.start_pos = start_pos ? start_pos[i] : 0;
    e.len = (int32_t)(cu_seqlens[i + 1] - cu_seqlens[i]);
    e.chunk_begin = cb;
    e.state_in = state_in_page ? state_in_page[i] : -1;
    e.state_out = state_out_page ? state_out_page[i] : -1;
    cb += e.len > 0 ? (e.len + 63) / 64 : (e.state_out >= 0 ? 1 : 0);
    e.ckpt_begin = ckpt_cu ? ckpt_cu[i] : 0;
    e.ckpt_end = ckpt_cu ? ckpt_cu[i + 1] : 0;
  }
  CkptEntry* ck = reinterpret_cast<CkptEntry*>(blob.data() + ml.ckpt_off);
  for (int32_t m = 0; m < num_ckpts; ++m) {
    ck[m].pos = ckpt_pos[m];
    ck[m].page = ckpt_page[m];
  }
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  s = ship_metadata(ws, blob, st);
  if (s != KDA_OK) return s;
  ConvArgs a{x, w, y, reinterpret_cast<const SeqEntry*>(ws + ml.seq_off),
             reinterpret_cast<const CkptEntry*>(ws + ml.ckpt_off), static_cast<uint8_t*>(cpool->base),
             cpool->page_bytes, num_seqs, cpool->channels, cpool->width, cpool->dtype == KDA_BF16,
             out_dtype == KDA_BF16, hash_block};
  Launch L("kda_short_conv", st);
  hipError_t e = launch_conv(a, (int32_t)total_chunks, st);
  if (e != hipSuccess) return hip_fail(e, "conv launch");
  return ok();
}

kda_status kda_short_conv_update(const kda_conv_pool* cpool, const void* x, const float* w, void* y,
                                 kda_dtype out_dtype, int32_t n, const int32_t* page_in,
                                 const int32_t* page_out, void* stream) {
  const char* what = "kda_short_conv_update";
  kda_status s = check_conv_pool(cpool);
  if (s != KDA_OK) return s;
  if (!valid_dtype(out_dtype)) return fail(KDA_ERR_DTYPE, "%s: unknown out dtype %d", what, (int)out_dtype);
  if (n < 0) return fail(KDA_ERR_SHAPE, "%s: n < 0", what);
  if (n == 0) return ok();
  if (!x || !y || !w || !page_in || !page_out)
    return fail(KDA_ERR_NULL, "%s: x, w, y, page_in and page_out must be non-NULL", what);
  for (const void* p : {x, static_cast<const void*>(y), static_cast<const void*>(w)})
    if (!aligned(p, 16)) return fail(KDA_ERR_SHAPE, "%s: x, y, w must be 16-byte aligned", what);
  if (x == y) return fail(KDA_ERR_SHAPE, "%s: y may not alias x", what);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const char* val = std::getenv("KDA_VALIDATE");
  if (val && val[0] == '1') {
    std::vector<int32_t> pin(n), pout(n);
    hipError_t e = hipMemcpyAsync(pin.data(), page_in, (size_t)n * 4, hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipMemcpyAsync(pout.data(), page_out, (size_t)n * 4, hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_fail(e, "page table read-back");
    std::unordered_set<int32_t> outs;
    for (int32_t r = 0; r < n; ++r) {
      if (pin[r] < 0 || pin[r] >= cpool->num_pages)
        return fail(KDA_ERR_PAGE_RANGE, "%s: request %d: page_in %d out of range", what, r, pin[r]);
      if (pout[r] < 0 || pout[r] >= cpool->num_pages)
        return fail(KDA_ERR_PAGE_RANGE, "%s: request %d: page_out %d out of range", what, r, pout[r]);
      if (!outs.insert(pout[r]).second) return fail(KDA_ERR_PAGE_ALIAS, "%s: page_out %d repeats", what, pout[r]);
    }
    for (int32_t r = 0; r < n; ++r)
      if (outs.count(pin[r]) && pout[r] != pin[r])
        return fail(KDA_ERR_PAGE_ALIAS, "%s: page_in[%d] = %d is another request's output", what, r, pin[r]);
  }
  ConvUpdateArgs a{x, w, y, page_in, page_out, static_cast<uint8_t*>(cpool->base), cpool->page_bytes,
                   cpool->num_pages, n, cpool->channels, cpool->width, cpool->dtype == KDA_BF16,
                   out_dtype == KDA_BF16};
  Launch L("kda_short_conv_update", st);
  hipError_t e = launch_conv_update(a, st);
  if (e != hipSuccess) return hip_fail(e, "conv update launch");
  return ok();
}

// ---- int8 compressed checkpoints ----------------------------------------------

int64_t kda_ckpt_int8_head_bytes(int32_t d_k, int32_t d_v) {
  if (d_k != d_v || (d_k != 64 && d_k != 128)) return -1;
  return int8_head_bytes(d_k);
}

static kda_status check_qpool(const char* what, const kda_pool* pool, const kda_pool* qpool) {
  kda_status s = check_pool(pool);
  if (s != KDA_OK) return s;
  if (!qpool) return fail(KDA_ERR_NULL, "%s: qpool descriptor is NULL", what);
  if (!qpool->base) return fail(KDA_ERR_POOL, "%s: qpool base is NULL", what);
  if (!aligned(qpool->base, 256)) return fail(KDA_ERR_POOL, "%s: qpool base must be 256-byte aligned", what);
  if (qpool->num_pages < 1) return fail(KDA_ERR_POOL, "%s: qpool needs num_pages >= 1", what);
  if (qpool->num_heads != pool->num_heads || qpool->d_k != pool->d_k || qpool->d_v != pool->d_v)
    return fail(KDA_ERR_SHAPE, "%s: qpool heads/dims (%d, %d, %d) differ from the pool's (%d, %d, %d)",
                what, qpool->num_heads, qpool->d_k, qpool->d_v, pool->num_heads, pool->d_k, pool->d_v);
  const int64_t need = (int64_t)qpool->num_heads * int8_head_bytes(qpool->d_k);
  if (qpool->page_bytes < need || qpool->page_bytes % 256 != 0)
    return fail(KDA_ERR_POOL, "%s: qpool page_bytes %lld must be a multiple of 256 and >= %lld", what,
                (long long)qpool->page_bytes, (long long)need);
  const uintptr_t p0 = reinterpret_cast<uintptr_t>(pool->base);
  const uintptr_t p1 = p0 + (uintptr_t)pool->num_pages * (uintptr_t)pool->page_bytes;
  const uintptr_t q0 = reinterpret_cast<uintptr_t>(qpool->base);
  const uintptr_t q1 = q0 + (uintptr_t)qpool->num_pages * (uintptr_t)qpool->page_bytes;
  if (p0 < q1 && q0 < p1) return fail(KDA_ERR_PAGE_ALIAS, "%s: pool and qpool byte ranges overlap", what);
  return KDA_OK;
}

// src pages index `src_pool`'s range, dst pages `dst_pool`'s.
static kda_status quant_pages(const char* what, bool to_int8, const kda_pool* pool,
                              const kda_pool* qpool, const int32_t* src, int32_t src_pages,
                              const int32_t* dst, int32_t dst_pages, int32_t n, void* stream) {
  kda_status s = check_qpool(what, pool, qpool);
  if (s != KDA_OK) return s;
  if (n < 0) return fail(KDA_ERR_SHAPE, "%s: n < 0", what);
  if (n == 0) return ok();
  if (!src || !dst) return fail(KDA_ERR_NULL, "%s: page arrays are NULL", what);
  std::unordered_set<int32_t> dsts;
  for (int32_t i = 0; i < n; ++i) {
    if (src[i] < 0 || src[i] >= src_pages || dst[i] < 0 || dst[i] >= dst_pages)
      return fail(KDA_ERR_PAGE_RANGE, "%s: pair %d (%d -> %d) out of range", what, i, src[i], dst[i]);
    if (!dsts.insert(dst[i]).second)
      return fail(KDA_ERR_PAGE_ALIAS, "%s: destination page %d repeats", what, dst[i]);
  }
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  for (int32_t b = 0; b < n; b += kCopyPairsPerLaunch) {
    QuantArgs a;
    a.pool = static_cast<uint8_t*>(pool->base);
    a.page_bytes = pool->page_bytes;
    a.qpool = static_cast<uint8_t*>(qpool->base);
    a.qpage_bytes = qpool->page_bytes;
    a.H = pool->num_heads;
    a.npairs = std::min(kCopyPairsPerLaunch, n - b);
    for (int32_t i = 0; i < a.npairs; ++i) {
      a.src[i] = src[b + i];
      a.dst[i] = dst[b + i];
    }
    Launch L(to_int8 ? "kda_ckpt_quant" : "kda_ckpt_dequant", st);
    hipError_t e = to_int8 ? launch_quant(pool->d_k, a, st) : launch_dequant(pool->d_k, a, st);
    if (e != hipSuccess) return hip_fail(e, to_int8 ? "quantise launch" : "dequantise launch");
  }
  return ok();
}

kda_status kda_checkpoint_write_int8(const kda_pool* pool, const int32_t* src_active,
                                     const kda_pool* qpool, const int32_t* dst_qckpt, int32_t n,
                                     void* stream) {
  if (!pool || !qpool) return fail(KDA_ERR_NULL, "kda_checkpoint_write_int8: pool descriptor is NULL");
  return quant_pages("kda_checkpoint_write_int8", true, pool, qpool, src_active, pool->num_pages,
                     dst_qckpt, qpool->num_pages, n, stream);
}

kda_status kda_checkpoint_restore_int8(const kda_pool* qpool, const int32_t* src_qckpt,
                                       const kda_pool* pool, const int32_t* dst_active, int32_t n,
                                       void* stream) {
  if (!pool || !qpool) return fail(KDA_ERR_NULL, "kda_checkpoint_restore_int8: pool descriptor is NULL");
  return quant_pages("kda_checkpoint_restore_int8", false, pool, qpool, src_qckpt, qpool->num_pages,
                     dst_active, pool->num_pages, n, stream);
}

kda_status kda_profile_enable(int32_t on) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_on = on != 0;
  return ok();
}

int32_t kda_profile_read(kda_kernel_stat* out, int32_t max_entries, int32_t reset) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (const TimedLaunch& t : g_prof_pending) {
    float ms = 0.f;
    if (hipEventSynchronize(t.ev1) == hipSuccess && hipEventElapsedTime(&ms, t.ev0, t.ev1) == hipSuccess) {
      auto it = std::find_if(g_prof_stats.begin(), g_prof_stats.end(),
                             [&](const kda_kernel_stat& s) { return std::strcmp(s.name, t.name) == 0; });
      if (it == g_prof_stats.end()) {
        kda_kernel_stat s;
        std::memset(&s, 0, sizeof(s));
        std::snprintf(s.name, sizeof(s.name), "%s", t.name);
        g_prof_stats.push_back(s);
        it = g_prof_stats.end() - 1;
      }
      it->launches += 1;
      it->total_ms += ms;
    }
    g_event_pool.push_back(t.ev0);
    g_event_pool.push_back(t.ev1);
  }
  g_prof_pending.clear();
  const int32_t n = std::min<int32_t>((int32_t)g_prof_stats.size(), std::max(0, max_entries));
  if (out)
    for (int32_t i = 0; i < n; ++i) out[i] = g_prof_stats[i];
  const int32_t total = (int32_t)g_prof_stats.size();
  if (reset) g_prof_stats.clear();
  return out ? n : total;
}

}  // extern "C"
