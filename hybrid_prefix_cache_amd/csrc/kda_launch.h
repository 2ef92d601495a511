// kda_launch.h -- kernel-argument structs and launch entry points shared by the
// host launcher (kda_api.cpp) and the kernel translation units.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kda.h"
#include "kda_meta.h"

namespace kda {

// Small calls carry their sequence and checkpoint tables inside the kernel
// arguments (read from the kernel-argument segment with scalar loads), which
// saves the table-fill launch; larger ones read them from the workspace.
constexpr int kInlineSeqs = 16;
constexpr int kInlineCkpts = 64;
struct InlineSeqs {
  SeqEntry e[kInlineSeqs];
  int32_t order[kInlineSeqs];  // the window's sequences by descending chunk count
};
struct InlineCkpts {
  CkptEntry e[kInlineCkpts];
};

struct PrepArgs {
  const void* q;
  const void* k;
  const void* g;
  const void* beta;
  const SeqEntry* seqs;  // workspace table (when !inline_meta)
  int32_t num_seqs;
  int32_t H;
  uint8_t* inter;         // block of chunk c, head h at ((c - chunk0) * H + h) * blk_bytes
  int64_t blk_bytes;
  int32_t inline_meta;
  int32_t chunk0;         // first global chunk of the window
  InlineSeqs iseq;
};

// One window of a prefill call: global chunks [c0, c0 + nch).  Each of its
// sequences runs the part of its chunks inside the window; a sequence that
// began in an earlier window enters with the carried state (carry_in), one
// that continues past the window leaves its state in carry_out.
struct ScanArgs {
  const void* v;
  void* o;
  int32_t out_bf16;
  int32_t H;
  const SeqEntry* seqs;
  const int32_t* order;  // the window's sequences by descending chunk count
  const CkptEntry* ckpts;
  int32_t npairs;  // (sequences in the window) * H
  int32_t c0;      // first global chunk of the window
  int32_t nch;     // chunks in the window
  int32_t pad;
  const uint8_t* inter;
  int64_t blk_bytes;
  uint8_t* pool;
  int64_t page_bytes;
  const float* carry_in;  // [H][D][D] fp32
  float* carry_out;       // [H][D][D] fp32 (never the same buffer as carry_in)
  int32_t inline_meta;
  int32_t pad2;
  InlineSeqs iseq;
  InlineCkpts ick;
};
static_assert(sizeof(ScanArgs) <= 4096 && sizeof(PrepArgs) <= 4096, "kernel argument budget");

constexpr int kMaxVerifyTokens = 64;  // tokens per request in one decode launch

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* g;
  const void* beta;
  void* o;
  const int32_t* page_in;
  const int32_t* page_out;
  uint8_t* pool;
  int64_t page_bytes;
  int32_t num_pages;
  int32_t H;
  int32_t out_bf16;
  int32_t n;   // requests
  int32_t K;   // tokens per request: rows r*K + t, state after token t -> page_out[r*K + t]
};

constexpr int kCopyPairsPerLaunch = 448;
constexpr int kPieceBytes = 4096;  // bytes per copy workgroup: one 16-byte vector per thread

struct CopyArgs {
  uint8_t* pool;
  int64_t page_bytes;
  int64_t state_bytes;  // bytes copied per page
  int32_t pieces;       // ceil(state_bytes / kPieceBytes)
  int32_t npairs;
  int32_t src[kCopyPairsPerLaunch];
  int32_t dst[kCopyPairsPerLaunch];
};
static_assert(sizeof(CopyArgs) <= 4096, "kernel argument budget");

// Page pairs of one int8 checkpoint write (src in pool, dst in qpool) or
// restore (src in qpool, dst in pool) launch.
struct QuantArgs {
  uint8_t* pool;
  int64_t page_bytes;
  uint8_t* qpool;
  int64_t qpage_bytes;
  int32_t H;
  int32_t npairs;
  int32_t src[kCopyPairsPerLaunch];
  int32_t dst[kCopyPairsPerLaunch];
};
static_assert(sizeof(QuantArgs) <= 4096, "kernel argument budget");

// Bytes of one head in a compressed page: int8 q[d][d], then fp32 scale[d].
constexpr int64_t int8_head_bytes(int D) { return (int64_t)D * D + 4LL * D; }
static_assert(sizeof(MetaFillArgs) <= 4096, "kernel argument budget");

hipError_t launch_meta_fill(const MetaFillArgs& a, hipStream_t st);
hipError_t launch_prep(int D, bool bf16, const PrepArgs& a, int total_chunks, hipStream_t st);
hipError_t launch_scan(int D, bool bf16, const ScanArgs& a, hipStream_t st);
hipError_t launch_decode(int D, bool bf16, const DecodeArgs& a, hipStream_t st);
// Sequence owning a global chunk index: the largest s with
// seqs[s].chunk_begin <= chunk (chunk tables are increasing).
template <typename SeqPtr>
__device__ __forceinline__ int find_seq(SeqPtr seqs, int n, int chunk) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (seqs[mid].chunk_begin <= chunk) lo = mid; else hi = mid - 1;
  }
  return lo;
}
// The sequence table seen through the constant address space: uniform reads
// of it are scalar loads even after the kernel has stored to global memory.
typedef const __attribute__((address_space(4))) SeqEntry* ConstSeqPtr;
// The checkpoint table through the constant address space (scalar loads).
typedef const __attribute__((address_space(4))) CkptEntry* ConstCkptPtr;

__device__ __forceinline__ SeqEntry load_seq(ConstSeqPtr p, int i) {
  SeqEntry e;
  e.row_begin = p[i].row_begin;
  e.start_pos = p[i].start_pos;
  e.len = p[i].len;
  e.chunk_begin = p[i].chunk_begin;
  e.state_in = p[i].state_in;
  e.state_out = p[i].state_out;
  e.ckpt_begin = p[i].ckpt_begin;
  e.ckpt_end = p[i].ckpt_end;
  return e;
}
// Sequence i of a prefill call, from the kernel arguments or from the
// workspace table.
template <typename Args>
__device__ __forceinline__ SeqEntry seq_at(const Args& a, int i) {
  return a.inline_meta ? a.iseq.e[i] : load_seq((ConstSeqPtr)(a.seqs), i);
}
// Largest s with seq_at(a, s).chunk_begin <= chunk.
template <typename Args>
__device__ __forceinline__ int find_seq_in(const Args& a, int chunk) {
  int lo = 0, hi = a.num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (seq_at(a, mid).chunk_begin <= chunk) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// One kda_short_conv call: 16-token blocks of the 64-token chunks of the
// sequence table, by channel groups.
struct ConvArgs {
  const void* x;
  const float* w;
  void* y;
  const SeqEntry* seqs;
  const CkptEntry* ckpts;
  uint8_t* cpool;
  int64_t cpage_bytes;
  int32_t num_seqs;
  int32_t C;
  int32_t W;
  int32_t in_bf16;
  int32_t out_bf16;
  int32_t hash_block;
};

// The chunked prefill behind kda_prefill_chunked (scratch == nullptr) and
// kda_prefill_chunked_noalloc (scratch supplies the static workspace after
// validation).
kda_status prefill_impl(const kda_pool* pool, const void* q, const void* k, const void* v,
                        const void* g, const void* beta, kda_dtype in_dtype, void* o,
                        kda_dtype out_dtype, int32_t num_seqs, const int64_t* cu_seqlens,
                        const int64_t* start_pos, const int32_t* state_in_page,
                        const int32_t* state_out_page, const int32_t* ckpt_cu,
                        const int64_t* ckpt_pos, const int32_t* ckpt_page, int32_t chunk_size,
                        int32_t hash_block, void* workspace, size_t workspace_bytes,
                        kda_status (*scratch)(void**), void* stream);

// One kda_short_conv_update call: request r's window page_in[r] and token
// row r of x -> y row r and the next window in page_out[r].
struct ConvUpdateArgs {
  const void* x;
  const float* w;
  void* y;
  const int32_t* page_in;   // device [n]
  const int32_t* page_out;  // device [n]
  uint8_t* cpool;
  int64_t cpage_bytes;
  int32_t num_pages;
  int32_t n;
  int32_t C;
  int32_t W;
  int32_t in_bf16;
  int32_t out_bf16;
};

hipError_t launch_copy(const CopyArgs& a, hipStream_t st);
hipError_t launch_conv(const ConvArgs& a, int32_t total_chunks, hipStream_t st);
hipError_t launch_conv_update(const ConvUpdateArgs& a, hipStream_t st);
hipError_t launch_quant(int D, const QuantArgs& a, hipStream_t st);
hipError_t launch_dequant(int D, const QuantArgs& a, hipStream_t st);

}  // namespace kda
