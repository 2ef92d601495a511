// kda_meta.h -- per-call metadata tables shared by the host launcher and the
// prefill kernels.  The host validates the caller's arrays, packs these tables,
// and ships them into the caller's workspace through kernel arguments.
#pragma once
#include <stdint.h>

namespace kda {

// One packed sequence of a prefill call.
struct SeqEntry {
  int64_t row_begin;    // first token row in q/k/v/g/beta/o
  int64_t start_pos;    // absolute position of that token (multiple of 64)
  int32_t len;          // tokens in this call
  int32_t chunk_begin;  // global index of the sequence's first 64-token chunk
  int32_t state_in;     // page with the entering state, or -1 (zero state)
  int32_t state_out;    // page receiving the final state, or -1
  int32_t ckpt_begin;   // [ckpt_begin, ckpt_end) in the checkpoint table
  int32_t ckpt_end;
};
static_assert(sizeof(SeqEntry) == 40, "SeqEntry layout");

struct CkptEntry {
  int64_t pos;   // absolute position P: the state after P tokens
  int32_t page;  // destination page
  int32_t pad;
};
static_assert(sizeof(CkptEntry) == 16, "CkptEntry layout");

// Workspace bytes per (chunk, head) block of prefill intermediates, element
// type Op (bf16 or fp32):
//   Keff [64][D], Qt [64][D], KendT [D][64], T [64][64], Aq [64][64],
//   then gammaC [D] fp32; padded to 256 bytes.  With bf16 operands the two
//   16x32 fragments right of the diagonal in row tiles 0 and 1 of T and of
//   Aq are zero, never written and never read.
inline constexpr int64_t inter_elems(int D) { return 3LL * 64 * D + 2LL * 64 * 64; }
inline constexpr int64_t inter_block_bytes(int D, int op_bytes) {
  return ((inter_elems(D) * op_bytes + 4LL * D) + 255) / 256 * 256;
}

constexpr int kMetaChunkBytes = 2048;  // payload of one metadata-fill launch

struct MetaFillArgs {
  uint8_t* dst;
  uint32_t nwords;
  uint32_t pad;
  uint32_t words[kMetaChunkBytes / 4];
};

}  // namespace kda
