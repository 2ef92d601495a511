// kda_plan.h -- host-side planning of a chunked prefill call into windows.
//
// A window is a run of consecutive 64-token chunks of the packed call (global
// chunk indices, sequences back to back).  Per window the library launches the
// prep of its chunks and the scan of the sequences that own them, so the
// workspace holds one window of (chunk, head) blocks instead of the whole
// call's.  A sequence cut by a window edge carries its fp32 state to the next
// window through one of two carry buffers (alternating, so that a window
// never reads and writes the same one); the state is stored and reloaded
// unchanged, so the results do not depend on the window size.
#pragma once
#include <stdint.h>

#include <algorithm>
#include <vector>

#include "kda_meta.h"

namespace kda {

// Workspace layout of a prefill call:
//   [sequence table | window order table | checkpoint table | 2 carry states | wc * H blocks]
struct PrefillLayout {
  int64_t seq_off, order_off, ckpt_off, carry_off, inter_off;
};

inline int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

inline PrefillLayout prefill_layout(int32_t num_seqs, int32_t num_ckpts, int H, int D) {
  PrefillLayout m;
  m.seq_off = 0;
  m.order_off = align256((int64_t)num_seqs * (int64_t)sizeof(SeqEntry));
  m.ckpt_off = m.order_off + align256((int64_t)num_seqs * 4);
  m.carry_off = m.ckpt_off + align256((int64_t)num_ckpts * (int64_t)sizeof(CkptEntry));
  m.inter_off = m.carry_off + 2LL * H * D * D * 4;
  return m;
}

// Preferred window: 2048 (chunk, head) blocks (64 chunks = 4096 tokens at 32
// heads, 135 MB of bf16 blocks at d = 128).  A window that small stays in the
// memory-side cache (256 MB) between the prep that writes it and the scan
// that reads it: an 8K-token, 32-head call runs 7% faster as two windows
// than as one.
inline int32_t default_window_chunks(int H) { return std::max(1, 2048 / std::max(H, 1)); }

// Chunks per window for `avail` workspace bytes: the preferred window clipped
// to the call, or the largest that fits; 0 if not even one chunk fits.
inline int32_t fit_window_chunks(const PrefillLayout& m, int H, int64_t blk, int64_t total_chunks,
                                 int64_t avail) {
  const int64_t want = std::min<int64_t>(default_window_chunks(H), std::max<int64_t>(total_chunks, 1));
  const int64_t room = avail - m.inter_off;
  if (room < (int64_t)H * blk) return 0;
  return (int32_t)std::min<int64_t>(want, room / ((int64_t)H * blk));
}

struct Window {
  int32_t c0, nch;                // global chunks [c0, c0 + nch)
  std::vector<int32_t> seqs;      // sequences run in this window, by descending chunk count
};

// Windows of at most `wc` chunks over the packed call.  A sequence appears in
// every window holding one of its chunks; an empty sequence in the window
// holding its chunk_begin (the last window when it is past every chunk).
inline std::vector<Window> plan_windows(const SeqEntry* seqs, int32_t num_seqs, int64_t total_chunks,
                                        int32_t wc) {
  std::vector<Window> wins;
  for (int64_t c0 = 0; c0 < total_chunks || wins.empty(); c0 += wc) {
    Window w;
    w.c0 = (int32_t)c0;
    w.nch = (int32_t)std::min<int64_t>(wc, total_chunks - c0);
    wins.push_back(w);
  }
  std::vector<std::vector<std::pair<int32_t, int32_t>>> lists(wins.size());
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int64_t cb = seqs[s].chunk_begin, nc = (seqs[s].len + 63) / 64;
    if (nc == 0) {
      const size_t w = std::min<size_t>((size_t)(cb / wc), wins.size() - 1);
      lists[w].push_back({0, s});
      continue;
    }
    for (int64_t w = cb / wc; w < (int64_t)wins.size() && (int64_t)wins[w].c0 < cb + nc; ++w) {
      const int64_t lo = std::max<int64_t>(cb, wins[w].c0);
      const int64_t hi = std::min<int64_t>(cb + nc, (int64_t)wins[w].c0 + wins[w].nch);
      lists[w].push_back({(int32_t)(hi - lo), s});
    }
  }
  for (size_t w = 0; w < wins.size(); ++w) {
    // longest first (the scan's cost per sequence is its chunk count); ties by index
    std::stable_sort(lists[w].begin(), lists[w].end(),
                     [](const std::pair<int32_t, int32_t>& a, const std::pair<int32_t, int32_t>& b) {
                       return a.first > b.first;
                     });
    for (const auto& e : lists[w]) wins[w].seqs.push_back(e.second);
  }
  return wins;
}

}  // namespace kda
