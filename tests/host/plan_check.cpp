// Randomised check of the prefill window planner (kda_plan.h), host only:
// for packed calls of random sequence lengths (empty ones included) and random
// window sizes, every chunk of every sequence is run by exactly one window,
// each window's sequences own a chunk in it (or are empty and listed once in
// the window holding their chunk_begin), the order lists descend in the
// sequence's chunk count inside the window, and windows tile [0, total) in
// order.  The workspace sizing is checked too: the chosen window fits the
// bytes given, and the minimum size admits one chunk per window.
#include <cstdio>
#include <random>
#include <vector>

#include "../../hybrid_prefix_cache_amd/csrc/kda_plan.h"

using namespace kda;

static int fail(const char* what, int trial) {
  std::printf("FAIL %s (trial %d)\n", what, trial);
  return 1;
}

int main() {
  std::mt19937 rng(12345);
  for (int trial = 0; trial < 20000; ++trial) {
    const int ns = 1 + (int)(rng() % 24);
    std::vector<SeqEntry> s(ns);
    int cb = 0;
    for (int i = 0; i < ns; ++i) {
      s[i] = SeqEntry{};
      s[i].len = rng() % 4 == 0 ? 0 : (int)(rng() % 5000);
      s[i].chunk_begin = cb;
      cb += (s[i].len + 63) / 64;
    }
    const int wc = 1 + (int)(rng() % 70);
    const std::vector<Window> w = plan_windows(s.data(), ns, cb, wc);
    std::vector<int> cov(cb, 0), empty_seen(ns, 0);
    int next_c0 = 0;
    for (const Window& win : w) {
      if (win.c0 != next_c0 || win.nch < 0 || win.nch > wc) return fail("tiling", trial);
      next_c0 += win.nch;
      int prev = 1 << 30;
      for (int si : win.seqs) {
        if (si < 0 || si >= ns) return fail("index", trial);
        const int nc = (s[si].len + 63) / 64;
        const int lo = std::max(win.c0 - s[si].chunk_begin, 0);
        const int hi = std::min(win.c0 + win.nch - s[si].chunk_begin, nc);
        if (nc == 0) {
          ++empty_seen[si];
          if (hi - lo != 0) return fail("empty range", trial);
        } else if (lo >= hi) {
          return fail("listed without a chunk", trial);
        }
        const int here = std::max(hi - lo, 0);
        if (here > prev) return fail("order", trial);
        prev = here;
        for (int n = lo; n < hi; ++n) ++cov[s[si].chunk_begin + n];
      }
    }
    if (next_c0 != cb) return fail("tiling end", trial);
    for (int c = 0; c < cb; ++c)
      if (cov[c] != 1) return fail("coverage", trial);
    for (int i = 0; i < ns; ++i)
      if (s[i].len == 0 && empty_seen[i] != 1) return fail("empty sequence", trial);
    // sizing
    const int H = 1 + (int)(rng() % 64), D = rng() % 2 ? 64 : 128;
    const int64_t blk = inter_block_bytes(D, rng() % 2 ? 2 : 4);
    const PrefillLayout m = prefill_layout(ns, (int)(rng() % 50), H, D);
    const int64_t least = m.inter_off + (int64_t)H * blk;
    if (fit_window_chunks(m, H, blk, cb, least - 1) != 0) return fail("below minimum", trial);
    if (fit_window_chunks(m, H, blk, cb, least) != 1) return fail("minimum", trial);
    const int64_t avail = least + (int64_t)(rng() % 100) * H * blk / 7;
    const int32_t got = fit_window_chunks(m, H, blk, cb, avail);
    if (m.inter_off + (int64_t)got * H * blk > avail) return fail("fits", trial);
    if (got > default_window_chunks(H) || got > std::max(cb, 1)) return fail("cap", trial);
  }
  std::printf("ok\n");
  return 0;
}
