// kda_conv.hip -- short causal convolution with a checkpointed window state,
// gfx950.
//
// Page "KIMI K3 경량 복제에서 본 KDA의 AI 인프라 과제" (acpost.vercel.app),
// sections 8.2.3 (in prefill, q, k and v each pass through a causal
// convolution before the recurrence), 8.2.4 (the checkpoint kernel writes the
// convolution history and the recurrent checkpoint in the same pass) and 6.5
// (the convolution state is the window of recent inputs, kept at full
// precision; a restore needs it as well as the recurrent state).  Width W and
// the absence of an activation are this implementation's reading (the pages fix
// neither):  y[t][c] = sum_{j < W} w[c][j] * x[t - (W-1) + j][c].
//
// Work unit: a 16-token block of one 64-token chunk of the sequence table, for
// one channel group (8 bf16 or 4 fp32 channels = 16 bytes) per thread.  The
// thread holds the W-1 rows before its block and the block's rows as raw
// 16-byte words, all loads in flight before the first output: rows before the
// block come from x, or from the state page before the sequence start (zeros
// without one).  At a checkpoint position P inside the block, and at the end
// of the sequence, it writes the W-1 most recent inputs (positions P-W+1 ..
// P-1) to the page, token-major in the input dtype, as copies of those words.
// A wave reads and writes whole 1 KB rows of channels; outputs are stored
// non-temporally (written once, read by the next kernel from HBM anyway).
// Consecutive workgroup ids take the channel columns of one time block, so
// the workgroups in flight read whole rows of x (all channels of a few
// tokens) rather than one column's slice of many rows: with x not in the
// memory-side cache this streams 7% faster than giving each XCD a contiguous
// run of one column's time blocks (whose shared W-1 rows then come from its
// L2), which only wins when x is already cached.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

constexpr int kConvBlock = 16;  // tokens per thread

template <typename In> struct ConvVec;
template <> struct ConvVec<uint16_t> {
  static constexpr int N = 8;
  __device__ static u32x4_t raw(const uint16_t* p) { return *reinterpret_cast<const u32x4_t*>(p); }
  __device__ static void unpack(const u32x4_t r, float (&v)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(r[i] << 16);
      v[2 * i + 1] = __uint_as_float(r[i] & 0xffff0000u);
    }
  }
};
template <> struct ConvVec<float> {
  static constexpr int N = 4;
  __device__ static u32x4_t raw(const float* p) { return *reinterpret_cast<const u32x4_t*>(p); }
  __device__ static void unpack(const u32x4_t r, float (&v)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(r[i]);
  }
};

template <typename In, int W>
__global__ __launch_bounds__(256) void conv_kernel(ConvArgs a) {
  using CV = ConvVec<In>;
  constexpr int N = CV::N;
  // linear workgroup id -> (time block, channel column), channel columns of a
  // time block adjacent
  const int tile = blockIdx.x + gridDim.x * blockIdx.y;
  const int by = tile % gridDim.y, bx = tile / gridDim.y;
  const int cg = by * 256 + threadIdx.x;
  const int c0 = cg * N;
  if (c0 >= a.C) return;  // no barriers in this kernel
  const int chunk = bx / (64 / kConvBlock), sub = bx % (64 / kConvBlock);
  const SeqEntry se = a.seqs[find_seq(a.seqs, a.num_seqs, chunk)];
  const int lc = chunk - se.chunk_begin;
  const int nchunks = (se.len + 63) / 64 > 0 ? (se.len + 63) / 64 : 1;
  const int t0 = 64 * lc + kConvBlock * sub;  // first token of the block (sequence-relative)
  const int nt = max(0, min(kConvBlock, se.len - t0));
  const bool last_block = lc == nchunks - 1 && (t0 + kConvBlock >= se.len);
  if (nt == 0 && !(last_block && sub == 0)) return;  // a block past the end, except an empty sequence's slot
  const In* x = reinterpret_cast<const In*>(a.x);
  const int64_t C = a.C;

  // Every load is issued before the first is used (no branch between them, so
  // the waits stay exact): the W-1 rows before the block come from x, from the
  // entering window page, or -- when they are zeros -- from a harmless
  // in-bounds address (this thread's taps); the block rows repeat the last
  // valid row past the end of the sequence (and read the taps for an empty one).
  float wt[W][N];  // taps first: the first output needs them and the oldest rows
#pragma unroll
  for (int i = 0; i < N; ++i)
#pragma unroll
    for (int j = 0; j < W; ++j) wt[j][i] = a.w[(int64_t)(c0 + i) * W + j];

  // rows[0 .. W-2]: the W-1 inputs before the block; rows[W-1+t]: block row t.
  // Output t reads rows[t .. t+W-1]; the window after token t is
  // rows[t+1 .. t+W-1], stored as raw words (an exact copy of the inputs).
  const In* sp = se.state_in >= 0
                     ? reinterpret_cast<const In*>(a.cpool + (int64_t)se.state_in * a.cpage_bytes)
                     : nullptr;
  const In* dummy = reinterpret_cast<const In*>(a.w + (int64_t)c0 * W);
  u32x4_t rows[W - 1 + kConvBlock];
#pragma unroll
  for (int j = 0; j < W - 1; ++j) {
    const int r = t0 - (W - 1) + j;
    const In* p = r >= 0 ? x + (se.row_begin + r) * C + c0
                         : (sp ? sp + (int64_t)(W - 1 + r) * C + c0 : dummy);
    rows[j] = CV::raw(p);
    __builtin_amdgcn_sched_barrier(0);
  }
  const In* xb = nt > 0 ? x + (se.row_begin + t0) * C + c0 : dummy;
  const int tlast = max(nt - 1, 0);
#pragma unroll
  for (int t = 0; t < kConvBlock; ++t) {
    rows[W - 1 + t] = CV::raw(xb + (int64_t)min(t, tlast) * C);
    __builtin_amdgcn_sched_barrier(0);  // keep row order: row t is waited for by count
  }
#pragma unroll
  for (int j = 0; j < W - 1; ++j)  // zeros before the start when there is no entering window
    if (t0 - (W - 1) + j < 0 && !sp) rows[j] = u32x4_t{0u, 0u, 0u, 0u};

  // checkpoint inside this block: the first multiple of hash_block after the block start
  const int64_t a0 = se.start_pos + t0, a1 = se.start_pos + t0 + nt;
  const int64_t cand = (a0 / a.hash_block + 1) * a.hash_block;
  int ck_page = -1;
  int64_t ck_pos = -1;
  if (cand <= a1 && se.ckpt_end > se.ckpt_begin) {
    int lo = se.ckpt_begin, hi = se.ckpt_end - 1;  // binary search for cand
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (a.ckpts[mid].pos < cand) lo = mid + 1; else hi = mid;
    }
    if (a.ckpts[lo].pos == cand) {
      ck_pos = cand;
      ck_page = a.ckpts[lo].page;
    }
  }
  // window rows rows[first .. first+W-2] to a page
  auto write_window = [&](int page, int first) {
    uint8_t* dp = a.cpool + (int64_t)page * a.cpage_bytes + (int64_t)c0 * sizeof(In);
#pragma unroll
    for (int j = 0; j < W - 1; ++j)
      *reinterpret_cast<u32x4_t*>(dp + (int64_t)j * C * sizeof(In)) = rows[first + j];
  };
  if (nt == 0) {  // empty sequence: the output window is the input window
    if (se.state_out >= 0) write_window(se.state_out, 0);
    return;
  }
#pragma unroll
  for (int t = 0; t < kConvBlock; ++t) {
    if (t >= nt) continue;
    float yv[N];
#pragma unroll
    for (int i = 0; i < N; ++i) yv[i] = 0.f;
#pragma unroll
    for (int j = 0; j < W; ++j) {
      float xv[N];
      CV::unpack(rows[t + j], xv);
#pragma unroll
      for (int i = 0; i < N; ++i) yv[i] = fmaf(wt[j][i], xv[i], yv[i]);
    }
    const int64_t yo = (se.row_begin + t0 + t) * C + c0;
    if (a.out_bf16) {
      u32x4_t r;
#pragma unroll
      for (int i = 0; i < N / 2; ++i) r[i] = pack_bf16x2(yv[2 * i], yv[2 * i + 1]);
      if constexpr (N == 8) {
        __builtin_nontemporal_store(r, reinterpret_cast<u32x4_t*>(reinterpret_cast<uint16_t*>(a.y) + yo));
      } else {
        __builtin_nontemporal_store(u32x2_t{r[0], r[1]},
                                    reinterpret_cast<u32x2_t*>(reinterpret_cast<uint16_t*>(a.y) + yo));
      }
    } else {
#pragma unroll
      for (int i = 0; i < N; i += 4)
        __builtin_nontemporal_store(f32x4{yv[i], yv[i + 1], yv[i + 2], yv[i + 3]},
                                    reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.y) + yo + i));
    }
    if (se.start_pos + t0 + t + 1 == ck_pos) write_window(ck_page, t + 1);
    if (t0 + t + 1 == se.len && se.state_out >= 0) write_window(se.state_out, t + 1);
  }
}

// Decode-step update: one token per request.  Workgroup (R consecutive
// requests, column of 256 channel groups): the thread loads the taps of its
// 16-byte channel group once, then for each of its requests reads the window
// (W-1 rows) from page_in[r] and the token row of x, writes y and the shifted
// window (the last W-2 window rows and the token) to page_out[r].  All loads
// of the R requests are issued before any store, so page_out[r] may equal
// page_in[r].  A page index outside the pool touches no page and gives NaN
// outputs.  Same taps and summation order as conv_kernel: bit-identical
// outputs and windows for the same inputs.
constexpr int kConvUpdateReqs = 4;  // requests per workgroup

template <typename In, int W>
__global__ __launch_bounds__(256) void conv_update_kernel(ConvUpdateArgs a) {
  using CV = ConvVec<In>;
  constexpr int N = CV::N, R = kConvUpdateReqs;
  const int r0 = blockIdx.x * R;
  const int c0 = (blockIdx.y * 256 + threadIdx.x) * N;
  if (c0 >= a.C) return;
  const int64_t C = a.C;
  float wt[W][N];
#pragma unroll
  for (int i = 0; i < N; ++i)
#pragma unroll
    for (int j = 0; j < W; ++j) wt[j][i] = a.w[(int64_t)(c0 + i) * W + j];
  bool ok[R];
  int pout[R];
  u32x4_t rows[R][W];
#pragma unroll
  for (int q = 0; q < R; ++q) {
    const int r = r0 + q;
    ok[q] = false;
    pout[q] = 0;
    if (r >= a.n) continue;
    const int pin = a.page_in[r], po = a.page_out[r];  // uniform: scalar loads
    ok[q] = pin >= 0 && pin < a.num_pages && po >= 0 && po < a.num_pages;
    pout[q] = po;
    if (!ok[q]) continue;
    const In* sp = reinterpret_cast<const In*>(a.cpool + (int64_t)pin * a.cpage_bytes);
#pragma unroll
    for (int j = 0; j < W - 1; ++j) rows[q][j] = CV::raw(sp + (int64_t)j * C + c0);
    rows[q][W - 1] = CV::raw(reinterpret_cast<const In*>(a.x) + (int64_t)r * C + c0);
  }
#pragma unroll
  for (int q = 0; q < R; ++q) {
    const int r = r0 + q;
    if (r >= a.n) continue;
    const int64_t yo = (int64_t)r * C + c0;
    float yv[N];
    if (ok[q]) {
#pragma unroll
      for (int i = 0; i < N; ++i) yv[i] = 0.f;
#pragma unroll
      for (int j = 0; j < W; ++j) {
        float xv[N];
        CV::unpack(rows[q][j], xv);
#pragma unroll
        for (int i = 0; i < N; ++i) yv[i] = fmaf(wt[j][i], xv[i], yv[i]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < N; ++i) yv[i] = __builtin_nanf("");
    }
    if (a.out_bf16) {
      u32x4_t qv;
#pragma unroll
      for (int i = 0; i < N / 2; ++i) qv[i] = pack_bf16x2(yv[2 * i], yv[2 * i + 1]);
      if constexpr (N == 8) {
        __builtin_nontemporal_store(qv, reinterpret_cast<u32x4_t*>(reinterpret_cast<uint16_t*>(a.y) + yo));
      } else {
        __builtin_nontemporal_store(u32x2_t{qv[0], qv[1]},
                                    reinterpret_cast<u32x2_t*>(reinterpret_cast<uint16_t*>(a.y) + yo));
      }
    } else {
#pragma unroll
      for (int i = 0; i < N; i += 4)
        __builtin_nontemporal_store(f32x4{yv[i], yv[i + 1], yv[i + 2], yv[i + 3]},
                                    reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.y) + yo + i));
    }
    if (!ok[q]) continue;
    uint8_t* dp = a.cpool + (int64_t)pout[q] * a.cpage_bytes + (int64_t)c0 * sizeof(In);
#pragma unroll
    for (int j = 0; j < W - 1; ++j)
      *reinterpret_cast<u32x4_t*>(dp + (int64_t)j * C * sizeof(In)) = rows[q][j + 1];
  }
}

template <typename In>
static hipError_t launch_conv_update_t(const ConvUpdateArgs& a, hipStream_t st) {
  constexpr int N = ConvVec<In>::N;
  const dim3 grid((unsigned)((a.n + kConvUpdateReqs - 1) / kConvUpdateReqs), (unsigned)((a.C / N + 255) / 256));
  if (a.W == 2) hipLaunchKernelGGL((conv_update_kernel<In, 2>), grid, dim3(256), 0, st, a);
  else if (a.W == 3) hipLaunchKernelGGL((conv_update_kernel<In, 3>), grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL((conv_update_kernel<In, 4>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_conv_update(const ConvUpdateArgs& a, hipStream_t st) {
  return a.in_bf16 ? launch_conv_update_t<uint16_t>(a, st) : launch_conv_update_t<float>(a, st);
}

template <typename In>
static hipError_t launch_conv_t(const ConvArgs& a, int32_t total_chunks, hipStream_t st) {
  constexpr int N = ConvVec<In>::N;
  const dim3 grid((unsigned)total_chunks * (64 / kConvBlock), (unsigned)((a.C / N + 255) / 256));
  if (a.W == 2) hipLaunchKernelGGL((conv_kernel<In, 2>), grid, dim3(256), 0, st, a);
  else if (a.W == 3) hipLaunchKernelGGL((conv_kernel<In, 3>), grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL((conv_kernel<In, 4>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_conv(const ConvArgs& a, int32_t total_chunks, hipStream_t st) {
  return a.in_bf16 ? launch_conv_t<uint16_t>(a, total_chunks, st) : launch_conv_t<float>(a, total_chunks, st);
}

}  // namespace kda
