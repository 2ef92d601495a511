// kda_device.h -- device-side helpers shared by the libkda kernels (gfx950).
//
// Matrix-core fragments.  Two instructions are used:
//   v_mfma_f32_16x16x32_bf16  (bf16 operands, 8 per lane, fp32 accumulate)
//   v_mfma_f32_16x16x4_f32    (fp32 operands, 1 per lane)
// For both, lane l of a wave64 supplies row (l % 16) of the A tile and column
// (l % 16) of the B tile, with the K index split over the four 16-lane groups
// (l / 16); the 16x16 fp32 result lands as acc[r] = C[4 * (l / 16) + r][l % 16].
// A and B use the same lane -> K mapping, so the product does not depend on how
// K is permuted inside a group.
//
// LDS operand convention used by every tile product here: both operands are
// stored "K-contiguous": A as [M][K] and B as [N][K] (i.e. B transposed), each
// with its own row stride.  bf16 fragments are then one 16-byte LDS read.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kChunk = 64;     // tokens per chunk (C)
constexpr int kThreads = 256;  // 4 waves per workgroup

// ---- bf16 <-> fp32 --------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest even: gfx950 converts in hardware
// (v_cvt_pk_bf16_f32), two values per instruction when paired.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
// two / four values packed in one conversion each pair
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2_t v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}

// ---- storage-type traits --------------------------------------------------
// Op = uint16_t (bf16 bits) or float.  kK = K covered by one MFMA.
template <typename Op> struct OpT;
template <> struct OpT<uint16_t> {
  static constexpr int kK = 32;
  __device__ static __forceinline__ float to_f(uint16_t x) { return bf16_to_f32(x); }
  __device__ static __forceinline__ uint16_t from_f(float x) { return f32_to_bf16(x); }
};
template <> struct OpT<float> {
  static constexpr int kK = 4;
  __device__ static __forceinline__ float to_f(float x) { return x; }
  __device__ static __forceinline__ float from_f(float x) { return x; }
};

__device__ __forceinline__ float load_as_f(const uint16_t* p) { return bf16_to_f32(*p); }
__device__ __forceinline__ float load_as_f(const float* p) { return *p; }

// ---- one MFMA step on a fragment pair ---------------------------------------
// Fragment for Op=bf16: 8 values (K-group of lane); for Op=float: 1 value.
template <typename Op> struct Frag;
template <> struct Frag<uint16_t> { u16x8 v; };
template <> struct Frag<float> { float v; };

__device__ __forceinline__ void mfma(f32x4& acc, const Frag<uint16_t>& a, const Frag<uint16_t>& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a.v),
                                                __builtin_bit_cast(bf16x8, b.v), acc, 0, 0, 0);
}
__device__ __forceinline__ void mfma(f32x4& acc, const Frag<float>& a, const Frag<float>& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v, b.v, acc, 0, 0, 0);
}

// Fragment of a K-contiguous matrix X (row stride ld elements): rows r0..r0+15,
// K columns k0.. k0+kK-1.  Works for LDS and global pointers.
template <typename Op>
__device__ __forceinline__ Frag<Op> frag(const Op* x, int ld, int r0, int k0, int lane);
template <>
__device__ __forceinline__ Frag<uint16_t> frag<uint16_t>(const uint16_t* x, int ld, int r0, int k0,
                                                         int lane) {
  Frag<uint16_t> f;
  f.v = *reinterpret_cast<const u16x8*>(x + (r0 + (lane & 15)) * ld + k0 + 8 * (lane >> 4));
  return f;
}
template <>
__device__ __forceinline__ Frag<float> frag<float>(const float* x, int ld, int r0, int k0, int lane) {
  Frag<float> f;
  f.v = x[(r0 + (lane & 15)) * ld + k0 + (lane >> 4)];
  return f;
}

// fp32 B fragment from an N-contiguous matrix X[K][N] (row stride ld).
__device__ __forceinline__ Frag<float> frag_kn(const float* x, int ld, int n0, int k0, int lane) {
  Frag<float> f;
  f.v = x[(k0 + (lane >> 4)) * ld + n0 + (lane & 15)];
  return f;
}

// acc += A[m0:m0+16, k-range] * B[n0:n0+16, k-range]^T, k-range = [kb, ke)
// (kb, ke multiples of OpT<Op>::kK).  A: [M][K] stride lda; B: [N][K] stride ldb.
template <typename Op>
__device__ __forceinline__ void tile_mma(f32x4& acc, const Op* A, int lda, int m0, const Op* B,
                                         int ldb, int n0, int kb, int ke, int lane) {
  constexpr int KK = OpT<Op>::kK;
#pragma unroll 4
  for (int k = kb; k < ke; k += KK) {
    Frag<Op> a = frag<Op>(A, lda, m0, k, lane);
    Frag<Op> b = frag<Op>(B, ldb, n0, k, lane);
    mfma(acc, a, b);
  }
}

// fp32 only: as tile_mma but B stored [K][N] (N-contiguous), stride ldb.
__device__ __forceinline__ void tile_mma_kn(f32x4& acc, const float* A, int lda, int m0,
                                            const float* B, int ldb, int n0, int kb, int ke,
                                            int lane) {
#pragma unroll 4
  for (int k = kb; k < ke; k += 4) {
    Frag<float> a = frag<float>(A, lda, m0, k, lane);
    Frag<float> b = frag_kn(B, ldb, n0, k, lane);
    mfma(acc, a, b);
  }
}

__device__ __forceinline__ u16x4 pack_bf16x4(float a, float b, float c, float d) {
  bf16x4_t v = {static_cast<__bf16>(a), static_cast<__bf16>(b), static_cast<__bf16>(c),
                static_cast<__bf16>(d)};
  return __builtin_bit_cast(u16x4, v);
}

// Fragment-major storage of an MFMA operand X[rows][K] (the layout the
// prefill prep kernel writes its per-chunk intermediates in): fragment
// (row tile, k step) is 64 lanes x (KK/4) contiguous elements, lane-major, so a
// wave loads one fragment as one contiguous 1 KB (bf16) / 256 B (fp32) block.
template <int KK>
__host__ __device__ __forceinline__ int frag_off(int row, int k, int K) {
  constexpr int E = KK / 4;  // elements per lane
  const int f = (row >> 4) * (K / KK) + k / KK;
  const int ln = (row & 15) + 16 * ((k % KK) / E);
  return (f * 64 + ln) * E + (k % E);
}

template <typename Op>
__device__ __forceinline__ Frag<Op> frag_fm(const Op* x, int row_tile, int k_step, int K, int lane) {
  constexpr int KK = OpT<Op>::kK, E = KK / 4;
  const Op* p = x + ((row_tile * (K / KK) + k_step) * 64 + lane) * E;
  Frag<Op> f;
  if constexpr (E == 8) f.v = *reinterpret_cast<const u16x8*>(p);
  else f.v = *p;
  return f;
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Row/column of element r (0..3) of a 16x16 accumulator held by `lane`.
__device__ __forceinline__ int acc_row(int lane, int r) { return 4 * (lane >> 4) + r; }
__device__ __forceinline__ int acc_col(int lane) { return lane & 15; }

}  // namespace kda
