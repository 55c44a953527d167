// Device building blocks shared by the forward and backward attention kernels
// (gfx950 / CDNA4, wave64).
//
// Matrix-core layouts used throughout (v_mfma_f32_32x32x16_{bf16,f16} and,
// for fp32, eight v_mfma_f32_32x32x2_f32 per 16-deep step).  For lane l of a
// wave let c = l % 32 and h = l / 32:
//   A operand  (32 x 16): lane holds row c, eight k-slots (h, s), s = 0..7;
//   B operand  (16 x 32): lane holds column c, the same eight k-slots (h, s);
//   accumulator (32 x 32, 16 fp32): register r of lane l holds
//              row 8*(r/4) + 4*h + (r%4), column c.
// The hardware pairs A's and B's k-slots; which k index a slot carries is our
// choice as long as both operands agree.  Two slot maps are used:
//   contiguous:  slot (h, s) <-> k = 8*h + s       (rows of Q, K, dO: d-major)
//   acc-ordered: slot (h, s) <-> k = 4*h + s        for s < 4,
//                               k = 8 + 4*h + s-4  for s >= 4
// The acc-ordered map is exactly how registers 8*t .. 8*t+7 of an accumulator
// tile cover rows 16*t .. 16*t+15, so a probability (or dS) tile computed with
// keys as accumulator rows feeds the next product as a B operand straight from
// registers, with no trip through LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

template <typename T> struct Traits;

template <> struct Traits<__bf16> {
  typedef uint16_t raw;
  typedef __bf16 frag __attribute__((ext_vector_type(8)));
  static __device__ __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

template <> struct Traits<_Float16> {
  typedef uint16_t raw;
  typedef _Float16 frag __attribute__((ext_vector_type(8)));
  static __device__ __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

template <> struct Traits<float> {
  typedef uint32_t raw;
  typedef float frag __attribute__((ext_vector_type(8)));
  static __device__ __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
#pragma unroll
    for (int s = 0; s < 8; ++s) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[s], b[s], c, 0, 0, 0);
    return c;
  }
};

template <typename T> using frag_t = typename Traits<T>::frag;
template <typename T> using raw_t = typename Traits<T>::raw;
template <typename T> using raw4_t = raw_t<T> __attribute__((ext_vector_type(4)));
template <typename T> using raw8_t = raw_t<T> __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

template <typename T> __device__ __forceinline__ frag_t<T> zero_frag() {
  frag_t<T> z;
#pragma unroll
  for (int i = 0; i < 8; ++i) z[i] = (T)0.f;
  return z;
}

// Eight contiguous elements (contiguous slot map) from LDS or global memory.
template <typename T> __device__ __forceinline__ frag_t<T> load_frag(const raw_t<T>* p) {
  return *reinterpret_cast<const frag_t<T>*>(p);
}

// Acc-ordered operand from a k-contiguous row: elements p[4h .. 4h+3] and
// p[8+4h .. 8+4h+3], where p points at the start of a 16-wide k step.
template <typename T> __device__ __forceinline__ frag_t<T> load_frag_acc_order(
    const raw_t<T>* p, int h) {
  raw4_t<T> lo = *reinterpret_cast<const raw4_t<T>*>(p + 4 * h);
  raw4_t<T> hi = *reinterpret_cast<const raw4_t<T>*>(p + 8 + 4 * h);
  raw8_t<T> r;
#pragma unroll
  for (int i = 0; i < 4; ++i) { r[i] = lo[i]; r[4 + i] = hi[i]; }
  return __builtin_bit_cast(frag_t<T>, r);
}

// Registers 8*t .. 8*t+7 of an fp32 accumulator tile, rounded to T, as a B
// operand with the acc-ordered slot map.
template <typename T> __device__ __forceinline__ frag_t<T> acc_to_frag(const f32x16& a, int t) {
  frag_t<T> f;
#pragma unroll
  for (int s = 0; s < 8; ++s) f[s] = (T)a[8 * t + s];
  return f;
}

// Row of accumulator register r for half h.
__device__ __forceinline__ int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// Combine a value with the one held by lane l ^ 32 (the other half of the wave).
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Work-group id -> (tile, head) for a grid of ntiles * BH work-groups.
// Work-groups are dispatched round-robin over the 8 XCDs (id % 8); when BH is a
// multiple of 8 every tile of one head is kept on one XCD so that its K/V (or
// Q/dO) re-reads hit that XCD's L2.  With reverse set, tiles are handed out
// from the last (heaviest under a causal mask) to the first.
__device__ __forceinline__ void map_tile(int bid, int ntiles, int BH, bool reverse,
                                         int& tile, int& bh) {
  int ti;
  if ((BH & 7) == 0) {
    const int xcd = bid & 7, slot = bid >> 3, hpx = BH >> 3;
    ti = slot / hpx;
    bh = (slot - ti * hpx) * 8 + xcd;
  } else {
    ti = bid / BH;
    bh = bid - ti * BH;
  }
  tile = reverse ? ntiles - 1 - ti : ti;
}

}  // namespace fa
