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
typedef float f32x4 __attribute__((ext_vector_type(4)));

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

// ---------------------------------------------------------------- LDS staging
// Byte address of a __shared__ object within LDS.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Direct HBM -> LDS copy: lane i's 16 bytes at g land at LDS byte lds + 16 i.
// Written as inline asm so that the compiler does not order every later LDS
// read behind it; callers wait for completion with wait_vmcnt and a barrier.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(lds)
               : "memory", "m0");
}

// Same copy with a wave-uniform base address in SGPRs and a per-lane 32-bit
// byte offset: no per-lane address arithmetic.
__device__ __forceinline__ void dma16s(uint32_t voff, const void* sbase, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Wait until at most N of this wave's vector-memory operations are in flight.
template <int N> __device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (((N >> 4) & 3) << 14) | (7 << 4) | (15 << 8));
}

// Race check build (FA_SERIALIZE_STAGES): every LDS ring stage is fenced on
// both sides, each copy completed and the whole work-group synchronised right
// after it is issued and again after each step's reads, so no tile is read
// before it lands or overwritten while read.  Same arithmetic in the same
// order; the results must equal the normal build's bit for bit.
#ifdef FA_SERIALIZE_STAGES
#define FA_STAGE_FENCE() \
  do {                   \
    wait_vmcnt<0>();     \
    __syncthreads();     \
  } while (0)
#else
#define FA_STAGE_FENCE() \
  do {                   \
  } while (0)
#endif

// 4-byte variant (lane i's word lands at LDS byte lds + 4 i).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma4s(uint32_t voff, const void* sbase, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Row-major tiles in LDS are stored as 16-byte chunks, with the chunk index of
// row r XORed by a swizzle of r so that reads hit distinct banks (there is no
// room for row padding: a DMA wave writes 1 KB contiguously).  Model: one LDS
// cycle serves 256 B = 16 chunk-wide bank groups, group = (r*CPR + chunk) % 16.
//   kRows  row reads (ds_read_b128, 16 lanes on 16 consecutive rows, one chunk
//          each): conflict-free;
//   kTr    transposed reads (ds_read_b64_tr_b16, 8 rows x 4 chunks per wave):
//          each group hit twice, the minimum;
//   kBoth  both of the above at once (tiles read both ways).
enum SwzKind { kRows = 0, kTr = 1, kBoth = 2 };
template <int CPR, int KIND> __device__ __forceinline__ int swz(int r) {
  if constexpr (KIND == kRows) return CPR >= 16 ? (r & 15) : ((r >> 1) & 7);
  if constexpr (KIND == kTr) return CPR >= 16 ? ((r & 3) << 2) : (((r >> 1) & 1) << 2);
  if constexpr (CPR == 8) return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  if constexpr (CPR == 16) return ((r & 3) << 2) | ((r >> 2) & 3);
  return r & 15;  // 32 chunks per row (fp32, d = 128): row reads only
}

// Copies rows row0 .. row0+ROWS-1 (D elements each, row-major in HBM; rows
// past N-1 repeat row N-1) into an LDS tile at byte address `lds` with the
// given chunk swizzle.  The tile is split over the work-group's NW waves; each
// wave issues ROWS*D*sizeof(raw)/(1024*NW) DMA instructions.
template <typename raw, int ROWS, int D, int KIND, int NW = 4>
__device__ __forceinline__ void dma_tile(const raw* __restrict__ g, int row0, int N, uint32_t lds,
                                         int wave, int lane) {
  constexpr int CPR = D * (int)sizeof(raw) / 16;  // chunks per row
  constexpr int VEC = 16 / (int)sizeof(raw);
  constexpr int NI = ROWS * CPR / (64 * NW);      // instructions per wave
  static_assert(ROWS * CPR % (64 * NW) == 0, "tile must split into 1 KB per-wave pieces");
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int blk = i * NW + wave;       // 1 KB block of the tile
    const int pos = blk * 64 + lane;     // chunk position within the tile
    const int r = pos / CPR, cs = pos % CPR;
    const int c = cs ^ swz<CPR, KIND>(r);
    const int row = min(row0 + r, N - 1);
    dma16(g + (size_t)row * D + c * VEC, __builtin_amdgcn_readfirstlane(lds + blk * 1024));
  }
}

// The same tile copy for tiles whose ROWS rows all exist: this lane's byte
// offsets within the tile are computed once, each copy only supplies the
// tile's (wave-uniform) first-row address.
template <typename raw, int ROWS, int D, int KIND, int NW = 4>
struct DmaPlan {
  static constexpr int CPR = D * (int)sizeof(raw) / 16;
  static constexpr int VEC = 16 / (int)sizeof(raw);
  static constexpr int NI = ROWS * CPR / (64 * NW);
  static_assert(ROWS * CPR % (64 * NW) == 0, "tile must split into 1 KB per-wave pieces");
  uint32_t off[NI];
  int wave;
  __device__ __forceinline__ void init(int wave_, int lane) {
    wave = wave_;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int pos = (i * NW + wave) * 64 + lane;
      const int r = pos / CPR, cs = pos % CPR;
      const int c = cs ^ swz<CPR, KIND>(r);
      off[i] = (uint32_t)((r * D + c * VEC) * (int)sizeof(raw));
    }
  }
  __device__ __forceinline__ void issue(const raw* first_row, uint32_t lds) const {
    // The base address and the LDS address are wave-uniform; stating it keeps
    // them in scalar registers wherever the compiler cannot prove it.
    const uint64_t a = (uint64_t)first_row;
    const raw* base = (const raw*)(((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)) << 32) |
                                   (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a));
#pragma unroll
    for (int i = 0; i < NI; ++i)
      dma16s(off[i], base, __builtin_amdgcn_readfirstlane(lds + (i * NW + wave) * 1024));
  }
  // rows row0 .. row0+ROWS-1 of g, or the clamped copy if the tile is ragged
  __device__ __forceinline__ void copy(const raw* g, int row0, int N, uint32_t lds,
                                       int lane) const {
    if (row0 + ROWS <= N) issue(g + (size_t)row0 * D, lds);
    else dma_tile<raw, ROWS, D, KIND, NW>(g, row0, N, lds, wave, lane);
  }
};

// Eight contiguous elements of row `row` starting at element `col` (a multiple
// of 8) from a swizzled row-major tile: the contiguous-slot operand.
template <typename T, int D, int KIND>
__device__ __forceinline__ frag_t<T> load_frag_swz(const raw_t<T>* tile, int row, int col) {
  constexpr int CPR = D * (int)sizeof(raw_t<T>) / 16;
  constexpr int VEC = 16 / (int)sizeof(raw_t<T>);
  const raw_t<T>* rp = tile + row * D;
  const int sw = swz<CPR, KIND>(row);
  if constexpr (VEC == 8) {
    return load_frag<T>(rp + (((col / VEC) ^ sw) * VEC));
  } else {
    typedef raw_t<T> raw4v __attribute__((ext_vector_type(4)));
    const raw4v lo = *reinterpret_cast<const raw4v*>(rp + (((col / VEC) ^ sw) * VEC));
    const raw4v hi = *reinterpret_cast<const raw4v*>(rp + ((((col / VEC) + 1) ^ sw) * VEC));
    raw8_t<T> r8;
#pragma unroll
    for (int i = 0; i < 4; ++i) { r8[i] = lo[i]; r8[4 + i] = hi[i]; }
    return __builtin_bit_cast(frag_t<T>, r8);
  }
}

// Acc-ordered A operand of a product whose contraction runs over the ROWS of a
// row-major tile (e.g. V^T P^T: rows = keys): lane (c, h) receives elements
// (k0 + pi(h, s), col0 + c), pi the acc-ordered slot map.  16-bit types use
// two transposed LDS reads (ds_read_b64_tr_b16: within each 16-lane group,
// lane j takes element j % 4 of the 8-byte rows addressed by lanes
// j / 4 + 4t, t = 0..3).  fp32 reads the eight elements one by one.
template <typename T, int D, int KIND>
__device__ __forceinline__ frag_t<T> load_frag_tr(const raw_t<T>* tile, int k0, int col0,
                                                  int lane) {
  typedef raw_t<T> raw;
  constexpr int CPR = D * (int)sizeof(raw) / 16;
  if constexpr (sizeof(raw) == 2) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const int g = lane >> 4, s = lane & 15;
    const int r0 = k0 + 4 * (g >> 1) + (s >> 2);
    const int col = col0 + 16 * (g & 1) + 4 * (s & 3);  // 4 elements = half a chunk
    auto addr = [&](int r) {
      const int chunk = (col >> 3) ^ swz<CPR, KIND>(r);
      return (lds_s16x4*)(const __attribute__((address_space(3))) raw*)(tile + r * D + chunk * 8 +
                                                                          (col & 7));
    };
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(addr(r0));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(addr(r0 + 8));
    raw8_t<T> r8;
#pragma unroll
    for (int i = 0; i < 4; ++i) { r8[i] = (raw)lo[i]; r8[4 + i] = (raw)hi[i]; }
    return __builtin_bit_cast(frag_t<T>, r8);
  } else {
    const int c = lane & 31, h = lane >> 5;
    const int col = col0 + c;
    raw8_t<T> r8;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int r = k0 + (u < 4 ? 4 * h + u : 8 + 4 * h + (u - 4));
      r8[u] = tile[r * D + (((col / 4) ^ swz<CPR, KIND>(r)) * 4) + (col & 3)];
    }
    return __builtin_bit_cast(frag_t<T>, r8);
  }
}

// Compute units per XCD of MI355X (256 in 8 XCDs).
constexpr int kCusPerXcd = 32;

// Work-group id -> (tile, head) for a grid of ntiles * BH work-groups.
// Work-groups are dispatched round-robin over the 8 XCDs (id % 8); when BH is a
// multiple of 8 every tile of one head is kept on one XCD so that its K/V (or
// Q/dO) re-reads hit that XCD's L2.  Each XCD takes its BH / 8 heads in
// groups of `group` heads (all of them when group >= BH / 8), and within a
// group hands out the heads' tiles by tile index: with reverse set from the
// last (heaviest under a causal mask) to the first.  Groups bound how many
// heads' streamed operands share the XCD's L2 at a time.  With snake set,
// every other complete round of kCusPerXcd slots is taken in reverse, so that
// when an XCD's work-groups land on its CUs round by round the heaviest of one
// round shares a CU with the lightest of the next (causal dQ pass: 3.5-5%
// faster at N = 2K-4K, within 1% elsewhere; the forward measured up to 19%
// slower on grids of several rounds, whose heaviest-first order it breaks, and
// the dK/dV pass slower too, so the dQ pass uses it, and the forward only
// when its whole grid is resident at once).  Whole rounds only: the slot stays
// a bijection on [0, ntiles * BH / 8).
__device__ __forceinline__ void map_tile(int bid, int ntiles, int BH, bool reverse, int group,
                                         int& tile, int& bh, bool snake = false) {
  int ti;
  if ((BH & 7) == 0) {
    const int xcd = bid & 7, hpx = BH >> 3;
    int slot = bid >> 3;
    if (snake) {
      constexpr int C = kCusPerXcd;
      const int r = slot / C, c = slot - r * C;
      if ((r & 1) && (r + 1) * C <= ntiles * hpx) slot = r * C + (C - 1 - c);
    }
    const int G = group > 0 && group < hpx ? group : hpx;
    const int g = slot / (G * ntiles);          // groups before this one are full
    const int r = slot - g * G * ntiles;
    const int Gg = min(G, hpx - g * G);         // heads in this group
    ti = r / Gg;
    bh = (g * G + (r - ti * Gg)) * 8 + xcd;
  } else {
    ti = bid / BH;
    bh = bid - ti * BH;
  }
  tile = reverse ? ntiles - 1 - ti : ti;
}

}  // namespace fa
