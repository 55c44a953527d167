// Unit issue rates on gfx950 (a measurement library, libfa_rates.so; the
// attention library does not contain it).
//
// The attention steps are built from a handful of instruction kinds: the
// bf16 matrix product v_mfma_f32_32x32x16_bf16, and on the vector side the
// score scaling (v_fma_f32), the base-2 exponential (v_exp_f32), fp32 adds
// (row sums) and the packing of probabilities to bf16 (v_cvt_pk_bf16_f32).
// Their cost per step is the step's count of each kind times the SIMD cycles
// one wave instruction of that kind takes.  These kernels measure the second
// factor: every wave runs a straight loop of one kind, with enough
// independent chains per wave (and waves per SIMD) to cover the latency, and
// lane 0 records the shader clock (s_memtime) and the 100 MHz wall clock
// (s_memrealtime) before and after its loop.  SIMD cycles per instruction =
// loop cycles / (instructions per wave x waves per SIMD), with every wave of
// the grid resident at once (the caller sizes the grid to the chip).
//
// Two mixed kernels test overlap: kMixSelf interleaves one matrix product
// with four exponentials inside each wave; kMixWaves runs work-groups of 8
// waves, waves 0-3 the matrix loop and waves 4-7 the exponential loop, so
// that each SIMD holds one of each.  If vector work runs beside the matrix
// cores, the mixed loops take about as long as their matrix part alone.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_common.h"  // (the attention kernels' LDS operand reads, for op 8)

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

enum Op {
  kMfma = 0, kExp = 1, kFma = 2, kAdd = 3, kCvt = 4, kMixSelf = 5, kMixWaves = 6,
  kLds128 = 7, kLdsTr = 8
};

constexpr int kChains = 16;  // independent vector chains per lane
constexpr int kAccs = 4;     // independent matrix accumulators per wave

// Per wave: shader clock start and end, wall clock start and end, and where
// the wave ran: the XCD (XCC_ID) in bits 32 and up, the HW_ID register below
// (SIMD, CU, shader array and engine fields), so that the waves of one SIMD
// can be grouped.
constexpr int kRecordWords = 5;
__device__ __forceinline__ void record(unsigned long long* rec, unsigned long long t0,
                                       unsigned long long r0, unsigned long long t1,
                                       unsigned long long r1) {
  // s_getreg operands: (size - 1) << 11 | offset << 6 | register id
  const unsigned hw_id = __builtin_amdgcn_s_getreg((31 << 11) | 4);    // HW_REG_HW_ID
  const unsigned xcc_id = __builtin_amdgcn_s_getreg((31 << 11) | 20);  // HW_REG_XCC_ID
  rec[0] = t0;
  rec[1] = t1;
  rec[2] = r0;
  rec[3] = r1;
  rec[4] = ((unsigned long long)xcc_id << 32) | hw_id;
}

// One loop iteration of each kind: kAccs matrix products, or kChains vector
// instructions.
__device__ __forceinline__ void mfma_iter(f32x16 (&acc)[kAccs], bf16x8 a, bf16x8 b) {
#pragma unroll
  for (int j = 0; j < kAccs; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
}

__device__ __forceinline__ void exp_iter(float (&x)[kChains]) {
  // (the chains overflow to +inf within a few steps and stay there; the
  // plain operand form is the one the attention kernels issue)
#pragma unroll
  for (int j = 0; j < kChains; ++j) x[j] = __builtin_amdgcn_exp2f(x[j]);
}

// LDS reads: each wave reads its work-group's LDS buffer, 16 reads per
// iteration: ds_read_b128 (16 contiguous bytes per lane, 1 KB per read) or
// ds_read_b64_tr_b16 (the transposing read the attention kernels use for the
// V^T, dO^T and Q^T operands, 512 bytes per read) addressed exactly as the
// kernels address a swizzled tile, and folds every element read into a
// running xor so that no read is dead.
constexpr int kLdsBytes = 32768;  // two 16 KB tiles (op 8); op 7 reads 17 KB of it
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) u32x4 lds_u4;

// Waves per work-group: 4, or 8 for kMixWaves.
template <int OP> constexpr int waves_per_group() { return OP == kMixWaves ? 8 : 4; }

template <int OP>
__global__ __launch_bounds__(64 * waves_per_group<OP>()) void rates_kernel(
    int iters, float seed, float* sink, unsigned long long* clocks) {
  constexpr int WPG = waves_per_group<OP>();
  const int lane = threadIdx.x & 63;
  const int wave = (int)(blockIdx.x * WPG + (threadIdx.x >> 6));
  const float base = seed * (float)(threadIdx.x + 1);
  float x[kChains];
#pragma unroll
  for (int j = 0; j < kChains; ++j) x[j] = base + 0.001f * j;
  f32x16 acc[kAccs];
#pragma unroll
  for (int j = 0; j < kAccs; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
  bf16x8 a, b;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    a[s] = (__bf16)(base + s);
    b[s] = (__bf16)(base - s);
  }
  const float m = 1.0f - 0.5f * seed;  // (wave-uniform: a scalar operand)
  const float add = 0.25f * base;      // (a vector operand)
  const bool mfma_wave = (threadIdx.x >> 6) < 4;  // (kMixWaves)
  __shared__ __attribute__((aligned(1024))) char lds[OP == kLds128 || OP == kLdsTr ? kLdsBytes : 4];
  unsigned fold = 0;
  __attribute__((address_space(3))) char* const lb = (__attribute__((address_space(3))) char*)lds;
  if constexpr (OP == kLds128 || OP == kLdsTr) {
    for (int i = threadIdx.x; i < kLdsBytes / 4; i += 64 * WPG)
      reinterpret_cast<unsigned*>(lds)[i] = (unsigned)i * 2654435761u;
    __syncthreads();
  }

  __builtin_amdgcn_sched_barrier(0);
  const unsigned long long t0 = __builtin_readcyclecounter();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (OP == kMixWaves) {
    // wave-uniform choice of loop
    if (mfma_wave) {
      for (int it = 0; it < iters; ++it) mfma_iter(acc, a, b);
    } else {
      for (int it = 0; it < iters; ++it) exp_iter(x);
    }
  } else {
  for (int it = 0; it < iters; ++it) {
    if constexpr (OP == kMfma) {
      mfma_iter(acc, a, b);
    } else if constexpr (OP == kExp) {
      exp_iter(x);
    } else if constexpr (OP == kFma) {
#pragma unroll
      for (int j = 0; j < kChains; ++j) x[j] = fmaf(x[j], m, add);
    } else if constexpr (OP == kAdd) {
#pragma unroll
      for (int j = 0; j < kChains; ++j) x[j] = x[j] + add;
    } else if constexpr (OP == kCvt) {
      // pack a float twice to bf16 and reuse the packed bits as the next input
#pragma unroll
      for (int j = 0; j < kChains; ++j) {
        const bf16x2 p = {(__bf16)x[j], (__bf16)x[j]};
        x[j] = __builtin_bit_cast(float, p);
      }
    } else if constexpr (OP == kLds128) {
      // lane l reads bytes 16 l .. 16 l + 15 of each 1 KB row j, from a base
      // that alternates between 0 and 512 so that no read is loop-invariant
      const __attribute__((address_space(3))) char* const b = lb + (it & 1) * 512 + lane * 16;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const u32x4 v = *(const lds_u4*)(b + j * 1024);
        fold ^= v[0] ^ v[1] ^ v[2] ^ v[3];
      }
    } else if constexpr (OP == kLdsTr) {
      // the V^T operand reads of the forward: eight 32 x 16 fragments of a
      // 64-key x 128-d bf16 tile stored with the transposed-read swizzle,
      // each two ds_read_b64_tr_b16 (512 bytes each), from one of two tiles
      const uint16_t* tile = reinterpret_cast<const uint16_t*>(lds) + (it & 1) * 64 * 128;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const fa::frag_t<__bf16> v =
            fa::load_frag_tr<__bf16, 128, fa::kTr>(tile, 16 * (j & 3), 32 * (j >> 2), lane);
        const uint32_t* w = reinterpret_cast<const uint32_t*>(&v);
        fold ^= w[0] ^ w[1] ^ w[2] ^ w[3];
      }
    } else if constexpr (OP == kMixSelf) {
      // per iteration kAccs products and kChains exponentials, issued as
      // one product then four exponentials (the order held by scheduling
      // barriers)
      constexpr int E = kChains / kAccs;
#pragma unroll
      for (int j = 0; j < kAccs; ++j) {
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < E; ++u) x[E * j + u] = __builtin_amdgcn_exp2f(x[E * j + u]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  }
  __builtin_amdgcn_sched_barrier(0);
  // the last results must have landed before the closing clock read
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kAccs; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
#pragma unroll
  for (int j = 0; j < kChains; ++j) s += x[j];
  s += (float)(fold & 1);
  __builtin_amdgcn_sched_barrier(0);
  const unsigned long long t1 = __builtin_readcyclecounter();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  sink[(size_t)blockIdx.x * 64 * WPG + threadIdx.x] = s;
  if (lane == 0) record(clocks + kRecordWords * (size_t)wave, t0, r0, t1, r1);
}

template <int OP>
hipError_t launch(int grid, int iters, float* sink, unsigned long long* clocks,
                  hipStream_t stream) {
  hipLaunchKernelGGL(rates_kernel<OP>, dim3(grid), dim3(64 * waves_per_group<OP>()), 0, stream,
                     iters, 0.001f, sink, clocks);
  return hipGetLastError();
}

}  // namespace

// Runs one rates kernel (op: 0 matrix products, 1 exponentials, 2 fma, 3 add,
// 4 bf16 packing, 5 products and exponentials in one wave, 6 in separate
// waves, 7 ds_read_b128, 8 ds_read_b64_tr_b16): `grid` work-groups of W waves (W = 4, or 8 for op 6; the dispatcher
// spreads a work-group's waves over the CU's four SIMDs), each wave `iters`
// loop iterations of 4 matrix products, 16 vector instructions (op 5: both)
// or 16 KB of LDS reads per wave (ops 7, 8).
// sink: grid * 64 * W floats (device); clocks: grid * W * 5 uint64 (device):
// per wave (shader clock start, end, wall clock start, end, XCD << 32 |
// HW_ID).  Asynchronous on
// `stream`.  Returns 0, 1 for arguments out of range, or 2 + the HIP error.
extern "C" int fa_rates_run(int op, int grid, int iters, void* sink, void* clocks, void* stream) {
  if (op < 0 || op > kLdsTr || grid <= 0 || grid > (1 << 16) || iters <= 0 || !sink || !clocks)
    return 1;
  float* s = static_cast<float*>(sink);
  unsigned long long* c = static_cast<unsigned long long*>(clocks);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  switch (op) {
    case kMfma: e = launch<kMfma>(grid, iters, s, c, st); break;
    case kExp: e = launch<kExp>(grid, iters, s, c, st); break;
    case kFma: e = launch<kFma>(grid, iters, s, c, st); break;
    case kAdd: e = launch<kAdd>(grid, iters, s, c, st); break;
    case kCvt: e = launch<kCvt>(grid, iters, s, c, st); break;
    case kMixSelf: e = launch<kMixSelf>(grid, iters, s, c, st); break;
    case kMixWaves: e = launch<kMixWaves>(grid, iters, s, c, st); break;
    case kLds128: e = launch<kLds128>(grid, iters, s, c, st); break;
    case kLdsTr: e = launch<kLdsTr>(grid, iters, s, c, st); break;
  }
  return e == hipSuccess ? 0 : 2 + (int)e;
}
