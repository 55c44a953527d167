// Tiled exact attention, forward pass, for gfx950.
//
// FlashAttention forward (review page "Method"; slides steps 01-04; visual
// guide, "online softmax"): each work-group owns one tile of BR = 128 query
// rows of one (b, h) head and streams the key/value tiles that tile needs
// through LDS.  Scores never leave the compute unit; only O and the per-row
// logsumexp are written.  The pages' pseudocode runs key/value blocks in the
// outer loop and carries per-query-block state through memory; here the
// query tile is the outer (grid) dimension so that its state (running max m,
// denominator l, fp32 accumulator) stays in registers for the whole sweep.
// Both orders give the same result in exact arithmetic.
//
// Work split: 4 waves, wave w owns queries i0 + 32w .. i0 + 32w + 31.  Each
// step a wave forms the transposed score tile S^T (keys x queries) for a
// BC = 64-key tile: A = K tile rows from LDS, B = the wave's Q rows, held in
// registers for the whole kernel.  With keys as accumulator rows, each lane
// owns one query column, so the row max and row sum of the softmax are an
// in-register reduction plus one exchange with the lane 32 apart, and the
// exponentiated tile is already the B operand of O^T += V^T P^T (V^T is
// written to LDS transposed when the tile is staged).
//
// Pipeline: K/V tile j+1 is fetched from HBM into registers while tile j is
// being multiplied; it is written to the other half of a double buffer in LDS
// after the step, and one barrier per step separates the two.
//
// Masks are decided per tile: tiles beyond the causal diagonal, past the key
// length or with a zero block-mask entry are skipped (never loaded); only the
// tiles that straddle a boundary apply an element mask.

#include "fa_common.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kFwdWaves = 4;
constexpr int kFwdBR = 32 * kFwdWaves;  // query rows per work-group
constexpr int kFwdBC = 64;              // keys per staged K/V tile
constexpr int kMaskBlock = 128;         // block-mask granularity (keys and queries)

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int32_t* key_lens;
  const uint8_t* block_mask;
  int H, N, BH, nq, nblk;
  float scale;
  float c;  // scale * log2(e): exponents are taken base 2
  int causal;
};

template <typename T, int D>
struct FwdSmem {
  typedef raw_t<T> raw;
  static constexpr int VEC = 16 / sizeof(raw);       // elements per 16-byte chunk
  static constexpr int KS = D + VEC;                 // K row stride (+16 B against bank conflicts)
  static constexpr int VTS = kFwdBC + 4;              // V^T row stride (+4 elements)
  static constexpr int K_ELEMS = kFwdBC * KS;
  static constexpr int V_ELEMS = D * VTS;
  static constexpr int STAGE = K_ELEMS + V_ELEMS;
};

template <typename T, int D>
// Two waves per SIMD: one wave's softmax can run while the other's matrix
// products do.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void fa_fwd_kernel(
    FwdParams p) {
  typedef raw_t<T> raw;
  typedef raw4_t<T> raw4;
  typedef Traits<T> Tr;
  typedef FwdSmem<T, D> L;
  constexpr int BC = kFwdBC;
  constexpr int VEC = L::VEC;
  constexpr int KCH = BC * D / VEC / 256;  // 16-byte K chunks per thread
  constexpr int VBL = BC * D / 16 / 256;   // 4x4 V blocks per thread
  static_assert(KCH >= 1 && VBL >= 1, "tile too small for 256 threads");

  __shared__ __attribute__((aligned(16))) raw smem[2 * L::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;
  const int hh = lane >> 5;

  int qt, bh;
  map_tile(blockIdx.x, p.nq, p.BH, p.causal != 0, qt, bh);
  const int b = bh / p.H;
  const int N = p.N;
  const int i0 = qt * kFwdBR;
  const int qw0 = i0 + 32 * w;  // first query of this wave

  int kend = N;
  if (p.key_lens) kend = min(max(p.key_lens[b], 0), N);
  int kv_end = kend;
  if (p.causal) kv_end = min(kv_end, i0 + kFwdBR);
  const int nkt = kv_end > 0 ? (kv_end + BC - 1) / BC : 0;
  const uint8_t* bm = p.block_mask ? p.block_mask + (size_t)(i0 / kMaskBlock) * p.nblk : nullptr;
  auto kept = [&](int j) { return bm == nullptr || bm[(j * BC) / kMaskBlock] != 0; };
  auto next_kept = [&](int j) {
    while (j < nkt && !kept(j)) ++j;
    return j;
  };

  const size_t head = (size_t)bh * N * D;
  const raw* __restrict__ Qg = reinterpret_cast<const raw*>(p.q) + head;
  const raw* __restrict__ Kg = reinterpret_cast<const raw*>(p.k) + head;
  const raw* __restrict__ Vg = reinterpret_cast<const raw*>(p.v) + head;

  // The wave's Q rows as B operands (contiguous slot map over d).
  frag_t<T> qf[D / 16];
  {
    const int qrow = qw0 + col;
#pragma unroll
    for (int kc = 0; kc < D / 16; ++kc)
      qf[kc] = qrow < N ? load_frag<T>(Qg + (size_t)qrow * D + kc * 16 + hh * 8) : zero_frag<T>();
  }

  // Staging registers for one K/V tile.
  uint4 kreg[KCH];
  raw4 vreg[VBL][4];
  auto fetch = [&](int j) {
    const int kt0 = j * BC;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + 256 * i;
      const int row = c / (D / VEC), cv = c % (D / VEC);
      kreg[i] = kt0 + row < N
                    ? *reinterpret_cast<const uint4*>(Kg + (size_t)(kt0 + row) * D + cv * VEC)
                    : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < VBL; ++i) {
      const int c = tid + 256 * i;
      const int a = c / (D / 4), bc = c % (D / 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = kt0 + 4 * a + e;
        if (row < N) {
          vreg[i][e] = *reinterpret_cast<const raw4*>(Vg + (size_t)row * D + 4 * bc);
        } else {
#pragma unroll
          for (int t = 0; t < 4; ++t) vreg[i][e][t] = 0;
        }
      }
    }
  };
  auto stash = [&](int buf) {
    raw* Ks = smem + buf * L::STAGE;
    raw* Vt = Ks + L::K_ELEMS;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + 256 * i;
      const int row = c / (D / VEC), cv = c % (D / VEC);
      *reinterpret_cast<uint4*>(Ks + row * L::KS + cv * VEC) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < VBL; ++i) {
      const int c = tid + 256 * i;
      const int a = c / (D / 4), bc = c % (D / 4);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        raw4 col4;
#pragma unroll
        for (int e = 0; e < 4; ++e) col4[e] = vreg[i][e][t];
        *reinterpret_cast<raw4*>(Vt + (4 * bc + t) * L::VTS + 4 * a) = col4;
      }
    }
  };

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = zero16();
  float m_run = kNegInf;  // running max of raw scores q.k for this lane's query
  float l_run = 0.f;      // this lane's half of the running denominator
  const float c = p.c;
  const int myq = qw0 + col;

  int j = next_kept(0);
  if (j < nkt) {
    fetch(j);
    stash(0);
  }
  __syncthreads();
  int buf = 0;
  while (j < nkt) {
    const int jn = next_kept(j + 1);
    if (jn < nkt) fetch(jn);
    const int kt0 = j * BC;
    const raw* Ks = smem + buf * L::STAGE;
    const raw* Vt = Ks + L::K_ELEMS;

    if (!p.causal || kt0 <= qw0 + 31) {
      // S^T = K_j Q^T for this wave's 32 queries.
      f32x16 sacc[BC / 32];
#pragma unroll
      for (int kb = 0; kb < BC / 32; ++kb) {
        sacc[kb] = zero16();
#pragma unroll
        for (int kc = 0; kc < D / 16; ++kc) {
          const frag_t<T> a = load_frag<T>(Ks + (kb * 32 + col) * L::KS + kc * 16 + hh * 8);
          sacc[kb] = Tr::mma(a, qf[kc], sacc[kb]);
        }
      }
      const bool masked = (p.causal && kt0 + BC - 1 > qw0) || (kt0 + BC > kend);
      if (masked) {
#pragma unroll
        for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kt0 + kb * 32 + acc_row(r, hh);
            if (key >= kend || (p.causal && key > myq)) sacc[kb][r] = kNegInf;
          }
      }
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
      mx = pair_max(mx);
      const float m_new = fmaxf(m_run, mx);
      const float m_use = m_new == kNegInf ? 0.f : m_new;
      const float alpha = m_run == kNegInf ? 0.f : fast_exp2((m_run - m_use) * c);
      const float mc = m_use * c;
      float rs = 0.f;
      if (masked) {
#pragma unroll
        for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float s = sacc[kb][r];
            const float e = s == kNegInf ? 0.f : fast_exp2(fmaf(s, c, -mc));
            sacc[kb][r] = e;
            rs += e;
          }
      } else {
#pragma unroll
        for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float e = fast_exp2(fmaf(sacc[kb][r], c, -mc));
            sacc[kb][r] = e;
            rs += e;
          }
      }
      l_run = fmaf(l_run, alpha, rs);
      m_run = m_new;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;

      // O^T += V_j^T P^T.
      frag_t<T> pf[BC / 16];
#pragma unroll
      for (int kb = 0; kb < BC / 32; ++kb) {
        pf[2 * kb] = acc_to_frag<T>(sacc[kb], 0);
        pf[2 * kb + 1] = acc_to_frag<T>(sacc[kb], 1);
      }
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int kc = 0; kc < BC / 16; ++kc) {
          const frag_t<T> a = load_frag_acc_order<T>(Vt + (db * 32 + col) * L::VTS + kc * 16, hh);
          oacc[db] = Tr::mma(a, pf[kc], oacc[db]);
        }
    }

    if (jn < nkt) stash(buf ^ 1);
    __syncthreads();
    buf ^= 1;
    j = jn;
  }

  // Epilogue: O = acc / l, LSE = scale * m + ln(l).
  const float l_tot = pair_sum(l_run);
  if (myq < N) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    raw* Og = reinterpret_cast<raw*>(p.o) + head + (size_t)myq * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        raw4 out;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const T val = (T)(oacc[db][4 * g + t] * inv);
          out[t] = __builtin_bit_cast(raw, val);
        }
        *reinterpret_cast<raw4*>(Og + db * 32 + 8 * g + 4 * hh) = out;
      }
    if (hh == 0)
      p.lse[(size_t)bh * N + myq] = l_tot > 0.f ? m_run * p.scale + __logf(l_tot) : kNegInf;
  }
}

template <typename T, int D>
hipError_t launch_fwd_t(const Problem& pb, const FwdTensors& t) {
  FwdParams p;
  p.q = t.q; p.k = t.k; p.v = t.v; p.o = t.o; p.lse = t.lse;
  p.key_lens = pb.key_lens;
  p.block_mask = pb.block_mask;
  p.H = pb.H;
  p.N = pb.N;
  p.BH = pb.B * pb.H;
  p.nq = (pb.N + kFwdBR - 1) / kFwdBR;
  p.nblk = (pb.N + kMaskBlock - 1) / kMaskBlock;
  p.scale = pb.scale;
  p.c = pb.scale * kLog2e;
  p.causal = pb.causal;
  const unsigned grid = (unsigned)p.nq * (unsigned)p.BH;
  timing_begin(kFwd, pb.stream);
  hipLaunchKernelGGL((fa_fwd_kernel<T, D>), dim3(grid), dim3(256), 0, pb.stream, p);
  hipError_t e = hipGetLastError();
  timing_end(kFwd, pb.stream);
  return e;
}

}  // namespace

hipError_t launch_forward(const Problem& p, const FwdTensors& t) {
  switch (p.dtype * 1000 + p.d) {
    case 0 * 1000 + 64: return launch_fwd_t<float, 64>(p, t);
    case 0 * 1000 + 128: return launch_fwd_t<float, 128>(p, t);
    case 1 * 1000 + 64: return launch_fwd_t<_Float16, 64>(p, t);
    case 1 * 1000 + 128: return launch_fwd_t<_Float16, 128>(p, t);
    case 2 * 1000 + 64: return launch_fwd_t<__bf16, 64>(p, t);
    case 2 * 1000 + 128: return launch_fwd_t<__bf16, 128>(p, t);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa
