// Tiled exact attention, backward pass, for gfx950.
//
// The backward recomputes each probability tile on chip from the saved
// logsumexp instead of reading an N x N matrix (review page, "Method" and
// claim C7).  With P = exp(S - LSE) and D = rowsum(dO * O):
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  dK = scale dS^T Q,
//   dQ = scale dS K.
//
// Three launches on the caller's stream:
//   1. fa_bwd_preprocess_kernel: D for every row (reads O and dO once).
//   2. fa_bwd_dkdv_kernel: one work-group per 128 keys of a head; its four
//      waves keep K, V (as matrix operands) and the dK, dV accumulators in
//      registers and sweep the query tiles that see those keys.  The score
//      tile is formed with queries as accumulator rows, so P and dS are the B
//      operands of dV^T += dO^T P and dK^T += Q^T dS straight from registers;
//      Q and dO are staged in LDS both row-major and transposed.
//   3. fa_bwd_dq_kernel: one work-group per 128 queries; the same
//      recomputation with keys as accumulator rows (as in the forward) feeds
//      dQ^T += K^T dS^T, with K staged row-major and transposed.
// Splitting dQ into its own pass recomputes S and dP once more (6 d flops per
// pair on top of the 8 d of the dK/dV pass) but needs no atomics, keeps every
// accumulator in registers and makes the result deterministic.

#include "fa_common.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kMaskBlock = 128;

template <typename T> __device__ __forceinline__ float to_f32(raw_t<T> r);
template <> __device__ __forceinline__ float to_f32<__bf16>(uint16_t r) {
  return __uint_as_float((uint32_t)r << 16);
}
template <> __device__ __forceinline__ float to_f32<_Float16>(uint16_t r) {
  return (float)__builtin_bit_cast(_Float16, r);
}
template <> __device__ __forceinline__ float to_f32<float>(uint32_t r) { return __uint_as_float(r); }

// ----------------------------------------------------------------------------
// Stager for an R x D tile read as 4 x 4 element blocks: one global pass feeds
// a row-major copy and/or a transposed copy in LDS.  Rows at or past `limit`
// are read from row limit-1 (a valid address; no predicated loads): every use
// of such a row is masked by the caller.
template <typename T, int R, int D>
struct Stager {
  typedef raw_t<T> raw;
  typedef raw4_t<T> raw4;
  static constexpr int NB = R * D / 16 / 256;
  static_assert(NB >= 1 && (R * D / 16) % 256 == 0, "tile does not split over 256 threads");
  raw4 reg[NB][4];

  __device__ __forceinline__ void fetch(const raw* __restrict__ g, int row0, int limit, int tid) {
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int c = tid + 256 * i;
      const int a = c / (D / 4), bc = c % (D / 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = min(row0 + 4 * a + e, limit - 1);
        reg[i][e] = *reinterpret_cast<const raw4*>(g + (size_t)row * D + 4 * bc);
      }
    }
  }
  __device__ __forceinline__ void store_rows(raw* s, int stride, int tid) const {
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int c = tid + 256 * i;
      const int a = c / (D / 4), bc = c % (D / 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) *reinterpret_cast<raw4*>(s + (4 * a + e) * stride + 4 * bc) = reg[i][e];
    }
  }
  __device__ __forceinline__ void store_transposed(raw* s, int stride, int tid) const {
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int c = tid + 256 * i;
      const int a = c / (D / 4), bc = c % (D / 4);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        raw4 col4;
#pragma unroll
        for (int e = 0; e < 4; ++e) col4[e] = reg[i][e][t];
        *reinterpret_cast<raw4*>(s + (4 * bc + t) * stride + 4 * a) = col4;
      }
    }
  }
};

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* dvec;
  const int32_t* key_lens;
  const uint8_t* block_mask;
  int H, N, BH, nblk;
  float scale;
  float c;  // scale * log2(e)
  int causal;
};

// ----------------------------------------------------------------------------
// 1. D_i = sum_k dO_ik O_ik, float32, one row per group of TPR threads.
template <typename T, int D>
__global__ __launch_bounds__(256) void fa_bwd_preprocess_kernel(BwdParams p, long long rows) {
  typedef raw_t<T> raw;
  constexpr int VEC = 16 / sizeof(raw);
  constexpr int TPR = D / VEC;  // threads per row
  const int tid = threadIdx.x;
  const long long row = (long long)blockIdx.x * (256 / TPR) + tid / TPR;
  const int sub = tid % TPR;
  float acc = 0.f;
  if (row < rows) {
    const raw* O = reinterpret_cast<const raw*>(p.o) + row * D + sub * VEC;
    const raw* dO = reinterpret_cast<const raw*>(p.dout) + row * D + sub * VEC;
    const uint4 a = *reinterpret_cast<const uint4*>(O);
    const uint4 b = *reinterpret_cast<const uint4*>(dO);
    const raw* ar = reinterpret_cast<const raw*>(&a);
    const raw* br = reinterpret_cast<const raw*>(&b);
#pragma unroll
    for (int i = 0; i < VEC; ++i) acc = fmaf(to_f32<T>(ar[i]), to_f32<T>(br[i]), acc);
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, TPR);
  if (row < rows && sub == 0) p.dvec[row] = acc;
}

// ----------------------------------------------------------------------------
// 2. dK, dV.  Work-group: 4 waves x 32 keys; query tiles of BQ rows.
template <typename T, int D>
struct DkDvCfg {
  typedef raw_t<T> raw;
  // 64 query rows per step.  At d = 128 the persistent per-wave state (K, V
  // operands and the dK, dV accumulators: 192 VGPRs) only fits one wave per
  // SIMD, so one work-group per CU may use 140 KB of double-buffered LDS.
  static constexpr int BQ = (sizeof(raw) == 4 && D == 128) ? 32 : 64;
  static constexpr int WAVES_PER_SIMD = D == 128 ? 1 : 2;
  static constexpr int RS = D + 16 / (int)sizeof(raw);  // row-major stride (+16 B)
  static constexpr int TS = BQ + 4;                      // transposed stride
  static constexpr int Q_ELEMS = BQ * RS;
  static constexpr int QT_ELEMS = D * TS;
  // per stage: Q, dO (row-major), Q^T, dO^T, then 2*BQ floats (LSE*log2e, D)
  static constexpr int STAGE_RAW = 2 * Q_ELEMS + 2 * QT_ELEMS;
  static constexpr int STAGE_BYTES = STAGE_RAW * sizeof(raw) + 2 * BQ * 4;
};

template <typename T, int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(
    DkDvCfg<T, D>::WAVES_PER_SIMD))) void fa_bwd_dkdv_kernel(BwdParams p) {
  typedef raw_t<T> raw;
  typedef raw4_t<T> raw4;
  typedef Traits<T> Tr;
  typedef DkDvCfg<T, D> L;
  constexpr int BQ = L::BQ;
  constexpr int BK = 128;

  __shared__ __attribute__((aligned(16))) char smem_bytes[2 * L::STAGE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;
  const int hh = lane >> 5;
  const int N = p.N;
  const int nkt = (N + BK - 1) / BK;

  int kt, bh;
  map_tile(blockIdx.x, nkt, p.BH, false, kt, bh);
  const int b = bh / p.H;
  const int j0 = kt * BK;
  const int kw0 = j0 + 32 * w;  // first key of this wave
  const int myk = kw0 + col;

  int kend = N;
  if (p.key_lens) kend = min(max(p.key_lens[b], 0), N);

  const size_t head = (size_t)bh * N * D;
  const raw* __restrict__ Qg = reinterpret_cast<const raw*>(p.q) + head;
  const raw* __restrict__ Kg = reinterpret_cast<const raw*>(p.k) + head;
  const raw* __restrict__ Vg = reinterpret_cast<const raw*>(p.v) + head;
  const raw* __restrict__ dOg = reinterpret_cast<const raw*>(p.dout) + head;
  const float* __restrict__ lse = p.lse + (size_t)bh * N;
  const float* __restrict__ dvec = p.dvec + (size_t)bh * N;

  f32x16 dk_acc[D / 32], dv_acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    dk_acc[db] = zero16();
    dv_acc[db] = zero16();
  }

  // Query-tile range that sees keys [j0, j0 + BK).
  const int nqt = (N + BQ - 1) / BQ;
  int t_begin = p.causal ? j0 / BQ : 0;
  int t_end = j0 < kend ? nqt : t_begin;  // no visible key in this tile: nothing to do
  const uint8_t* bm_col = p.block_mask ? p.block_mask + j0 / kMaskBlock : nullptr;
  auto kept = [&](int t) {
    return bm_col == nullptr || bm_col[(size_t)((t * BQ) / kMaskBlock) * p.nblk] != 0;
  };
  auto next_kept = [&](int t) {
    while (t < t_end && !kept(t)) ++t;
    return t;
  };

  if (t_begin < t_end) {
    // K and V of this wave's keys as B operands (contiguous slot map over d).
    frag_t<T> kf[D / 16], vf[D / 16];
#pragma unroll
    for (int kc = 0; kc < D / 16; ++kc) {
      const bool ok = myk < N;
      kf[kc] = ok ? load_frag<T>(Kg + (size_t)myk * D + kc * 16 + hh * 8) : zero_frag<T>();
      vf[kc] = ok ? load_frag<T>(Vg + (size_t)myk * D + kc * 16 + hh * 8) : zero_frag<T>();
    }

    Stager<T, BQ, D> sq, sdo;
    float lse2_r = 0.f, dvec_r = 0.f;
    auto fetch = [&](int t) {
      const int i0 = t * BQ;
      sq.fetch(Qg, i0, N, tid);
      sdo.fetch(dOg, i0, N, tid);
      if (tid < BQ) {
        const int i = i0 + tid;
        const float l = i < N ? lse[i] : kNegInf;
        // Rows without any visible key (LSE = -inf) and rows past N get
        // +inf here, so that their recomputed probabilities are exactly 0.
        lse2_r = l == kNegInf ? __builtin_inff() : l * kLog2e;
        dvec_r = i < N ? dvec[i] : 0.f;
      }
    };
    auto stash = [&](int buf) {
      raw* base = reinterpret_cast<raw*>(smem_bytes + buf * L::STAGE_BYTES);
      sq.store_rows(base, L::RS, tid);
      sdo.store_rows(base + L::Q_ELEMS, L::RS, tid);
      sq.store_transposed(base + 2 * L::Q_ELEMS, L::TS, tid);
      sdo.store_transposed(base + 2 * L::Q_ELEMS + L::QT_ELEMS, L::TS, tid);
      float* f = reinterpret_cast<float*>(base + L::STAGE_RAW);
      if (tid < BQ) {
        f[tid] = lse2_r;
        f[BQ + tid] = dvec_r;
      }
    };

    const float c = p.c;
    int t = next_kept(t_begin);
    if (t < t_end) {
      fetch(t);
      stash(0);
    }
    __syncthreads();
    int buf = 0;
    while (t < t_end) {
      const int tn = next_kept(t + 1);
      if (tn < t_end) fetch(tn);
      const int qi0 = t * BQ;
      const raw* Qs = reinterpret_cast<const raw*>(smem_bytes + buf * L::STAGE_BYTES);
      const raw* dOs = Qs + L::Q_ELEMS;
      const raw* QTs = Qs + 2 * L::Q_ELEMS;
      const raw* dOTs = QTs + L::QT_ELEMS;
      const float* lse2s = reinterpret_cast<const float*>(Qs + L::STAGE_RAW);
      const float* dvs = lse2s + BQ;

      if (!p.causal || kw0 <= qi0 + BQ - 1) {
        // S (queries x keys) and dP, with queries as accumulator rows.
        f32x16 sacc[BQ / 32], pacc[BQ / 32];
#pragma unroll
        for (int qb = 0; qb < BQ / 32; ++qb) {
          sacc[qb] = zero16();
          pacc[qb] = zero16();
#pragma unroll
          for (int kc = 0; kc < D / 16; ++kc) {
            const frag_t<T> aq = load_frag<T>(Qs + (qb * 32 + col) * L::RS + kc * 16 + hh * 8);
            sacc[qb] = Tr::mma(aq, kf[kc], sacc[qb]);
            const frag_t<T> ad = load_frag<T>(dOs + (qb * 32 + col) * L::RS + kc * 16 + hh * 8);
            pacc[qb] = Tr::mma(ad, vf[kc], pacc[qb]);
          }
        }
        const bool masked =
            (p.causal && kw0 + 31 > qi0) || (kw0 + 32 > kend) || (qi0 + BQ > N);
#pragma unroll
        for (int qb = 0; qb < BQ / 32; ++qb)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int r0 = qb * 32 + 8 * g + 4 * hh;  // first of 4 consecutive query rows
            const float4 l4 = *reinterpret_cast<const float4*>(lse2s + r0);
            const float4 d4 = *reinterpret_cast<const float4*>(dvs + r0);
            const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
            const float dv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const int r = 4 * g + u;
              float pr = fast_exp2(fmaf(sacc[qb][r], c, -lv[u]));
              if (masked) {
                const int qi = qi0 + r0 + u;
                if (myk >= kend || qi >= N || (p.causal && myk > qi)) pr = 0.f;
              }
              sacc[qb][r] = pr;                        // P
              pacc[qb][r] = pr * (pacc[qb][r] - dv[u]);  // dS = P (dP - D)
            }
          }
        // dV^T += dO^T P,  dK^T += Q^T dS  (k = queries, acc-ordered slots).
#pragma unroll
        for (int qc = 0; qc < BQ / 16; ++qc) {
          const frag_t<T> pf = acc_to_frag<T>(sacc[qc / 2], qc % 2);
          const frag_t<T> sf = acc_to_frag<T>(pacc[qc / 2], qc % 2);
#pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            const frag_t<T> ado = load_frag_acc_order<T>(dOTs + (db * 32 + col) * L::TS + qc * 16, hh);
            dv_acc[db] = Tr::mma(ado, pf, dv_acc[db]);
            const frag_t<T> aq = load_frag_acc_order<T>(QTs + (db * 32 + col) * L::TS + qc * 16, hh);
            dk_acc[db] = Tr::mma(aq, sf, dk_acc[db]);
          }
        }
      }

      if (tn < t_end) stash(buf ^ 1);
      __syncthreads();
      buf ^= 1;
      t = tn;
    }
  }

  // Store dK = scale * (dK^T)^T and dV; lane owns key `myk`, rows d of its half.
  if (myk < N) {
    raw* dKg = reinterpret_cast<raw*>(p.dk) + head + (size_t)myk * D;
    raw* dVg = reinterpret_cast<raw*>(p.dv) + head + (size_t)myk * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        raw4 ok, ov;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          ok[u] = __builtin_bit_cast(raw, (T)(dk_acc[db][4 * g + u] * p.scale));
          ov[u] = __builtin_bit_cast(raw, (T)dv_acc[db][4 * g + u]);
        }
        *reinterpret_cast<raw4*>(dKg + db * 32 + 8 * g + 4 * hh) = ok;
        *reinterpret_cast<raw4*>(dVg + db * 32 + 8 * g + 4 * hh) = ov;
      }
  }
}

// ----------------------------------------------------------------------------
// 3. dQ.  Work-group: 4 waves x 32 queries; key tiles of BC rows.
template <typename T, int D>
struct DqCfg {
  typedef raw_t<T> raw;
  // 64 keys per step at d = 64; 32 at d = 128 so that two work-groups
  // (double-buffered stages) fit in one CU's LDS.
  static constexpr int BC = D == 128 ? 32 : 64;
  static constexpr int RS = D + 16 / (int)sizeof(raw);
  static constexpr int TS = BC + 4;
  static constexpr int K_ELEMS = BC * RS;
  static constexpr int KT_ELEMS = D * TS;
  static constexpr int STAGE = 2 * K_ELEMS + KT_ELEMS;  // K, V row-major; K^T
};

template <typename T, int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void fa_bwd_dq_kernel(
    BwdParams p) {
  typedef raw_t<T> raw;
  typedef raw4_t<T> raw4;
  typedef Traits<T> Tr;
  typedef DqCfg<T, D> L;
  constexpr int BC = L::BC;
  constexpr int BR = 128;

  __shared__ __attribute__((aligned(16))) raw smem[2 * L::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;
  const int hh = lane >> 5;
  const int N = p.N;
  const int nq = (N + BR - 1) / BR;

  int qt, bh;
  map_tile(blockIdx.x, nq, p.BH, p.causal != 0, qt, bh);
  const int b = bh / p.H;
  const int i0 = qt * BR;
  const int qw0 = i0 + 32 * w;
  const int myq = qw0 + col;

  int kend = N;
  if (p.key_lens) kend = min(max(p.key_lens[b], 0), N);
  int kv_end = kend;
  if (p.causal) kv_end = min(kv_end, i0 + BR);
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
  const raw* __restrict__ dOg = reinterpret_cast<const raw*>(p.dout) + head;

  frag_t<T> qf[D / 16], df[D / 16];
#pragma unroll
  for (int kc = 0; kc < D / 16; ++kc) {
    const bool ok = myq < N;
    qf[kc] = ok ? load_frag<T>(Qg + (size_t)myq * D + kc * 16 + hh * 8) : zero_frag<T>();
    df[kc] = ok ? load_frag<T>(dOg + (size_t)myq * D + kc * 16 + hh * 8) : zero_frag<T>();
  }
  float lse2 = __builtin_inff(), dval = 0.f;
  if (myq < N) {
    const float l = p.lse[(size_t)bh * N + myq];
    lse2 = l == kNegInf ? __builtin_inff() : l * kLog2e;
    dval = p.dvec[(size_t)bh * N + myq];
  }

  f32x16 dq_acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) dq_acc[db] = zero16();

  Stager<T, BC, D> sk, sv;
  auto fetch = [&](int j) {
    sk.fetch(Kg, j * BC, N, tid);
    sv.fetch(Vg, j * BC, N, tid);
  };
  auto stash = [&](int buf) {
    raw* Ks = smem + buf * L::STAGE;
    sk.store_rows(Ks, L::RS, tid);
    sv.store_rows(Ks + L::K_ELEMS, L::RS, tid);
    sk.store_transposed(Ks + 2 * L::K_ELEMS, L::TS, tid);
  };

  const float c = p.c;
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
    const raw* Vs = Ks + L::K_ELEMS;
    const raw* KTs = Ks + 2 * L::K_ELEMS;

    if (!p.causal || kt0 <= qw0 + 31) {
      f32x16 sacc[BC / 32], pacc[BC / 32];
#pragma unroll
      for (int kb = 0; kb < BC / 32; ++kb) {
        sacc[kb] = zero16();
        pacc[kb] = zero16();
#pragma unroll
        for (int kc = 0; kc < D / 16; ++kc) {
          const frag_t<T> ak = load_frag<T>(Ks + (kb * 32 + col) * L::RS + kc * 16 + hh * 8);
          sacc[kb] = Tr::mma(ak, qf[kc], sacc[kb]);
          const frag_t<T> av = load_frag<T>(Vs + (kb * 32 + col) * L::RS + kc * 16 + hh * 8);
          pacc[kb] = Tr::mma(av, df[kc], pacc[kb]);
        }
      }
      const bool masked = (p.causal && kt0 + BC - 1 > qw0) || (kt0 + BC > kend);
#pragma unroll
      for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float pr = fast_exp2(fmaf(sacc[kb][r], c, -lse2));
          if (masked) {
            const int key = kt0 + kb * 32 + acc_row(r, hh);
            if (key >= kend || (p.causal && key > myq)) pr = 0.f;
          }
          pacc[kb][r] = pr * (pacc[kb][r] - dval);  // dS^T
        }
      // dQ^T += K^T dS^T  (k = keys, acc-ordered slots).
#pragma unroll
      for (int kc = 0; kc < BC / 16; ++kc) {
        const frag_t<T> sf = acc_to_frag<T>(pacc[kc / 2], kc % 2);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const frag_t<T> a = load_frag_acc_order<T>(KTs + (db * 32 + col) * L::TS + kc * 16, hh);
          dq_acc[db] = Tr::mma(a, sf, dq_acc[db]);
        }
      }
    }

    if (jn < nkt) stash(buf ^ 1);
    __syncthreads();
    buf ^= 1;
    j = jn;
  }

  if (myq < N) {
    raw* dQg = reinterpret_cast<raw*>(p.dq) + head + (size_t)myq * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        raw4 out;
#pragma unroll
        for (int u = 0; u < 4; ++u)
          out[u] = __builtin_bit_cast(raw, (T)(dq_acc[db][4 * g + u] * p.scale));
        *reinterpret_cast<raw4*>(dQg + db * 32 + 8 * g + 4 * hh) = out;
      }
  }
}

template <typename T, int D>
hipError_t launch_bwd_t(const Problem& pb, const BwdTensors& t) {
  BwdParams p;
  p.q = t.q; p.k = t.k; p.v = t.v; p.o = t.o; p.dout = t.dout; p.lse = t.lse;
  p.dq = t.dq; p.dk = t.dk; p.dv = t.dv; p.dvec = t.dvec;
  p.key_lens = pb.key_lens;
  p.block_mask = pb.block_mask;
  p.H = pb.H;
  p.N = pb.N;
  p.BH = pb.B * pb.H;
  p.nblk = (pb.N + kMaskBlock - 1) / kMaskBlock;
  p.scale = pb.scale;
  p.c = pb.scale * kLog2e;
  p.causal = pb.causal;

  const long long rows = (long long)p.BH * pb.N;
  constexpr int TPR = D * (int)sizeof(raw_t<T>) / 16;
  const unsigned pre_grid = (unsigned)((rows + (256 / TPR) - 1) / (256 / TPR));
  timing_begin(kBwdPre, pb.stream);
  hipLaunchKernelGGL((fa_bwd_preprocess_kernel<T, D>), dim3(pre_grid), dim3(256), 0, pb.stream, p,
                     rows);
  hipError_t e = hipGetLastError();
  timing_end(kBwdPre, pb.stream);
  if (e != hipSuccess) return e;

  const unsigned tiles128 = (unsigned)((pb.N + 127) / 128);
  timing_begin(kBwdDkDv, pb.stream);
  hipLaunchKernelGGL((fa_bwd_dkdv_kernel<T, D>), dim3(tiles128 * p.BH), dim3(256), 0, pb.stream, p);
  e = hipGetLastError();
  timing_end(kBwdDkDv, pb.stream);
  if (e != hipSuccess) return e;

  timing_begin(kBwdDq, pb.stream);
  hipLaunchKernelGGL((fa_bwd_dq_kernel<T, D>), dim3(tiles128 * p.BH), dim3(256), 0, pb.stream, p);
  e = hipGetLastError();
  timing_end(kBwdDq, pb.stream);
  return e;
}

}  // namespace

hipError_t launch_backward(const Problem& p, const BwdTensors& t) {
  switch (p.dtype * 1000 + p.d) {
    case 0 * 1000 + 64: return launch_bwd_t<float, 64>(p, t);
    case 0 * 1000 + 128: return launch_bwd_t<float, 128>(p, t);
    case 1 * 1000 + 64: return launch_bwd_t<_Float16, 64>(p, t);
    case 1 * 1000 + 128: return launch_bwd_t<_Float16, 128>(p, t);
    case 2 * 1000 + 64: return launch_bwd_t<__bf16, 64>(p, t);
    case 2 * 1000 + 128: return launch_bwd_t<__bf16, 128>(p, t);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa
