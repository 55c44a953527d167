// Tiled exact attention, backward pass, for gfx950 (kernel templates; the
// instances live in fa_bwd.hip (16-bit) and fa_bwd_f32.hip (fp32)).
//
// The backward recomputes each probability tile on chip from the saved
// logsumexp instead of reading an N x N matrix (review page, "Method" and
// claim C7).  With P = exp(S - LSE) and D = rowsum(dO * O):
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  dK = scale dS^T Q,
//   dQ = scale dS K.
//
// Two launches on the caller's stream:
//   1. fa_bwd_dq_kernel: one work-group per 128 queries; scores recomputed
//      with keys as accumulator rows (as in the forward) feed
//      dQ^T += K^T dS^T, K^T by transposing LDS reads.  Each lane holds its
//      query's Q and dO rows; it also reads the O row, forms
//      D = rowsum(dO * O) and writes -D and LSE * log2(e) to the caller's
//      workspace for the second pass.
//   2. fa_bwd_dkdv_kernel: one work-group per 128 keys of a head; its four
//      waves keep K, V (as matrix operands) and the dK, dV accumulators in
//      registers and sweep the query tiles that see those keys.  The score
//      tile is formed with queries as accumulator rows, so P and dS are the B
//      operands of dV^T += dO^T P and dK^T += Q^T dS straight from registers;
//      dO^T and Q^T come from the row-major tiles by transposing LDS reads.
//      At d = 128 those registers would allow one wave per SIMD, so by
//      default eight waves share each query tile instead (two per 32-key
//      block, one 32-query half each) and read K and V from LDS.
// Splitting dQ into its own pass recomputes S and dP once more (6 d flops per
// pair on top of the 8 d of the dK/dV pass) but needs no atomics, keeps every
// accumulator in registers and makes the result deterministic.
//
// Streaming (both passes): the tiles of the streamed operand go from HBM
// straight into a 4-slot LDS ring by direct-to-LDS loads, requested two steps
// before use; one barrier per step.
//
// Long block-sparse rows and columns (a "global" block row attends every key
// block, a global column is seen by every query block) would make one
// work-group's sweep the whole kernel's critical path.  The split instances
// (SPLIT) therefore hand out each row (dQ pass) or column (dK/dV pass) in
// items of chunk_blocks kept mask blocks, one work-group per item
// (gridDim.y = items of the longest row).  A tile with at most chunk_blocks
// kept blocks is one item and writes its result directly; the items of a
// longer one write fp32 partials that fa_bwd_split_reduce_kernel sums in item
// order, so the result stays deterministic.
//
// Masks: tiles that straddle a causal, padding or sequence boundary apply the
// element mask after the exponentials, in a loop of their own behind one
// wave-uniform branch (or as selects in the interleaved step); a run-time
// mask flag tested inside the exponential loop compiles to one branch per
// element.

#pragma once

#include "fa_common.h"

#include <type_traits>
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kMaskBlock = 128;
constexpr int kMaxMaskBlocks = 1024;   // block-mask row cached in LDS (N <= 131072)

template <typename T> __device__ __forceinline__ float to_f32(raw_t<T> r);
template <> __device__ __forceinline__ float to_f32<__bf16>(uint16_t r) {
  return __uint_as_float((uint32_t)r << 16);
}
template <> __device__ __forceinline__ float to_f32<_Float16>(uint16_t r) {
  return (float)__builtin_bit_cast(_Float16, r);
}
template <> __device__ __forceinline__ float to_f32<float>(uint32_t r) { return __uint_as_float(r); }

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
  float* lse2;   // workspace: LSE * log2(e), +inf for rows without a visible key
  float* dvec;   // workspace: -D = -rowsum(dO * O)
  const int32_t* key_lens;
  const uint8_t* block_mask;
  int H, N, BH, nblk;
  int hgroup;  // heads per XCD dispatched together (map_tile)
  float scale;
  float c;  // scale * log2(e)
  int causal;
  // Split by kept mask blocks (SPLIT instances): work-group (tile, item)
  // takes kept blocks item * chunk_blocks .. of its row or column; tiles
  // with more than chunk_blocks kept blocks write fp32 partials
  // [item][BH][N][d] (dK scaled), summed by fa_bwd_split_reduce_kernel.
  int chunk_blocks;
  float* part_dq;
  float* part_dk;
  float* part_dv;
  // Written by fa_bwd_split_prep_kernel: kept blocks of each mask row, then
  // of each column ([2][nblk], whole rows and columns: an upper bound on
  // what a pass counts, enough to drop items that cannot exist before they
  // load anything), and the mask transposed ([nblk][nblk], so that the dK/dV
  // pass reads its column contiguously).
  int* split_counts;
  uint8_t* mask_t;
};

// Split backward, before both passes: per mask row and column the kept
// blocks, and the transposed mask.  One work-group per mask row r.
__global__ __launch_bounds__(256) void fa_bwd_split_prep_kernel(BwdParams p) {
  const int r = (int)blockIdx.x, nb = p.nblk;
  int rows = 0, cols = 0;
  for (int base = 0; base < nb; base += 256) {
    const int i = base + (int)threadIdx.x;
    const bool in = i < nb;
    const uint8_t mr = in ? p.block_mask[(size_t)r * nb + i] : 0;
    const uint8_t mc = in ? p.block_mask[(size_t)i * nb + r] : 0;
    if (in) p.mask_t[(size_t)r * nb + i] = mc;
    rows += __syncthreads_count(mr != 0);
    cols += __syncthreads_count(mc != 0);
  }
  if (threadIdx.x == 0) {
    p.split_counts[r] = rows;
    p.split_counts[nb + r] = cols;
  }
}

// Kept blocks among m[lo, hi) (LDS copy of a mask row or column; every wave
// computes the same wave-uniform count).
__device__ __forceinline__ int count_kept(const uint8_t* m, int lo, int hi, int lane) {
  int n = 0;
  for (int base = lo; base < hi; base += 64) {
    const int i = base + lane;
    n += __builtin_popcountll(__builtin_amdgcn_ballot_w64(i < hi && m[i] != 0));
  }
  return n;
}

// Index of the kept block of rank `rank` (0-based) among m[lo, hi), or hi if
// there are not that many.
__device__ __forceinline__ int kth_kept(const uint8_t* m, int lo, int hi, int rank, int lane) {
  int before = 0;
  for (int base = lo; base < hi; base += 64) {
    const int i = base + lane;
    const bool kept = i < hi && m[i] != 0;
    const uint64_t bits = __builtin_amdgcn_ballot_w64(kept);
    const int n = __builtin_popcountll(bits);
    if (rank < before + n) {
      const int r = __builtin_popcountll(bits & ((1ull << lane) - 1ull));
      const uint64_t hit = __builtin_amdgcn_ballot_w64(kept && r == rank - before);
      return base + (int)__builtin_ctzll(hit);
    }
    before += n;
  }
  return hi;
}

// ----------------------------------------------------------------------------
// dK, dV.  Work-group: NW waves x 32 keys (4 by default; 2 and 8 are a
// tile-size option); query tiles of BQ rows.
//
// QS (16-bit, d = 128, 8 waves): the two waves of each 32-key block share
// every query tile, one 32-query half each, so that two waves per SIMD fit:
// K and V are read from LDS rather than held in registers.
template <typename T, int D, int NW = 4, bool QS = false>
struct DkDvCfg {
  typedef raw_t<T> raw;
  static constexpr int BQ = (sizeof(raw) == 4 && D == 128) ? 32 : 64;
  static constexpr int NS = 4;
  static constexpr int TILE_BYTES = BQ * D * (int)sizeof(raw);   // one of Q, dO
  static constexpr int ROWV_BYTES = 64 * 4;                      // LSE2 or D words (one DMA)
  static constexpr int SLOT_BYTES = 2 * TILE_BYTES + 2 * ROWV_BYTES;
  static constexpr int LPT = 2 * TILE_BYTES / (1024 * NW);       // 16-byte DMAs per wave per tile
  // At d = 128 the persistent per-wave state (K, V operands and the dK, dV
  // accumulators: 192 VGPRs) only fits one wave per SIMD; with QS the K and
  // V operands come from LDS and two waves fit.
  static constexpr int WAVES_PER_SIMD = D == 128 && !QS ? 1 : 2;
  // Read each group of matrix operands one group ahead of its products
  // (explicit, fenced with scheduling barriers): the compiler otherwise reads
  // each operand just before its product.  Groups of GK k-steps: 4 at
  // d = 128 (one wave per SIMD, registers to spare), 2 at d = 64 (two waves
  // per SIMD, 256 VGPRs).
  static constexpr bool PREFETCH = true;
  static constexpr int GK = D == 64 ? 2 : 4;
  // One wave per SIMD (16-bit, d = 128): no other wave overlaps this one's
  // softmax with matrix work, so the step interleaves them itself (the
  // softmax of query block 0 beside the score products of block 1, that of
  // block 1 beside the first gradient products).
  static constexpr bool ILV = D == 128 && sizeof(raw) == 2 && !QS;
};

// GF32: store dK, dV as float32 (16-bit inputs; an option for exact
// comparisons, compiled as separate instances so that the usual instances'
// register allocation is untouched).
//
// KG = 2 (dense problems at d = 64, chosen by the caller): the NW waves form
// two key groups of NW / 2 that share the keys and sweep the first and
// second half of the query tiles, each through its own ring; group 1 adds
// its dK, dV accumulators into group 0's through LDS.
//
// QS (with KG = 2, 16-bit, d = 128): the groups split every query tile
// instead of the tile range: group g takes query block g (32 of the tile's
// 64 queries) of each tile, from one 2-slot ring that both read; K and V of
// the work-group's 128 keys sit in LDS beside it (64 KB), which frees the 64
// registers per wave that hold them otherwise, so two waves per SIMD fit.
template <typename T, int D, bool GF32 = false, bool SPLIT = false, int NW = 4, int KG = 1,
          bool QS = false>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(
    DkDvCfg<T, D, NW / KG, QS>::WAVES_PER_SIMD))) void fa_bwd_dkdv_kernel(BwdParams p) {
  static_assert(KG == 1 || (KG == 2 && !SPLIT), "key groups: unsplit passes");
  static_assert(!QS || (KG == 2 && sizeof(raw_t<T>) == 2), "split query tiles: two groups, 16-bit");
  constexpr int RW = NW / KG;  // waves per key group (32 keys each)
  typedef raw_t<T> raw;
  typedef raw4_t<T> raw4;
  typedef Traits<T> Tr;
  typedef DkDvCfg<T, D, RW, QS> L;
  constexpr int BQ = L::BQ;
  constexpr int BK = 32 * RW;  // keys of this work-group (at most one mask block)
  static_assert(BK <= kMaskBlock || !SPLIT, "split columns come in whole mask blocks");
  constexpr int LPT = L::LPT;
  // QS: one 2-slot ring shared by both groups, then K and V (row-major).
  constexpr int NSL = QS ? 2 : L::NS;
  constexpr int RING_BYTES = (QS ? 1 : KG) * NSL * L::SLOT_BYTES;
  constexpr int KV_TILE = QS ? BK * D * (int)sizeof(raw) : 0;

  __shared__ __attribute__((aligned(1024))) char ring[RING_BYTES + 2 * KV_TILE];
  __shared__ uint8_t mask_col[kMaxMaskBlocks];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wg_wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kgrp = KG > 1 ? wg_wave / RW : 0;        // key group of this wave
  const int w = KG > 1 ? wg_wave % RW : wg_wave;     // key wave within the group
  char* const gring = ring + (QS ? 0 : kgrp * L::NS * L::SLOT_BYTES);  // this group's ring
  const uint32_t ring_lds = lds_addr(gring);
  const int col = lane & 31;
  const int hh = lane >> 5;
  const int N = p.N;
  const int nkt = (N + BK - 1) / BK;

  int kt, bh;
  map_tile(blockIdx.x, nkt, p.BH, false, p.hgroup, kt, bh);
  if constexpr (SPLIT) {
    // an item past every kept block of this column: nothing to do
    if (blockIdx.y > 0 && (int)blockIdx.y * p.chunk_blocks >= p.split_counts[p.nblk + kt]) return;
  }
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
  const float* __restrict__ lse2g = p.lse2 + (size_t)bh * N;
  const float* __restrict__ dvecg = p.dvec + (size_t)bh * N;

  // Query tiles that see keys [j0, j0 + BK); the block-mask column of this
  // key block is cached in LDS.
  const int nqt = (N + BQ - 1) / BQ;
  int t_begin = p.causal ? j0 / BQ : 0;
  int t_end = j0 < kend ? nqt : t_begin;  // no visible key in this tile: nothing to do
  const bool sparse = p.block_mask != nullptr;
  if (sparse) {
    for (int i = tid; i < p.nblk; i += 64 * NW)
      mask_col[i] = SPLIT ? p.mask_t[(size_t)(j0 / kMaskBlock) * p.nblk + i]
                          : p.block_mask[(size_t)i * p.nblk + j0 / kMaskBlock];
  }

  f32x16 dk_acc[D / 32], dv_acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    dk_acc[db] = zero16();
    dv_acc[db] = zero16();
  }
  // K and V of this wave's keys as B operands (contiguous slot map over d).
  frag_t<T> kf[D / 16], vf[D / 16];
  if constexpr (!QS) {
#pragma unroll
    for (int kc = 0; kc < D / 16; ++kc) {
      const bool ok = myk < N;
      kf[kc] = ok ? load_frag<T>(Kg + (size_t)myk * D + kc * 16 + hh * 8) : zero_frag<T>();
      vf[kc] = ok ? load_frag<T>(Vg + (size_t)myk * D + kc * 16 + hh * 8) : zero_frag<T>();
    }
  }
  // QS: K and V rows of the work-group's keys in LDS (copied by all waves;
  // rows past N repeat row N-1, and no key past N is stored).
  const raw* const Kt = reinterpret_cast<const raw*>(ring + RING_BYTES);
  const raw* const Vt = Kt + BK * D;
  if constexpr (QS) {
    DmaPlan<raw, BK, D, kRows, NW> kvplan;
    kvplan.init(wg_wave, lane);
    kvplan.copy(Kg, j0, N, lds_addr(ring) + RING_BYTES, lane);
    kvplan.copy(Vg, j0, N, lds_addr(ring) + RING_BYTES + KV_TILE, lane);
  }
  __syncthreads();  // mask_col visible

  // Split: this work-group's item of the column's kept query blocks.
  bool multi = false;  // the column has more than one item: write partials
  const int item = SPLIT ? (int)blockIdx.y : 0;
  if constexpr (SPLIT) {
    const int qlo = (t_begin * BQ) / kMaskBlock;
    const int qhi = min((t_end * BQ + kMaskBlock - 1) / kMaskBlock, p.nblk);
    const int total = count_kept(mask_col, qlo, qhi, lane);
    const int C = p.chunk_blocks;
    if (item > 0 && item * C >= total) return;  // whole work-group, no barrier pending
    multi = total > C;
    const int b0 = kth_kept(mask_col, qlo, qhi, item * C, lane);
    const int b1 = kth_kept(mask_col, qlo, qhi, (item + 1) * C, lane);
    t_begin = max(t_begin, b0 * (kMaskBlock / BQ));
    t_end = min(t_end, b1 * (kMaskBlock / BQ));
    if (t_end < t_begin) t_end = t_begin;
  }

  auto next_kept = [&](int t) {
    if (!sparse) return t;
    while (t < t_end && mask_col[(t * BQ) / kMaskBlock] == 0) ++t;
    return t;
  };

  // (a key group copies its own tiles; with QS all waves copy the shared ones)
  DmaPlan<raw, BQ, D, kBoth, QS ? NW : RW> plan;
  plan.init(QS ? wg_wave : w, lane);
  // Q, dO rows of tile t, plus (waves 0 and 1) its LSE2 and D words.
  auto issue = [&](int t, int s) {
    const uint32_t base = ring_lds + s * L::SLOT_BYTES;
    const int qi0 = t * BQ;
    plan.copy(Qg, qi0, N, base, lane);
    plan.copy(dOg, qi0, N, base + L::TILE_BYTES, lane);
    if ((QS ? wg_wave : w) < 2) {
      const uint32_t voff = (uint32_t)min(qi0 + lane, N - 1) * 4u;
      dma4s(voff, w == 0 ? (const void*)lse2g : (const void*)dvecg,
            base + 2 * L::TILE_BYTES + w * L::ROWV_BYTES);
    }
  };
  // wait until at most `tiles` whole tiles of this wave's DMAs are in flight
  auto wait_tiles = [&](int tiles) {
    if (w < 2) {
      if (tiles == 2) wait_vmcnt<2 * (LPT + 1)>();
      else if (tiles == 1) wait_vmcnt<LPT + 1>();
      else wait_vmcnt<0>();
    } else {
      if (tiles == 2) wait_vmcnt<2 * LPT>();
      else if (tiles == 1) wait_vmcnt<LPT>();
      else wait_vmcnt<0>();
    }
  };

  const float c = p.c;
  typedef f32x16 qblk[BQ / 32];
  // -D of the accumulator rows of query block qb of the tile in `slot`
  // (queries qb*32 + 8g + 4hh + u), read from the words staged beside Q, dO.
  auto dneg_of = [&](const char* slot, int qb) {
    const float* dns = reinterpret_cast<const float*>(slot + 2 * L::TILE_BYTES) + 64;
    f32x16 dneg;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float4 d4 = *reinterpret_cast<const float4*>(dns + qb * 32 + 8 * g + 4 * hh);
      dneg[4 * g] = d4.x;
      dneg[4 * g + 1] = d4.y;
      dneg[4 * g + 2] = d4.z;
      dneg[4 * g + 3] = d4.w;
    }
    return dneg;
  };
  // S (queries x keys) and dP = dO V^T of the query tile in `slot`, with
  // queries as accumulator rows.
  auto sdp = [&](const char* slot, qblk& sacc, qblk& pacc) {
    const raw* Qs = reinterpret_cast<const raw*>(slot);
    const raw* dOs = reinterpret_cast<const raw*>(slot + L::TILE_BYTES);
    if constexpr (L::PREFETCH) {
      // groups of GK k-steps of one query block, read one group ahead
      constexpr int GK = L::GK, NG = D / 16 / GK;
      frag_t<T> fq[2][GK], fd[2][GK];
      auto ld = [&](int g, int b) {
        const int qb = g / NG, k0 = (g % NG) * GK;
#pragma unroll
        for (int j = 0; j < GK; ++j) {
          fq[b][j] = load_frag_swz<T, D, kBoth>(Qs, qb * 32 + col, (k0 + j) * 16 + hh * 8);
          fd[b][j] = load_frag_swz<T, D, kBoth>(dOs, qb * 32 + col, (k0 + j) * 16 + hh * 8);
        }
      };
      ld(0, 0);
      f32x16 dneg;
#pragma unroll
      for (int g = 0; g < BQ / 32 * NG; ++g) {
        const int qb = g / NG, k0 = (g % NG) * GK;
        if (k0 == 0) dneg = dneg_of(slot, qb);
        if (g + 1 < BQ / 32 * NG) ld(g + 1, (g + 1) & 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < GK; ++j) {
          const int kc = k0 + j;
          sacc[qb] = Tr::mma(fq[g & 1][j], kf[kc], kc == 0 ? zero16() : sacc[qb]);
          pacc[qb] = Tr::mma(fd[g & 1][j], vf[kc], kc == 0 ? dneg : pacc[qb]);  // dP - D
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int qb = 0; qb < BQ / 32; ++qb) {
        const f32x16 dneg = dneg_of(slot, qb);
#pragma unroll
        for (int kc = 0; kc < D / 16; ++kc) {
          const frag_t<T> aq = load_frag_swz<T, D, kBoth>(Qs, qb * 32 + col, kc * 16 + hh * 8);
          sacc[qb] = Tr::mma(aq, kf[kc], kc == 0 ? zero16() : sacc[qb]);
          const frag_t<T> ad = load_frag_swz<T, D, kBoth>(dOs, qb * 32 + col, kc * 16 + hh * 8);
          pacc[qb] = Tr::mma(ad, vf[kc], kc == 0 ? dneg : pacc[qb]);  // dP - D
        }
      }
    }
  };
  // Queries that see this lane's key: qlo <= i < qhi (the element mask).
  const int qlo = p.causal ? myk : 0;
  const int qhi = myk < kend ? N : 0;
  // In place: P = exp2(c S - LSE2) into sacc, dS = P (dP - D) into pacc.
  // On boundary tiles the mask is applied in a loop of its own behind one
  // wave-uniform branch: a mask test inside the exponential loop compiles to
  // one branch per element.
  auto soft = [&](const char* slot, int qi0, bool masked, qblk& sacc, qblk& pacc) {
    const float* lse2s = reinterpret_cast<const float*>(slot + 2 * L::TILE_BYTES);
#pragma unroll
    for (int qb = 0; qb < BQ / 32; ++qb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int r0 = qb * 32 + 8 * g + 4 * hh;  // first of 4 consecutive query rows
        const float4 l4 = *reinterpret_cast<const float4*>(lse2s + r0);
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
        for (int u = 0; u < 4; ++u)
          sacc[qb][4 * g + u] = fast_exp2(fmaf(sacc[qb][4 * g + u], c, -lv[u]));  // P
      }
    if (masked) {
#pragma unroll
      for (int qb = 0; qb < BQ / 32; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qi = qi0 + qb * 32 + acc_row(r, hh);
          sacc[qb][r] = (qi >= qlo) & (qi < qhi) ? sacc[qb][r] : 0.f;
        }
    }
#pragma unroll
    for (int qb = 0; qb < BQ / 32; ++qb)
#pragma unroll
      for (int r = 0; r < 16; ++r) pacc[qb][r] = sacc[qb][r] * pacc[qb][r];  // dS = P (dP - D)
  };
  // P and dS of a tile as B operands over the query dimension.
  typedef frag_t<T> qfrag[BQ / 16];
  auto to_frags = [&](const qblk& sacc, const qblk& pacc, qfrag& pf, qfrag& sf) {
#pragma unroll
    for (int qc = 0; qc < BQ / 16; ++qc) {
      pf[qc] = acc_to_frag<T>(sacc[qc / 2], qc % 2);
      sf[qc] = acc_to_frag<T>(pacc[qc / 2], qc % 2);
    }
  };
  // dV^T += dO^T P,  dK^T += Q^T dS  (k = queries, acc-ordered slots).
  auto grads = [&](const char* slot, const qfrag& pf, const qfrag& sf) {
    const raw* Qs = reinterpret_cast<const raw*>(slot);
    const raw* dOs = reinterpret_cast<const raw*>(slot + L::TILE_BYTES);
    if constexpr (L::PREFETCH) {
      frag_t<T> ga[2][D / 32], gq[2][D / 32];
      auto ld = [&](int qc, int b) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          ga[b][db] = load_frag_tr<T, D, kBoth>(dOs, qc * 16, db * 32, lane);
          gq[b][db] = load_frag_tr<T, D, kBoth>(Qs, qc * 16, db * 32, lane);
        }
      };
      ld(0, 0);
#pragma unroll
      for (int qc = 0; qc < BQ / 16; ++qc) {
        if (qc + 1 < BQ / 16) ld(qc + 1, (qc + 1) & 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          dv_acc[db] = Tr::mma(ga[qc & 1][db], pf[qc], dv_acc[db]);
          dk_acc[db] = Tr::mma(gq[qc & 1][db], sf[qc], dk_acc[db]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int qc = 0; qc < BQ / 16; ++qc)
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const frag_t<T> ado = load_frag_tr<T, D, kBoth>(dOs, qc * 16, db * 32, lane);
          dv_acc[db] = Tr::mma(ado, pf[qc], dv_acc[db]);
          const frag_t<T> aq = load_frag_tr<T, D, kBoth>(Qs, qc * 16, db * 32, lane);
          dk_acc[db] = Tr::mma(aq, sf[qc], dk_acc[db]);
        }
    }
  };
  auto slot_of = [&](int s) { return gring + (s & 3) * L::SLOT_BYTES; };
  // Query tile t reaches this wave's keys (under a causal mask the first
  // tiles may not; once a tile does, every later one does).
  auto active = [&](int t) { return !p.causal || kw0 <= t * BQ + BQ - 1; };
  auto masked = [&](int t) {
    const int qi0 = t * BQ;
    return (p.causal && kw0 + 31 > qi0) || (kw0 + 32 > kend) || (qi0 + BQ > N);
  };
  // The whole step (sdp, soft, to_frags, grads) with the softmax of each
  // query block placed beside independent matrix products of the same wave:
  //   score groups of block 1   + softmax of block 0 (halves 0, 1)
  //   gradient products qc 0, 1 + softmax of block 1 (halves 0, 1)
  // Half t of a block is its accumulator registers 8t .. 8t+7, which is
  // exactly the B operand pf / sf[2 qb + t] of the gradient products.
  auto step_ilv = [&](const char* slot, int qi0, bool msk) {
    static_assert(!L::ILV || (BQ == 64 && L::PREFETCH), "interleaved step: two 32-query blocks");
    const raw* Qs = reinterpret_cast<const raw*>(slot);
    const raw* dOs = reinterpret_cast<const raw*>(slot + L::TILE_BYTES);
    const float* lse2s = reinterpret_cast<const float*>(slot + 2 * L::TILE_BYTES);
    qblk sacc, pacc;
    qfrag pf, sf;
    auto soft_half = [&](int qb, int t) {
#pragma unroll
      for (int g = 2 * t; g < 2 * t + 2; ++g) {
        const int r0 = qb * 32 + 8 * g + 4 * hh;  // first of 4 consecutive query rows
        const float4 l4 = *reinterpret_cast<const float4*>(lse2s + r0);
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int r = 4 * g + u;
          float pr = fast_exp2(fmaf(sacc[qb][r], c, -lv[u]));
          if (msk) {  // selects only: no branch per element
            const int qi = qi0 + r0 + u;
            pr = (qi >= qlo) & (qi < qhi) ? pr : 0.f;
          }
          sacc[qb][r] = pr;                // P
          pacc[qb][r] = pr * pacc[qb][r];  // dS = P (dP - D)
        }
      }
      pf[2 * qb + t] = acc_to_frag<T>(sacc[qb], t);
      sf[2 * qb + t] = acc_to_frag<T>(pacc[qb], t);
    };
    constexpr int GK = L::GK, NG = D / 16 / GK, NGRP = BQ / 32 * NG;
    // Matrix products of a region (NP of them: 2 GK score products or
    // 2 D / 32 gradient products), one at a time, each followed by a share
    // of the region's vector work (a softmax half: about 36 instructions),
    // with its two LSE reads first.
    constexpr int NP = 2 * GK;
    static_assert(!L::ILV || (NG == 2 && NP == 2 * (D / 32)), "one softmax half per region");
    auto interleave = [&]() {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, (36 + NP - 1) / NP, 0);
      }
    };
    frag_t<T> fq[2][GK], fd[2][GK];
    auto ld = [&](int g, int b) {
      const int qb = g / NG, k0 = (g % NG) * GK;
#pragma unroll
      for (int j = 0; j < GK; ++j) {
        fq[b][j] = load_frag_swz<T, D, kBoth>(Qs, qb * 32 + col, (k0 + j) * 16 + hh * 8);
        fd[b][j] = load_frag_swz<T, D, kBoth>(dOs, qb * 32 + col, (k0 + j) * 16 + hh * 8);
      }
    };
    frag_t<T> ga[2][D / 32], gq[2][D / 32];
    auto gld = [&](int qc, int b) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        ga[b][db] = load_frag_tr<T, D, kBoth>(dOs, qc * 16, db * 32, lane);
        gq[b][db] = load_frag_tr<T, D, kBoth>(Qs, qc * 16, db * 32, lane);
      }
    };
    ld(0, 0);
    f32x16 dneg;
#pragma unroll
    for (int g = 0; g < NGRP; ++g) {
      const int qb = g / NG, k0 = (g % NG) * GK;
      if (k0 == 0) dneg = dneg_of(slot, qb);
      if (g + 1 < NGRP) ld(g + 1, (g + 1) & 1);
      else gld(0, 0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < GK; ++j) {
        const int kc = k0 + j;
        sacc[qb] = Tr::mma(fq[g & 1][j], kf[kc], kc == 0 ? zero16() : sacc[qb]);
        pacc[qb] = Tr::mma(fd[g & 1][j], vf[kc], kc == 0 ? dneg : pacc[qb]);  // dP - D
      }
      if (qb == 1) {
        soft_half(0, g % NG);
        interleave();
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int qc = 0; qc < BQ / 16; ++qc) {
      if (qc + 1 < BQ / 16) gld(qc + 1, (qc + 1) & 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        dv_acc[db] = Tr::mma(ga[qc & 1][db], pf[qc], dv_acc[db]);
        dk_acc[db] = Tr::mma(gq[qc & 1][db], sf[qc], dk_acc[db]);
      }
      if (qc < 2) {
        soft_half(1, qc);
        interleave();
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // QS: one query block (this wave's group) of the tile in `slot`: S and dP
  // with the K and V operands read from LDS, the softmax, then dV and dK
  // over the block's two 16-query chunks.
  auto step_qs = [&](const char* slot, int qi0, bool msk) {
    const raw* Qs = reinterpret_cast<const raw*>(slot);
    const raw* dOs = reinterpret_cast<const raw*>(slot + L::TILE_BYTES);
    const float* lse2s = reinterpret_cast<const float*>(slot + 2 * L::TILE_BYTES);
    const int qb = kgrp;
    f32x16 sacc, pacc;
    const f32x16 dneg = dneg_of(slot, qb);
#pragma unroll
    for (int kc = 0; kc < D / 16; ++kc) {
      const frag_t<T> aq = load_frag_swz<T, D, kBoth>(Qs, qb * 32 + col, kc * 16 + hh * 8);
      const frag_t<T> bk = load_frag_swz<T, D, kRows>(Kt, w * 32 + col, kc * 16 + hh * 8);
      sacc = Tr::mma(aq, bk, kc == 0 ? zero16() : sacc);
      const frag_t<T> ad = load_frag_swz<T, D, kBoth>(dOs, qb * 32 + col, kc * 16 + hh * 8);
      const frag_t<T> bv = load_frag_swz<T, D, kRows>(Vt, w * 32 + col, kc * 16 + hh * 8);
      pacc = Tr::mma(ad, bv, kc == 0 ? dneg : pacc);  // dP - D
    }
    // P = exp2(c S - LSE2) and dS = P (dP - D); boundary tiles only select
    // masked elements to 0 (one copy of the loop each, behind one
    // wave-uniform branch).
    auto soft_qs = [&](auto masked_c) {
      constexpr bool M = decltype(masked_c)::value;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int r0 = qb * 32 + 8 * g + 4 * hh;  // first of 4 consecutive query rows
        const float4 l4 = *reinterpret_cast<const float4*>(lse2s + r0);
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int r = 4 * g + u;
          float pr = fast_exp2(fmaf(sacc[r], c, -lv[u]));
          if constexpr (M) {
            const int qi = qi0 + r0 + u;
            pr = (qi >= qlo) & (qi < qhi) ? pr : 0.f;
          }
          sacc[r] = pr;            // P
          pacc[r] = pr * pacc[r];  // dS = P (dP - D)
        }
      }
    };
    if (msk) soft_qs(std::true_type{});
    else soft_qs(std::false_type{});
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const frag_t<T> pf = acc_to_frag<T>(sacc, t);
      const frag_t<T> sf = acc_to_frag<T>(pacc, t);
      const int qc = 2 * qb + t;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const frag_t<T> ado = load_frag_tr<T, D, kBoth>(dOs, qc * 16, db * 32, lane);
        dv_acc[db] = Tr::mma(ado, pf, dv_acc[db]);
        const frag_t<T> aqt = load_frag_tr<T, D, kBoth>(Qs, qc * 16, db * 32, lane);
        dk_acc[db] = Tr::mma(aqt, sf, dk_acc[db]);
      }
    }
  };

  if constexpr (QS) {
    // Both groups walk the same kept tiles [t_begin, t_end), one tile ahead
    // in the 2-slot ring: step i waits for tile i (slot i % 2; on the first
    // step also K and V), and once the barrier shows every wave done with
    // step i - 1 requests the next kept tile into the other slot.
    int t = t_begin < t_end ? next_kept(t_begin) : t_end;
    if (t < t_end) {
      issue(t, 0);
      FA_STAGE_FENCE();
      for (int step = 0;; ++step) {
        wait_vmcnt<0>();
        __syncthreads();
        const int tn = t + 1 < t_end ? next_kept(t + 1) : t_end;
        if (tn < t_end) issue(tn, (step + 1) & 1);
        FA_STAGE_FENCE();
        if (active(t)) step_qs(gring + (step & 1) * L::SLOT_BYTES, t * BQ, masked(t));
        FA_STAGE_FENCE();
        t = tn;
        if (t >= t_end) break;
      }
    }
    wait_vmcnt<0>();  // (no copy may still land in LDS once it is reused below)
  } else {
    // Kept query tiles in order; tl[k] is the tile of step i + k.  Step i
    // forms S and dP of tile i, its softmax, then the dV, dK products.
    // The split instances (long sparse masks, whose tiles come from HBM rather
    // than L2) request tiles three steps ahead, using the ring's fourth slot;
    // the others two.
    //
    // This key group's query tiles [tb, te): all of [t_begin, t_end), or its
    // first or second half (the first group takes the extra tile of an odd
    // count).  With two key groups the loop's condition is the work-group's,
    // and both groups take the first group's number of steps, so that their
    // barriers pair up; a group past its last tile only joins the barriers.
    int tb = t_begin, te = t_end;
    if constexpr (KG > 1) {
      const int tmid = t_begin + (t_end - t_begin + 1) / 2;
      tb = kgrp ? tmid : t_begin;
      te = kgrp ? t_end : tmid;
    }
    constexpr bool LA3 = SPLIT;
    int tl[4];
    tl[0] = tb < te ? next_kept(tb) : te;
    tl[1] = tl[0] < te ? next_kept(tl[0] + 1) : te;
    tl[2] = tl[1] < te ? next_kept(tl[1] + 1) : te;
    tl[3] = LA3 && tl[2] < te ? next_kept(tl[2] + 1) : te;
    if (KG > 1 ? t_begin < t_end : tl[0] < te) {
      if (tl[0] < te) issue(tl[0], 0);
      if (tl[1] < te) issue(tl[1], 1);
      if (LA3 && tl[2] < te) issue(tl[2], 2);
      FA_STAGE_FENCE();
      // The K and V fragments arrived by ordinary loads issued before these
      // copies.  Waiting for everything once here tells the compiler they have
      // landed; otherwise it waits for them (vmcnt(0)) at their first use
      // inside the loop, on every step, which also stalls on the tile just
      // requested.
      wait_vmcnt<0>();
      // Dense interior: every wave's keys see tile t in full, and tiles t+1,
      // t+2 are whole.
      int lo = te, hi = -1;
      if (!sparse && j0 + BK <= kend) {
        lo = p.causal ? (j0 + BK - 1 + BQ - 1) / BQ : tb;
        hi = min(N / BQ - 3, te - 3);
      }
      const int steps = KG > 1 ? (t_end - t_begin + 1) / 2 : 0;
      int step = 0;
      while (true) {
        const int t = tl[0];
        if (KG > 1 && t >= te) {
          __syncthreads();  // (the step's one barrier)
          FA_STAGE_FENCE();
        } else if (t >= lo && t <= hi) {
          wait_tiles(1);    // tile t landed; t+1 may be in flight
          __syncthreads();  // every wave is done with step i-1: slot (i+2)%4 is free
          const uint32_t base = ring_lds + ((step + 2) & 3) * L::SLOT_BYTES;
          const int qn = (t + 2) * BQ;
          plan.issue(Qg + (size_t)qn * D, base);
          plan.issue(dOg + (size_t)qn * D, base + L::TILE_BYTES);
          // 64 words per copy; with 32-row tiles (fp32, d = 128) lanes 32..63
          // would reach past the head, so the row is clamped as in issue().
          if (w < 2)
            dma4s((uint32_t)min(qn + lane, N - 1) * 4u,
                  w == 0 ? (const void*)lse2g : (const void*)dvecg,
                  base + 2 * L::TILE_BYTES + w * L::ROWV_BYTES);
          FA_STAGE_FENCE();
          if constexpr (L::ILV) {
            step_ilv(slot_of(step), t * BQ, false);
          } else {
            qblk sacc, pacc;
            qfrag pf, sf;
            sdp(slot_of(step), sacc, pacc);
            soft(slot_of(step), t * BQ, false, sacc, pacc);
            to_frags(sacc, pacc, pf, sf);
            grads(slot_of(step), pf, sf);
          }
          tl[0] = t + 1;
          tl[1] = t + 2;
          tl[2] = min(t + 3, te);
        } else {
          if constexpr (LA3) {
            wait_tiles((tl[1] < te) + (tl[2] < te));  // tile t landed
            __syncthreads();  // every wave is done with step i-1: slot (i+3)%4 is free
            if (tl[3] < te) issue(tl[3], (step + 3) & 3);
          } else {
            wait_tiles(tl[1] < te ? 1 : 0);  // tile t landed; tl[1] may be in flight
            __syncthreads();  // every wave is done with step i-1: slot (i+2)%4 is free
            if (tl[2] < te) issue(tl[2], (step + 2) & 3);
          }
          FA_STAGE_FENCE();
          if (active(t)) {
            if constexpr (L::ILV) {
              step_ilv(slot_of(step), t * BQ, masked(t));
            } else {
              qblk sacc, pacc;
              qfrag pf, sf;
              sdp(slot_of(step), sacc, pacc);
              soft(slot_of(step), t * BQ, masked(t), sacc, pacc);
              to_frags(sacc, pacc, pf, sf);
              grads(slot_of(step), pf, sf);
            }
          }
          tl[0] = tl[1];
          tl[1] = tl[2];
          if constexpr (LA3) {
            tl[2] = tl[3];
            tl[3] = tl[3] < te ? next_kept(tl[3] + 1) : te;
          } else {
            tl[2] = tl[2] < te ? next_kept(tl[2] + 1) : te;
          }
        }
        FA_STAGE_FENCE();
        ++step;
        if (KG > 1 ? step >= steps : tl[0] >= te) break;
      }
    }
  }

  if constexpr (KG > 1) {
    // Key group 1 adds its dK, dV accumulators into group 0's through the
    // idle rings, lane for lane; group 0 alone stores them (group 1 stays for
    // the staged store's barriers).
    constexpr int XF = 2 * (D / 32) * 16;
    static_assert(RW * XF * 64 * 4 <= (int)sizeof(ring), "hand-over fits in the rings");
    float* const xs = reinterpret_cast<float*>(ring) + w * XF * 64;
    __syncthreads();  // every wave is done with both rings
    if (kgrp == 1) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          xs[(db * 16 + r) * 64 + lane] = dk_acc[db][r];
          xs[((D / 32 + db) * 16 + r) * 64 + lane] = dv_acc[db][r];
        }
    }
    __syncthreads();
    if (kgrp == 0) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          dk_acc[db][r] += xs[(db * 16 + r) * 64 + lane];
          dv_acc[db][r] += xs[((D / 32 + db) * 16 + r) * 64 + lane];
        }
    }
  }

  if constexpr (SPLIT) {
    if (multi) {
      // One item of a long column: fp32 partials of scale * dK and dV.
      if (myk < N) {
        const size_t prow = ((size_t)item * p.BH + bh) * N + myk;
        float* const dkg = p.part_dk + prow * D;
        float* const dvg = p.part_dv + prow * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            f32x4 k4, v4;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              k4[u] = dk_acc[db][4 * g + u] * p.scale;
              v4[u] = dv_acc[db][4 * g + u];
            }
            *reinterpret_cast<f32x4*>(dkg + db * 32 + 8 * g + 4 * hh) = k4;
            *reinterpret_cast<f32x4*>(dvg + db * 32 + 8 * g + 4 * hh) = v4;
          }
      }
      return;
    }
  }
  // Store dK = scale * dK and dV.  A lane holds four consecutive d of one key
  // (key `myk`), so storing straight from the accumulators makes every
  // instruction write 16 bytes into each of 32 rows; lines that leave L2 half
  // written cost HBM a read and a write each (measured at N = 1K: 1.7x the
  // dK, dV bytes written and as much again fetched).  Each tensor goes through
  // LDS instead (the ring is idle by now), one at a time, and is stored as
  // whole rows: every store instruction writes 64 lanes x 16 bytes of
  // complete rows.  With float32 gradients requested (an option for exact
  // comparisons, not a fast path), each lane stores its fp32 values directly.
  if constexpr (GF32) {
    if (myk < N && kgrp == 0) {
      float* const dkg = reinterpret_cast<float*>(p.dk) + head + (size_t)myk * D;
      float* const dvg = reinterpret_cast<float*>(p.dv) + head + (size_t)myk * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 k4, v4;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            k4[u] = dk_acc[db][4 * g + u] * p.scale;
            v4[u] = dv_acc[db][4 * g + u];
          }
          *reinterpret_cast<f32x4*>(dkg + db * 32 + 8 * g + 4 * hh) = k4;
          *reinterpret_cast<f32x4*>(dvg + db * 32 + 8 * g + 4 * hh) = v4;
        }
    }
  } else {
    constexpr int RB = D * (int)sizeof(raw);  // bytes per row
    constexpr int RS = RB + 16;               // padded LDS row stride
    constexpr int CPR = RB / 16;              // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;             // rows per store instruction
    static_assert(RW * 32 * RS <= (int)sizeof(ring), "staging fits in the ring");
    char* const stage = ring + w * 32 * RS;
    // (with two key groups, group 0 stores; group 1 joins the barriers)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      __syncthreads();  // no wave reads the ring (or the previous tensor) any more
      if (kgrp == 0) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            raw4 r4;
#pragma unroll
            for (int u = 0; u < 4; ++u)
              r4[u] = __builtin_bit_cast(raw, t == 0 ? (T)(dk_acc[db][4 * g + u] * p.scale)
                                                     : (T)dv_acc[db][4 * g + u]);
            *reinterpret_cast<raw4*>(stage + col * RS +
                                     (db * 32 + 8 * g + 4 * hh) * (int)sizeof(raw)) = r4;
          }
      }
      __syncthreads();
      char* const out = reinterpret_cast<char*>(t == 0 ? p.dk : p.dv) + head * sizeof(raw);
#pragma unroll
      for (int r0 = 0; r0 < 32; r0 += RPI) {
        const int r = r0 + lane / CPR, c = lane % CPR;
        if (kgrp == 0 && kw0 + r < N)
          *reinterpret_cast<uint4*>(out + (size_t)(kw0 + r) * RB + c * 16) =
              *reinterpret_cast<const uint4*>(stage + r * RS + c * 16);
      }
    }
  }
}

// ----------------------------------------------------------------------------
// dQ (and D).  Work-group: 4 waves x 32 queries; key tiles of BC rows.
template <typename T, int D, int NW = 4>
struct DqCfg {
  typedef raw_t<T> raw;
  // 64 keys per step at d = 64; 32 at d = 128 (two work-groups per CU).
  static constexpr int BC = D == 128 ? 32 : 64;
  static constexpr int NS = 4;
  static constexpr int TILE_BYTES = BC * D * (int)sizeof(raw);   // one of K, V
  static constexpr int SLOT_BYTES = 2 * TILE_BYTES;
  static constexpr int LPT = 2 * TILE_BYTES / (1024 * NW);
  static constexpr int WAVES_PER_SIMD = sizeof(raw) == 4 ? 1 : 2;
  // Score/dP operand prefetch group (k-steps; 0: read each operand just
  // before its product).  One k-step ahead at 16-bit d = 128 (dQ 3.6%
  // faster at N = 16K); at d = 64 groups of 1, 2 and 4 measured 1-2% slower,
  // and groups of 4 at d = 128 spill (1.8x slower).
  static constexpr int GK = (sizeof(raw) == 2 && D == 128) ? 1 : 0;
};

// Work-group: NW waves x 32 queries (4 by default; 2 and 8 are a tile-size
// option); key tiles of BC rows.  KG = 2 (dense problems, chosen by the
// caller): the NW waves form two key groups of NW / 2 that share the query
// rows and sweep the first and second half of the key tiles, each through
// its own ring; group 1 adds its dQ accumulator into group 0's through LDS.
template <typename T, int D, bool GF32 = false, bool SPLIT = false, int NW = 4, int KG = 1>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(
    DqCfg<T, D, NW / KG>::WAVES_PER_SIMD))) void fa_bwd_dq_kernel(BwdParams p) {
  static_assert(KG == 1 || (KG == 2 && !SPLIT), "key groups: unsplit passes");
  constexpr int RW = NW / KG;  // waves per key group (32 query rows each)
  typedef raw_t<T> raw;
  typedef raw4_t<T> raw4;
  typedef Traits<T> Tr;
  typedef DqCfg<T, D, RW> L;
  constexpr int BC = L::BC;
  constexpr int BR = 32 * RW;  // queries of this work-group (at most one mask block)
  static_assert(BR <= kMaskBlock || !SPLIT, "split rows come in whole mask blocks");
  constexpr int LPT = L::LPT;

  __shared__ __attribute__((aligned(1024))) char ring[KG * L::NS * L::SLOT_BYTES];
  __shared__ uint8_t mask_row[kMaxMaskBlocks];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wg_wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kgrp = KG > 1 ? wg_wave / RW : 0;        // key group of this wave
  const int w = KG > 1 ? wg_wave % RW : wg_wave;     // row wave within the group
  char* const gring = ring + kgrp * L::NS * L::SLOT_BYTES;  // this group's ring
  const uint32_t ring_lds = lds_addr(gring);
  const int col = lane & 31;
  const int hh = lane >> 5;
  const int N = p.N;
  const int nq = (N + BR - 1) / BR;

  int qt, bh;
  map_tile(blockIdx.x, nq, p.BH, p.causal != 0, p.hgroup, qt, bh, p.causal != 0);
  if constexpr (SPLIT) {
    // an item past every kept block of this row: nothing to do
    if (blockIdx.y > 0 && (int)blockIdx.y * p.chunk_blocks >= p.split_counts[qt]) return;
  }
  const int b = bh / p.H;
  const int i0 = qt * BR;
  const int qw0 = i0 + 32 * w;
  const int myq = qw0 + col;

  int kend = N;
  if (p.key_lens) kend = min(max(p.key_lens[b], 0), N);
  int kv_end = kend;
  if (p.causal) kv_end = min(kv_end, i0 + BR);
  int nkt = kv_end > 0 ? (kv_end + BC - 1) / BC : 0;
  const bool sparse = p.block_mask != nullptr;
  if (sparse) {
    const uint8_t* bm = p.block_mask + (size_t)(i0 / kMaskBlock) * p.nblk;
    for (int i = tid; i < p.nblk; i += 64 * NW) mask_row[i] = bm[i];
  }

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
  // D = rowsum(dO * O) of this lane's query (each lane holds half of d) and
  // LSE * log2(e); both also go to the workspace for the dK/dV pass, which
  // runs after this one.  Rows without a visible key get LSE2 = +inf, so that
  // every probability recomputed for them is exp2(-inf) = 0.
  float part = 0.f, lse2 = __builtin_inff();
  if (myq < N) {
    const raw* Og = reinterpret_cast<const raw*>(p.o) + head + (size_t)myq * D;
#pragma unroll
    for (int kc = 0; kc < D / 16; ++kc) {
      const frag_t<T> of = load_frag<T>(Og + kc * 16 + hh * 8);
#pragma unroll
      for (int u = 0; u < 8; ++u) part = fmaf((float)of[u], (float)df[kc][u], part);
    }
    const float l = p.lse[(size_t)bh * N + myq];
    lse2 = l == kNegInf ? __builtin_inff() : l * kLog2e;
  }
  const float dneg = -pair_sum(part);  // -D
  if (myq < N && hh == 0 && (!SPLIT || blockIdx.y == 0) && kgrp == 0) {
    p.dvec[(size_t)bh * N + myq] = dneg;
    p.lse2[(size_t)bh * N + myq] = lse2;
  }
  f32x16 dinit;  // C operand starting each dP^T product: it delivers dP^T - D
#pragma unroll
  for (int r = 0; r < 16; ++r) dinit[r] = dneg;
  __syncthreads();  // mask_row visible

  // Split: this work-group's item of the row's kept key blocks.
  int kt_first = 0;
  bool multi = false;  // the row has more than one item: write partials
  const int item = SPLIT ? (int)blockIdx.y : 0;
  if constexpr (SPLIT) {
    const int nb = min((max(kv_end, 0) + kMaskBlock - 1) / kMaskBlock, p.nblk);
    const int total = count_kept(mask_row, 0, nb, lane);
    const int C = p.chunk_blocks;
    if (item > 0 && item * C >= total) return;  // whole work-group, no barrier pending
    multi = total > C;
    const int b0 = kth_kept(mask_row, 0, nb, item * C, lane);
    const int b1 = kth_kept(mask_row, 0, nb, (item + 1) * C, lane);
    kt_first = b0 * (kMaskBlock / BC);
    nkt = min(nkt, b1 * (kMaskBlock / BC));
  }

  auto next_kept = [&](int j) {
    if (!sparse) return j;
    while (j < nkt && mask_row[(j * BC) / kMaskBlock] == 0) ++j;
    return j;
  };

  f32x16 dq_acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) dq_acc[db] = zero16();

  DmaPlan<raw, BC, D, kBoth, RW> kplan;  // (a key group copies its own tiles)
  DmaPlan<raw, BC, D, kRows, RW> vplan;
  kplan.init(w, lane);
  vplan.init(w, lane);
  auto issue = [&](int t, int s) {
    const uint32_t base = ring_lds + s * L::SLOT_BYTES;
    kplan.copy(Kg, t * BC, N, base, lane);
    vplan.copy(Vg, t * BC, N, base + L::TILE_BYTES, lane);
  };
  auto wait_tiles = [&](int tiles) {
    if (tiles == 2) wait_vmcnt<2 * LPT>();
    else if (tiles == 1) wait_vmcnt<LPT>();
    else wait_vmcnt<0>();
  };

  const float c = p.c;
  auto step_math = [&](const char* slot, int kt0) {
    const raw* Ks = reinterpret_cast<const raw*>(slot);
    const raw* Vs = reinterpret_cast<const raw*>(slot + L::TILE_BYTES);
    f32x16 sacc[BC / 32], pacc[BC / 32];
    if constexpr (L::GK > 0) {
      // K and V operands read in groups of GK k-steps, one group ahead of
      // their products (fenced so that the compiler keeps the order).
      constexpr int GK = L::GK, NKC = D / 16, NGR = BC / 32 * NKC / GK;
      static_assert((BC / 32 * NKC) % GK == 0, "whole groups");
      frag_t<T> fk[2][GK], fv[2][GK];
      auto ld = [&](int g, int b) {
#pragma unroll
        for (int j = 0; j < GK; ++j) {
          const int i = g * GK + j, kb = i / NKC, kc = i % NKC;
          fk[b][j] = load_frag_swz<T, D, kBoth>(Ks, kb * 32 + col, kc * 16 + hh * 8);
          fv[b][j] = load_frag_swz<T, D, kRows>(Vs, kb * 32 + col, kc * 16 + hh * 8);
        }
      };
      ld(0, 0);
#pragma unroll
      for (int g = 0; g < NGR; ++g) {
        if (g + 1 < NGR) ld(g + 1, (g + 1) & 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < GK; ++j) {
          const int i = g * GK + j, kb = i / NKC, kc = i % NKC;
          sacc[kb] = Tr::mma(fk[g & 1][j], qf[kc], kc == 0 ? zero16() : sacc[kb]);
          pacc[kb] = Tr::mma(fv[g & 1][j], df[kc], kc == 0 ? dinit : pacc[kb]);
        }
        // (no fence after the last group: the exponentials may start beside it)
        if (g + 1 < NGR) __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int kb = 0; kb < BC / 32; ++kb) {
#pragma unroll
        for (int kc = 0; kc < D / 16; ++kc) {
          const frag_t<T> ak = load_frag_swz<T, D, kBoth>(Ks, kb * 32 + col, kc * 16 + hh * 8);
          sacc[kb] = Tr::mma(ak, qf[kc], kc == 0 ? zero16() : sacc[kb]);
          const frag_t<T> av = load_frag_swz<T, D, kRows>(Vs, kb * 32 + col, kc * 16 + hh * 8);
          pacc[kb] = Tr::mma(av, df[kc], kc == 0 ? dinit : pacc[kb]);
        }
      }
    }
    // P^T in place, then (tiles on a mask boundary only) the element mask in
    // a loop of its own behind one wave-uniform branch, then dS^T.  A mask
    // test inside the exponential loop compiles to one branch per element,
    // on every tile.
#pragma unroll
    for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb][r] = fast_exp2(fmaf(sacc[kb][r], c, -lse2));
    if ((p.causal && kt0 + BC - 1 > qw0) || (kt0 + BC > kend)) {
      // first key this lane's query does not see
      const int lim = p.causal ? min(kend, myq + 1) : kend;
#pragma unroll
      for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          sacc[kb][r] = kt0 + kb * 32 + acc_row(r, hh) < lim ? sacc[kb][r] : 0.f;
    }
#pragma unroll
    for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) pacc[kb][r] = sacc[kb][r] * pacc[kb][r];  // dS^T = P^T (dP^T - D)
    // dQ^T += K^T dS^T  (k = keys, acc-ordered slots).
#pragma unroll
    for (int kc = 0; kc < BC / 16; ++kc) {
      const frag_t<T> sf = acc_to_frag<T>(pacc[kc / 2], kc % 2);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const frag_t<T> a = load_frag_tr<T, D, kBoth>(Ks, kc * 16, db * 32, lane);
        dq_acc[db] = Tr::mma(a, sf, dq_acc[db]);
      }
    }
  };

  // This key group's tiles [tb, te): all of [kt_first, nkt), or its first or
  // second half (the first group takes the extra tile of an odd count).
  int tb = kt_first, te = nkt;
  if constexpr (KG > 1) {
    const int tmid = kt_first + (nkt - kt_first + 1) / 2;
    tb = kgrp ? tmid : kt_first;
    te = kgrp ? nkt : tmid;
  }
  // As in the dK/dV pass: three tiles ahead in the split instances.
  constexpr bool LA3 = SPLIT;
  int tl[4];
  tl[0] = tb < te ? next_kept(tb) : te;
  tl[1] = tl[0] < te ? next_kept(tl[0] + 1) : te;
  tl[2] = tl[1] < te ? next_kept(tl[1] + 1) : te;
  tl[3] = LA3 && tl[2] < te ? next_kept(tl[2] + 1) : te;
  // (With two key groups the condition is the work-group's, and both groups
  // take the first group's number of steps, so that their barriers pair up;
  // a group past its last tile only joins the barriers.)
  if (KG > 1 ? kt_first < nkt : tl[0] < te) {
    if (tl[0] < te) issue(tl[0], 0);
    if (tl[1] < te) issue(tl[1], 1);
    if (tl[2] < te) issue(tl[2], 2);
    if (LA3 && tl[3] < te) issue(tl[3], 3);
    FA_STAGE_FENCE();
    // As in the dK/dV pass: the Q and dO fragments came by ordinary loads;
    // wait for them here, once, rather than inside the loop.
    wait_vmcnt<0>();
    const int steps = KG > 1 ? (nkt - kt_first + 1) / 2 : 0;
    int step = 0;
    while (true) {
      if constexpr (LA3) {
        wait_tiles((tl[1] < te) + (tl[2] < te));
        __syncthreads();  // every wave is done with step i-1
        if (step > 0 && tl[3] < te) issue(tl[3], (step + 3) & 3);
      } else {
        wait_tiles((tl[1] < te) + (step == 0 && tl[2] < te));
        __syncthreads();  // every wave is done with step i-1
        if (step > 0 && tl[2] < te) issue(tl[2], (step + 2) & 3);
      }
      FA_STAGE_FENCE();
      const int kt0 = tl[0] * BC;
      if ((KG == 1 || tl[0] < te) && (!p.causal || kt0 <= qw0 + 31))
        step_math(gring + (step & 3) * L::SLOT_BYTES, kt0);
      tl[0] = tl[1];
      tl[1] = tl[2];
      if constexpr (LA3) {
        tl[2] = tl[3];
        tl[3] = tl[3] < te ? next_kept(tl[3] + 1) : te;
      } else {
        tl[2] = tl[2] < te ? next_kept(tl[2] + 1) : te;
      }
      FA_STAGE_FENCE();
      ++step;
      if (KG > 1 ? step >= steps : tl[0] >= te) break;
    }
  }
  if constexpr (KG > 1) {
    // Key group 1 adds its dQ accumulator into group 0's through the idle
    // rings, lane for lane; group 0 alone stores.
    constexpr int XF = D / 32 * 16;
    static_assert(RW * XF * 64 * 4 <= KG * L::NS * L::SLOT_BYTES, "hand-over fits in the rings");
    float* const xs = reinterpret_cast<float*>(ring) + w * XF * 64;
    __syncthreads();  // every wave is done with both rings
    if (kgrp == 1) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) xs[(db * 16 + r) * 64 + lane] = dq_acc[db][r];
    }
    __syncthreads();
    if (kgrp == 1) return;  // (no barrier follows)
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) dq_acc[db][r] += xs[(db * 16 + r) * 64 + lane];
  }

  if (SPLIT && multi) {
    // One item of a long row: fp32 partial of scale * dQ.
    if (myq < N) {
      float* const dQg = p.part_dq + (((size_t)item * p.BH + bh) * N + myq) * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 out;
#pragma unroll
          for (int u = 0; u < 4; ++u) out[u] = dq_acc[db][4 * g + u] * p.scale;
          *reinterpret_cast<f32x4*>(dQg + db * 32 + 8 * g + 4 * hh) = out;
        }
    }
  } else if constexpr (GF32) {
    if (myq < N) {
      float* const dQg = reinterpret_cast<float*>(p.dq) + head + (size_t)myq * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 out;
#pragma unroll
          for (int u = 0; u < 4; ++u) out[u] = dq_acc[db][4 * g + u] * p.scale;
          *reinterpret_cast<f32x4*>(dQg + db * 32 + 8 * g + 4 * hh) = out;
        }
    }
  } else if (myq < N) {
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

// Sums, in item order, the fp32 partials of the tiles whose mask row (dQ;
// COLS false) or column (dK and dV; COLS true) has more than chunk_blocks
// kept blocks, and writes the gradients of those tiles.  One work-group per
// 128-row tile of a head; the kept blocks are counted over the same range as
// in the pass that wrote the partials, so both agree on which tiles are split.
template <typename T, int D, bool COLS>
__global__ __launch_bounds__(256) void fa_bwd_split_reduce_kernel(BwdParams p) {
  typedef raw_t<T> raw;
  typedef raw4_t<T> raw4;
  const int N = p.N;
  const int nt = (N + 127) / 128;
  const int tile = (int)blockIdx.x % nt;
  const int bh = (int)blockIdx.x / nt;
  const int b = bh / p.H;
  int kend = N;
  if (p.key_lens) kend = min(max(p.key_lens[b], 0), N);
  const int r0 = tile * 128;
  if (p.split_counts[(COLS ? p.nblk : 0) + tile] <= p.chunk_blocks) return;  // one item at most
  int lo, hi;
  if constexpr (!COLS) {
    const int kv_end = p.causal ? min(kend, r0 + 128) : kend;
    lo = 0;
    hi = min((max(kv_end, 0) + kMaskBlock - 1) / kMaskBlock, p.nblk);
  } else {
    constexpr int BQ = DkDvCfg<T, D>::BQ;
    const int nqt = (N + BQ - 1) / BQ;
    const int t_begin = p.causal ? r0 / BQ : 0;
    const int t_end = r0 < kend ? nqt : t_begin;
    lo = (t_begin * BQ) / kMaskBlock;
    hi = min((t_end * BQ + kMaskBlock - 1) / kMaskBlock, p.nblk);
  }
  int total = 0;
  for (int base = lo; base < hi; base += 256) {
    const int i = base + (int)threadIdx.x;
    const bool kept = i < hi && (COLS ? p.mask_t : p.block_mask)[(size_t)tile * p.nblk + i] != 0;
    total += __syncthreads_count(kept);
  }
  const int C = p.chunk_blocks;
  if (total <= C) return;  // one item: its pass wrote the gradients directly
  const int items = (total + C - 1) / C;
  const int rows = min(128, N - r0);
  constexpr int V4 = D / 4;  // float4 per row
  for (int e = (int)threadIdx.x; e < rows * V4; e += 256) {
    const int r = e / V4, c4 = e - r * V4;
    const size_t row = (size_t)bh * N + r0 + r;
#pragma unroll
    for (int o = 0; o < (COLS ? 2 : 1); ++o) {
      const float* part = COLS ? (o ? p.part_dv : p.part_dk) : p.part_dq;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int s = 0; s < items; ++s)
        acc += *reinterpret_cast<const f32x4*>(part + ((size_t)s * p.BH * N + row) * D + 4 * c4);
      raw4 out;
#pragma unroll
      for (int u = 0; u < 4; ++u) out[u] = __builtin_bit_cast(raw, (T)acc[u]);
      raw* dst = reinterpret_cast<raw*>(COLS ? (o ? p.dv : p.dk) : p.dq);
      *reinterpret_cast<raw4*>(dst + row * D + 4 * c4) = out;
    }
  }
}

// SPLIT: the split instances, launched with one work-group per item
// (gridDim.y = pb.split_items), each pass followed by its reduce kernel.
// One pass with NW waves in KG key groups (32 NW / KG rows) per work-group.
template <typename T, int D, bool GF32, bool SPLIT, int NW, int KG = 1>
hipError_t launch_dq_pass(const BwdParams& p, const Problem& pb, unsigned items) {
  constexpr int BR = 32 * NW / KG;
  const unsigned tiles = (unsigned)((pb.N + BR - 1) / BR);
  hipLaunchKernelGGL((fa_bwd_dq_kernel<T, D, GF32, SPLIT, NW, KG>), dim3(tiles * p.BH, items),
                     dim3(64 * NW), 0, pb.stream, p);
  return hipGetLastError();
}
template <typename T, int D, bool GF32, bool SPLIT, int NW, int KG = 1, bool QS = false>
hipError_t launch_dkdv_pass(const BwdParams& p, const Problem& pb, unsigned items) {
  constexpr int BK = 32 * NW / KG;
  const unsigned tiles = (unsigned)((pb.N + BK - 1) / BK);
  hipLaunchKernelGGL((fa_bwd_dkdv_kernel<T, D, GF32, SPLIT, NW, KG, QS>),
                     dim3(tiles * p.BH, items), dim3(64 * NW), 0, pb.stream, p);
  return hipGetLastError();
}

template <typename T, int D, bool GF32 = false, bool SPLIT = false>
hipError_t launch_bwd_t(const Problem& pb, const BwdTensors& t) {
  static_assert(!(GF32 && SPLIT), "split backward: gradients in the input type");
  BwdParams p;
  p.q = t.q; p.k = t.k; p.v = t.v; p.o = t.o; p.dout = t.dout; p.lse = t.lse;
  p.dq = t.dq; p.dk = t.dk; p.dv = t.dv;
  const size_t rows_total = (size_t)pb.B * pb.H * pb.N;
  p.dvec = t.workspace;
  p.lse2 = t.workspace + rows_total;
  p.key_lens = pb.key_lens;
  p.block_mask = pb.block_mask;
  p.H = pb.H;
  p.N = pb.N;
  p.BH = pb.B * pb.H;
  p.nblk = (pb.N + kMaskBlock - 1) / kMaskBlock;
  // each pass streams two [N, d] operands per head (K and V, or Q and dO)
  p.hgroup = head_group(p.BH, 2LL * pb.N * pb.d * (long long)sizeof(raw_t<T>));
  p.scale = pb.scale;
  p.c = pb.scale * kLog2e;
  p.causal = pb.causal;
  p.chunk_blocks = SPLIT ? pb.chunk_blocks : 0;
  p.part_dq = pb.part_dq;
  p.part_dk = pb.part_dk;
  p.part_dv = pb.part_dv;
  p.split_counts = pb.split_counts;
  p.mask_t = pb.mask_t;

  const unsigned tiles128 = (unsigned)((pb.N + 127) / 128);
  if constexpr (SPLIT) {
    hipLaunchKernelGGL(fa_bwd_split_prep_kernel, dim3(p.nblk), dim3(256), 0, pb.stream, p);
    hipError_t e0 = hipGetLastError();
    if (e0 != hipSuccess) return e0;
  }
  const unsigned items = SPLIT ? (unsigned)pb.split_items : 1u;
  hipError_t e = hipSuccess;
  // Run-time choices among the unsplit 16-bit instances (checked by the
  // caller): two key groups (128 rows; the dK/dV pass at d = 64 splits the
  // tile range, at d = 128 each tile's queries, with K and V in LDS), or
  // other tile heights than 128 rows (gradients in the input type).
  const bool two_groups = pb.bwd_kgroups == 2;
  if (pb.bwd_passes & kPassDq) {
    if constexpr (SPLIT || sizeof(T) == 4) {
      e = launch_dq_pass<T, D, GF32, SPLIT, 4>(p, pb, items);
    } else if (two_groups) {
      e = launch_dq_pass<T, D, GF32, false, 8, 2>(p, pb, items);
    } else if (GF32 || pb.bwd_dq_rows == 128) {
      e = launch_dq_pass<T, D, GF32, false, 4>(p, pb, items);
    } else {
      e = pb.bwd_dq_rows == 64 ? launch_dq_pass<T, D, false, false, 2>(p, pb, items)
                               : launch_dq_pass<T, D, false, false, 8>(p, pb, items);
    }
    if (e != hipSuccess) return e;
    if constexpr (SPLIT) {
      hipLaunchKernelGGL((fa_bwd_split_reduce_kernel<T, D, false>), dim3(tiles128 * p.BH),
                         dim3(256), 0, pb.stream, p);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  if (pb.bwd_passes & kPassDkDv) {
    if constexpr (SPLIT || sizeof(T) == 4) {
      e = launch_dkdv_pass<T, D, GF32, SPLIT, 4>(p, pb, items);
    } else if (two_groups && D == 64) {
      if constexpr (D == 64) e = launch_dkdv_pass<T, D, GF32, false, 8, 2>(p, pb, items);
    } else if (D == 128 && pb.bwd_dkdv_qs) {
      if constexpr (D == 128) e = launch_dkdv_pass<T, D, GF32, false, 8, 2, true>(p, pb, items);
    } else if (GF32 || pb.bwd_dkdv_rows == 128) {
      e = launch_dkdv_pass<T, D, GF32, false, 4>(p, pb, items);
    } else {
      e = pb.bwd_dkdv_rows == 64 ? launch_dkdv_pass<T, D, false, false, 2>(p, pb, items)
                                 : launch_dkdv_pass<T, D, false, false, 8>(p, pb, items);
    }
    if (e != hipSuccess) return e;
    if constexpr (SPLIT) {
      hipLaunchKernelGGL((fa_bwd_split_reduce_kernel<T, D, true>), dim3(tiles128 * p.BH),
                         dim3(256), 0, pb.stream, p);
      e = hipGetLastError();
    }
  }
  return e;
}

}  // namespace
}  // namespace fa
