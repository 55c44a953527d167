// Tiled exact attention, forward pass, for gfx950.
//
// FlashAttention forward (review page "Method"; slides steps 01-04; visual
// guide, "online softmax"): each work-group owns one tile of 32 NW query
// rows of one (b, h) head (NW = 4 waves, 128 rows; 256 rows by default for
// large 16-bit d = 128 problems; 64 and 256 rows on request) and streams the
// key/value tiles that tile needs through
// LDS.  Scores never leave the compute unit; only O and the per-row
// logsumexp are written.  The pages' pseudocode runs key/value blocks in the
// outer loop and carries per-query-block state through memory; here the
// query tile is the outer (grid) dimension so that its state (running max m,
// denominator l, fp32 accumulator) stays in registers for the whole sweep.
// Both orders give the same result in exact arithmetic.
//
// Work split: NW waves, wave w owns queries i0 + 32w .. i0 + 32w + 31.  For
// each sub-tile of 32 keys a wave forms the transposed score tile S^T (keys x
// queries): A = K rows from LDS, B = the wave's Q rows, held in registers for
// the whole kernel.  With keys as accumulator rows each lane owns one query
// column, so row reductions are in-register plus one exchange with the lane
// 32 apart, and the exponentiated tile is already the B operand of
// O^T += V^T P^T.
//
// Staging: K and V tiles (64 keys for 16-bit types, 32 for fp32) go
// from HBM straight into an LDS ring of NS slots by direct-to-LDS loads (no
// staging registers, no vector instructions); a tile is requested NS - 1
// steps before its keys are used.  K is read as row-major matrix operands;
// V^T, the A operand of O^T += V^T P^T, is read from the row-major V tile
// with the transposing LDS read.  One barrier per ring tile.
//
// 16-bit instances keep several waves per SIMD resident (3 at d = 64, 2 at
// d = 128), which interleave matrix and vector work across waves; within a
// wave, the block of a tile's second sub-tile is ordered so that the first
// sub-tile's P V products run beside the second one's exponentials.  The
// fp32 instances (one wave per SIMD) use a software pipeline instead: K runs
// one sub-tile ahead of V, the next sub-tile's score products issuing while
// the current one is exponentiated.  Dense interior tiles (visible in full
// to every wave, whole tiles ahead) run a loop with no per-tile decisions.
//
// Online softmax with a lazy reference: each probability is
// exp2(fma(s, c, -ra)), s the fp32 score, c = scale * log2(e) and ra the
// row's reference point in exp2 units.  A sub-tile is accepted as is when
// every lane's sum of its probabilities is at most 2^8 (which bounds each
// one), so no per-tile max is taken; only otherwise, or before a row's first
// visible key, is the sub-tile max formed and the reference moved, with the
// accumulator and denominator rescaled.  Dense self-attention first tries
// an unchecked sweep with the reference fixed from each row's first 32 keys
// and falls back to the checked one only if a denominator passes 2^64 or an
// accumulator is not finite.  The result is the same exact softmax either
// way: the reference cancels in O = acc / l.  (Pre-multiplying Q by c
// would save the multiply but round c q to the input type, an error that
// grows with the size of the scores.)
//
// Masks are decided per sub-tile: tiles past the causal diagonal, past the
// key length or with a zero block-mask entry are skipped (never loaded); only
// sub-tiles that straddle a boundary apply an element mask.

#include "fa_common.h"
#include "fa_internal.h"

#include <type_traits>

namespace fa {
namespace {

constexpr int kMaskBlock = 128;         // block-mask granularity (keys and queries)

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int32_t* key_lens;
  const uint8_t* block_mask;
  int H, N, BH, nq, nblk;  // N: query rows per head; nq: query tiles per head
  int hgroup;              // heads per XCD dispatched together (map_tile)
  int snake;               // map_tile's snake order (causal grids of one round)
  int nk;                  // key (and value) rows per head: N for self-attention
  float scale;
  float c;  // scale * log2(e): exponents are taken base 2
  int causal;
  // Causal alignment: 0 = top-left (query i sees keys j <= i); 1 = bottom-right
  // to the visible key count L (query i sees keys j <= i + L - N).
  int causal_br;
  // Key range split over gridDim.y work-groups per query tile: split s covers
  // keys [s * chunk, (s + 1) * chunk) (chunk a multiple of the key tile) and
  // writes its normalised partial O (fp32) and LSE to opart / lpart at
  // [s][bh][row]; with one split (opart null) O and LSE are written directly.
  int chunk;
  float* opart;
  float* lpart;
  // Packed variable-length batch (cu_q null: the [B, H, N, d] layout):
  // sequence b owns rows cu_q[b] .. cu_q[b+1]-1 of Q and O ([H, Tq, d]) and
  // cu_k[b] .. cu_k[b+1]-1 of K and V ([H, Tk, d]); N is then the longest
  // query count, which sizes the grid.
  const int32_t* cu_q;
  const int32_t* cu_k;
  int Tq, Tk;
};

constexpr int kMaxMaskBlocks = 1024;    // block-mask row cached in LDS (N <= 131072)

// Step timeline build (FA_STEP_STAMPS, a separate library for measurement
// only): lane 0 of waves 0..3 of up to eight chosen work-groups records
// (shader clock, 100 MHz wall clock, event code) at fixed points of
// fa_fwd_kernel's sweep into a device buffer that fa_stamps_read returns.
// Codes: 1000 + query tile at the start; 5 prologue done (first tiles
// landed); interior step: 1 top, 2 tile landed, 3 past the barrier, 4 math
// done; generic step: 11 top, 12 tile landed, 13 past the barrier, 14 math
// done; 20 epilogue start, 21 end.  The stores add to the wave's count of
// memory operations in flight, so the waits for tiles are stricter there.
#ifdef FA_STEP_STAMPS
constexpr int kStampWgs = 8, kStampEvents = 340;
__device__ unsigned long long g_stamps[kStampWgs * 4][3 * kStampEvents];
__device__ int g_stamp_wgs[kStampWgs];
#endif

// NW waves per work-group, 32 query rows each (BR = 32 NW rows per tile).
// BC: keys per K/V tile, or 0 for the default width.
template <typename T, int D, int NW, int BC = 0>
struct FwdCfg {
  typedef raw_t<T> raw;
  static constexpr int BR = 32 * NW;
  static constexpr bool B16 = sizeof(raw) == 2;
  // BT keys per ring slot (one DMA tile, one barrier); the math runs on
  // 32-key sub-tiles, NSUB per slot.  By default 64 keys (16-bit) or 32
  // (fp32); the key-tile width option of the 16-bit forward also takes 32
  // and 128 (tile-size sweeps: the width sets the step count and the ring's
  // granularity, not the bytes each query tile reads).
  static constexpr int BT = BC ? BC : (B16 ? 64 : 32);
  static_assert(BT == 32 || (B16 && (BT == 64 || BT == 128)), "key tile of 32, 64 or 128 keys");
  static constexpr int NSUB = BT / 32;
  // Software pipelining across sub-tiles (a second score buffer); the 16-bit
  // instances instead keep more waves resident, which interleave matrix and
  // vector work across waves and hide the LDS latency.
  static constexpr bool PIPE = !B16;
  // Resident waves per SIMD (VGPR budget 512 / WAVES_PER_SIMD) and LDS ring
  // slots: at d = 64, 3 waves (<= 168 VGPRs) and a 3-slot ring (49 KB, three
  // work-groups per CU); at d = 128 the VGPRs allow 2 waves, and a 2-slot
  // ring of 64-key tiles (64 KB) fits two work-groups per CU.  The ring does
  // not depend on NW, so LDS caps the work-groups per CU whatever their
  // height: 64-row tiles (NW = 2) hold half the default's waves per CU (6 at
  // d = 64, 4 at d = 128), and 256-row tiles (NW = 8) one work-group, 8
  // waves, since two of them would need more VGPRs than a SIMD holds.  The
  // fp32 instances (accuracy, not speed) take the whole register file, and
  // so does the one-wave d = 128 tile (inference with few queries), which
  // would spill to fit two.
  static constexpr int WAVES_PER_SIMD = B16 ? (D == 64 ? 3 : (NW == 1 ? 1 : 2)) : 1;
  // (Other key-tile widths keep the default ring's bytes where 2 to 4 slots
  // allow it: 4 slots of 32 keys, 2 of 128.)
  static constexpr int RING_TARGET = D == 64 ? 3 * 2 * 64 * 64 * 2 : 2 * 2 * 64 * 128 * 2;
  static constexpr int NS_FIT = RING_TARGET / (2 * BT * D * (int)sizeof(raw));
  static constexpr int NS = B16 ? (NS_FIT < 2 ? 2 : (NS_FIT > 4 ? 4 : NS_FIT)) : 4;
  static constexpr int TILE_BYTES = BT * D * (int)sizeof(raw);  // one K or V tile
  static constexpr int SLOT_BYTES = 2 * TILE_BYTES;             // K then V
  static constexpr int LPT = 2 * TILE_BYTES / (1024 * NW);      // DMA instructions per wave per tile
  static_assert(!PIPE || NS == 4, "the pipelined loop uses a 4-slot ring");
};

// This lane's share of a sub-tile's row sum: sixteen probabilities, added as
// a pairwise tree of fp32 adds of the values before rounding to the input
// type.  (Summing the rounded 16-bit values with packed dot products would
// match the P V operands exactly, but on gfx950 those dot products wait for
// the matrix core whenever another wave's matrix products run on the same
// SIMD, which serialises the softmax behind them; plain fp32 adds run beside
// the matrix products.  The two sums differ by the rounding of P, the same
// order as the rounding P already carries into P V.)
__device__ __forceinline__ float sum16(const float (&e)[16]) {
  float a[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = e[2 * i] + e[2 * i + 1];
#pragma unroll
  for (int i = 0; i < 4; ++i) a[i] = a[2 * i] + a[2 * i + 1];
  return (a[0] + a[1]) + (a[2] + a[3]);
}

// One work-group's query tile (the body of the forward kernels below).
// KG key groups: with KG = 2 the NW waves form two groups of NW / 2 that
// share the tile's query rows and split its key range in halves, each group
// streaming its half through its own LDS ring; the two online-softmax states
// are merged through LDS at the end (review page, "Method": the per-block
// states combine exactly by rescaling to a common reference).  Dense
// self-attention only (the caller chooses it).
template <typename T, int D, int NW, int BC, int KG = 1>
__device__ __forceinline__ void fwd_tile(FwdParams p) {
  static_assert(KG == 1 || KG == 2, "one or two key groups");
  static_assert(KG == 1 || sizeof(raw_t<T>) == 2, "key groups: 16-bit types");
  constexpr int RW = NW / KG;  // waves per key group (32 query rows each)
  typedef raw_t<T> raw;
  typedef raw4_t<T> raw4;
  typedef Traits<T> Tr;
  typedef FwdCfg<T, D, RW, BC> L;
  constexpr int BR = L::BR;
  constexpr int BT = L::BT;
  constexpr int NSUB = L::NSUB;

  constexpr int LPT = L::LPT;
  constexpr int VSWZ = sizeof(raw) == 2 ? kTr : kRows;  // V^T via transposing reads

  __shared__ __attribute__((aligned(1024))) char ring[KG * L::NS * L::SLOT_BYTES];
  __shared__ uint8_t mask_row[kMaxMaskBlocks];
  __shared__ int wg_redo;  // unchecked sweep overflowed somewhere in the work-group
  __shared__ float ref_x[KG > 1 ? RW * 64 : 1];  // key group 0's fixed references

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wg_wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kgrp = KG > 1 ? wg_wave / RW : 0;  // key group of this wave
  const int w = KG > 1 ? wg_wave % RW : wg_wave;  // row wave within the group
  char* const gring = ring + kgrp * L::NS * L::SLOT_BYTES;  // this group's ring
  const uint32_t ring_lds = lds_addr(gring);
  auto ktile = [&](int s) { return reinterpret_cast<const raw*>(gring + s * L::SLOT_BYTES); };
  auto vtile = [&](int s) {
    return reinterpret_cast<const raw*>(gring + s * L::SLOT_BYTES + L::TILE_BYTES);
  };
  const int col = lane & 31;
  const int hh = lane >> 5;

  int qt, bh;
  map_tile(blockIdx.x, p.nq, p.BH, p.causal != 0, p.hgroup, qt, bh, p.snake != 0);
#ifdef FA_STEP_STAMPS
  int stamp_slot = -1;
  for (int i = 0; i < kStampWgs; ++i)
    if (g_stamp_wgs[i] == (int)blockIdx.x && blockIdx.y == 0) stamp_slot = i;
  int stamp_ev = 0;
  auto stamp = [&](int code) {
    __builtin_amdgcn_sched_barrier(0);
    const unsigned long long t = __builtin_readcyclecounter();
    const unsigned long long rt = __builtin_amdgcn_s_memrealtime();
    if (stamp_slot >= 0 && wg_wave < 4 && lane == 0 && stamp_ev < kStampEvents) {
      unsigned long long* rec = g_stamps[stamp_slot * 4 + wg_wave] + 3 * stamp_ev;
      rec[0] = t;
      rec[1] = rt;
      rec[2] = (unsigned long long)code;
    }
    ++stamp_ev;
    __builtin_amdgcn_sched_barrier(0);
  };
#else
  auto stamp = [](int) {};
#endif
  stamp(1000 + qt);
  const int b = bh / p.H;
  int N = p.N;    // query rows of this head
  int NK = p.nk;  // key rows
  size_t head = (size_t)bh * N * D;    // Q and O rows of this head
  size_t khead = (size_t)bh * NK * D;  // K and V rows
  size_t lrow = (size_t)bh * N;        // LSE of query row 0
  if (p.cu_q) {
    // Packed sequences: offsets clamped into the tensors, whatever cu holds.
    const int h = bh - b * p.H;
    const int q0 = min(max(p.cu_q[b], 0), p.Tq), q1 = min(max(p.cu_q[b + 1], q0), p.Tq);
    const int k0 = min(max(p.cu_k[b], 0), p.Tk), k1 = min(max(p.cu_k[b + 1], k0), p.Tk);
    N = q1 - q0;
    NK = k1 - k0;
    head = ((size_t)h * p.Tq + q0) * D;
    khead = ((size_t)h * p.Tk + k0) * D;
    lrow = (size_t)h * p.Tq + q0;
    if (qt * BR >= N) return;  // past this sequence's queries: the whole work-group, before any barrier
  }
  const int i0 = qt * BR;
  const int qw0 = i0 + 32 * w;  // first query of this wave
  const int myq = qw0 + col;

  int kend = NK;
  if (p.key_lens) kend = min(max(p.key_lens[b], 0), NK);
  // Query i sees keys j <= i + shift under the causal mask.
  const int shift = p.causal_br ? kend - N : 0;
  // This work-group's key range: [kbeg, kv_end), whole key tiles from kbeg.
  const int kbeg = blockIdx.y * p.chunk;
  int kv_end = min(kend, kbeg + p.chunk);
  if (p.causal) kv_end = min(kv_end, i0 + BR + shift);
  const int t0 = kbeg / BT;  // first key tile of the range
  const int nkt = kv_end > kbeg ? (kv_end + BT - 1) / BT : t0;
  // This key group's tiles [tbeg, tend): all of [t0, nkt), or its first or
  // second half (the first group takes the extra tile of an odd count).
  int tbeg = t0, tend = nkt;
  if constexpr (KG > 1) {
    const int tmid = t0 + (nkt - t0 + 1) / 2;
    tbeg = kgrp ? tmid : t0;
    tend = kgrp ? nkt : tmid;
  }
  const bool sparse = p.block_mask != nullptr;
  if (sparse) {
    const uint8_t* bm = p.block_mask + (size_t)(i0 / kMaskBlock) * p.nblk;
    for (int i = tid; i < p.nblk; i += 64 * NW) mask_row[i] = bm[i];
  }
  auto next_kept = [&](int j) {
    if (!sparse) return j;
    while (j < nkt && mask_row[(j * BT) / kMaskBlock] == 0) ++j;
    return j;
  };
  const raw* __restrict__ Qg = reinterpret_cast<const raw*>(p.q) + head;
  const raw* __restrict__ Kg = reinterpret_cast<const raw*>(p.k) + khead;
  const raw* __restrict__ Vg = reinterpret_cast<const raw*>(p.v) + khead;
  const float c = p.c;

  // The wave's Q rows as B operands (contiguous slot map over d).
  frag_t<T> qf[D / 16];
#pragma unroll
  for (int kc = 0; kc < D / 16; ++kc) {
    qf[kc] = myq < N ? load_frag<T>(Qg + (size_t)myq * D + kc * 16 + hh * 8) : zero_frag<T>();
  }
  __syncthreads();  // mask_row visible

  // K and V of tile t into ring slot s (LPT DMA instructions per wave).  Only
  // the ragged last tile computes clamped per-lane addresses.
  DmaPlan<raw, BT, D, kRows, RW> kplan;  // (a key group copies its own tiles)
  DmaPlan<raw, BT, D, VSWZ, RW> vplan;
  kplan.init(w, lane);
  vplan.init(w, lane);
  auto issue = [&](int t, int s) __attribute__((always_inline)) {
    const uint32_t base = ring_lds + s * L::SLOT_BYTES;
    kplan.copy(Kg, t * BT, NK, base, lane);
    vplan.copy(Vg, t * BT, NK, base + L::TILE_BYTES, lane);
  };

  // ---- per-wave math
  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = zero16();
  // Reference point of this lane's query row in exp2 units: probabilities are
  // p = exp2(c s - ra).  ra is the row max (times c) as of its last move and
  // moves only when a sub-tile's probabilities would exceed 2^8.
  float ra = 0.f;
  float l_run = 0.f;      // this lane's half of the denominator, relative to ra
  bool ref = false;       // ra is a row max (pair-uniform); before that, O = l = 0
  bool all_ref = false;   // wave-uniform: ref holds on every lane

  // Sub-tile (t, h): keys t*BT + 32h .. +31.  A wave skips sub-tiles wholly
  // past its causal diagonal and element-masks those that straddle a boundary.
  auto active = [&](int t, int h) { return !p.causal || t * BT + 32 * h <= qw0 + 31 + shift; };
  auto masked = [&](int t, int h) {
    const int k0 = t * BT + 32 * h;
    return (p.causal && k0 + 31 > qw0 + shift) || (k0 + 32 > kend);
  };
  // S^T of one sub-tile: rows = keys, columns = queries.
  auto scores = [&](const raw* Ks, int h, f32x16& s) {
#pragma unroll
    for (int kc = 0; kc < D / 16; ++kc) {
      const frag_t<T> a = load_frag_swz<T, D, kRows>(Ks, 32 * h + col, kc * 16 + hh * 8);
      s = Tr::mma(a, qf[kc], kc == 0 ? zero16() : s);
    }
  };
  auto apply_mask = [&](int t, int h, f32x16& s) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = t * BT + 32 * h + acc_row(r, hh);
      if (key >= kend || (p.causal && key > myq + shift)) s[r] = kNegInf;
    }
  };
  // P = exp2(c s - ra) rounded to T, as B operands; returns this lane's sum
  // (sum16).  Masked keys hold -inf and give 0 (selected
  // explicitly: with scale 0, c s would be NaN).
  auto expo = [&](const f32x16& s, frag_t<T> (&pf)[2], bool has_mask) {
    float e[16];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      frag_t<T> f;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float x = s[8 * h2 + u];
        float v = fast_exp2(fmaf(x, c, -ra));
        if (has_mask) v = x == kNegInf ? 0.f : v;
        e[8 * h2 + u] = v;
        f[u] = (T)v;
      }
      pf[h2] = f;
    }
    return sum16(e);
  };
  // Accept the sub-tile if every lane's probabilities are at most 2^8 (their
  // sum bounds each one) and the row has a reference; otherwise (wave-uniform
  // branch, rare) move the reference of the rows whose sub-tile max exceeds
  // it, rescale their accumulator and denominator and redo the exponentials.
  auto settle = [&](const f32x16& s, frag_t<T> (&pf)[2], float rs, bool has_mask) {
    // (The ballot is taken unconditionally so that the exponentials above
    // stay on the straight-line path.)
    const uint64_t over = __builtin_amdgcn_ballot_w64(!(rs <= 256.f));
    if (over != 0 || !all_ref) {
      float mx = kNegInf;
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
      mx = pair_max(mx);
      const float m2 = mx == kNegInf ? kNegInf : mx * c;
      const bool move = m2 != kNegInf && (!ref || m2 > ra);
      const float alpha = move && ref ? fast_exp2(ra - m2) : 1.f;
      ra = move ? m2 : ra;
      ref = ref || move;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
      rs = expo(s, pf, has_mask);
      all_ref = __builtin_amdgcn_ballot_w64(!ref) == 0;
    }
    l_run += rs;
  };
  auto pv = [&](const raw* Vs, int h, const frag_t<T> (&pf)[2]) {
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const frag_t<T> a = load_frag_tr<T, D, VSWZ>(Vs, 32 * h + kc * 16, db * 32, lane);
        oacc[db] = Tr::mma(a, pf[kc], oacc[db]);
      }
  };
  // Sub-step with both sub-tiles visible in full: the next one's products
  // overlap this one's exponentials.
  auto interior = [&](f32x16& scur, f32x16& snext, int hc, const raw* Vc, int hn,
                      const raw* Kn) {
    frag_t<T> pf[2];
    scores(Kn, hn, snext);
    const float rs = expo(scur, pf, false);
    settle(scur, pf, rs, false);
    pv(Vc, hc, pf);
  };
  // One sub-step: exponentiate sub-tile (tc, hc), whose scores are in scur,
  // and add its P V, while the products of the next sub-tile (tn, hn), if
  // any, form in snext: one wave always has independent matrix-core and
  // vector work in flight.
  auto substep = [&](f32x16& scur, f32x16& snext, int tc, int hc, const raw* Vc, int tn, int hn,
                     const raw* Kn, bool has_next) {
    const bool act_c = active(tc, hc);
    const bool act_n = has_next && active(tn, hn);
    if (act_c && act_n && !masked(tc, hc) && !masked(tn, hn)) {
      interior(scur, snext, hc, Vc, hn, Kn);
    } else {
      if (act_n) {
        scores(Kn, hn, snext);
        apply_mask(tn, hn, snext);
      }
      if (act_c) {
        frag_t<T> pf[2];
        const bool mc = masked(tc, hc);
        const float rs = expo(scur, pf, mc);
        settle(scur, pf, rs, mc);
        pv(Vc, hc, pf);
      }
    }
  };

  bool one_ref = false;  // the kept sweep was the unchecked one (one fixed reference)
  // Kept tiles of this work-group, in order; tl[k] is the tile of step i + k.
  int tl[4];
  tl[0] = next_kept(t0);
  tl[1] = tl[0] < nkt ? next_kept(tl[0] + 1) : nkt;
  tl[2] = tl[1] < nkt ? next_kept(tl[1] + 1) : nkt;
  tl[3] = tl[2] < nkt ? next_kept(tl[2] + 1) : nkt;
  if constexpr (L::PIPE) {
    if (tl[0] < nkt) {
      issue(tl[0], 0);
      if (tl[1] < nkt) issue(tl[1], 1);
      if (tl[2] < nkt) issue(tl[2], 2);
      FA_STAGE_FENCE();
      // wait for tile 0 (later tiles may stay in flight)
      if (tl[2] < nkt) wait_vmcnt<2 * LPT>();
      else if (tl[1] < nkt) wait_vmcnt<LPT>();
      else wait_vmcnt<0>();
      __syncthreads();

      f32x16 sa, sb;
      if (active(tl[0], 0)) {
        scores(ktile(0), 0, sa);
        if (masked(tl[0], 0)) apply_mask(tl[0], 0, sa);
      }

      // Step i works on the tile in ring slot i % 4: on entry its first
      // sub-tile's scores are formed; on exit, those of the next tile.
      int step = 0;
      auto body = [&](f32x16& s0, f32x16& s1) {
        if (tl[1] < nkt) {
          // tile tl[1] must have landed; tl[2] may still be in flight
          if (tl[2] < nkt) wait_vmcnt<LPT>();
          else wait_vmcnt<0>();
        }
        __syncthreads();  // every wave is done with step i-1: slot (i+3)%4 is free
        if (tl[3] < nkt) issue(tl[3], (step + 3) & 3);
        FA_STAGE_FENCE();
        const raw* Kc = ktile(step & 3);
        const raw* Kn = ktile((step + 1) & 3);
        const raw* Vc = vtile(step & 3);
        const bool more = tl[1] < nkt;
        if constexpr (NSUB == 2) {
          substep(s0, s1, tl[0], 0, Vc, tl[0], 1, Kc, true);
          substep(s1, s0, tl[0], 1, Vc, tl[1], 0, Kn, more);
        } else {
          substep(s0, s1, tl[0], 0, Vc, tl[1], 0, Kn, more);
        }
        tl[0] = tl[1];
        tl[1] = tl[2];
        tl[2] = tl[3];
        tl[3] = tl[3] < nkt ? next_kept(tl[3] + 1) : nkt;
        FA_STAGE_FENCE();
        ++step;
      };
      while (true) {
        body(sa, sb);
        if (tl[0] >= nkt) break;
        body(NSUB == 2 ? sa : sb, NSUB == 2 ? sb : sa);
        if (tl[0] >= nkt) break;
      }
    }
  } else if (KG > 1 ? t0 < nkt : tl[0] < nkt) {
    // Without the pipeline: step i forms, exponentiates and multiplies into
    // O the scores of tile i, from ring slot i % NS, with the next NS - 1
    // tiles requested ahead (several work-groups per CU hide the latency).
    //
    // Dense self-attention first takes an unchecked sweep: each row's
    // reference point is fixed at the largest score among keys 0 .. 31
    // (key 0 is visible to every row here) and no sub-tile is checked on the
    // way, so a step has no branch and the compiler interleaves its matrix and
    // vector work across both sub-tiles.  Probabilities may then exceed 1.
    // The sweep is kept if every row's denominator is at most 2^64 and every
    // accumulator is finite: no probability, product or sum has then lost
    // range.  Otherwise the work-group starts over with the checked sweep
    // (the lazy reference above), which is also the only sweep for masked,
    // split or packed problems.
    constexpr int NS = L::NS, PD = NS - 1;
    static_assert(PD >= 1 && PD <= 3, "ring of 2 to 4 slots");
    auto sweep = [&](auto checked_c) {
      constexpr bool CHECKED = decltype(checked_c)::value;
      int tl[PD + 1];
      tl[0] = next_kept(tbeg);
#pragma unroll
      for (int k = 1; k <= PD; ++k) tl[k] = tl[k - 1] < tend ? next_kept(tl[k - 1] + 1) : tend;
      // (tile indices are wave-uniform; the copies take them as scalars)
#pragma unroll
      for (int k = 0; k <= PD; ++k) tl[k] = __builtin_amdgcn_readfirstlane(tl[k]);
#pragma unroll
      for (int k = 0; k < PD; ++k)
        if (tl[k] < tend) issue(tl[k], k);
      FA_STAGE_FENCE();
      // The Q fragments arrived by ordinary loads issued before these copies.
      // Waiting for everything once here tells the compiler they have landed;
      // otherwise it waits for them (vmcnt(0)) at their first use inside the
      // loop, on every step, which also stalls on the tiles just requested.
      wait_vmcnt<0>();
      stamp(5);
      if constexpr (!CHECKED) {
        // Reference points: sub-tile 0 of tile 0, the keys each row sees
        // (in the first key group's ring; the second group takes them from
        // there through LDS).
        __syncthreads();
        if (kgrp == 0) {
          f32x16 sc;
          scores(ktile(0), 0, sc);
          apply_mask(0, 0, sc);
          float mx = kNegInf;
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[r]);
          ra = pair_max(mx) * c;
        }
        if constexpr (KG > 1) {
          if (kgrp == 0) ref_x[w * 64 + lane] = ra;
          __syncthreads();
          if (kgrp == 1) ra = ref_x[w * 64 + lane];
        }
      }
      // Per sub-tile bookkeeping: the checked sweep's settle, or the sum.
      auto take = [&](const f32x16& s, frag_t<T> (&pf)[2], float rs, bool has_mask) {
        if constexpr (CHECKED) settle(s, pf, rs, has_mask);
        else l_run += rs;
      };
      int cur = 0, nxt = PD;  // ring slots of tile i and of tile i + PD
      // One ring tile seen in full by this wave: NSUB sub-tiles, each with its
      // scores, exponentials and P V products.
      auto full_tile = [&](const raw* Kc, const raw* Vc) {
#pragma unroll
        for (int h = 0; h < NSUB; ++h) {
          f32x16 sc;
          frag_t<T> pf[2];
          scores(Kc, h, sc);
          const float rs = expo(sc, pf, false);
          if (CHECKED && h > 0) {
            // This block also holds the P V products of sub-tile h-1 (after
            // its settle branch): score reads and products first, then each
            // P V product beside a share of the exponentials.
            __builtin_amdgcn_sched_group_barrier(0x100, D / 16, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, D / 16, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 4 * D / 32, 0);
#pragma unroll
            for (int i = 0; i < 2 * D / 32; ++i) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
              __builtin_amdgcn_sched_group_barrier(0x002, 40 / (2 * D / 32), 0);
            }
          }
          take(sc, pf, rs, false);
          pv(Vc, h, pf);
        }
      };
      // Dense interior: whole tiles seen in full by every wave, tile i+PD whole.
      int lo = tend, hi = -1;
      if (!sparse) {
        lo = tbeg;
        hi = min(min(tend, NK / BT) - 1 - PD, kend / BT - 1);
        // whole tile visible to query i0: (t + 1) BT - 1 <= i0 + shift
        if (p.causal) hi = min(hi, i0 + shift + 1 >= 0 ? (i0 + shift + 1) / BT - 1 : -1);
      }
      // With two key groups both take the same number of steps (the first
      // group's tile count, the larger), so that their barriers pair up; a
      // group past its last tile only joins the barriers.
      const int steps = KG > 1 ? (nkt - t0 + 1) / 2 : 0;
      for (int iter = 0;; ++iter) {
        const int t = __builtin_amdgcn_readfirstlane(tl[0]);
        const raw* Kc = ktile(cur);
        const raw* Vc = vtile(cur);
        if (KG > 1 && t >= tend) {
          __syncthreads();  // (the step's one barrier)
          FA_STAGE_FENCE();
        } else if (t >= lo && t <= hi) {
          stamp(1);
          wait_vmcnt<(PD - 1) * LPT>();  // tile t landed; t+1 .. t+PD-1 may be in flight
          stamp(2);
          __syncthreads();               // every wave is done with step i-1: slot nxt is free
          stamp(3);
          const uint32_t nb = ring_lds + nxt * L::SLOT_BYTES;
          kplan.issue(Kg + (size_t)(t + PD) * BT * D, nb);
          vplan.issue(Vg + (size_t)(t + PD) * BT * D, nb + L::TILE_BYTES);
          FA_STAGE_FENCE();
          full_tile(Kc, Vc);
          stamp(4);
#pragma unroll
          for (int k = 0; k < PD; ++k) tl[k] = tl[k + 1];
          tl[PD] = min(t + PD + 1, tend);
        } else {
          stamp(11);
          int inflight = 0;  // later tiles requested so far (at most PD - 1)
#pragma unroll
          for (int k = 1; k < PD; ++k) inflight += tl[k] < tend;
          if constexpr (PD >= 3) {
            if (inflight >= 2) wait_vmcnt<2 * LPT>();
            else if (inflight == 1) wait_vmcnt<LPT>();
            else wait_vmcnt<0>();
          } else if constexpr (PD == 2) {
            if (inflight == 1) wait_vmcnt<LPT>();
            else wait_vmcnt<0>();
          } else {
            wait_vmcnt<0>();
          }
          stamp(12);
          __syncthreads();  // every wave is done with step i-1: slot nxt is free
          stamp(13);
          if (tl[PD] < tend) issue(tl[PD], nxt);
          FA_STAGE_FENCE();
          // A tile this wave sees in full (every sub-tile active and unmasked;
          // wave-uniform) takes the interior's interleaved order.
          bool full = true;
#pragma unroll
          for (int h = 0; h < NSUB; ++h) full = full && active(t, h) && !masked(t, h);
          if (full) {
            full_tile(Kc, Vc);
          } else {
#pragma unroll
            for (int h = 0; h < NSUB; ++h) {
              if (active(t, h)) {
                f32x16 sc;
                frag_t<T> pf[2];
                scores(Kc, h, sc);
                const bool mc = masked(t, h);
                if (mc) apply_mask(t, h, sc);
                const float rs = expo(sc, pf, mc);
                take(sc, pf, rs, mc);
                pv(Vc, h, pf);
              }
            }
          }
          stamp(14);
#pragma unroll
          for (int k = 0; k < PD; ++k) tl[k] = tl[k + 1];
          tl[PD] = __builtin_amdgcn_readfirstlane(tl[PD] < tend ? next_kept(tl[PD] + 1) : tend);
        }
        FA_STAGE_FENCE();
        cur = cur + 1 == NS ? 0 : cur + 1;
        nxt = nxt + 1 == NS ? 0 : nxt + 1;
        if (KG > 1 ? iter + 1 >= steps : tl[0] >= tend) break;
      }
    };
    // (One-wave tiles, for inference with few queries, keep only the checked
    // sweep: both would not fit its registers at d = 128.)
    bool checked = NW == 1 || sparse || p.causal_br || p.cu_q || p.opart;
    if constexpr (NW > 1) {
      if (!checked) {
        sweep(std::false_type{});
        // (with two key groups, half the bound, so that their sum stays finite)
        constexpr float kMaxAcc = KG > 1 ? 0x1p126f : 0x1p127f;
        bool bad = !(l_run <= 0x1p64f);
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) bad = bad || !(__builtin_fabsf(oacc[db][r]) <= kMaxAcc);
        // Work-group wide: every wave is done with the ring before the flag is
        // read, and any wave's overflow sends the whole work-group back.
        if (tid == 0) wg_redo = 0;
        __syncthreads();
        if (__builtin_amdgcn_ballot_w64(bad) != 0 && lane == 0) wg_redo = 1;
        __syncthreads();
        checked = __builtin_amdgcn_readfirstlane(wg_redo) != 0;
        if (checked) {
          ra = 0.f;
          l_run = 0.f;
#pragma unroll
          for (int db = 0; db < D / 32; ++db) oacc[db] = zero16();
        }
      }
    }
    if (checked) sweep(std::true_type{});
    one_ref = !checked;
  }

  if constexpr (KG > 1) {
    // Key group 1 hands its state (O accumulator, denominator, reference) to
    // group 0 through the idle ring, lane for lane; group 0 merges and alone
    // stores the tile.  Under the unchecked sweep both groups share one
    // reference point, so the states simply add; otherwise each is rescaled
    // to the larger reference.
    constexpr int XF = D / 32 * 16 + 3;
    static_assert(RW * XF * 64 * 4 <= KG * L::NS * L::SLOT_BYTES, "hand-over fits in the rings");
    float* const xs = reinterpret_cast<float*>(ring) + w * XF * 64;
    __syncthreads();  // every wave is done with both rings
    if (kgrp == 1) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) xs[(db * 16 + r) * 64 + lane] = oacc[db][r];
      xs[(XF - 3) * 64 + lane] = l_run;
      xs[(XF - 2) * 64 + lane] = ra;
      xs[(XF - 1) * 64 + lane] = ref ? 1.f : 0.f;
    }
    __syncthreads();
    if (kgrp == 1) return;  // (no barrier follows)
    const float l1 = xs[(XF - 3) * 64 + lane];
    const float ra1 = xs[(XF - 2) * 64 + lane];
    const bool ref1 = xs[(XF - 1) * 64 + lane] != 0.f;
    if (one_ref) {
      l_run += l1;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] += xs[(db * 16 + r) * 64 + lane];
    } else if (ref1) {  // (ref, ref1 are the same on both lanes of a row)
      const float r = ref ? fmaxf(ra, ra1) : ra1;
      const float f0 = ref ? fast_exp2(ra - r) : 0.f;
      const float f1 = fast_exp2(ra1 - r);
      l_run = l_run * f0 + l1 * f1;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r2 = 0; r2 < 16; ++r2)
          oacc[db][r2] = oacc[db][r2] * f0 + xs[(db * 16 + r2) * 64 + lane] * f1;
      ra = r;
      ref = true;
    }
  }

  stamp(20);
  // Epilogue: O = acc / l, LSE = ln(2^ra l) = ra ln(2) + ln(l).
  const float l_tot = pair_sum(l_run);
  if (p.opart && myq < N) {
    // One split of the key range: fp32 partial results for the combine pass.
    // A row that saw no key in this split gets LSE = -inf only: the combine
    // pass never reads the partial O of such a row.
    const size_t prow = ((size_t)blockIdx.y * p.BH + bh) * N + myq;
    if (l_tot > 0.f) {
      const float inv = 1.f / l_tot;
      float* Op = p.opart + prow * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 out;
#pragma unroll
          for (int u = 0; u < 4; ++u) out[u] = oacc[db][4 * g + u] * inv;
          *reinterpret_cast<f32x4*>(Op + db * 32 + 8 * g + 4 * hh) = out;
        }
    }
    if (hh == 0) p.lpart[prow] = l_tot > 0.f ? ra * kLn2 + __logf(l_tot) : kNegInf;
  } else if (myq < N) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    raw* Og = reinterpret_cast<raw*>(p.o) + head + (size_t)myq * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        raw4 out;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const T val = (T)(oacc[db][4 * g + u] * inv);
          out[u] = __builtin_bit_cast(raw, val);
        }
        *reinterpret_cast<raw4*>(Og + db * 32 + 8 * g + 4 * hh) = out;
      }
    if (hh == 0) {
      p.lse[lrow + myq] = l_tot > 0.f ? ra * kLn2 + __logf(l_tot) : kNegInf;
    }
  }
  stamp(21);
}

template <typename T, int D, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(
    FwdCfg<T, D, NW>::WAVES_PER_SIMD))) void fa_fwd_kernel(FwdParams p) {
  fwd_tile<T, D, NW, 0>(p);
}

// 128-row tiles with another key-tile width (16-bit types; tile-size option).
template <typename T, int D, int BC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(
    FwdCfg<T, D, 4, BC>::WAVES_PER_SIMD))) void fa_fwd_keys_kernel(FwdParams p) {
  fwd_tile<T, D, 4, BC>(p);
}

// 128-row tiles whose key range two groups of four waves split (16-bit dense
// self-attention): half the sequential steps per tile, for grids too small
// to fill the GPU, where the longest causal tiles set the kernel's time.  Two
// rings take one work-group (two waves per SIMD) per CU.
template <typename T, int D>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void
fa_fwd_kgroups_kernel(FwdParams p) {
  fwd_tile<T, D, 8, 0, 2>(p);
}

// Merge of the key-range splits of one query row (the online-softmax merge of
// per-block states, applied across work-groups): with split results (O_s,
// LSE_s), LSE = ln sum_s exp(LSE_s) and O = sum_s exp(LSE_s - LSE) O_s.  A row
// that no split saw keys for gets O = 0, LSE = -inf.  D / 4 threads per row,
// four output elements each.
struct CombineParams {
  const float* opart;
  const float* lpart;
  void* o;
  float* lse;
  int rows;    // B * H * N
  int splits;
};

template <typename T, int D>
__global__ __launch_bounds__(256) void fa_fwd_combine_kernel(CombineParams p) {
  typedef raw_t<T> raw;
  constexpr int TPR = D / 4;
  constexpr int RPB = 256 / TPR;
  const int row = blockIdx.x * RPB + (int)threadIdx.x / TPR;
  if (row >= p.rows) return;
  const int c4 = ((int)threadIdx.x % TPR) * 4;
  float m = kNegInf;
  for (int s = 0; s < p.splits; ++s) m = fmaxf(m, p.lpart[(size_t)s * p.rows + row]);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float sum = 0.f;
  if (m != kNegInf) {
    for (int s = 0; s < p.splits; ++s) {
      const float ls = p.lpart[(size_t)s * p.rows + row];
      if (ls == kNegInf) continue;
      const float wgt = expf(ls - m);
      const f32x4 os = *reinterpret_cast<const f32x4*>(p.opart + ((size_t)s * p.rows + row) * D + c4);
      sum += wgt;
      acc += wgt * os;
    }
  }
  const float inv = sum > 0.f ? 1.f / sum : 0.f;
  raw* Og = reinterpret_cast<raw*>(p.o) + (size_t)row * D + c4;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const T val = (T)(acc[u] * inv);
    Og[u] = __builtin_bit_cast(raw, val);
  }
  if (c4 == 0) p.lse[row] = sum > 0.f ? m + logf(sum) : kNegInf;
}

template <typename T, int D>
hipError_t launch_fwd_combine(const Problem& pb, const FwdTensors& t, int splits) {
  constexpr int RPB = 256 / (D / 4);
  CombineParams c;
  c.opart = pb.opart;
  c.lpart = pb.lpart;
  c.o = t.o;
  c.lse = t.lse;
  c.rows = pb.B * pb.H * pb.N;
  c.splits = splits;
  const unsigned grid = (unsigned)((c.rows + RPB - 1) / RPB);
  hipLaunchKernelGGL((fa_fwd_combine_kernel<T, D>), dim3(grid), dim3(256), 0, pb.stream, c);
  return hipGetLastError();
}

template <typename T, int D, int NW, int BC = 0, int KG = 1>
hipError_t launch_fwd_t(const Problem& pb, const FwdTensors& t) {
  constexpr int BR = FwdCfg<T, D, NW / KG, BC>::BR;
  FwdParams p;
  p.q = t.q; p.k = t.k; p.v = t.v; p.o = t.o; p.lse = t.lse;
  p.key_lens = pb.key_lens;
  p.block_mask = pb.block_mask;
  p.H = pb.H;
  p.N = pb.N;
  p.nk = pb.nk < 0 ? pb.N : pb.nk;
  p.BH = pb.B * pb.H;
  // K and V stream through every query tile of a head
  p.hgroup = head_group(p.BH, 2LL * (pb.cu_q ? (pb.Tk + pb.B - 1) / std::max(pb.B, 1) : p.nk) * D *
                                  (long long)sizeof(raw_t<T>));
  p.nq = (pb.N + BR - 1) / BR;
  // Causal grids that the chip holds in one round (three work-groups per CU
  // for this instance's ring and registers) are all resident from the start,
  // so the snake order pairs heavy and light tiles on each CU instead of
  // three of similar weight (GPT-2 shape, 768 tiles: 3.5-6.5% faster).
  p.snake = D == 64 && NW == 4 && BC == 0 && KG == 1 && pb.causal && !pb.cu_q &&
            (long long)p.nq * p.BH <= 3 * 256;
  p.nblk = (pb.N + kMaskBlock - 1) / kMaskBlock;
  p.scale = pb.scale;
  p.c = pb.scale * kLog2e;
  p.causal = pb.causal;
  p.causal_br = pb.causal_br;
  const int splits = pb.splits > 1 ? pb.splits : 1;
  p.chunk = splits > 1 ? pb.chunk : max(p.nk, 1);
  p.opart = splits > 1 ? pb.opart : nullptr;
  p.lpart = splits > 1 ? pb.lpart : nullptr;
  p.cu_q = pb.cu_q;
  p.cu_k = pb.cu_k;
  p.Tq = pb.Tq;
  p.Tk = pb.Tk;
  const unsigned grid = (unsigned)p.nq * (unsigned)p.BH;
  if constexpr (KG == 2) {
    static_assert(NW == 8 && BC == 0, "two key groups of four waves, 64-key tiles");
    hipLaunchKernelGGL((fa_fwd_kgroups_kernel<T, D>), dim3(grid, splits), dim3(512), 0, pb.stream,
                       p);
  } else if constexpr (BC != 0) {
    static_assert(NW == 4, "other key-tile widths come with 128-row tiles");
    hipLaunchKernelGGL((fa_fwd_keys_kernel<T, D, BC>), dim3(grid, splits), dim3(256), 0,
                       pb.stream, p);
  } else {
    hipLaunchKernelGGL((fa_fwd_kernel<T, D, NW>), dim3(grid, splits), dim3(64 * NW), 0,
                       pb.stream, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  return launch_fwd_combine<T, D>(pb, t, splits);
}

// Query rows per tile (work-group): 128 or 256 (chosen on the host), 64 on request;
// 32 (one wave, 16-bit types) for inference with few queries.
template <typename T, int D>
hipError_t launch_fwd_rows(const Problem& pb, const FwdTensors& t) {
  if constexpr (sizeof(T) == 2) {
    // 128-row tiles of 32 or 128 keys, or split between two key groups
    // (checked by the caller)
    if (pb.fwd_kgroups == 2) return launch_fwd_t<T, D, 8, 0, 2>(pb, t);
    if (pb.fwd_keys == 32) return launch_fwd_t<T, D, 4, 32>(pb, t);
    if (pb.fwd_keys == 128) return launch_fwd_t<T, D, 4, 128>(pb, t);
  }
  switch (pb.fwd_rows) {
    case 32:
      if constexpr (sizeof(T) == 2) return launch_fwd_t<T, D, 1>(pb, t);
      else return launch_fwd_t<T, D, 2>(pb, t);
    case 64: return launch_fwd_t<T, D, 2>(pb, t);
    case 256:
      // (float32 at d = 128 takes at most 128 rows: refused by the caller)
      if constexpr (sizeof(T) == 4 && D == 128) return hipErrorInvalidValue;
      else return launch_fwd_t<T, D, 8>(pb, t);
    default: return launch_fwd_t<T, D, 4>(pb, t);
  }
}

}  // namespace

#ifdef FA_STEP_STAMPS
// Step timeline build only (not part of the C ABI): choose the work-groups
// (blockIdx.x, up to 8; -1 unused) and clear the buffer, then read it back
// after the launches ([32][3 * 340] uint64: work-group slot * 4 + wave).
extern "C" int fa_stamps_arm(const int* wgs) {
  static unsigned long long zero[kStampWgs * 4][3 * kStampEvents];
  hipError_t e = hipMemcpyToSymbol(HIP_SYMBOL(g_stamps), zero, sizeof(zero), 0,
                                   hipMemcpyHostToDevice);
  if (e == hipSuccess)
    e = hipMemcpyToSymbol(HIP_SYMBOL(g_stamp_wgs), wgs, kStampWgs * sizeof(int), 0,
                          hipMemcpyHostToDevice);
  return (int)e;
}
extern "C" int fa_stamps_read(void* host, size_t bytes) {
  if (bytes > sizeof(g_stamps)) bytes = sizeof(g_stamps);
  return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(g_stamps), bytes, 0, hipMemcpyDeviceToHost);
}
#endif

hipError_t launch_forward(const Problem& p, const FwdTensors& t) {
  switch (p.dtype * 1000 + p.d) {
    case 0 * 1000 + 64: return launch_fwd_rows<float, 64>(p, t);
    case 0 * 1000 + 128: return launch_fwd_rows<float, 128>(p, t);
    case 1 * 1000 + 64: return launch_fwd_rows<_Float16, 64>(p, t);
    case 1 * 1000 + 128: return launch_fwd_rows<_Float16, 128>(p, t);
    case 2 * 1000 + 64: return launch_fwd_rows<__bf16, 64>(p, t);
    case 2 * 1000 + 128: return launch_fwd_rows<__bf16, 128>(p, t);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa
