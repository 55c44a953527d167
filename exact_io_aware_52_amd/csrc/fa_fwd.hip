// Tiled exact attention, forward pass, for gfx950.
//
// FlashAttention forward (review page "Method"; slides steps 01-04; visual
// guide, "online softmax"): each work-group owns one tile of 128 query rows
// of one (b, h) head and streams the key/value tiles that tile needs through
// LDS.  Scores never leave the compute unit; only O and the per-row
// logsumexp are written.  The pages' pseudocode runs key/value blocks in the
// outer loop and carries per-query-block state through memory; here the
// query tile is the outer (grid) dimension so that its state (running max m,
// denominator l, fp32 accumulator) stays in registers for the whole sweep.
// Both orders give the same result in exact arithmetic.
//
// Work split: 4 waves, wave w owns queries i0 + 32w .. i0 + 32w + 31.  For a
// tile of BC keys a wave forms the transposed score tile S^T (keys x
// queries): A = K rows from LDS, B = the wave's Q rows, held in registers for
// the whole kernel.  With keys as accumulator rows each lane owns one query
// column, so the row max and row sum are in-register reductions plus one
// exchange with the lane 32 apart, and the exponentiated tile is already the
// B operand of O^T += V^T P^T (V^T is written to LDS transposed when staged).
//
// Staging: K and V tiles go from HBM straight into a 4-slot LDS ring by
// direct-to-LDS loads (no staging registers, no vector instructions); a tile
// is requested two steps before its keys are first used.  K is read as
// row-major matrix operands; V^T, the A operand of O^T += V^T P^T, is read
// from the row-major V tile with the transposing LDS read.
//
// Software pipeline: K runs one tile ahead of V.  In step i a wave issues
// the matrix products of the next tile's scores while it exponentiates the
// current tile and accumulates P V for it, so one wave always has
// independent matrix-core and vector work in flight.  One barrier per step.
//
// Online softmax with lazy rescaling: the running max m only moves (and the
// accumulator and denominator are rescaled) when a new tile's max exceeds it
// by more than 2^8 in exp2 units; otherwise probabilities are taken relative
// to the stale max (at most 256, exactly representable scale).  The result is
// the same exact softmax.
//
// Masks are decided per tile: tiles past the causal diagonal, past the key
// length or with a zero block-mask entry are skipped (never loaded); only
// tiles that straddle a boundary apply an element mask, on a slower path.

#include "fa_common.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kFwdWaves = 4;
constexpr int kFwdBR = 32 * kFwdWaves;  // query rows per work-group
constexpr int kMaskBlock = 128;         // block-mask granularity (keys and queries)
constexpr float kLazy = 8.0f;           // rescale when the max grows by > 2^8

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

constexpr int kMaxMaskBlocks = 1024;    // block-mask row cached in LDS (N <= 131072)

template <typename T, int D>
struct FwdCfg {
  typedef raw_t<T> raw;
  static constexpr int BC = D == 128 ? 32 : 64;                // keys per step
  static constexpr int NKB = BC / 32;                           // 32-key blocks per step
  static constexpr int NS = 4;                                  // LDS ring slots
  static constexpr int TILE_BYTES = BC * D * (int)sizeof(raw);  // one K or V tile
  static constexpr int SLOT_BYTES = 2 * TILE_BYTES;             // K then V
  static constexpr int LPT = 2 * TILE_BYTES / 4096;             // DMA instructions per wave per tile
  // Two waves per SIMD for 16-bit inputs; the fp32 instances (accuracy, not
  // speed) take the whole register file.
  static constexpr int WAVES_PER_SIMD = sizeof(raw) == 4 ? 1 : 2;
  // Software pipelining (next tile's scores during this tile's softmax) pays
  // at d = 64, where exponentials rival the matrix products; at d = 128 the
  // products dominate and the second score buffer would not fit 256 VGPRs.
  static constexpr bool PIPE = D == 64;
};

// Sum of the eight probabilities of a B-operand fragment, added to acc.  For
// 16-bit types the sum is taken over the rounded values the P V product uses.
__device__ __forceinline__ float frag_sum(const frag_t<__bf16>& f, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = {(__bf16)1.f, (__bf16)1.f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16x2 pr = {f[2 * i], f[2 * i + 1]};
    acc = __builtin_amdgcn_fdot2_f32_bf16(pr, one, acc, false);
  }
  return acc;
}
__device__ __forceinline__ float frag_sum(const frag_t<_Float16>& f, float acc) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  const f16x2 one = {(_Float16)1.f, (_Float16)1.f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f16x2 pr = {f[2 * i], f[2 * i + 1]};
    acc = __builtin_amdgcn_fdot2(pr, one, acc, false);
  }
  return acc;
}
__device__ __forceinline__ float frag_sum(const frag_t<float>& f, float acc) {
#pragma unroll
  for (int i = 0; i < 8; ++i) acc += f[i];
  return acc;
}

template <typename T, int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(
    FwdCfg<T, D>::WAVES_PER_SIMD))) void fa_fwd_kernel(FwdParams p) {
  typedef raw_t<T> raw;
  typedef raw4_t<T> raw4;
  typedef Traits<T> Tr;
  typedef FwdCfg<T, D> L;
  constexpr int BC = L::BC;
  constexpr int NKB = L::NKB;

  constexpr int LPT = L::LPT;
  constexpr int VSWZ = sizeof(raw) == 2 ? kTr : kRows;  // V^T via transposing reads

  __shared__ __attribute__((aligned(1024))) char ring[L::NS * L::SLOT_BYTES];
  __shared__ uint8_t mask_row[kMaxMaskBlocks];
  const uint32_t ring_lds = lds_addr(ring);
  auto ktile = [&](int s) { return reinterpret_cast<const raw*>(ring + s * L::SLOT_BYTES); };
  auto vtile = [&](int s) {
    return reinterpret_cast<const raw*>(ring + s * L::SLOT_BYTES + L::TILE_BYTES);
  };

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
  const int myq = qw0 + col;

  int kend = N;
  if (p.key_lens) kend = min(max(p.key_lens[b], 0), N);
  int kv_end = kend;
  if (p.causal) kv_end = min(kv_end, i0 + kFwdBR);
  const int nkt = kv_end > 0 ? (kv_end + BC - 1) / BC : 0;
  const bool sparse = p.block_mask != nullptr;
  if (sparse) {
    const uint8_t* bm = p.block_mask + (size_t)(i0 / kMaskBlock) * p.nblk;
    for (int i = tid; i < p.nblk; i += 256) mask_row[i] = bm[i];
  }
  auto next_kept = [&](int j) {
    if (!sparse) return j;
    while (j < nkt && mask_row[(j * BC) / kMaskBlock] == 0) ++j;
    return j;
  };
  // Tile t holds keys t*BC .. t*BC+BC-1.  A wave skips tiles wholly past its
  // causal diagonal and element-masks tiles that straddle a boundary.
  auto active = [&](int t) { return !p.causal || t * BC <= qw0 + 31; };
  auto masked = [&](int t) {
    return (p.causal && t * BC + BC - 1 > qw0) || (t * BC + BC > kend);
  };

  const size_t head = (size_t)bh * N * D;
  const raw* __restrict__ Qg = reinterpret_cast<const raw*>(p.q) + head;
  const raw* __restrict__ Kg = reinterpret_cast<const raw*>(p.k) + head;
  const raw* __restrict__ Vg = reinterpret_cast<const raw*>(p.v) + head;

  // The wave's Q rows as B operands (contiguous slot map over d).
  frag_t<T> qf[D / 16];
#pragma unroll
  for (int kc = 0; kc < D / 16; ++kc)
    qf[kc] = myq < N ? load_frag<T>(Qg + (size_t)myq * D + kc * 16 + hh * 8) : zero_frag<T>();
  __syncthreads();  // mask_row visible

  // K and V of tile t into ring slot s (LPT DMA instructions per wave).  Only
  // the ragged last tile computes clamped per-lane addresses.
  DmaPlan<raw, BC, D, kRows> kplan;
  DmaPlan<raw, BC, D, VSWZ> vplan;
  kplan.init(w, lane);
  vplan.init(w, lane);
  auto issue = [&](int t, int s) {
    const uint32_t base = ring_lds + s * L::SLOT_BYTES;
    kplan.copy(Kg, t * BC, N, base, lane);
    vplan.copy(Vg, t * BC, N, base + L::TILE_BYTES, lane);
  };

  // ---- per-wave math
  const float c = p.c;
  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = zero16();
  float m_run = kNegInf;  // running (possibly stale) max of raw scores, this lane's query
  float l_run = 0.f;      // this lane's half of the denominator, relative to m_run

  // S^T for one tile: rows = keys of the tile, columns = this wave's queries.
  auto scores = [&](const raw* Ks, f32x16 (&s)[NKB]) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) s[kb] = zero16();
#pragma unroll
    for (int kc = 0; kc < D / 16; ++kc)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const frag_t<T> a = load_frag_swz<T, D, kRows>(Ks, kb * 32 + col, kc * 16 + hh * 8);
        s[kb] = Tr::mma(a, qf[kc], s[kb]);
      }
  };
  auto apply_mask = [&](int t, f32x16 (&s)[NKB]) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = t * BC + kb * 32 + acc_row(r, hh);
        if (key >= kend || (p.causal && key > myq)) s[kb][r] = kNegInf;
      }
  };
  auto tile_max = [&](const f32x16 (&s)[NKB]) {
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    return pair_max(mx);
  };
  // Move the running max if this tile's max outruns it (wave-uniform branch).
  auto maybe_rescale = [&](float m_tile) {
    const bool need = m_tile > m_run && (m_run == kNegInf || (m_tile - m_run) * c > kLazy);
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
      const float m_new = fmaxf(m_run, m_tile);
      const float alpha = m_run == kNegInf ? 0.f : fast_exp2((m_run - m_new) * c);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    }
  };
  // P = exp2(c*s - c*m) rounded to T, as B operands; accumulates the row sum.
  auto softmax = [&](const f32x16 (&s)[NKB], frag_t<T> (&pf)[2 * NKB], bool has_mask) {
    const float mc = m_run == kNegInf ? 0.f : m_run * c;
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        frag_t<T> f;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float x = s[kb][8 * t + u];
          float e = fast_exp2(fmaf(x, c, -mc));
          if (has_mask) e = x == kNegInf ? 0.f : e;
          f[u] = (T)e;
        }
        pf[2 * kb + t] = f;
        rs = frag_sum(f, rs);
      }
    l_run += rs;
  };
  auto pv = [&](const raw* Vs, const frag_t<T> (&pf)[2 * NKB]) {
#pragma unroll
    for (int kc = 0; kc < BC / 16; ++kc)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const frag_t<T> a = load_frag_tr<T, D, VSWZ>(Vs, kc * 16, db * 32, lane);
        oacc[db] = Tr::mma(a, pf[kc], oacc[db]);
      }
  };

  // Kept tiles of this work-group, in order; tl[k] is the tile of step i + k.
  int tl[4];
  tl[0] = next_kept(0);
  tl[1] = tl[0] < nkt ? next_kept(tl[0] + 1) : nkt;
  tl[2] = tl[1] < nkt ? next_kept(tl[1] + 1) : nkt;
  tl[3] = tl[2] < nkt ? next_kept(tl[2] + 1) : nkt;
  if (tl[0] < nkt) {
    issue(tl[0], 0);
    if (tl[1] < nkt) issue(tl[1], 1);
    if (tl[2] < nkt) issue(tl[2], 2);
    // wait for tile 0 (later tiles may stay in flight)
    if (tl[2] < nkt) wait_vmcnt<2 * LPT>();
    else if (tl[1] < nkt) wait_vmcnt<LPT>();
    else wait_vmcnt<0>();
    __syncthreads();

    f32x16 sa[NKB], sb[NKB];
    float m_tile_a = kNegInf, m_tile_b = kNegInf;
    if (active(tl[0])) {
      scores(ktile(0), sa);
      if (masked(tl[0])) apply_mask(tl[0], sa);
      m_tile_a = tile_max(sa);
    }

    // Step i: tile tl[0] (scores in scur, max m_cur) is exponentiated and
    // multiplied into O; tile tl[1]'s scores go to snext.
    int step = 0;
    auto body = [&](f32x16 (&scur)[NKB], f32x16 (&snext)[NKB], float m_cur, float& m_next) {
      const int t_cur = tl[0], t_nxt = tl[1];
      if (t_nxt < nkt) {
        // tile tl[1] must have landed; tl[2] may still be in flight
        if (tl[2] < nkt) wait_vmcnt<LPT>();
        else wait_vmcnt<0>();
      }
      __syncthreads();  // every wave is done with step i-1: slot (i+3)%4 is free
      if (tl[3] < nkt) issue(tl[3], (step + 3) & 3);
      const raw* Kn = ktile((step + 1) & 3);
      const raw* Vc = vtile(step & 3);
      const bool act_cur = active(t_cur);
      const bool act_nxt = t_nxt < nkt && active(t_nxt);
      if (act_cur) maybe_rescale(m_cur);
      frag_t<T> pf[2 * NKB];
      if (act_cur && act_nxt && !masked(t_cur) && !masked(t_nxt)) {
        // interior: straight-line, next tile's products overlap this softmax
        scores(Kn, snext);
        softmax(scur, pf, false);
        pv(Vc, pf);
        m_next = tile_max(snext);
      } else {
        if (act_nxt) {
          scores(Kn, snext);
          if (masked(t_nxt)) apply_mask(t_nxt, snext);
          m_next = tile_max(snext);
        }
        if (act_cur) {
          softmax(scur, pf, masked(t_cur));
          pv(Vc, pf);
        }
      }
      tl[0] = tl[1];
      tl[1] = tl[2];
      tl[2] = tl[3];
      tl[3] = tl[3] < nkt ? next_kept(tl[3] + 1) : nkt;
      ++step;
    };
    if constexpr (L::PIPE) {
      while (true) {
        body(sa, sb, m_tile_a, m_tile_b);
        if (tl[0] >= nkt) break;
        body(sb, sa, m_tile_b, m_tile_a);
        if (tl[0] >= nkt) break;
      }
    } else {
      // Step i: scores, softmax and P V of tile tl[0] from ring slot i % 4.
      while (true) {
        const int t_cur = tl[0];
        frag_t<T> pf[2 * NKB];
        if (step > 0) {
          // tile tl[0] must have landed; tl[1] may still be in flight
          if (tl[1] < nkt) wait_vmcnt<LPT>();
          else wait_vmcnt<0>();
          __syncthreads();  // every wave is done with step i-1: slot (i+2)%4 is free
          if (tl[2] < nkt) issue(tl[2], (step + 2) & 3);
          if (active(t_cur)) {
            scores(ktile(step & 3), sa);
            if (masked(t_cur)) apply_mask(t_cur, sa);
            m_tile_a = tile_max(sa);
          }
        }
        if (active(t_cur)) {
          maybe_rescale(m_tile_a);
          softmax(sa, pf, masked(t_cur));
          pv(vtile(step & 3), pf);
        }
        tl[0] = tl[1];
        tl[1] = tl[2];
        tl[2] = tl[3];
        tl[3] = tl[3] < nkt ? next_kept(tl[3] + 1) : nkt;
        ++step;
        if (tl[0] >= nkt) break;
      }
    }
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
        for (int u = 0; u < 4; ++u) {
          const T val = (T)(oacc[db][4 * g + u] * inv);
          out[u] = __builtin_bit_cast(raw, val);
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
