// Host-side interface between the C ABI layer (fa_api.cpp) and the kernel
// launchers (fa_fwd.hip, fa_bwd.hip).  Arguments arrive here validated.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

// Backward passes a call launches (Problem::bwd_passes): the dQ pass (which
// also writes -D and LSE * log2(e) to the workspace) and the dK/dV pass that
// reads them.
enum BwdPass { kPassDq = 1, kPassDkDv = 2, kPassBoth = 3 };

struct Problem {
  int B, H, N, d;
  float scale;
  int causal;
  const int32_t* key_lens;    // device, may be null
  const uint8_t* block_mask;  // device, may be null
  int dtype;                  // fa_dtype
  hipStream_t stream;
  int fwd_rows = 128;         // forward: query rows per work-group (32, 64, 128, 256)
  int fwd_keys = 0;           // forward: keys per K/V tile (0: the type's default)
  int fwd_kgroups = 1;        // forward: wave groups splitting each tile's key range (1, 2)
  // Forward of N queries against nk keys (inference): nk < 0 means nk = N.
  int nk = -1;
  int causal_br = 0;          // causal aligned bottom-right to the visible key count
  int splits = 1;             // key-range splits per query tile
  int chunk = 0;              // keys per split (a multiple of 64)
  float* opart = nullptr;     // [splits][B*H][N][d] fp32 partial O (splits > 1)
  float* lpart = nullptr;     // [splits][B*H][N] fp32 partial LSE
  // Packed variable-length batch: Q/O [H, Tq, d], K/V [H, Tk, d], sequence b
  // at rows cu_q[b] .. and cu_k[b] ..; N is the longest query count and nk = Tk.
  const int32_t* cu_q = nullptr;
  const int32_t* cu_k = nullptr;
  int Tq = 0, Tk = 0;
  int bwd_passes = kPassBoth;  // backward: which passes to launch (BwdPass bits)
  int grad_f32 = 0;            // backward, 16-bit inputs: float32 dQ, dK, dV
  int bwd_dq_rows = 128;       // backward: query rows per dQ work-group (64, 128, 256)
  int bwd_dkdv_rows = 128;     // backward: keys per dK/dV work-group (64, 128, 256)
  int bwd_kgroups = 1;         // backward: wave groups splitting each tile's sweep (1, 2)
  // backward, d = 128: the dK/dV pass splits each query tile between two wave
  // groups (one 32-query half each, K and V in LDS)
  bool bwd_dkdv_qs = false;
  // Block-sparse backward split by kept mask blocks (chunk_blocks > 0): items
  // of chunk_blocks kept blocks per mask row (dQ) or column (dK, dV), at most
  // split_items per tile; fp32 partials [split_items][B*H][N][d] each.
  int chunk_blocks = 0;
  int split_items = 1;
  float* part_dq = nullptr;
  float* part_dk = nullptr;
  float* part_dv = nullptr;
  int* split_counts = nullptr;  // [2][ceil(N/128)] kept blocks per mask row, column
  uint8_t* mask_t = nullptr;    // [ceil(N/128)]^2 transposed block mask
};

// Heads per XCD dispatched together (map_tile's group).  The XCDs of MI355X
// each hold 4 MB of L2: when an XCD's BH / 8 heads stream more than that per
// sweep, their re-reads would miss it, so heads go two at a time (measured:
// pairs beat groups of 3 or 4 and the ungrouped order there, and lose to the
// ungrouped order when everything fits).
inline int head_group(int BH, long long streamed_bytes_per_head) {
  const int hpx = BH / 8;
  if (BH % 8 != 0 || hpx <= 2) return hpx;
  if ((long long)hpx * streamed_bytes_per_head <= (4LL << 20)) return hpx;
  return 2;
}

struct FwdTensors {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
};

struct BwdTensors {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* workspace;  // caller's workspace: -D = -rowsum(dO * O), then LSE * log2(e),
                    // each float32 [B, H, N]
};

// Device scratch of the allocation-free backward (fa_backward_noalloc): its
// size, and its address on the current device (looked up once per device;
// thread-safe).  It holds the backward workspace of any problem up to that size.
constexpr size_t kScratchBytes = size_t(16) << 20;
hipError_t scratch_workspace(void** ptr);

hipError_t launch_forward(const Problem& p, const FwdTensors& t);
hipError_t launch_backward(const Problem& p, const BwdTensors& t);

}  // namespace fa
