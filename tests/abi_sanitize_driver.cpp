// Host-only driver for fa_api.cpp (argument validation, planning, status
// strings), built with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_abi_sanitize.py.  The kernel launchers are replaced by stubs
// that record the problem they were handed, so every path of the C ABI layer
// runs without a GPU: rejected arguments, empty problems, the tile-height
// rule, the inference split plan, the split workspace layout and a launch
// failure.  Pointers are fake and never dereferenced (the layer only checks
// them).  Exit status 0 when every check holds.

#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "fa.h"
#include "fa_internal.h"

namespace {
int g_calls = 0;
hipError_t g_result = hipSuccess;
fa::Problem g_last{};
int g_failures = 0;

void check(bool ok, const char* what, int line) {
  if (!ok) {
    std::fprintf(stderr, "FAIL line %d: %s (detail: %s)\n", line, what, fa_last_error_detail());
    ++g_failures;
  }
}
#define CHECK(x) check((x), #x, __LINE__)

void* P(uintptr_t x) { return reinterpret_cast<void*>(x); }
const uintptr_t kA = 0x10000;       // 16-byte aligned fake address
const uintptr_t kBad = 0x10002;     // misaligned
}  // namespace

namespace fa {
hipError_t launch_forward(const Problem& p, const FwdTensors&) {
  ++g_calls;
  g_last = p;
  return g_result;
}
hipError_t launch_backward(const Problem& p, const BwdTensors&) {
  ++g_calls;
  g_last = p;
  return g_result;
}
hipError_t scratch_workspace(void** ptr) {
  *ptr = reinterpret_cast<void*>(0x200000);
  return hipSuccess;
}
}  // namespace fa

extern "C" const char* hipGetErrorString(hipError_t) { return "stub launch error"; }

int main() {
  void* a = P(kA);
  float* f = static_cast<float*>(a);
  // ---- forward: rejections launch nothing
  g_calls = 0;
  CHECK(fa_forward(nullptr, a, a, a, f, 1, 1, 64, 64, 0.1f, 0, nullptr, FA_BF16, nullptr) ==
        FA_ERR_INVALID_ARG);
  CHECK(std::strstr(fa_last_error_detail(), "q is NULL") != nullptr);
  CHECK(fa_forward(P(kBad), a, a, a, f, 1, 1, 64, 64, 0.1f, 0, nullptr, FA_BF16, nullptr) ==
        FA_ERR_INVALID_ARG);
  CHECK(fa_forward(a, a, a, a, f, -1, 1, 64, 64, 0.1f, 0, nullptr, FA_BF16, nullptr) ==
        FA_ERR_INVALID_ARG);
  CHECK(fa_forward(a, a, a, a, f, 1, 1, 64, 96, 0.1f, 0, nullptr, FA_BF16, nullptr) ==
        FA_ERR_UNSUPPORTED);
  CHECK(fa_forward(a, a, a, a, f, 1, 1, 64, 64, -1.f, 0, nullptr, FA_BF16, nullptr) ==
        FA_ERR_UNSUPPORTED);
  CHECK(fa_forward(a, a, a, a, f, 1, 1, 64, 64, 1.f / 0.f, 0, nullptr, FA_BF16, nullptr) ==
        FA_ERR_INVALID_ARG);
  CHECK(fa_forward(a, a, a, a, f, 1, 1, 64, 64, 0.1f, 0, nullptr, (fa_dtype)9, nullptr) ==
        FA_ERR_INVALID_ARG);
  CHECK(fa_forward(a, a, a, a, f, 1 << 20, 1 << 12, 1 << 16, 64, 0.1f, 0, nullptr, FA_BF16,
                   nullptr) == FA_ERR_INVALID_ARG);  // grid beyond 2^31 work-groups
  CHECK(fa_forward(a, a, a, a, f, 1, 1, 64, 64, 0.1f, 0, reinterpret_cast<const int32_t*>(kA + 2),
                   FA_BF16, nullptr) == FA_ERR_INVALID_ARG);
  CHECK(fa_forward(nullptr, nullptr, nullptr, nullptr, nullptr, 0, 1, 64, 64, 0.1f, 0, nullptr,
                   FA_BF16, nullptr) == FA_OK);  // empty: nothing checked, nothing launched
  CHECK(g_calls == 0);
  // ---- forward: accepted calls and the tile-height rule
  CHECK(fa_forward(a, a, a, a, f, 2, 8, 16384, 128, 0.1f, 1, nullptr, FA_BF16, nullptr) == FA_OK);
  CHECK(g_calls == 1 && g_last.fwd_rows == 256 && g_last.splits == 1 && g_last.causal == 1);
  CHECK(fa_forward(a, a, a, a, f, 2, 8, 4096, 128, 0.1f, 1, nullptr, FA_BF16, nullptr) == FA_OK);
  CHECK(g_last.fwd_rows == 128);
  for (int rows : {64, 128, 256}) {
    CHECK(fa_forward_ex(a, a, a, a, f, 1, 2, 300, 64, 0.1f, 0, nullptr, nullptr, 128, rows, 0, 0,
                        FA_F16, nullptr) == FA_OK);
    CHECK(g_last.fwd_rows == rows && g_last.fwd_keys == 0);
  }
  CHECK(fa_forward_ex(a, a, a, a, f, 1, 2, 300, 64, 0.1f, 0, nullptr, nullptr, 128, 32, 0, 0, FA_F16,
                      nullptr) == FA_ERR_UNSUPPORTED);
  // key-tile widths: 32 and 128 with 128-row tiles (0 rows means 128); 64,
  // the 16-bit default, is no option at all
  for (int keys : {32, 64, 128}) {
    CHECK(fa_forward_ex(a, a, a, a, f, 2, 8, 16384, 128, 0.1f, 1, nullptr, nullptr, 128, 0, keys, 0,
                        FA_BF16, nullptr) == FA_OK);
    CHECK(g_last.fwd_keys == (keys == 64 ? 0 : keys) && g_last.fwd_rows == (keys == 64 ? 256 : 128));
  }
  CHECK(fa_forward_ex(a, a, a, a, f, 1, 2, 300, 64, 0.1f, 0, nullptr, nullptr, 128, 256, 128, 0,
                      FA_BF16, nullptr) == FA_ERR_UNSUPPORTED);
  CHECK(fa_forward_ex(a, a, a, a, f, 1, 2, 300, 64, 0.1f, 0, nullptr, nullptr, 128, 0, 128, 0,
                      FA_F32, nullptr) == FA_ERR_UNSUPPORTED);
  CHECK(fa_forward_ex(a, a, a, a, f, 1, 2, 300, 64, 0.1f, 0, nullptr, nullptr, 128, 0, 256, 0,
                      FA_BF16, nullptr) == FA_ERR_UNSUPPORTED);
  // key groups: automatic for small 16-bit dense grids (at most 512 tiles of 128 rows)
  CHECK(fa_forward(a, a, a, a, f, 2, 8, 4096, 64, 0.1f, 1, nullptr, FA_BF16, nullptr) == FA_OK);
  CHECK(g_last.fwd_kgroups == 2 && g_last.fwd_rows == 128);
  CHECK(fa_forward(a, a, a, a, f, 2, 8, 16384, 64, 0.1f, 1, nullptr, FA_BF16, nullptr) == FA_OK);
  CHECK(g_last.fwd_kgroups == 1 && g_last.fwd_rows == 128);
  CHECK(fa_forward(a, a, a, a, f, 2, 8, 4096, 64, 0.1f, 1, nullptr, FA_F32, nullptr) == FA_OK);
  CHECK(g_last.fwd_kgroups == 1);
  CHECK(fa_forward_ex(a, a, a, a, f, 2, 8, 4096, 64, 0.1f, 1, nullptr, nullptr, 128, 128, 0, 0,
                      FA_BF16, nullptr) == FA_OK);
  CHECK(g_last.fwd_kgroups == 1);  // an explicit height: no automatic key groups
  CHECK(fa_forward_ex(a, a, a, a, f, 2, 8, 4096, 64, 0.1f, 1, nullptr, nullptr, 128, 0, 0, 1,
                      FA_BF16, nullptr) == FA_OK);
  CHECK(g_last.fwd_kgroups == 1);
  CHECK(fa_forward_ex(a, a, a, a, f, 2, 8, 16384, 128, 0.1f, 1, nullptr, nullptr, 128, 0, 0, 2,
                      FA_F16, nullptr) == FA_OK);
  CHECK(g_last.fwd_kgroups == 2 && g_last.fwd_rows == 128);
  CHECK(fa_forward_ex(a, a, a, a, f, 2, 8, 4096, 64, 0.1f, 1, nullptr, nullptr, 128, 0, 0, 3,
                      FA_BF16, nullptr) == FA_ERR_UNSUPPORTED);
  const uint8_t* bm = static_cast<const uint8_t*>(a);
  CHECK(fa_forward_blocksparse(a, a, a, a, f, 2, 8, 4096, 64, 0.1f, 1, nullptr, bm, 128, FA_BF16,
                               nullptr) == FA_OK);
  CHECK(g_last.fwd_kgroups == 1);
  CHECK(fa_forward_ex(a, a, a, a, f, 2, 8, 4096, 64, 0.1f, 1, nullptr, bm, 128, 0, 0, 2, FA_BF16,
                      nullptr) == FA_ERR_UNSUPPORTED);
  CHECK(fa_forward_ex(a, a, a, a, f, 1, 2, 300, 64, 0.1f, 0, nullptr, bm, 128, 256, 0, 0, FA_F16,
                      nullptr) == FA_ERR_UNSUPPORTED);
  CHECK(fa_forward_ex(a, a, a, a, f, 1, 2, 300, 64, 0.1f, 0, nullptr, bm, 128, 0, 32, 0, FA_F16,
                      nullptr) == FA_OK);
  CHECK(g_last.fwd_keys == 32 && g_last.fwd_rows == 128 && g_last.block_mask == bm);
  CHECK(fa_forward_blocksparse(a, a, a, a, f, 1, 1, 300, 64, 0.1f, 0, nullptr, nullptr, 128,
                               FA_BF16, nullptr) == FA_ERR_INVALID_ARG);  // mask required
  CHECK(fa_forward_blocksparse(a, a, a, a, f, 1, 1, 300, 64, 0.1f, 0, nullptr, bm, 64, FA_BF16,
                               nullptr) == FA_ERR_UNSUPPORTED);
  CHECK(fa_forward_blocksparse(a, a, a, a, f, 1, 1, 131073, 64, 0.1f, 0, nullptr, bm, 128,
                               FA_BF16, nullptr) == FA_ERR_UNSUPPORTED);
  CHECK(fa_forward_blocksparse(a, a, a, a, f, 1, 1, 131072, 64, 0.1f, 0, nullptr, bm, 128,
                               FA_BF16, nullptr) == FA_OK);
  CHECK(g_last.block_mask == bm && g_last.fwd_rows == 128);
  // ---- split block-sparse forward: workspace layout
  const size_t wsz = fa_forward_blocksparse_split_workspace_bytes(1, 8, 65536, 64, 16384);
  CHECK(wsz == 4ull * 8 * 65536 * 64 * 4 + 4ull * 8 * 65536 * 4);
  CHECK(fa_forward_blocksparse_split_workspace_bytes(1, 8, 1000, 64, 1024) == 0);  // one split
  CHECK(fa_forward_blocksparse_split_workspace_bytes(1, 8, 1000, 64, 100) == 0);   // bad chunk
  CHECK(fa_forward_blocksparse_split(a, a, a, a, f, 1, 8, 65536, 64, 0.1f, 0, nullptr, bm, 128,
                                     16384, FA_BF16, a, wsz - 1, nullptr) == FA_ERR_WORKSPACE);
  CHECK(fa_forward_blocksparse_split(a, a, a, a, f, 1, 8, 65536, 64, 0.1f, 0, nullptr, bm, 128,
                                     16384, FA_BF16, a, wsz, nullptr) == FA_OK);
  CHECK(g_last.splits == 4 && g_last.chunk == 16384 && g_last.opart == f &&
        reinterpret_cast<char*>(g_last.lpart) == static_cast<char*>(a) + 4ull * 8 * 65536 * 64 * 4);
  CHECK(fa_forward_blocksparse_split(a, a, a, a, f, 1, 1, 65536, 64, 0.1f, 0, nullptr, bm, 128,
                                     64, FA_BF16, a, 1ull << 40, nullptr) == FA_OK);  // 1024 splits
  CHECK(fa_forward_blocksparse_split(a, a, a, a, f, 1, 1, 65600, 64, 0.1f, 0, nullptr, bm, 128,
                                     64, FA_BF16, a, 1ull << 40, nullptr) == FA_ERR_UNSUPPORTED);
  // ---- inference forward: split plan and workspace
  const size_t kvw = fa_forward_kv_workspace_bytes(16, 16, 1, 8192, 128, FA_BF16);
  CHECK(kvw > 0 && kvw % 256 == 0);
  CHECK(fa_forward_kv(a, a, a, a, f, 16, 16, 1, 8192, 128, 0.1f, 1, nullptr, FA_BF16, a, kvw,
                      nullptr) == FA_OK);
  CHECK(g_last.splits > 1 && g_last.fwd_rows == 32 && g_last.causal_br == 1 &&
        g_last.nk == 8192 && g_last.chunk % 64 == 0 &&
        (long long)g_last.splits * g_last.chunk >= 8192);
  CHECK(fa_forward_kv(a, a, a, a, f, 16, 16, 1, 8192, 128, 0.1f, 1, nullptr, FA_BF16, a, kvw - 1,
                      nullptr) == FA_ERR_WORKSPACE);
  CHECK(fa_forward_kv(a, nullptr, nullptr, a, f, 2, 2, 5, 0, 64, 0.1f, 1, nullptr, FA_BF16,
                      nullptr, 0, nullptr) == FA_OK);  // empty cache: k, v unused
  CHECK(fa_forward_kv(a, a, a, a, f, 2, 2, 5, -1, 64, 0.1f, 1, nullptr, FA_BF16, nullptr, 0,
                      nullptr) == FA_ERR_INVALID_ARG);
  // ---- packed variable-length forward
  const int32_t* cu = static_cast<const int32_t*>(a);
  CHECK(fa_forward_varlen(a, a, a, a, f, cu, cu, 16, 16, 25815, 25815, 4096, 128, 0.1f, 1,
                          FA_BF16, nullptr) == FA_OK);
  CHECK(g_last.cu_q == cu && g_last.Tq == 25815 && g_last.N == 4096 && g_last.fwd_rows == 128);
  CHECK(fa_forward_varlen(a, a, a, a, f, cu, cu, 16, 16, 100, 100, 101, 128, 0.1f, 1, FA_BF16,
                          nullptr) == FA_ERR_INVALID_ARG);
  // ---- backward and its passes
  const size_t bw = fa_backward_workspace_bytes(2, 3, 100, 64);
  CHECK(bw == 2 * 2 * 3 * 100 * 4 + 256 - (2 * 2 * 3 * 100 * 4) % 256);
  CHECK(fa_backward(a, a, a, a, a, f, a, a, a, 2, 3, 100, 64, 0.1f, 1, nullptr, nullptr, 128,
                    FA_BF16, a, bw, nullptr) == FA_OK);
  CHECK(g_last.bwd_passes == fa::kPassBoth);
  CHECK(fa_backward_dq(a, a, a, a, a, f, a, 2, 3, 100, 64, 0.1f, 1, nullptr, nullptr, 128,
                       FA_BF16, 0, a, bw, nullptr) == FA_OK);
  CHECK(g_last.bwd_passes == fa::kPassDq && g_last.bwd_dq_rows == 128);
  CHECK(fa_backward_dkdv(a, a, a, a, a, a, 2, 3, 100, 64, 0.1f, 1, nullptr, nullptr, 128,
                         FA_BF16, 0, a, bw, nullptr) == FA_OK);
  CHECK(g_last.bwd_passes == fa::kPassDkDv && g_last.bwd_dkdv_rows == 128);
  CHECK(fa_backward_dq(a, a, a, a, a, f, a, 2, 3, 100, 64, 0.1f, 1, nullptr, nullptr, 128,
                       FA_BF16, 256, a, bw, nullptr) == FA_OK);
  CHECK(g_last.bwd_dq_rows == 256 && g_last.bwd_dkdv_rows == 128);
  CHECK(fa_backward_dkdv(a, a, a, a, a, a, 2, 3, 100, 64, 0.1f, 1, nullptr, nullptr, 128,
                         FA_BF16, 64, a, bw, nullptr) == FA_OK);
  CHECK(g_last.bwd_dq_rows == 128 && g_last.bwd_dkdv_rows == 64);
  CHECK(fa_backward_dkdv(a, a, a, a, a, a, 2, 3, 100, 64, 0.1f, 1, nullptr, nullptr, 128,
                         FA_BF16, 32, a, bw, nullptr) == FA_ERR_UNSUPPORTED);
  CHECK(fa_backward(a, a, a, a, a, f, a, a, a, 2, 3, 100, 64, 0.1f, 1, nullptr, nullptr, 128,
                    FA_BF16, a, bw - 1, nullptr) == FA_ERR_WORKSPACE);
  CHECK(fa_backward(a, a, a, a, a, f, nullptr, a, a, 2, 3, 100, 64, 0.1f, 1, nullptr, nullptr,
                    128, FA_BF16, a, bw, nullptr) == FA_ERR_INVALID_ARG);
  CHECK(fa_backward_dkdv(a, a, a, a, nullptr, a, 2, 3, 100, 64, 0.1f, 1, nullptr, nullptr, 128,
                         FA_BF16, 0, a, bw, nullptr) == FA_ERR_INVALID_ARG);
  // ---- float32 gradients for 16-bit inputs
  CHECK(fa_backward_ex(a, a, a, a, a, f, a, a, a, 2, 3, 100, 64, 0.1f, 1, nullptr, nullptr, 128,
                       FA_BF16, FA_F32, 0, 0, 0, a, bw, nullptr) == FA_OK);
  CHECK(g_last.grad_f32 == 1 && g_last.bwd_passes == fa::kPassBoth);
  CHECK(g_last.bwd_dq_rows == 128 && g_last.bwd_dkdv_rows == 128);
  CHECK(fa_backward_ex(a, a, a, a, a, f, a, a, a, 2, 3, 100, 64, 0.1f, 1, nullptr, nullptr, 128,
                       FA_BF16, FA_BF16, 0, 0, 0, a, bw, nullptr) == FA_OK);
  CHECK(g_last.grad_f32 == 0);
  CHECK(fa_backward_ex(a, a, a, a, a, f, a, a, a, 2, 3, 100, 64, 0.1f, 1, nullptr, nullptr, 128,
                       FA_BF16, FA_F16, 0, 0, 0, a, bw, nullptr) == FA_ERR_INVALID_ARG);
  CHECK(fa_backward_ex(a, a, a, a, a, f, a, a, a, 2, 3, 100, 64, 0.1f, 1, nullptr, nullptr, 128,
                       FA_F32, FA_F32, 0, 0, 0, a, bw, nullptr) == FA_OK);
  CHECK(g_last.grad_f32 == 0);  // float32 inputs: float32 gradients already
  // ---- backward tile sizes: 64, 128, 256 rows per work-group of each pass
  for (int dqr : {0, 64, 128, 256})
    for (int kvr : {0, 64, 128, 256}) {
      CHECK(fa_backward_ex(a, a, a, a, a, f, a, a, a, 2, 3, 100, 64, 0.1f, 1, nullptr, nullptr,
                           128, FA_F16, FA_F16, dqr, kvr, 0, a, bw, nullptr) == FA_OK);
      CHECK(g_last.bwd_dq_rows == (dqr ? dqr : 128) && g_last.bwd_dkdv_rows == (kvr ? kvr : 128));
    }
  CHECK(fa_backward_ex(a, a, a, a, a, f, a, a, a, 2, 3, 100, 64, 0.1f, 1, nullptr, nullptr, 128,
                       FA_BF16, FA_BF16, 32, 0, 0, a, bw, nullptr) == FA_ERR_UNSUPPORTED);
  CHECK(fa_backward_ex(a, a, a, a, a, f, a, a, a, 2, 3, 100, 64, 0.1f, 1, nullptr, nullptr, 128,
                       FA_BF16, FA_BF16, 0, 512, 0, a, bw, nullptr) == FA_ERR_UNSUPPORTED);
  CHECK(fa_backward_ex(a, a, a, a, a, f, a, a, a, 2, 3, 100, 64, 0.1f, 1, nullptr, nullptr, 128,
                       FA_BF16, FA_F32, 64, 0, 0, a, bw, nullptr) == FA_ERR_UNSUPPORTED);
  CHECK(fa_backward_ex(a, a, a, a, a, f, a, a, a, 2, 3, 100, 64, 0.1f, 1, nullptr, nullptr, 128,
                       FA_F32, FA_F32, 0, 256, 0, a, bw, nullptr) == FA_ERR_UNSUPPORTED);
  CHECK(fa_backward_ex(a, a, a, a, a, f, a, a, a, 2, 3, 100, 64, 0.1f, 1, nullptr, nullptr, 128,
                       FA_F32, FA_F32, 128, 128, 0, a, bw, nullptr) == FA_OK);
  {
    const uint8_t* bmk = static_cast<const uint8_t*>(a);
    CHECK(fa_backward_ex(a, a, a, a, a, f, a, a, a, 2, 3, 100, 64, 0.1f, 1, nullptr, bmk, 128,
                         FA_BF16, FA_BF16, 64, 64, 0, a, bw, nullptr) == FA_OK);
    CHECK(fa_backward_ex(a, a, a, a, a, f, a, a, a, 2, 3, 100, 64, 0.1f, 1, nullptr, bmk, 128,
                         FA_BF16, FA_BF16, 256, 0, 0, a, bw, nullptr) == FA_ERR_UNSUPPORTED);
    CHECK(fa_backward_ex(a, a, a, a, a, f, a, a, a, 2, 3, 100, 64, 0.1f, 1, nullptr, bmk, 128,
                         FA_BF16, FA_BF16, 0, 256, 0, a, bw, nullptr) == FA_ERR_UNSUPPORTED);
  }
  // ---- backward key groups: automatic for 16-bit dense grids of at most 512 tiles
  CHECK(fa_backward(a, a, a, a, a, f, a, a, a, 2, 3, 100, 64, 0.1f, 1, nullptr, nullptr, 128,
                    FA_BF16, a, bw, nullptr) == FA_OK);
  CHECK(g_last.bwd_kgroups == 2);
  CHECK(fa_backward(a, a, a, a, a, f, a, a, a, 2, 3, 100, 64, 0.1f, 1, nullptr, nullptr, 128,
                    FA_F32, a, bw, nullptr) == FA_OK);
  CHECK(g_last.bwd_kgroups == 1);
  CHECK(fa_backward_ex(a, a, a, a, a, f, a, a, a, 2, 3, 100, 64, 0.1f, 1, nullptr, nullptr, 128,
                       FA_BF16, FA_F32, 0, 0, 0, a, bw, nullptr) == FA_OK);
  CHECK(g_last.bwd_kgroups == 2 && g_last.grad_f32 == 1);
  CHECK(fa_backward_ex(a, a, a, a, a, f, a, a, a, 2, 3, 100, 64, 0.1f, 1, nullptr, nullptr, 128,
                       FA_BF16, FA_BF16, 64, 0, 0, a, bw, nullptr) == FA_OK);
  CHECK(g_last.bwd_kgroups == 1);  // another height: one group
  CHECK(fa_backward_ex(a, a, a, a, a, f, a, a, a, 2, 3, 100, 64, 0.1f, 1, nullptr, nullptr, 128,
                       FA_BF16, FA_BF16, 0, 0, 1, a, bw, nullptr) == FA_OK);
  CHECK(g_last.bwd_kgroups == 1);
  CHECK(fa_backward_ex(a, a, a, a, a, f, a, a, a, 2, 3, 100, 64, 0.1f, 1, nullptr, nullptr, 128,
                       FA_BF16, FA_BF16, 128, 0, 2, a, bw, nullptr) == FA_OK);
  CHECK(g_last.bwd_kgroups == 2);
  CHECK(fa_backward_ex(a, a, a, a, a, f, a, a, a, 2, 3, 100, 64, 0.1f, 1, nullptr, nullptr, 128,
                       FA_F32, FA_F32, 0, 0, 2, a, bw, nullptr) == FA_ERR_UNSUPPORTED);
  {
    const uint8_t* bmk = static_cast<const uint8_t*>(a);
    CHECK(fa_backward(a, a, a, a, a, f, a, a, a, 2, 3, 100, 64, 0.1f, 1, nullptr, bmk, 128,
                      FA_BF16, a, bw, nullptr) == FA_OK);
    CHECK(g_last.bwd_kgroups == 1 && !g_last.bwd_dkdv_qs);
  }
  // ---- the d = 128 dK/dV pass splits its query tiles unless one group is asked for
  {
    const size_t bw128 = fa_backward_workspace_bytes(2, 3, 100, 128);
    const uint8_t* bmk = static_cast<const uint8_t*>(a);
    CHECK(fa_backward(a, a, a, a, a, f, a, a, a, 2, 3, 100, 128, 0.1f, 1, nullptr, nullptr, 128,
                      FA_BF16, a, bw128, nullptr) == FA_OK);
    CHECK(g_last.bwd_dkdv_qs);
    CHECK(fa_backward(a, a, a, a, a, f, a, a, a, 2, 3, 100, 128, 0.1f, 1, nullptr, bmk, 128,
                      FA_F16, a, bw128, nullptr) == FA_OK);
    CHECK(g_last.bwd_dkdv_qs);  // block masks too
    CHECK(fa_backward_ex(a, a, a, a, a, f, a, a, a, 2, 3, 100, 128, 0.1f, 1, nullptr, nullptr,
                         128, FA_BF16, FA_BF16, 0, 0, 1, a, bw128, nullptr) == FA_OK);
    CHECK(!g_last.bwd_dkdv_qs);  // one group asked for
    CHECK(fa_backward_ex(a, a, a, a, a, f, a, a, a, 2, 3, 100, 128, 0.1f, 1, nullptr, nullptr,
                         128, FA_BF16, FA_BF16, 0, 0, 2, a, bw128, nullptr) == FA_OK);
    CHECK(g_last.bwd_dkdv_qs);
    CHECK(fa_backward_ex(a, a, a, a, a, f, a, a, a, 2, 3, 100, 128, 0.1f, 1, nullptr, nullptr,
                         128, FA_BF16, FA_F32, 0, 0, 0, a, bw128, nullptr) == FA_OK);
    CHECK(g_last.bwd_dkdv_qs && g_last.grad_f32);  // float32 gradients: the same sums
    CHECK(fa_backward_ex(a, a, a, a, a, f, a, a, a, 2, 3, 100, 128, 0.1f, 1, nullptr, nullptr,
                         128, FA_BF16, FA_BF16, 0, 64, 0, a, bw128, nullptr) == FA_OK);
    CHECK(!g_last.bwd_dkdv_qs);  // another tile height
    CHECK(fa_backward(a, a, a, a, a, f, a, a, a, 2, 3, 100, 128, 0.1f, 1, nullptr, nullptr, 128,
                      FA_F32, a, bw128, nullptr) == FA_OK);
    CHECK(!g_last.bwd_dkdv_qs);
    CHECK(fa_backward(a, a, a, a, a, f, a, a, a, 2, 3, 100, 64, 0.1f, 1, nullptr, nullptr, 128,
                      FA_BF16, a, bw, nullptr) == FA_OK);
    CHECK(!g_last.bwd_dkdv_qs);  // d = 64
  }
  // (the sizes are checked before anything else is read, empty problems too)
  CHECK(fa_backward_ex(nullptr, a, a, a, a, f, a, a, a, 0, 3, 100, 64, 0.1f, 1, nullptr, nullptr,
                       128, FA_BF16, FA_BF16, 96, 0, 0, nullptr, 0, nullptr) == FA_ERR_UNSUPPORTED);
  // ---- allocation-free backward: the library's device scratch, size-limited
  const size_t max_rows = fa_backward_noalloc_max_rows();
  CHECK(max_rows == (size_t(16) << 20) / 8);
  CHECK(fa_backward_noalloc(a, a, a, a, a, f, a, a, a, 2, 8, 16384, 128, 0.1f, 1, nullptr,
                            nullptr, 128, FA_BF16, nullptr) == FA_OK);
  CHECK(g_last.bwd_passes == fa::kPassBoth);
  CHECK(fa_backward_noalloc(a, a, a, a, a, f, a, a, a, 1, 1, (int)max_rows + 256, 64, 0.1f, 1,
                            nullptr, nullptr, 128, FA_BF16, nullptr) == FA_ERR_UNSUPPORTED);
  CHECK(fa_backward_noalloc(a, a, a, a, a, f, nullptr, a, a, 2, 3, 100, 64, 0.1f, 1, nullptr,
                            nullptr, 128, FA_BF16, nullptr) == FA_ERR_INVALID_ARG);
  // ---- block-sparse backward split by kept blocks: item count and the
  // three float32 partial arrays placed after the unsplit workspace
  {
    const uint8_t* bm2 = reinterpret_cast<const uint8_t*>(a);
    const size_t base = fa_backward_workspace_bytes(1, 8, 65536, 64);
    const size_t part = 8ull * 8 * 65536 * 64 * 4;  // 512 blocks per row in items of 64: 8
    const size_t need = fa_backward_blocksparse_split_workspace_bytes(1, 8, 65536, 64, 64);
    const size_t masks = 4096 + 512ull * 512;  // int32 counts [2][512], transposed mask
    CHECK(need == base + 3 * part + masks);
    char* ws = static_cast<char*>(a);
    CHECK(fa_backward_blocksparse_split(a, a, a, a, a, f, a, a, a, 1, 8, 65536, 64, 0.1f, 0,
                                        nullptr, bm2, 128, 64, FA_BF16, ws, need,
                                        nullptr) == FA_OK);
    CHECK(g_last.chunk_blocks == 64 && g_last.split_items == 8 &&
          g_last.part_dq == reinterpret_cast<float*>(ws + base) &&
          g_last.part_dk == reinterpret_cast<float*>(ws + base + part) &&
          g_last.part_dv == reinterpret_cast<float*>(ws + base + 2 * part) &&
          g_last.split_counts == reinterpret_cast<int*>(ws + base + 3 * part) &&
          g_last.mask_t == reinterpret_cast<uint8_t*>(ws + base + 3 * part + 4096) &&
          g_last.bwd_passes == fa::kPassBoth && g_last.grad_f32 == 0);
    CHECK(fa_backward_blocksparse_split(a, a, a, a, a, f, a, a, a, 1, 8, 65536, 64, 0.1f, 0,
                                        nullptr, bm2, 128, 64, FA_BF16, ws, need - 1,
                                        nullptr) == FA_ERR_WORKSPACE);
    CHECK(fa_backward_blocksparse_split(a, a, a, a, a, f, a, a, a, 1, 8, 65536, 64, 0.1f, 0,
                                        nullptr, nullptr, 128, 64, FA_BF16, ws, need,
                                        nullptr) == FA_ERR_INVALID_ARG);
    CHECK(fa_backward_blocksparse_split(a, a, a, a, a, f, a, a, a, 1, 8, 65536, 64, 0.1f, 0,
                                        nullptr, bm2, 128, 0, FA_BF16, ws, need,
                                        nullptr) == FA_ERR_UNSUPPORTED);
    CHECK(fa_backward_blocksparse_split(a, a, a, a, a, f, a, a, a, 1, 8, 65536, 64, 0.1f, 0,
                                        nullptr, bm2, 128, 64, FA_F32, ws, need,
                                        nullptr) == FA_ERR_UNSUPPORTED);
    // a later unsplit call carries no split state
    CHECK(fa_backward(a, a, a, a, a, f, a, a, a, 2, 3, 100, 64, 0.1f, 1, nullptr, nullptr, 128,
                      FA_BF16, a, bw, nullptr) == FA_OK);
    CHECK(g_last.chunk_blocks == 0 && g_last.part_dq == nullptr);
  }
  // ---- a failed launch is reported, with its message
  g_result = hipErrorInvalidValue;
  CHECK(fa_forward(a, a, a, a, f, 1, 1, 64, 64, 0.1f, 0, nullptr, FA_BF16, nullptr) == FA_ERR_HIP);
  CHECK(std::strstr(fa_last_error_detail(), "stub launch error") != nullptr);
  CHECK(fa_backward(a, a, a, a, a, f, a, a, a, 2, 3, 100, 64, 0.1f, 1, nullptr, nullptr, 128,
                    FA_BF16, a, bw, nullptr) == FA_ERR_HIP);
  g_result = hipSuccess;
  // ---- status strings and the automatic tile height
  for (int st = -1; st < 7; ++st) CHECK(fa_status_string(st) != nullptr);
  CHECK(fa_forward_block_rows_for(2, 8, 16384, 128, FA_BF16, 0) == 256);
  CHECK(fa_forward_block_rows_for(2, 8, 16384, 128, FA_BF16, 1) == 128);
  CHECK(fa_forward_block_rows_for(2, 8, 16384, 64, FA_BF16, 0) == 128);
  if (g_failures) {
    std::fprintf(stderr, "%d check(s) failed\n", g_failures);
    return 1;
  }
  std::printf("abi sanitize driver: all checks passed\n");
  return 0;
}
