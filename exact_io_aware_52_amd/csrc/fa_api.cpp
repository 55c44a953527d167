// C ABI of the tiled attention library: argument validation, dispatch to the
// kernel launchers and status strings.  No state is kept between calls apart
// from the thread-local detail text of the last failure.
// Every check runs on the host before any HIP call, so a rejected call has
// launched nothing.

#include "fa.h"

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>

#include "fa_internal.h"

namespace {

thread_local char g_detail[256] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_detail, sizeof(g_detail), fmt, ap);
  va_end(ap);
  return status;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Query rows per forward work-group when the caller leaves the choice to the
// library.  256-row tiles halve the K/V bytes each query reads at L2 and, at
// 16-bit d = 128, run as fast or faster than 128 once the grid still holds
// two rounds of work-groups (one 256-row work-group fits a compute unit):
// measured N = 8K -4.3%, 16K -3.5% forward time, but N = 4K (one round)
// +14%.  Otherwise 128.
constexpr long long kAutoTallMinGroups = 2LL * 256;  // two per CU of MI355X's 256
int auto_fwd_rows(int B, int H, int N, int d, fa_dtype dtype, bool sparse) {
  if (dtype == FA_F32 || d != 128 || sparse) return 128;
  const long long groups = (long long)B * H * ((N + 255) / 256);
  return groups >= kAutoTallMinGroups ? 256 : 128;
}

// Two key groups per 128-row tile (fa_fwd_kgroups_kernel: 8 waves, one
// work-group per CU) when the default grid of 16-bit dense self-attention
// holds at most two work-groups per CU: the plain kernel then keeps no more
// waves resident than the split one, and the longest causal tiles set its
// time.  Measured forward times, key groups 2 against 1 (B2 H8, causal):
// N = 2K -10% (d = 64) and -21% (d = 128), N = 4K -4% and -13%; with more
// work-groups the split kernel's single work-group per CU costs more than
// the shorter chains save (GPT-2 shape, 768 tiles: +44%; N = 8K: +18%, +15%).
constexpr long long kAutoKgroupsMaxGroups = 2LL * 256;
int auto_fwd_kgroups(int B, int H, int N, int d, fa_dtype dtype, bool sparse) {
  if (dtype == FA_F32 || sparse || auto_fwd_rows(B, H, N, d, dtype, sparse) != 128) return 1;
  const long long groups = (long long)B * H * ((N + 127) / 128);
  return groups <= kAutoKgroupsMaxGroups ? 2 : 1;
}

// The backward's two passes: their 4-slot rings already hold them to two
// 4-wave work-groups per CU, so one 8-wave work-group per CU keeps as many
// waves and halves the chains.  Measured backward times, key groups 2
// against 1 (B2 H8, causal): N = 2K -15% (d = 64) and -8% (d = 128, measured
// with only the dQ pass split), N = 4K -4% and +1%; N = 8K +4%, +3%; the GPT-2
// shape (768 tiles) +26%.  So at most 512 tiles at d = 64, 256 at d = 128.
// (At d = 128 the dK/dV pass takes its own two-group form whatever this
// returns: see backward_impl.)
int auto_bwd_kgroups(int B, int H, int N, int d, fa_dtype dtype, bool sparse) {
  if (dtype == FA_F32 || sparse) return 1;
  const long long groups = (long long)B * H * ((N + 127) / 128);
  return groups <= (d == 64 ? kAutoKgroupsMaxGroups : kAutoKgroupsMaxGroups / 2) ? 2 : 1;
}

}  // namespace

namespace {

int check_common(int B, int H, int N, int d, float scale, fa_dtype dtype, bool* empty) {
  if (B < 0 || H < 0 || N < 0)
    return fail(FA_ERR_INVALID_ARG, "negative size B=%d H=%d N=%d", B, H, N);
  *empty = (B == 0 || H == 0 || N == 0);
  if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16)
    return fail(FA_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "head dim d=%d (supported: 64, 128)", d);
  if (!std::isfinite(scale)) return fail(FA_ERR_INVALID_ARG, "scale is not finite");
  if (scale < 0.f) return fail(FA_ERR_UNSUPPORTED, "negative scale %g", (double)scale);
  if (*empty) return FA_OK;
  // One work-group per 64, 128 or 256 query rows (forward) or 128 keys
  // (backward) per head; the bound is taken for the smallest tile.
  const long long tiles = ((long long)N + 63) / 64;
  if ((long long)B * H * tiles > 0x7fffffffLL)
    return fail(FA_ERR_INVALID_ARG, "problem too large: B*H*ceil(N/64) exceeds 2^31-1");
  if ((long long)N * d > 0x7fffffffLL) return fail(FA_ERR_INVALID_ARG, "N*d exceeds 2^31-1");
  return FA_OK;
}

int check_tensor(const void* p, const char* name, size_t align) {
  if (!p) return fail(FA_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned(p, align)) return fail(FA_ERR_INVALID_ARG, "%s is not %zu-byte aligned", name, align);
  return FA_OK;
}

// Kernels cache one row of the block mask in LDS: at most 1024 blocks.
constexpr int kMaxMaskBlocks = 1024;

int check_block(const uint8_t* block_mask, int block_size, int N, bool required) {
  if (!block_mask) {
    if (required) return fail(FA_ERR_INVALID_ARG, "block_mask is NULL");
    return FA_OK;
  }
  if (block_size != 128)
    return fail(FA_ERR_UNSUPPORTED, "block_size=%d (supported: 128)", block_size);
  if ((N + 127) / 128 > kMaxMaskBlocks)
    return fail(FA_ERR_UNSUPPORTED, "block mask for N=%d exceeds %d blocks per row", N,
                kMaxMaskBlocks);
  return FA_OK;
}

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Key-range splits of the block-sparse forward with key_chunk keys each, and
// the workspace their fp32 partial O and LSE take ([splits][B*H][N][d], then
// [splits][B*H][N], each rounded up to 256 bytes).
constexpr int kMaxSplits = 1024;
int sparse_splits(int N, int key_chunk) { return (N + key_chunk - 1) / key_chunk; }
size_t split_workspace(int B, int H, int N, int d, int splits) {
  if (splits <= 1) return 0;
  const size_t rows = (size_t)splits * B * H * N;
  return round_up(rows * d * sizeof(float), 256) + round_up(rows * sizeof(float), 256);
}

// Block-sparse backward split: items per mask row or column, and the bytes of
// one float32 partial array [items][B*H][N][d] (rounded up to 256 bytes).
int bwd_split_items(int N, int chunk_blocks) {
  const int nblk = (N + 127) / 128;
  return (nblk + chunk_blocks - 1) / chunk_blocks;
}
size_t bwd_split_part_bytes(int B, int H, int N, int d, int chunk_blocks) {
  return round_up((size_t)bwd_split_items(N, chunk_blocks) * B * H * N * d * sizeof(float), 256);
}
// Kept-block counts per mask row and column (int32 [2][nblk]), then the
// transposed mask ([nblk][nblk] bytes), each rounded up to 256 bytes.
size_t bwd_split_mask_bytes(int N) {
  const size_t nblk = (size_t)(N + 127) / 128;
  return round_up(2 * nblk * sizeof(int32_t), 256) + round_up(nblk * nblk, 256);
}

// Key-range split of one forward call (splits = 1: none).
struct SplitArgs {
  int key_chunk = 0;
  void* workspace = nullptr;
  size_t workspace_bytes = 0;
};

int forward_impl(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                 int N, int d, float scale, int causal, const int32_t* key_lens,
                 const uint8_t* block_mask, int block_size, bool sparse, fa_dtype dtype,
                 hipStream_t stream, const SplitArgs& split = SplitArgs(), int block_rows = 0,
                 int block_keys = 0, int key_groups = 0) {
  g_detail[0] = 0;
  bool empty = false;
  int st = check_common(B, H, N, d, scale, dtype, &empty);
  if (st != FA_OK) return st;
  if ((st = check_block(block_mask, block_size, N, sparse)) != FA_OK) return st;
  if (block_rows != 0 && block_rows != 64 && block_rows != 128 && block_rows != 256)
    return fail(FA_ERR_UNSUPPORTED,
                "block_rows=%d (supported: 0 = automatic, 64, 128, 256)", block_rows);
  if (block_keys != 0 && block_keys != 32 && block_keys != 64 && block_keys != 128)
    return fail(FA_ERR_UNSUPPORTED,
                "block_keys=%d (supported: 0 = the type's default, 32, 64, 128)", block_keys);
  // Key tiles other than the type's default (64 keys for 16-bit types, 32 for
  // float32) exist for 16-bit types with 128-row tiles.
  const int default_keys = dtype == FA_F32 ? 32 : 64;
  const bool other_keys = block_keys != 0 && block_keys != default_keys;
  if (other_keys && dtype == FA_F32)
    return fail(FA_ERR_UNSUPPORTED, "float32 forward with %d keys per tile (32 only)", block_keys);
  if (other_keys && block_rows != 0 && block_rows != 128)
    return fail(FA_ERR_UNSUPPORTED,
                "%d keys per tile with %d query rows per tile (128 rows only)", block_keys,
                block_rows);
  if (key_groups < 0 || key_groups > 2)
    return fail(FA_ERR_UNSUPPORTED, "key_groups=%d (supported: 0 = automatic, 1, 2)", key_groups);
  if (key_groups == 2 && (dtype == FA_F32 || block_mask || other_keys ||
                          (block_rows != 0 && block_rows != 128) || split.key_chunk > 0))
    return fail(FA_ERR_UNSUPPORTED, "key_groups=2 takes 16-bit dense self-attention with 128-row "
                "tiles of 64 keys");
  const int rows = other_keys ? 128
                   : block_rows ? block_rows
                                : auto_fwd_rows(B, H, N, d, dtype, block_mask != nullptr);
  int kgroups = key_groups;
  if (kgroups == 0)
    kgroups = block_rows == 0 && !other_keys && split.key_chunk == 0
                  ? auto_fwd_kgroups(B, H, N, d, dtype, block_mask != nullptr)
                  : 1;
  if (block_mask && rows > 128)
    return fail(FA_ERR_UNSUPPORTED, "block-sparse forward with %d query rows per tile (at most 128)",
                rows);
  // Eight fp32 waves at d = 128 need more registers than a CU holds.
  if (dtype == FA_F32 && d == 128 && rows > 128)
    return fail(FA_ERR_UNSUPPORTED, "float32 forward at d=128 with %d query rows per tile "
                "(at most 128)", rows);
  if (empty) return FA_OK;
  if ((st = check_tensor(q, "q", 16)) || (st = check_tensor(k, "k", 16)) ||
      (st = check_tensor(v, "v", 16)) || (st = check_tensor(o, "o", 16)) ||
      (st = check_tensor(lse, "lse", 4)))
    return st;
  if (key_lens && !aligned(key_lens, 4)) return fail(FA_ERR_INVALID_ARG, "key_lens misaligned");
  fa::Problem p{B, H, N, d, scale, causal ? 1 : 0, key_lens, block_mask, (int)dtype, stream, rows};
  p.fwd_keys = other_keys ? block_keys : 0;
  p.fwd_rows = kgroups == 2 ? 128 : p.fwd_rows;
  p.fwd_kgroups = kgroups;
  const int splits = split.key_chunk > 0 ? sparse_splits(N, split.key_chunk) : 1;
  if (splits > 1) {
    const size_t need = split_workspace(B, H, N, d, splits);
    if (!split.workspace)
      return fail(FA_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
    if (!aligned(split.workspace, 16))
      return fail(FA_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
    if (split.workspace_bytes < need)
      return fail(FA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", split.workspace_bytes,
                  need);
    const size_t prow = (size_t)splits * B * H * N;
    p.splits = splits;
    p.chunk = split.key_chunk;
    p.opart = static_cast<float*>(split.workspace);
    p.lpart = reinterpret_cast<float*>(static_cast<char*>(split.workspace) +
                                       round_up(prow * d * sizeof(float), 256));
  }
  fa::FwdTensors t{q, k, v, o, lse};
  hipError_t e = fa::launch_forward(p, t);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "forward launch: %s", hipGetErrorString(e));
  return FA_OK;
}

// Inference forward plan: query rows per work-group and key-range splits.
// Few queries against a long cache leave too few work-groups to fill the
// chip (and to keep enough key/value reads in flight), so the key range is
// split until the work-groups fill one round of the slots the chip holds at
// once (256 CUs times the work-groups whose K/V ring fits one CU's 160 KB of
// LDS: 3 for 16-bit d = 64, 2 for 16-bit d = 128 and fp32 d = 64, 1 for
// fp32 d = 128), each split keeping at least 256 keys; a second pass merges
// the split results.  Measured on the inference workloads: one round beats
// two or four (partial results cost traffic) and no split (idle CUs).
struct KvPlan {
  int rows;    // 32 (one wave; 16-bit types), 64 or 128
  int splits;  // 1: no workspace, O and LSE written directly
  int chunk;   // keys per split, a multiple of 64
};

KvPlan kv_plan(int B, int H, int Nq, int Nk, int d, fa_dtype dtype) {
  KvPlan pl;
  pl.rows = (Nq <= 32 && dtype != FA_F32) ? 32 : (Nq <= 64 ? 64 : 128);
  pl.splits = 1;
  pl.chunk = 0;
  const int per_cu = dtype == FA_F32 ? (d == 64 ? 2 : 1) : (d == 64 ? 3 : 2);
  const long long slots = 256LL * per_cu;
  const long long groups = (long long)B * H * ((Nq + pl.rows - 1) / pl.rows);
  const long long ktiles = ((long long)Nk + 63) / 64;
  if (groups <= 0 || ktiles <= 0 || groups >= slots) return pl;
  long long s = (slots + groups - 1) / groups;
  s = std::min<long long>(s, std::max<long long>(ktiles / 4, 1));
  s = std::min<long long>(s, 64);
  if (s <= 1) return pl;
  const long long per = (ktiles + s - 1) / s;  // key tiles per split
  pl.chunk = (int)(per * 64);
  pl.splits = (int)((ktiles + per - 1) / per);
  if (pl.splits <= 1) pl.splits = 1, pl.chunk = 0;
  return pl;
}

size_t kv_workspace(int B, int H, int Nq, int d, const KvPlan& pl) {
  if (pl.splits <= 1) return 0;
  const size_t rows = (size_t)pl.splits * B * H * Nq;
  return round_up(rows * d * sizeof(float), 256) + round_up(rows * sizeof(float), 256);
}

int check_key_chunk(int key_chunk, int N) {
  if (key_chunk <= 0 || key_chunk % 64 != 0)
    return fail(FA_ERR_UNSUPPORTED, "key_chunk=%d (a positive multiple of 64)", key_chunk);
  if (N > 0 && sparse_splits(N, key_chunk) > kMaxSplits)
    return fail(FA_ERR_UNSUPPORTED, "N=%d with key_chunk=%d gives more than %d splits", N,
                key_chunk, kMaxSplits);
  return FA_OK;
}

}  // namespace

namespace {

// Shared by fa_backward and its two passes.  Pointers a pass does not read
// (passes = the dQ pass only: dk, dv; the dK/dV pass only: o, lse, dq) are
// not checked and may be NULL.
int backward_impl(const void* q, const void* k, const void* v, const void* o, const void* dout,
                  const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d,
                  float scale, int causal, const int32_t* key_lens, const uint8_t* block_mask,
                  int block_size, fa_dtype dtype, void* workspace, size_t workspace_bytes,
                  hipStream_t stream, int passes, fa_dtype grad_dtype, int chunk_blocks = 0,
                  int dq_rows = 0, int dkdv_rows = 0, int key_groups = 0) {
  g_detail[0] = 0;
  bool empty = false;
  int st = check_common(B, H, N, d, scale, dtype, &empty);
  if (st != FA_OK) return st;
  if (grad_dtype != dtype && grad_dtype != FA_F32)
    return fail(FA_ERR_INVALID_ARG, "grad_dtype %d (the input dtype %d or FA_F32)",
                (int)grad_dtype, (int)dtype);
  // Tile sizes of the two passes: 128 rows by default; 64 and 256 for 16-bit
  // inputs with gradients in the input type, 256 without a block mask (a
  // work-group's rows then span two 128-token mask blocks).
  for (int i = 0; i < 2; ++i) {
    const int rows = i == 0 ? dq_rows : dkdv_rows;
    const char* name = i == 0 ? "dq_rows" : "dkdv_rows";
    if (rows != 0 && rows != 64 && rows != 128 && rows != 256)
      return fail(FA_ERR_UNSUPPORTED, "%s=%d (supported: 0 = 128, 64, 128, 256)", name, rows);
    if (rows == 0 || rows == 128) continue;
    if (dtype == FA_F32 || grad_dtype != dtype)
      return fail(FA_ERR_UNSUPPORTED, "%s=%d needs 16-bit inputs and gradients (128 only "
                  "otherwise)", name, rows);
    if (rows == 256 && block_mask)
      return fail(FA_ERR_UNSUPPORTED, "%s=256 with a block mask (at most 128)", name);
  }
  const bool rows128 = (dq_rows == 0 || dq_rows == 128) && (dkdv_rows == 0 || dkdv_rows == 128);
  if (key_groups < 0 || key_groups > 2)
    return fail(FA_ERR_UNSUPPORTED, "key_groups=%d (supported: 0 = automatic, 1, 2)", key_groups);
  if (key_groups == 2 && (dtype == FA_F32 || block_mask || !rows128 || chunk_blocks > 0))
    return fail(FA_ERR_UNSUPPORTED, "key_groups=2 takes 16-bit dense problems with 128-row "
                "tiles");
  const int kgroups = key_groups ? key_groups
                      : rows128 && chunk_blocks == 0
                          ? auto_bwd_kgroups(B, H, N, d, dtype, block_mask != nullptr)
                          : 1;
  if ((st = check_block(block_mask, block_size, N, false)) != FA_OK) return st;
  if (empty) return FA_OK;
  const bool pdq = (passes & fa::kPassDq) != 0, pkv = (passes & fa::kPassDkDv) != 0;
  if ((st = check_tensor(q, "q", 16)) || (st = check_tensor(k, "k", 16)) ||
      (st = check_tensor(v, "v", 16)) || (st = check_tensor(dout, "dout", 16)))
    return st;
  if (pdq && ((st = check_tensor(o, "o", 16)) || (st = check_tensor(lse, "lse", 4)) ||
              (st = check_tensor(dq, "dq", 16))))
    return st;
  if (pkv && ((st = check_tensor(dk, "dk", 16)) || (st = check_tensor(dv, "dv", 16)))) return st;
  if (key_lens && !aligned(key_lens, 4)) return fail(FA_ERR_INVALID_ARG, "key_lens misaligned");
  const size_t need = chunk_blocks > 0
                         ? fa_backward_blocksparse_split_workspace_bytes(B, H, N, d, chunk_blocks)
                         : fa_backward_workspace_bytes(B, H, N, d);
  if (!workspace) return fail(FA_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if (!aligned(workspace, 16)) return fail(FA_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
  if (workspace_bytes < need)
    return fail(FA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
  fa::Problem p{B, H, N, d, scale, causal ? 1 : 0, key_lens, block_mask, (int)dtype, stream};
  p.bwd_passes = passes;
  p.grad_f32 = grad_dtype == FA_F32 && dtype != FA_F32;
  p.bwd_dq_rows = dq_rows ? dq_rows : 128;
  p.bwd_dkdv_rows = dkdv_rows ? dkdv_rows : 128;
  p.bwd_kgroups = kgroups;
  // At d = 128 the dK/dV pass (16-bit inputs, 128-key tiles, unsplit) runs
  // two wave groups on each query tile unless one group is asked for: each
  // group's waves hold half the queries' products, which leaves room for two
  // waves per SIMD.
  p.bwd_dkdv_qs = dtype != FA_F32 && d == 128 && p.bwd_dkdv_rows == 128 && chunk_blocks == 0 &&
                  key_groups != 1;
  if (chunk_blocks > 0) {
    const size_t base = fa_backward_workspace_bytes(B, H, N, d);
    const size_t part = bwd_split_part_bytes(B, H, N, d, chunk_blocks);
    char* const w = static_cast<char*>(workspace);
    p.chunk_blocks = chunk_blocks;
    p.split_items = bwd_split_items(N, chunk_blocks);
    p.part_dq = reinterpret_cast<float*>(w + base);
    p.part_dk = reinterpret_cast<float*>(w + base + part);
    p.part_dv = reinterpret_cast<float*>(w + base + 2 * part);
    const size_t nblk = (size_t)(N + 127) / 128;
    p.split_counts = reinterpret_cast<int32_t*>(w + base + 3 * part);
    p.mask_t = reinterpret_cast<uint8_t*>(w + base + 3 * part +
                                          round_up(2 * nblk * sizeof(int32_t), 256));
  }
  fa::BwdTensors t{q, k, v, o, dout, lse, dq, dk, dv, static_cast<float*>(workspace)};
  hipError_t e = fa::launch_backward(p, t);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "backward launch: %s", hipGetErrorString(e));
  return FA_OK;
}

}  // namespace

extern "C" {

int fa_forward(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
               int N, int d, float scale, int causal, const int32_t* key_lens, fa_dtype dtype,
               hipStream_t stream) {
  return forward_impl(q, k, v, o, lse, B, H, N, d, scale, causal, key_lens, nullptr, 128, false,
                      dtype, stream);
}

int fa_forward_blocksparse(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int H, int N, int d, float scale, int causal,
                           const int32_t* key_lens, const uint8_t* block_mask, int block_size,
                           fa_dtype dtype, hipStream_t stream) {
  return forward_impl(q, k, v, o, lse, B, H, N, d, scale, causal, key_lens, block_mask,
                      block_size, true, dtype, stream);
}

size_t fa_forward_blocksparse_split_workspace_bytes(int B, int H, int N, int d, int key_chunk) {
  if (B <= 0 || H <= 0 || N <= 0 || d <= 0 || key_chunk <= 0 || key_chunk % 64 != 0) return 0;
  const int splits = sparse_splits(N, key_chunk);
  if (splits > kMaxSplits) return 0;
  return split_workspace(B, H, N, d, splits);
}

int fa_forward_blocksparse_split(const void* q, const void* k, const void* v, void* o, float* lse,
                                 int B, int H, int N, int d, float scale, int causal,
                                 const int32_t* key_lens, const uint8_t* block_mask,
                                 int block_size, int key_chunk, fa_dtype dtype, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  g_detail[0] = 0;
  const int st = check_key_chunk(key_chunk, N);
  if (st != FA_OK) return st;
  SplitArgs split;
  split.key_chunk = key_chunk;
  split.workspace = workspace;
  split.workspace_bytes = workspace_bytes;
  return forward_impl(q, k, v, o, lse, B, H, N, d, scale, causal, key_lens, block_mask,
                      block_size, true, dtype, stream, split);
}

size_t fa_forward_kv_workspace_bytes(int B, int H, int Nq, int Nk, int d, fa_dtype dtype) {
  if (B <= 0 || H <= 0 || Nq <= 0 || Nk <= 0 || d <= 0) return 0;
  return kv_workspace(B, H, Nq, d, kv_plan(B, H, Nq, Nk, d, dtype));
}

int fa_forward_kv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                  int Nq, int Nk, int d, float scale, int causal, const int32_t* key_lens,
                  fa_dtype dtype, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  g_detail[0] = 0;
  if (Nk < 0) return fail(FA_ERR_INVALID_ARG, "negative size Nk=%d", Nk);
  bool empty = false;
  int st = check_common(B, H, Nq, d, scale, dtype, &empty);
  if (st != FA_OK) return st;
  if (empty) return FA_OK;
  if ((long long)Nk * d > 0x7fffffffLL) return fail(FA_ERR_INVALID_ARG, "Nk*d exceeds 2^31-1");
  if ((st = check_tensor(q, "q", 16)) || (st = check_tensor(o, "o", 16)) ||
      (st = check_tensor(lse, "lse", 4)))
    return st;
  if (Nk > 0 && ((st = check_tensor(k, "k", 16)) || (st = check_tensor(v, "v", 16)))) return st;
  if (key_lens && !aligned(key_lens, 4)) return fail(FA_ERR_INVALID_ARG, "key_lens misaligned");
  const KvPlan pl = kv_plan(B, H, Nq, Nk, d, dtype);
  const size_t need = kv_workspace(B, H, Nq, d, pl);
  if (need > 0) {
    if (!workspace) return fail(FA_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
    if (!aligned(workspace, 16)) return fail(FA_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
    if (workspace_bytes < need)
      return fail(FA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
  }
  fa::Problem p{B, H, Nq, d, scale, causal ? 1 : 0, key_lens, nullptr, (int)dtype, stream, pl.rows};
  p.nk = Nk;
  p.causal_br = 1;
  p.splits = pl.splits;
  p.chunk = pl.chunk;
  if (pl.splits > 1) {
    const size_t rows = (size_t)pl.splits * B * H * Nq;
    p.opart = static_cast<float*>(workspace);
    p.lpart = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                       round_up(rows * d * sizeof(float), 256));
  }
  fa::FwdTensors t{q, k, v, o, lse};
  hipError_t e = fa::launch_forward(p, t);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "forward launch: %s", hipGetErrorString(e));
  return FA_OK;
}

int fa_forward_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                      const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int B, int H,
                      int Tq, int Tk, int max_seqlen_q, int d, float scale, int causal,
                      fa_dtype dtype, hipStream_t stream) {
  g_detail[0] = 0;
  if (Tq < 0 || Tk < 0 || max_seqlen_q < 0)
    return fail(FA_ERR_INVALID_ARG, "negative size Tq=%d Tk=%d max_seqlen_q=%d", Tq, Tk,
                max_seqlen_q);
  bool empty = false;
  int st = check_common(B, H, max_seqlen_q, d, scale, dtype, &empty);
  if (st != FA_OK) return st;
  if (empty || Tq == 0) return FA_OK;
  if (max_seqlen_q > Tq)
    return fail(FA_ERR_INVALID_ARG, "max_seqlen_q=%d exceeds Tq=%d", max_seqlen_q, Tq);
  if ((st = check_tensor(q, "q", 16)) || (st = check_tensor(o, "o", 16)) ||
      (st = check_tensor(lse, "lse", 4)) || (st = check_tensor(cu_seqlens_q, "cu_seqlens_q", 4)) ||
      (st = check_tensor(cu_seqlens_k, "cu_seqlens_k", 4)))
    return st;
  if (Tk > 0 && ((st = check_tensor(k, "k", 16)) || (st = check_tensor(v, "v", 16)))) return st;
  const int rows = (max_seqlen_q <= 32 && dtype != FA_F32) ? 32 : (max_seqlen_q <= 64 ? 64 : 128);
  fa::Problem p{B, H, max_seqlen_q, d, scale, causal ? 1 : 0, nullptr, nullptr, (int)dtype, stream,
                rows};
  p.nk = Tk;
  p.causal_br = 1;
  p.cu_q = cu_seqlens_q;
  p.cu_k = cu_seqlens_k;
  p.Tq = Tq;
  p.Tk = Tk;
  fa::FwdTensors t{q, k, v, o, lse};
  hipError_t e = fa::launch_forward(p, t);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "forward launch: %s", hipGetErrorString(e));
  return FA_OK;
}

int fa_forward_ex(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                  int N, int d, float scale, int causal, const int32_t* key_lens,
                  const uint8_t* block_mask, int block_size, int block_rows, int block_keys,
                  int key_groups, fa_dtype dtype, hipStream_t stream) {
  return forward_impl(q, k, v, o, lse, B, H, N, d, scale, causal, key_lens, block_mask,
                      block_size, false, dtype, stream, SplitArgs(), block_rows, block_keys,
                      key_groups);
}

int fa_forward_block_rows_for(int B, int H, int N, int d, fa_dtype dtype, int sparse) {
  return auto_fwd_rows(B, H, N, d, dtype, sparse != 0);
}

int fa_forward_key_groups_for(int B, int H, int N, int d, fa_dtype dtype, int sparse) {
  return auto_fwd_kgroups(B, H, N, d, dtype, sparse != 0);
}

int fa_backward_key_groups_for(int B, int H, int N, int d, fa_dtype dtype, int sparse) {
  return auto_bwd_kgroups(B, H, N, d, dtype, sparse != 0);
}

size_t fa_backward_workspace_bytes(int B, int H, int N, int d) {
  if (B <= 0 || H <= 0 || N <= 0 || d <= 0) return 0;
  return round_up(2 * (size_t)B * H * N * sizeof(float), 256);
}

int fa_backward(const void* q, const void* k, const void* v, const void* o, const void* dout,
                const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d,
                float scale, int causal, const int32_t* key_lens, const uint8_t* block_mask,
                int block_size, fa_dtype dtype, void* workspace, size_t workspace_bytes,
                hipStream_t stream) {
  return backward_impl(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale, causal, key_lens,
                       block_mask, block_size, dtype, workspace, workspace_bytes, stream,
                       fa::kPassBoth, dtype);
}

int fa_backward_ex(const void* q, const void* k, const void* v, const void* o, const void* dout,
                   const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d,
                   float scale, int causal, const int32_t* key_lens, const uint8_t* block_mask,
                   int block_size, fa_dtype dtype, fa_dtype grad_dtype, int dq_rows,
                   int dkdv_rows, int key_groups, void* workspace, size_t workspace_bytes,
                   hipStream_t stream) {
  return backward_impl(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale, causal, key_lens,
                       block_mask, block_size, dtype, workspace, workspace_bytes, stream,
                       fa::kPassBoth, grad_dtype, 0, dq_rows, dkdv_rows, key_groups);
}

int fa_backward_dq(const void* q, const void* k, const void* v, const void* o, const void* dout,
                   const float* lse, void* dq, int B, int H, int N, int d, float scale,
                   int causal, const int32_t* key_lens, const uint8_t* block_mask,
                   int block_size, fa_dtype dtype, int rows, void* workspace,
                   size_t workspace_bytes, hipStream_t stream) {
  return backward_impl(q, k, v, o, dout, lse, dq, nullptr, nullptr, B, H, N, d, scale, causal,
                       key_lens, block_mask, block_size, dtype, workspace, workspace_bytes,
                       stream, fa::kPassDq, dtype, 0, rows, 0);
}

int fa_backward_dkdv(const void* q, const void* k, const void* v, const void* dout, void* dk,
                     void* dv, int B, int H, int N, int d, float scale, int causal,
                     const int32_t* key_lens, const uint8_t* block_mask, int block_size,
                     fa_dtype dtype, int rows, void* workspace, size_t workspace_bytes,
                     hipStream_t stream) {
  return backward_impl(q, k, v, nullptr, dout, nullptr, nullptr, dk, dv, B, H, N, d, scale,
                       causal, key_lens, block_mask, block_size, dtype, workspace,
                       workspace_bytes, stream, fa::kPassDkDv, dtype, 0, 0, rows);
}

size_t fa_backward_blocksparse_split_workspace_bytes(int B, int H, int N, int d,
                                                     int chunk_blocks) {
  if (B <= 0 || H <= 0 || N <= 0 || d <= 0 || chunk_blocks <= 0) return 0;
  if (bwd_split_items(N, chunk_blocks) > kMaxSplits) return 0;
  return fa_backward_workspace_bytes(B, H, N, d) +
         3 * bwd_split_part_bytes(B, H, N, d, chunk_blocks) + bwd_split_mask_bytes(N);
}

int fa_backward_blocksparse_split(const void* q, const void* k, const void* v, const void* o,
                                  const void* dout, const float* lse, void* dq, void* dk,
                                  void* dv, int B, int H, int N, int d, float scale, int causal,
                                  const int32_t* key_lens, const uint8_t* block_mask,
                                  int block_size, int chunk_blocks, fa_dtype dtype,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
  g_detail[0] = 0;
  if (chunk_blocks <= 0)
    return fail(FA_ERR_UNSUPPORTED, "chunk_blocks=%d (at least 1)", chunk_blocks);
  if (N > 0 && bwd_split_items(N, chunk_blocks) > kMaxSplits)
    return fail(FA_ERR_UNSUPPORTED, "N=%d with chunk_blocks=%d gives more than %d items", N,
                chunk_blocks, kMaxSplits);
  if (dtype == FA_F32)
    return fail(FA_ERR_UNSUPPORTED, "split backward for float32 inputs (use fa_backward)");
  if (!block_mask) return fail(FA_ERR_INVALID_ARG, "block_mask is NULL");
  return backward_impl(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale, causal, key_lens,
                       block_mask, block_size, dtype, workspace, workspace_bytes, stream,
                       fa::kPassBoth, dtype, chunk_blocks);
}

int fa_backward_noalloc(const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse, void* dq, void* dk, void* dv, int B,
                        int H, int N, int d, float scale, int causal, const int32_t* key_lens,
                        const uint8_t* block_mask, int block_size, fa_dtype dtype,
                        hipStream_t stream) {
  g_detail[0] = 0;
  bool empty = false;
  int st = check_common(B, H, N, d, scale, dtype, &empty);
  if (st != FA_OK) return st;
  if (empty) return FA_OK;
  const size_t need = fa_backward_workspace_bytes(B, H, N, d);
  if (need > fa::kScratchBytes)
    return fail(FA_ERR_UNSUPPORTED,
                "problem needs %zu bytes of scratch; the allocation-free backward holds %zu "
                "(B*H*N <= %zu)",
                need, fa::kScratchBytes, fa::kScratchBytes / 8);
  void* ws = nullptr;
  const hipError_t e = fa::scratch_workspace(&ws);
  if (e != hipSuccess)
    return fail(FA_ERR_HIP, "scratch address lookup: %s", hipGetErrorString(e));
  return backward_impl(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale, causal, key_lens,
                       block_mask, block_size, dtype, ws, fa::kScratchBytes, stream,
                       fa::kPassBoth, dtype);
}

size_t fa_backward_noalloc_max_rows(void) { return fa::kScratchBytes / 8; }

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE";
    case FA_ERR_HIP: return "FA_ERR_HIP";
  }
  return "FA_ERR_UNKNOWN";
}

const char* fa_last_error_detail(void) { return g_detail; }

}  // extern "C"
