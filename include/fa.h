/*
 * fa.h - tiled exact attention for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libfa.so.  Every tensor argument is a DEVICE pointer owned by the
 * caller; the library never allocates, frees or synchronises memory it was
 * handed, and it launches all work asynchronously on the caller's stream.
 * It keeps no settings between calls (the only state is the thread-local
 * text of fa_last_error_detail), so calls from several threads are safe as
 * long as calls sharing a workspace are ordered on one stream.
 * Asynchronous kernel faults surface at the caller's next synchronisation.
 *
 * Method (FlashAttention, as summarised by the review page "FlashAttention"
 * of agent-readings, section "Method", and the slides' steps 01-04): exact
 * softmax(scale * Q K^T) V is computed tile by tile.  Q, K and V are cut into
 * blocks that fit in on-chip memory, each score tile is formed on chip, a
 * running row maximum and denominator (online softmax, visual guide,
 * "online softmax" paragraph) rescale the partial outputs, and only the
 * output O and one normalisation value per row (the logsumexp) reach HBM.
 * The backward pass recomputes score tiles from that logsumexp instead of
 * reading an N x N matrix (review page, claim C7).
 *
 * Common conventions
 *   Layout     Q, K, V, O, dO, dQ, dK, dV: [B, H, N, d] contiguous, d fastest.
 *              LSE: [B, H, N] float32, natural log: LSE_i = ln sum_j exp(S_ij)
 *              over the keys visible to query i, S = scale * Q K^T.
 *   dtype      FA_F32, FA_F16 or FA_BF16 for all of Q, K, V, O, dO, dQ, dK, dV.
 *              16-bit inputs use bf16/fp16 matrix cores with fp32 accumulation;
 *              probabilities are rounded to the input dtype (round to nearest
 *              even) before the P V product.  FA_F32 computes in fp32 only.
 *   d          64 or 128.
 *   scale      finite and >= 0 (the usual value is 1/sqrt(d)).
 *   causal     nonzero: key j is visible to query i only if j <= i.
 *   key_lens   int32[B] on the device, or NULL.  Key j of batch b is visible
 *              only if j < key_lens[b] (values are clamped to [0, N]); query
 *              rows are never masked by it.
 *   block_mask uint8[nb][nb] on the device, nb = ceil(N / block_size), one
 *              mask shared by every (b, h); entry (I, J) != 0 keeps the keys
 *              of block J for the queries of block I (visual guide,
 *              block-sparse paragraph).  block_size must be 128 and
 *              nb <= 1024 (N <= 131072) when a block mask is given.
 *   Masks combine by logical AND.  A query row with no visible key gets
 *   O = 0 and LSE = -inf and contributes nothing to any gradient.
 *   Empty problems (B, H or N equal to 0) return FA_OK and launch nothing.
 *   Alignment  tensors of the input dtype and the workspace: 16 bytes;
 *              LSE, key_lens: 4 bytes.
 *
 * Errors: every argument is checked on the host before any HIP call.  A bad
 * argument returns FA_ERR_INVALID_ARG or FA_ERR_UNSUPPORTED and nothing is
 * launched; a failed launch returns FA_ERR_HIP.  fa_last_error_detail() then
 * describes the failure (thread-local text, valid until the next call on the
 * same thread).  No C++ exception crosses this interface.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { FA_F32 = 0, FA_F16 = 1, FA_BF16 = 2 } fa_dtype;

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = 1,   /* null pointer, negative size, misalignment, ... */
  FA_ERR_UNSUPPORTED = 2,   /* well-formed but not provided: d, block_size, scale < 0 */
  FA_ERR_WORKSPACE = 3,     /* workspace missing or smaller than required */
  FA_ERR_HIP = 4            /* the HIP runtime reported an error */
} fa_status;

/*
 * Forward pass (review page, "Method": tiles of Q, K, V in on-chip memory,
 * online softmax, write only the output and small normalisation values).
 * Reads q, k, v; writes o [B,H,N,d] (dtype) and lse [B,H,N] (float32).
 */
int fa_forward(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int N, int d, float scale, int causal,
               const int32_t* key_lens, fa_dtype dtype, hipStream_t stream);

/*
 * Block-sparse forward (visual guide, block-sparse paragraph; review page,
 * "Method", last step): as fa_forward, with key/value tiles whose block_mask
 * entry is zero never loaded.  block_mask must not be NULL.  The result is
 * exact attention under the block mask.
 */
int fa_forward_blocksparse(const void* q, const void* k, const void* v, void* o,
                           float* lse, int B, int H, int N, int d, float scale,
                           int causal, const int32_t* key_lens,
                           const uint8_t* block_mask, int block_size,
                           fa_dtype dtype, hipStream_t stream);

/*
 * fa_forward_blocksparse with the key range of every query tile split over
 * ceil(N / key_chunk) work-groups, whose float32 partial O and LSE a second
 * pass merges (the online-softmax merge of per-block states, taken across
 * work-groups).  For masks that give a few query tiles far more kept blocks
 * than the rest (a global row), whose single work-group would otherwise run
 * the whole key range alone.  key_chunk: keys per split, a positive multiple
 * of 64 (FA_ERR_UNSUPPORTED otherwise, or beyond 1024 splits); a split with
 * no kept block contributes nothing.  workspace: caller-owned device memory
 * of at least fa_forward_blocksparse_split_workspace_bytes(B,H,N,d,key_chunk)
 * bytes, 16-byte aligned, not initialised (NULL when that is 0, i.e. one
 * split: then the call is fa_forward_blocksparse); calls that share it must
 * be ordered on one stream.  Same results as fa_forward_blocksparse up to the
 * rounding of the merge.
 */
int fa_forward_blocksparse_split(const void* q, const void* k, const void* v, void* o, float* lse,
                                 int B, int H, int N, int d, float scale, int causal,
                                 const int32_t* key_lens, const uint8_t* block_mask,
                                 int block_size, int key_chunk, fa_dtype dtype, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream);
size_t fa_forward_blocksparse_split_workspace_bytes(int B, int H, int N, int d, int key_chunk);

/*
 * Inference forward: Nq new queries against a key/value cache of Nk entries
 * (review page, "Caveats": the kernel later became central to inference
 * stacks; "Agent Infrastructure Takeaways": for long contexts, memory
 * traffic and key/value residency dominate the cost).  The pages give no
 * detail; the reading here: q, o [B,H,Nq,d]; k, v [B,H,Nk,d]; lse [B,H,Nq]
 * float32.  key_lens (int32[B] on device, or NULL for all Nk) gives the
 * filled part of each batch's cache, L_b = key_lens[b] clamped to [0, Nk];
 * keys j >= L_b are never visible.  The queries are the newest Nq positions
 * of that sequence, so with causal set query i sees key j iff
 * j <= i + L_b - Nq (aligned bottom-right; with Nq = Nk = L_b this is
 * fa_forward's causal mask).  A row that sees no key gets O = 0 and
 * LSE = -inf.  Nk may be 0 (every row sees no key).
 * With few queries (decode) the key range is split over several
 * work-groups, whose float32 partial results a second pass merges; they go
 * to workspace, caller-owned device memory of at least
 * fa_forward_kv_workspace_bytes(B,H,Nq,Nk,d,dtype) bytes, 16-byte aligned,
 * need not be initialised.  workspace may be NULL when that size is 0.
 * Calls that share a workspace must be ordered on one stream.  The tile
 * height is chosen from Nq.
 */
int fa_forward_kv(const void* q, const void* k, const void* v, void* o, float* lse,
                  int B, int H, int Nq, int Nk, int d, float scale, int causal,
                  const int32_t* key_lens, fa_dtype dtype, void* workspace,
                  size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes fa_forward_kv needs for these sizes (0: none needed). */
size_t fa_forward_kv_workspace_bytes(int B, int H, int Nq, int Nk, int d, fa_dtype dtype);

/*
 * Packed variable-length forward (same passages as fa_forward_kv): B
 * sequences of different lengths stored back to back without padding.
 * q, o: [H, Tq, d]; k, v: [H, Tk, d]; lse: [H, Tq] float32 (head-major, like
 * the [B,H,N,d] layout with the batch folded into the rows).  cu_seqlens_q
 * and cu_seqlens_k: int32[B+1] on device, prefix sums starting at 0:
 * sequence b owns query rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 and key
 * rows cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1 of every head, and attends to
 * its own keys only, with fa_forward_kv's visibility (nq, nk = its own
 * counts; causal aligned bottom-right, top-left when they are equal).
 * Offsets are clamped into [0, Tq] / [0, Tk] on the device.  max_seqlen_q
 * must be at least every sequence's query count (it sizes the grid; query
 * rows of a longer sequence past it, rounded up to the tile, would not be
 * written; the library cannot check it, since the prefix sums live on the
 * device, and the Python binding checks it when they are given on the host).
 * Rows outside every sequence are not written.  No workspace.
 */
int fa_forward_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                      const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                      int B, int H, int Tq, int Tk, int max_seqlen_q, int d, float scale,
                      int causal, fa_dtype dtype, hipStream_t stream);

/*
 * Backward pass (review page, "Method" and claim C7: recompute the attention
 * tiles on chip from the saved normalisation values).  Gradient of
 * L = sum(dout * o): with P = exp(S - LSE), D = rowsum(dout * o),
 * dV = P^T dout, dP = dout V^T, dS = P * (dP - D), dQ = scale * dS K,
 * dK = scale * dS^T Q.
 * o and lse must come from fa_forward / fa_forward_blocksparse(_split) called with
 * the same q, k, v, sizes, scale and masks.  block_mask may be NULL (dense);
 * block_size is ignored then.  Overwrites dq, dk, dv (dtype).
 * workspace: device memory of at least fa_backward_workspace_bytes(B,H,N,d)
 * bytes, 16-byte aligned, owned by the caller, contents need not be
 * initialised; the dQ pass fills it with -D = -rowsum(dout * o) and
 * LSE * log2(e), each float32 [B,H,N], which the dK/dV pass that follows
 * reads.  Calls that share a workspace must be ordered on one stream.
 */
int fa_backward(const void* q, const void* k, const void* v, const void* o,
                const void* dout, const float* lse, void* dq, void* dk, void* dv,
                int B, int H, int N, int d, float scale, int causal,
                const int32_t* key_lens, const uint8_t* block_mask, int block_size,
                fa_dtype dtype, void* workspace, size_t workspace_bytes,
                hipStream_t stream);

/*
 * fa_backward with the gradients' storage type and the tile sizes chosen
 * per call.
 *   grad_dtype  the input dtype (then this is fa_backward) or FA_F32, which
 *               writes dq, dk, dv as float32 [B,H,N,d] (4-byte elements,
 *               16-byte aligned).  The computation is the same; only the
 *               final rounding to a 16-bit type is left out, so the 16-bit
 *               results of fa_backward are exactly the round-to-nearest-even
 *               of these.  Meant for callers that accumulate gradients in
 *               float32 and for measuring the computation's error apart from
 *               the output rounding (the output rounding of a bf16 value of
 *               magnitude 4 to 8 is already 2^-6).  Any other grad_dtype is
 *               FA_ERR_INVALID_ARG.
 *   dq_rows     query rows per work-group of the dQ pass, and
 *   dkdv_rows   keys per work-group of the dK/dV pass: 0 (= 128), 64, 128 or
 *               256 (review page, claims C2 and C3, applied to the backward:
 *               each work-group streams the other side's tiles through
 *               on-chip memory once, so those re-reads fall as its rows
 *               grow).  64 and 256 take 16-bit inputs with grad_dtype = dtype,
 *               256 no block mask; other combinations and values are
 *               FA_ERR_UNSUPPORTED.  Results agree to rounding for every
 *               value (the accumulation order over tiles is unchanged, so
 *               they are in fact bitwise equal).
 *   key_groups  groups of waves per work-group that split each tile's sweep
 *               (the dQ pass's key tiles, the dK/dV pass's query tiles) in
 *               halves and add their partial gradients on chip: 1, 2, or 0
 *               to let the library choose (fa_backward_key_groups_for; with
 *               128-row tiles only).  2 takes 16-bit inputs, no block mask
 *               and 128-row tiles, else FA_ERR_UNSUPPORTED.  At d = 128 the
 *               dK/dV pass (16-bit inputs, 128-key tiles, any mask)
 *               splits every query tile between two groups, one
 *               32-query half each, with K and V read from LDS, whenever
 *               key_groups is not 1; with 1 it keeps one group, one wave
 *               per SIMD.  Results agree to rounding (the halves are added
 *               in another order).
 */
int fa_backward_ex(const void* q, const void* k, const void* v, const void* o,
                   const void* dout, const float* lse, void* dq, void* dk, void* dv,
                   int B, int H, int N, int d, float scale, int causal,
                   const int32_t* key_lens, const uint8_t* block_mask, int block_size,
                   fa_dtype dtype, fa_dtype grad_dtype, int dq_rows, int dkdv_rows,
                   int key_groups, void* workspace, size_t workspace_bytes,
                   hipStream_t stream);

/*
 * Key groups (see fa_backward_ex) that a backward of these sizes uses when
 * key_groups is 0 and the tiles are 128 rows: 2 for 16-bit dense problems
 * whose grid holds at most 512 tiles at d = 64 (two per compute unit) or 256
 * at d = 128, else 1.  (At d = 128 this is the dQ pass's choice; the dK/dV
 * pass splits its query tiles whenever key_groups is not 1.)  Host
 * arithmetic only.
 */
int fa_backward_key_groups_for(int B, int H, int N, int d, fa_dtype dtype, int sparse);

/*
 * The two passes of fa_backward, for callers that schedule them separately
 * (and for timing each).  fa_backward is fa_backward_dq followed by
 * fa_backward_dkdv on the same stream, with the same arguments and workspace.
 *   fa_backward_dq    writes dq; fills the workspace with -D = -rowsum(dout * o)
 *                     and LSE * log2(e) (float32 [B,H,N] each).  Reads q, k, v,
 *                     o, dout, lse.
 *   fa_backward_dkdv  writes dk, dv; reads q, k, v, dout and the workspace
 *                     that a preceding fa_backward_dq with the same q, k, v,
 *                     o, dout, lse, sizes, scale and masks filled (unchanged
 *                     since).  It may be called again on that workspace.
 *   rows              the pass's tile height: dq_rows or dkdv_rows of
 *                     fa_backward_ex (0 = 128), under the same rules; the
 *                     workspace does not depend on it.  Key groups as
 *                     fa_backward_ex with key_groups 0.
 * Other arguments, validation and errors as fa_backward.
 */
int fa_backward_dq(const void* q, const void* k, const void* v, const void* o,
                   const void* dout, const float* lse, void* dq,
                   int B, int H, int N, int d, float scale, int causal,
                   const int32_t* key_lens, const uint8_t* block_mask, int block_size,
                   fa_dtype dtype, int rows, void* workspace, size_t workspace_bytes,
                   hipStream_t stream);
int fa_backward_dkdv(const void* q, const void* k, const void* v, const void* dout,
                     void* dk, void* dv, int B, int H, int N, int d, float scale,
                     int causal, const int32_t* key_lens, const uint8_t* block_mask,
                     int block_size, fa_dtype dtype, int rows, void* workspace,
                     size_t workspace_bytes, hipStream_t stream);

/*
 * Block-sparse backward for masks with a few very long block rows or columns
 * (visual guide, block-sparse paragraph: long-context results; a "global"
 * row attends every key block, a global column is seen by every query
 * block).  As fa_backward with block_mask required, except that each mask
 * row (dQ pass) and each mask column (dK/dV pass) is handed out in items of
 * chunk_blocks kept blocks, one work-group per item, instead of one
 * work-group sweeping the whole row or column.  A row or column with at most
 * chunk_blocks kept blocks is one item and writes its gradients directly;
 * the items of a longer one write float32 partials to the workspace, which a
 * reduction sums in item order (deterministic).  Arguments:
 *   chunk_blocks  kept mask blocks per item, >= 1 (FA_ERR_UNSUPPORTED
 *                 otherwise, or beyond 1024 items per row);
 *   dtype         FA_F16 or FA_BF16 (FA_F32: FA_ERR_UNSUPPORTED; gradients
 *                 come back in dtype);
 *   workspace     caller-owned device memory of at least
 *                 fa_backward_blocksparse_split_workspace_bytes(B,H,N,d,
 *                 chunk_blocks) bytes, 16-byte aligned, not initialised:
 *                 fa_backward's workspace, then three float32 partial arrays
 *                 [items][B,H,N,d] (items = ceil(ceil(N/128) / chunk_blocks)),
 *                 of which only split rows and columns touch their part, then
 *                 the kept-block counts of every mask row and column and the
 *                 transposed mask.  Calls that share a workspace must be
 *                 ordered on one stream.
 * Same results as fa_backward up to the rounding of the partial sums.
 */
int fa_backward_blocksparse_split(const void* q, const void* k, const void* v,
                                  const void* o, const void* dout, const float* lse,
                                  void* dq, void* dk, void* dv, int B, int H, int N,
                                  int d, float scale, int causal,
                                  const int32_t* key_lens, const uint8_t* block_mask,
                                  int block_size, int chunk_blocks, fa_dtype dtype,
                                  void* workspace, size_t workspace_bytes,
                                  hipStream_t stream);
size_t fa_backward_blocksparse_split_workspace_bytes(int B, int H, int N, int d,
                                                     int chunk_blocks);

/*
 * Forward with the tile sizes chosen per call (review page, claims C2 and
 * C3: tiling reduces HBM reads and writes, and the IO cost depends on the
 * on-chip memory size; K and V are read once per query tile, so that traffic
 * falls as the tile height B_r grows, whatever the key-tile width B_c).  As
 * fa_forward, plus:
 *   block_mask, block_size  as fa_forward_blocksparse, or block_mask NULL
 *                           (dense; block_size is then ignored);
 *   block_rows  query rows per work-group: 64, 128 or 256, or 0 to let the
 *               library choose (fa_forward_block_rows_for).  The block-sparse
 *               forward takes 64 or 128 (FA_ERR_UNSUPPORTED for 256, since a
 *               128-token mask block must hold a whole tile), and so does the
 *               float32 forward at d = 128 (eight float32 waves would need
 *               more registers than a compute unit holds); any other value
 *               is FA_ERR_UNSUPPORTED.
 *   block_keys  keys per K/V tile streamed through on-chip memory: 0 for the
 *               default (64 for 16-bit types, 32 for float32), or 32, 64,
 *               128.  Widths other than the default take 16-bit types and
 *               128 query rows per tile (block_rows 0 or 128; 0 then means
 *               128); other combinations and values are FA_ERR_UNSUPPORTED.
 *   key_groups  groups of waves that split each query tile's key range and
 *               merge their online-softmax states on chip (review page,
 *               "Method": per-block states combine exactly after rescaling
 *               to a common reference): 1, 2, or 0 to let the library choose
 *               (fa_forward_key_groups_for; only with block_rows 0 and the
 *               default block_keys).  2 takes 16-bit types without a block
 *               mask, 128-row tiles (block_rows 0 or 128) and the default
 *               key-tile width; otherwise FA_ERR_UNSUPPORTED.
 * Tuning and measurement options: results agree to rounding for every
 * value.  fa_forward and fa_forward_blocksparse are this call with
 * block_rows = 0, block_keys = 0 and key_groups = 0.
 */
int fa_forward_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                  int B, int H, int N, int d, float scale, int causal,
                  const int32_t* key_lens, const uint8_t* block_mask, int block_size,
                  int block_rows, int block_keys, int key_groups, fa_dtype dtype,
                  hipStream_t stream);

/*
 * Query rows per work-group that a forward of these sizes uses when
 * block_rows is 0 (sparse != 0: a block mask is given): 256 for 16-bit
 * d = 128 dense problems whose 256-row grid holds at least 512 work-groups,
 * else 128.  Host arithmetic only.
 */
int fa_forward_block_rows_for(int B, int H, int N, int d, fa_dtype dtype, int sparse);

/*
 * Key groups (see fa_forward_ex) that a forward of these sizes uses when
 * key_groups is 0: 2 for 16-bit dense problems whose tiles are 128 rows and
 * whose grid holds at most 512 of them (two per compute unit: too few to keep
 * every unit busy until the longest causal tile ends), else 1.  Host
 * arithmetic only.
 */
int fa_forward_key_groups_for(int B, int H, int N, int d, fa_dtype dtype, int sparse);

/*
 * fa_backward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same computation and results, with the workspace taken from a device array
 * inside the library instead of a caller buffer.  Calls no allocating
 * routine.  The array holds 16 MiB on each GPU the library runs on, until the
 * process ends; problems whose workspace (fa_backward_workspace_bytes, 8 bytes
 * per query row) exceeds it, i.e. B * H * N > fa_backward_noalloc_max_rows(),
 * return FA_ERR_UNSUPPORTED before anything is launched.  The array of the
 * current device is used, so stream must belong to the current device.
 * Every call on a GPU shares that GPU's array: calls that overlap on one GPU
 * (different streams, or other threads) race and must not be made; calls
 * ordered on one stream are safe.  Nothing in the array needs clearing
 * between calls (the first pass writes every entry the second reads).
 */
int fa_backward_noalloc(const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse, void* dq, void* dk, void* dv,
                        int B, int H, int N, int d, float scale, int causal,
                        const int32_t* key_lens, const uint8_t* block_mask, int block_size,
                        fa_dtype dtype, hipStream_t stream);
size_t fa_backward_noalloc_max_rows(void);

/* Workspace bytes fa_backward needs for these sizes (0 for an empty problem). */
size_t fa_backward_workspace_bytes(int B, int H, int N, int d);

/* Name of a status code; never NULL. */
const char* fa_status_string(int status);

/* Detail of the last non-OK return on the calling thread ("" if none). */
const char* fa_last_error_detail(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
