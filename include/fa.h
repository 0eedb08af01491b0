/*
 * fa.h -- C ABI of the MI355X (gfx950) FlashAttention forward library.
 *
 * The operation is attention as the page "Android Transformer Optimization:
 * Attention and Mobile GPU Bottlenecks" states it in its section "The
 * Self-Attention Bottleneck Is Memory Traffic, Not Compute": for every
 * (batch b, head h),
 *
 *     O = softmax(scale * Q K^T [+ causal mask]) V,
 *
 * the softmax taken along each row, with the softmax scale of "Flash
 * Attention on Android: tiled SGEMM with RenderScript", section
 * "Architecture: tiled attention with RenderScript BLAS" (1/sqrt(headDim)
 * there; any finite factor here).  It is computed the way the first page's
 * sections "The Essence of FlashAttention: Reordering the Computation" and
 * "A Complete Tile Loop" describe: Q, K and V are cut into tiles, each score
 * tile stays on chip, an online softmax keeps a running row maximum and
 * denominator and rescales the output accumulator, and O is divided by the
 * denominator once at the end; the N x N score matrix never reaches memory.
 *
 * All entry points are plain C, take plain pointers and sizes, never throw,
 * never print and never allocate device memory (the three-pass comparison
 * path at the end takes its scratch space from the caller).
 */
#ifndef FA_H_
#define FA_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage type of q, k, v and o (all four share it).  16-bit inputs are
 * multiplied on the matrix cores with fp32 accumulation, softmax and
 * accumulators in fp32 (the mixed precision that "Optimizing for Mobile
 * GPUs", section "Exploit 16-bit Precision", recommends: 16-bit storage,
 * fp32 accumulation).  fp32 inputs form their scores on the fp64 matrix
 * cores (exact products, fp64 sums) and the rest in fp32. */
typedef enum fa_dtype {
  FA_F32 = 0,  /* IEEE binary32 */
  FA_F16 = 1,  /* IEEE binary16 */
  FA_BF16 = 2  /* bfloat16 */
} fa_dtype;

/* Status codes.  Every failure is reported before anything is launched, so a
 * failed call writes nothing. */
typedef enum fa_status {
  FA_OK = 0,
  FA_ERR_NULL = -1,           /* q, k, v or o is NULL (with N > 0) */
  FA_ERR_DIM = -2,            /* B < 1, H < 1, N < 0 or D < 1 */
  FA_ERR_UNSUPPORTED_D = -3,  /* head dimension not in {64, 96, 128} */
  FA_ERR_DTYPE = -4,          /* dtype not an fa_dtype value, or not taken by the call */
  FA_ERR_ALIGN = -5,          /* a pointer is not 16-byte aligned */
  FA_ERR_ALIAS = -6,          /* o overlaps q, k or v */
  FA_ERR_LAUNCH = -7,         /* the HIP runtime refused the launch */
  FA_ERR_SCALE = -8,          /* scale is NaN or infinite */
  FA_ERR_TOO_LARGE = -9,      /* N*D >= 2^31, or the grid would overflow */
  FA_ERR_DEVICE = -10,        /* current device is not gfx950, or no device */
  FA_ERR_WORKSPACE = -11,     /* workspace NULL, misaligned, too small or overlapping */
  FA_ERR_SPLITS = -12,        /* num_splits outside 0..64 */
  FA_ERR_STRIDE = -13,        /* negative strides, rows shorter than D, overlapping o rows */
  FA_ERR_SCRATCH = -14        /* fa_forward_ex_noalloc: the partials exceed the fixed scratch */
} fa_status;

/*
 * fa_forward -- attention forward pass, O = softmax(scale*QK^T [+mask]) V.
 *
 *   q, k, v  device pointers to [B, H, N, D] tensors, dense, row-major (D
 *            fastest, then N, then H, then B), storage type `dtype`,
 *            16-byte aligned.  Read only; they may alias one another.
 *   o        device pointer to the [B, H, N, D] output, same layout and
 *            type, 16-byte aligned, must not overlap q, k or v.  Every
 *            element is written; nothing outside it is.
 *   B, H     batch size and number of heads (>= 1).  Heads are independent.
 *   N        sequence length of queries and keys (>= 0; 0 is a no-op).
 *   D        head dimension: 64, 96 or 128.
 *   scale    softmax scale (finite; 1/sqrt(D) is the usual choice; 0 gives
 *            the mean of the visible V rows; negative values are allowed).
 *   causal   0: every query sees all N keys.  Non-zero: query i sees keys
 *            j <= i only (top-left aligned, diagonal included).
 *   dtype    an fa_dtype value.
 *   stream   hipStream_t to enqueue on; NULL means the default stream.
 *
 * The call is asynchronous: it validates its arguments on the host,
 * enqueues one kernel on `stream` and returns.  The caller owns all buffers
 * and synchronises.  The library holds no state between calls apart from a
 * per-device cache of the device check and CU count, and allocates nothing.
 * When B*H times the 16-bit kernel's query blocks leave much of the device
 * idle (few heads, short rows; fa_key_groups_suggest), each workgroup's
 * waves split its key tiles in two groups whose partial results are merged
 * in LDS by the rescaling rule of the online softmax; the arithmetic order
 * changes, the result agrees to the same tolerance.
 * Pointers must be device memory of the current HIP device.
 * Returns FA_OK or a negative fa_status.
 */
int fa_forward(const void* q, const void* k, const void* v, void* o, int64_t B, int64_t H,
               int64_t N, int64_t D, float scale, int causal, int dtype, void* stream);

/*
 * fa_forward_strided -- fa_forward on tensors laid out by strides, with
 * grouped key/value heads.  The operation is fa_forward's, per (b, h), with
 * query head h attending to key/value head h / (H / H_kv): H_kv == H is
 * ordinary multi-head attention, 1 < H_kv < H grouped-query attention,
 * H_kv == 1 multi-query attention (the sharing of K/V heads is not on the
 * pages; it is how LLM layers lay out the same computation).
 *
 *   q, o        device pointers, H heads: element (b, h, n, d) at
 *               base[b*s[0] + h*s[1] + n*s[2] + d] with s = q_strides /
 *               o_strides (host arrays of 3 int64, in elements).
 *   k, v        the same with H_kv heads and k_strides / v_strides.
 *               Dense [B, H, N, D] is {H*N*D, N*D, D}; the [B, N, H, D]
 *               layout of many LLM stacks is {N*H*D, D, H*D}.
 *   B, H, H_kv  batch, query heads, key/value heads (H % H_kv == 0).
 *   N, D, scale, causal, dtype, stream   as for fa_forward.
 *
 * Requirements, checked in this order after fa_forward's dtype, size, head
 * dimension, scale and N == 0 checks: no NULL pointer (FA_ERR_NULL);
 * strides >= 0 (FA_ERR_STRIDE); pointers 16-byte aligned and every stride a
 * multiple of 16 bytes (FA_ERR_ALIGN); every row stride >= D, and the
 * (b, h, n) rows of o pairwise disjoint (FA_ERR_STRIDE); N*D < 2^31 and
 * max(N, 64) row strides below 2^32 bytes for every tensor (FA_ERR_TOO_LARGE);
 * the span of o overlapping none of the spans of q, k, v (FA_ERR_ALIAS);
 * the device (FA_ERR_DEVICE).  Inputs may overlap one another.
 * Asynchronous, one kernel, allocates nothing.
 */
int fa_forward_strided(const void* q, const int64_t* q_strides, const void* k,
                       const int64_t* k_strides, const void* v, const int64_t* v_strides, void* o,
                       const int64_t* o_strides, int64_t B, int64_t H, int64_t H_kv, int64_t N,
                       int64_t D, float scale, int causal, int dtype, void* stream);

/*
 * fa_forward_ex -- fa_forward with two additions beside the same tile loop:
 *
 * Log-sum-exp output.  The online softmax of "Android Transformer
 * Optimization: Attention and Mobile GPU Bottlenecks", sections "The
 * Essence of FlashAttention: Reordering the Computation" and "A Complete
 * Tile Loop", ends each row with a running maximum m and denominator l;
 * lse = m + ln l = ln sum_j exp(scale * q_i . k_j) over the visible keys,
 * in natural-log units of the scaled scores.
 *
 * Split-KV.  Each query block's key tiles are cut into num_splits even
 * ranges, one workgroup each, so that short or few heads still fill the
 * device.  Each range leaves its own normalised partial O_r and lse_r in
 * the workspace; a second kernel merges them by the same rescaling rule
 * that the tile loop applies between tiles: with lse = ln sum_r
 * exp(lse_r), O = sum_r exp(lse_r - lse) O_r.
 *
 *   q, k, v, o, B, H, N, D, scale, causal, dtype, stream
 *                    as for fa_forward.
 *   lse              NULL, or device pointer to B*H*N floats ([B, H, N],
 *                    4-byte aligned, overlapping none of q, k, v, o) that
 *                    receive each row's log-sum-exp.
 *   num_splits       1: no split (workspace unused, may be NULL);
 *                    2..64: that many key ranges per query block;
 *                    0: the value fa_splitkv_suggest returns.
 *   workspace        for num_splits != 1: device memory of the current
 *                    device, 256-byte aligned, at least
 *                    fa_forward_ex_workspace_bytes(...) bytes, overlapping
 *                    none of q, k, v, o, lse.  Layout: fp32 partials
 *                    [splits, B*H, N, D], then their log-sum-exp
 *                    [splits, B*H, N], each on a 256-byte boundary.  Owned by
 *                    the caller; calls that share it and overlap in time
 *                    race.
 *   workspace_bytes  its size.
 *
 * Checks as fa_forward, then FA_ERR_SPLITS, FA_ERR_ALIGN / FA_ERR_ALIAS for
 * lse, FA_ERR_TOO_LARGE for the larger grid, FA_ERR_WORKSPACE, in that
 * order, all before anything is enqueued.  Enqueues one kernel (two with
 * splits: the ranges, then the merge).  O agrees with fa_forward's to the
 * same tolerance; the ranges change the order of the arithmetic only.
 */
int fa_forward_ex(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                  int64_t H, int64_t N, int64_t D, float scale, int causal, int dtype,
                  int num_splits, void* workspace, int64_t workspace_bytes, void* stream);

/*
 * fa_forward_ex_noalloc -- fa_forward_ex for callers that cannot allocate
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments without workspace / workspace_bytes, the
 * same kernels and results.  The split-KV partials go to a scratch array of
 * FA_NOALLOC_SCRATCH_BYTES that the library holds in each device's memory
 * from the first call on that device until the process ends; the call
 * allocates nothing and clears nothing (every partial the merge reads is
 * written earlier in the same call).
 *
 * A call whose partials (fa_forward_ex_workspace_bytes for the same
 * arguments) exceed FA_NOALLOC_SCRATCH_BYTES returns FA_ERR_SCRATCH and
 * enqueues nothing; num_splits resolving to 1 needs no scratch.  Other
 * checks and codes as fa_forward_ex (FA_ERR_DEVICE also when the scratch
 * address cannot be looked up).  All calls on one device share its scratch
 * array: calls that overlap in time on one device (two streams, two host
 * threads) race and must be serialised by the caller.
 */
#define FA_NOALLOC_SCRATCH_BYTES (64LL * 1024 * 1024)
int fa_forward_ex_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                          int64_t B, int64_t H, int64_t N, int64_t D, float scale, int causal,
                          int dtype, int num_splits, void* stream);

/*
 * fa_forward_ex_workspace_bytes -- workspace bytes fa_forward_ex needs
 * (0 when num_splits resolves to 1 or N == 0).  num_splits 0 resolves as
 * fa_splitkv_suggest does (so it queries the current device).  Negative
 * fa_status on bad arguments (FA_ERR_SPLITS, FA_ERR_DTYPE, FA_ERR_DIM,
 * FA_ERR_UNSUPPORTED_D, FA_ERR_TOO_LARGE, FA_ERR_DEVICE).
 */
int64_t fa_forward_ex_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t D, int dtype,
                                      int causal, int num_splits);

/*
 * fa_splitkv_suggest -- key ranges per query block that fill the current
 * device: 1 when B*H times the query blocks already occupy every resident
 * workgroup slot, else enough ranges to do so, at most 16 and leaving each
 * range at least 16 key tiles (shorter ranges lose more to the merge than
 * they gain); for FA_F32 also 1 where fa_forward's own workgroup shape
 * (fa_workgroup_shape: fewer rows, more key groups) leaves less key-tile
 * work on one SIMD than the ranges would.  Returns >= 1, or a negative fa_status
 * (FA_ERR_DTYPE, FA_ERR_DIM, FA_ERR_UNSUPPORTED_D, FA_ERR_TOO_LARGE,
 * FA_ERR_DEVICE when no device is current).
 */
int fa_splitkv_suggest(int64_t B, int64_t H, int64_t N, int64_t D, int dtype, int causal);

/*
 * fa_key_groups_suggest -- how many key groups the workgroups of fa_forward,
 * fa_forward_strided and fa_forward_ex (with one key range) use on the
 * current device for these sizes, when dtype is FA_F16 or FA_BF16 and
 * N > 64:
 *   - non-causal: B*H times the blocks of 256 rows is at most a quarter of
 *     the CU count (4 at D = 96 and 128, else 2), or at most half of it for
 *     D = 64 and 128 (2); or
 *   - causal: B*H times the one-group kernel's query blocks (256 rows; 128
 *     for D = 64 and 96) fill at most half of the device's workgroup slots
 *     (one per CU; two for D = 64; 4 at D = 96 and 128, else 2), or at most
 *     three quarters (2), except bf16 at D = 96 and 128 in that last band,
 *     or at most once with N >= 4096 (2; 4 at D = 96; bf16 at D = 128
 *     excepted);
 * for FA_F32 (16 query rows per wave, 32-key tiles; f = B*H times the
 * blocks of 64 rows over the CUs): for f < 1, and causal f <= 1, the shape
 * with the least key-tile work per SIMD among 32 rows in four groups, 16
 * rows in four, 32 rows in two and 64 rows in two (4 or 2); causal with
 * 1 < f <= 2, 2 (32 rows per group at D = 64, 64 at D = 96 and 128);
 * non-causal D = 128 with f >= 2, 1; else 2 when N >= 256 (64 rows in each
 * group), 1 below, and 1 whenever N <= 32 (fa_workgroup_shape names the
 * rows).  With 2 the waves of
 * a 16-bit workgroup (64 query rows, or 128 on the
 * fuller of those grids) form two groups that take alternate key tiles;
 * with 4, eight waves over 64 query rows form four groups that take every
 * fourth 32-key tile.  The groups' running maxima, denominators and
 * accumulators are merged in LDS by the rescaling rule of the online
 * softmax ("Android Transformer Optimization: Attention and Mobile GPU
 * Bottlenecks", section "A Complete Tile Loop").  Host only; returns 1, 2,
 * 4 or a negative fa_status
 * (FA_ERR_DTYPE, FA_ERR_DIM, FA_ERR_UNSUPPORTED_D, FA_ERR_TOO_LARGE,
 * FA_ERR_DEVICE when no device is current).
 */
int fa_key_groups_suggest(int64_t B, int64_t H, int64_t N, int64_t D, int dtype, int causal);

/*
 * fa_workgroup_shape -- the workgroup shape fa_forward (and fa_forward_ex
 * with one key range, and fa_forward_strided) launches on the current
 * device for these sizes: *waves wave64s per workgroup, *key_groups (1, 2
 * or 4, as fa_key_groups_suggest) and *block_n keys per LDS tile (32 or
 * 64), the tile loop of "Android Transformer Optimization: Attention and
 * Mobile GPU Bottlenecks", section "A Complete Tile Loop", sized as "Flash
 * Attention on Android: tiled SGEMM with RenderScript", section "The detail
 * that breaks naive ports: tile calibration", asks (measured per device).
 * Each wave owns 32 query rows of its group for FA_F16 and FA_BF16, 16 for
 * FA_F32 (always 32-key tiles).  Any output pointer may be NULL.  Host
 * only; returns FA_OK or FA_ERR_DTYPE, FA_ERR_DIM, FA_ERR_UNSUPPORTED_D,
 * FA_ERR_TOO_LARGE, FA_ERR_DEVICE.
 */
int fa_workgroup_shape(int64_t B, int64_t H, int64_t N, int64_t D, int dtype, int causal, int* waves,
                       int* key_groups, int* block_n);

/*
 * The three-pass ("naive") attention that tiling is measured against:
 * "Android Transformer Optimization: Attention and Mobile GPU Bottlenecks",
 * section "The Self-Attention Bottleneck Is Memory Traffic, Not Compute",
 * and "Flash Attention on Android: tiled SGEMM with RenderScript", sections
 * "The bottleneck most engineers misdiagnose" and "Benchmark results:
 * Snapdragon vs. Dimensity", describe it: the full N x N score matrix is
 * written to memory, read back for the row softmax, and the probabilities
 * are read back once more for the product with V.  It computes the same O
 * as fa_forward (same arguments, same masking) and exists to measure what
 * the tiled pass saves.  Three kernels are enqueued on `stream`:
 *
 *   scores:  S[i][j] = scale * q_i . k_j, fp32, [B*H, N, NP] row-major
 *            with NP = N rounded up to 64 (keys N..NP-1 are not written;
 *            causal: only the 32-key blocks up to each row block's
 *            diagonal are);
 *   softmax: P[i][j] = exp(S[i][j] - max_j S[i][j]) / sum_j exp(...), the
 *            storage type, [B*H, N, NP] (keys past N, and under the causal
 *            mask keys past i up to the end of i's 64-key block, get 0);
 *            within every aligned group of 16 keys the entries are stored
 *            in the key order 0-3, 8-11, 4-7, 12-15 (the order in which the
 *            third kernel's matrix-core operand takes them); for FA_BF16 P
 *            is kept as two bf16 arrays, a rounded value and the rounded
 *            remainder, whose sum carries 16 significant bits;
 *   P V:     O = P V, the storage type.
 *
 * Only FA_F16 and FA_BF16 are taken (FA_F32 returns FA_ERR_DTYPE).
 */

/*
 * fa_naive_workspace_bytes -- bytes of workspace fa_naive_forward needs for
 * these sizes: B*H*N*NP*4 (S), then B*H*N*NP*2 (P), then for FA_BF16 another
 * B*H*N*NP*2 (the remainders of P), each part starting on a 256-byte
 * boundary.  0 when N == 0.  Returns a negative fa_status instead for an
 * unsupported dtype (FA_ERR_DTYPE), B < 1, H < 1 or N < 0 (FA_ERR_DIM), or
 * a size that does not fit in int64_t (FA_ERR_TOO_LARGE).  Host only; no
 * device call.
 */
int64_t fa_naive_workspace_bytes(int64_t B, int64_t H, int64_t N, int dtype);

/*
 * fa_naive_forward -- O = softmax(scale*QK^T [+mask]) V in three passes
 * through the caller's workspace.
 *
 *   q, k, v, o, B, H, N, D, scale, causal, stream
 *                    as for fa_forward (dtype FA_F16 or FA_BF16 only).
 *   workspace        device memory of the current device, 256-byte
 *                    aligned, at least fa_naive_workspace_bytes(B, H, N,
 *                    dtype) bytes, overlapping none of q, k, v, o.  Its
 *                    contents on entry do not matter; on return (once the
 *                    stream has run) it holds S and P as laid out above.
 *                    The caller owns it and must not use it until the
 *                    stream has finished the call.
 *   workspace_bytes  its size in bytes.
 *
 * Checks and status codes as for fa_forward, in the same order, then
 * FA_ERR_TOO_LARGE for N > 2^20, then FA_ERR_WORKSPACE for a NULL,
 * misaligned, short or overlapping workspace (all before anything is
 * enqueued).  Asynchronous; allocates nothing.
 * Calls that share a workspace and overlap in time race.
 */
int fa_naive_forward(const void* q, const void* k, const void* v, void* o, int64_t B, int64_t H,
                     int64_t N, int64_t D, float scale, int causal, int dtype, void* workspace,
                     int64_t workspace_bytes, void* stream);

/* Properties of the current HIP device that a measurement reports beside its
 * figures: *cus = compute units, *max_clock_khz = peak shader clock (kHz),
 * both from the HIP runtime.  Either pointer may be NULL.  Returns FA_OK, or
 * FA_ERR_DEVICE when no device is current or the runtime refuses the query
 * (outputs untouched).  Synchronous; enqueues nothing. */
int fa_device_info(int* cus, int* max_clock_khz);

/* Human-readable text for a status code (static storage, never NULL). */
const char* fa_status_string(int status);

/* Library version and target, e.g. "fa-mi355x 0.1.0 gfx950" (static). */
const char* fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
