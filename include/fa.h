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
 * never print and never allocate device memory.
 */
#ifndef FA_H_
#define FA_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage type of q, k, v and o (all four share it).  Arithmetic is fp32
 * (scores, softmax, accumulators) whatever the storage type; 16-bit inputs
 * are multiplied on the matrix cores with fp32 accumulation (the mixed
 * precision that "Optimizing for Mobile GPUs", section "Exploit 16-bit
 * Precision", recommends: 16-bit storage, fp32 accumulation). */
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
  FA_ERR_DTYPE = -4,          /* dtype is not an fa_dtype value */
  FA_ERR_ALIGN = -5,          /* a pointer is not 16-byte aligned */
  FA_ERR_ALIAS = -6,          /* o overlaps q, k or v */
  FA_ERR_LAUNCH = -7,         /* the HIP runtime refused the launch */
  FA_ERR_SCALE = -8,          /* scale is NaN or infinite */
  FA_ERR_TOO_LARGE = -9,      /* N*D >= 2^31, or the grid would overflow */
  FA_ERR_DEVICE = -10         /* current device is not gfx950, or no device */
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
 * per-device cache of the device check, and allocates nothing.
 * Pointers must be device memory of the current HIP device.
 * Returns FA_OK or a negative fa_status.
 */
int fa_forward(const void* q, const void* k, const void* v, void* o, int64_t B, int64_t H,
               int64_t N, int64_t D, float scale, int causal, int dtype, void* stream);

/* Human-readable text for a status code (static storage, never NULL). */
const char* fa_status_string(int status);

/* Library version and target, e.g. "fa-mi355x 0.1.0 gfx950" (static). */
const char* fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
