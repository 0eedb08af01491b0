/*
 * fa_tune.h -- C ABI of the tile-calibration library (libfa_tune.so).
 *
 * "Android Transformer Optimization: Attention and Mobile GPU Bottlenecks",
 * section "Implementation Recommendations" (size tiles from the device's
 * on-chip memory), and "Flash Attention on Android: tiled SGEMM with
 * RenderScript", section "The detail that breaks naive ports: tile
 * calibration" (the best size differs between devices and has to be
 * measured on each).  This library is built from the same kernel
 * sources as libfa.so, with every workgroup shape of the calibration sweep
 * instantiated (16-bit kernel: 32 query rows per wave; 32-, 64- or
 * 128-key tiles; one, two or four key groups; fp32 kernel: 16 query rows
 * per wave, 64-, 32- or 16-row workgroups in one, two or four key groups),
 * so that a sweep can time each shape on the device.  libfa.so itself
 * launches the shape its rules name and is not changed by loading this
 * library.
 *
 * Status codes are fa_status values from fa.h.  Nothing here allocates.
 */
#ifndef FA_TUNE_H_
#define FA_TUNE_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * fa_tune_shapes -- the workgroup shapes the sweep covers for head
 * dimension D: writes up to `capacity` (waves per workgroup, waves_per_eu
 * hint, key groups, keys per LDS tile) quadruples into waves[] /
 * occupancy[] / key_groups[] / block_n[] (any may be NULL) and returns how
 * many there are (14 for D = 64, 8 for D = 96 and 128), or
 * FA_ERR_UNSUPPORTED_D.  Key groups 2: the waves form two groups over the
 * same 32 * waves / 2 query rows, taking alternate key tiles, merged in LDS
 * at the end (64-key tiles only).  block_n is the number of keys staged in
 * LDS per tile, per barrier: 32, 64 or 128 (128 at D = 64 only, where four
 * ring slots of K and V take 128 KiB of the 160 KiB; the softmax and the
 * products then run on its two 64-key halves).  Host only.
 */
int fa_tune_shapes(int64_t D, int* waves, int* occupancy, int* key_groups, int* block_n,
                   int capacity);

/*
 * fa_tune_forward -- fa_forward (same arguments, same checks and status
 * codes, dense [B, H, N, D], FA_F16 or FA_BF16 only) with the workgroup
 * shape given: `waves` waves per workgroup in `key_groups` groups (32 query
 * rows per wave of a group), the compiler's waves_per_eu hint `occupancy`,
 * and `block_n` keys per LDS tile.  A quadruple that fa_tune_shapes does
 * not list for D returns FA_ERR_UNSUPPORTED_D.  One kernel on `stream`.
 */
int fa_tune_forward(const void* q, const void* k, const void* v, void* o, int64_t B, int64_t H,
                    int64_t N, int64_t D, float scale, int causal, int dtype, int waves,
                    int occupancy, int key_groups, int block_n, void* stream);

/*
 * fa_tune_f32_shapes -- the workgroup shapes of the fp32 (matrix-core)
 * kernel the sweep covers for head dimension D: writes up to `capacity`
 * pairs into row_waves[] and key_groups[] (either may be NULL) and returns
 * how many there are (5: (4, 1), (4, 2), (2, 2), (2, 4), (1, 4)), or
 * FA_ERR_UNSUPPORTED_D.  A workgroup owns 16 * row_waves query rows, 16
 * per wave, in key_groups groups of row_waves waves that take every
 * key_groups-th key tile (32 keys) of the rows and merge their results at
 * the end.  Host only.
 */
int fa_tune_f32_shapes(int64_t D, int* row_waves, int* key_groups, int capacity);

/*
 * fa_tune_forward_f32 -- fa_forward with dtype FA_F32 (same arguments
 * otherwise, same checks and status codes, dense [B, H, N, D]) on the fp32
 * kernel with the shape (row_waves, key_groups).  A pair that
 * fa_tune_f32_shapes does not list returns FA_ERR_UNSUPPORTED_D.  One
 * kernel on `stream`.
 */
int fa_tune_forward_f32(const void* q, const void* k, const void* v, void* o, int64_t B, int64_t H,
                        int64_t N, int64_t D, float scale, int causal, int row_waves, int key_groups,
                        void* stream);

/*
 * fa_tune_split_merge -- the merge kernel of fa_forward_ex's split-KV path
 * on its own, for checks of its combination rule ("Android Transformer
 * Optimization: Attention and Mobile GPU Bottlenecks", sections "The
 * Essence of FlashAttention: Reordering the Computation" and "A Complete
 * Tile Loop": partial results against different maxima are brought to a
 * common one by exp(m_old - m_new)) on partials the caller writes:
 *
 *   part_o    device fp32 [splits, rows, D], 16-byte aligned: each range's
 *             O normalised by its own denominator;
 *   part_lse  device fp32 [splits, rows]: each range's log-sum-exp, -inf
 *             for a range that saw no key of the row;
 *   o         device [rows, D] in the storage type `dtype` (FA_F32, FA_F16,
 *             FA_BF16), 16-byte aligned;
 *   lse       NULL or device fp32 [rows].
 *
 * With M = max_r lse_r and L = sum_r exp(lse_r - M):
 * o = sum_r exp(lse_r - M) O_r / L and lse = M + ln L; a row with L = 0 gets
 * o = 0 and lse = -inf.  D in {64, 96, 128}, 1 <= splits <= 64.  Returns
 * FA_OK or FA_ERR_DTYPE / FA_ERR_DIM / FA_ERR_SPLITS / FA_ERR_NULL /
 * FA_ERR_ALIGN / FA_ERR_DEVICE / FA_ERR_LAUNCH.  One kernel on `stream`.
 */
int fa_tune_split_merge(const float* part_o, const float* part_lse, void* o, float* lse, int64_t rows,
                        int64_t D, int splits, int dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_TUNE_H_ */
