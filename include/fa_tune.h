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
 * instantiated (32 query rows per wave; 64-key tiles; one or two key
 * groups), so that a sweep can time each shape on the device.  libfa.so
 * itself launches the shape its table names and is not changed by loading
 * this library.
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
 * hint, key groups) triples into waves[] / occupancy[] / key_groups[] (any
 * may be NULL) and returns how many there are (7 for D = 64, 5 for D = 96
 * and 128), or FA_ERR_UNSUPPORTED_D.  Key groups 2: the waves form two
 * groups over the same 32 * waves / 2 query rows, taking alternate key
 * tiles, merged in LDS at the end.  Host only.
 */
int fa_tune_shapes(int64_t D, int* waves, int* occupancy, int* key_groups, int capacity);

/*
 * fa_tune_forward -- fa_forward (same arguments, same checks and status
 * codes, dense [B, H, N, D], FA_F16 or FA_BF16 only) with the workgroup
 * shape given: `waves` waves per workgroup in `key_groups` groups (32 query
 * rows per wave of a group) and the compiler's waves_per_eu hint
 * `occupancy`.  A triple that fa_tune_shapes does not list for D returns
 * FA_ERR_UNSUPPORTED_D.  One kernel on `stream`.
 */
int fa_tune_forward(const void* q, const void* k, const void* v, void* o, int64_t B, int64_t H,
                    int64_t N, int64_t D, float scale, int causal, int dtype, int waves,
                    int occupancy, int key_groups, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_TUNE_H_ */
