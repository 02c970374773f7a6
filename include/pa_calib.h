/*
 * pa_calib.h - C ABI of libpacalib.so, the read-bandwidth calibration kernels
 * that the benchmark runs beside the paged decode.
 *
 * Paged decode is bound by HBM reads ([INFRA] "【infra之路】10-PagedAttention 与
 * KV Cache 管理" §1.2: each decode step reads the whole cache to produce one
 * token). These two kernels measure what plain reads reach on the device the
 * decode runs on, so that the decode's rate can be set against a ceiling that
 * was measured, not only against the data-sheet peak:
 *
 *   pa_calib_stream_read  every byte of one contiguous buffer, once;
 *   pa_calib_tile_read    whole tiles of a buffer in the order a list gives
 *                         (a shuffled list reads scattered tiles, as a paged
 *                         decode reads scattered blocks; [INFRA] FAQ puts the
 *                         cost of non-contiguous reads under 5%).
 *
 * Both issue 16-byte non-temporal loads, 64 lanes x 16 bytes = 1 KiB per wave
 * instruction, with `loads_in_flight` (1..16) loads of each lane outstanding,
 * and write nothing but a rarely taken store into `sink` (4 bytes, device
 * memory) that keeps the loads alive. Pointers are device pointers owned by the
 * caller; nothing is allocated or synchronised; work is enqueued on `stream`.
 *
 * Return value: 0 on success; 1 for a NULL pointer; 2 for a size out of range
 * or misaligned (buffers and tile sizes must be multiples of 16 KiB and 1 KiB
 * and 16-byte aligned); 5 when the launch failed (the codes of pagedattn.h).
 */
#ifndef PA_CALIB_H
#define PA_CALIB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Reads bytes of buf (a multiple of 16384) once. workgroups of 256 threads
 * (0: 4 per compute unit) walk it in a grid-stride loop; each lane keeps
 * loads_in_flight 16-byte loads outstanding.
 */
int32_t pa_calib_stream_read(const void *buf, size_t bytes, int32_t workgroups,
                             int32_t loads_in_flight, uint32_t *sink, void *stream);

/*
 * Reads tiles tiles[0..num_tiles) of buf, each tile_bytes long (a multiple of
 * 1024, at most 65536), tile i starting at byte tiles[i] * tile_bytes. tiles is
 * int32 device memory; entries must lie in [0, num_buf_tiles) (entries outside
 * are skipped). Wave g of the grid reads tiles g, g + W, g + 2W, ... (W =
 * waves in the grid), with its lanes' loads_in_flight loads outstanding.
 */
int32_t pa_calib_tile_read(const void *buf, int64_t num_buf_tiles, const int32_t *tiles,
                           int32_t num_tiles, int32_t tile_bytes, int32_t workgroups,
                           int32_t loads_in_flight, uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_CALIB_H */
