/*
 * fc_internal.h -- measurement helpers of libfc.so, not part of the codec's
 * interface (include/fc.h). The benchmark uses them to measure the bandwidth
 * ceiling that plain streaming kernels reach on this GPU for the traffic
 * shapes of the codec's kernels, and the engine clock while the pipeline runs.
 */
#ifndef FC_INTERNAL_H_
#define FC_INTERNAL_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * One streaming pass over `bytes` bytes of `src` (device pointers, 16-byte
 * aligned, bytes % 16 == 0), enqueued on `stream` (a hipStream_t; NULL = the
 * default stream):
 *   kind 0  copy:             dst[0 .. bytes) = src[0 .. bytes)
 *   kind 1  read 4, write 1:  reads src, writes bytes/4 bytes of dst (one
 *           4-byte word per 16 bytes read: the xor of its four words)
 *   kind 2  read:             reads src, writes one 4-byte word per wave
 *           tile (dst must hold 4 * ceil(bytes / (slots * 1024)) bytes)
 *   kind 3  read 1, write 4:  reads src, writes 4 * bytes bytes of dst (16
 *           bytes per 4 read)
 * slots: 16-byte loads each lane keeps in flight (1, 2, 4 or 8).
 * Returns 0, or 1 (NULL pointer), 2 (bad kind or slots), 4 (alignment or
 * size not a multiple of 16), 6 (launch error). bytes == 0 enqueues nothing.
 * The caller owns both buffers; nothing is allocated.
 */
int fc_internal_stream_probe(int kind, int slots, const void *src, void *dst, size_t bytes,
                             void *stream);

/*
 * The engine clock at the point of the stream where it is enqueued: one wave
 * runs `iters` (1 .. 2^20) dependent fused multiply-adds and writes three
 * uint64 values to `out` (device pointer, 8-byte aligned, 24 bytes):
 * out[0] shader-clock cycles elapsed (s_memtime), out[1] ticks of the
 * constant 100 MHz counter (s_memrealtime) over the same interval, out[2] a
 * value that keeps the work alive. Clock in MHz = 100 * out[0] / out[1].
 * Returns 0, or 1 (NULL), 2 (iters out of range), 4 (alignment), 6 (launch).
 */
int fc_internal_clock_probe(void *out, int iters, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* FC_INTERNAL_H_ */
