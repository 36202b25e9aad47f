/*
 * kaio_roof.h -- measurement aid shipped beside libkaio (libkaio_roof.so).
 *
 * Not an operation of the pages and not part of libkaio's ABI: a plain
 * streaming read of device memory and a read of the packed-weight layout by
 * column strips, used by the benchmark as the measured ceilings an HBM-bound
 * kernel moving the same bytes is compared with, MFMA work alone (the same for
 * the MFMA-bound kernels), and a shader-clock probe.
 */
#ifndef KAIO_ROOF_H
#define KAIO_ROOF_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Reads `bytes` (a multiple of 16) from the device buffer `src` (16-byte
 * aligned) with 16-byte loads: ceil(bytes / (16 * loads_per_thread * threads))
 * workgroups of `threads` threads, each thread issuing its `loads_per_thread`
 * loads before using any.  Nothing is written in practice; `sink` must be a
 * device buffer of kaio_roof_sink_bytes(bytes, loads_per_thread, threads)
 * bytes all the same (the kernel may store there).  Supported
 * (loads_per_thread, threads): (1|2|4|8|16, 256), (4|8|16, 512), (4|8|16, 1024); a
 * negative loads_per_thread selects the same shape with non-temporal loads.
 * Returns 0 on a queued launch, 1 for a bad pointer or size, 2 for an
 * unsupported shape, 3 if the launch failed.
 */
int kaio_roof_stream_read(const void* src, size_t bytes, void* sink, int loads_per_thread, int threads,
                          void* stream);
size_t kaio_roof_sink_bytes(size_t bytes, int loads_per_thread, int threads);

/*
 * Reads three arrays of `rows` x `cols` u32 (row major, 16-byte aligned
 * device buffers a0, a1, a2; rows a multiple of 128, cols of 64, both at most
 * 2^20) by column strips, with non-temporal loads:
 *   strip_cols = 64: 3*cols/64 workgroups of 16 waves, one per 64-column
 *     strip of one array; each wave a contiguous row range, 16-byte loads, so
 *     each row is read in 256-byte segments (the packed-weight reads of the
 *     decode kernel);
 *   strip_cols = 16: cols/16 workgroups of 8 waves, one per 16-column strip
 *     of all three arrays; 4-byte loads, 64-byte row segments.
 * `sink` must be a device buffer of kaio_roof_strip_sink_bytes(cols,
 * strip_cols) bytes (the kernel may store there).  Returns 0 on a queued
 * launch, 1 for a bad pointer or size, 2 for an unsupported strip width, 3 if
 * the launch failed.
 */
int kaio_roof_strip_read(const void* a0, const void* a1, const void* a2, unsigned rows, unsigned cols,
                         int strip_cols, void* sink, void* stream);
size_t kaio_roof_strip_sink_bytes(unsigned cols, int strip_cols);

/*
 * One wave that reads the shader-clock counter and the constant-rate real-time
 * counter, sleeps until `ticks` real-time ticks have passed, and stores
 * {shader cycles, real-time ticks, start tick, end tick} (four u64) to the
 * device buffer `out` (8-byte aligned).  Launched on a side stream while
 * another kernel runs, it reports the shader clock under that load:
 * MHz = cycles / ticks * kaio_roof_wall_clock_khz() / 1000.
 * Returns 0 on a queued launch, 1 for a bad pointer, 3 if the launch failed.
 */
int kaio_roof_clock_probe(void* out, unsigned long long ticks, void* stream);
/*
 * MFMA work alone: `workgroups` workgroups of 4 waves, each wave issuing
 * iters x 8 dense f16 MFMAs (16x16x32, f32 accumulate) on register operands,
 * with no memory traffic but one 4-byte store per thread at the end, into
 * `sink` (a device buffer of workgroups * 256 floats, 4-byte aligned).  Its
 * sustained rate is the ceiling of matrix-core work under the chip's power
 * limit, against which the MFMA-bound kernels are weighed beside the nominal
 * peak.  iters: a multiple of 4 in [4, 2^20]; workgroups in [1, 2^20].
 * Returns 0 on a queued launch, 1 for a bad argument, 3 if the launch failed.
 * kaio_roof_mfma_flops gives the flops of one launch.
 */
int kaio_roof_mfma(void* sink, int iters, int workgroups, void* stream);
double kaio_roof_mfma_flops(int iters, int workgroups);

/* Rate of the real-time counter of the current device in kHz (0 if unknown). */
int kaio_roof_wall_clock_khz(void);

#ifdef __cplusplus
}
#endif

#endif /* KAIO_ROOF_H */
