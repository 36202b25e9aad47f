/*
 * kaio_roof.h -- measurement aid shipped beside libkaio (libkaio_roof.so).
 *
 * Not an operation of the pages and not part of libkaio's ABI: a plain
 * streaming read of device memory, used by the benchmark as the measured
 * ceiling an HBM-bound kernel moving the same bytes is compared with.
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
 * One wave that reads the shader-clock counter and the constant-rate real-time
 * counter, sleeps until `ticks` real-time ticks have passed, and stores
 * {shader cycles, real-time ticks, start tick, end tick} (four u64) to the
 * device buffer `out` (8-byte aligned).  Launched on a side stream while
 * another kernel runs, it reports the shader clock under that load:
 * MHz = cycles / ticks * kaio_roof_wall_clock_khz() / 1000.
 * Returns 0 on a queued launch, 1 for a bad pointer, 3 if the launch failed.
 */
int kaio_roof_clock_probe(void* out, unsigned long long ticks, void* stream);
/* Rate of the real-time counter of the current device in kHz (0 if unknown). */
int kaio_roof_wall_clock_khz(void);

#ifdef __cplusplus
}
#endif

#endif /* KAIO_ROOF_H */
