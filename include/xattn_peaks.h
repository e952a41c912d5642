/*
 * xattn_peaks.h — C ABI of libxattn_peaks.so: microbenchmarks that measure the
 * peak rates the attention library is compared against on one MI355X
 * (gfx950). Measurement code only, separate from libxattn.so.
 *
 * Every call only enqueues work on `stream` (a hipStream_t passed as void*,
 * NULL = the null stream) and returns a hipError_t value (0 = success); the
 * caller times the launch (e.g. with events on the same stream) and owns every
 * buffer, all of them device memory.
 */
#ifndef XATTN_PEAKS_H
#define XATTN_PEAKS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Waves per workgroup of xattn_peak_mfma (two per SIMD). */
int32_t xattn_peak_mfma_waves_per_block(void);

/*
 * Matrix-core rate: `blocks` workgroups, each wave running `iters` rounds of
 * 16 v_mfma_f32_32x32x16_bf16 (2*32*32*16 FLOP each) on four independent
 * accumulators, no memory traffic. FLOP per launch = blocks * waves_per_block
 * * iters * 16 * 32768.
 *  sink  device float[blocks * 64 * waves_per_block]: written, keeps the loop live.
 *  clk   device uint64[2 * blocks] or NULL: per workgroup, the core-clock
 *        counter delta (s_memtime) and the 100 MHz reference counter delta
 *        (s_memrealtime) over the loop, so clock = 100 MHz * clk[0] / clk[1].
 */
int32_t xattn_peak_mfma(int32_t blocks, int32_t iters, float* sink, unsigned long long* clk, void* stream);

/*
 * HBM stream copy of `bytes` (a non-zero multiple of 16) from src to dst with
 * 16-byte vector loads and stores; bytes moved = 2 * bytes.
 */
int32_t xattn_peak_copy(const void* src, void* dst, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* XATTN_PEAKS_H */
