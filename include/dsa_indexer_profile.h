/*
 * dsa_indexer_profile.h -- optional per-kernel timing of the indexer library.
 *
 * For benchmarks and tuning: while a profiling window is open, every kernel
 * the library launches is bracketed by two HIP events recorded on the
 * caller's stream (the stream the kernel runs on).  Closing the window waits
 * for those events and reports, per kernel name, the number of launches and
 * their mean duration.  Outside a window the library records no events.
 *
 * The events come from a pool that opening a window tops up to 1024 pairs
 * (on the current device; the pool is rebuilt when the device changes), so
 * a window of up to 1024 launches creates no events while it is open.
 *
 * Not thread-safe: open, run and close a window from one host thread.
 */
#ifndef DSA_INDEXER_PROFILE_H_
#define DSA_INDEXER_PROFILE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Open a window (discarding any previous one).  Returns 0. */
int dsa_indexer_profile_begin(void);

/* Close the window: synchronise its events and write up to `max_kernels`
 * entries: names[i] (static strings), launches[i], mean_ms[i].  Returns the
 * number of distinct kernels seen (which may exceed max_kernels), or -1 on a
 * HIP error. */
int dsa_indexer_profile_end(const char** names, int32_t* launches, double* mean_ms, int max_kernels);

/* Sustained rate of the score step on this part: the routine that scores
 * (query, key) pairs (the index-score equation of the DeepSeek DSA FLOPs
 * notes, section "Lightning Indexer FLOPs") run on synthetic operands held in
 * registers and LDS, with no memory traffic.  No Top-K path calls it; it
 * gives the rate an MFMA-bound scoring kernel can reach once the clock has
 * settled under that load, next to the nominal peak.
 *
 * dtype: DSA_BF16 or DSA_FP8_E4M3 of dsa_indexer.h (full-entropy codes).  mode 0: the MFMAs and
 * key-fragment LDS reads alone; mode 1: also the ReLU-weighted head sum and
 * the cross-half combine of every 32-key block, as the streaming Top-K issues
 * them; mode 2 (bf16 only): the head sum in the form (w/2)(x + |x|), one FMA
 * with an absolute-value source per head and key, plus the linear term on a
 * 16-row MFMA block (8 more 16x16x32 MFMAs per 32 keys; its FLOPs are not
 * counted below).  The launch has *workgroups (two per compute unit of the current
 * device) workgroups of four waves; each wave scores `iters` (even, >= 2)
 * blocks of 32 keys against 64 heads x 128 dims, so a launch does
 * (*workgroups) * 4 * iters * 2 * 64 * 32 * 128 MFMA FLOP.  The caller times
 * it (events on `stream`, a hipStream_t or NULL).
 *
 * out: device buffer of out_len floats, at least (*workgroups) * 256 (per-lane
 * sinks that keep the work live; contents unspecified), or NULL to report
 * *workgroups only, launching nothing.  workgroups must not be NULL.
 * Returns 0 or a DSA_ERR_* code of dsa_indexer.h: DSA_ERR_INVALID_ARG (dtype, mode or iters out of range, mode 2
 * with fp8, out_len too small, workgroups NULL); DSA_ERR_HIP (device query or launch failed). */
int dsa_indexer_mfma_ceiling(int32_t dtype, int32_t mode, int32_t iters, float* out, size_t out_len, void* stream,
                             int32_t* workgroups);

#ifdef __cplusplus
}
#endif
#endif /* DSA_INDEXER_PROFILE_H_ */
