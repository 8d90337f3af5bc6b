/*
 * dsa_indexer_profile.h -- optional per-kernel timing of the indexer library.
 *
 * For benchmarks and tuning: while a profiling window is open, every kernel
 * the library launches is bracketed by two HIP events recorded on the
 * caller's stream (the stream the kernel runs on).  Closing the window waits
 * for those events and reports, per kernel name, the number of launches and
 * their mean duration.  Outside a window the library records no events.
 *
 * Not thread-safe: open, run and close a window from one host thread.
 */
#ifndef DSA_INDEXER_PROFILE_H_
#define DSA_INDEXER_PROFILE_H_

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

#ifdef __cplusplus
}
#endif
#endif /* DSA_INDEXER_PROFILE_H_ */
