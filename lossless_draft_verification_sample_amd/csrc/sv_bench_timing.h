/*
 * sv_bench_timing.h - per-kernel event timing of the benchmark build
 * (libspecverify_bench.so). Not part of the verifier's interface: the product
 * library (libspecverify.so) has neither these calls nor the event records.
 *
 * The benchmark build exports every entry point of spec_verify.h with the same
 * kernels; while a profile is active, each of its launches records a HIP event
 * pair around the kernel on the caller's stream.
 *
 *   sv_bench_profile_start(n)  creates event pairs for up to n launches of each
 *                              kernel (host side, not thread-safe; one profile
 *                              at a time per process). SV_EINVAL when n < 1 or
 *                              a profile is already active, SV_EHIP when an
 *                              event cannot be created.
 *   sv_bench_profile_stop(ms, launches)
 *                              synchronises on those events, writes the summed
 *                              milliseconds and the launch count of each kernel
 *                              (arrays of SV_NUM_KERNELS entries, indexed by
 *                              SV_K_*; either may be NULL) and releases them.
 *                              SV_EINVAL without an active profile.
 */
#ifndef SV_BENCH_TIMING_H
#define SV_BENCH_TIMING_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SV_K_ROW_STATS 0
#define SV_K_DRAW 1
#define SV_K_GREEDY_ARGMAX 2
#define SV_K_GREEDY_SCAN 3
#define SV_K_OVERLAP 4
#define SV_K_COMMIT 5
#define SV_NUM_KERNELS 6

int sv_bench_profile_start(int32_t max_launches_per_kernel);
int sv_bench_profile_stop(double* total_ms, int32_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* SV_BENCH_TIMING_H */
