/*
 * moe_testing.h -- hooks of libmoe_shard.so for tests of its error paths.
 *
 * Not part of the layer: production callers never need these.  They let a
 * test reach a failure the device would otherwise only meet by chance, with
 * every kernel still ending normally.
 */
#ifndef MOE_TESTING_H
#define MOE_TESTING_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Bound of the grouped GEMM's wait for rows that another tile of the same
 * launch produces (the one-launch kernel's second GEMM waits for the first
 * GEMM's tiles of its rows), for every later call in this process:
 *   spins  > 0  that many sleeps (about 50 ns each) before a tile gives up;
 *   spins == 0  the default (about 0.2 s, far beyond any tile's work);
 *   spins  < 0  a tile gives up at once, without waiting.
 * A tile that gives up leaves its rows of expert_out unwritten and reports
 * MOE_ERR_GEMM_WAIT (moe_shard.h).  Returns MOE_OK. */
int moe_testing_set_gemm_wait_limit(int32_t spins);

#ifdef __cplusplus
}
#endif

#endif /* MOE_TESTING_H */
