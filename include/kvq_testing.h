/*
 * kvq_testing.h - test and tuning hooks of libkvq.so, outside the C ABI of
 * kvq.h. Nothing here is needed to use the library; the defaults are what
 * the decode entry points are tuned for.
 */
#ifndef KVQ_TESTING_H
#define KVQ_TESTING_H

#include <stdint.h>

#include "kvq.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Aim the context-split planner of this cache's decode calls at
 * `target_wgs` workgroups per launch (0 = the library default: 512 for GQA,
 * 256 for MLA). The value is kept in the host handle, so
 * kvq_decode_workspace_bytes and every decode entry point on this handle
 * plan the same splits until it is set again. Tests use it to force one
 * split (the direct output path) or many (up to the 128-split cap).
 * Errors: KVQ_ERR_ARG (null handle, target outside [0, 2^20]). */
int kvq_testing_set_split_target(kvq_cache* cache, int32_t target_wgs);

#ifdef __cplusplus
}
#endif
#endif /* KVQ_TESTING_H */
