/*
 * mla_measure: a bandwidth reference for the benchmark of this library's
 * kernels on AMD MI355X (gfx950). Not a step of the computed path.
 *
 * The fused kernels are bound by HBM reads (mla_post reads its partial rows
 * once; everything else is small). A plain read of the same bytes, with the
 * same 16-byte non-temporal loads, measured on the same device in the same
 * run, is the tight ceiling they are compared with, next to AMD's published
 * 8 TB/s.
 *
 * Conventions as in mla_post.h (C linkage, caller-owned device memory,
 * asynchronous on the caller's stream, MLA_POST_* status codes).
 */
#ifndef MLA_MEASURE_H
#define MLA_MEASURE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Read `bytes` bytes at `p` (16-byte aligned, bytes a multiple of 16, at
 * most 2^40) once, with 16-byte non-temporal loads from every CU, and fold
 * them into a value that is stored to `sink` (16 bytes of device memory,
 * 16-byte aligned) only if it equals a constant no real data folds to, so
 * the loads cannot be dropped and nothing else is written in practice.
 * Returns MLA_POST_OK, MLA_POST_EINVAL, MLA_POST_EALIGN or MLA_POST_ELAUNCH.
 */
int mla_measure_read(const void* p, int64_t bytes, void* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_MEASURE_H */
