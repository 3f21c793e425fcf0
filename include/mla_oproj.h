/*
 * mla_oproj: o_proj, the consumer of mla_post's core, on AMD MI355X (gfx950).
 *
 * The vLLM API-docs page for module
 * vllm.models.kimi_k3.amd.specialized_decode.mono.attention.mla_back
 * describes its path as running from the attention's decode output to
 * o_proj's input (module docstring): core [S, 1536] bf16, one
 * tensor-parallel rank's 12 heads x 128 columns, is that input. The page
 * says nothing more about o_proj. This library takes it as a bias-free
 * linear layer over those columns:
 *
 *   out[t, d] = bf16( sum_k core[t, k] * w_o[d, k] ),  t < S, d < D, k < K,
 *
 * with W_O in the linear layer's [D, K] row-major layout, bf16 operands,
 * float32 accumulation (bf16 matrix-core instructions) and one rounding to
 * bf16 (round to nearest even). Under tensor parallelism each rank's out is a
 * partial sum that an all-reduce completes; that reduction is not part of
 * this one-GPU library.
 *
 * Conventions as in mla_post.h: host functions with C linkage; caller-owned
 * device memory; nothing allocated or kept; asynchronous on the caller's
 * stream; the status codes are mla_post.h's MLA_POST_*; validation errors
 * launch nothing and leave out untouched.
 */
#ifndef MLA_OPROJ_H
#define MLA_OPROJ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_OPROJ_KMAX 16384 /* largest K accepted */

/*
 * Enqueue out = bf16(core @ w_o^T) on `stream` (a hipStream_t; NULL is the
 * default stream).
 *   core   bf16 [S, K]: row t at core + t*core_stride elements; 16-byte aligned
 *   w_o    bf16 [D, K]: row d at w_o + d*w_stride elements; 16-byte aligned
 *   out    bf16 [S, D]: row t at out + t*out_stride elements; 16-byte aligned;
 *          every element (t < S, d < D) is written, nothing else is
 * S >= 0 (0: no-op), D >= 1 a multiple of 8, K >= 64 a multiple of 64 and at
 * most MLA_OPROJ_KMAX (K = 1536 for core). Strides are in elements, >= 0 and
 * multiples of 8.
 * Returns MLA_POST_OK, MLA_POST_EINVAL (null pointer, sizes out of range),
 * MLA_POST_ESTRIDE, MLA_POST_EALIGN, MLA_POST_ERANGE (offsets overflow
 * 64-bit arithmetic), MLA_POST_EUNSUPPORTED (D or K not a multiple of 8 or
 * 64, K above MLA_OPROJ_KMAX) or MLA_POST_ELAUNCH.
 */
int mla_oproj(const void* core, int64_t core_stride, int32_t S, int32_t K, const void* w_o, int64_t w_stride,
              int32_t D, void* out, int64_t out_stride, void* stream);

/* The validation of mla_oproj alone: host only, touches no device memory. */
int mla_oproj_check(const void* core, int64_t core_stride, int32_t S, int32_t K, const void* w_o,
                    int64_t w_stride, int32_t D, const void* out, int64_t out_stride);

/* The launch mla_oproj makes for S x D on a device of `cus` compute units
 * (cus <= 0: the current device): *tile_m x *tile_n outputs per workgroup (of
 * 512 threads for 256 x 256 tiles, else 256), *workgroups in the grid. Host
 * only. Returns a status code. */
int mla_oproj_plan(int32_t S, int32_t D, int32_t cus, int32_t* tile_m, int32_t* tile_n, int32_t* workgroups);

#ifdef __cplusplus
}
#endif

#endif /* MLA_OPROJ_H */
