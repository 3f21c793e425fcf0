/*
 * mla_post: MLA decode post-attention on AMD MI355X (gfx950).
 *
 * The operation is the one the vLLM API-docs page for module
 * vllm.models.kimi_k3.amd.specialized_decode.mono.attention.mla_back
 * describes (module docstring; functions mla_post, host_args,
 * stage_combine, combine_splits, combine_ranks, sane, stage_uv, wv_loads).
 * For every token t < S and head h < 12:
 *
 *   1. merge the n bf16 partial rows o[j, t, h, 0:512] with their float32
 *      natural-log LSEs (NaN and +inf count as -inf; m = max LSE, 0 when all
 *      are -inf; w_j = exp(lse_j - m) / sum exp; a row of weight 0 is not
 *      read and contributes nothing). With n == 1 and lse == NULL the row is
 *      the final attention output and is used as is;
 *   2. round the float32 sum to bf16 latents (round to nearest even);
 *   3. quantise each block of 32 latents to MXFP4: E8M0 scale code
 *      c = max(1, Eb(amax) + [mantissa fraction of amax >= 0.75] - 2), amax
 *      the largest bf16 magnitude in the block; E2M1 elements of x / 2^(c-127)
 *      rounded to nearest, ties to the even code, saturating at 6, sign kept;
 *   4. multiply by the head's MXFP4 W_V[h] (128 x 512) with scaled FP4 MFMA
 *      (float32 accumulation);
 *   5. core[t, 128 h + v] = bf16( bf16(acc[v]) * gate[t, 128 h + v] ).
 *
 * All entry points are host functions with C linkage. Device pointers are
 * caller-owned device memory; the library keeps no pointer after a call
 * returns and allocates nothing per call. Its only mutable global state is a
 * per-device cache of the compute-unit count (asked of the runtime on first
 * use, then only read; atomic) and a per-thread copy of the last HIP launch
 * error's message (mla_post_last_hip_error). Neither carries data from one
 * call into another's results, so calls are thread-safe, and calls on
 * different streams may run at the same time. Work is enqueued
 * asynchronously on the caller's HIP stream. Validation failures are
 * reported synchronously, launch nothing and leave every output untouched.
 */
#ifndef MLA_POST_H
#define MLA_POST_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_POST_VERSION 5

/* Fixed shapes (the page's per-rank Kimi-K3 shapes at 8-way tensor parallelism). */
#define MLA_POST_HEADS 12   /* local heads */
#define MLA_POST_KVL 512    /* latent width */
#define MLA_POST_VD 128     /* W_V rows (value width) per head */
#define MLA_POST_GROWS 1536 /* gate / core row length = 12 * 128 */
#define MLA_POST_NMAX 512   /* largest number of partials per (token, head) */
#define MLA_POST_SMAX (1 << 30) /* largest number of tokens per call */

/* Status codes (0 = success, negative = error). */
#define MLA_POST_OK 0
#define MLA_POST_EINVAL (-1)       /* null pointer, bad size (S above MLA_POST_SMAX among them), lse NULL with n > 1 */
#define MLA_POST_ESTRIDE (-2)      /* a stride that is negative or not a multiple the loads need */
#define MLA_POST_EALIGN (-3)       /* a pointer not aligned as its loads or stores need */
#define MLA_POST_ERANGE (-4)       /* an offset that overflows 64-bit arithmetic */
#define MLA_POST_EUNSUPPORTED (-5) /* n > MLA_POST_NMAX, or cols not a multiple of 32 */
#define MLA_POST_ELAUNCH (-6)      /* the HIP runtime refused the launch (message: mla_post_last_hip_error) */

/*
 * Arguments of one mla_post call. Strides of o and lse are in elements; those
 * of w_v and w_v_scale are in bytes. The partial row j of (t, h) is the 512
 * contiguous bf16 at o + j*o_sj + t*o_st + h*o_sh (the innermost stride is 1,
 * as the page's host_args asserts). One layout covers the three cases the page
 * names:
 *   - split-KV partials, dense [n, S, 12, 512]: (o_sj, o_st, o_sh) = (S*6144, 6144, 512);
 *   - decode-context-parallel partials gathered on one GPU, o [S, >= n*12, 512]
 *     with rank r's partial of local head h at gathered head r*12 + h:
 *     (o_sj, o_st, o_sh) = (12*512, head_rows*512, 512);
 *   - one partial, no LSE (n == 1, lse == NULL): o [S, 12, 512].
 * A row whose merge weight is 0 (LSE -inf, NaN or +inf, or masked below)
 * never contributes, whatever it holds (NaN and inf included). The kernels
 * skip loading most such rows but not all (the small-batch kernel loads a
 * token's rows together with its LSEs), so every row j < n of every token
 * t < S must lie in readable device memory.
 */
typedef struct mla_post_args {
  uint32_t struct_size; /* sizeof(mla_post_args), or MLA_POST_ARGS_V1_SIZE */
  int32_t n;            /* partials per (token, head): splits or ranks, 1..MLA_POST_NMAX */
  int32_t S;            /* tokens, 0..MLA_POST_SMAX; 0 is a no-op */
  int32_t reserved;

  const void* o;            /* bf16 partials, device, 16-byte aligned */
  int64_t o_sj, o_st, o_sh; /* >= 0, multiples of 8 elements */

  const float* lse;         /* float32 LSEs, device, or NULL only when n == 1 */
  int64_t l_sj, l_st, l_sh; /* >= 0 */

  const uint8_t* w_v;  /* MXFP4 W_V codes, logical (12, 128, 256) bytes: byte of
                          (h, v, k) at w_v + h*w_sh + v*w_sv + k/2, element 2i
                          in the low nibble of byte i; 16-byte aligned */
  int64_t w_sh, w_sv;  /* bytes, >= 0, multiples of 16 */

  const uint8_t* w_v_scale;  /* E8M0 scales, logical (12, 128, 16): byte of
                                (h, v, b) at + h*s_sh + v*s_sv + b*s_sb */
  int64_t s_sh, s_sv, s_sb;  /* bytes, >= 0 */

  const void* gate; /* bf16 [S, 1536] dense, 16-byte aligned */
  void* core;       /* bf16 [S, 1536] dense, 16-byte aligned; every row t < S is
                       written, nothing else is */

  /* Optional stage outputs (NULL to skip), written by the same kernel with
   * the same arithmetic: latents bf16 [S, 12, 512] (16-byte aligned), MXFP4
   * latent codes u8 [S, 12, 256] (4-byte aligned), E8M0 latent scale codes
   * u8 [S, 12, 16]. */
  void* dbg_lat;
  void* dbg_codes;
  void* dbg_scales;

  /* ---- since version 2; a caller whose struct_size ends above leaves them off.
   * Request-major split slices and push-side masking (the page's
   * combine_splits addressing and stage_push masking). With R = S / q requests
   * of q consecutive tokens, token t belongs to request r = t / q:
   *   row (j, t, h) = o + j*o_sj + r*o_sr + t*o_st + h*o_sh,
   *   LSE (j, t, h) = lse + j*l_sj + r*l_sr + t*l_st + h*l_sh.
   * The page's dense layout of per = P / R slices per request in one tensor
   * [P, S, 12, 512] is (o_sj, o_sr, o_st) = (S*6144, per*S*6144, 6144) with
   * n = per. Partial j of token t is empty (LSE taken as -inf, its row never
   * used) when kv_lens[j*kl_sj + r] == 0, or for every j when t >= qsl[R]. */
  int32_t q;              /* tokens per request; 0 or 1 = one token each. S % q == 0 */
  int32_t reserved2;
  int64_t o_sr, l_sr;     /* elements per request index, >= 0; o_sr a multiple of 8 */
  const int32_t* kv_lens; /* NULL, or int32 KV lengths, entry (j, r) at j*kl_sj + r; 4-byte aligned */
  int64_t kl_sj;          /* >= 0; 0 shares one row of R lengths among all partials */
  const int32_t* qsl;     /* NULL, or int32 [R + 1] query start offsets; tokens >= qsl[R] are past the batch */
} mla_post_args;

/* Size of the version-1 prefix of mla_post_args (fields up to dbg_scales). */
#define MLA_POST_ARGS_V1_SIZE 176

/* Validate and enqueue one mla_post call on `stream` (a hipStream_t; NULL is
 * the default stream). Returns MLA_POST_OK or a negative status. */
int mla_post(const mla_post_args* a, void* stream);

/* The validation of mla_post alone: host only, touches no device memory and
 * needs no GPU. Returns what mla_post would return before launching. */
int mla_post_check(const mla_post_args* a);

/* Since version 3: the launch mla_post makes for a call. */
#define MLA_POST_KERNEL_NONE 0       /* S == 0: nothing is launched */
#define MLA_POST_KERNEL_ONE_TILE 1   /* one token tile per workgroup, every load issued up front */
#define MLA_POST_KERNEL_PERSISTENT 2 /* workgroups that each keep one head and walk its tiles */
#define MLA_POST_KERNEL_SPLIT_ROWS 3 /* one small token tile per workgroup, 8 / tile_tokens waves sharing the
                                        partials of each token (many partials, few tokens) */
#define MLA_POST_KERNEL_STREAM 4     /* since version 4: workgroups that each keep one head and walk its tiles,
                                        loading each tile's rows two tiles ahead straight into LDS (one or
                                        two partials, many tokens); since version 5 two per CU */

typedef struct mla_post_plan {
  int32_t kernel;              /* MLA_POST_KERNEL_* */
  int32_t tile_tokens;         /* tokens of a full tile: 8 or 16 (split-rows kernel: 1, 2 or 4; streaming
                                  kernel: 16 / n) */
  int32_t rows_held;           /* one-tile kernel: partial rows per token held at once (1, 2, 4, 8 or 16);
                                  split-rows kernel: rows each wave holds at once (8 or 16); streaming
                                  kernel: n; else 0 */
  int32_t lse_chunks;          /* persistent and split-rows kernels: 64-lane chunks of partials per token
                                  (1, 2, 4 or 8); else 1 */
  int32_t workgroups_per_head; /* the grid is 12 times this, except for the streaming kernel (since version
                                  5): its grid is `workgroups`, workgroup b taking head b mod 12; heads
                                  h < workgroups mod 12 have workgroups_per_head workgroups, the others
                                  one fewer */
  int32_t workgroups;          /* grid size (workgroups of 512 threads) */
  int32_t full_tiles;          /* persistent and streaming kernels: full tiles of every workgroup (streaming
                                  kernel: of a head with workgroups_per_head workgroups) */
  int32_t short_tokens;        /* persistent and streaming kernels: tokens of one more, shorter tile per
                                  workgroup (at most tile_tokens; the last workgroups of a head may get
                                  fewer or none); 0: none */
  int32_t pair_rows;           /* persistent kernel: rows of each of a wave's two tokens issued a tile ahead
                                  (4, for n <= 4 with LSEs); 0: 8 rows of its first token only */
  int32_t cus;                 /* compute units the plan was made for */
} mla_post_plan;

/* Since version 3: validate like mla_post_check and, on MLA_POST_OK, fill
 * *out with the launch mla_post would make for these arguments on a device
 * with `cus` compute units (cus <= 0: the current HIP device, asked of the
 * runtime once; 256 when it cannot tell). Host only; touches no device
 * memory and needs no GPU when cus > 0. Returns a status code; out == NULL
 * is MLA_POST_EINVAL. */
int mla_post_plan_for(const mla_post_args* a, int32_t cus, mla_post_plan* out);

/*
 * Quantise `rows` rows of `cols` bf16 values (cols a multiple of 32, at most
 * 8192) to MXFP4 with the same rule as step 3 above: row r's values at
 * x + r*x_stride (elements, 16-byte aligned rows), its codes (cols/2 bytes) to
 * codes + r*c_stride and its E8M0 scale codes (cols/32 bytes) to
 * scales + r*s_stride (bytes). This is how W_V is put into MXFP4 from bf16.
 * Asynchronous on `stream`; same status codes (rows above 2^34 give
 * MLA_POST_ERANGE).
 */
int mla_quantize_mxfp4(const void* x, int64_t rows, int32_t cols, int64_t x_stride, uint8_t* codes,
                       int64_t c_stride, uint8_t* scales, int64_t s_stride, void* stream);

/* Static description of a status code. */
const char* mla_post_strerror(int status);

/* The HIP error string of the last MLA_POST_ELAUNCH on this thread, or "". */
const char* mla_post_last_hip_error(void);

/* MLA_POST_VERSION of the library. */
int mla_post_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_POST_H */
