/*
 * mla_decode: split-KV MLA decode attention fused with mla_post on AMD
 * MI355X (gfx950), one launch.
 *
 * The vLLM API-docs page for module
 * vllm.models.kimi_k3.amd.specialized_decode.mono.attention.mla_back names
 * the producer of mla_post's split partials (module docstring: M1c's
 * mla_attn writes o / lse per KV split; combine_splits: a token merges its
 * request's splits, request-major) and a launch that runs that producer and
 * the merge + W_UV together (module docstring: K2; combine_splits polls the
 * producer's per-split ready flags; combine_tasks / stage_uv: core stored at
 * device scope). The page does not show the attention itself; this library
 * computes the plainest split-KV MLA decode attention with those outputs:
 *
 *   for request r (q consecutive tokens, KV rows kv[indptr[r] .. indptr[r+1])),
 *   split j < n covering its rows floor(j L / n) .. floor((j+1) L / n) - 1,
 *   token t of r and head h:
 *     s_i    = scale * (qry[t, h, 0:576] . kv[i, 0:576])      (absorbed MLA:
 *              512 latent + 64 rotary dims; all heads share the cache row)
 *     o_j    = bf16( sum_i softmax_j(s)_i kv[i, 0:512] )      (float32 sums)
 *     lse_j  = ln sum_i exp(s_i)                              (float32)
 *   an empty split: o_j = 0, lse_j = -inf;
 *
 * and then, for every token and head, exactly mla_post's steps on those n
 * partials (include/mla_post.h: merge, bf16 latents, MXFP4, W_UV, gate).
 *
 * The handoff is this library's own, not the page's: no workgroup ever
 * waits for another. The launch has two workgroups per CU (fewer when there
 * are fewer units); each takes (request, split) units in order, its first
 * by its block index and each later one from a queue counter in the
 * workspace (a vector atomic at device scope), until none is left, then
 * counts itself out on a second counter; the last one out sets both back
 * to 0. After a unit's attention the workgroup writes its partials to the
 * workspace with stores that go through to the device's coherence point
 * (device-scope cache policy), waits for them to complete, then adds 1 to
 * its request's counter; the workgroup that brings the counter to n reads
 * that request's partials with loads of the same policy, merges them and
 * runs W_UV for its tokens, then sets the counter back to 0. So the launch
 * cannot deadlock whatever order or placement its workgroups get, and a
 * call leaves the counters as it found them.
 *
 * Conventions as in mla_post.h (C linkage, caller-owned device memory,
 * asynchronous on the caller's stream, MLA_POST_* status codes, validation
 * errors launch nothing).
 */
#ifndef MLA_DECODE_H
#define MLA_DECODE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_DECODE_DQK 576    /* query / cache row width: 512 latent + 64 rotary */
#define MLA_DECODE_QMAX 4     /* most query tokens per request */
#define MLA_DECODE_NMAX 64    /* most KV splits per request */

typedef struct mla_decode_args {
  uint32_t struct_size; /* sizeof(mla_decode_args) */
  int32_t R;            /* requests, >= 0 (0: no-op) */
  int32_t q;            /* query tokens per request, 1..MLA_DECODE_QMAX; S = R * q */
  int32_t n;            /* KV splits per request, 1..MLA_DECODE_NMAX */

  const void* qry;        /* bf16 queries: token t, head h at qry + t*q_st + h*q_sh (576 contiguous); 16-byte aligned */
  int64_t q_st, q_sh;     /* elements, >= 0, multiples of 8 */
  const void* kv;         /* bf16 cache: row i at kv + i*kv_st (576 contiguous); 16-byte aligned */
  int64_t kv_st;          /* elements, >= 576, a multiple of 8 */
  const int32_t* indptr;  /* int32 [R + 1], non-decreasing: request r's rows indptr[r] .. indptr[r+1] - 1 */
  float scale;            /* softmax scale applied to the dot products */
  int32_t reserved;

  const uint8_t* w_v;       /* as mla_post_args: MXFP4 W_V, logical (12, 128, 256), 16-byte aligned */
  int64_t w_sh, w_sv;       /* bytes, multiples of 16 */
  const uint8_t* w_v_scale; /* E8M0 scales, logical (12, 128, 16) */
  int64_t s_sh, s_sv, s_sb; /* bytes */
  const void* gate;         /* bf16 [S, 1536] dense, 16-byte aligned */
  void* core;               /* bf16 [S, 1536] dense, 16-byte aligned: every row written */

  void* workspace;         /* device memory of mla_decode_workspace's size, 256-byte aligned; its
                              counters must be zero before the first call (mla_decode_workspace_init)
                              and are zero again after every call. Counters that are not zero give
                              wrong or missing results, never an access outside the arguments'
                              buffers: a queue value outside the batch names no unit */
  int64_t workspace_bytes;

  /* optional stage outputs of the merge (NULL to skip), as mla_post's:
   * latents bf16 [S, 12, 512], codes u8 [S, 12, 256], scale codes u8 [S, 12, 16] */
  void* dbg_lat;
  void* dbg_codes;
  void* dbg_scales;
} mla_decode_args;

/* Workspace bytes for R requests of q tokens and n splits, and where its
 * parts start (byte offsets): counters int32 [R + 2] (one per request, then
 * the unit queue's two); partials bf16
 * [R, n, q, 12, 512] (split j of token t = r q + tt, head h at row
 * ((r n + j) q + tt) 12 + h); LSEs float32 [R, n, q, 12] (same order).
 * After a call the partials and LSEs of that call stay there. Any output
 * pointer may be NULL. Host only. */
int mla_decode_workspace(int32_t R, int32_t q, int32_t n, int64_t* bytes, int64_t* off_counters,
                         int64_t* off_partials, int64_t* off_lse);

/* Zero the workspace's R + 2 counters (a small fill kernel on `stream`; no
 * memset, so it may be captured in a graph). Needed once, before the first
 * call (mla_decode or mla_decode_partials) on a new workspace. */
int mla_decode_workspace_init(void* workspace, int32_t R, void* stream);

/* One launch: the split-KV attention of every (request, split) and, in the
 * same kernel, mla_post of every request's tokens (the handoff above). */
int mla_decode(const mla_decode_args* a, void* stream);

/* The attention alone: every (request, split) partial and LSE into the
 * workspace, nothing merged (the request counters untouched, the queue's
 * used and left at 0; core not written). With
 * mla_post on the workspace's partials (request-major: n = n, q = q,
 * o_sj = q*6144, o_sr = (n-1)*q*6144, o_st = 6144, o_sh = 512, and the same
 * strides over the LSEs divided by 512) it gives the same core as
 * mla_decode, in two launches. */
int mla_decode_partials(const mla_decode_args* a, void* stream);

/* The validation of mla_decode alone: host only, touches no device memory. */
int mla_decode_check(const mla_decode_args* a);

/* Size of the library's own device scratch array for mla_decode_noalloc. */
#define MLA_DECODE_SCRATCH_BYTES (64ll << 20)

/*
 * mla_decode without a caller workspace and without any allocation, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc). The workspace is a
 * file-scope device array of MLA_DECODE_SCRATCH_BYTES (64 MiB) that every GPU
 * the library runs on holds until the process ends; its address is asked of
 * the runtime once per device. a->workspace must be NULL (workspace_bytes is
 * ignored). Calls whose workspace (mla_decode_workspace) exceeds the array
 * return MLA_POST_EUNSUPPORTED and launch nothing. Each call first clears the
 * array's counters with a small fill kernel on `stream`, then makes the fused
 * launch; the partials and LSEs stay in the array until the next call. All
 * calls on one GPU share the array: calls that overlap on one GPU (other
 * streams, other threads) race, and must be ordered by the caller.
 * Calls no hipMalloc, hipFree or allocating routine. Same results as
 * mla_decode with a workspace, bit for bit.
 */
int mla_decode_noalloc(const mla_decode_args* a, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_H */
