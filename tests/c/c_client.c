/*
 * A C host program that runs one mla_post call through the HIP runtime's C
 * API alone (no Python, no torch): it reads the inputs of a dense split-KV
 * batch from a file, allocates and fills device memory, calls mla_post on
 * the default stream, and writes core back to a file.
 *
 *   c_client IN OUT
 *
 * IN : int32 n, int32 S, then o (n*S*12*512 bf16), lse (n*S*12 float32),
 *      W_V codes (12*128*256 u8), W_V scale codes (12*128*16 u8),
 *      gate (S*1536 bf16), all dense and little-endian.
 * OUT: core (S*1536 bf16).
 * Exit status 0 on success; any HIP or library error is printed and exits 1.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "mla_post.h"

#define HIP_OK(call)                                                       \
  do {                                                                     \
    hipError_t e_ = (call);                                                \
    if (e_ != hipSuccess) {                                                \
      fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));    \
      exit(1);                                                             \
    }                                                                      \
  } while (0)

static void* read_block(FILE* f, size_t bytes) {
  void* p = malloc(bytes ? bytes : 1);
  if (!p || fread(p, 1, bytes, f) != bytes) {
    fprintf(stderr, "short input file\n");
    exit(1);
  }
  return p;
}

static void* to_device(const void* host, size_t bytes) {
  void* d = NULL;
  HIP_OK(hipMalloc(&d, bytes ? bytes : 16));
  if (bytes) HIP_OK(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice));
  return d;
}

int main(int argc, char** argv) {
  int32_t hdr[2];
  FILE* f;
  size_t o_bytes, lse_bytes, wv_bytes, ws_bytes, g_bytes;
  void *o_h, *lse_h, *wv_h, *ws_h, *g_h, *core_h;
  void *o_d, *lse_d, *wv_d, *ws_d, *g_d, *core_d;
  mla_post_args a = {0};
  int st;

  if (argc != 3) {
    fprintf(stderr, "usage: %s IN OUT\n", argv[0]);
    return 2;
  }
  f = fopen(argv[1], "rb");
  if (!f || fread(hdr, sizeof hdr, 1, f) != 1) {
    fprintf(stderr, "cannot read %s\n", argv[1]);
    return 1;
  }
  if (hdr[0] < 1 || hdr[0] > MLA_POST_NMAX || hdr[1] < 0) {
    fprintf(stderr, "bad header n=%d S=%d\n", hdr[0], hdr[1]);
    return 1;
  }
  o_bytes = (size_t)hdr[0] * hdr[1] * MLA_POST_HEADS * MLA_POST_KVL * 2;
  lse_bytes = (size_t)hdr[0] * hdr[1] * MLA_POST_HEADS * 4;
  wv_bytes = (size_t)MLA_POST_HEADS * MLA_POST_VD * (MLA_POST_KVL / 2);
  ws_bytes = (size_t)MLA_POST_HEADS * MLA_POST_VD * (MLA_POST_KVL / 32);
  g_bytes = (size_t)hdr[1] * MLA_POST_GROWS * 2;
  o_h = read_block(f, o_bytes);
  lse_h = read_block(f, lse_bytes);
  wv_h = read_block(f, wv_bytes);
  ws_h = read_block(f, ws_bytes);
  g_h = read_block(f, g_bytes);
  fclose(f);

  o_d = to_device(o_h, o_bytes);
  lse_d = to_device(lse_h, lse_bytes);
  wv_d = to_device(wv_h, wv_bytes);
  ws_d = to_device(ws_h, ws_bytes);
  g_d = to_device(g_h, g_bytes);
  HIP_OK(hipMalloc(&core_d, g_bytes ? g_bytes : 16));

  /* dense split-KV partials [n, S, 12, 512] and LSEs [n, S, 12] */
  a.struct_size = (uint32_t)sizeof a;
  a.n = hdr[0];
  a.S = hdr[1];
  a.o = o_d;
  a.o_sj = (int64_t)hdr[1] * MLA_POST_HEADS * MLA_POST_KVL;
  a.o_st = MLA_POST_HEADS * MLA_POST_KVL;
  a.o_sh = MLA_POST_KVL;
  a.lse = (const float*)lse_d;
  a.l_sj = (int64_t)hdr[1] * MLA_POST_HEADS;
  a.l_st = MLA_POST_HEADS;
  a.l_sh = 1;
  a.w_v = (const uint8_t*)wv_d;
  a.w_sh = MLA_POST_VD * (MLA_POST_KVL / 2);
  a.w_sv = MLA_POST_KVL / 2;
  a.w_v_scale = (const uint8_t*)ws_d;
  a.s_sh = MLA_POST_VD * (MLA_POST_KVL / 32);
  a.s_sv = MLA_POST_KVL / 32;
  a.s_sb = 1;
  a.gate = g_d;
  a.core = core_d;

  st = mla_post(&a, NULL);
  if (st != MLA_POST_OK) {
    fprintf(stderr, "mla_post: %s %s\n", mla_post_strerror(st), mla_post_last_hip_error());
    return 1;
  }
  HIP_OK(hipDeviceSynchronize());

  core_h = malloc(g_bytes ? g_bytes : 1);
  if (!core_h) return 1;
  if (g_bytes) HIP_OK(hipMemcpy(core_h, core_d, g_bytes, hipMemcpyDeviceToHost));
  f = fopen(argv[2], "wb");
  if (!f || fwrite(core_h, 1, g_bytes, f) != g_bytes) {
    fprintf(stderr, "cannot write %s\n", argv[2]);
    return 1;
  }
  fclose(f);

  HIP_OK(hipFree(o_d));
  HIP_OK(hipFree(lse_d));
  HIP_OK(hipFree(wv_d));
  HIP_OK(hipFree(ws_d));
  HIP_OK(hipFree(g_d));
  HIP_OK(hipFree(core_d));
  free(o_h);
  free(lse_h);
  free(wv_h);
  free(ws_h);
  free(g_h);
  free(core_h);
  printf("c_client ok n=%d S=%d\n", hdr[0], hdr[1]);
  return 0;
}
