/*
 * C client of the mla_post library, host side only (no GPU needed): built
 * with a plain C compiler against include/mla_post.h, it prints the struct
 * layout as C sees it and the statuses that validation gives for a set of
 * argument structs, so a test can compare them with the header's contract
 * and with the Python binding's struct. Device addresses are fake: nothing
 * is dereferenced and nothing is launched (every call below either fails
 * validation or has S == 0).
 */
#include <stddef.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "mla_post.h"

#define FIELD(name) printf("offset %s %zu\n", #name, offsetof(mla_post_args, name))
#define PFIELD(name) printf("plan_offset %s %zu\n", #name, offsetof(mla_post_plan, name))

static mla_post_args good(int n, int S) {
  mla_post_args a;
  memset(&a, 0, sizeof a);
  a.struct_size = (uint32_t)sizeof(mla_post_args);
  a.n = n;
  a.S = S;
  a.o = (const void*)(uintptr_t)0x100000;
  a.o_sj = (int64_t)S * 6144;
  a.o_st = 6144;
  a.o_sh = 512;
  a.lse = (const float*)(uintptr_t)0x200000;
  a.l_sj = (int64_t)S * 12;
  a.l_st = 12;
  a.l_sh = 1;
  a.w_v = (const uint8_t*)(uintptr_t)0x300000;
  a.w_sh = 128 * 256;
  a.w_sv = 256;
  a.w_v_scale = (const uint8_t*)(uintptr_t)0x400000;
  a.s_sh = 128 * 16;
  a.s_sv = 16;
  a.s_sb = 1;
  a.gate = (const void*)(uintptr_t)0x500000;
  a.core = (void*)(uintptr_t)0x600000;
  return a;
}

static void status(const char* name, int st) { printf("status %s %d %s\n", name, st, mla_post_strerror(st)); }

int main(void) {
  mla_post_args a;

  printf("sizeof %zu\n", sizeof(mla_post_args));
  printf("v1_size %d\n", MLA_POST_ARGS_V1_SIZE);
  printf("header_version %d\n", MLA_POST_VERSION);
  printf("library_version %d\n", mla_post_version());
  FIELD(struct_size); FIELD(n); FIELD(S); FIELD(reserved);
  FIELD(o); FIELD(o_sj); FIELD(o_st); FIELD(o_sh);
  FIELD(lse); FIELD(l_sj); FIELD(l_st); FIELD(l_sh);
  FIELD(w_v); FIELD(w_sh); FIELD(w_sv);
  FIELD(w_v_scale); FIELD(s_sh); FIELD(s_sv); FIELD(s_sb);
  FIELD(gate); FIELD(core); FIELD(dbg_lat); FIELD(dbg_codes); FIELD(dbg_scales);
  FIELD(q); FIELD(reserved2); FIELD(o_sr); FIELD(l_sr); FIELD(kv_lens); FIELD(kl_sj); FIELD(qsl);

  a = good(4, 8);
  status("valid", mla_post_check(&a));
  status("null_struct", mla_post_check(NULL));
  a = good(4, 8); a.o = NULL;
  status("null_o", mla_post_check(&a));
  a = good(4, 8); a.lse = NULL;
  status("null_lse_n4", mla_post_check(&a));
  a = good(1, 8); a.lse = NULL;
  status("null_lse_n1", mla_post_check(&a));
  a = good(4, 8); a.o_st = 6143;
  status("odd_o_stride", mla_post_check(&a));
  a = good(4, 8); a.core = (void*)(uintptr_t)0x600008;
  status("misaligned_core", mla_post_check(&a));
  a = good(MLA_POST_NMAX + 1, 8);
  status("n_too_large", mla_post_check(&a));
  a = good(4, 8); a.S = -1;
  status("negative_S", mla_post_check(&a));
  a = good(4, 8); a.q = 3;
  status("q_not_dividing_S", mla_post_check(&a));
  a = good(4, 8); a.struct_size = MLA_POST_ARGS_V1_SIZE; a.q = 3;
  status("v1_ignores_q", mla_post_check(&a));
  a = good(4, 8); a.struct_size = 8;
  status("struct_too_small", mla_post_check(&a));

  /* mla_post itself: validation is synchronous and launches nothing */
  a = good(4, 8); a.o_st = 6143;
  status("launch_odd_o_stride", mla_post(&a, NULL));
  a = good(4, 0);
  status("launch_empty", mla_post(&a, NULL));
  status("quantize_bad_cols", mla_quantize_mxfp4((const void*)(uintptr_t)0x100000, 4, 33, 64,
                                                 (uint8_t*)(uintptr_t)0x200000, 32,
                                                 (uint8_t*)(uintptr_t)0x300000, 2, NULL));
  printf("last_hip_error '%s'\n", mla_post_last_hip_error());

  /* the launch plan, for 256 CUs (host only) */
  {
    mla_post_plan p;
    printf("plan_sizeof %zu\n", sizeof(mla_post_plan));
    PFIELD(kernel); PFIELD(tile_tokens); PFIELD(rows_held); PFIELD(lse_chunks); PFIELD(workgroups_per_head);
    PFIELD(workgroups); PFIELD(full_tiles); PFIELD(short_tokens); PFIELD(pair_rows); PFIELD(cus);
    a = good(16, 4096);
    status("plan_large", mla_post_plan_for(&a, 256, &p));
    printf("plan_large %d %d %d %d\n", p.kernel, p.workgroups, p.full_tiles, p.cus);
    a = good(2, 4);
    status("plan_tiny", mla_post_plan_for(&a, 256, &p));
    printf("plan_tiny %d %d %d %d\n", p.kernel, p.tile_tokens, p.rows_held, p.workgroups);
    a = good(4, 8); a.o_st = 6143;
    status("plan_bad_stride", mla_post_plan_for(&a, 256, &p));
    status("plan_null_out", mla_post_plan_for(&a, 256, NULL));
  }
  return 0;
}
