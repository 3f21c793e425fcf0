// mla_post: fused MLA decode post-attention for AMD MI355X (gfx950 / CDNA4).
//
// One launch does the whole path the vLLM API-docs page for module
// vllm.models.kimi_k3.amd.specialized_decode.mono.attention.mla_back
// describes (module docstring; stage_combine, combine_splits, combine_ranks,
// sane, stage_uv, wv_loads): LSE merge of bf16 partial rows -> bf16 latents
// -> MXFP4 -> scaled FP4 MFMA against W_V[h] -> bf16 x gate -> core.
//
// Decomposition (this library's own, not the page's):
//   workgroup = 8 waves of 64 lanes that own one head h for the whole launch
//     and walk its 16-token tiles (k workgroups per head, WG_PER_CU per CU
//     in the grid); W_V[h]'s operands stay in registers throughout; the 12
//     heads of one token tile run as consecutive workgroups of one XCD, so
//     they read each (token, split) 12 KiB block together behind one L2;
//   merge: per tile, wave w owns tokens 2w and 2w+1; a token's partial row
//     is 1 KiB = 64 lanes x 16 B, so each row is one coalesced non-temporal
//     16-byte load per lane, ROWS_IN_FLIGHT rows in flight, rows of weight 0
//     not loaded (but for the first rows of a workgroup's first tile, issued
//     with its LSEs); software-pipelined over tiles: before the barrier of a
//     tile a wave computes the next tile's weights (LSEs loaded a tile
//     earlier, DPP reductions) and issues that tile's first rows, so it
//     keeps loads in flight through the barrier and the MFMAs;
//   the merged latents never go to memory: each lane rounds its 8 latents
//     to bf16, the 4 lanes of a 32-element block agree on the E8M0 code with
//     two DPP steps, and the hardware scaled convert packs the 8 FP4 codes;
//     codes and scales go to (double-buffered) LDS as the MFMA B operand;
//   W_UV: wave w multiplies W_V[h] rows 16w..16w+15 (A operand) by the 16
//     tokens' latent codes, four 16x16x128 scaled FP4 MFMAs over K = 512, so
//     all 16 MFMA columns carry live tokens (the page fills 4 of 16);
//   epilogue: bf16(acc) x gate -> bf16 tiles are held in LDS and written
//     when the workgroup's tiles are done: 16-byte non-temporal stores,
//     tokens < S only.
// Small batches (one token tile per workgroup fills the device at most once;
// n <= 16 with 8-token tiles, n <= 8 with 16-token tiles) take a one-tile
// instance that issues every load up front, with 8-token tiles while that
// grid is at most 3 workgroups per CU.

#include <hip/hip_runtime.h>

#include <stdint.h>

#include <string.h>

#include <algorithm>
#include <string>

#include "device.h"
#include "launch.h"
#include "mla_post.h"
#include "post_common.h"

namespace {

constexpr int NH = MLA_POST_HEADS;
constexpr int KVL = MLA_POST_KVL;
constexpr int VD = MLA_POST_VD;
constexpr int GROWS = MLA_POST_GROWS;
constexpr int TILE_T = 16;                     // tokens per workgroup (MFMA N)
constexpr int WAVES = VD / 16;                 // 8 waves x 16 W_V rows
constexpr int THREADS = WAVES * 64;            // 512
constexpr int TOK_PER_WAVE = TILE_T / WAVES;   // 2
constexpr int ROWS_IN_FLIGHT = 8;              // partial rows a wave loads before it sums
constexpr int PF_ROWS = ROWS_IN_FLIGHT;        // first rows of the next tile issued before the barrier
constexpr bool NT_ROWS = true;                 // partial rows loaded non-temporally
constexpr int WG_PER_CU = 3;                   // workgroups per CU in the grid (2 resident at a time)
constexpr int NBLK = KVL / 32;                 // 16 MXFP4 blocks per latent row
constexpr int CODE_ROW = TILE_T * 16 + 16;     // LDS bytes per block row (+16 B skew)
constexpr int LDS_CODES = NBLK * CODE_ROW;     // 4352 B per buffer
constexpr int LDS_SCALES = TILE_T * NBLK;      // 256 B per buffer
constexpr int OUT_ROW = VD * 2 + 16;           // LDS bytes per token of the output tile (+16 B skew)
constexpr int LDS_OUT = TILE_T * OUT_ROW;      // 4352 B
constexpr int STORE_LANES = TILE_T * VD * 2 / 16;  // 256 16-byte pieces per output tile
constexpr int OUT_TILES = 8;                   // output tiles held in LDS before they are written
constexpr int SPREAD_MIN_N = 6;                // n from which leftover tokens are dealt out evenly
constexpr int ONE_TILE_SMAX = 1 << 20;         // largest S sent to the one-tile instance beyond its fill

struct KArgs {
  const uint8_t* o;
  int64_t o_sj, o_st, o_sh;  // bytes
  const float* lse;
  int64_t l_sj, l_st, l_sh;  // elements
  const uint8_t* w_v;
  int64_t w_sh, w_sv;
  const uint8_t* w_vs;
  int64_t s_sh, s_sv, s_sb;
  const uint8_t* gate;
  uint8_t* core;
  uint8_t* dbg_lat;
  uint8_t* dbg_codes;
  uint8_t* dbg_scales;
  int32_t n, S;
  int32_t q;                // tokens per request, >= 1
  int64_t o_sr;             // bytes per request index
  int64_t l_sr;             // elements per request index
  const int32_t* kv_lens;   // NULL or (j, r) at j * kl_sj + r
  int64_t kl_sj;
  const int32_t* qsl;       // NULL or [S / q + 1]
};

// The LSEs and KV lengths of one (t, h) as they are stored, one per lane:
// lane j of chunk c takes partial 64c + j. Every lane issues the same two
// loads on every path (lanes past n re-read partial n - 1; without KV
// lengths the second load re-reads the first LSE, and its value is ignored),
// so the number of loads in flight is fixed and nothing waits for the values
// here: finish_lse sanitises and masks them when they are used.
template <int NCH>
__device__ __forceinline__ void issue_lse(const KArgs& a, int t, int h, int lane, float x[NCH], int kv[NCH]) {
  const int r = t / a.q;
  const bool masked = a.kv_lens != nullptr;
  const int32_t* kvp = masked ? a.kv_lens : reinterpret_cast<const int32_t*>(a.lse);
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int j = min(64 * c + lane, a.n - 1);
    x[c] = a.lse[(int64_t)j * a.l_sj + (int64_t)r * a.l_sr + (int64_t)t * a.l_st + (int64_t)h * a.l_sh];
    kv[c] = kvp[masked ? (int64_t)j * a.kl_sj + r : 0];
  }
}

// Raw LSEs from issue_lse -> sanitised and masked: NaN / +inf -> -inf
// ([mla_back: sane]), -inf past n and for partials whose request has no KV
// ([mla_back: stage_push]).
template <int NCH>
__device__ __forceinline__ void finish_lse(const KArgs& a, int lane, float x[NCH], const int kv[NCH]) {
  const bool masked = a.kv_lens != nullptr;
#pragma unroll
  for (int c = 0; c < NCH; ++c) x[c] = (64 * c + lane < a.n && !(masked && kv[c] == 0)) ? sane(x[c]) : -INFINITY;
}

// One 1 KiB partial row: 16 B per lane. The rows are read once, so they are
// loaded non-temporally and do not push W_V out of L2.
// The row start p is the same for the whole wave: it goes into a scalar
// buffer resource that covers exactly the row's 1024 bytes, and the lane's
// 16 bytes are fetched at offset 16 lane (one vector register for every row,
// instead of a 64-bit address per row; an offset past the row would read 0).
__device__ __forceinline__ uint4 load_row16(const uint8_t* p, int lane) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p), (short)0, KVL * 2, BUF_WORD3);
  const v4u t = (v4u)__builtin_amdgcn_raw_buffer_load_b128(r, lane * 16, 0, NT_ROWS ? 2 : 0);  // 2: nt
  return make_uint4(t.x, t.y, t.z, t.w);
}

// Rows j0 .. j0 + R - 1 of chunk c of one (t, h): one 16-byte piece per lane
// each, and their wave-uniform weights. A row of weight 0, or past n, is
// loaded through a buffer resource of zero bytes, which returns zeros without
// touching memory, so every call issues exactly R loads: the number of loads
// in flight never depends on the data, and later waits (the gate, W_V) can
// leave them in flight.
template <int R>
__device__ __forceinline__ void issue_rows(const KArgs& a, const uint8_t* rowbase, int lane, int wbits, int c, int j0,
                                           uint4 v[R], float w[R]) {
  const int nc = min(64, a.n - 64 * c);
#pragma unroll
  for (int b = 0; b < R; ++b) {
    const int jl = j0 + b;
    int wb = __builtin_amdgcn_readlane(wbits, jl & 63);
    if (jl >= nc) wb = 0;
    w[b] = __int_as_float(wb);
    const uint8_t* p = rowbase + (int64_t)(64 * c + min(jl, nc - 1)) * a.o_sj;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(p), (short)0, (wb & 0x7FFFFFFF) ? KVL * 2 : 0, BUF_WORD3);
    const v4u t = (v4u)__builtin_amdgcn_raw_buffer_load_b128(r, lane * 16, 0, NT_ROWS ? 2 : 0);  // 2: nt
    v[b] = make_uint4(t.x, t.y, t.z, t.w);
  }
}

// acc += the weighted rows of one (t, h), in the order j = 0, 1, .., n - 1;
// the first NPRE rows of chunk 0 are already in flight (pv, pw), and those
// of weight 0 are skipped (a workgroup's first tile loads them before it
// knows the weights). Skipping a row of weight 0 gives the same bits as
// adding its 0 * 0: the sum starts at +0 and never becomes -0. REST: rows
// past the first NPRE may exist (false when the caller guarantees n <= NPRE).
template <int NCH, int NPRE, bool REST>
__device__ __forceinline__ void merge_token(const KArgs& a, const uint8_t* rowbase, int lane, const float wts[NCH],
                                            const uint4* pv, const float* pw, float acc[8]) {
#pragma unroll
  for (int b = 0; b < NPRE; ++b)
    if (__float_as_int(pw[b]) & 0x7FFFFFFF) fma_row(pw[b], pv[b], acc);
  if constexpr (!REST) return;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int nc = min(64, a.n - 64 * c);
    const int wbits = __float_as_int(wts[c]);
    for (int j0 = c == 0 ? NPRE : 0; j0 < nc; j0 += ROWS_IN_FLIGHT) {
      uint4 v[ROWS_IN_FLIGHT];
      float w[ROWS_IN_FLIGHT];
      issue_rows<ROWS_IN_FLIGHT>(a, rowbase, lane, wbits, c, j0, v, w);
#pragma unroll
      for (int b = 0; b < ROWS_IN_FLIGHT; ++b) fma_row(w[b], v[b], acc);
    }
  }
}

// W_V[h] rows wave*16 + tl, K block kb of each of the 4 K steps
// ([mla_back: wv_loads]); the four scale bytes packed into one word, byte st
// for K step st.
__device__ __forceinline__ void load_wv_codes(const KArgs& a, int h, int wave, int tl, int kb, uint4 wv[4]) {
  const uint8_t* wrow = a.w_v + h * a.w_sh + (wave * 16 + tl) * a.w_sv + kb * 16;
#pragma unroll
  for (int st = 0; st < 4; ++st) wv[st] = *reinterpret_cast<const uint4*>(wrow + st * 64);
}

__device__ __forceinline__ int load_wv_scales(const KArgs& a, int h, int wave, int tl, int kb) {
  const uint8_t* srow = a.w_vs + h * a.s_sh + (wave * 16 + tl) * a.s_sv;
  int sa = 0;
#pragma unroll
  for (int st = 0; st < 4; ++st) sa |= (int)srow[(st * 4 + kb) * a.s_sb] << (8 * st);
  return sa;
}

__device__ __forceinline__ void load_wv(const KArgs& a, int h, int wave, int tl, int kb, uint4 wv[4], int& sa) {
  load_wv_codes(a, h, wave, tl, kb, wv);
  sa = load_wv_scales(a, h, wave, tl, kb);
}

// bf16 latents of token t (tile slot tt) -> MXFP4 codes and scale into LDS
// (the MFMA B operand) and, if asked, the stage outputs. Slots of tokens past
// S get zero codes.
__device__ __forceinline__ void quant_to_lds(const KArgs& a, int t, int tt, int h, int lane, bool live,
                                             const uint32_t lat[4], uint8_t* s_codes, uint8_t* s_scales) {
  int code;
  const uint32_t pk = quant8(lat, code);
  const int b = lane >> 2;  // this lane's block
  *reinterpret_cast<uint32_t*>(s_codes + b * CODE_ROW + tt * 16 + (lane & 3) * 4) = live ? pk : 0u;
  if ((lane & 3) == 0) s_scales[tt * NBLK + (b & 3) * 4 + (b >> 2)] = (uint8_t)code;
  if (live) {
    const int64_t th = (int64_t)t * NH + h;
    if (a.dbg_lat)
      reinterpret_cast<uint4*>(a.dbg_lat + th * (KVL * 2))[lane] = make_uint4(lat[0], lat[1], lat[2], lat[3]);
    if (a.dbg_codes) reinterpret_cast<uint32_t*>(a.dbg_codes + th * (KVL / 2))[lane] = pk;
    if (a.dbg_scales && (lane & 3) == 0) a.dbg_scales[th * NBLK + b] = (uint8_t)code;
  }
}

__device__ __forceinline__ const uint8_t* row_base(const KArgs& a, int t, int h) {
  return a.o + (int64_t)t * a.o_st + (int64_t)h * a.o_sh + (int64_t)(t / a.q) * a.o_sr;
}

// The LSE of token t's one partial (n = 1), or 0 without LSEs; t is clamped
// to S - 1, so the load is valid for tokens a tile does not own.
__device__ __forceinline__ float lse_one(const KArgs& a, int t, int h) {
  if (!a.lse) return 0.f;
  const int tc = min(t, a.S - 1);
  return a.lse[(int64_t)(tc / a.q) * a.l_sr + (int64_t)tc * a.l_st + (int64_t)h * a.l_sh];
}

// Two bf16 values in one word with -0 made +0, the rest unchanged: a half's
// sign bit is kept only where its magnitude bits are not all zero (adding
// 0x7FFF to a magnitude of at most 0x7FFF sets bit 15 exactly when the
// magnitude is nonzero, and never carries into the other half).
__device__ __forceinline__ uint32_t plus_zero2(uint32_t w) {
  const uint32_t m = w & 0x7FFF7FFFu;
  return m | ((m + 0x7FFF7FFFu) & w & 0x80008000u);
}

// One partial: token t's row (tile slot tt, already loaded: v) is its
// latents, unless its request is masked as having no KV, the token lies
// past the batch (`empty`) or, with an LSE, that LSE sanitises to -inf.
// With an LSE this is the merge of one partial exactly: its weight is
// exp(0) / 1 = 1 or 0, and 1 * x + 0 is x except that -0 becomes +0 (the
// merge's sum starts at +0), so -0 elements are made +0 here. -> MXFP4 into
// LDS.
__device__ __forceinline__ void copy_stage(const KArgs& a, int t, int tt, int h, int lane, bool live, bool empty,
                                           const uint4& v, float lse, uint8_t* s_codes, uint8_t* s_scales) {
  uint32_t lat[4] = {0u, 0u, 0u, 0u};
  const bool dead = a.lse != nullptr && sane(lse) == -INFINITY;
  if (live && !empty && !dead && !(a.kv_lens && a.kv_lens[t / a.q] == 0)) {
    lat[0] = v.x; lat[1] = v.y; lat[2] = v.z; lat[3] = v.w;
    if (a.lse) {
#pragma unroll
      for (int k = 0; k < 4; ++k) lat[k] = plus_zero2(lat[k]);
    }
  }
  quant_to_lds(a, t, tt, h, lane, live, lat, s_codes, s_scales);
}

// Token t (tile slot tt) of the persistent kernel with LSEs: merged latents
// -> bf16 -> MXFP4 into LDS. Its first NPRE rows are in flight (pv, pw).
template <int NCH, int NPRE, bool REST>
__device__ __forceinline__ void merge_stage(const KArgs& a, int t, int tt, int h, int lane, bool live, bool empty,
                                            const float wts[NCH], const uint4* pv, const float* pw,
                                            uint8_t* s_codes, uint8_t* s_scales) {
  uint32_t lat[4] = {0u, 0u, 0u, 0u};
  if (live && !empty) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    merge_token<NCH, NPRE, REST>(a, row_base(a, t, h), lane, wts, pv, pw, acc);
#pragma unroll
    for (int k = 0; k < 4; ++k) lat[k] = pack_bf16(acc[2 * k], acc[2 * k + 1]);
  }
  quant_to_lds(a, t, tt, h, lane, live, lat, s_codes, s_scales);
}

// Raw LSEs of this wave's two tokens of the tile starting at token t0
// (issue_lse). The loads are issued for every tile and token, the token
// index clamped to S - 1, so that their number never varies; tokens the
// tile does not own, tokens past the batch and tiles that do not exist never
// use them.
template <int NCH>
__device__ __forceinline__ void prefetch_lse(const KArgs& a, int t0, int h, int wave, int lane, float lA[NCH],
                                             int kA[NCH], float lB[NCH], int kB[NCH]) {
  const int tA = t0 + wave * TOK_PER_WAVE;
  issue_lse<NCH>(a, min(tA, a.S - 1), h, lane, lA, kA);
  issue_lse<NCH>(a, min(tA + 1, a.S - 1), h, lane, lB, kB);
}

// Merge weights of this wave's two tokens of the tile [t0, tend) from their
// raw LSEs (loaded a tile earlier); all zero for tokens at or past tend or
// past the batch, and for tiles that do not exist (tend <= t0).
template <int NCH>
__device__ __forceinline__ void tile_weights(const KArgs& a, int t0, int tend, int batch_end, int wave, int lane,
                                             const float lA[NCH], const int kA[NCH], const float lB[NCH],
                                             const int kB[NCH], float wA[NCH], float wB[NCH]) {
  const int tA = t0 + wave * TOK_PER_WAVE, tB = tA + 1;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    wA[c] = lA[c];
    wB[c] = lB[c];
  }
  if (tA < tend && tA < batch_end) {
    finish_lse<NCH>(a, lane, wA, kA);
    lse_to_weights<NCH>(wA);
  } else {
#pragma unroll
    for (int c = 0; c < NCH; ++c) wA[c] = 0.f;
  }
  if (tB < tend && tB < batch_end) {
    finish_lse<NCH>(a, lane, wB, kB);
    lse_to_weights<NCH>(wB);
  } else {
#pragma unroll
    for (int c = 0; c < NCH; ++c) wB[c] = 0.f;
  }
}

// Rows of this wave's tokens of the tile starting at token t0 that are
// issued before the barrier of the tile ahead of it (weights wA, wB): with
// PAIR = 0 the first PF_ROWS rows of the first token; with PAIR > 0 the
// first PAIR rows of each of the two tokens (slots 0..PAIR-1 and
// PAIR..2 PAIR-1), which for n <= PAIR is every row of the tile. A row of
// weight 0, or of a token the tile does not own, reads nothing.
template <int NCH, int PAIR>
__device__ __forceinline__ void issue_next_rows(const KArgs& a, int t0, int h, int wave, int lane, const float wA[NCH],
                                                const float wB[NCH], uint4* pv, float* pw) {
  const int tA = min(t0 + wave * TOK_PER_WAVE, a.S - 1);
  if constexpr (PAIR == 0) {
    issue_rows<PF_ROWS>(a, row_base(a, tA, h), lane, __float_as_int(wA[0]), 0, 0, pv, pw);
  } else {
    const int tB = min(t0 + wave * TOK_PER_WAVE + 1, a.S - 1);
    issue_rows<PAIR>(a, row_base(a, tA, h), lane, __float_as_int(wA[0]), 0, 0, pv, pw);
    issue_rows<PAIR>(a, row_base(a, tB, h), lane, __float_as_int(wB[0]), 0, 0, pv + PAIR, pw + PAIR);
  }
}

// The first tile of a workgroup: the rows issue_next_rows would issue for
// it, issued together with its LSE loads, before the weights are known, so
// that the first tile does not wait one more memory round trip. Only a token
// the tile [t0, tend) does not own or past the batch, or a row past n, reads
// nothing (a buffer resource of zero bytes); rows of weight 0 are loaded but
// never used (the merge skips them by a uniform branch, so NaN or inf stored
// there cannot reach the sum).
template <int R>
__device__ __forceinline__ void issue_rows_early(const KArgs& a, int t, int tend, int batch_end, int h, int lane,
                                                 uint4* pv) {
  const bool use = t < tend && t < batch_end;
  const uint8_t* rowbase = row_base(a, min(t, a.S - 1), h);
  const int nc = min(64, a.n);
#pragma unroll
  for (int b = 0; b < R; ++b) {
    const uint8_t* p = rowbase + (int64_t)min(b, nc - 1) * a.o_sj;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(p), (short)0, (use && b < nc) ? KVL * 2 : 0, BUF_WORD3);
    const v4u v = (v4u)__builtin_amdgcn_raw_buffer_load_b128(r, lane * 16, 0, NT_ROWS ? 2 : 0);  // 2: nt
    pv[b] = make_uint4(v.x, v.y, v.z, v.w);
  }
}

template <int PAIR>
__device__ __forceinline__ void issue_first_rows_early(const KArgs& a, int t0, int tend, int batch_end, int h,
                                                       int wave, int lane, uint4* pv) {
  const int t = t0 + wave * TOK_PER_WAVE;
  if constexpr (PAIR == 0) {
    issue_rows_early<PF_ROWS>(a, t, tend, batch_end, h, lane, pv);
  } else {
    issue_rows_early<PAIR>(a, t, tend, batch_end, h, lane, pv);
    issue_rows_early<PAIR>(a, t + 1, tend, batch_end, h, lane, pv + PAIR);
  }
}

// The weights of R early rows once known (w0: chunk 0's weights, lane j
// holding partial j's): 0 past n.
template <int R>
__device__ __forceinline__ void early_row_weights(const KArgs& a, float w0, float* pw) {
  const int nc = min(64, a.n);
#pragma unroll
  for (int b = 0; b < R; ++b) {
    int wb = __builtin_amdgcn_readlane(__float_as_int(w0), b);
    if (b >= nc) wb = 0;
    pw[b] = __int_as_float(wb);
  }
}

template <int PAIR>
__device__ __forceinline__ void first_row_weights(const KArgs& a, float wA0, float wB0, float* pw) {
  if constexpr (PAIR == 0) {
    early_row_weights<PF_ROWS>(a, wA0, pw);
  } else {
    early_row_weights<PAIR>(a, wA0, pw);
    early_row_weights<PAIR>(a, wB0, pw + PAIR);
  }
}

// 8 bf16 W_UV results times 8 bf16 gate values, each rounded once to bf16
// (the product of two bf16 values is exact in float32).
__device__ __forceinline__ uint4 gate_mul(const uint4& av, const uint4& g8) {
  return make_uint4(pack_bf16(bf_lo(av.x) * bf_lo(g8.x), bf_hi(av.x) * bf_hi(g8.x)),
                    pack_bf16(bf_lo(av.y) * bf_lo(g8.y), bf_hi(av.y) * bf_hi(g8.y)),
                    pack_bf16(bf_lo(av.z) * bf_lo(g8.z), bf_hi(av.z) * bf_hi(g8.z)),
                    pack_bf16(bf_lo(av.w) * bf_lo(g8.w), bf_hi(av.w) * bf_hi(g8.w)));
}

// The token tiles of one slot of a head, out of k slots per head. Every slot
// takes `main` full 16-token tiles at stride k (tiles slot, slot + k, ..);
// the tokens past those, fewer than 16 k, go out as one more tile of at
// most `chunk` consecutive tokens per slot. With `spread` they are dealt out
// evenly (chunk = ceil(rest / k) <= 16), so every workgroup's share of a head
// differs from another's by at most one short tile and the CUs, each running
// the same number of workgroups, end together; otherwise whole 16-token tiles
// go to the first slots. Measured with 16 splits: S = 2064 72.9 -> 63.4 us,
// 4112 124.3 -> 121.3 us, 4608 139.7 -> 135.1 us spread; with 6 to 12 splits
// spreading is as good or better at most sizes, with 2 or 4 splits (little
// data per tile, so an extra short tile costs a whole memory round trip)
// it loses as often as it wins, so those keep whole tiles. The schedule's
// arithmetic costs about 0.3% where nothing is left over (S = 4096: 120.8
// -> 121.2 us in an A/B run).
struct TileSched {
  int S, k, slot;
  int main;   // full tiles of every slot
  int base;   // the first token past them
  int chunk;  // tokens of a slot's short tile
  int count;  // tiles of this slot
};

// Full tiles per slot and the short tile's token count (host and device),
// for tiles of TT tokens.
template <int TT = TILE_T>
__host__ __device__ inline void tile_counts(int S, int k, bool spread, int& main, int& chunk) {
  main = S / (TT * k);
  const int rest = S - main * TT * k;
  chunk = spread ? (rest + k - 1) / k : (rest < TT ? rest : TT);
}

// Whether leftover tokens are dealt out evenly (see TileSched): for one
// partial (copied) and from SPREAD_MIN_N partials.
__host__ __device__ inline bool spread_leftover(bool copy, int n) { return copy || n >= SPREAD_MIN_N; }

template <int TT = TILE_T>
__device__ __forceinline__ TileSched tile_sched(int S, int k, int slot, bool spread) {
  TileSched t;
  t.S = S;
  t.k = k;
  t.slot = slot;
  tile_counts<TT>(S, k, spread, t.main, t.chunk);
  t.base = t.main * TT * k;
  t.count = t.main + (t.base + slot * t.chunk < S ? 1 : 0);
  return t;
}

// Tokens [t0, tend) of tile i of the slot; t0 = tend = S for an i past its
// tiles.
template <int TT = TILE_T>
__device__ __forceinline__ void tile_span(const TileSched& t, int i, int& t0, int& tend) {
  if (i < t.main) {
    t0 = (t.slot + i * t.k) * TT;
    tend = t0 + TT;
  } else if (i < t.count) {
    t0 = t.base + t.slot * t.chunk;
    tend = min(t0 + t.chunk, t.S);
  } else {
    t0 = tend = t.S;
  }
}

// Write `count` staged output tiles (final core values) of head h, the slot's
// tiles first, first + 1, ..: each token's 256 bytes of the head go out as 16
// coalesced 16-byte pieces; the whole workgroup shares the pieces.
__device__ __forceinline__ void flush_tiles(const KArgs& a, const TileSched& ts, int h, int first, int count,
                                            uint8_t (*s_out)[LDS_OUT]) {
  for (int i = threadIdx.x; i < count * STORE_LANES; i += THREADS) {
    const int k = i / STORE_LANES, piece = i % STORE_LANES;
    const int tok = piece >> 4, col = (piece & 15) * 8;
    int t0, tend;
    tile_span(ts, first + k, t0, tend);
    const int t = t0 + tok;
    if (t >= tend) continue;
    const int64_t off = ((int64_t)t * GROWS + h * VD + col) * 2;
    store_nt16(a.core + off, *reinterpret_cast<const uint4*>(s_out[k] + tok * OUT_ROW + col * 2));
  }
}

// ---------------------------------------------------------------- the fused kernel

// The device deals workgroups to its 8 XCDs in turn (workgroup i to XCD
// i mod 8), each XCD with its own L2. When the grid is a multiple of 8 x 12,
// the 12 heads of one token-tile slot go to consecutive workgroups of one
// XCD, so they run at the same time behind the same L2: the LSE lines they
// share are fetched once, and the 12 pieces of each core row are written
// together. Otherwise workgroup i takes head i mod 12 and slot i / 12. Either
// way the map is one to one onto (head, slot).
constexpr int XCDS = 8;

__device__ __forceinline__ void head_and_slot(int& h, int& slot) {
  if (gridDim.x % (XCDS * NH) == 0) {
    const int xcd = blockIdx.x % XCDS, k = blockIdx.x / XCDS;
    h = k % NH;
    slot = xcd + XCDS * (k / NH);
  } else {
    h = blockIdx.x % NH;
    slot = blockIdx.x / NH;
  }
}

// COPY: one partial, copied (copy_stage) rather than merged. PAIR: rows of
// each of a wave's two tokens issued a tile ahead (instantiated with 4, for
// 2 <= n <= 4; 0: the first PF_ROWS rows of the first token only).
template <bool COPY, int NCH, int PAIR>
__global__ __launch_bounds__(THREADS) void mla_post_kernel(const KArgs a, int wg_per_head) {
  static_assert(PAIR == 0 || (NCH == 1 && !COPY), "both tokens' rows ahead only for merged partials, n <= 64");
  constexpr int NPF = PAIR ? 2 * PAIR : PF_ROWS;  // rows in flight across the barrier
  constexpr int NPRE_A = PAIR ? PAIR : PF_ROWS, NPRE_B = PAIR;
  // two LDS buffers: a wave may merge tile i+1 while others still read tile i
  __shared__ __attribute__((aligned(16))) uint8_t s_codes[2][LDS_CODES];
  __shared__ __attribute__((aligned(16))) uint8_t s_scales[2][LDS_SCALES];
  __shared__ __attribute__((aligned(16))) uint8_t s_out[OUT_TILES][LDS_OUT];

  const int lane = threadIdx.x & 63;
  // wave index as a scalar: everything derived from it (tokens, row bases)
  // stays in scalar registers, and row loads take a scalar base plus the
  // lane's 32-bit offset
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int h, slot;  // this workgroup's head, fixed, and its slot of the head's tiles
  head_and_slot(h, slot);
  const TileSched ts = tile_sched(a.S, wg_per_head, slot, spread_leftover(COPY, a.n));
  const int tl = lane & 15;  // MFMA row / column index of this lane
  const int kb = lane >> 4;  // MFMA K block of this lane

  // W_V[h]'s operands for this wave's 16 rows stay in registers for every
  // tile of the head (loaded below, after the first tile's loads).
  uint4 wv[4];
  int sa = 0;
  // tokens at or past qsl[R] lie past the batch: every partial is empty
  const int batch_end = a.qsl ? a.qsl[a.S / a.q] : a.S;

  // Software pipeline over the workgroup's tiles, so that a wave keeps loads
  // in flight while it waits at the barrier and runs the MFMAs: before the
  // barrier of tile i it turns tile i+1's LSEs (loaded during tile i-1) into
  // weights, issues tile i+2's LSE loads and tile i+1's first PF_ROWS rows.
  float lA[NCH], lB[NCH];  // raw LSEs of the next tile
  int kA[NCH], kB[NCH];
  float wA[NCH], wB[NCH];  // weights of the current tile
  uint4 pv[NPF];           // its first rows, in flight
  float pw[NPF];
  // The first tile's LSEs and first rows go out together; W_V goes out after
  // them, so that waiting for the LSEs does not wait for W_V (loads complete
  // in issue order), which only the first MFMAs need. Measured on the large
  // decode batch: 122.9 -> 121.5 us for W_V last, 120.7 us with the rows
  // issued early.
  // tokens of the current tile and of the next one
  int t0, tend, n0, nend;
  tile_span(ts, 0, t0, tend);
  tile_span(ts, 1, n0, nend);
  float pl[TOK_PER_WAVE] = {0.f, 0.f};  // one partial: the LSEs (if any) of the rows in flight
  if constexpr (COPY) {
    // one partial: a token's one row (and LSE) is issued a tile ahead, both tokens'
    pl[0] = lse_one(a, t0 + wave * TOK_PER_WAVE, h);
    pl[1] = lse_one(a, t0 + wave * TOK_PER_WAVE + 1, h);
    issue_rows_early<1>(a, t0 + wave * TOK_PER_WAVE, tend, batch_end, h, lane, pv);
    issue_rows_early<1>(a, t0 + wave * TOK_PER_WAVE + 1, tend, batch_end, h, lane, pv + 1);
  } else {
    prefetch_lse<NCH>(a, t0, h, wave, lane, lA, kA, lB, kB);
    issue_first_rows_early<PAIR>(a, t0, tend, batch_end, h, wave, lane, pv);
    tile_weights<NCH>(a, t0, tend, batch_end, wave, lane, lA, kA, lB, kB, wA, wB);
    first_row_weights<PAIR>(a, wA[0], wB[0], pw);
    prefetch_lse<NCH>(a, n0, h, wave, lane, lA, kA, lB, kB);
  }
  load_wv(a, h, wave, tl, kb, wv, sa);

#pragma unroll 1
  for (int it = 0; it < ts.count; ++it) {
    uint8_t* codes = s_codes[it & 1];
    uint8_t* scales = s_scales[it & 1];
    int m0, mend;  // the tile after the next
    tile_span(ts, it + 2, m0, mend);
    // ---- merge + quantise: wave owns tile slots 2 wave and 2 wave + 1
    const int ttA = wave * TOK_PER_WAVE, ttB = ttA + 1;
    const int tA = t0 + ttA, tB = t0 + ttB;
    const bool liveA = tA < tend, liveB = tB < tend;
    const bool emptyA = tA >= batch_end, emptyB = tB >= batch_end;
    // the 4 gate values of this lane's outputs (token tl, rows v0..v0+3),
    // loaded now so that their latency hides behind the merge; a token past
    // S re-reads row S - 1 (a token the tile does not own is never stored)
    const int t_out = min(t0 + tl, a.S - 1);
    const uint2 g4 = load_nt8(a.gate + ((int64_t)t_out * GROWS + h * VD + wave * 16 + kb * 4) * 2);
    if constexpr (COPY) {
      copy_stage(a, tA, ttA, h, lane, liveA, emptyA, pv[0], pl[0], codes, scales);
      copy_stage(a, tB, ttB, h, lane, liveB, emptyB, pv[1], pl[1], codes, scales);
      pl[0] = lse_one(a, n0 + wave * TOK_PER_WAVE, h);
      pl[1] = lse_one(a, n0 + wave * TOK_PER_WAVE + 1, h);
      issue_rows_early<1>(a, n0 + wave * TOK_PER_WAVE, nend, batch_end, h, lane, pv);
      issue_rows_early<1>(a, n0 + wave * TOK_PER_WAVE + 1, nend, batch_end, h, lane, pv + 1);
    } else {
      // with PAIR > 0 the call has n <= PAIR: every row is among those issued ahead
      merge_stage<NCH, NPRE_A, PAIR == 0>(a, tA, ttA, h, lane, liveA, emptyA, wA, pv, pw, codes, scales);
      merge_stage<NCH, NPRE_B, PAIR == 0>(a, tB, ttB, h, lane, liveB, emptyB, wB, pv + NPRE_A, pw + NPRE_A, codes,
                                           scales);
    }
    if constexpr (!COPY) {
      tile_weights<NCH>(a, n0, nend, batch_end, wave, lane, lA, kA, lB, kB, wA, wB);
      prefetch_lse<NCH>(a, m0, h, wave, lane, lA, kA, lB, kB);
      issue_next_rows<NCH, PAIR>(a, n0, h, wave, lane, wA, wB, pv, pw);
    }
    // One barrier per tile: it publishes this tile's codes, and since every
    // wave finished the previous tile's MFMAs before merging this one, the
    // other buffer is free for the next tile.
    __syncthreads();

    // ---- W_UV: D[v][token] = sum_k W_V[h][v][k] * L[token][k]
    const int sb = *reinterpret_cast<const int*>(scales + tl * NBLK + kb * 4);
    v4f acc = {0.f, 0.f, 0.f, 0.f};
    {
      const uint8_t* brow = codes + tl * 16;
      acc = mfma_step<0>(wv[0], *reinterpret_cast<const uint4*>(brow + (0 * 4 + kb) * CODE_ROW), acc, sa, sb);
      acc = mfma_step<1>(wv[1], *reinterpret_cast<const uint4*>(brow + (1 * 4 + kb) * CODE_ROW), acc, sa, sb);
      acc = mfma_step<2>(wv[2], *reinterpret_cast<const uint4*>(brow + (2 * 4 + kb) * CODE_ROW), acc, sa, sb);
      acc = mfma_step<3>(wv[3], *reinterpret_cast<const uint4*>(brow + (3 * 4 + kb) * CODE_ROW), acc, sa, sb);
    }
    // The MFMAs read operands from all 64 lanes, so they must run with the
    // whole wave active: their result goes straight to an unconditional LDS
    // store below, before any lane-dependent branch, so no lane condition can
    // enclose them (a CPU test checks the built code for MFMAs under a
    // narrowed exec mask).

    // ---- gate and stage ([mla_back: stage_uv]): the lane holds rows
    // v0..v0+3 (v0 = 16 wave + 4 kb) of token tl. The finished core values
    // are kept in LDS and written when OUT_TILES have gathered or the
    // workgroup's tiles are done: the writes then come in bursts, mostly
    // after the read stream, instead of competing with it all along.
    // core = bf16( bf16(acc) * gate ): the product of two bf16 values is
    // exact in float32, so that is one rounding
    const int slot_out = it % OUT_TILES;
    const uint2 ab = make_uint2(pack_bf16(acc[0], acc[1]), pack_bf16(acc[2], acc[3]));
    *reinterpret_cast<uint2*>(s_out[slot_out] + tl * OUT_ROW + (wave * 16 + kb * 4) * 2) =
        make_uint2(pack_bf16(bf_lo(ab.x) * bf_lo(g4.x), bf_hi(ab.x) * bf_hi(g4.x)),
                   pack_bf16(bf_lo(ab.y) * bf_lo(g4.y), bf_hi(ab.y) * bf_hi(g4.y)));
    const bool last = it + 1 == ts.count;
    if (slot_out == OUT_TILES - 1 || last) {
      __syncthreads();
      flush_tiles(a, ts, h, it - slot_out, slot_out + 1, s_out);
      if (!last) __syncthreads();  // the staging buffers are reused
    }
    t0 = n0;
    tend = nend;
    n0 = m0;
    nend = mend;
  }
}

// ---------------------------------------------------------------- the latency-regime kernel

// The output piece a thread of a one-tile workgroup writes: token tok of the
// tile (thread / 16), columns col .. col + 7 of head h's 128, and the gate
// values of those columns, loaded at once (a thread whose token lies past S
// or past the tile's TT tokens loads and stores nothing).
struct OutPiece {
  int tok, col;
  bool live;
  int64_t off;  // byte offset in gate and core
  uint4 g8;
};

__device__ __forceinline__ OutPiece out_piece(const KArgs& a, int h, int t0, int tt) {
  OutPiece o;
  o.tok = threadIdx.x >> 4;
  o.col = (threadIdx.x & 15) * 8;
  const int t = t0 + o.tok;
  o.live = o.tok < tt && t < a.S;
  o.off = ((int64_t)t * GROWS + h * VD + o.col) * 2;
  o.g8 = make_uint4(0u, 0u, 0u, 0u);
  if (o.live) o.g8 = load_nt16(a.gate + o.off);
  return o;
}

// The tile's MXFP4 latents in LDS (after a barrier) times this wave's 16 rows
// of W_V[h] (wv, sa) -> bf16 -> s_out; after a barrier each thread with a
// live output piece writes bf16(that * gate) to core.
__device__ __forceinline__ void tile_wuv_store(const KArgs& a, int wave, int tl, int kb, const uint4 wv[4], int sa,
                                               const uint8_t* s_codes, const uint8_t* s_scales, uint8_t* s_out,
                                               const OutPiece& out) {
  const int sb = *reinterpret_cast<const int*>(s_scales + tl * NBLK + kb * 4);
  v4f acc = {0.f, 0.f, 0.f, 0.f};
  {
    const uint8_t* brow = s_codes + tl * 16;
    acc = mfma_step<0>(wv[0], *reinterpret_cast<const uint4*>(brow + (0 * 4 + kb) * CODE_ROW), acc, sa, sb);
    acc = mfma_step<1>(wv[1], *reinterpret_cast<const uint4*>(brow + (1 * 4 + kb) * CODE_ROW), acc, sa, sb);
    acc = mfma_step<2>(wv[2], *reinterpret_cast<const uint4*>(brow + (2 * 4 + kb) * CODE_ROW), acc, sa, sb);
    acc = mfma_step<3>(wv[3], *reinterpret_cast<const uint4*>(brow + (3 * 4 + kb) * CODE_ROW), acc, sa, sb);
  }
  // the result is stored unconditionally before any lane-dependent branch, so
  // the MFMAs run with the whole wave active (see the persistent kernel)
  *reinterpret_cast<uint2*>(s_out + tl * OUT_ROW + (wave * 16 + kb * 4) * 2) =
      make_uint2(pack_bf16(acc[0], acc[1]), pack_bf16(acc[2], acc[3]));
  __syncthreads();
  if (out.live) {
    const uint4 av = *reinterpret_cast<const uint4*>(s_out + out.tok * OUT_ROW + out.col * 2);
    store_nt16(a.core + out.off, gate_mul(av, out.g8));
  }
}

// When the whole grid is resident at once (one token tile per workgroup) and
// n <= lat_nmax(TT), bandwidth is not the bound; the chain of dependent memory
// round trips is (LSEs -> weights -> rows of one token -> rows of the other
// -> gate). This kernel issues everything at once: W_V, the gate, the LSEs
// and every partial row of both tokens, speculatively, before the weights
// are known; a row whose weight turns out to be 0 is then left out of the
// sum by a uniform branch, so NaN or inf stored in it cannot reach the
// result. Same arithmetic, same order of summation as the main kernel.
constexpr int LAT_NMAX = 8;

// Rows per token the one-tile instance can hold in registers at once: with
// 8-token tiles a wave owns one token, so it can hold twice as many.
constexpr int lat_nmax(int tt) { return tt <= WAVES ? 2 * LAT_NMAX : LAT_NMAX; }

// TT tokens per workgroup (16 or 8): with fewer tokens per workgroup a
// small batch spreads over more CUs. Wave w owns token slots w and w + 8;
// slots at or past TT are empty (zero codes, nothing loaded, nothing stored),
// so MFMA columns of those slots carry zeros.
// NM: rows per token held at once (the instance for n <= NM). COPY: one
// partial, copied (copy_stage) rather than merged.
template <bool COPY, int TT, int NM>
__global__ __launch_bounds__(THREADS) void mla_post_latency_kernel(const KArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t s_codes[LDS_CODES];
  __shared__ __attribute__((aligned(16))) uint8_t s_scales[LDS_SCALES];
  __shared__ __attribute__((aligned(16))) uint8_t s_out[LDS_OUT];

  const int lane = threadIdx.x & 63;
  // wave index as a scalar: everything derived from it (tokens, row bases)
  // stays in scalar registers, and row loads take a scalar base plus the
  // lane's 32-bit offset
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = blockIdx.x % NH;
  const int tile = blockIdx.x / NH;
  const int t0 = tile * TT;
  const int tl = lane & 15;
  const int kb = lane >> 4;
  const int batch_end = a.qsl ? a.qsl[a.S / a.q] : a.S;

  uint4 wv[4];
  int sa = 0;
  load_wv(a, h, wave, tl, kb, wv, sa);
  const OutPiece out = out_piece(a, h, t0, TT);

  const int ttA = wave, ttB = wave + WAVES;
  const int tA = t0 + ttA, tB = t0 + ttB;
  const bool liveA = ttA < TT && tA < a.S, liveB = ttB < TT && tB < a.S;
  const bool useA = liveA && tA < batch_end, useB = liveB && tB < batch_end;
  uint32_t latA[4] = {0u, 0u, 0u, 0u}, latB[4] = {0u, 0u, 0u, 0u};
  if constexpr (COPY) {
    // one partial: its row, kept as copy_stage keeps it
    const float lsA = lse_one(a, tA, h), lsB = lse_one(a, tB, h);
    uint4 vA = make_uint4(0u, 0u, 0u, 0u), vB = make_uint4(0u, 0u, 0u, 0u);
    if (useA) vA = load_row16(row_base(a, tA, h), lane);
    if (useB) vB = load_row16(row_base(a, tB, h), lane);
    copy_stage(a, tA, ttA, h, lane, liveA, !useA, vA, lsA, s_codes, s_scales);
    copy_stage(a, tB, ttB, h, lane, liveB, !useB, vB, lsB, s_codes, s_scales);
  } else {
    // LSE loads first, then every row, and only then anything that waits
    float lA[1] = {-INFINITY}, lB[1] = {-INFINITY};
    int kA[1] = {1}, kB[1] = {1};
    if (useA) issue_lse<1>(a, tA, h, lane, lA, kA);
    if (useB) issue_lse<1>(a, tB, h, lane, lB, kB);
    // a second token per wave only when the tile has 16 tokens
    static_assert(NM <= lat_nmax(TT), "rows held at once");
    constexpr int NB = TT > WAVES ? NM : 1;
    uint4 rA[NM], rB[NB];
    const uint8_t* baseA = row_base(a, tA, h);
    const uint8_t* baseB = row_base(a, tB, h);
#pragma unroll
    for (int j = 0; j < NM; ++j) {
      rA[j] = make_uint4(0u, 0u, 0u, 0u);
      if (useA && j < a.n) rA[j] = load_row16(baseA + (int64_t)j * a.o_sj, lane);
      if constexpr (TT > WAVES) {
        rB[j] = make_uint4(0u, 0u, 0u, 0u);
        if (useB && j < a.n) rB[j] = load_row16(baseB + (int64_t)j * a.o_sj, lane);
      }
    }
    if (useA) {
      finish_lse<1>(a, lane, lA, kA);
      lse_to_weights<1>(lA);
    }
    if (useB) {
      finish_lse<1>(a, lane, lB, kB);
      lse_to_weights<1>(lB);
    }
    float accA[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float accB[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < NM; ++j) {
      const int wa = useA && j < a.n ? __builtin_amdgcn_readlane(__float_as_int(lA[0]), j) : 0;
      if (wa & 0x7FFFFFFF) fma_row(__int_as_float(wa), rA[j], accA);
      if constexpr (TT > WAVES) {
        const int wb = useB && j < a.n ? __builtin_amdgcn_readlane(__float_as_int(lB[0]), j) : 0;
        if (wb & 0x7FFFFFFF) fma_row(__int_as_float(wb), rB[j], accB);
      }
    }
    if (useA) {
#pragma unroll
      for (int k = 0; k < 4; ++k) latA[k] = pack_bf16(accA[2 * k], accA[2 * k + 1]);
    }
    if (useB) {
#pragma unroll
      for (int k = 0; k < 4; ++k) latB[k] = pack_bf16(accB[2 * k], accB[2 * k + 1]);
    }
    quant_to_lds(a, tA, ttA, h, lane, liveA, latA, s_codes, s_scales);
    quant_to_lds(a, tB, ttB, h, lane, liveB, latB, s_codes, s_scales);
  }
  __syncthreads();
  tile_wuv_store(a, wave, tl, kb, wv, sa, s_codes, s_scales, s_out, out);
}

// ---------------------------------------------------------------- the split-rows kernel

// Many partials and few tokens (a long context split many ways in a small
// decode batch): the other kernels give each wave whole tokens, so a wave
// walks a token's n rows in sequence while the grid holds few workgroups.
// Here G waves share each token: a workgroup takes TT = 8 / G tokens of one
// head, and wave w takes token w / G and its partials j = g, g + G, g + 2G,
// .. (g = w mod G). The LSEs, the first SPLIT_RB (at most) of those rows, W_V
// and the gate are all issued before anything waits; further rows stream
// through the same registers, each issued as the row before it in its
// register is summed. A wave sums its rows in that order (skipping weight-0 rows as
// the other kernels do); the G sums of a token are then added in LDS in the
// order g = 0, 1, .., G - 1. So the order of summation differs from the other
// kernels' j = 0, 1, .., n - 1 (the merge admits any order; the float32
// rounding stays within the same bound) and is fixed, so results repeat.
constexpr int SPLIT_RB = 16;  // rows a wave holds at once
constexpr int SPLIT_NB = 8;   // most batches of SPLIT_RB rows a wave streams

// Batches of rows per wave of the instance for G waves per token and NCH LSE
// chunks (n <= 64 NCH): 64 NCH / G rows.
constexpr int split_batches(int g, int nch) { return 64 * nch / g <= SPLIT_RB ? 1 : 64 * nch / g / SPLIT_RB; }

// Zero codes for tile slot tt, whose token does not exist (an MFMA column of
// zeros, never stored).
__device__ __forceinline__ void empty_slot(const KArgs& a, int tt, int h, int lane, uint8_t* s_codes,
                                           uint8_t* s_scales) {
  const uint32_t zero[4] = {0u, 0u, 0u, 0u};
  quant_to_lds(a, 0, tt, h, lane, false, zero, s_codes, s_scales);
}

template <int G, int NCH>
__global__ __launch_bounds__(THREADS) void mla_post_split_kernel(const KArgs a) {
  static_assert(G == 1 || G == 2 || G == 4 || G == 8, "waves per token");
  static_assert(split_batches(G, NCH) <= SPLIT_NB, "rows per wave");
  constexpr int TT = WAVES / G;
  constexpr int RMAX = 64 * NCH / G;                    // most rows of one wave (n <= 64 NCH)
  constexpr int RB = RMAX < SPLIT_RB ? RMAX : SPLIT_RB;  // rows held at once
  constexpr int NB = RMAX / RB;                         // batches of RB rows
  constexpr int NRED = WAVES - TT;                      // waves whose sums go through LDS
  __shared__ __attribute__((aligned(16))) uint8_t s_codes[LDS_CODES];
  __shared__ __attribute__((aligned(16))) uint8_t s_scales[LDS_SCALES];
  __shared__ __attribute__((aligned(16))) uint8_t s_out[LDS_OUT];
  __shared__ __attribute__((aligned(16))) float4 s_red[NRED > 0 ? NRED : 1][2][64];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = blockIdx.x % NH;
  const int t0 = (blockIdx.x / NH) * TT;
  const int tl = lane & 15, kb = lane >> 4;
  const int batch_end = a.qsl ? a.qsl[a.S / a.q] : a.S;
  const int tt = wave / G, g = wave % G;
  const int t = t0 + tt;
  const bool live = t < a.S;
  const bool use = live && t < batch_end;
  // rows of this wave: j = g + G i for i < mine
  const int mine = use ? (a.n - g + G - 1) / G : 0;
  const uint8_t* base = row_base(a, use ? t : 0, h);
  const int64_t step = (int64_t)G * a.o_sj;

  float l[NCH];
  int kv[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    l[c] = -INFINITY;
    kv[c] = 1;
  }
  if (use) issue_lse<NCH>(a, t, h, lane, l, kv);
  // row i of this wave through a buffer resource of 1 KiB, or of 0 bytes
  // (zeros, no memory access) when the wave has no row i
  auto row = [&](int i) {
    const uint8_t* p = base + (int64_t)g * a.o_sj + (int64_t)i * step;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(i < mine ? p : base), (short)0, i < mine ? KVL * 2 : 0, BUF_WORD3);
    const v4u x = (v4u)__builtin_amdgcn_raw_buffer_load_b128(r, lane * 16, 0, NT_ROWS ? 2 : 0);  // 2: nt
    return make_uint4(x.x, x.y, x.z, x.w);
  };
  uint4 v[RB];
#pragma unroll
  for (int i = 0; i < RB; ++i) v[i] = row(i);

  uint4 wv[4];
  int sa = 0;
  load_wv(a, h, wave, tl, kb, wv, sa);
  const OutPiece out = out_piece(a, h, t0, TT);
  // slots past the tile's tokens: zero codes
#pragma unroll
  for (int e = TT + wave; e < TILE_T; e += WAVES) empty_slot(a, e, h, lane, s_codes, s_scales);

  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (use) {
    finish_lse<NCH>(a, lane, l, kv);
    lse_to_weights<NCH>(l);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (b == 0 || b * RB < mine) {
#pragma unroll
        for (int k = 0; k < RB; ++k) {
          const int i = b * RB + k;
          // partial j = g + G i: chunk (G i) / 64 (g < G and G divides 64), lane j mod 64
          const int wb = i < mine ? __builtin_amdgcn_readlane(__float_as_int(l[(G * i) >> 6]), (g + G * i) & 63) : 0;
          if (wb & 0x7FFFFFFF) fma_row(__int_as_float(wb), v[k], acc);
          if (b + 1 < NB) v[k] = row(i + RB);
        }
      }
    }
  }
  // the G sums of each token: waves g > 0 hand theirs to wave g = 0
  if (g > 0) {
    float4* r = s_red[tt * (G - 1) + g - 1][0];
    r[lane] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    r[64 + lane] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  }
  __syncthreads();
  if (g == 0) {
#pragma unroll
    for (int k = 1; k < G; ++k) {
      const float4* r = s_red[tt * (G - 1) + k - 1][0];
      const float4 x = r[lane], y = r[64 + lane];
      acc[0] += x.x; acc[1] += x.y; acc[2] += x.z; acc[3] += x.w;
      acc[4] += y.x; acc[5] += y.y; acc[6] += y.z; acc[7] += y.w;
    }
    uint32_t lat[4] = {0u, 0u, 0u, 0u};
    if (use) {
#pragma unroll
      for (int k = 0; k < 4; ++k) lat[k] = pack_bf16(acc[2 * k], acc[2 * k + 1]);
    }
    quant_to_lds(a, t, tt, h, lane, live, lat, s_codes, s_scales);
  }
  __syncthreads();
  tile_wuv_store(a, wave, tl, kb, wv, sa, s_codes, s_scales, s_out, out);
}

// ---------------------------------------------------------------- the streaming kernel

// One or two partials per (token, head) over many tokens. A 16-token tile
// then reads only 16 KiB of rows; the persistent kernel keeps one tile's rows
// in flight in registers and loads each tile's gate as it goes, so it waits
// about one memory round trip per tile and spends much of each tile on
// scalar address arithmetic. Here a tile's partial rows move straight from
// memory into LDS by buffer-to-LDS loads, which hold no registers while in
// flight, and its gate values and LSEs (a few bytes a lane) into registers,
// issued together three tiles ahead of the tile being merged. Each wave
// loads and merges only its own tokens' rows, so a tile needs one barrier,
// between the merge and the MFMAs; the row buffer is refilled as soon as
// the wave has merged it, and the codes and the staged output have a buffer
// per tile in flight. Every load of a tile shares one scalar base at its
// first token, with per-lane offsets fixed for the launch. Workgroups keep
// one head and walk its tiles as the persistent kernel's do, W_V[h] in
// registers; each tile's core rows are staged in LDS and written at the next
// tile, 16 bytes a lane, so every token's 256 bytes of the head go out as
// whole cache lines (8-byte stores straight from the MFMA's result, each
// lane's piece of a token, measured slower). NR = n partials per token (1: copied, 2: merged); a tile has 16 /
// NR tokens, so a wave owns 2 / NR tokens and 2 partial rows of every tile
// either way. Same arithmetic and order of summation as the other kernels.
constexpr int STREAM_NBUF = 3;  // tiles in LDS (rows, codes, staged output): the one being merged and two in flight

template <int NR>
struct StreamTile {
  static constexpr int TT = TILE_T / NR;      // tokens per tile
  static constexpr int TPW = TT / WAVES;      // tokens per wave
  static constexpr int BYTES = TILE_T * KVL * 2;  // rows: token slot tt, partial j at (tt NR + j) KiB
  static constexpr int LOADS = NR * TPW + 2;  // loads a wave issues per tile: its rows, gate values, LSEs
};

// One tile's values that travel in registers: the gate values of this
// lane's four output elements and, in lanes 0 and 1, one LSE each.
struct StreamRegs {
  v2u g;
  float l;
};

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt
// in 6:4, lgkmcnt in 11:8): at most n vector memory operations outstanding;
// no LDS operation outstanding.
constexpr int wait_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int WAIT_LGKM0 = 15 | (3 << 14) | (7 << 4);

// A workgroup barrier that leaves vector memory loads in flight: the wave's
// own LDS writes are complete, then s_barrier. (__syncthreads also waits
// for every outstanding buffer-to-LDS load, which here are the next tiles'.)
// The empty asm statements keep the compiler from moving memory accesses
// across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(WAIT_LGKM0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

typedef __attribute__((address_space(3))) void lds_void;

// Where a workgroup's loads and stores go, fixed for the whole launch. The
// streaming kernel takes only layouts where a (token, head) row, its gate
// row and its LSEs move by a fixed stride per token (no request-major
// offset), with strides that keep every offset within a tile below 2^31 (the
// host checks): each tile's loads then use a scalar base at the tile's first
// token and per-lane offsets computed here once.
struct StreamAddr {
  const uint8_t* o_h[2];  // partial j's row of token 0, head h
  const uint8_t* g_h;     // gate row of token 0, head h
  uint8_t* c_h;           // core row of token 0, head h
  const uint8_t* l_h;     // LSE of partial 0, token 0, head h (the gate when there are none)
  int o_stb, l_st4;       // bytes per token
  int lse_tail;           // LSE bytes a token's loads span
  uint32_t vrow[2];       // this lane's offset in the wave's k-th token's row
  uint32_t vgate;         // .. of its 4 gate values (token slot lane & 15, the MFMA output's rows)
  uint32_t vlse;          // .. among the LSEs
  uint32_t vout;          // this thread's piece of a staged output tile in core
};

template <int NR>
__device__ __forceinline__ StreamAddr stream_addr(const KArgs& a, int h, int wave, int lane) {
  using L = StreamTile<NR>;
  StreamAddr s;
  // the partials' strides are in bytes here, the LSEs' in elements
  s.o_h[0] = a.o + (int64_t)h * a.o_sh;
  s.o_h[1] = s.o_h[0] + (NR > 1 ? a.o_sj : 0);
  s.g_h = a.gate + h * VD * 2;
  s.c_h = a.core + h * VD * 2;
  s.l_h = a.lse ? reinterpret_cast<const uint8_t*>(a.lse + (int64_t)h * a.l_sh) : a.gate;
  s.o_stb = (int)a.o_st;
  s.l_st4 = (int)(a.l_st * 4);
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int tt = wave * L::TPW + (k < L::TPW ? k : 0);
    s.vrow[k] = (uint32_t)(tt * s.o_stb + lane * 16);
  }
  s.vgate = (uint32_t)((lane & 15) * GROWS * 2 + (wave * 16 + (lane >> 4) * 4) * 2);
  // LSEs, 4 B a lane: with two partials lane j takes partial min(j, 1) of
  // the wave's token; with one, lane 0 the LSE of the wave's first token and
  // the other lanes that of its second
  if constexpr (NR == 2) {
    s.vlse = (uint32_t)(wave * s.l_st4 + min(lane, 1) * (int)(a.l_sj * 4));
    s.lse_tail = (int)(a.l_sj * 4) + 4;
  } else {
    s.vlse = (uint32_t)((wave * 2 + min(lane, 1)) * s.l_st4);
    s.lse_tail = 4;
  }
  s.vout = (uint32_t)((threadIdx.x >> 4) * GROWS * 2 + (threadIdx.x & 15) * 16);
  return s;
}

// The loads of the tile [t0, tend): its rows into its LDS buffer
// (stream_rows), then its gate values and LSEs into the registers returned
// (stream_regs), with no other vector memory operation between the two.
// Every wave issues exactly StreamTile<NR>::LOADS of them, for every tile
// index, also past its last tile, so the number in flight is fixed. The
// rows and LSEs of tokens past tend or the batch end, and the gate values of
// tokens past tend, lie beyond the end of their buffer resource (each
// token's bytes start past the previous token's end): nothing is read, the
// registers get zeros and what the LDS then holds is never used. Without
// LSEs the LSE resource has zero bytes.
template <int NR>
__device__ __forceinline__ void stream_rows(const StreamAddr& s, int t0, int tend, int batch_end, int wave,
                                            uint8_t* buf) {
  using L = StreamTile<NR>;
  const int use = max(0, min(tend, batch_end) - t0);  // tokens with partials to read
  const uint64_t orow = (uint64_t)(uint32_t)t0 * (uint32_t)s.o_stb;
#pragma unroll
  for (int j = 0; j < NR; ++j) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(s.o_h[j] + orow), (short)0, use ? (use - 1) * s.o_stb + KVL * 2 : 0, BUF_WORD3);
#pragma unroll
    for (int k = 0; k < L::TPW; ++k)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(buf + ((wave * L::TPW + k) * NR + j) * KVL * 2), 16,
                                               s.vrow[k], 0, 0, NT_ROWS ? 2 : 0);  // 2: nt
  }
}

template <int NR>
__device__ __forceinline__ StreamRegs stream_regs(const KArgs& a, const StreamAddr& s, int t0, int tend,
                                                  int batch_end) {
  const int live = max(0, tend - t0);                 // tokens of the tile
  const int use = max(0, min(tend, batch_end) - t0);  // .. with partials to read
  StreamRegs out;
  {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(s.g_h + (uint64_t)(uint32_t)t0 * (GROWS * 2)), (short)0,
        live ? (live - 1) * (GROWS * 2) + VD * 2 : 0, BUF_WORD3);
    out.g = (v2u)__builtin_amdgcn_raw_buffer_load_b64(r, s.vgate, 0, 0);
  }
  {
    const bool have = a.lse != nullptr && use > 0;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(s.l_h + (a.lse ? (uint64_t)(uint32_t)t0 * (uint32_t)s.l_st4 : 0)), (short)0,
        have ? (use - 1) * s.l_st4 + s.lse_tail : 0, BUF_WORD3);
    out.l = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, s.vlse, 0, 0));
  }
  return out;
}

// The merge weights of two partials from their raw LSEs (wave-uniform), as
// wave-uniform bits: the same values, bit for bit, as lse_to_weights over a
// wave whose other lanes hold -inf (the maximum of two values is exact, each
// exp is the same call on the same argument, and adding the zeros of the
// other lanes to e0 + e1 leaves it unchanged), without its two 64-lane
// reductions: lane 0 computes e0 and its weight, the other lanes e1 and its.
__device__ __forceinline__ void two_weights(float l0, float l1, int& w0, int& w1) {
  l0 = sane(l0);
  l1 = sane(l1);
  float m = fmaxf(l0, l1);
  if (m == -INFINITY) m = 0.f;
  const float e = expf(((threadIdx.x & 63) ? l1 : l0) - m);
  const float tot = lane_f(e, 0) + lane_f(e, 1);
  const float w = (tot == 0.f || e == 0.f) ? 0.f : e / tot;
  w0 = __float_as_int(lane_f(w, 0));
  w1 = __float_as_int(lane_f(w, 1));
}

// Write the staged output tile (final core values) of the tokens [t0, tend)
// of head h: thread i writes piece i, 16 bytes of token i / 16, so each
// token's 256 bytes of the head go out whole. Every thread stores, with no
// branch: pieces of tokens past the tile (threads 16 TT and up included) lie
// beyond the end of the buffer resource and are dropped. The stored value is
// returned so that the caller keeps it live until the loop's next wait, when
// the store has certainly read it: the compiler then never reuses its
// registers early, which would make it wait for every load in flight.
template <int TT>
__device__ __forceinline__ uint4 stream_flush(const StreamAddr& s, int t0, int tend, const uint8_t* s_out) {
  const int tok = min((int)(threadIdx.x >> 4), TILE_T - 1);
  const uint4 v = *reinterpret_cast<const uint4*>(s_out + tok * OUT_ROW + (threadIdx.x & 15) * 16);
  const int live = max(0, tend - t0);
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      s.c_h + (uint64_t)(uint32_t)min(t0, tend) * (GROWS * 2), (short)0, live ? (live - 1) * (GROWS * 2) + VD * 2 : 0,
      BUF_WORD3);
  __builtin_amdgcn_raw_buffer_store_b128((v4u){v.x, v.y, v.z, v.w}, r, s.vout, 0, 2);  // 2: nt
  return v;
}

// The wave's issue priority (s_setprio takes an immediate). Two workgroups
// share a CU; at equal priority the older one's waves issue first, so it
// runs ahead and the younger one finishes alone, later. The streaming kernel
// sets priority 3, 2, 1, 0 at tiles 0, 1, 2, 3 (mod 4): a workgroup one to
// three tiles behind the other then has the higher priority at most tiles,
// which keeps the two together (measured: two partials at S = 16384, 90.8
// -> 86.0 us; one partial unchanged).
__device__ __forceinline__ void issue_priority(int p) {
  switch (p) {
    case 3: __builtin_amdgcn_s_setprio(3); break;
    case 2: __builtin_amdgcn_s_setprio(2); break;
    case 1: __builtin_amdgcn_s_setprio(1); break;
    default: __builtin_amdgcn_s_setprio(0);
  }
}

// One tile of the streaming kernel, tile `it`. Its rows are in LDS buffer
// `rows` (each wave loads and merges only its own tokens' rows there), its
// gate values and LSEs in `regs`. The wave merges its tokens into the code
// buffer (codes, scales), issues tile it + NBUF's rows into its part of
// `rows`, and meets the other waves at the one barrier of the tile: then
// every token's codes are complete and every wave is done with tile it - 1
// (its MFMAs read the other code buffer, and the output tile staged for it,
// out_prev, is written now). The MFMAs' result, times the gate, is staged
// in out_cur; then tile it + NBUF's gate values and LSEs go to `regs` (a
// register reloaded while its old value is still needed would be copied at
// the loop's back edge, which waits for the load). The buffers are distinct
// LDS variables named at compile time at each step: the compiler then knows
// that reading one does not touch what the loads in flight write to the
// others, and leaves those in flight.
template <bool COPY, int NR>
__device__ __forceinline__ void stream_step(const KArgs& a, const TileSched& ts, int it, int h, int wave, int lane,
                                            int batch_end, const StreamAddr& sad, const uint4 wv[4], int sa,
                                            uint8_t* rows, StreamRegs& regs, uint8_t* codes, uint8_t* scales,
                                            uint8_t* out_cur, const uint8_t* out_prev, int& p0, int& pend) {
  using L = StreamTile<NR>;
  constexpr int TT = L::TT;
  const int tl = lane & 15;
  const int kb = lane >> 4;
  issue_priority(3 - (it & 3));
  // This wave's share of tile it has landed when at most the loads of the
  // tiles issued after it are outstanding (loads complete in order).
  __builtin_amdgcn_s_waitcnt(wait_vm((STREAM_NBUF - 1) * L::LOADS));
  int t0, tend;
  tile_span<TT>(ts, it, t0, tend);
  // lanes 0 and 1: the LSEs of the wave's two tokens (one partial) or of
  // its token's two partials
  const float l0 = lane_f(regs.l, 0), l1 = lane_f(regs.l, 1);
  // ---- merge (or copy) + quantise this wave's tokens
#pragma unroll
  for (int k = 0; k < L::TPW; ++k) {
    const int tt = wave * L::TPW + k;
    const int t = t0 + tt;
    const bool live = t < tend, empty = t >= batch_end;
    const uint4 v0 = *reinterpret_cast<const uint4*>(rows + tt * NR * KVL * 2 + lane * 16);
    if constexpr (COPY) {
      copy_stage(a, t, tt, h, lane, live, empty, v0, k ? l1 : l0, codes, scales);
    } else {
      const uint4 v1 = *reinterpret_cast<const uint4*>(rows + (tt * NR + 1) * KVL * 2 + lane * 16);
      uint32_t lat[4] = {0u, 0u, 0u, 0u};
      if (live && !empty) {
        int w0, w1;
        two_weights(l0, l1, w0, w1);
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (w0 & 0x7FFFFFFF) fma_row(__int_as_float(w0), v0, acc);
        if (w1 & 0x7FFFFFFF) fma_row(__int_as_float(w1), v1, acc);
#pragma unroll
        for (int q = 0; q < 4; ++q) lat[q] = pack_bf16(acc[2 * q], acc[2 * q + 1]);
      }
      quant_to_lds(a, t, tt, h, lane, live, lat, codes, scales);
    }
  }
  // the wave's rows of tile it are read (their values are used above): its
  // part of the buffer takes tile it + NBUF's rows
  int n0, nend;
  tile_span<TT>(ts, it + STREAM_NBUF, n0, nend);
  stream_rows<NR>(sad, n0, nend, batch_end, wave, rows);
  lds_barrier();  // every token's codes are complete; every wave is done with tile it - 1
  const uint4 kept = stream_flush<TT>(sad, p0, pend, out_prev);

  // ---- W_UV, gate: the lane holds rows v0..v0+3 (v0 = 16 wave + 4 kb) of
  // token slot tl (slots past an 8-token tile have gate values 0 and are
  // never stored)
  const int sb = *reinterpret_cast<const int*>(scales + tl * NBLK + kb * 4);
  v4f acc = {0.f, 0.f, 0.f, 0.f};
  {
    const uint8_t* brow = codes + tl * 16;
    acc = mfma_step<0>(wv[0], *reinterpret_cast<const uint4*>(brow + (0 * 4 + kb) * CODE_ROW), acc, sa, sb);
    acc = mfma_step<1>(wv[1], *reinterpret_cast<const uint4*>(brow + (1 * 4 + kb) * CODE_ROW), acc, sa, sb);
    acc = mfma_step<2>(wv[2], *reinterpret_cast<const uint4*>(brow + (2 * 4 + kb) * CODE_ROW), acc, sa, sb);
    acc = mfma_step<3>(wv[3], *reinterpret_cast<const uint4*>(brow + (3 * 4 + kb) * CODE_ROW), acc, sa, sb);
  }
  // computed and written by every lane, before any lane-dependent branch:
  // the MFMAs run with the whole wave active
  const uint2 ab = make_uint2(pack_bf16(acc[0], acc[1]), pack_bf16(acc[2], acc[3]));
  const uint2 cv = make_uint2(pack_bf16(bf_lo(ab.x) * bf_lo(regs.g.x), bf_hi(ab.x) * bf_hi(regs.g.x)),
                              pack_bf16(bf_lo(ab.y) * bf_lo(regs.g.y), bf_hi(ab.y) * bf_hi(regs.g.y)));
  *reinterpret_cast<uint2*>(out_cur + tl * OUT_ROW + (wave * 16 + kb * 4) * 2) = cv;
  regs = stream_regs<NR>(a, sad, n0, nend, batch_end);
  p0 = t0;
  pend = tend;
  // the stored values stay live until here, after the tile's other memory
  // operations: their registers are not reused while the store may still
  // read them, which would make the compiler wait for every load in flight
  asm volatile("" ::"v"(kept.x), "v"(kept.y), "v"(kept.z), "v"(kept.w));
}

// Step I on the buffers of tile slot B (rows, registers RG, codes, output),
// the previous tile's output in slot P.
#define STREAM_STEP(I, B, RG, P)                                                                                \
  stream_step<COPY, NR>(a, ts, I, h, wave, lane, batch_end, sad, wv, sa, s_buf##B, RG, s_codes##B, s_scales##B, \
                        s_out##B, s_out##P, p0, pend)

template <bool COPY, int NR>
__global__ __launch_bounds__(THREADS) void mla_post_stream_kernel(const KArgs a) {
  static_assert(COPY == (NR == 1), "one partial is copied, two are merged");
  using L = StreamTile<NR>;
  constexpr int TT = L::TT;
  __shared__ __attribute__((aligned(16))) uint8_t s_buf0[L::BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t s_buf1[L::BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t s_buf2[L::BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t s_codes0[LDS_CODES];
  __shared__ __attribute__((aligned(16))) uint8_t s_codes1[LDS_CODES];
  __shared__ __attribute__((aligned(16))) uint8_t s_codes2[LDS_CODES];
  __shared__ __attribute__((aligned(16))) uint8_t s_scales0[LDS_SCALES];
  __shared__ __attribute__((aligned(16))) uint8_t s_scales1[LDS_SCALES];
  __shared__ __attribute__((aligned(16))) uint8_t s_scales2[LDS_SCALES];
  __shared__ __attribute__((aligned(16))) uint8_t s_out0[LDS_OUT];
  __shared__ __attribute__((aligned(16))) uint8_t s_out1[LDS_OUT];
  __shared__ __attribute__((aligned(16))) uint8_t s_out2[LDS_OUT];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // workgroup b: head b mod 12, slot b / 12 of that head's k workgroups
  const int h = blockIdx.x % NH, slot = blockIdx.x / NH;
  const int k = gridDim.x / NH + (h < (int)(gridDim.x % NH) ? 1 : 0);
  const TileSched ts = tile_sched<TT>(a.S, k, slot, true);
  const int batch_end = a.qsl ? a.qsl[a.S / a.q] : a.S;

  // W_V[h] first (the first MFMAs wait for it anyway), then the first tiles
  uint4 wv[4];
  int sa = 0;
  load_wv(a, h, wave, lane & 15, lane >> 4, wv, sa);
  const StreamAddr sad = stream_addr<NR>(a, h, wave, lane);
  StreamRegs r0, r1, r2;
  {
    int t0, tend;
    tile_span<TT>(ts, 0, t0, tend);
    stream_rows<NR>(sad, t0, tend, batch_end, wave, s_buf0);
    r0 = stream_regs<NR>(a, sad, t0, tend, batch_end);
    tile_span<TT>(ts, 1, t0, tend);
    stream_rows<NR>(sad, t0, tend, batch_end, wave, s_buf1);
    r1 = stream_regs<NR>(a, sad, t0, tend, batch_end);
    tile_span<TT>(ts, 2, t0, tend);
    stream_rows<NR>(sad, t0, tend, batch_end, wave, s_buf2);
    r2 = stream_regs<NR>(a, sad, t0, tend, batch_end);
  }
  // 8-token tiles: MFMA columns 8..15 never hold a token, zero codes once
  if constexpr (TT < TILE_T) {
    empty_slot(a, TT + wave, h, lane, s_codes0, s_scales0);
    empty_slot(a, TT + wave, h, lane, s_codes1, s_scales1);
    empty_slot(a, TT + wave, h, lane, s_codes2, s_scales2);
  }

  int p0 = a.S, pend = a.S;  // tokens of the tile whose output is staged
  // Whole rounds of three tiles, then the last one or two, with no exit from
  // the middle of a round: an early exit would give the compiler a path from
  // inside the round back to its start, along which it would count the
  // latest loads as just issued and wait for them.
  int it = 0;
#pragma unroll 1
  for (; it + 3 <= ts.count; it += 3) {
    STREAM_STEP(it, 0, r0, 2);
    STREAM_STEP(it + 1, 1, r1, 0);
    STREAM_STEP(it + 2, 2, r2, 1);
  }
  const uint8_t* last = s_out2;
  if (it < ts.count) {
    STREAM_STEP(it, 0, r0, 2);
    last = s_out0;
    if (it + 1 < ts.count) {
      STREAM_STEP(it + 1, 1, r1, 0);
      last = s_out1;
    }
  }
  lds_barrier();
  stream_flush<TT>(sad, p0, pend, last);
  // the loads issued for tile indices past the last are still in flight:
  // they read nothing, but the wave waits for them (and its stores) before
  // it ends
  __builtin_amdgcn_s_waitcnt(wait_vm(0));
}
#undef STREAM_STEP

// ---------------------------------------------------------------- stand-alone quantiser

constexpr int QWAVES = 4;
constexpr int64_t QMAX_BLOCKS = 1 << 16;

__global__ __launch_bounds__(QWAVES * 64) void quantize_kernel(const uint8_t* x, int64_t rows, int cols,
                                                               int64_t xs_bytes, uint8_t* codes, int64_t cs,
                                                               uint8_t* scales, int64_t ss) {
  const int lane = threadIdx.x & 63;
  // a wave per row, striding over the grid (the grid is capped; r is the
  // same for the whole wave)
  const int64_t stride = (int64_t)gridDim.x * QWAVES;
  for (int64_t r = (int64_t)blockIdx.x * QWAVES + (threadIdx.x >> 6); r < rows; r += stride) {
    for (int c0 = 0; c0 < cols; c0 += 512) {
      const int c = c0 + lane * 8;
      const bool in = c < cols;  // cols is a multiple of 32: whole quads are in or out
      uint32_t w[4] = {0u, 0u, 0u, 0u};
      if (in) {
        const uint4 v = *reinterpret_cast<const uint4*>(x + r * xs_bytes + (int64_t)c * 2);
        w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
      }
      int code;
      const uint32_t pk = quant8(w, code);
      if (in) {
        *reinterpret_cast<uint32_t*>(codes + r * cs + c / 2) = pk;
        if ((lane & 3) == 0) scales[r * ss + c / 32] = (uint8_t)code;
      }
    }
  }
}

// ---------------------------------------------------------------- host side

bool mul_ok(int64_t a, int64_t b, int64_t* out) { return !__builtin_mul_overflow(a, b, out); }
bool add_ok(int64_t a, int64_t b, int64_t* out) { return !__builtin_add_overflow(a, b, out); }

// largest byte offset reached by index (n0-1, n1-1, n2-1) with the given byte strides, plus `tail`
bool span_ok(int64_t n0, int64_t s0, int64_t n1, int64_t s1, int64_t n2, int64_t s2, int64_t tail) {
  int64_t a, b, c, x, y;
  return mul_ok(n0 - 1, s0, &a) && mul_ok(n1 - 1, s1, &b) && mul_ok(n2 - 1, s2, &c) && add_ok(a, b, &x) &&
         add_ok(x, c, &y) && add_ok(y, tail, &x);
}

bool aligned(const void* p, uintptr_t al) { return (reinterpret_cast<uintptr_t>(p) & (al - 1)) == 0; }

// Copy the caller's arguments into the current layout: a version-1 caller's
// struct ends after dbg_scales, and the later fields read as zero (off).
int normalize(const mla_post_args* in, mla_post_args* out) {
  if (!in || in->struct_size < MLA_POST_ARGS_V1_SIZE) return MLA_POST_EINVAL;
  memset(out, 0, sizeof(*out));
  memcpy(out, in, in->struct_size < sizeof(*out) ? in->struct_size : sizeof(*out));
  out->struct_size = sizeof(*out);
  return MLA_POST_OK;
}

// largest byte offset of a 4-index span: sum_i (n_i - 1) * s_i + tail fits int64
bool span4_ok(const int64_t n[4], const int64_t s[4], int64_t tail) {
  int64_t acc = tail;
  for (int i = 0; i < 4; ++i) {
    int64_t term;
    if (n[i] < 1) continue;
    if (!mul_ok(n[i] - 1, s[i], &term) || !add_ok(acc, term, &acc)) return false;
  }
  return true;
}

int check_args(const mla_post_args* in) {
  mla_post_args na;
  const int st = normalize(in, &na);
  if (st != MLA_POST_OK) return st;
  const mla_post_args* a = &na;
  if (a->n < 1 || a->S < 0 || a->S > MLA_POST_SMAX || a->q < 0) return MLA_POST_EINVAL;
  if (a->n > MLA_POST_NMAX) return MLA_POST_EUNSUPPORTED;
  if (a->S == 0) return MLA_POST_OK;
  if (!a->o || !a->w_v || !a->w_v_scale || !a->gate || !a->core) return MLA_POST_EINVAL;
  if (!a->lse && a->n != 1) return MLA_POST_EINVAL;
  if (a->o_sj < 0 || a->o_st < 0 || a->o_sh < 0) return MLA_POST_ESTRIDE;
  if ((a->o_sj % 8) || (a->o_st % 8) || (a->o_sh % 8)) return MLA_POST_ESTRIDE;
  if (a->lse && (a->l_sj < 0 || a->l_st < 0 || a->l_sh < 0)) return MLA_POST_ESTRIDE;
  if (a->w_sh < 0 || a->w_sv < 0 || (a->w_sh % 16) || (a->w_sv % 16)) return MLA_POST_ESTRIDE;
  if (a->s_sh < 0 || a->s_sv < 0 || a->s_sb < 0) return MLA_POST_ESTRIDE;
  if (!aligned(a->o, 16) || !aligned(a->w_v, 16) || !aligned(a->gate, 16) || !aligned(a->core, 16))
    return MLA_POST_EALIGN;
  if (a->lse && !aligned(a->lse, 4)) return MLA_POST_EALIGN;
  if ((a->dbg_lat && !aligned(a->dbg_lat, 16)) || (a->dbg_codes && !aligned(a->dbg_codes, 4))) return MLA_POST_EALIGN;
  const int q = a->q > 1 ? a->q : 1;
  if (a->S % q) return MLA_POST_EINVAL;
  const int64_t R = a->S / q;
  if (a->o_sr < 0 || a->l_sr < 0 || (a->o_sr % 8) || a->kl_sj < 0) return MLA_POST_ESTRIDE;
  if ((a->kv_lens && !aligned(a->kv_lens, 4)) || (a->qsl && !aligned(a->qsl, 4))) return MLA_POST_EALIGN;
  // every byte offset the kernel forms must fit int64
  {
    const int64_t n4[4] = {a->n, R, a->S, NH};
    int64_t b4[4];
    if (!mul_ok(a->o_sj, 2, &b4[0]) || !mul_ok(a->o_sr, 2, &b4[1]) || !mul_ok(a->o_st, 2, &b4[2]) ||
        !mul_ok(a->o_sh, 2, &b4[3]) || !span4_ok(n4, b4, KVL * 2))
      return MLA_POST_ERANGE;
    if (a->lse && (!mul_ok(a->l_sj, 4, &b4[0]) || !mul_ok(a->l_sr, 4, &b4[1]) || !mul_ok(a->l_st, 4, &b4[2]) ||
                   !mul_ok(a->l_sh, 4, &b4[3]) || !span4_ok(n4, b4, 4)))
      return MLA_POST_ERANGE;
    const int64_t nk[4] = {a->n, R, 1, 1};
    int64_t bk[4] = {0, 4, 0, 0};
    if (a->kv_lens && (!mul_ok(a->kl_sj, 4, &bk[0]) || !span4_ok(nk, bk, 4))) return MLA_POST_ERANGE;
  }
  if (!span_ok(NH, a->w_sh, VD, a->w_sv, 1, 0, KVL / 2)) return MLA_POST_ERANGE;
  if (!span_ok(NH, a->s_sh, VD, a->s_sv, NBLK, a->s_sb, 1)) return MLA_POST_ERANGE;
  if (!span_ok(a->S, (int64_t)GROWS * 2, 1, 0, 1, 0, GROWS * 2)) return MLA_POST_ERANGE;
  return MLA_POST_OK;
}

using mla_dev::device_cus;
using mla_dev::launch;

// Workgroups per head of the persistent kernel (the grid is 12 times that).
// `fill` is WG_PER_CU workgroups per CU in the grid, 2 of them resident (64
// at 256 CUs); `one_round` the most that are all resident at once (2 per CU,
// a multiple of 8 so that the 12 heads of a slot share an XCD: 40).
// - At most one workgroup per CU with one tile each: one per tile.
// - Up to one_round tiles: one_round, each workgroup one short tile of S /
//   one_round tokens, all resident and every CU with at most 2 (one tile
//   per workgroup would put 2 full tiles on the CUs past the first round).
//   Except with at most 128 splits when only the last tile is past the first
//   round and one tile per workgroup leaves fewer tokens on the busiest CU
//   (its 16 and the last tile's, against 2 short tiles). With more splits 2
//   workgroups per CU stream faster than one alone, and one_round stays.
// - Up to 2 workgroups per CU with one tile each: one per tile.
// - Up to fill tiles: fill, every CU running 3 workgroups of S / fill tokens
//   (one tile each would leave some CUs 3 full tiles, others 2).
// - Up to 1.5 fill tiles: one_round, so that every workgroup runs about two
//   tiles back to back in one round instead of a full and a short tile in 1.5
//   rounds. Measured at 65 to 96 tiles (S = 1040 to 1536) with 4 to 24
//   splits, 40 against 64: 16 splits S = 1100 43.5 -> 36.7 us, S = 1280 45.4
//   -> 40.3 us, within 2% either way at S = 1536, and 64 ahead again from
//   about 100 tiles.
// - Beyond that, fill.
// Measured at 256 CUs, 16 to 256 splits, S = 337 to 960, against one tile
// per workgroup up to fill tiles (the rule before) and against 40 and 64
// workgroups per head throughout: within 1.5% of the fastest of the three at
// every point, and up to 26% faster than before (64 splits: S = 352 66.2 ->
// 49.7 us, S = 704 101.9 -> 87.7 us; 16 splits, S = 768: 30.3 -> 28.2 us).
int workgroups_per_head(int S, int n, int cus) {
  const int ntiles = (S + TILE_T - 1) / TILE_T;
  const int fill = max(1, cus * WG_PER_CU / NH);
  const int one_round = (2 * cus / NH) / XCDS * XCDS;
  if ((int64_t)NH * ntiles <= cus) return ntiles;
  if (one_round > 0 && ntiles <= one_round) {
    const int last = S - (ntiles - 1) * TILE_T;
    const int short_tile = (S + one_round - 1) / one_round;
    if (n <= 128 && (int64_t)NH * (ntiles - 1) < cus && TILE_T + last < 2 * short_tile) return ntiles;
    return one_round;
  }
  if ((int64_t)NH * ntiles <= 2 * (int64_t)cus) return min(ntiles, fill);
  if (ntiles <= fill) return fill;
  if (2 * ntiles <= 3 * fill && one_round > 0) return one_round;
  return fill;
}

// Tokens per workgroup of the one-tile instance: 8 while that grid stays
// within 3 workgroups per CU, else 16 (with n > 8 the call then goes to the
// persistent kernel). Measured at 256 CUs with n = 4, 8 and 16: 8-token tiles
// are 8-19% faster up to S = 512 and 2-9% slower at S = 640 (1.25 waves of
// workgroups); 4-token tiles are slower than 8.
int latency_tile(int S, int cus) {
  const int64_t wg8 = (int64_t)NH * ((S + TILE_T / 2 - 1) / (TILE_T / 2));
  return wg8 <= 3 * (int64_t)cus ? TILE_T / 2 : TILE_T;
}

// 64-lane LSE chunks the persistent kernel is instantiated for.
int lse_chunks(int n) { return n <= 64 ? 1 : n <= 128 ? 2 : n <= 256 ? 4 : 8; }

// Tokens per workgroup of the split-rows kernel for a call with LSEs, or 0
// when the call does not take it: more partials than the one-tile instance
// holds, and at most half as many 16-token tiles as CUs (S <= 160 at 256
// CUs), 9/16 as many with 64 partials or more (S <= 192). The tile (8, 4, 2 or 1 tokens; at most SPLIT_NB batches of rows per
// wave) is the one whose busiest CU finishes first by a simple model: a CU
// runs ceil(grid / CUs) workgroups one after another, each costing a fixed
// SPLIT_ROUND_ROWS plus its tile's token rows (TT n). On a tie, the larger
// tile. Checked at 256 CUs against every tile forced in turn (17 to 512
// splits, S = 16 to 160): the model's tile was the fastest, or within 2.5%
// of it, at every point; the largest tile that fits one workgroup per CU
// lost up to 16% (a grid just past the CU count: 200 and 256 splits at S = 96),
// and tiles of at most 4 tokens and two batches up to 27%. Against the
// persistent kernel: S = 16 10.8 -> 5.5 us (17 splits), 24.7 -> 6.1 (64),
// 171.0 -> 21.8 (512); S = 160 13.1 -> 9.4 (17), 29.4 -> 20.0 (64), 212.4
// -> 163.3 (512). Past S = 160 the persistent kernel is 5-11% ahead with up
// to 32 splits (S = 176: 13.1 against 14.4 us with 17); with 64 to 512 the
// split-rows kernel is ahead or level up to S = 192 (S = 161, one round of
// 8-token tiles: 28.2 -> 19.4 us with 64, 52.2 -> 39.0 with 128; S = 176:
// 29.2 -> 28.7 with 64, level with 128, 208.9 -> 186.6 with 512) and within
// 2% either way at S = 256.
constexpr int SPLIT_ROUND_ROWS = 150;
int split_tile(int n, int S, int cus) {
  const int64_t ntiles = (S + TILE_T - 1) / TILE_T;
  const int64_t bound = (n >= 64 ? 9 : 8) * (int64_t)cus;  // 16 x 12 x tiles at most
  if (n <= 2 * LAT_NMAX || 16 * NH * ntiles > bound) return 0;
  const int nch = lse_chunks(n);
  int cap = WAVES;
  while (cap > 1 && split_batches(WAVES / cap, nch) > SPLIT_NB) cap /= 2;
  int best = cap;
  int64_t best_cost = INT64_MAX;
  for (int tt = cap; tt >= 1; tt /= 2) {
    const int64_t grid = (int64_t)NH * ((S + tt - 1) / tt);
    const int64_t cost = (grid + cus - 1) / cus * (SPLIT_ROUND_ROWS + (int64_t)tt * n);
    if (cost < best_cost) {
      best = tt;
      best_cost = cost;
    }
  }
  return best;
}

// The launch for a validated call with S > 0 on a device of `cus` CUs: the
// one-tile instance when one token tile per workgroup fills the device at
// most once and the instance can hold every row of a token, or when n == 2
// with LSEs; the split-rows kernel for many partials and few tokens; else
// the persistent kernel. One partial is copied. mla_post launches exactly
// this.
// Workgroups of the streaming kernel: as many as are resident at once, two
// per CU (its LDS), so that every CU holds two: workgroup b takes head
// b mod 12, and heads below (workgroups mod 12) get one workgroup more than
// the others (43 and 42 at 256 CUs). A grid of whole rounds of 12 (40 per
// head) left 32 of 256 CUs with one workgroup, which finished early and then
// idled (512 workgroups: 3-5% faster at S = 4096..16384).
constexpr int STREAM_WG_PER_CU = 2;
int stream_workgroups(int cus) { return max(NH, STREAM_WG_PER_CU * cus); }

// Whether the streaming kernel takes the call: one or two partials, no KV
// length masks, a layout where rows and LSEs move by a fixed stride per token
// (no request-major offset), each token's row past the previous one's end
// (o_st >= 512) and its LSEs past the previous ones (l_st >= 1), offsets
// within a tile below 2^31, and at least STREAM_MIN_TOKENS_PER_CU tokens per
// CU. Measured at 256 CUs against the one-tile and persistent kernels, with
// the large decode batch's distributions: ahead from S = 1536 with one
// partial (with an LSE: S = 1536 12.7 -> 10.6 us, 4096 20.2 -> 17.7, 8192
// 35.6 -> 29.9, 16384 66.1 -> 56.7; without: 8192 31.7 -> 29.6) and with two
// (S = 1536 14.8 -> 14.5, 4096 30.5 -> 28.1, 8192 56.4 -> 50.3, 16384 107.3
// -> 96.7), behind at S = 1024 (one partial 8.5 -> 9.0 us, two 10.6 -> 12.2).
constexpr int STREAM_MIN_TOKENS_PER_CU = 6;
bool stream_takes(const mla_post_args* a, int cus) {
  if (a->n > 2 || a->kv_lens || a->o_sr) return false;
  const int64_t lim = (int64_t(1) << 31) - 4096;
  if (a->o_st < KVL || a->o_st > lim / (2 * TILE_T)) return false;
  if (a->lse && (a->l_sr || a->l_st < 1 || a->l_st > lim / (8 * TILE_T) || a->l_sj > lim / 8)) return false;
  return (int64_t)a->S >= (int64_t)STREAM_MIN_TOKENS_PER_CU * cus;
}

mla_post_plan make_plan(const mla_post_args* a, int cus) {
  mla_post_plan p;
  memset(&p, 0, sizeof(p));
  p.cus = cus;
  if (stream_takes(a, cus)) {
    const int tt = TILE_T / a->n;
    p.kernel = MLA_POST_KERNEL_STREAM;
    p.tile_tokens = tt;
    p.rows_held = a->n;
    p.lse_chunks = 1;
    p.workgroups = stream_workgroups(cus);
    p.workgroups_per_head = (p.workgroups + NH - 1) / NH;
    if (tt == TILE_T)
      tile_counts<TILE_T>(a->S, p.workgroups_per_head, true, p.full_tiles, p.short_tokens);
    else
      tile_counts<TILE_T / 2>(a->S, p.workgroups_per_head, true, p.full_tiles, p.short_tokens);
    return p;
  }
  // one partial (with or without an LSE) is copied rather than merged
  const bool copy = a->n == 1;
  const int S = a->S, n = a->n;
  const int nch = lse_chunks(n);
  const int ntiles = (S + TILE_T - 1) / TILE_T;
  const int wph = workgroups_per_head(S, n, cus);
  // Two partials with LSEs take the one-tile instance at every size: a
  // 16-token tile then holds 2 rows per token (59 registers, 4 workgroups
  // per CU), and the device refills CUs with new workgroups as others end.
  // Measured against the persistent kernel: S = 2048 19.9 -> 16.9 us, equal
  // at 8192; with 3 or 4 splits it was slower beyond S = 1024. Up to S =
  // 2^20: a dispatch counts its work-items in 32 bits, and 12 workgroups of
  // 512 per 16 tokens would overflow that past S = 11M. One partial, with an
  // LSE or without, takes the copy instances (the one-tile one while it
  // fits, else the persistent kernel's): with an LSE, against merging it in
  // the one-tile instance as two partials are, S = 4096 26.8 -> 20.2 us,
  // S = 16384 94.7 -> 64.3 us, S = 256 6.3 -> 5.8 us.
  const bool fits = ntiles <= max(1, cus * WG_PER_CU / NH) && nch == 1;
  if (fits || (!copy && n <= 2 && S <= ONE_TILE_SMAX)) {
    const int tt = fits ? latency_tile(S, cus) : TILE_T;
    if (copy || n <= lat_nmax(tt)) {
      p.kernel = MLA_POST_KERNEL_ONE_TILE;
      p.tile_tokens = tt;
      // rows held per token: the fewest instantiated that hold all n (fewer
      // registers, so more workgroups resident at once)
      p.rows_held = copy ? 1 : n <= 2 ? 2 : n <= 4 ? 4 : n <= LAT_NMAX ? LAT_NMAX : 2 * LAT_NMAX;
      p.lse_chunks = 1;
      p.workgroups_per_head = (S + tt - 1) / tt;
      p.workgroups = NH * p.workgroups_per_head;
      return p;
    }
  }
  const int stt = copy ? 0 : split_tile(n, S, cus);
  if (stt > 0) {
    p.kernel = MLA_POST_KERNEL_SPLIT_ROWS;
    p.tile_tokens = stt;
    p.lse_chunks = nch;
    p.rows_held = min(SPLIT_RB, 64 * nch * stt / WAVES);
    p.workgroups_per_head = (S + stt - 1) / stt;
    p.workgroups = NH * p.workgroups_per_head;
    return p;
  }
  p.kernel = MLA_POST_KERNEL_PERSISTENT;
  p.tile_tokens = TILE_T;
  p.lse_chunks = nch;
  // n <= 4: both tokens' rows a tile ahead (the 8 slots hold all of them).
  // Measured with 1 to 4 splits: S = 4096 40.1 -> 29.5 us (n = 1), 41.3 ->
  // 31.2 (n = 2), 45.1 -> 39.4 (n = 4), S = 8192 by 14-30%. Eight rows of
  // each token for n <= 8 needs 141 registers, one resident workgroup per CU,
  // and was 20-30% slower with 6 and 8 splits.
  p.pair_rows = !copy && nch == 1 && n <= PF_ROWS / 2 ? PF_ROWS / 2 : 0;
  p.workgroups_per_head = wph;
  p.workgroups = NH * wph;
  tile_counts(S, wph, spread_leftover(copy, n), p.full_tiles, p.short_tokens);
  return p;
}

template <bool COPY, int TT>
int launch_one_tile(const KArgs& k, const mla_post_plan& p, hipStream_t stream) {
  const dim3 grid((unsigned)p.workgroups), block(THREADS);
  if constexpr (COPY) {
    return launch(mla_post_latency_kernel<true, TT, LAT_NMAX>, grid, block, stream, k);
  } else {
    if (p.rows_held == 2) return launch(mla_post_latency_kernel<false, TT, 2>, grid, block, stream, k);
    if (p.rows_held == 4) return launch(mla_post_latency_kernel<false, TT, 4>, grid, block, stream, k);
    if (p.rows_held == LAT_NMAX) return launch(mla_post_latency_kernel<false, TT, LAT_NMAX>, grid, block, stream, k);
    if constexpr (lat_nmax(TT) > LAT_NMAX)
      return launch(mla_post_latency_kernel<false, TT, 2 * LAT_NMAX>, grid, block, stream, k);
    return MLA_POST_EUNSUPPORTED;
  }
}

// Instances exist for the (tile, LSE chunks) pairs the plan can give; any
// other pair is refused (the plan never makes one).
template <int G, int NCH>
int launch_split(const KArgs& k, const mla_post_plan& p, hipStream_t stream) {
  if constexpr (split_batches(G, NCH) <= SPLIT_NB) {
    return launch(mla_post_split_kernel<G, NCH>, dim3((unsigned)p.workgroups), dim3(THREADS), stream, k);
  } else {
    return MLA_POST_EUNSUPPORTED;
  }
}

template <int G>
int launch_split_chunks(const KArgs& k, const mla_post_plan& p, hipStream_t stream) {
  switch (p.lse_chunks) {
    case 1: return launch_split<G, 1>(k, p, stream);
    case 2: return launch_split<G, 2>(k, p, stream);
    case 4: return launch_split<G, 4>(k, p, stream);
    default: return launch_split<G, 8>(k, p, stream);
  }
}

int launch_plan(const KArgs& k, const mla_post_plan& p, bool copy, hipStream_t stream) {
  if (p.kernel == MLA_POST_KERNEL_SPLIT_ROWS) {
    switch (p.tile_tokens) {
      case 8: return launch_split_chunks<1>(k, p, stream);
      case 4: return launch_split_chunks<2>(k, p, stream);
      case 2: return launch_split_chunks<4>(k, p, stream);
      default: return launch_split_chunks<8>(k, p, stream);
    }
  }
  if (p.kernel == MLA_POST_KERNEL_ONE_TILE) {
    if (p.tile_tokens == TILE_T)
      return copy ? launch_one_tile<true, TILE_T>(k, p, stream) : launch_one_tile<false, TILE_T>(k, p, stream);
    return copy ? launch_one_tile<true, TILE_T / 2>(k, p, stream) : launch_one_tile<false, TILE_T / 2>(k, p, stream);
  }
  const dim3 grid((unsigned)p.workgroups), block(THREADS);
  const int wph = p.workgroups_per_head;
  if (p.kernel == MLA_POST_KERNEL_STREAM)
    return copy ? launch(mla_post_stream_kernel<true, 1>, grid, block, stream, k)
                : launch(mla_post_stream_kernel<false, 2>, grid, block, stream, k);
  if (copy) return launch(mla_post_kernel<true, 1, 0>, grid, block, stream, k, wph);
  if (p.pair_rows == PF_ROWS / 2) return launch(mla_post_kernel<false, 1, PF_ROWS / 2>, grid, block, stream, k, wph);
  if (p.lse_chunks == 1) return launch(mla_post_kernel<false, 1, 0>, grid, block, stream, k, wph);
  if (p.lse_chunks == 2) return launch(mla_post_kernel<false, 2, 0>, grid, block, stream, k, wph);
  if (p.lse_chunks == 4) return launch(mla_post_kernel<false, 4, 0>, grid, block, stream, k, wph);
  return launch(mla_post_kernel<false, 8, 0>, grid, block, stream, k, wph);
}

}  // namespace

extern "C" {

int mla_post_check(const mla_post_args* a) { return check_args(a); }

int mla_post(const mla_post_args* in, void* stream) {
  const int st = check_args(in);
  if (st != MLA_POST_OK || in->S == 0) return st;
  mla_post_args na;
  normalize(in, &na);
  const mla_post_args* a = &na;
  KArgs k;
  k.o = static_cast<const uint8_t*>(a->o);
  k.o_sj = a->o_sj * 2;
  k.o_st = a->o_st * 2;
  k.o_sh = a->o_sh * 2;
  k.lse = a->lse;
  k.l_sj = a->l_sj;
  k.l_st = a->l_st;
  k.l_sh = a->l_sh;
  k.w_v = a->w_v;
  k.w_sh = a->w_sh;
  k.w_sv = a->w_sv;
  k.w_vs = a->w_v_scale;
  k.s_sh = a->s_sh;
  k.s_sv = a->s_sv;
  k.s_sb = a->s_sb;
  k.gate = static_cast<const uint8_t*>(a->gate);
  k.core = static_cast<uint8_t*>(a->core);
  k.dbg_lat = static_cast<uint8_t*>(a->dbg_lat);
  k.dbg_codes = static_cast<uint8_t*>(a->dbg_codes);
  k.dbg_scales = static_cast<uint8_t*>(a->dbg_scales);
  k.n = a->n;
  k.S = a->S;
  k.q = a->q > 1 ? a->q : 1;
  k.o_sr = a->o_sr * 2;
  k.l_sr = a->l_sr;
  k.kv_lens = a->kv_lens;
  k.kl_sj = a->kl_sj;
  k.qsl = a->qsl;
  return launch_plan(k, make_plan(a, device_cus()), a->n == 1, static_cast<hipStream_t>(stream));
}

int mla_post_plan_for(const mla_post_args* in, int32_t cus, mla_post_plan* out) {
  if (!out) return MLA_POST_EINVAL;
  const int st = check_args(in);
  if (st != MLA_POST_OK) return st;
  const int c = cus > 0 ? cus : device_cus();
  if (in->S == 0) {
    memset(out, 0, sizeof(*out));
    out->cus = c;
    return MLA_POST_OK;
  }
  mla_post_args na;
  normalize(in, &na);
  *out = make_plan(&na, c);
  return MLA_POST_OK;
}

int mla_quantize_mxfp4(const void* x, int64_t rows, int32_t cols, int64_t x_stride, uint8_t* codes, int64_t c_stride,
                       uint8_t* scales, int64_t s_stride, void* stream) {
  if (rows < 0 || cols < 0) return MLA_POST_EINVAL;
  if (rows == 0 || cols == 0) return MLA_POST_OK;
  if (!x || !codes || !scales) return MLA_POST_EINVAL;
  if ((cols % 32) || cols > 8192) return MLA_POST_EUNSUPPORTED;
  if (rows > (int64_t(1) << 34)) return MLA_POST_ERANGE;
  if (x_stride < 0 || c_stride < 0 || s_stride < 0 || (x_stride % 8) || (c_stride % 4)) return MLA_POST_ESTRIDE;
  if (!aligned(x, 16) || !aligned(codes, 4)) return MLA_POST_EALIGN;
  int64_t xsb;
  if (!mul_ok(x_stride, 2, &xsb) || !span_ok(rows, xsb, 1, 0, 1, 0, (int64_t)cols * 2) ||
      !span_ok(rows, c_stride, 1, 0, 1, 0, cols / 2) ||
      !span_ok(rows, s_stride, 1, 0, 1, 0, cols / 32))
    return MLA_POST_ERANGE;
  // at most 2^16 workgroups, each wave striding over the rows: the grid's
  // work-item count must fit the 32 bits of a dispatch
  const int64_t blocks = std::min<int64_t>((rows + QWAVES - 1) / QWAVES, QMAX_BLOCKS);
  return launch(quantize_kernel, dim3((unsigned)blocks), dim3(QWAVES * 64), static_cast<hipStream_t>(stream),
                static_cast<const uint8_t*>(x), rows, cols, (int64_t)(x_stride * 2), codes, c_stride, scales, s_stride);
}

const char* mla_post_strerror(int status) {
  switch (status) {
    case MLA_POST_OK: return "ok";
    case MLA_POST_EINVAL: return "invalid argument (null pointer, size out of range, or lse NULL with n > 1)";
    case MLA_POST_ESTRIDE: return "stride negative or not a multiple the vector loads need";
    case MLA_POST_EALIGN: return "pointer not aligned for its vector loads or stores";
    case MLA_POST_ERANGE: return "an operand's byte offsets overflow 64-bit arithmetic";
    case MLA_POST_EUNSUPPORTED: return "unsupported size (n above MLA_POST_NMAX, or cols not a multiple of 32)";
    case MLA_POST_ELAUNCH: return "HIP launch failed";
    default: return "unknown status";
  }
}

const char* mla_post_last_hip_error(void) { return mla_dev::g_hip_error.c_str(); }

int mla_post_version(void) { return MLA_POST_VERSION; }

}  // extern "C"
