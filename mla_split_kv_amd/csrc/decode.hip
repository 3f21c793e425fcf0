// mla_decode: split-KV MLA decode attention fused with mla_post, for AMD
// MI355X (gfx950).
//
// The vLLM API-docs page for module
// vllm.models.kimi_k3.amd.specialized_decode.mono.attention.mla_back has its
// merge + W_UV consume the split partials of an attention kernel (M1c), and
// runs both in one launch (module docstring: K2; combine_splits,
// combine_tasks, stage_uv). The attention computed here is the plainest one
// with those outputs (include/mla_decode.h states it); the merge and W_UV
// are mla_post's arithmetic, from the same device helpers.
//
// One workgroup of 4 waves per (request, split) unit:
//   queries: the unit's q x 12 query rows (token tt, head h as row
//     12 tt + h) in tiles of 16, one tile per wave (waves past the last tile
//     only stage KV); a wave keeps its 16 queries' 576 dims in registers as
//     the B operand of the score MFMAs;
//   KV: blocks of 64 cache rows through two LDS buffers (1168-byte rows, 16 B
//     of skew), every thread holding its share of the next block in
//     registers while the waves compute on this one; one barrier per block;
//   scores: S^T[kv][query] = K . Q^T with v_mfma_f32_16x16x32_bf16 (18 steps
//     over the 576 dims, 4 tiles of 16 rows); online softmax in base 2 per
//     query column (running max and sum, cross-lane by shuffles);
//   values: O^T[col][query] += V^T . P^T: the MFMA's K index runs over the
//     block's kv rows in the order the score tiles leave them in the lanes
//     (a sum, so any order both operands share is correct), so P needs no
//     shuffle; the V^T operand is gathered from the staged rows 2 bytes at a
//     time (8 rows per operand);
//   partials: O / sum rounded to bf16 and the natural-log LSE into the
//     workspace, request-major.
// Fused, each unit then fences its partials at device scope and adds 1 to
// its request's counter; the workgroup that completes the count merges the
// request's partials (mla_post's weights, float32 sums in split order, bf16
// latents, MXFP4 by the hardware scaled convert), runs the scaled FP4 MFMAs
// against W_V for all 12 heads, gates and writes core, and resets the
// counter. No workgroup waits for another.
// Units are numbered so that the splits of one request run on one XCD (the
// device deals workgroup b to XCD b mod 8), behind one L2.

#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <atomic>

#include "device.h"
#include "launch.h"
#include "mla_decode.h"
#include "mla_post.h"
#include "post_common.h"

namespace {

using mla_dev::launch;

constexpr int NH = MLA_POST_HEADS;
constexpr int KVL = MLA_POST_KVL;
constexpr int VD = MLA_POST_VD;
constexpr int GROWS = MLA_POST_GROWS;
constexpr int NBLK = KVL / 32;               // MXFP4 blocks per latent row
constexpr int DQK = MLA_DECODE_DQK;          // 576
constexpr int DW = 4;                        // waves per workgroup
constexpr int DTHREADS = DW * 64;
constexpr int BC = 32;                       // KV rows per block (one MFMA K step of the value product)
constexpr float RESCALE_AT = 8.f;            // base-2 headroom of the softmax reference
constexpr int NBUF = 2;                      // LDS blocks: the one computed on and the next in flight
constexpr int MROW = KVL * 2 + 16;           // LDS bytes per block row of the 512 latent dims (+16 B skew)
constexpr int TROW = (DQK - KVL) * 2;        // LDS bytes per block row of the 64 rotary dims
constexpr int TAIL = BC * MROW;              // offset of a block's rotary part
constexpr int BLOCK_BYTES = TAIL + BC * TROW;  // one LDS block
constexpr int LOADS_PER_WAVE = BC / DW + BC / 8 / DW;  // a wave's 16-byte-per-lane loads of one block
constexpr int KSTEPS = DQK / 32;             // score MFMA steps over the 576 dims
constexpr int NCOLT = KVL / 16;              // value column tiles (32)
constexpr float LN2 = 0.69314718055994530942f;
constexpr float LOG2E = 1.44269504088896340736f;
// consumer LDS (reuses the KV buffers): codes and scales of 12 heads, core rows
constexpr int CODE_ROW = 16 * 16 + 16;       // LDS bytes per MXFP4 block row of 16 token slots
constexpr int LDS_CODES = NBLK * CODE_ROW;
constexpr int LDS_SCALES = 16 * NBLK;
constexpr int CORE_ROW = GROWS * 2 + 16;
constexpr int LDS_BYTES = NBUF * BLOCK_BYTES;
static_assert(BC % (8 * DW) == 0 && LOADS_PER_WAVE <= 15, "whole loads per wave; the waits count them");
static_assert(NH * (LDS_CODES + LDS_SCALES) + ((MLA_DECODE_QMAX + 1) * CORE_ROW > MLA_DECODE_QMAX * NH * 64 * 4
                                                    ? (MLA_DECODE_QMAX + 1) * CORE_ROW
                                                    : MLA_DECODE_QMAX * NH * 64 * 4) <= LDS_BYTES,
              "consumer fits the KV buffers (merge weights and staged core rows share bytes)");

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Cache policy of the partials' stores and loads: coherent at device (agent)
// scope (sc1), so the units of a request and the unit that merges them
// exchange the partials without writing back or invalidating whole caches.
constexpr int CPOL_AGENT = 16;
// Cache policy of the KV rows: non-temporal (each row is read once per
// split), so the stream does not push the queries, the partials on their
// way to the merge and W_V out of the L2 (measured on the large decode batch:
// the fused launch 1290 -> 1208-1219 us, the attention alone 1186 -> 1174).
constexpr int CPOL_NT = 2;

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt in
// 6:4, lgkmcnt in 11:8): wait until at most n vector memory operations are
// outstanding; wait for every LDS operation.
constexpr int WAITCNT_VM(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int WAITCNT_LGKM0 = 15 | (3 << 14) | (7 << 4);

// A workgroup barrier for LDS hazards alone: the wave's LDS operations are
// complete, then s_barrier (__syncthreads also waits for every vector memory
// operation in flight). The empty asm statements keep the compiler from
// moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(WAITCNT_LGKM0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

struct DArgs {
  const uint8_t* qry;
  int64_t q_st, q_sh;  // bytes
  const uint8_t* kv;
  int64_t kv_st;  // bytes
  const int32_t* indptr;
  float scale2;  // softmax scale times log2(e)
  int32_t R, q, n;
  const uint8_t* w_v;
  int64_t w_sh, w_sv;
  const uint8_t* w_vs;
  int64_t s_sh, s_sv, s_sb;
  const uint8_t* gate;
  uint8_t* core;
  int32_t* cnt;
  uint8_t* po;  // partials bf16 [R, n, q, 12, 512]
  float* pl;    // LSEs [R, n, q, 12]
  uint8_t* dbg_lat;
  uint8_t* dbg_codes;
  uint8_t* dbg_scales;
};

// Row of split j of token tt (of request r), head h in the workspace.
__device__ __forceinline__ int64_t part_row(const DArgs& a, int r, int j, int tt, int h) {
  return ((int64_t)(r * a.n + j) * a.q + tt) * NH + h;
}

__device__ __forceinline__ float xor_max(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}

__device__ __forceinline__ float xor_sum(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}


// ---------------------------------------------------------------- the consumer

// The merge + W_UV + gate of request r's tokens, from the workspace's n
// partials per (token, head) (mla_post's steps and helpers). It runs once per
// request, in whichever unit completes the request, so it is written as
// compact loops: unrolled code of this size would be fetched anew from L2 at
// every run (the instruction cache holds the attention loop), which measured
// several times slower than its memory round trips.
__device__ void consume(const DArgs& a, int r, uint8_t* lds) {
  int tid = threadIdx.x;  // opaque, as in decode_unit
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  uint8_t* s_codes = lds;                        // [12][LDS_CODES]
  uint8_t* s_scales = lds + NH * LDS_CODES;      // [12][16 slots][16 blocks]
  uint8_t* s_core = s_scales + NH * LDS_SCALES;  // [q + 1 spare][CORE_ROW]
  // [4 waves][12][64] weights, in the same bytes as s_core: read only by the
  // merge, s_core written only after the barrier that ends it
  float* s_w = reinterpret_cast<float*>(s_core);
  const int qrows = NH * a.q;
  // token slots past q: zero codes, scale code 1 (MFMA columns of zeros)
  for (int i = tid; i < NH * NBLK * (16 - a.q); i += DTHREADS) {
    const int h = i / (NBLK * (16 - a.q)), rest = i % (NBLK * (16 - a.q));
    const int b = rest / (16 - a.q), slot = a.q + rest % (16 - a.q);
    *reinterpret_cast<uint4*>(s_codes + h * LDS_CODES + b * CODE_ROW + slot * 16) = make_uint4(0u, 0u, 0u, 0u);
    s_scales[h * LDS_SCALES + slot * NBLK + b] = 1;
  }
  // merge: wave w takes (token, head) rows p = w, w + 4, .. (np of them), the
  // partial rows of two (token, head) pairs at a time (32 rows in flight).
  // The LSE loads go out first, then the first pair's rows, so the weights
  // are computed while those rows are in flight; the weights wait in LDS.
  const __amdgpu_buffer_rsrc_t rres = __builtin_amdgcn_make_buffer_rsrc(
      a.po + part_row(a, r, 0, 0, 0) * (KVL * 2), (short)0, a.n * qrows * KVL * 2, BUF_WORD3);
  const int np = (qrows - wave + DW - 1) / DW;  // wave-uniform, at most 12
  float* w_wave = s_w + wave * (MLA_DECODE_QMAX * NH / DW) * 64;
  uint4 v[2][16];
  // every row is loaded (an empty split's partial is +0, written by its
  // unit), then added with its weight: a weight of 0 adds +0, which leaves
  // the sum's bits as skipping the row would (the sum starts at +0 and never
  // becomes -0). The rows are read once: non-temporal (measured: the fused
  // launch 1207 -> 1188 us on the large decode batch)
  auto load_rows = [&](int i0, int j0) {
    const int p0 = wave + DW * i0, p1 = wave + DW * min(i0 + 1, np - 1);
#pragma unroll
    for (int b = 0; b < 16; ++b) {
      const int j = min(j0 + b, a.n - 1);
      const v4u x0 = (v4u)__builtin_amdgcn_raw_buffer_load_b128(
          rres, (int)(part_row(a, 0, j, p0 / NH, p0 % NH) * (KVL * 2)) + lane * 16, 0, CPOL_AGENT | CPOL_NT);
      const v4u x1 = (v4u)__builtin_amdgcn_raw_buffer_load_b128(
          rres, (int)(part_row(a, 0, j, p1 / NH, p1 % NH) * (KVL * 2)) + lane * 16, 0, CPOL_AGENT | CPOL_NT);
      v[0][b] = make_uint4(x0.x, x0.y, x0.z, x0.w);
      v[1][b] = make_uint4(x1.x, x1.y, x1.z, x1.w);
    }
  };
  {
    // every lane loads (split min(lane, n - 1) of pair min(i, np - 1)) and
    // takes -inf where the split or the pair does not exist: no branch
    // around the loads
    float l[MLA_DECODE_QMAX * NH / DW];
#pragma unroll
    for (int i = 0; i < MLA_DECODE_QMAX * NH / DW; ++i) {
      const int p = wave + DW * min(i, np - 1);
      l[i] = __hip_atomic_load(a.pl + part_row(a, r, min(lane, a.n - 1), p / NH, p % NH), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
    load_rows(0, 0);
#pragma unroll
    for (int i = 0; i < MLA_DECODE_QMAX * NH / DW; ++i)
      w_wave[i * 64 + lane] = (i < np && lane < a.n) ? sane(l[i]) : -INFINITY;
  }
#pragma unroll 1
  for (int i = 0; i < np; ++i) {
    float w1[1] = {w_wave[i * 64 + lane]};
    lse_to_weights<1>(w1);
    w_wave[i * 64 + lane] = w1[0];
  }
#pragma unroll 1
  for (int i0 = 0; i0 < np; i0 += 2) {
    float acc[2][8];
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[e][k] = 0.f;
#pragma unroll 1
    for (int j0 = 0; j0 < a.n; j0 += 16) {
      if (i0 | j0) load_rows(i0, j0);  // the first pair's rows are in flight already
#pragma unroll
      for (int b = 0; b < 16; ++b) {
        const int j = j0 + b;
        const float wa = j < a.n ? w_wave[i0 * 64 + (j & 63)] : 0.f;
        const float wb = j < a.n ? w_wave[min(i0 + 1, np - 1) * 64 + (j & 63)] : 0.f;
        fma_row(wa, v[0][b], acc[0]);
        fma_row(wb, v[1][b], acc[1]);
      }
    }
    const int p0 = wave + DW * i0, p1 = wave + DW * min(i0 + 1, np - 1);
#pragma unroll 1
    for (int e = 0; e < 2 && i0 + e < np; ++e) {
      const int p = e ? p1 : p0;
      const int tt = p / NH, h = p % NH;
      uint32_t lat[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) lat[k] = pack_bf16(e ? acc[1][2 * k] : acc[0][2 * k], e ? acc[1][2 * k + 1] : acc[0][2 * k + 1]);
      int code;
      const uint32_t pk = quant8(lat, code);
      const int b = lane >> 2;
      *reinterpret_cast<uint32_t*>(s_codes + h * LDS_CODES + b * CODE_ROW + tt * 16 + (lane & 3) * 4) = pk;
      if ((lane & 3) == 0) s_scales[h * LDS_SCALES + tt * NBLK + (b & 3) * 4 + (b >> 2)] = (uint8_t)code;
      const int64_t th = (int64_t)(r * a.q + tt) * NH + h;
      if (a.dbg_lat)
        reinterpret_cast<uint4*>(a.dbg_lat + th * (KVL * 2))[lane] = make_uint4(lat[0], lat[1], lat[2], lat[3]);
      if (a.dbg_codes) reinterpret_cast<uint32_t*>(a.dbg_codes + th * (KVL / 2))[lane] = pk;
      if (a.dbg_scales && (lane & 3) == 0) a.dbg_scales[th * NBLK + b] = (uint8_t)code;
    }
  }
  // W_UV: wave w takes heads w, w + 4, w + 8; per head 8 tiles of 16 W_V
  // rows. The head's W_V operands for all 8 row tiles come in one round
  // trip; the first head's are requested before the barrier that ends the
  // merge (which waits for LDS only), so they are in flight while the other
  // waves finish it.
  const int tl = lane & 15, kb = lane >> 4;
  const int tok = min(tl, a.q - 1);  // gate row of this lane's column (columns past q are never stored)
  uint4 wv[VD / 16][4];
  int sa[VD / 16];
  auto load_head = [&](int h) {
#pragma unroll
    for (int rt = 0; rt < VD / 16; ++rt) {
      const int vrow = rt * 16 + tl;
      const uint8_t* wrow = a.w_v + h * a.w_sh + vrow * a.w_sv + kb * 16;
      const uint8_t* srow = a.w_vs + h * a.s_sh + vrow * a.s_sv;
      sa[rt] = 0;
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        wv[rt][st] = *reinterpret_cast<const uint4*>(wrow + st * 64);
        sa[rt] |= (int)srow[(st * 4 + kb) * a.s_sb] << (8 * st);
      }
    }
  };
  load_head(wave);
  lds_barrier();
#pragma unroll 1
  for (int h = wave; h < NH; h += DW) {
    if (h != wave) load_head(h);
    // the gate values, used after the MFMAs
    uint2 g4[VD / 16];
#pragma unroll
    for (int rt = 0; rt < VD / 16; ++rt)
      g4[rt] = *reinterpret_cast<const uint2*>(a.gate + ((int64_t)(r * a.q + tok) * GROWS + h * VD + rt * 16 + kb * 4) * 2);
    const int sb = *reinterpret_cast<const int*>(s_scales + h * LDS_SCALES + tl * NBLK + kb * 4);
    const uint8_t* brow = s_codes + h * LDS_CODES + tl * 16;
#pragma unroll
    for (int rt = 0; rt < VD / 16; ++rt) {
      v4f acc = {0.f, 0.f, 0.f, 0.f};
      acc = mfma_step<0>(wv[rt][0], *reinterpret_cast<const uint4*>(brow + (0 * 4 + kb) * CODE_ROW), acc, sa[rt], sb);
      acc = mfma_step<1>(wv[rt][1], *reinterpret_cast<const uint4*>(brow + (1 * 4 + kb) * CODE_ROW), acc, sa[rt], sb);
      acc = mfma_step<2>(wv[rt][2], *reinterpret_cast<const uint4*>(brow + (2 * 4 + kb) * CODE_ROW), acc, sa[rt], sb);
      acc = mfma_step<3>(wv[rt][3], *reinterpret_cast<const uint4*>(brow + (3 * 4 + kb) * CODE_ROW), acc, sa[rt], sb);
      // rows 16 rt + 4 kb + i of token column tl: bf16(bf16(acc) * gate),
      // staged in LDS by every lane (columns past q go to a spare row that is
      // never written out), so the MFMAs' result is used unconditionally
      const int col = h * VD + rt * 16 + kb * 4;
      const uint2 ab = make_uint2(pack_bf16(acc[0], acc[1]), pack_bf16(acc[2], acc[3]));
      const uint2 cv = make_uint2(pack_bf16(bf_lo(ab.x) * bf_lo(g4[rt].x), bf_hi(ab.x) * bf_hi(g4[rt].x)),
                                  pack_bf16(bf_lo(ab.y) * bf_lo(g4[rt].y), bf_hi(ab.y) * bf_hi(g4[rt].y)));
      *reinterpret_cast<uint2*>(s_core + (tl < a.q ? tl : MLA_DECODE_QMAX) * CORE_ROW + col * 2) = cv;
    }
  }
  __syncthreads();
  // core rows of the request's tokens: 16-byte pieces
  for (int i = tid; i < a.q * (GROWS * 2 / 16); i += DTHREADS) {
    const int tt = i / (GROWS * 2 / 16), c = (i % (GROWS * 2 / 16)) * 16;
    store_nt16(a.core + (int64_t)(r * a.q + tt) * (GROWS * 2) + c, *reinterpret_cast<const uint4*>(s_core + tt * CORE_ROW + c));
  }
}

// ---------------------------------------------------------------- the attention (and the fused launch)

// One thread's atomic add of 1 at device scope, returning the old value.
// The address is made a per-lane value, so the compiler issues the one
// atomic as it stands instead of its wave-wide form, which takes the
// returned value at once (a wait for the round trip where the atomic is
// issued rather than where its value is used).
__device__ __forceinline__ int count_in(int32_t* c) {
  int zero = 0;
  asm volatile("" : "+v"(zero));
  return __hip_atomic_fetch_add(c + zero, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Thread 0's claim of the workgroup's next unit: the queue counter's old
// value.
__device__ __forceinline__ int claim_unit(int32_t* q_next) { return count_in(q_next); }

// One unit: the attention of request r's split j (and, fused, the merge of
// request r when this unit completes it). lds: the workgroup's LDS (KV
// blocks, then the consumer's buffers); s_last, s_next: words past them.
// Thread 0 claims the workgroup's next unit and puts the claim in s_next
// before the unit's end. Attention alone: the claim is `next`, issued before
// the unit's loads, and is stored once the KV loop has waited for every load
// (so for the claim too). Fused: the claim goes out with the partial stores
// (a claim held through the KV loop would take one of the registers the
// loop has none left of), and the wait for the stores covers it.
//
// Handoff. The partials are written coherent at device scope (sc1,
// write-through to the device's coherence point); every wave waits for its
// stores to complete before the barrier that precedes the counter's atomic
// add, as a device-scope release (a writeback of the whole L2, then the same
// wait) would order them, without the writeback. The workgroup that brings
// the counter to n merges the request at once (consume), reading the
// partials with sc1 loads, which a stale line cannot satisfy, in place of a
// device-scope acquire (an invalidation of the whole L2). (Counting a unit
// in one unit later, after the next unit's KV loop has waited for its
// stores, measured 5% slower: the merges then read partials written a unit
// earlier, and took 10% longer.)
template <bool FUSED>
__device__ __forceinline__ void decode_unit(const DArgs& a, int r, int j, uint8_t* lds, int* s_last, int* s_next,
                                            int32_t* q_next, int next) {
  // the thread index as the compiler cannot tell from one unit to the next:
  // values derived from it are then computed within the unit, not hoisted
  // out of the unit loop and held (spilled) across it
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qrows = NH * a.q;
  // indptr does not change during the launch: read through the constant
  // address space, as scalar loads
  typedef const __attribute__((address_space(4))) int32_t const_i32;
  const_i32* ip = (const_i32*)(uintptr_t)a.indptr;
  const int base = ip[r];
  const int L = max(ip[r + 1] - base, 0);
  const int k0 = base + (int)((int64_t)j * L / a.n);
  const int nrows = base + (int)((int64_t)(j + 1) * L / a.n) - k0;
  const int nblk = (nrows + BC - 1) / BC;
  const int g = lane >> 4, c16 = lane & 15;
  const int qi = wave * 16 + c16;            // this lane's query row
  const bool compute = wave * 16 < qrows;    // wave-uniform

  // the 16 queries of this wave, as score MFMA B operands (lane: query c16,
  // dims 32 k + 8 g .. + 7 of step k); rows past the unit's are zero
  bf16x8 qreg[KSTEPS];
  {
    const int tt = min(qi / NH, a.q - 1), h = qi % NH;
    const uint8_t* qp = a.qry + (int64_t)(r * a.q + tt) * a.q_st + (int64_t)h * a.q_sh + g * 16;
    const bool live = compute && qi < qrows;
#pragma unroll
    for (int k = 0; k < KSTEPS; ++k) {
      uint4 x = make_uint4(0u, 0u, 0u, 0u);
      if (live) x = *reinterpret_cast<const uint4*>(qp + k * 64);
      qreg[k] = __builtin_bit_cast(bf16x8, x);
    }
  }

  // KV block b into LDS block b mod NBUF by direct loads (buffer_load ... lds:
  // lane i of an instruction writes 16 bytes at the instruction's LDS address
  // + 16 i, no registers). Wave w loads the 512 latent dims of rows w, w + 4,
  // .. (one instruction per row: 64 lanes x 16 B) and the 64 rotary dims of
  // rows 8 w .. 8 w + 7 (one instruction: 8 lanes per row). Rows past the
  // split's end load the split's last row instead (their scores are masked
  // to -inf, so their probabilities are 0 and their finite values add 0).
  const int vlane16 = lane * 16;
  int tail_off = 0;  // the rotary loads' per-lane offset, kept live until the block's reads are done
  auto load_block = [&](int b) {
    const int rows = min(nrows - b * BC, BC);  // 0 for block 0 of an empty split: nothing is read
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(a.kv + (int64_t)(k0 + b * BC) * a.kv_st), (short)0,
        rows > 0 ? (rows - 1) * (int)a.kv_st + DQK * 2 : 0, BUF_WORD3);
    uint8_t* dst = lds + (b % NBUF) * BLOCK_BYTES;
    // the row's offset is the same for the whole wave: the scalar offset;
    // the lane's, fixed for the launch, the vector one (so no vector
    // register is written per block for them, which the compiler would then
    // have to keep from reuse until the loads had read it)
#pragma unroll
    for (int i = 0; i < BC / DW; ++i) {
      const int row = wave + DW * i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(dst + row * MROW), 16, vlane16,
                                               max(min(row, rows - 1), 0) * (int)a.kv_st, 0, CPOL_NT);
    }
#pragma unroll
    for (int i = 0; i < BC / 8 / DW; ++i) {
      const int grp = wave + DW * i;  // rows 8 grp .. 8 grp + 7
      tail_off = max(min(8 * grp + (lane >> 3), rows - 1), 0) * (int)a.kv_st + KVL * 2 + (lane & 7) * 16;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(dst + TAIL + 8 * grp * TROW), 16, tail_off, 0, 0,
                                               CPOL_NT);
    }
  };

  // Online softmax in base 2 with a lazily raised reference: p = 2^(s - m2),
  // m2 raised (and the sums rescaled) only when a score exceeds it by more
  // than RESCALE_AT, so most blocks skip the rescale of the 128 accumulator
  // registers; p stays below 2^RESCALE_AT, far inside float32 and bf16 range,
  // and the final division by the sum of the same p cancels the reference.
  float m2 = -INFINITY, lsum = 0.f;  // query qi's reference (base-2 units) and sum
  v4f acc[NCOLT];                    // O^T: value columns 16 c + 4 g + i, query c16
#pragma unroll
  for (int c = 0; c < NCOLT; ++c) acc[c] = v4f{0.f, 0.f, 0.f, 0.f};
  // Block 0's loads (issued even for an empty split, reading nothing, so
  // that the count of loads in flight is known here), then the queries are
  // waited for (block 0 stays in flight; the compiler then knows the queries
  // are in registers and does not wait again inside the loop), then blocks 1
  // and 2.
  load_block(0);
#pragma unroll
  for (int k = 0; k < KSTEPS; k += 6) {
    const uint4 q0 = __builtin_bit_cast(uint4, qreg[k]), q1 = __builtin_bit_cast(uint4, qreg[k + 1]),
                q2 = __builtin_bit_cast(uint4, qreg[k + 2]), q3 = __builtin_bit_cast(uint4, qreg[k + 3]),
                q4 = __builtin_bit_cast(uint4, qreg[k + 4]), q5 = __builtin_bit_cast(uint4, qreg[k + 5]);
    asm volatile("" ::"v"(q0.x), "v"(q1.x), "v"(q2.x), "v"(q3.x), "v"(q4.x), "v"(q5.x));
  }
  for (int b = 1; b < min(nblk, NBUF - 1); ++b) load_block(b);
  auto block = [&](int b) {
    // Block b is complete when at most the loads of the blocks issued after
    // it are outstanding (vector memory operations complete in order); then
    // every wave's share of it is, after the barrier. The barrier also tells
    // every wave that all of them are done reading block b - 1, whose LDS
    // block the loads of block b + NBUF - 1 reuse. The LDS reads of block
    // b - 1 have returned (lgkmcnt(0)) before a wave reaches it.
    const int later = min(nblk - 1 - b, NBUF - 2);
    if (later >= 2)
      __builtin_amdgcn_s_waitcnt(WAITCNT_VM(2 * LOADS_PER_WAVE));
    else if (later == 1)
      __builtin_amdgcn_s_waitcnt(WAITCNT_VM(LOADS_PER_WAVE));
    else
      __builtin_amdgcn_s_waitcnt(WAITCNT_VM(0));
    __builtin_amdgcn_s_barrier();
    if (b + NBUF - 1 < nblk) load_block(b + NBUF - 1);
    const uint8_t* blk = lds + (b % NBUF) * BLOCK_BYTES;
    if (compute) {
      // scores: tile t holds kv rows 16 t + 4 g + i for query c16; dims
      // 0..511 from the latent part, 512..575 from the rotary part
      v4f s[BC / 16];
#pragma unroll
      for (int t = 0; t < BC / 16; ++t) s[t] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < KSTEPS; ++k)
#pragma unroll
        for (int t = 0; t < BC / 16; ++t) {
          const int row = 16 * t + c16;
          const uint8_t* ap = k < KVL / 32 ? blk + row * MROW + k * 64 + g * 16
                                           : blk + TAIL + row * TROW + (k - KVL / 32) * 64 + g * 16;
          s[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8*>(ap), qreg[k], s[t], 0, 0, 0);
        }
      const int valid = nrows - b * BC;
      float bmax = -INFINITY;
#pragma unroll
      for (int t = 0; t < BC / 16; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float x = (16 * t + 4 * g + i < valid) ? s[t][i] * a.scale2 : -INFINITY;
          s[t][i] = x;
          bmax = fmaxf(bmax, x);
        }
      bmax = xor_max(bmax);  // finite: a block has a valid row
      if (__any(bmax > m2 + RESCALE_AT)) {  // wave-uniform
        const float mn = fmaxf(m2, bmax);
        const float alpha = exp2f(m2 - mn);  // 0 on the first block
        lsum *= alpha;
#pragma unroll
        for (int c = 0; c < NCOLT; ++c) acc[c] *= alpha;
        m2 = mn;
      }
      float rs = 0.f;
#pragma unroll
      for (int t = 0; t < BC / 16; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = exp2f(s[t][i] - m2);
          s[t][i] = p;
          rs += p;
        }
      lsum += xor_sum(rs);
      // P^T operand: kv rows 4 g + i, then 16 + 4 g + i (the score tiles'
      // own lane order; the V^T operand takes the same rows)
      const bf16x8 pb = bf16x8{(__bf16)s[0][0], (__bf16)s[0][1], (__bf16)s[0][2], (__bf16)s[0][3],
                               (__bf16)s[1][0], (__bf16)s[1][1], (__bf16)s[1][2], (__bf16)s[1][3]};
      // V^T operands by transposed LDS reads: in each 16-lane group, lane i
      // points at row base + i / 4, columns 16 c + 4 (i mod 4) .. + 3, and
      // lane j receives rows base .. base + 3 of column 16 c + j. The reads
      // are issued by hand, four column tiles at a time, each batch ending in
      // its own wait for them: the compiler cannot tell which LDS block the
      // builtin's reads touch, so for it it waits for every load in flight
      // (the next blocks' too) first. Block b is complete and visible here
      // (the wait and barrier above), and the next barrier comes after this
      // wave's reads have returned. The outputs are early-clobber: the first
      // read's result lands while later reads still use the address.
      const uint32_t vaddr = (uint32_t)(uintptr_t)(lds + (b % NBUF) * BLOCK_BYTES + (4 * g + (c16 >> 2)) * MROW +
                                                   (c16 & 3) * 8);
#pragma unroll
      for (int c0 = 0; c0 < NCOLT; c0 += 4) {
        v2u lo0, lo1, lo2, lo3, hi0, hi1, hi2, hi3;
        asm volatile(
            "ds_read_b64_tr_b16 %0, %8 offset:%9\n"
            "ds_read_b64_tr_b16 %1, %8 offset:%10\n"
            "ds_read_b64_tr_b16 %2, %8 offset:%11\n"
            "ds_read_b64_tr_b16 %3, %8 offset:%12\n"
            "ds_read_b64_tr_b16 %4, %8 offset:%13\n"
            "ds_read_b64_tr_b16 %5, %8 offset:%14\n"
            "ds_read_b64_tr_b16 %6, %8 offset:%15\n"
            "ds_read_b64_tr_b16 %7, %8 offset:%16\n"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(lo0), "=&v"(lo1), "=&v"(lo2), "=&v"(lo3), "=&v"(hi0), "=&v"(hi1), "=&v"(hi2), "=&v"(hi3)
            : "v"(vaddr), "i"(32 * c0), "i"(32 * c0 + 32), "i"(32 * c0 + 64), "i"(32 * c0 + 96),
              "i"(16 * MROW + 32 * c0), "i"(16 * MROW + 32 * c0 + 32), "i"(16 * MROW + 32 * c0 + 64),
              "i"(16 * MROW + 32 * c0 + 96));
        const v2u lo[4] = {lo0, lo1, lo2, lo3}, hi[4] = {hi0, hi1, hi2, hi3};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const v4u w = {lo[c].x, lo[c].y, hi[c].x, hi[c].y};
          acc[c0 + c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w), pb, acc[c0 + c], 0, 0, 0);
        }
      }
    }
    // this wave's LDS reads of block b have returned before the next barrier
    __builtin_amdgcn_s_waitcnt(WAITCNT_LGKM0);
    asm volatile("" ::"v"(tail_off), "v"(vlane16));
  };
  // The first block outside the loop: there the compiler sees that the
  // query loads precede the KV loads and waits only for them, where at the
  // top of a loop it cannot tell the first pass from later ones and would
  // wait for every KV block in flight.
  if (nblk > 0) block(0);
#pragma unroll 1
  for (int b = 1; b < nblk; ++b) block(b);
  if constexpr (!FUSED) {
    if (tid == 0) *s_next = next;
  }
  lds_barrier();  // every wave is done with the KV blocks

  // partials: bf16(O / sum) and ln(sum exp) of each query row (an empty split:
  // zeros and -inf). Each compute wave stages its 16 rows in LDS (the KV
  // blocks are free after the barrier above) and writes each row's 1 KiB as
  // one store of 16 bytes per lane: whole cache lines, since the partials are
  // written through to the device's coherence point (sc1). The attention
  // alone also stores them non-temporal: they are read by another launch,
  // long after, so keeping them in the caches only pushes out the queries
  // (measured on the large decode batch: 1030 -> 1005 us; in the fused launch
  // the merge reads them soon after, and non-temporal stores were slower).
  uint8_t* ot = lds + wave * 16 * MROW;  // this wave's rows, MROW bytes apart
  const bool any = nblk > 0;
  if (compute) {
    const float inv = any ? 1.f / lsum : 0.f;
#pragma unroll
    for (int c = 0; c < NCOLT; ++c)
      *reinterpret_cast<uint2*>(ot + c16 * MROW + (16 * c + 4 * g) * 2) =
          make_uint2(pack_bf16(acc[c][0] * inv, acc[c][1] * inv), pack_bf16(acc[c][2] * inv, acc[c][3] * inv));
  }
  if (compute) {
    const float lse = any ? (m2 + __log2f(lsum)) * LN2 : -INFINITY;
    __builtin_amdgcn_s_waitcnt(WAITCNT_LGKM0);  // this wave's rows are in LDS (the wave reads only its own)
    for (int i = 0; i < 16; ++i) {
      const int qrow = wave * 16 + i;
      if (qrow >= qrows) break;  // wave-uniform
      const int64_t row = part_row(a, r, j, qrow / NH, qrow % NH);
      const uint4 v = *reinterpret_cast<const uint4*>(ot + i * MROW + lane * 16);
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc(a.po + row * (KVL * 2), (short)0, KVL * 2, BUF_WORD3);
      __builtin_amdgcn_raw_buffer_store_b128((v4u){v.x, v.y, v.z, v.w}, rs, lane * 16, 0,
                                             FUSED ? CPOL_AGENT : CPOL_AGENT | CPOL_NT);
    }
    if (g == 0 && qi < qrows)
      __hip_atomic_store(a.pl + part_row(a, r, j, qi / NH, qi % NH), lse, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  if constexpr (FUSED) {
    // the claim of the next unit goes out with the partial stores; the wait
    // for them covers it
    if (tid == 0) next = claim_unit(q_next);
    __builtin_amdgcn_s_waitcnt(0);
    next = __builtin_amdgcn_readfirstlane(next);  // lane 0's (thread 0's) value, taken on every path
    if (tid == 0) *s_next = next;
    lds_barrier();  // every wave's partial stores are complete
    if (tid == 0) *s_last = count_in(a.cnt + r) == a.n - 1;
    lds_barrier();
    // the same value on every lane: read as a scalar, so the branch is uniform
    // and the consumer's MFMAs run with the whole wave active
    if (__builtin_amdgcn_readfirstlane(*s_last)) {
      consume(a, r, lds);
      if (tid == 0) __hip_atomic_store(a.cnt + r, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// The launch: DECODE_WG_PER_CU workgroups per CU (or one per unit, if fewer),
// each taking units u = (request u / n, split u mod n) in order until none is
// left: its first by its block index, each later one from the queue counter
// (units gridDim.x, gridDim.x + 1, ..), claimed while the unit before it
// runs, so the claim's round trip overlaps that unit. A request's splits
// are consecutive units, so they run at about the same time and the merge
// follows them closely. Units are not tied to XCDs or to dispatch order: a
// grid of one workgroup per unit, dispatched in order to the XCDs in turn,
// left slots idle on every XCD behind the one where merges held workgroups
// longest (about 200 of 512 slots on average in the fused launch). A
// workgroup with no unit left counts itself out; the last one sets both
// counters back to zero for the next launch.
template <bool FUSED>
__global__ __launch_bounds__(DTHREADS, 2) void mla_decode_kernel(const DArgs a) {
  // One LDS variable (the flag words below live past the KV blocks): with a
  // single one the compiler does not order this wave's LDS reads behind the
  // buffer-to-LDS loads in flight, whose completion the block loop waits for
  // itself; with several it treats every access to the KV array as touching
  // the block being loaded.
  __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_BYTES + 16];
  int* const s_last = reinterpret_cast<int*>(lds + LDS_BYTES);
  int* const s_next = s_last + 1;
  int32_t* const q_next = a.cnt + a.R;  // units handed out past the first gridDim.x
  int32_t* const q_done = q_next + 1;   // workgroups with no unit left
  const int units = a.R * a.n;
  int u = blockIdx.x;
  while (u < units) {
    int next = 0;
    if (!FUSED && threadIdx.x == 0) next = claim_unit(q_next);
    decode_unit<FUSED>(a, u / a.n, u % a.n, lds, s_last, s_next, q_next, next);
    // every wave is done with the unit's LDS before any starts the next (the
    // attention's partial stores stay in flight)
    lds_barrier();
    // a claim past the batch ends the loop; so does any value a counter
    // that was not zero at the launch can give, so no unit outside the
    // batch is ever named
    const int c = __builtin_amdgcn_readfirstlane(*s_next);
    u = c >= 0 && c < units - (int)gridDim.x ? (int)gridDim.x + c : units;
  }
  if (threadIdx.x == 0 &&
      __hip_atomic_fetch_add(q_done, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (int)gridDim.x - 1) {
    // every workgroup has made its last claim (each counts itself out after
    // its claim has returned)
    __hip_atomic_store(q_next, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(q_done, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

__global__ void zero_counters(int32_t* c, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) c[i] = 0;
}

// The workspace of mla_decode_noalloc: a file-scope device array that every
// GPU the library runs on holds until the process ends. In host code its name
// is not a device address; its address on the current device comes from
// hipGetSymbolAddress, asked once per device (scratch_on_device).
constexpr int64_t SCRATCH_BYTES = MLA_DECODE_SCRATCH_BYTES;
__device__ __align__(256) uint8_t scratch[SCRATCH_BYTES];

// ---------------------------------------------------------------- host side

bool aligned(const void* p, uintptr_t al) { return (reinterpret_cast<uintptr_t>(p) & (al - 1)) == 0; }

struct WsLayout {
  int64_t bytes, cnt, part, lse;
};

bool ws_layout(int64_t R, int64_t q, int64_t n, WsLayout* w) {
  auto up = [](int64_t x) { return (x + 255) / 256 * 256; };
  const int64_t rows = R * n * q * NH;  // R <= 2^24, n <= 64, q <= 4: no overflow
  w->cnt = 0;  // R request counters, then the unit queue's two
  w->part = up((R + 2) * 4);
  w->lse = w->part + up(rows * KVL * 2);
  w->bytes = w->lse + up(rows * 4);
  return true;
}

int check(const mla_decode_args* a) {
  if (!a || a->struct_size < sizeof(mla_decode_args)) return MLA_POST_EINVAL;
  if (a->R < 0 || a->R > (1 << 24) || a->q < 1 || a->q > MLA_DECODE_QMAX || a->n < 1) return MLA_POST_EINVAL;
  if (a->n > MLA_DECODE_NMAX) return MLA_POST_EUNSUPPORTED;
  if (a->R == 0) return MLA_POST_OK;
  if (!a->qry || !a->kv || !a->indptr || !a->w_v || !a->w_v_scale || !a->gate || !a->core || !a->workspace)
    return MLA_POST_EINVAL;
  if (a->q_st < 0 || a->q_sh < 0 || (a->q_st % 8) || (a->q_sh % 8)) return MLA_POST_ESTRIDE;
  if (a->kv_st < DQK || (a->kv_st % 8)) return MLA_POST_ESTRIDE;
  if (a->w_sh < 0 || a->w_sv < 0 || (a->w_sh % 16) || (a->w_sv % 16)) return MLA_POST_ESTRIDE;
  if (a->s_sh < 0 || a->s_sv < 0 || a->s_sb < 0) return MLA_POST_ESTRIDE;
  if (!aligned(a->qry, 16) || !aligned(a->kv, 16) || !aligned(a->indptr, 4) || !aligned(a->w_v, 16) ||
      !aligned(a->gate, 16) || !aligned(a->core, 16) || !aligned(a->workspace, 256))
    return MLA_POST_EALIGN;
  if ((a->dbg_lat && !aligned(a->dbg_lat, 16)) || (a->dbg_codes && !aligned(a->dbg_codes, 4))) return MLA_POST_EALIGN;
  // a block's rows are read with 32-bit buffer offsets; token and head offsets in 64 bits
  if ((int64_t)BC * a->kv_st * 2 >= (int64_t(1) << 31)) return MLA_POST_ERANGE;
  {
    int64_t x, y;
    const int64_t S = (int64_t)a->R * a->q;
    if (__builtin_mul_overflow(S - 1, a->q_st, &x) || __builtin_mul_overflow(NH - 1, a->q_sh, &y) ||
        __builtin_add_overflow(x, y, &x) || __builtin_add_overflow(x, DQK, &x) || __builtin_mul_overflow(x, 2, &x))
      return MLA_POST_ERANGE;
  }
  WsLayout w;
  ws_layout(a->R, a->q, a->n, &w);
  if (a->workspace_bytes < w.bytes) return MLA_POST_EINVAL;
  return MLA_POST_OK;
}

DArgs device_args(const mla_decode_args* a) {
  WsLayout w;
  ws_layout(a->R, a->q, a->n, &w);
  DArgs d;
  d.qry = static_cast<const uint8_t*>(a->qry);
  d.q_st = a->q_st * 2;
  d.q_sh = a->q_sh * 2;
  d.kv = static_cast<const uint8_t*>(a->kv);
  d.kv_st = a->kv_st * 2;
  d.indptr = a->indptr;
  d.scale2 = a->scale * LOG2E;
  d.R = a->R;
  d.q = a->q;
  d.n = a->n;
  d.w_v = a->w_v;
  d.w_sh = a->w_sh;
  d.w_sv = a->w_sv;
  d.w_vs = a->w_v_scale;
  d.s_sh = a->s_sh;
  d.s_sv = a->s_sv;
  d.s_sb = a->s_sb;
  d.gate = static_cast<const uint8_t*>(a->gate);
  d.core = static_cast<uint8_t*>(a->core);
  uint8_t* ws = static_cast<uint8_t*>(a->workspace);
  d.cnt = reinterpret_cast<int32_t*>(ws + w.cnt);
  d.po = ws + w.part;
  d.pl = reinterpret_cast<float*>(ws + w.lse);
  d.dbg_lat = static_cast<uint8_t*>(a->dbg_lat);
  d.dbg_codes = static_cast<uint8_t*>(a->dbg_codes);
  d.dbg_scales = static_cast<uint8_t*>(a->dbg_scales);
  return d;
}

// scratch's address on the current device, or nullptr (with the HIP error
// recorded) when the runtime cannot give it. Cached per device.
void* scratch_on_device() {
  constexpr int MAX_DEVICES = 64;
  static std::atomic<void*> cached[MAX_DEVICES];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= MAX_DEVICES) {
    mla_dev::g_hip_error = e != hipSuccess ? hipGetErrorString(e) : "device index out of range";
    return nullptr;
  }
  void* p = cached[dev].load(std::memory_order_acquire);
  if (p) return p;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !p) {
    mla_dev::g_hip_error = hipGetErrorString(e);
    return nullptr;
  }
  cached[dev].store(p, std::memory_order_release);
  return p;
}

constexpr int DECODE_WG_PER_CU = 2;  // resident at once: two KV blocks of LDS each, 256 VGPRs

unsigned decode_grid(const mla_decode_args* a) {
  return (unsigned)std::min<int64_t>((int64_t)a->R * a->n, (int64_t)DECODE_WG_PER_CU * mla_dev::device_cus());
}

template <bool FUSED>
int run(const mla_decode_args* a, void* stream) {
  const int st = check(a);
  if (st != MLA_POST_OK || a->R == 0) return st;
  const DArgs d = device_args(a);
  return launch(mla_decode_kernel<FUSED>, dim3(decode_grid(a)), dim3(DTHREADS), static_cast<hipStream_t>(stream), d);
}

}  // namespace

extern "C" {

int mla_decode_workspace(int32_t R, int32_t q, int32_t n, int64_t* bytes, int64_t* off_counters, int64_t* off_partials,
                         int64_t* off_lse) {
  if (R < 0 || R > (1 << 24) || q < 1 || q > MLA_DECODE_QMAX || n < 1) return MLA_POST_EINVAL;
  if (n > MLA_DECODE_NMAX) return MLA_POST_EUNSUPPORTED;
  WsLayout w;
  ws_layout(R, q, n, &w);
  if (bytes) *bytes = w.bytes;
  if (off_counters) *off_counters = w.cnt;
  if (off_partials) *off_partials = w.part;
  if (off_lse) *off_lse = w.lse;
  return MLA_POST_OK;
}

int mla_decode_workspace_init(void* workspace, int32_t R, void* stream) {
  if (R < 0 || R > (1 << 24)) return MLA_POST_EINVAL;
  if (R == 0) return MLA_POST_OK;
  if (!workspace) return MLA_POST_EINVAL;
  if (!aligned(workspace, 256)) return MLA_POST_EALIGN;
  return launch(zero_counters, dim3((unsigned)((R + 2 + 255) / 256)), dim3(256), static_cast<hipStream_t>(stream),
                static_cast<int32_t*>(workspace), (int)R + 2);
}

int mla_decode(const mla_decode_args* a, void* stream) { return run<true>(a, stream); }

int mla_decode_partials(const mla_decode_args* a, void* stream) { return run<false>(a, stream); }

int mla_decode_check(const mla_decode_args* a) { return check(a); }

int mla_decode_noalloc(const mla_decode_args* a, void* stream) {
  if (!a || a->struct_size < sizeof(mla_decode_args)) return MLA_POST_EINVAL;
  if (a->workspace) return MLA_POST_EINVAL;  // the workspace is the library's scratch array
  if (a->R < 0 || a->R > (1 << 24) || a->q < 1 || a->q > MLA_DECODE_QMAX || a->n < 1) return MLA_POST_EINVAL;
  if (a->n > MLA_DECODE_NMAX) return MLA_POST_EUNSUPPORTED;
  WsLayout w;
  ws_layout(a->R, a->q, a->n, &w);
  if (w.bytes > SCRATCH_BYTES) return MLA_POST_EUNSUPPORTED;
  if (a->R == 0) return check(a);
  mla_decode_args b = *a;
  b.struct_size = sizeof(mla_decode_args);
  b.workspace = reinterpret_cast<void*>(256);  // stand-in for validation only (non-null, aligned)
  b.workspace_bytes = SCRATCH_BYTES;
  const int st = check(&b);
  if (st != MLA_POST_OK) return st;
  void* p = scratch_on_device();
  if (!p) return MLA_POST_ELAUNCH;
  b.workspace = p;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  // the counters must start at zero: a fill kernel (no memset, so the call
  // may be captured in a graph)
  const int z =
      launch(zero_counters, dim3((unsigned)((a->R + 2 + 255) / 256)), dim3(256), s, static_cast<int32_t*>(p), (int)a->R + 2);
  if (z != MLA_POST_OK) return z;
  const DArgs d = device_args(&b);
  return launch(mla_decode_kernel<true>, dim3(decode_grid(&b)), dim3(DTHREADS), s, d);
}

}  // extern "C"
