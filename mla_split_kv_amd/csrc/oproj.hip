// o_proj for AMD MI355X (gfx950): out[t, d] = bf16( sum_k core[t, k] * W_O[d, k] ).
//
// The consumer of mla_post's core (the vLLM API-docs page for module
// vllm.models.kimi_k3.amd.specialized_decode.mono.attention.mla_back: the
// path runs up to o_proj's input, module docstring). A dense contraction, so
// it runs on the bf16 matrix cores: v_mfma_f32_32x32x16_bf16, float32
// accumulation, one rounding to bf16 at the end.
//
// Decomposition: a workgroup of 4 waves owns a BM x BN tile of out (BM
// tokens x BN outputs), the waves a 2 x 2 grid of (BM/2) x (BN/2) sub-tiles.
// K advances BK = 64 at a time through two LDS stages: while the waves run
// the MFMAs of stage i, every thread holds its share of stage i + 1's rows in
// registers (issued before the MFMAs), and writes them to the other LDS
// buffer after; one barrier per K step. LDS rows are 128 B of K plus a 16 B
// skew, so the 32 lanes that read one MFMA operand (32 rows, same K) hit
// distinct banks. The MFMA's A operand is W_O's rows (outputs d) and its B
// operand core's rows (tokens t), so a lane's 16 results are 4 runs of 4
// consecutive outputs of one token: they go to an LDS output tile as 8-byte
// pieces, and the workgroup writes the tile as whole 16-byte row pieces.
// Rows past S or D are read clamped (valid memory) and never stored.
// Workgroups are dealt to the 8 XCDs in turn; consecutive tile numbers are
// put on one XCD and ordered in groups of 8 token tiles, so the tiles an XCD
// runs at once share W_O and core rows in its L2.

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "device.h"
#include "launch.h"
#include "mla_oproj.h"
#include "mla_post.h"

namespace {

using mla_dev::launch;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

constexpr int BUF_WORD3 = 0x00020000;  // raw buffer, 32-bit data format (gfx9 family)

constexpr int OP_THREADS = 256;        // 4 waves
constexpr int KALIGN = 64;             // K must be a multiple of this (every K step divides it)
constexpr int XCDS = 8;
constexpr int GROUP_M = 8;             // token tiles per group of the tile order
constexpr int TILE_MAX = 256;          // the largest tile side

struct OArgs {
  const uint8_t* core;
  int64_t core_st;  // bytes
  const uint8_t* w;
  int64_t w_st;  // bytes
  uint8_t* out;
  int64_t out_st;  // bytes
  int32_t M, N, K;  // S, D, K
};

template <int BM, int BN, int BK>
struct Tiling {
  static constexpr int ROWB = BK * 2 + 16;          // LDS bytes per staged row (+16 B skew)
  static constexpr int PIECES_PER_ROW = BK * 2 / 16;  // 16-byte pieces of a staged row
  static constexpr int WM = BM / 2, WN = BN / 2;    // a wave's tokens x outputs
  static constexpr int TM = WM / 32, TN = WN / 32;  // its 32 x 32 MFMA tiles
  static constexpr int ROWS = BN + BM;              // staged rows per stage: W_O's, then core's
  static constexpr int PIECES = ROWS * PIECES_PER_ROW / OP_THREADS;  // 16 B pieces a thread stages
  static constexpr int STAGE = ROWS * ROWB;
  static constexpr int OUTB = BN * 2 + 16;          // LDS bytes per output row (+16 B skew)
  static_assert(BM % 64 == 0 && BN % 64 == 0, "two waves of 32-row MFMA tiles each way");
  static_assert((ROWS * PIECES_PER_ROW) % OP_THREADS == 0, "whole pieces per thread");
  static_assert(BN % (OP_THREADS / PIECES_PER_ROW) == 0, "a piece row is all W_O or all core");
  static_assert(KALIGN % BK == 0 && BK % 16 == 0, "K steps of whole MFMAs that divide K");
  static constexpr int LDS = 2 * STAGE > BM * OUTB ? 2 * STAGE : BM * OUTB;  // the output tile reuses the stages
};

// Tile (tm, tn) of workgroup b out of g: consecutive tile numbers on one XCD
// (the device deals workgroup b to XCD b mod 8), then groups of GROUP_M token
// tiles walked output-tile-major, so the tiles running at once on an XCD
// share rows of both operands.
__device__ __forceinline__ void tile_of(int b, int g, int nm, int nn, int& tm, int& tn) {
  const int per = g / XCDS;
  const int l = (g % XCDS == 0) ? (b % XCDS) * per + b / XCDS : b;
  const int group = l / (GROUP_M * nn);
  const int first = group * GROUP_M;
  const int size = min(nm - first, GROUP_M);
  const int in = l - group * GROUP_M * nn;
  tm = first + in % size;
  tn = in / size;
}

template <int BM, int BN, int BK>
__global__ __launch_bounds__(OP_THREADS) void oproj_kernel(const OArgs a) {
  using T = Tiling<BM, BN, BK>;
  constexpr int ROWB = T::ROWB, PIECES_PER_ROW = T::PIECES_PER_ROW;
  __shared__ __attribute__((aligned(16))) uint8_t lds[T::LDS];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int nm = (a.M + BM - 1) / BM, nn = (a.N + BN - 1) / BN;
  int tm, tn;
  tile_of(blockIdx.x, gridDim.x, nm, nn, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  // The pieces this thread stages: piece i is row tid / 8 + 32 i of the
  // stage (W_O's rows first, then core's), 16 bytes at K offset 16 (tid % 8).
  // Each operand's rows of this tile are read through a buffer resource that
  // ends after its last row in range, so rows past D or S read as zeros
  // (never stored); the lane's offset is one register and the piece's row
  // step a scalar.
  constexpr int RSTEP = OP_THREADS / PIECES_PER_ROW;  // rows between a thread's pieces
  const int nrow = min(BN, a.N - n0), mrow = min(BM, a.M - m0);
  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(a.w + (int64_t)n0 * a.w_st), (short)0, (int)((nrow - 1) * a.w_st + a.K * 2), BUF_WORD3);
  const __amdgpu_buffer_rsrc_t cres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(a.core + (int64_t)m0 * a.core_st), (short)0, (int)((mrow - 1) * a.core_st + a.K * 2),
      BUF_WORD3);
  const int r0 = tid / PIECES_PER_ROW, c0 = (tid % PIECES_PER_ROW) * 16;
  const int wvo = r0 * (int)a.w_st + c0, cvo = r0 * (int)a.core_st + c0;
  const int dst0 = r0 * ROWB + c0;
  uint4 stage[T::PIECES];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int i = 0; i < T::PIECES; ++i) {
      const int r = i * RSTEP;  // row of the stage, less r0
      v4u v;
      // the whole offset in the vector operand: the range check of a raw
      // buffer covers the vector offset, not the scalar one
      if (r < BN)
        v = (v4u)__builtin_amdgcn_raw_buffer_load_b128(wres, wvo + r * (int)a.w_st + k0 * 2, 0, 0);
      else
        v = (v4u)__builtin_amdgcn_raw_buffer_load_b128(cres, cvo + (r - BN) * (int)a.core_st + k0 * 2, 0, 0);
      stage[i] = make_uint4(v.x, v.y, v.z, v.w);
    }
  };
  auto put = [&](int buf) {
#pragma unroll
    for (int i = 0; i < T::PIECES; ++i)
      *reinterpret_cast<uint4*>(lds + buf * T::STAGE + dst0 + i * RSTEP * ROWB) = stage[i];
  };

  f32x16 acc[T::TN][T::TM];
#pragma unroll
  for (int i = 0; i < T::TN; ++i)
#pragma unroll
    for (int j = 0; j < T::TM; ++j) acc[i][j] = f32x16{};

  // this lane's operand rows: MFMA row / column lane % 32, K half lane / 32
  const int arow = (wn * T::WN + (lane & 31)) * ROWB + (lane >> 5) * 16;
  const int brow = (BN + wm * T::WM + (lane & 31)) * ROWB + (lane >> 5) * 16;

  const int ksteps = a.K / BK;
  fetch(0);
  put(0);
  __syncthreads();
#pragma unroll 1
  for (int ks = 0; ks < ksteps; ++ks) {
    const int buf = ks & 1;
    if (ks + 1 < ksteps) fetch((ks + 1) * BK);
    const uint8_t* s = lds + buf * T::STAGE;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8 av[T::TN], bv[T::TM];
#pragma unroll
      for (int i = 0; i < T::TN; ++i) av[i] = *reinterpret_cast<const bf16x8*>(s + arow + i * 32 * ROWB + kk * 32);
#pragma unroll
      for (int j = 0; j < T::TM; ++j) bv[j] = *reinterpret_cast<const bf16x8*>(s + brow + j * 32 * ROWB + kk * 32);
#pragma unroll
      for (int i = 0; i < T::TN; ++i)
#pragma unroll
        for (int j = 0; j < T::TM; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
    }
    if (ks + 1 < ksteps) put(buf ^ 1);
    __syncthreads();
  }

  // Output tile in LDS, [token][output] bf16: lane holds outputs
  // 8 (r / 4) + 4 (lane / 32) + r % 4 of MFMA tile i for token lane % 32 of
  // tile j; each run of 4 is one 8-byte piece. Every wave passed the last
  // barrier after its last LDS read, so the staging buffers are free.
#pragma unroll
  for (int i = 0; i < T::TN; ++i)
#pragma unroll
    for (int j = 0; j < T::TM; ++j) {
      const int tok = wm * T::WM + j * 32 + (lane & 31);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = wn * T::WN + i * 32 + 8 * g + 4 * (lane >> 5);
        const bf16x4 v = {(__bf16)acc[i][j][4 * g], (__bf16)acc[i][j][4 * g + 1], (__bf16)acc[i][j][4 * g + 2],
                          (__bf16)acc[i][j][4 * g + 3]};
        *reinterpret_cast<bf16x4*>(lds + tok * T::OUTB + col * 2) = v;
      }
    }
  __syncthreads();
  constexpr int ROW_PIECES = BN * 2 / 16;
  for (int p = tid; p < BM * ROW_PIECES; p += OP_THREADS) {
    const int r = p / ROW_PIECES, c = (p % ROW_PIECES) * 8;
    const int m = m0 + r, n = n0 + c;
    if (m < a.M && n < a.N)
      *reinterpret_cast<uint4*>(a.out + (int64_t)m * a.out_st + (int64_t)n * 2) =
          *reinterpret_cast<const uint4*>(lds + r * T::OUTB + c * 2);
  }
}

// ---------------------------------------------------------------- large tiles

// The instance for large calls: a 256 x 256 tile of out per workgroup of 8
// waves in a 2 x 4 grid, each wave 128 tokens x 64 outputs (4 x 2 MFMA tiles
// of 32 x 32, 128 float32 accumulators a lane), two waves per SIMD, one
// workgroup per CU. Per 16 of K a wave reads 6 operand rows of 1 KiB from
// LDS for 8 MFMAs, against 4 for 4 in the 128 x 128 instance, whose LDS reads
// bound it. K advances 32 at a time through two LDS stages of 32 KiB (W_O's
// 256 rows, then core's 256, 64 bytes of K each): every thread loads its 4
// 16-byte pieces of step ks + 2 into registers while the waves run the MFMAs
// of step ks, then writes those of step ks + 1 (loaded during step ks - 1)
// to the other stage; one barrier per step, with the MFMAs of each 16-wide
// slice running beside the LDS reads of the next (across steps too). (Buffer-to-LDS loads, which need
// no registers, moved only about 17 bytes per clock per CU from L2 here:
// the loads alone took 65 us of the call.) Rows are not skewed; the 16-byte
// piece p of row r sits in slot p XOR ((r >> 2) mod 4): the 16 lanes of an
// LDS cycle then cover all 64 banks, for the piece writes (4 rows x 4
// pieces) and for the MFMA operand reads (16 rows, one piece). The output
// tile is staged in LDS, a quarter of its tokens per 32 KiB, the 8-byte piece
// g of token t's row in slot g XOR 2 (t mod 32) (the 32 tokens of an MFMA
// tile write distinct banks; pieces stay paired, so rows are read back as
// 16-byte pieces), and written as 16-byte row pieces. Rows past S or D load
// a clamped row (valid memory); their results are never stored.
constexpr int BIG = 256;                       // tile side
constexpr int BIG_BK = 32;                     // K per step
constexpr int BIG_ROWB = BIG_BK * 2;           // bytes per staged row
constexpr int BIG_STAGE = 2 * BIG * BIG_ROWB;  // 32 KiB: W_O's rows, then core's
constexpr int BIG_WAVES = 8;                   // 2 x 4: 128 tokens x 64 outputs each
constexpr int BIG_THREADS = BIG_WAVES * 64;
constexpr int BIG_PIECES = BIG_STAGE / 16 / BIG_THREADS;  // 16-byte pieces a thread moves per step (4)

constexpr int WAIT_LGKM0 = 15 | (3 << 14) | (7 << 4);  // s_waitcnt lgkmcnt(0), other counters not waited
constexpr int wait_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// A workgroup barrier for LDS hazards (after this wave's LDS operations are
// complete); __syncthreads would also wait for the global loads of the step
// ahead.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(WAIT_LGKM0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// A thread's pieces: piece i is row (tid / 4) + 128 i of the stage (W_O's
// rows 0..255, then core's), 16-byte piece tid mod 4 of its 64 bytes of K.
struct BigPieces {
  const uint8_t* wbase;       // W_O's first row of the tile
  const uint8_t* cbase;       // core's
  int wbytes, cbytes;         // their extents (rows clamped to the valid ones)
  uint32_t voff[BIG_PIECES];  // the piece's offset in its operand, less the step's K
  uint32_t lds[BIG_PIECES];   // its swizzled slot in a stage
};

// Issue step ks's loads (live false: past the last step, through buffer
// resources of no bytes, which read nothing; the count in flight is then the
// same at every step).
__device__ __forceinline__ void big_load(const BigPieces& P, int k0, bool live, uint4 (&r)[BIG_PIECES]) {
  const __amdgpu_buffer_rsrc_t wr =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(P.wbase), (short)0, live ? P.wbytes : 0, BUF_WORD3);
  const __amdgpu_buffer_rsrc_t cr =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(P.cbase), (short)0, live ? P.cbytes : 0, BUF_WORD3);
#pragma unroll
  for (int i = 0; i < BIG_PIECES; ++i) {
    const v4u v = (v4u)__builtin_amdgcn_raw_buffer_load_b128(i < BIG_PIECES / 2 ? wr : cr, P.voff[i], k0 * 2, 0);
    r[i] = make_uint4(v.x, v.y, v.z, v.w);
  }
}

__device__ __forceinline__ void big_put(const BigPieces& P, uint8_t* st, const uint4 (&r)[BIG_PIECES]) {
#pragma unroll
  for (int i = 0; i < BIG_PIECES; ++i) *reinterpret_cast<uint4*>(st + P.lds[i]) = r[i];
}

// The operands of one 16-wide K slice from stage st: the wave's 2 W_O rows
// (outputs) and 4 core rows (tokens) of 32.
__device__ __forceinline__ void big_read(const uint8_t* st, uint32_t roff, int wm, int wn, bf16x8 (&av)[2],
                                         bf16x8 (&bv)[4]) {
#pragma unroll
  for (int i = 0; i < 2; ++i) av[i] = *reinterpret_cast<const bf16x8*>(st + roff + (wn * 64 + i * 32) * BIG_ROWB);
#pragma unroll
  for (int j = 0; j < 4; ++j) bv[j] = *reinterpret_cast<const bf16x8*>(st + roff + (BIG + wm * 128 + j * 32) * BIG_ROWB);
}

__device__ __forceinline__ void big_mfma(const bf16x8 (&av)[2], const bf16x8 (&bv)[4], f32x16 (&acc)[2][4]) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
}

// One K step, software-pipelined across steps so that every group of MFMAs
// has LDS reads in flight beside it (the workgroup is alone on its CU, and
// its waves meet at every barrier): on entry the operands of step ks's first
// 16-wide slice are in (a0, b0). Step ks + 2's loads go out into `ahead`;
// the second slice's operands are read from `cur`; the first slice's MFMAs;
// step ks + 1's pieces (`held`, loaded during the step before; at most
// `ahead`'s loads still outstanding) go to stage `nxt`; the barrier (every
// wave's pieces of `nxt` written, every wave done reading `cur`); step ks +
// 1's first slice read from `nxt` into (a0, b0); the second slice's MFMAs.
// Scheduling barriers keep the compiler from moving reads next to their
// MFMAs.
__device__ __forceinline__ void big_step(const BigPieces& P, const uint8_t* cur, uint8_t* nxt, uint4 (&held)[BIG_PIECES],
                                         uint4 (&ahead)[BIG_PIECES], const uint32_t* roff, int ks, int ksteps, int wm,
                                         int wn, f32x16 (&acc)[2][4], bf16x8 (&a0)[2], bf16x8 (&b0)[4]) {
  static_assert(BIG_BK == 32, "two K slices per step");
  big_load(P, (ks + 2) * BIG_BK, ks + 2 < ksteps, ahead);
  bf16x8 a1[2], b1[4];
  big_read(cur, roff[1], wm, wn, a1, b1);
  __builtin_amdgcn_sched_barrier(0);
  big_mfma(a0, b0, acc);
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(wait_vm(BIG_PIECES));
  big_put(P, nxt, held);
  lds_barrier();
  big_read(nxt, roff[0], wm, wn, a0, b0);
  __builtin_amdgcn_sched_barrier(0);
  big_mfma(a1, b1, acc);
  __builtin_amdgcn_sched_barrier(0);
}

__global__ __launch_bounds__(BIG_THREADS, 1) void oproj_big_kernel(const OArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t s0[BIG_STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t s1[BIG_STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t s2[BIG_STAGE];  // output staging only
  __shared__ __attribute__((aligned(16))) uint8_t s3[BIG_STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;  // the wave's token half and output quarter
  const int nm = (a.M + BIG - 1) / BIG, nn = (a.N + BIG - 1) / BIG;
  int tm, tn;
  tile_of(blockIdx.x, gridDim.x, nm, nn, tm, tn);
  const int m0 = tm * BIG, n0 = tn * BIG;

  BigPieces P;
  {
    const int nvalid = min(BIG, a.N - n0), mvalid = min(BIG, a.M - m0);
    P.wbase = a.w + (int64_t)n0 * a.w_st;
    P.cbase = a.core + (int64_t)m0 * a.core_st;
    P.wbytes = (int)((nvalid - 1) * a.w_st + a.K * 2);
    P.cbytes = (int)((mvalid - 1) * a.core_st + a.K * 2);
    const int piece = tid & 3;
#pragma unroll
    for (int i = 0; i < BIG_PIECES; ++i) {
      const int r = (tid >> 2) + 128 * i;  // row of the stage: W_O's for i < 2, then core's
      const bool isw = i < BIG_PIECES / 2;
      const int rr = isw ? min(r, nvalid - 1) : min(r - BIG, mvalid - 1);
      P.voff[i] = (uint32_t)(rr * (int)(isw ? a.w_st : a.core_st) + piece * 16);
      P.lds[i] = (uint32_t)(r * BIG_ROWB + ((piece ^ ((r >> 2) & 3)) << 4));
    }
  }
  // this lane's operand reads: MFMA row lane mod 32, K piece 2 kk + lane / 32
  // of a 32-row group (its rows' keys depend on the lane alone)
  uint32_t roff[BIG_BK / 16];
#pragma unroll
  for (int kk = 0; kk < BIG_BK / 16; ++kk) {
    const int r = lane & 31, piece = 2 * kk + (lane >> 5);
    roff[kk] = (uint32_t)(r * BIG_ROWB + ((piece ^ ((r >> 2) & 3)) << 4));
  }

  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  const int ksteps = a.K / BIG_BK;  // even: K is a multiple of 64
  uint4 r0[BIG_PIECES], r1[BIG_PIECES];
  big_load(P, 0, true, r0);
  big_load(P, BIG_BK, ksteps > 1, r1);
  __builtin_amdgcn_s_waitcnt(wait_vm(BIG_PIECES));
  big_put(P, s0, r0);
  lds_barrier();
  bf16x8 a0[2], b0[4];
  big_read(s0, roff[0], wm, wn, a0, b0);
#pragma unroll 1
  for (int ks = 0; ks < ksteps; ks += 2) {
    big_step(P, s0, s1, r1, r0, roff, ks, ksteps, wm, wn, acc, a0, b0);
    big_step(P, s1, s0, r0, r1, roff, ks + 1, ksteps, wm, wn, acc, a0, b0);
  }
  lds_barrier();  // every wave is done reading the stages (the last step read one more slice)

  // Output tile: token quarter q (64 tokens) in 32 KiB of LDS ([64 tokens][256
  // outputs] bf16, 512 bytes a row, 8-byte piece g in slot g ^ 2 (t mod 32)).
  // The lane holds, of MFMA tile (i, j), outputs 8 (r / 4) + 4 (lane / 32) + r
  // mod 4 of token lane mod 32 of tile j: 4 pieces of 4. Every wave passed
  // the last barrier after its last operand read.
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int q = 2 * wm + j / 2;
    uint8_t* ot = q == 0 ? s0 : q == 1 ? s1 : q == 2 ? s2 : s3;
    const int t = (j & 1) * 32 + (lane & 31);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int piece = (wn * 64 + i * 32 + 8 * g + 4 * (lane >> 5)) >> 2;
        const bf16x4 v = {(__bf16)acc[i][j][4 * g], (__bf16)acc[i][j][4 * g + 1], (__bf16)acc[i][j][4 * g + 2],
                          (__bf16)acc[i][j][4 * g + 3]};
        *reinterpret_cast<bf16x4*>(ot + t * 512 + ((piece ^ ((t & 31) << 1)) << 3)) = v;
      }
  }
  lds_barrier();
  // 16-byte pieces: quarter q, token t, pair p (outputs 8 p .. 8 p + 7)
  for (int i = tid; i < 4 * 64 * 32; i += BIG_THREADS) {
    const int q = i >> 11, t = (i >> 5) & 63, p = i & 31;
    const int m = m0 + q * 64 + t, n = n0 + p * 8;
    const uint8_t* ot = q == 0 ? s0 : q == 1 ? s1 : q == 2 ? s2 : s3;
    const uint4 v = *reinterpret_cast<const uint4*>(ot + t * 512 + (((2 * p) ^ ((t & 31) << 1)) << 3));
    if (m < a.M && n < a.N) *reinterpret_cast<uint4*>(a.out + (int64_t)m * a.out_st + (int64_t)n * 2) = v;
  }
}

bool mul_ok(int64_t a, int64_t b, int64_t* out) { return !__builtin_mul_overflow(a, b, out); }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// (rows - 1) * stride + cols elements of bf16 fit int64 bytes
bool span_ok(int64_t rows, int64_t stride, int64_t cols) {
  int64_t a, b;
  return mul_ok(rows - 1, stride, &a) && !__builtin_add_overflow(a, cols, &b) && mul_ok(b, 2, &a);
}

int check(const void* core, int64_t cst, int32_t S, int32_t K, const void* w, int64_t wst, int32_t D, const void* out,
          int64_t ost) {
  if (S < 0 || D < 1 || K < 1) return MLA_POST_EINVAL;
  if ((D % 8) || (K % KALIGN) || K > MLA_OPROJ_KMAX) return MLA_POST_EUNSUPPORTED;
  if (S == 0) return MLA_POST_OK;
  if (!core || !w || !out) return MLA_POST_EINVAL;
  if (cst < 0 || wst < 0 || ost < 0 || (cst % 8) || (wst % 8) || (ost % 8)) return MLA_POST_ESTRIDE;
  if (!aligned16(core) || !aligned16(w) || !aligned16(out)) return MLA_POST_EALIGN;
  if (!span_ok(S, cst, K) || !span_ok(D, wst, K) || !span_ok(S, ost, D)) return MLA_POST_ERANGE;
  // a tile's rows of each operand are read with 32-bit buffer offsets
  if ((int64_t)TILE_MAX * (cst > K ? cst : K) * 2 >= (int64_t(1) << 31) ||
      (int64_t)TILE_MAX * (wst > K ? wst : K) * 2 >= (int64_t(1) << 31))
    return MLA_POST_ERANGE;
  return MLA_POST_OK;
}

// Tile of a call: 256 x 256 while that grid gives every CU a workgroup
// (one is resident per CU), else 128 x 128 while that grid gives every CU at
// least two, else 64 x 128, else 64 x 64 (small batches, where the call
// streams W_O and wants many workgroups reading it).
void plan(int S, int D, int cus, int& bm, int& bn) {
  auto grid = [&](int m, int n) { return (int64_t)((S + m - 1) / m) * ((D + n - 1) / n); };
  if (grid(BIG, BIG) >= (int64_t)cus) {
    bm = BIG, bn = BIG;
  } else if (grid(128, 128) >= 2 * (int64_t)cus) {
    bm = 128, bn = 128;
  } else if (grid(64, 128) >= 2 * (int64_t)cus) {
    bm = 64, bn = 128;
  } else {
    bm = 64, bn = 64;
  }
}

}  // namespace

extern "C" {

int mla_oproj_check(const void* core, int64_t core_stride, int32_t S, int32_t K, const void* w_o, int64_t w_stride,
                    int32_t D, const void* out, int64_t out_stride) {
  return check(core, core_stride, S, K, w_o, w_stride, D, out, out_stride);
}

int mla_oproj_plan(int32_t S, int32_t D, int32_t cus, int32_t* tile_m, int32_t* tile_n, int32_t* workgroups) {
  if (!tile_m || !tile_n || !workgroups || S < 0 || D < 1) return MLA_POST_EINVAL;
  int bm, bn;
  plan(S, D, cus > 0 ? cus : mla_dev::device_cus(), bm, bn);
  *tile_m = bm;
  *tile_n = bn;
  *workgroups = (int32_t)(((int64_t)S + bm - 1) / bm * ((D + bn - 1) / bn));
  return MLA_POST_OK;
}

int mla_oproj(const void* core, int64_t core_stride, int32_t S, int32_t K, const void* w_o, int64_t w_stride,
              int32_t D, void* out, int64_t out_stride, void* stream) {
  const int st = check(core, core_stride, S, K, w_o, w_stride, D, out, out_stride);
  if (st != MLA_POST_OK || S == 0) return st;
  OArgs a;
  a.core = static_cast<const uint8_t*>(core);
  a.core_st = core_stride * 2;
  a.w = static_cast<const uint8_t*>(w_o);
  a.w_st = w_stride * 2;
  a.out = static_cast<uint8_t*>(out);
  a.out_st = out_stride * 2;
  a.M = S;
  a.N = D;
  a.K = K;
  int bm, bn;
  plan(S, D, mla_dev::device_cus(), bm, bn);
  const int64_t g = ((int64_t)S + bm - 1) / bm * ((D + bn - 1) / bn);
  if (g > 0x7FFFFFFF / OP_THREADS) return MLA_POST_ERANGE;
  const dim3 grid((unsigned)g), block(OP_THREADS);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (bm == BIG) return launch(oproj_big_kernel, grid, dim3(BIG_THREADS), s, a);
  if (bm == 128) return launch(oproj_kernel<128, 128, 64>, grid, block, s, a);
  if (bn == 128) return launch(oproj_kernel<64, 128, 64>, grid, block, s, a);
  return launch(oproj_kernel<64, 64, 64>, grid, block, s, a);
}

}  // extern "C"
