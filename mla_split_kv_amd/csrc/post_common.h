// Device helpers shared by the library's kernels: bf16 packing, wave
// reductions, the LSE -> weight step, the MXFP4 quantiser (the hardware scaled
// FP4 convert) and the scaled FP4 MFMA, streaming loads and stores.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- helpers

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two float32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Lane permutations within each row of 16 lanes (DPP controls): swap
// neighbours, swap pairs, mirror each half row, mirror the row. Applied in
// that order with an associative operation, they leave every lane of a row
// holding the row's reduction.
constexpr int DPP_XOR1 = 0xB1, DPP_XOR2 = 0x4E, DPP_HALF_MIRROR = 0x141, DPP_MIRROR = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float lane_f(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}

// Max over the 64 lanes, as a wave-uniform value: within rows by DPP, then
// the four rows' results combined from lanes 0, 16, 32 and 48.
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp<DPP_XOR1>(x));
  x = fmaxf(x, dpp<DPP_XOR2>(x));
  x = fmaxf(x, dpp<DPP_HALF_MIRROR>(x));
  x = fmaxf(x, dpp<DPP_MIRROR>(x));
  return fmaxf(fmaxf(lane_f(x, 0), lane_f(x, 16)), fmaxf(lane_f(x, 32), lane_f(x, 48)));
}

// Sum over the 64 lanes, as a wave-uniform value (same pattern as wave_max).
__device__ __forceinline__ float wave_sum(float x) {
  x += dpp<DPP_XOR1>(x);
  x += dpp<DPP_XOR2>(x);
  x += dpp<DPP_HALF_MIRROR>(x);
  x += dpp<DPP_MIRROR>(x);
  return (lane_f(x, 0) + lane_f(x, 16)) + (lane_f(x, 32) + lane_f(x, 48));
}

// LSE NaN / +inf -> -inf ([mla_back: sane]).
__device__ __forceinline__ float sane(float x) { return (x != x || x == INFINITY) ? -INFINITY : x; }

// MXFP4 quantisation of the 8 bf16 latents a lane holds (4 packed words);
// lanes 4b .. 4b+3 hold the 32 elements of block b. Returns the 8 E2M1
// codes (element 2i in the low nibble of byte i) and the block's E8M0 code.
// Scale code: max(1, ((amax_bits + 0x20) >> 7) - 2) over the 15-bit bf16
// magnitude patterns; the conversion divides by 2^(code-127) and rounds to
// nearest even with saturation (v_cvt_scalef32_pk_fp4_bf16).
__device__ __forceinline__ uint32_t quant8(const uint32_t w[4], int& code_out) {
  uint32_t am = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    am = max(am, w[i] & 0x7FFFu);
    am = max(am, (w[i] >> 16) & 0x7FFFu);
  }
  // quad reduction: xor 1 (quad_perm [1,0,3,2]) then xor 2 ([2,3,0,1])
  am = max(am, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)am, 0xB1, 0xF, 0xF, false));
  am = max(am, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)am, 0x4E, 0xF, 0xF, false));
  int code = max((int)((am + 0x20u) >> 7) - 2, 1);
  float scale = __uint_as_float((uint32_t)code << 23);
  int pk = 0;
  pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(pk, __builtin_bit_cast(bf2, w[0]), scale, 0);
  pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(pk, __builtin_bit_cast(bf2, w[1]), scale, 1);
  pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(pk, __builtin_bit_cast(bf2, w[2]), scale, 2);
  pk = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(pk, __builtin_bit_cast(bf2, w[3]), scale, 3);
  code_out = code;
  return (uint32_t)pk;
}

template <int ST>
__device__ __forceinline__ v4f mfma_step(const uint4& a, const uint4& b, v4f acc, int sa, int sb) {
  v8i av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  v8i bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
  // formats 4/4 = FP4 E2M1 for A and B; opsel ST picks byte ST of each scale word
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc, 4, 4, ST, sa, ST, sb);
}

// LSEs -> merge weights, in place ([mla_back: combine_splits],
// [mla_back: combine_ranks]): m = max, 0 when all are -inf; e = exp(lse - m);
// weight e / sum, 0 when e == 0 or the sum is 0.
template <int NCH>
__device__ __forceinline__ void lse_to_weights(float l[NCH]) {
  float m = l[0];
#pragma unroll
  for (int c = 1; c < NCH; ++c) m = fmaxf(m, l[c]);
  m = wave_max(m);
  if (m == -INFINITY) m = 0.f;
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    l[c] = expf(l[c] - m);
    s += l[c];
  }
  const float tot = wave_sum(s);
#pragma unroll
  for (int c = 0; c < NCH; ++c) l[c] = (tot == 0.f || l[c] == 0.f) ? 0.f : l[c] / tot;
}

typedef unsigned v4u __attribute__((ext_vector_type(4)));

typedef unsigned v2u __attribute__((ext_vector_type(2)));

// 8 bytes with the non-temporal hint (gate values, read once).
__device__ __forceinline__ uint2 load_nt8(const uint8_t* p) {
  const v2u t = __builtin_nontemporal_load(reinterpret_cast<const v2u*>(p));
  return make_uint2(t.x, t.y);
}

// 16 bytes with the non-temporal (streaming) hint, for data touched once.
__device__ __forceinline__ uint4 load_nt16(const uint8_t* p) {
  const v4u t = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}

// core is written once and not read back by this kernel: a streaming store.
// Measured on the large decode batch, the 12.6 MB of core writes cost about
// 18 us of a 131 us access skeleton as ordinary stores and 13 us as
// non-temporal ones (they compete with the read stream).
__device__ __forceinline__ void store_nt16(uint8_t* p, const uint4& v) {
  const v4u t = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(t, reinterpret_cast<v4u*>(p));
}

constexpr int BUF_WORD3 = 0x00020000;  // raw buffer, 32-bit data format (gfx9 family)

// acc[0..7] += w * (the 8 bf16 values of a lane's 16 bytes of a row)
__device__ __forceinline__ void fma_row(float w, const uint4& v, float acc[8]) {
  acc[0] = fmaf(w, bf_lo(v.x), acc[0]);
  acc[1] = fmaf(w, bf_hi(v.x), acc[1]);
  acc[2] = fmaf(w, bf_lo(v.y), acc[2]);
  acc[3] = fmaf(w, bf_hi(v.y), acc[3]);
  acc[4] = fmaf(w, bf_lo(v.z), acc[4]);
  acc[5] = fmaf(w, bf_hi(v.z), acc[5]);
  acc[6] = fmaf(w, bf_lo(v.w), acc[6]);
  acc[7] = fmaf(w, bf_hi(v.w), acc[7]);
}

}  // namespace
