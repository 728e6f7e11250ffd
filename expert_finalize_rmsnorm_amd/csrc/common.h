// common.h -- device helpers shared by the libmoetail kernels (gfx950, wave64).
//
// Build requirement: -ffp-contract=off.  Every FP32 expression below is
// meant to round after each operation (no fused multiply-add), which is
// what makes the finalize kernels bit-reproducible.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moetail {

constexpr int kWave = 64;        // CDNA wavefront
constexpr int kChunk = 8;        // BF16 columns per 16-byte access
constexpr int kBlockCols = kWave * kChunk;  // 512 columns: one wave-wide access

// ---------------------------------------------------------------- BF16 ---

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round-to-nearest-even FP32 -> BF16 bits.  Adding 0x7fff plus the kept
// LSB carries into the kept half exactly when the discarded half is above
// one half unit, or equal to it with an odd kept half.  NaN keeps its sign
// and becomes quiet.
__device__ __forceinline__ uint32_t bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Two FP32 values -> one word of two BF16 (low column in the low half) in
// one v_cvt_pk_bf16_f32.  The instruction rounds to nearest even, keeps
// denormals, and returns a NaN's upper half with the quiet bit set: on every
// one of the 2^32 inputs it gives the bits of bf16_bits above.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack2_rn(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// A -0 BF16 half (0x8000) leaves as +0.
__device__ __forceinline__ uint32_t plus_zero2(uint32_t w) {
  const uint32_t lo = (w & 0x7fffu) ? (w & 0xffffu) : 0u;
  const uint32_t hi = (w & 0x7fff0000u) ? (w & 0xffff0000u) : 0u;
  return lo | hi;
}

// pack2_rn with -0 written as +0 (for every BF16 word that leaves a kernel).
__device__ __forceinline__ uint32_t pack2_rn_pz(float lo, float hi) {
  return plus_zero2(pack2_rn(lo, hi));
}

// 16 bytes = 8 BF16 columns <-> 8 FP32.
__device__ __forceinline__ void unpack8(const uint4& q, float (&v)[8]) {
  v[0] = bf16_lo(q.x); v[1] = bf16_hi(q.x);
  v[2] = bf16_lo(q.y); v[3] = bf16_hi(q.y);
  v[4] = bf16_lo(q.z); v[5] = bf16_hi(q.z);
  v[6] = bf16_lo(q.w); v[7] = bf16_hi(q.w);
}
__device__ __forceinline__ uint4 pack8_pz(const float (&v)[8]) {
  return make_uint4(pack2_rn_pz(v[0], v[1]), pack2_rn_pz(v[2], v[3]),
                    pack2_rn_pz(v[4], v[5]), pack2_rn_pz(v[6], v[7]));
}
__device__ __forceinline__ uint4 pack8(const float (&v)[8]) {
  return make_uint4(pack2_rn(v[0], v[1]), pack2_rn(v[2], v[3]),
                    pack2_rn(v[4], v[5]), pack2_rn(v[6], v[7]));
}

// --------------------------------------------------------- reductions ---

// Wave-wide butterfly sum.  After the step that pairs aligned groups of o
// lanes, every lane of an aligned group of 2o lanes holds that group's sum,
// computed as (own group) + (partner group).  Every lane of a group holds
// the same value, so which partner lane is read does not change a bit, and
// FP32 addition commutes, so both partners agree: the result equals the xor
// butterfly with offsets 1, 2, 4, ..., 32.  Steps 1 and 2 use quad
// permutes, 4 and 8 the half-row and row mirrors (DPP: no LDS round trip),
// 16 and 32 a lane permute.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, true));
}
__device__ __forceinline__ float wave_butterfly_sum(float s) {
  s = s + dpp_f<0xb1>(s);   // quad_perm [1,0,3,2]: lane ^ 1
  s = s + dpp_f<0x4e>(s);   // quad_perm [2,3,0,1]: lane ^ 2
  s = s + dpp_f<0x141>(s);  // row_half_mirror: the other 4 of 8
  s = s + dpp_f<0x140>(s);  // row_mirror: the other 8 of 16
  s = s + __shfl_xor(s, 16, kWave);
  s = s + __shfl_xor(s, 32, kWave);
  return s;
}

// Sum of squares of one 8-column chunk, squares added one by one from 0.
__device__ __forceinline__ float chunk_sum_of_squares(const float (&v)[8]) {
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    float sq = v[c] * v[c];
    s = s + sq;
  }
  return s;
}

// 1 / sqrt(ss * (1/P) + eps): one FP32 multiply, one FP32 add, then the
// reciprocal square root correctly rounded through double precision
// (IEEE sqrt and divide), rounded once to FP32.
__device__ __forceinline__ float inv_rms(float ss, float inv_width, float eps) {
  float m = ss * inv_width;
  m = m + eps;
  return (float)(1.0 / __builtin_sqrt((double)m));
}

__device__ __forceinline__ int readlane_i(int v, int lane) {
  return __builtin_amdgcn_readlane(v, lane);
}
__device__ __forceinline__ float readlane_f(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

__device__ __forceinline__ uint4 load16(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}
// A 16-byte load marked non-temporal: for the large streams read once per
// call (weights, expert-TP K-partials), so that they pass the caches and
// what is read again stays in them.  (Marking the split partials', the
// expert rows' and the latent partials' loads the same way measured
// neutral.)
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load16_stream(const uint16_t* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ void store16(uint16_t* p, const uint4& q) {
  *reinterpret_cast<uint4*>(p) = q;
}

}  // namespace moetail
