// Device helpers shared by the exact-attention kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 2^x on the transcendental unit (v_exp_f32); 2^-inf = 0.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
// log2(x) on the transcendental unit (v_log_f32).
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }
// 1/x on the transcendental unit (v_rcp_f32).
__device__ __forceinline__ float rcp_hw(float x) { return __builtin_amdgcn_rcpf(x); }

// Two floats to two bf16 (round to nearest even, v_cvt_pk_bf16_f32), packed.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// 32x32x16 bf16 matrix-core product, float32 accumulate.
// Lane l supplies A[l%32][8*(l/32) + 0..7] and B[8*(l/32) + 0..7][l%32] (up to a
// permutation of the 16 contraction slots that is the same for A and B), and
// holds D[8*(r/4) + 4*(l/32) + r%4][l%32] in accumulator element r.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Reassemble 8 bf16 from two 64-bit halves.
__device__ __forceinline__ bf16x8 bf16x8_from(uint2 lo, uint2 hi) {
  uint4 u = {lo.x, lo.y, hi.x, hi.y};
  return __builtin_bit_cast(bf16x8, u);
}
__device__ __forceinline__ bf16x8 bf16x8_from(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

// Byte select: result bytes picked from {hi:lo} by `sel` (v_perm_b32).
__device__ __forceinline__ uint32_t perm_b32(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}
// Low 16-bit halves of two words: (lo.l16) | (hi.l16 << 16).
__device__ __forceinline__ uint32_t lo_halves(uint32_t lo, uint32_t hi) { return perm_b32(hi, lo, 0x05040100u); }
// High 16-bit halves of two words: (lo.h16) | (hi.h16 << 16).
__device__ __forceinline__ uint32_t hi_halves(uint32_t lo, uint32_t hi) { return perm_b32(hi, lo, 0x07060302u); }

__device__ __forceinline__ uint32_t word_of(const uint4& u, int i) {
  return i == 0 ? u.x : i == 1 ? u.y : i == 2 ? u.z : u.w;
}

// Workgroup id -> (batch*head, query block), with
//  * all query blocks of one (batch, head) on one XCD: the dispatcher hands
//    workgroup ids to the 8 XCDs round-robin, so consecutive logical ids are
//    gathered from ids that share id % 8;
//  * optionally the heaviest causal query blocks first (largest block index).
__device__ __forceinline__ void map_block_xcd(int w, int total, int nq, bool heavy_first, int& bh, int& qb) {
  const int per = total >> 3, rem = total & 7;
  const int x = w & 7, loc = w >> 3;
  const int logical = x * per + (x < rem ? x : rem) + loc;
  bh = logical / nq;
  const int i = logical - bh * nq;
  qb = heavy_first ? nq - 1 - i : i;
}

}  // namespace fa
