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
// Native vectors for raw 16/8-byte moves (HIP's uint4/uint2 are structs,
// which keeps some copies out of registers).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Multiplier taking a raw score q.k to the base-2 exponent domain:
// scale * log2(e).  The kernels hide a masked score by setting it to -inf
// before this multiply, which needs a strictly positive multiplier; for
// scale = 0 a multiplier of 1e-30 is used instead, under which every exponent
// of a finite score (|q.k| < 1e22) is below 2^-24, so exp2 returns exactly 1
// and the weights are exactly uniform, as with scale 0.
__host__ __device__ inline float score_coef(float scale) {
  const float c = scale * kLog2e;
  return c > 1e-30f ? c : 1e-30f;
}

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

// Buffer resource over `bytes` bytes at `base`: a raw buffer load whose byte
// offset is at or past `bytes` returns zero instead of reading memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
}

// The rows of one (batch, head) matrix, [N][W] elements of type T, as a
// buffer source.  from_row(r) is a buffer resource that starts at row r, so
// the per-lane offsets of a tile load stay the same from tile to tile (the
// tile's start moves into the scalar base address, not into every lane's
// offset); reads at or past row N still return zero.  Needs r <= N.
template <int W, typename T = uint16_t>
struct RowSrc {
  const T* p;
  uint32_t bytes;   // N * W * sizeof(T)
  __device__ __forceinline__ __amdgpu_buffer_rsrc_t from_row(int r) const {
    return make_rsrc(p + (size_t)r * W, bytes - (uint32_t)r * W * (uint32_t)sizeof(T));
  }
};

// LDS transpose read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane s supplies the address of 4 consecutive bf16 (a row segment); lane i
// of the group receives element i%4 of the segments of lanes i/4, i/4+4,
// i/4+8, i/4+12.  So when lane s points at row r0 + s/4, column c0 + 4*(s%4)
// of a row-major tile, lane i receives column c0 + i of rows r0 .. r0+3.
typedef short i16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* p) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(__attribute__((address_space(3))) uint16_t*)p);
  return __builtin_bit_cast(u32x2, v);
}

// Maximum that propagates NaN (v_maximum_f32 / v_maximum3_f32 on gfx950).
__device__ __forceinline__ float max_nan(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Value of x in this lane and in the lane 32 apart, via v_permlane32_swap:
// returns {x[lane % 32], x[32 + lane % 32]}.
__device__ __forceinline__ void halves(float x, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_halves(float x) {
  float a, b;
  halves(x, a, b);
  return max_nan(a, b);
}
__device__ __forceinline__ float sum_halves(float x) {
  float a, b;
  halves(x, a, b);
  return a + b;
}

// Reassemble 8 bf16 from two 64-bit halves.
__device__ __forceinline__ bf16x8 bf16x8_from(u32x2 lo, u32x2 hi) {
  u32x4 u = {lo.x, lo.y, hi.x, hi.y};
  return __builtin_bit_cast(bf16x8, u);
}
__device__ __forceinline__ bf16x8 bf16x8_from(u32x4 u) { return __builtin_bit_cast(bf16x8, u); }

// Byte select: result bytes picked from {hi:lo} by `sel` (v_perm_b32).
__device__ __forceinline__ uint32_t perm_b32(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}
// Low 16-bit halves of two words: (lo.l16) | (hi.l16 << 16).
__device__ __forceinline__ uint32_t lo_halves(uint32_t lo, uint32_t hi) { return perm_b32(hi, lo, 0x05040100u); }
// High 16-bit halves of two words: (lo.h16) | (hi.h16 << 16).
__device__ __forceinline__ uint32_t hi_halves(uint32_t lo, uint32_t hi) { return perm_b32(hi, lo, 0x07060302u); }

__device__ __forceinline__ uint32_t word_of(const u32x4& u, int i) { return u[i]; }

// Workgroup id -> (batch*head, block).  The dispatcher hands workgroup ids
// to the 8 XCDs round-robin (id % 8), each XCD with its own L2.
//  * order 0 (every block the same work): logical ids are gathered from
//    ids that share id % 8, so all blocks of one (batch, head) land on one
//    XCD and its K/V stay in that XCD's L2;
//  * order 1 / 2 (causal: the work grows with the block index / shrinks
//    with it): block-major order, the heaviest block of every head first,
//    so the last workgroups dispatched are the lightest and the tail stays
//    short.  Id w takes head w % BH; when BH is a multiple of 8 every head
//    still stays on one XCD.
__device__ __forceinline__ void map_block(int w, int total, int nq, int order, int& bh, int& blk) {
  if (order == 0) {
    const int per = total >> 3, rem = total & 7;
    const int x = w & 7, loc = w >> 3;
    const int logical = x * per + (x < rem ? x : rem) + loc;
    bh = logical / nq;
    blk = logical - bh * nq;
    return;
  }
  const int BH = total / nq;
  const int i = w / BH;
  bh = w - i * BH;
  blk = order == 1 ? nq - 1 - i : i;
}
__device__ __forceinline__ void map_block_xcd(int w, int total, int nq, bool heavy_first, int& bh, int& qb) {
  map_block(w, total, nq, heavy_first ? 1 : 0, bh, qb);
}

typedef __attribute__((address_space(3))) void lds_void;

// Direct HBM -> LDS load: lane l's 16 (or 4) bytes at byte `off` of the
// buffer land at dst + 16 l (4 l), dst wave-uniform; an offset past the
// buffer writes zeros.  Checked on the device: lane order, zero fill.
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t r, uint16_t* dst, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, off, 0, 0, 0);
}
__device__ __forceinline__ void lds_load4(__amdgpu_buffer_rsrc_t r, uint16_t* dst, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 4, off, 0, 0, 0);
}
// Wait until this wave's direct LDS loads (and all its other vector memory
// operations) are complete.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Sum over aligned groups of LPK (8 or 16) lanes; every lane of a group gets
// the same bits (each step adds a pair of values in both orders, and float
// addition is commutative).
template <int LPK>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp_mov<0xB1>(x);   // quad_perm [1,0,3,2]: partner lane ^ 1
  x += dpp_mov<0x4E>(x);   // quad_perm [2,3,0,1]: partner lane ^ 2
  x += dpp_mov<0x141>(x);  // row_half_mirror: lane i <-> 7 - i within 8
  if constexpr (LPK == 16) x += dpp_mov<0x140>(x);  // row_mirror: i <-> 15 - i within 16
  return x;
}

}  // namespace fa
