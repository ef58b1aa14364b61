// FP8 forward with incoherent processing, for gfx950 (d = 128).
//
// The page "FlashAttention-3 — FlashAttention-3" (section 「3. 量子化誤差を低減
// した低精度（FP8）」) multiplies Q and K by a random orthogonal matrix before
// quantising them to FP8: outliers spread over all coordinates and the FP8
// error drops, while Q K^T is unchanged.  Here:
//
//  * prepare: each row of Q and K is multiplied by a random sign vector and
//    by the Sylvester Hadamard matrix (float32 butterfly, widths 1, 2, ...,
//    64, each pair (a, b) -> (a + b, a - b); the 1/sqrt(128) of both is
//    folded into the softmax scale as 1/128),
//    then quantised to OCP E4M3 with one power-of-two scale per 32 elements
//    (the smallest 2^t with amax <= 448 * 2^t, so nothing saturates).  V is
//    quantised per column in blocks of 32 consecutive keys and stored
//    transposed.  Scales are E8M0 bytes (127 + t).
//  * attention: the FlashAttention-2 forward of fwd_bf16.hip with both
//    products on the block-scaled FP8 matrix cores
//    (v_mfma_scale_f32_32x32x64_f8f6f4): the hardware applies the E8M0
//    scales of the 32-element blocks, so dequantisation costs nothing.  P is
//    rounded to E4M3 (p <= 2^8 under the lazy rescale) for P V; the row sum
//    adds the float32 p.
//
// Operand layout of the 32x32x64 FP8 product (probed on gfx950): lane
// l = i + 32h supplies 32 bytes of row (column) i; bytes 0-15 are
// contraction slots 16h .. 16h+15 and bytes 16-31 are slots 32+16h ..
// 32+16h+15; the E8M0 scale in lane i + 32b applies to slots 32b .. 32b+31
// of row i.  Hence a lane reads two 16-byte pieces, at 16h and 32+16h, of
// each 64-byte stretch of its row.
//
// Buffer written by prepare (per section, (batch, head) major, each section
// starting at a 256-byte boundary; Np = N rounded up to 64):
//   Q8 [BH][Np][128], QE [BH][Np][4], K8 [BH][Np][128], KE [BH][Np][4],
//   V8 [BH][Np/64][128][64], VE [BH][Np/64][2][32][4]
// V8 row c of tile T holds, for each half b of the tile (keys 32b .. 32b+31),
// 32 bytes in which key 32b + 8j + 4g + i sits at byte 32b + 16g + 4j + i;
// VE[T][b][c % 32][c / 32] is the scale of keys 32b .. 32b+31 of column c.
// Rows and keys past N are zero.
#include <type_traits>

#include "fa_common.h"
#include "launch.h"

namespace fa {
namespace {

constexpr int FD = 128;       // head dimension of the FP8 path
constexpr int FBR = 128;      // queries per workgroup
constexpr int FBC = 64;       // keys per tile
constexpr int FNT = 256;
constexpr float FTAU = 8.0f;  // lazy-rescale threshold (log2 units); keeps p <= 256 < 448

typedef int v8i __attribute__((ext_vector_type(8)));

// Smallest t with amax <= 448 * 2^t (0 for amax = 0).  448 = 0.875 * 2^9.
__device__ __forceinline__ int block_exponent(float amax) {
  if (!(amax > 0.f)) return 0;
  int e;
  const float m = frexpf(amax, &e);
  return m <= 0.875f ? e - 9 : e - 8;
}

// Two floats to two E4M3 bytes in the low (hi = false) or high half of `old`.
__device__ __forceinline__ uint32_t cvt_fp8x2(float a, float b, uint32_t old, bool hi) {
  return hi ? (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, true)
            : (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, false);
}

// 32 floats scaled by 2^-t to 32 E4M3 bytes (8 words), in order.
__device__ __forceinline__ void quantize32(const float* x, int t, uint32_t* w) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t v = cvt_fp8x2(ldexpf(x[4 * i], -t), ldexpf(x[4 * i + 1], -t), 0u, false);
    w[i] = cvt_fp8x2(ldexpf(x[4 * i + 2], -t), ldexpf(x[4 * i + 3], -t), v, true);
  }
}

__device__ __forceinline__ uint8_t e8m0(int t) {
  const int b = 127 + t;
  return (uint8_t)(b < 0 ? 0 : b > 254 ? 254 : b);
}

// Q or K rows (BH * Np of them; rows past N become zero), 4 lanes per row:
// lane j holds elements 32j .. 32j+31, which is also its scale block, so each
// row is one coalesced 256-byte load and one 128-byte store.  The arithmetic
// is that of a serial pass over the row (sign flip, Walsh-Hadamard butterflies
// of widths 1, 2, ..., 64 in that order, block maximum, rounding), so the
// bytes are the same: widths 1 to 16 pair elements within a lane, widths 32
// and 64 pair lane j with lane j ^ 1 and j ^ 2, the lower keeping a + b and
// the upper a - b.
__global__ void __launch_bounds__(256)
fp8_quant_rows_kernel(const uint16_t* __restrict__ X, const float* __restrict__ signs, uint8_t* __restrict__ codes,
                      uint8_t* __restrict__ exps, int N, int Np, long long rows) {
  static_assert(FD == 128, "4 lanes of 32 elements per row");
  __shared__ float sg[FD];  // the signs, read by every row's lanes
  if (signs != nullptr && threadIdx.x < FD) sg[threadIdx.x] = signs[threadIdx.x];
  __syncthreads();
  const long long r = (long long)blockIdx.x * 64 + (threadIdx.x >> 2);
  const int j = threadIdx.x & 3;
  const bool live = r < rows;
  const long long bh = live ? r / Np : 0;
  const int n = live ? (int)(r - bh * Np) : N;
  float y[32];
  if (n < N) {
    const u32x4* src = reinterpret_cast<const u32x4*>(X + (bh * N + n) * FD + 32 * j);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const u32x4 w = src[c];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        y[8 * c + 2 * e] = bf16_lo(w[e]);
        y[8 * c + 2 * e + 1] = bf16_hi(w[e]);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) y[i] = 0.f;
  }
  if (signs != nullptr) {  // rows past N stay +0 (no sign flip, so no -0)
    if (n < N) {
#pragma unroll
      for (int i = 0; i < 32; ++i) y[i] *= sg[32 * j + i];
    }
#pragma unroll
    for (int h = 1; h < 32; h *= 2)
#pragma unroll
      for (int i = 0; i < 32; ++i)
        if ((i & h) == 0) {
          const float a = y[i], b = y[i + h];
          y[i] = a + b;
          y[i + h] = a - b;
        }
#pragma unroll
    for (int i = 0; i < 32; ++i) {  // width 32: lanes j ^ 1
      const float o = dpp_mov<0xB1>(y[i]);
      y[i] = (j & 1) ? o - y[i] : y[i] + o;
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) {  // width 64: lanes j ^ 2
      const float o = dpp_mov<0x4E>(y[i]);
      y[i] = (j & 2) ? o - y[i] : y[i] + o;
    }
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(y[i]));
  const int t = block_exponent(amax);
  uint32_t w[8];
  quantize32(y, t, w);
  uint32_t ex = (uint32_t)e8m0(t) << (8 * j);
  ex |= (uint32_t)__float_as_int(dpp_mov<0xB1>(__int_as_float((int)ex)));
  ex |= (uint32_t)__float_as_int(dpp_mov<0x4E>(__int_as_float((int)ex)));
  if (live) {
    u32x4* dst = reinterpret_cast<u32x4*>(codes + r * FD + 32 * j);
    dst[0] = u32x4{w[0], w[1], w[2], w[3]};
    dst[1] = u32x4{w[4], w[5], w[6], w[7]};
    if (j == 0) reinterpret_cast<uint32_t*>(exps)[r] = ex;
  }
}

// One thread per (batch*head, 32-key block, 4 adjacent columns); column
// groups fastest, so one wave-wide load of a key reads 512 contiguous bytes.
__global__ void __launch_bounds__(256)
fp8_quant_v_kernel(const uint16_t* __restrict__ V, uint8_t* __restrict__ v8, uint8_t* __restrict__ ve, int N, int Np,
                   long long total) {
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return;
  constexpr int CG = FD / 4;                 // column groups per key
  const int c0 = 4 * (int)(idx % CG);
  const long long rest = idx / CG;
  const int nb32 = Np / 32;
  const int blk = (int)(rest % nb32);
  const long long bh = rest / nb32;
  float x[4][32];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const int key = blk * 32 + i;
    u32x2 w = {0u, 0u};
    if (key < N) w = *reinterpret_cast<const u32x2*>(V + (bh * N + key) * FD + c0);
    x[0][i] = bf16_lo(w[0]);
    x[1][i] = bf16_hi(w[0]);
    x[2][i] = bf16_lo(w[1]);
    x[3][i] = bf16_hi(w[1]);
  }
  const int tile = blk >> 1, b = blk & 1;
  const long long tile_id = bh * (Np / 64) + tile;
#pragma unroll
  for (int cc = 0; cc < 4; ++cc) {
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(x[cc][i]));
    const int t = block_exponent(amax);
    // Key 8j + 4g + i of the block goes to byte 16g + 4j + i.
    float px[32];
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) px[16 * g + 4 * j + i] = x[cc][8 * j + 4 * g + i];
    uint32_t w[8];
    quantize32(px, t, w);
    const int c = c0 + cc;
    u32x4* dst = reinterpret_cast<u32x4*>(v8 + (tile_id * FD + c) * 64 + 32 * b);
    dst[0] = u32x4{w[0], w[1], w[2], w[3]};
    dst[1] = u32x4{w[4], w[5], w[6], w[7]};
    ve[((tile_id * 2 + b) * 32 + (c & 31)) * 4 + (c >> 5)] = e8m0(t);
  }
}

// Block-scaled FP8 32x32x64 product; OPA/OPB pick the scale byte.
template <int OPA, int OPB>
__device__ __forceinline__ f32x16 mfma8(v8i a, v8i b, f32x16 c, uint32_t sa, uint32_t sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, OPA, (int)sa, OPB, (int)sb);
}

__device__ __forceinline__ v8i v8i_from(u32x4 lo, u32x4 hi) {
  return v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

struct Fp8Lds {
  static constexpr int KSTR = FD + 16;     // bytes per K row (16-byte reads of 32 rows)
  static constexpr int VSTR = 64 + 16;     // bytes per V^T row
  static constexpr int K_BYTES = FBC * KSTR;
  static constexpr int KE_BYTES = FBC * 4;
  static constexpr int V_BYTES = FD * VSTR;
  static constexpr int VE_BYTES = 2 * 32 * 4;
  static constexpr int STAGE = K_BYTES + KE_BYTES + V_BYTES + VE_BYTES;
  static constexpr int BYTES = 2 * STAGE;
};

// One tile (K codes, K scales, V^T codes, V scales) by direct HBM -> LDS
// loads: each 16-byte load puts lane l's chunk 16 l bytes after its base, so
// the K rows (9 chunks each, 8 of data) take 9 loads and the V^T rows (5
// chunks, 4 of data) 10; lanes on padding get an offset past the buffer
// (zeros).  Each scale block is one 4-byte load.  Load j of the 21 is issued
// by wave j % 4.
struct Fp8TileDma {
  using L = Fp8Lds;
  static constexpr int KL = FBC * L::KSTR / 1024, VL = FD * L::VSTR / 1024;
  static_assert(KL * 1024 == FBC * L::KSTR && VL * 1024 == FD * L::VSTR, "tiles must be whole loads");
  static constexpr int NL = KL + 1 + VL + 1, PW = (NL + 3) / 4;
  uint32_t voff[PW];
  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int u = 0; u < PW; ++u) {
      const int j = wave + 4 * u;
      uint32_t o = 0x80000000u;
      if (j < KL) {
        const int p = 64 * j + lane, row = p / (L::KSTR / 16), col = p % (L::KSTR / 16);
        if (col < FD / 16) o = (uint32_t)(row * FD + col * 16);
      } else if (j == KL || j == NL - 1) {
        o = (uint32_t)lane * 4;
      } else if (j < NL) {
        const int p = 64 * (j - KL - 1) + lane, row = p / (L::VSTR / 16), col = p % (L::VSTR / 16);
        if (col < 4) o = (uint32_t)(row * 64 + col * 16);
      }
      voff[u] = o;
    }
  }
  // Tile starting at key kv0 (a multiple of FBC, below Np): the buffer
  // resources start at the tile (K and V codes kv0 * FD bytes in, their
  // scales kv0 * 4), so the per-lane offsets stay the same from tile to tile.
  __device__ __forceinline__ void issue(const RowSrc<FD, uint8_t>& k8s, const RowSrc<1, uint32_t>& kes,
                                        const RowSrc<FD, uint8_t>& v8s, const RowSrc<1, uint32_t>& ves, int kv0,
                                        uint8_t* st, int wave) const {
    const __amdgpu_buffer_rsrc_t k8 = k8s.from_row(kv0), ke = kes.from_row(kv0);
    const __amdgpu_buffer_rsrc_t v8 = v8s.from_row(kv0), ve = ves.from_row(kv0);
#pragma unroll
    for (int u = 0; u < PW; ++u) {
      const int j = wave + 4 * u;
      if (j < KL)
        lds_load16(k8, reinterpret_cast<uint16_t*>(st + 1024 * j), voff[u]);
      else if (j == KL)
        lds_load4(ke, reinterpret_cast<uint16_t*>(st + L::K_BYTES), voff[u]);
      else if (j < NL - 1)
        lds_load16(v8, reinterpret_cast<uint16_t*>(st + L::K_BYTES + L::KE_BYTES + 1024 * (j - KL - 1)), voff[u]);
      else if (j == NL - 1)
        lds_load4(ve, reinterpret_cast<uint16_t*>(st + L::K_BYTES + L::KE_BYTES + L::V_BYTES), voff[u]);
    }
  }
};

// One 64-key tile for this wave's 32 queries (same online softmax as the
// bf16 forward; see fwd_bf16.hip).  FIRST: the wave's first tile, where m is
// still -inf (the fast path would always fail) and the row sum and the
// accumulators are still zero (the rescale would leave them unchanged).
template <bool MASK, bool FIRST = false>
__device__ __forceinline__ void fp8_tile_step(const uint8_t* st, const v8i* qf, uint32_t qsc, f32x16* oacc, float& m,
                                              float& lsum, float c, int lim, int lane) {
  using L = Fp8Lds;
  const int l32 = lane & 31, h = lane >> 5;
  const uint8_t* Ks = st;
  const uint32_t* Ke = reinterpret_cast<const uint32_t*>(st + L::K_BYTES);
  const uint8_t* Vs = st + L::K_BYTES + L::KE_BYTES;
  const uint32_t* Ve = reinterpret_cast<const uint32_t*>(st + L::K_BYTES + L::KE_BYTES + L::V_BYTES);

  f32x16 s[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const uint8_t* row = Ks + (kb * 32 + l32) * L::KSTR + 16 * h;
    const v8i a0 = v8i_from(*reinterpret_cast<const u32x4*>(row), *reinterpret_cast<const u32x4*>(row + 32));
    const v8i a1 = v8i_from(*reinterpret_cast<const u32x4*>(row + 64), *reinterpret_cast<const u32x4*>(row + 96));
    const uint32_t ksc = Ke[kb * 32 + l32] >> (8 * h);
    s[kb] = mfma8<0, 0>(a0, qf[0], f32x16{}, ksc, qsc);
    s[kb] = mfma8<2, 2>(a1, qf[1], s[kb], ksc, qsc);
  }
  if (MASK) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (kb * 32 + 8 * (r >> 2) + (r & 3) > lim) s[kb][r] = -INFINITY;
  }
  // P^T operand: byte 16kb + r is p of accumulator element s[kb][r].  The
  // exponentials are first taken with the current reference max; only if
  // some p exceeds 2^FTAU (its 4-element block sum shows it) or the
  // reference is still -inf does the tile take the row max and the lazy
  // rescale, and P is recomputed (the bf16 forward does the same).
  uint32_t pw[8];
  auto probs = [&](float& l) {
    float ps[8];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int r = 4 * q4;
        const float p0 = exp2_hw(__builtin_fmaf(s[kb][r], c, -m));
        const float p1 = exp2_hw(__builtin_fmaf(s[kb][r + 1], c, -m));
        const float p2 = exp2_hw(__builtin_fmaf(s[kb][r + 2], c, -m));
        const float p3 = exp2_hw(__builtin_fmaf(s[kb][r + 3], c, -m));
        ps[4 * kb + q4] = (p0 + p1) + (p2 + p3);
        pw[4 * kb + q4] = cvt_fp8x2(p2, p3, cvt_fp8x2(p0, p1, 0u, false), true);
      }
    l += ((ps[0] + ps[1]) + (ps[2] + ps[3])) + ((ps[4] + ps[5]) + (ps[6] + ps[7]));
    return max_nan(max_nan(max_nan(ps[0], ps[1]), max_nan(ps[2], ps[3])),
                   max_nan(max_nan(ps[4], ps[5]), max_nan(ps[6], ps[7])));
  };
  float l = lsum;
  if (FIRST || __any(!(probs(l) <= 256.f))) {
    float m8[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int r = 8 * hh;
        const float a = max_nan(max_nan(s[kb][r], s[kb][r + 1]), s[kb][r + 2]);
        const float b = max_nan(max_nan(s[kb][r + 3], s[kb][r + 4]), s[kb][r + 5]);
        m8[2 * kb + hh] = max_nan(max_nan(a, b), max_nan(s[kb][r + 6], s[kb][r + 7]));
      }
    float mx = max_nan(max_nan(m8[0], m8[1]), max_nan(m8[2], m8[3]));
    mx = max_halves(mx) * c;
    if (__any(mx > m + FTAU)) {
      const float mn = fmaxf(m, mx);
      if constexpr (!FIRST) {
        const float alpha = exp2_hw(m - mn);
        lsum *= alpha;
#pragma unroll
        for (int i = 0; i < FD / 32; ++i) oacc[i] *= alpha;
      }
      m = mn;
    }
    l = lsum;
    probs(l);
  }
  lsum = l;
  const v8i pb = v8i{(int)pw[0], (int)pw[1], (int)pw[2], (int)pw[3], (int)pw[4], (int)pw[5], (int)pw[6], (int)pw[7]};
  const uint32_t vsc = Ve[h * 32 + l32];
  constexpr uint32_t ONE = 127u;
#define FA_FP8_PV(DB)                                                                                   \
  {                                                                                                     \
    const uint8_t* vr = Vs + ((DB)*32 + l32) * L::VSTR + 16 * h;                                        \
    const v8i va = v8i_from(*reinterpret_cast<const u32x4*>(vr), *reinterpret_cast<const u32x4*>(vr + 32)); \
    oacc[DB] = mfma8<DB, 0>(va, pb, oacc[DB], vsc, ONE);                                                \
  }
  FA_FP8_PV(0)
  FA_FP8_PV(1)
  FA_FP8_PV(2)
  FA_FP8_PV(3)
#undef FA_FP8_PV
}

// Three waves per SIMD: with the tiles loaded straight into LDS a wave
// needs ~160 VGPRs and a workgroup 40 KB of LDS (measured 10-12% faster than
// two waves per SIMD with register-staged tiles).
template <bool CAUSAL>
__global__ void __launch_bounds__(FNT) __attribute__((amdgpu_waves_per_eu(3, 3)))
fwd_fp8_kernel(const uint8_t* __restrict__ Q8, const uint8_t* __restrict__ QE, const uint8_t* __restrict__ K8,
               const uint8_t* __restrict__ KE, const uint8_t* __restrict__ V8, const uint8_t* __restrict__ VE,
               uint16_t* __restrict__ O, float* __restrict__ LSE, int N, int Np, int nqb, int total, float c) {
  using L = Fp8Lds;
  __shared__ __attribute__((aligned(16))) uint8_t smem[L::BYTES];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6) & (FNT / 64 - 1);  // wave-uniform, below 4
  const int l32 = lane & 31, h = lane >> 5;
  int bh, qb;
  map_block_xcd(blockIdx.x, total, nqb, CAUSAL, bh, qb);
  const size_t rows0 = (size_t)bh * Np;
  const uint32_t code_bytes = (uint32_t)Np * FD;
  const __amdgpu_buffer_rsrc_t qrs = make_rsrc(Q8 + rows0 * FD, code_bytes);
  const __amdgpu_buffer_rsrc_t qes = make_rsrc(QE + rows0 * 4, (uint32_t)Np * 4);
  // V's codes are stored in blocks of 64 keys x FD bytes, so a tile of V
  // starts kv0 * FD bytes in, as K's does.
  const RowSrc<FD, uint8_t> krs{K8 + rows0 * FD, code_bytes}, vrs{V8 + rows0 * FD, code_bytes};
  const RowSrc<1, uint32_t> kes{reinterpret_cast<const uint32_t*>(KE + rows0 * 4), (uint32_t)Np * 4},
      ves{reinterpret_cast<const uint32_t*>(VE + rows0 * 4), (uint32_t)Np * 4};
  const int q0 = qb * FBR;
  const int qw = q0 + wave * 32;
  const int myq = qw + l32;

  // Q^T operand: for product m, bytes 64m + 16h and 64m + 32 + 16h of the row.
  v8i qf[2];
#pragma unroll
  for (int mm = 0; mm < 2; ++mm) {
    const uint32_t off = (uint32_t)(myq * FD + 64 * mm + 16 * h);
    qf[mm] = v8i_from(buf_load16(qrs, off), buf_load16(qrs, off + 32));
  }
  const uint32_t qsc = __builtin_amdgcn_raw_buffer_load_b32(qes, (uint32_t)myq * 4, 0, 0) >> (8 * h);

  const int kv_end = CAUSAL ? min(N, q0 + FBR) : N;
  const int ntiles = (kv_end + FBC - 1) / FBC;

  f32x16 oacc[FD / 32];
#pragma unroll
  for (int i = 0; i < FD / 32; ++i) oacc[i] = f32x16{};
  float m = -INFINITY, lsum = 0.f;

  Fp8TileDma dma;
  dma.init(wave, lane);
  dma.issue(krs, kes, vrs, ves, 0, smem, wave);
  wait_vmem();
  __syncthreads();
  const int n_plain = min(CAUSAL ? q0 / FBC : ntiles, N / FBC);
  // Tile 0 holds key 0, which every query sees, and is every wave's first.
  auto step = [&](int j, auto mask_tag, auto first_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    constexpr bool FIRST = decltype(first_tag)::value;
    const uint8_t* st = smem + (j & 1) * L::STAGE;
    const int kv0 = j * FBC;
    if (j + 1 < ntiles) dma.issue(krs, kes, vrs, ves, kv0 + FBC, smem + ((j + 1) & 1) * L::STAGE, wave);
    if (!MASK || !CAUSAL || kv0 <= qw + 31) {
      const int lim = (CAUSAL ? min(myq, N - 1) : N - 1) - kv0 - 4 * h;
      fp8_tile_step<MASK, FIRST>(st, qf, qsc, oacc, m, lsum, c, lim, lane);
    }
    wait_vmem();
    __syncthreads();
  };
  int j = 1;
  if (n_plain > 0)
    step(0, std::false_type{}, std::true_type{});
  else
    step(0, std::true_type{}, std::true_type{});
  for (; j < n_plain; ++j) step(j, std::false_type{}, std::false_type{});
  for (; j < ntiles; ++j) step(j, std::true_type{}, std::false_type{});

  const float ltot = sum_halves(lsum);
  const float inv = rcp_hw(ltot);
  if (myq < N) {
    uint16_t* orow = O + ((size_t)bh * N + myq) * FD;
#pragma unroll
    for (int db = 0; db < FD / 32; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        u32x2 w = {pack_bf16x2(oacc[db][4 * a] * inv, oacc[db][4 * a + 1] * inv),
                   pack_bf16x2(oacc[db][4 * a + 2] * inv, oacc[db][4 * a + 3] * inv)};
        *reinterpret_cast<u32x2*>(orow + db * 32 + 8 * a + 4 * h) = w;
      }
    if (h == 0) LSE[(size_t)bh * N + myq] = (m + log2_hw(ltot)) * kLn2;
  }
}

}  // namespace

Fp8Buffer fp8_buffer_layout(long long BH, int N) {
  Fp8Buffer b;
  const long long Np = (N + 63) / 64 * 64;
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  size_t off = 0;
  b.q8 = off; off = up(off + (size_t)BH * Np * FD);
  b.qe = off; off = up(off + (size_t)BH * Np * 4);
  b.k8 = off; off = up(off + (size_t)BH * Np * FD);
  b.ke = off; off = up(off + (size_t)BH * Np * 4);
  b.v8 = off; off = up(off + (size_t)BH * Np * FD);
  b.ve = off; off = up(off + (size_t)BH * Np * 4);
  b.bytes = off;
  b.Np = (int)Np;
  return b;
}

hipError_t launch_fp8_prepare(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* signs, int BH,
                              int N, void* buf, hipStream_t stream) {
  const Fp8Buffer L = fp8_buffer_layout(BH, N);
  uint8_t* base = static_cast<uint8_t*>(buf);
  const long long rows = (long long)BH * L.Np;
  const long long vt = (long long)BH * (L.Np / 32) * (FD / 4);
  // the limits of these launches and of launch_fwd_fp8, checked before
  // anything is launched (fa_forward_fp8 runs this first)
  const long long nqb = (N + FBR - 1) / FBR;
  if ((rows + 63) / 64 > 0x7fffffffLL || (vt + 255) / 256 > 0x7fffffffLL || (long long)BH * nqb > 0x7fffffffLL ||
      (long long)L.Np * FD >= (1LL << 31))
    return hipErrorInvalidValue;
  const unsigned rb = (unsigned)((rows + 63) / 64);   // 64 rows per workgroup
  hipLaunchKernelGGL(fp8_quant_rows_kernel, dim3(rb), dim3(256), 0, stream, q, signs, base + L.q8, base + L.qe, N,
                     L.Np, rows);
  hipLaunchKernelGGL(fp8_quant_rows_kernel, dim3(rb), dim3(256), 0, stream, k, signs, base + L.k8, base + L.ke, N,
                     L.Np, rows);
  hipLaunchKernelGGL(fp8_quant_v_kernel, dim3((unsigned)((vt + 255) / 256)), dim3(256), 0, stream, v, base + L.v8,
                     base + L.ve, N, L.Np, vt);
  return hipGetLastError();
}

hipError_t launch_fwd_fp8(const void* buf, uint16_t* o, float* lse, int BH, int N, bool causal, float scale,
                          bool rotated, hipStream_t stream) {
  const Fp8Buffer L = fp8_buffer_layout(BH, N);
  const uint8_t* base = static_cast<const uint8_t*>(buf);
  const int nqb = (N + FBR - 1) / FBR;
  const long long total = (long long)BH * nqb;
  if (total > 0x7fffffffLL || (long long)L.Np * FD >= (1LL << 31)) return hipErrorInvalidValue;
  const float c = score_coef(scale) * (rotated ? 1.0f / FD : 1.0f);
  if (causal)
    hipLaunchKernelGGL((fwd_fp8_kernel<true>), dim3((unsigned)total), dim3(FNT), 0, stream, base + L.q8,
                       base + L.qe, base + L.k8, base + L.ke, base + L.v8, base + L.ve, o, lse, N, L.Np, nqb,
                       (int)total, c);
  else
    hipLaunchKernelGGL((fwd_fp8_kernel<false>), dim3((unsigned)total), dim3(FNT), 0, stream, base + L.q8,
                       base + L.qe, base + L.k8, base + L.ke, base + L.v8, base + L.ve, o, lse, N, L.Np, nqb,
                       (int)total, c);
  return hipGetLastError();
}

}  // namespace fa
