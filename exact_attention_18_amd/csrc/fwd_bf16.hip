// Forward exact attention, bf16 in/out, float32 accumulation, for gfx950.
//
// Algorithm (pages: "FlashAttention-2を読む：長い文脈のアテンションをGPUで効率化する仕組み",
// sections 「タイル分割でも全体の正規化を保つ」 and 「GPUの稼働率を高める三つの工夫」;
// "Flash Attention 2で打破するローカルLLMの「メモリの壁」：IO最適化の実践的エンジニアリング",
// section 「タイリング（Tiling）と再計算（Recomputation）の仕組み」):
//  * one workgroup per (batch*head, block of 128 queries); its 4 waves each own
//    32 queries and share every K/V tile (the query split across warps of
//    FlashAttention-2, on 64-wide waves);
//  * K/V tiles of 64 keys stream through a double-buffered LDS stage; tile j+1
//    is fetched into registers while tile j is computed;
//  * S^T = K Q^T and O^T += V^T P^T on the bf16 matrix cores.  Computing the
//    transposed products puts one query per lane (two lanes per query), so
//    the row max, the row sum and the output rescale are per-lane values;
//  * online softmax in the base-2 domain: scale*log2(e) is folded into one
//    multiply-add before v_exp_f32; the running max is only raised when a
//    tile's max exceeds it by more than 2^8 (the numerator and denominator
//    share the reference, so the result is unchanged); 1/l is applied once,
//    in the epilogue;
//  * causal: tiles above the diagonal are never loaded; the mask code runs
//    only on tiles that straddle the diagonal or the ragged end of N.
#include "fa_common.h"
#include "launch.h"

namespace fa {
namespace {

constexpr int BR = 128;       // queries per workgroup
constexpr int BC = 64;        // keys per tile
constexpr int NT = 256;       // threads per workgroup (4 waves)
constexpr float TAU = 8.0f;   // lazy-rescale threshold, log2 units

template <int D>
struct Lds {
  static constexpr int KS = D + 8;          // K tile row stride (elements)
  static constexpr int VS = BC + 4;         // V^T tile row stride (elements)
  static constexpr int K_ELEMS = BC * KS;
  static constexpr int V_ELEMS = D * VS;
  static constexpr int STAGE = K_ELEMS + V_ELEMS;
  static constexpr int ELEMS = 2 * STAGE;   // double buffer
  static constexpr int KCH = BC * D / 8 / NT;          // 16-byte K chunks per thread
  static constexpr int VBLK = BC / 4 * D / 8;          // 4-key x 8-column V blocks
  static constexpr int VPT = (VBLK + NT - 1) / NT;     // V blocks per thread
};

template <int D>
struct TileRegs {
  uint4 k[Lds<D>::KCH];
  uint4 v[Lds<D>::VPT][4];
};

template <int D>
__device__ __forceinline__ void load_tile(TileRegs<D>& r, const uint16_t* __restrict__ K,
                                          const uint16_t* __restrict__ V, int kv0, int N, int tid) {
  constexpr int CPR = D / 8;  // 16-byte chunks per row
#pragma unroll
  for (int i = 0; i < Lds<D>::KCH; ++i) {
    const int c = tid + NT * i;
    const int row = c / CPR, col = (c % CPR) * 8;
    const int key = kv0 + row;
    r.k[i] = key < N ? *reinterpret_cast<const uint4*>(K + (size_t)key * D + col) : uint4{0, 0, 0, 0};
  }
#pragma unroll
  for (int i = 0; i < Lds<D>::VPT; ++i) {
    const int b = tid + NT * i;
    if (b < Lds<D>::VBLK) {
      const int kq = b / CPR, col = (b % CPR) * 8;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = kv0 + 4 * kq + e;
        r.v[i][e] = key < N ? *reinterpret_cast<const uint4*>(V + (size_t)key * D + col) : uint4{0, 0, 0, 0};
      }
    }
  }
}

template <int D>
__device__ __forceinline__ void store_tile(const TileRegs<D>& r, uint16_t* Ks, uint16_t* Vt, int tid) {
  constexpr int CPR = D / 8;
  constexpr int KS = Lds<D>::KS, VS = Lds<D>::VS;
#pragma unroll
  for (int i = 0; i < Lds<D>::KCH; ++i) {
    const int c = tid + NT * i;
    const int row = c / CPR, col = (c % CPR) * 8;
    *reinterpret_cast<uint4*>(Ks + row * KS + col) = r.k[i];
  }
  // V is stored transposed (column d holds 64 consecutive keys) so that the
  // PV product can read 4 consecutive keys of one column with one 8-byte load.
#pragma unroll
  for (int i = 0; i < Lds<D>::VPT; ++i) {
    const int b = tid + NT * i;
    if (b < Lds<D>::VBLK) {
      const int kq = b / CPR, col = (b % CPR) * 8;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t w0 = word_of(r.v[i][0], p), w1 = word_of(r.v[i][1], p);
        const uint32_t w2 = word_of(r.v[i][2], p), w3 = word_of(r.v[i][3], p);
        uint2 even = {lo_halves(w0, w1), lo_halves(w2, w3)};
        uint2 odd = {hi_halves(w0, w1), hi_halves(w2, w3)};
        *reinterpret_cast<uint2*>(Vt + (col + 2 * p) * VS + 4 * kq) = even;
        *reinterpret_cast<uint2*>(Vt + (col + 2 * p + 1) * VS + 4 * kq) = odd;
      }
    }
  }
}

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
fwd_bf16_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
                float* __restrict__ LSE, int N, int nqb, int total, float c) {
  using L = Lds<D>;
  constexpr int KSTEPS = D / 16;   // contraction steps of S^T = K Q^T
  constexpr int DB = D / 32;       // 32-row blocks of O^T
  __shared__ __attribute__((aligned(16))) uint16_t smem[L::ELEMS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  int bh, qb;
  map_block_xcd(blockIdx.x, total, nqb, CAUSAL, bh, qb);
  const size_t base = (size_t)bh * N * D;
  const uint16_t* Kh = K + base;
  const uint16_t* Vh = V + base;
  const int q0 = qb * BR;
  const int qw = q0 + wave * 32;   // first query of this wave
  const int myq = qw + l32;        // query owned by this lane (with its partner lane)

  // Q fragment: lane holds Q[myq][16*ks + 8*g .. +8] for every contraction step.
  bf16x8 qf[KSTEPS];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
    uint4 u = {0, 0, 0, 0};
    if (myq < N) u = *reinterpret_cast<const uint4*>(Q + base + (size_t)myq * D + ks * 16 + 8 * g);
    qf[ks] = bf16x8_from(u);
  }

  const int kv_end = CAUSAL ? min(N, q0 + BR) : N;
  const int ntiles = (kv_end + BC - 1) / BC;

  f32x16 oacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) oacc[i] = f32x16{};
  float m = -INFINITY;   // running max of scale*log2e*s for query myq
  float lsum = 0.f;      // this lane's share of the running row sum

  TileRegs<D> regs;
  load_tile<D>(regs, Kh, Vh, 0, N, tid);
  store_tile<D>(regs, smem, smem + L::K_ELEMS, tid);
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    const uint16_t* Ks = smem + (j & 1) * L::STAGE;
    const uint16_t* Vt = Ks + L::K_ELEMS;
    const int kv0 = j * BC;
    if (j + 1 < ntiles) load_tile<D>(regs, Kh, Vh, kv0 + BC, N, tid);

    if (!CAUSAL || kv0 <= qw + 31) {
      // S^T tile: s[kb] element r is key kv0 + 32*kb + 8*(r/4) + 4*g + r%4, query myq.
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = f32x16{};
        const uint16_t* krow = Ks + (kb * 32 + l32) * L::KS + 8 * g;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
          const bf16x8 a = bf16x8_from(*reinterpret_cast<const uint4*>(krow + ks * 16));
          s[kb] = mfma32(a, qf[ks], s[kb]);
        }
      }

      const bool masked = (CAUSAL && kv0 + BC - 1 > qw) || (kv0 + BC > N);
      float mx = -INFINITY;
      if (masked) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kv0 + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
            const bool hide = key >= N || (CAUSAL && key > myq);
            const float t = hide ? -INFINITY : s[kb][r] * c;
            s[kb][r] = t;
            mx = fmaxf(mx, t);
          }
      } else {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
        mx *= c;
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32));

      // Raise the reference max only when some row's tile max exceeds it by
      // more than TAU; otherwise p stays below 2^TAU and nothing is rescaled.
      if (__any(mx > m + TAU)) {
        const float mn = fmaxf(m, mx);
        const float alpha = exp2_hw(m - mn);
        m = mn;
        lsum *= alpha;
#pragma unroll
        for (int i = 0; i < DB; ++i) oacc[i] *= alpha;
      }

      // P^T as the B operand of the PV product: 8 consecutive accumulator
      // elements (r = 8t .. 8t+7) of block kb form contraction step (kb, t).
      bf16x8 pf[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          uint32_t w[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 8 * t + 2 * e;
            float p0, p1;
            if (masked) {
              p0 = exp2_hw(s[kb][r] - m);
              p1 = exp2_hw(s[kb][r + 1] - m);
            } else {
              p0 = exp2_hw(__builtin_fmaf(s[kb][r], c, -m));
              p1 = exp2_hw(__builtin_fmaf(s[kb][r + 1], c, -m));
            }
            w[e] = pack_bf16x2(p0, p1);
            lsum += p0;
            lsum += p1;
          }
          pf[kb][t] = __builtin_bit_cast(bf16x8, uint4{w[0], w[1], w[2], w[3]});
        }

      // O^T += V^T P^T.  Slot (g, v) of step (kb, t) is key
      // 32*kb + 16*t + 8*(v/4) + 4*g + v%4: two 8-byte reads of V^T row d.
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const uint16_t* vp = Vt + (db * 32 + l32) * L::VS + kb * 32 + 16 * t + 4 * g;
            const bf16x8 a = bf16x8_from(*reinterpret_cast<const uint2*>(vp),
                                         *reinterpret_cast<const uint2*>(vp + 8));
            oacc[db] = mfma32(a, pf[kb][t], oacc[db]);
          }
        }
    }

    if (j + 1 < ntiles) store_tile<D>(regs, smem + ((j + 1) & 1) * L::STAGE,
                                      smem + ((j + 1) & 1) * L::STAGE + L::K_ELEMS, tid);
    __syncthreads();
  }

  // Epilogue: O = O^T / l, LSE = ln2 * (m + log2 l).
  const float ltot = lsum + __shfl_xor(lsum, 32);
  const float inv = rcp_hw(ltot);
  if (myq < N) {
    uint16_t* orow = O + base + (size_t)myq * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        uint2 w = {pack_bf16x2(oacc[db][4 * a] * inv, oacc[db][4 * a + 1] * inv),
                   pack_bf16x2(oacc[db][4 * a + 2] * inv, oacc[db][4 * a + 3] * inv)};
        *reinterpret_cast<uint2*>(orow + db * 32 + 8 * a + 4 * g) = w;
      }
    if (g == 0) LSE[(size_t)bh * N + myq] = (m + log2_hw(ltot)) * kLn2;
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, float* lse,
                  int BH, int N, float scale, hipStream_t stream) {
  const int nqb = (N + BR - 1) / BR;
  const long long total = (long long)BH * nqb;
  if (total > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL>), dim3((unsigned)total), dim3(NT), 0, stream,
                     q, k, v, o, lse, N, nqb, (int)total, scale * kLog2e);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                           float* lse, int BH, int N, int d, bool causal, float scale,
                           hipStream_t stream) {
  if (d == 64) return causal ? launch<64, true>(q, k, v, o, lse, BH, N, scale, stream)
                             : launch<64, false>(q, k, v, o, lse, BH, N, scale, stream);
  if (d == 128) return causal ? launch<128, true>(q, k, v, o, lse, BH, N, scale, stream)
                              : launch<128, false>(q, k, v, o, lse, BH, N, scale, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa
