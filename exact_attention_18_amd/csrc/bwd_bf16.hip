// Backward exact attention, bf16 in/out, float32 accumulation, for gfx950.
//
// The probabilities are recomputed from Q, K and the saved LSE instead of
// being stored (page "Flash Attention 2で打破するローカルLLMの「メモリの壁」：IO最適化の
// 実践的エンジニアリング", section 「タイリング（Tiling）と再計算（Recomputation）の仕組み」).
// With P = exp(scale*Q K^T - LSE) (masked entries 0) and delta = rowsum(dO * O):
//     dV = P^T dO,   dP = dO V^T,   dS = P * (dP - delta),
//     dQ = scale * dS K,   dK = scale * dS^T Q.
// Three launches on one stream, no atomics, so the result is bit-reproducible:
//   1. delta (row-dot pre-pass, in f32_path.hip);
//   2. dK/dV: one workgroup per (batch*head, 128 keys), each wave owning 32
//      keys and looping over query tiles of 32 (causal: from the diagonal on);
//   3. dQ: one workgroup per (batch*head, 128 queries), each wave owning 32
//      queries and looping over key tiles of 64 (causal: up to the diagonal).
// Every product runs on the 32x32x16 bf16 matrix cores.  Each kernel picks
// the orientation (S or S^T) in which the operand it keeps in registers sits
// on the lanes, and stages the other operands in LDS in both row-major and
// transposed form, so every matrix-core operand is read with 8- or 16-byte
// LDS loads.
#include "fa_common.h"
#include "launch.h"

namespace fa {
namespace {

constexpr int NT = 256;

// Stage rows [r0, r0+ROWS) of a [N][D] bf16 matrix into LDS, row-major with
// row stride RS elements; rows at or beyond N become zero.
template <int ROWS, int D, int RS>
__device__ __forceinline__ void stage_rm(uint16_t* dst, const uint16_t* __restrict__ src, int r0, int N,
                                         int tid) {
  constexpr int CPR = D / 8;
#pragma unroll
  for (int c = tid; c < ROWS * CPR; c += NT) {
    const int row = c / CPR, col = (c % CPR) * 8;
    u32x4 x = {0, 0, 0, 0};
    if (r0 + row < N) x = *reinterpret_cast<const u32x4*>(src + (size_t)(r0 + row) * D + col);
    *reinterpret_cast<u32x4*>(dst + row * RS + col) = x;
  }
}

// Stage the same rows both row-major (stride RS) and transposed (column c of
// the tile becomes row c of `dst_t`, stride TS, so 4 consecutive source rows
// of one column are one 8-byte word).
template <int ROWS, int D, int RS, int TS>
__device__ __forceinline__ void stage_rm_t(uint16_t* dst_rm, uint16_t* dst_t, const uint16_t* __restrict__ src,
                                           int r0, int N, int tid) {
  constexpr int CPR = D / 8;
#pragma unroll
  for (int b = tid; b < ROWS / 4 * CPR; b += NT) {
    const int rq = b / CPR, col = (b % CPR) * 8;
    u32x4 x[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = r0 + 4 * rq + e;
      x[e] = row < N ? *reinterpret_cast<const u32x4*>(src + (size_t)row * D + col) : u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(dst_rm + (4 * rq + e) * RS + col) = x[e];
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t w0 = word_of(x[0], p), w1 = word_of(x[1], p);
      const uint32_t w2 = word_of(x[2], p), w3 = word_of(x[3], p);
      *reinterpret_cast<u32x2*>(dst_t + (col + 2 * p) * TS + 4 * rq) = u32x2{lo_halves(w0, w1), lo_halves(w2, w3)};
      *reinterpret_cast<u32x2*>(dst_t + (col + 2 * p + 1) * TS + 4 * rq) = u32x2{hi_halves(w0, w1), hi_halves(w2, w3)};
    }
  }
}

// 8 bf16 MFMA-operand values of a transposed tile: row `row`, contraction
// slots (g, v) of step t mapped to columns 16t + 8(v/4) + 4g + v%4.
__device__ __forceinline__ bf16x8 read_t_operand(const uint16_t* t_row, int col16, int g) {
  const uint16_t* p = t_row + col16 + 4 * g;
  return bf16x8_from(*reinterpret_cast<const u32x2*>(p), *reinterpret_cast<const u32x2*>(p + 8));
}

// Accumulator elements r = 8t .. 8t+7 of `x` as one bf16 operand.
__device__ __forceinline__ bf16x8 acc_to_operand(const f32x16& x, int t) {
  u32x4 u = {pack_bf16x2(x[8 * t + 0], x[8 * t + 1]), pack_bf16x2(x[8 * t + 2], x[8 * t + 3]),
             pack_bf16x2(x[8 * t + 4], x[8 * t + 5]), pack_bf16x2(x[8 * t + 6], x[8 * t + 7])};
  return __builtin_bit_cast(bf16x8, u);
}

// Store a [D][32] accumulator set (D/32 blocks; lane holds column l%32) as
// rows of a [N][D] bf16 matrix: element r of block db is column
// 32*db + 8*(r/4) + 4*g + r%4 of row `row`.
template <int D>
__device__ __forceinline__ void store_acc_rows(uint16_t* __restrict__ dst_row, const f32x16 (&acc)[D / 32],
                                               float mul, int g) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      u32x2 w = {pack_bf16x2(acc[db][4 * a] * mul, acc[db][4 * a + 1] * mul),
                 pack_bf16x2(acc[db][4 * a + 2] * mul, acc[db][4 * a + 3] * mul)};
      *reinterpret_cast<u32x2*>(dst_row + db * 32 + 8 * a + 4 * g) = w;
    }
}

// ---------------------------------------------------------------- dK / dV
constexpr int KV_BLK = 128;   // keys per workgroup
constexpr int Q_TILE = 32;    // queries per tile

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(NT)
bwd_dkdv_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                const uint16_t* __restrict__ V, const float* __restrict__ LSE,
                const uint16_t* __restrict__ dO, const float* __restrict__ delta,
                uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int N, int nkb, int total,
                float c, float scale) {
  constexpr int RS = D + 8, TS = Q_TILE + 4, KSTEPS = D / 16, DB = D / 32;
  __shared__ __attribute__((aligned(16))) uint16_t Qs[Q_TILE * RS];
  __shared__ __attribute__((aligned(16))) uint16_t Qt[D * TS];
  __shared__ __attribute__((aligned(16))) uint16_t Gs[Q_TILE * RS];
  __shared__ __attribute__((aligned(16))) uint16_t Gt[D * TS];
  __shared__ float lse2[Q_TILE], dl[Q_TILE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int l32 = lane & 31, g = lane >> 5;
  int bh, kb;
  map_block_xcd(blockIdx.x, total, nkb, false, bh, kb);  // causal: low key blocks carry the most work
  const size_t base = (size_t)bh * N * D;
  const int k0 = kb * KV_BLK;
  const int kw = k0 + wave * 32;
  const int myk = kw + l32;

  // K and V rows of this lane's key, as B operands (K^T / V^T columns).
  bf16x8 kf[KSTEPS], vf[KSTEPS];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
    u32x4 a = {0, 0, 0, 0}, b = {0, 0, 0, 0};
    if (myk < N) {
      a = *reinterpret_cast<const u32x4*>(K + base + (size_t)myk * D + ks * 16 + 8 * g);
      b = *reinterpret_cast<const u32x4*>(V + base + (size_t)myk * D + ks * 16 + 8 * g);
    }
    kf[ks] = bf16x8_from(a);
    vf[ks] = bf16x8_from(b);
  }
  f32x16 dkt[DB], dvt[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) dkt[i] = dvt[i] = f32x16{};

  const int qstart = CAUSAL ? k0 : 0;
  for (int qt0 = qstart; qt0 < N; qt0 += Q_TILE) {
    stage_rm_t<Q_TILE, D, RS, TS>(Qs, Qt, Q + base, qt0, N, tid);
    stage_rm_t<Q_TILE, D, RS, TS>(Gs, Gt, dO + base, qt0, N, tid);
    if (tid < Q_TILE) {
      const int qi = qt0 + tid;
      lse2[tid] = qi < N ? LSE[(size_t)bh * N + qi] * kLog2e : INFINITY;
      dl[tid] = qi < N ? delta[(size_t)bh * N + qi] : 0.f;
    }
    __syncthreads();

    if (!CAUSAL || qt0 + Q_TILE - 1 >= kw) {
      // S and dP with queries in registers (element r: query qt0 + 8(r/4) + 4g + r%4)
      // and this lane's key on the lane.
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        const bf16x8 qa = bf16x8_from(*reinterpret_cast<const u32x4*>(Qs + l32 * RS + ks * 16 + 8 * g));
        const bf16x8 ga = bf16x8_from(*reinterpret_cast<const u32x4*>(Gs + l32 * RS + ks * 16 + 8 * g));
        s = mfma32(qa, kf[ks], s);
        dp = mfma32(ga, vf[ks], dp);
      }
      const bool masked = (CAUSAL && qt0 < kw + 31) || (k0 + KV_BLK > N);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qr = 8 * (r >> 2) + 4 * g + (r & 3);
        float p = exp2_hw(__builtin_fmaf(s[r], c, -lse2[qr]));
        if (masked && (myk >= N || (CAUSAL && myk > qt0 + qr))) p = 0.f;
        s[r] = p;
        dp[r] = p * (dp[r] - dl[qr]);
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const bf16x8 pb = acc_to_operand(s, t);
        const bf16x8 db_ = acc_to_operand(dp, t);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          dvt[db] = mfma32(read_t_operand(Gt + (db * 32 + l32) * TS, 16 * t, g), pb, dvt[db]);
          dkt[db] = mfma32(read_t_operand(Qt + (db * 32 + l32) * TS, 16 * t, g), db_, dkt[db]);
        }
      }
    }
    __syncthreads();
  }
  if (myk < N) {
    store_acc_rows<D>(dK + base + (size_t)myk * D, dkt, scale, g);
    store_acc_rows<D>(dV + base + (size_t)myk * D, dvt, 1.0f, g);
  }
}

// ---------------------------------------------------------------- dQ
constexpr int Q_BLK = 128;    // queries per workgroup
constexpr int K_TILE = 64;    // keys per tile

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(NT)
bwd_dq_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
              const uint16_t* __restrict__ V, const float* __restrict__ LSE,
              const uint16_t* __restrict__ dO, const float* __restrict__ delta,
              uint16_t* __restrict__ dQ, int N, int nqb, int total, float c, float scale) {
  constexpr int RS = D + 8, TS = K_TILE + 4, KSTEPS = D / 16, DB = D / 32;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[K_TILE * RS];
  __shared__ __attribute__((aligned(16))) uint16_t Kt[D * TS];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[K_TILE * RS];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int l32 = lane & 31, g = lane >> 5;
  int bh, qb;
  map_block_xcd(blockIdx.x, total, nqb, CAUSAL, bh, qb);
  const size_t base = (size_t)bh * N * D;
  const int q0 = qb * Q_BLK;
  const int qw = q0 + wave * 32;
  const int myq = qw + l32;

  bf16x8 qf[KSTEPS], gf[KSTEPS];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
    u32x4 a = {0, 0, 0, 0}, b = {0, 0, 0, 0};
    if (myq < N) {
      a = *reinterpret_cast<const u32x4*>(Q + base + (size_t)myq * D + ks * 16 + 8 * g);
      b = *reinterpret_cast<const u32x4*>(dO + base + (size_t)myq * D + ks * 16 + 8 * g);
    }
    qf[ks] = bf16x8_from(a);
    gf[ks] = bf16x8_from(b);
  }
  const float lse2 = myq < N ? LSE[(size_t)bh * N + myq] * kLog2e : INFINITY;
  const float dlv = myq < N ? delta[(size_t)bh * N + myq] : 0.f;
  f32x16 dqt[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) dqt[i] = f32x16{};

  const int kv_end = CAUSAL ? min(N, q0 + Q_BLK) : N;
  for (int kv0 = 0; kv0 < kv_end; kv0 += K_TILE) {
    stage_rm_t<K_TILE, D, RS, TS>(Ks, Kt, K + base, kv0, N, tid);
    stage_rm<K_TILE, D, RS>(Vs, V + base, kv0, N, tid);
    __syncthreads();
    if (!CAUSAL || kv0 <= qw + 31) {
      const bool masked = (CAUSAL && kv0 + K_TILE - 1 > qw) || (kv0 + K_TILE > N);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        // S^T and dP^T: element r is key kv0 + 32kb + 8(r/4) + 4g + r%4, query myq.
        f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
          const bf16x8 ka = bf16x8_from(*reinterpret_cast<const u32x4*>(Ks + (kb * 32 + l32) * RS + ks * 16 + 8 * g));
          const bf16x8 va = bf16x8_from(*reinterpret_cast<const u32x4*>(Vs + (kb * 32 + l32) * RS + ks * 16 + 8 * g));
          s = mfma32(ka, qf[ks], s);
          dp = mfma32(va, gf[ks], dp);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kv0 + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
          float p = exp2_hw(__builtin_fmaf(s[r], c, -lse2));
          if (masked && (key >= N || (CAUSAL && key > myq))) p = 0.f;
          dp[r] = p * (dp[r] - dlv);
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const bf16x8 dsb = acc_to_operand(dp, t);
#pragma unroll
          for (int db = 0; db < DB; ++db)
            dqt[db] = mfma32(read_t_operand(Kt + (db * 32 + l32) * TS, kb * 32 + 16 * t, g), dsb, dqt[db]);
        }
      }
    }
    __syncthreads();
  }
  if (myq < N) store_acc_rows<D>(dQ + base + (size_t)myq * D, dqt, scale, g);
}

template <int D, bool CAUSAL>
hipError_t launch_dkdv(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* lse,
                       const uint16_t* dO, const float* delta, uint16_t* dk, uint16_t* dv, int BH,
                       int N, float scale, hipStream_t stream) {
  const int nkb = (N + KV_BLK - 1) / KV_BLK;
  const long long tk = (long long)BH * nkb;
  if (tk > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3((unsigned)tk), dim3(NT), 0, stream, q, k, v, lse,
                     dO, delta, dk, dv, N, nkb, (int)tk, scale * kLog2e, scale);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_dq(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* lse,
                     const uint16_t* dO, const float* delta, uint16_t* dq, int BH, int N, float scale,
                     hipStream_t stream) {
  const int nqb = (N + Q_BLK - 1) / Q_BLK;
  const long long tq = (long long)BH * nqb;
  if (tq > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3((unsigned)tq), dim3(NT), 0, stream, q, k, v, lse,
                     dO, delta, dq, N, nqb, (int)tq, scale * kLog2e, scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_dkdv_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                const float* lse, const uint16_t* dO, const float* delta,
                                uint16_t* dk, uint16_t* dv, int BH, int N, int d, bool causal,
                                float scale, hipStream_t stream) {
  if (d == 64)
    return causal ? launch_dkdv<64, true>(q, k, v, lse, dO, delta, dk, dv, BH, N, scale, stream)
                  : launch_dkdv<64, false>(q, k, v, lse, dO, delta, dk, dv, BH, N, scale, stream);
  if (d == 128)
    return causal ? launch_dkdv<128, true>(q, k, v, lse, dO, delta, dk, dv, BH, N, scale, stream)
                  : launch_dkdv<128, false>(q, k, v, lse, dO, delta, dk, dv, BH, N, scale, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_dq_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              const float* lse, const uint16_t* dO, const float* delta,
                              uint16_t* dq, int BH, int N, int d, bool causal, float scale,
                              hipStream_t stream) {
  if (d == 64)
    return causal ? launch_dq<64, true>(q, k, v, lse, dO, delta, dq, BH, N, scale, stream)
                  : launch_dq<64, false>(q, k, v, lse, dO, delta, dq, BH, N, scale, stream);
  if (d == 128)
    return causal ? launch_dq<128, true>(q, k, v, lse, dO, delta, dq, BH, N, scale, stream)
                  : launch_dq<128, false>(q, k, v, lse, dO, delta, dq, BH, N, scale, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                           const uint16_t* o, const float* lse, const uint16_t* dO, uint16_t* dq,
                           uint16_t* dk, uint16_t* dv, int BH, int N, int d, bool causal,
                           float scale, float* delta, hipStream_t stream) {
  hipError_t e = launch_rowdot_bf16(o, dO, delta, (long long)BH * N, d, stream);
  if (e != hipSuccess) return e;
  e = launch_bwd_dkdv_bf16(q, k, v, lse, dO, delta, dk, dv, BH, N, d, causal, scale, stream);
  if (e != hipSuccess) return e;
  return launch_bwd_dq_bf16(q, k, v, lse, dO, delta, dq, BH, N, d, causal, scale, stream);
}

}  // namespace fa
