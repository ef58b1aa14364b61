// float32 debug path: forward and backward exact attention with float32
// storage and arithmetic on the vector ALUs.  Same tiling, online softmax,
// base-2 exponentials, deferred 1/l and diagonal-only masking as the bf16
// kernels; only the arithmetic type differs.  Also the row-dot pre-pass of
// the backward (delta_i = sum_c dO_ic O_ic) for both element types.
//
// Backward (pages only say the probabilities are recomputed rather than
// stored: "Flash Attention 2で打破するローカルLLMの「メモリの壁」：IO最適化の実践的
// エンジニアリング", section 「タイリング（Tiling）と再計算（Recomputation）の仕組み」):
// with P rebuilt as exp(scale*q.k - LSE), dV = P^T dO, dP = dO V^T,
// dS = P * (dP - delta), dQ = scale * dS K, dK = scale * dS^T Q.
//
// Thread layout: four consecutive threads share one row (a query row, or a
// key row in the dK/dV kernel); thread `part` owns the 4-wide column chunks
// part, part+4, part+8, ... of the head dimension (d <= 128, d % 4 == 0).
// Dot products are summed over the four threads with two xor shuffles.
#include "fa_common.h"
#include "launch.h"

namespace fa {
namespace {

constexpr int ROWS = 64;     // rows per workgroup
constexpr int TILE = 32;     // keys (or queries) per LDS tile
constexpr int NT = 256;
constexpr int MAXC = 8;      // chunks per thread: 8 x 4 = 32 columns = 128 / 4 threads

__device__ __forceinline__ float quad_sum(float x) {
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  return x;
}

// Load `rows_in_tile` rows starting at row r0 of a [N][d] matrix into an LDS
// tile with row stride 128 floats; rows at or beyond N become zero.
__device__ __forceinline__ void stage_rows(float* dst, const float* __restrict__ src, int r0, int N,
                                           int d, int tid) {
  const int cpr = d / 4;
  for (int c = tid; c < TILE * cpr; c += NT) {
    const int row = c / cpr, col = (c % cpr) * 4;
    float4 x = {0.f, 0.f, 0.f, 0.f};
    if (r0 + row < N) x = *reinterpret_cast<const float4*>(src + (size_t)(r0 + row) * d + col);
    *reinterpret_cast<float4*>(dst + row * 128 + col) = x;
  }
}

__device__ __forceinline__ void load_row(float (&x)[MAXC][4], const float* __restrict__ p, int d,
                                         int part, bool valid) {
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int col = (4 * i + part) * 4;
    float4 t = {0.f, 0.f, 0.f, 0.f};
    if (valid && col < d) t = *reinterpret_cast<const float4*>(p + col);
    x[i][0] = t.x; x[i][1] = t.y; x[i][2] = t.z; x[i][3] = t.w;
  }
}

__device__ __forceinline__ float dot_lds(const float (&x)[MAXC][4], const float* row, int d, int part) {
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int col = (4 * i + part) * 4;
    if (col < d) {
      const float4 y = *reinterpret_cast<const float4*>(row + col);
      acc = __builtin_fmaf(x[i][0], y.x, acc);
      acc = __builtin_fmaf(x[i][1], y.y, acc);
      acc = __builtin_fmaf(x[i][2], y.z, acc);
      acc = __builtin_fmaf(x[i][3], y.w, acc);
    }
  }
  return quad_sum(acc);
}

__device__ __forceinline__ void axpy_lds(float (&acc)[MAXC][4], float a, const float* row, int d, int part) {
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int col = (4 * i + part) * 4;
    if (col < d) {
      const float4 y = *reinterpret_cast<const float4*>(row + col);
      acc[i][0] = __builtin_fmaf(a, y.x, acc[i][0]);
      acc[i][1] = __builtin_fmaf(a, y.y, acc[i][1]);
      acc[i][2] = __builtin_fmaf(a, y.z, acc[i][2]);
      acc[i][3] = __builtin_fmaf(a, y.w, acc[i][3]);
    }
  }
}

__device__ __forceinline__ void store_row(float* __restrict__ p, const float (&x)[MAXC][4], float mul,
                                          int d, int part) {
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int col = (4 * i + part) * 4;
    if (col < d) {
      float4 t = {x[i][0] * mul, x[i][1] * mul, x[i][2] * mul, x[i][3] * mul};
      *reinterpret_cast<float4*>(p + col) = t;
    }
  }
}

template <bool CAUSAL>
__global__ void __launch_bounds__(NT)
fwd_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
               float* __restrict__ O, float* __restrict__ LSE, int N, int d, int nqb, float c) {
  __shared__ __attribute__((aligned(16))) float Ks[TILE * 128];
  __shared__ __attribute__((aligned(16))) float Vs[TILE * 128];
  const int tid = threadIdx.x, part = tid & 3;
  const int bh = blockIdx.x / nqb, qb = blockIdx.x % nqb;
  const int q0 = qb * ROWS, myq = q0 + (tid >> 2);
  const size_t base = (size_t)bh * N * d;
  float q[MAXC][4], o[MAXC][4];
  load_row(q, Q + base + (size_t)myq * d, d, part, myq < N);
#pragma unroll
  for (int i = 0; i < MAXC; ++i) o[i][0] = o[i][1] = o[i][2] = o[i][3] = 0.f;
  float m = -INFINITY, l = 0.f;

  const int kv_end = CAUSAL ? min(N, q0 + ROWS) : N;
  for (int kv0 = 0; kv0 < kv_end; kv0 += TILE) {
    stage_rows(Ks, K + base, kv0, N, d, tid);
    stage_rows(Vs, V + base, kv0, N, d, tid);
    __syncthreads();
    const bool masked = (CAUSAL && kv0 + TILE - 1 > q0) || (kv0 + TILE > N);
    float s[TILE];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < TILE; ++j) {
      float t = dot_lds(q, Ks + j * 128, d, part) * c;
      if (masked) {
        const int key = kv0 + j;
        if (key >= N || (CAUSAL && key > myq)) t = -INFINITY;
      }
      s[j] = t;
      mx = fmaxf(mx, t);
    }
    const float mn = fmaxf(m, mx);
    const float alpha = exp2_hw(m - mn);
    m = mn;
    l *= alpha;
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
      o[i][0] *= alpha; o[i][1] *= alpha; o[i][2] *= alpha; o[i][3] *= alpha;
    }
#pragma unroll
    for (int j = 0; j < TILE; ++j) {
      const float p = exp2_hw(s[j] - m);
      l += p;
      axpy_lds(o, p, Vs + j * 128, d, part);
    }
    __syncthreads();
  }
  if (myq < N) {
    store_row(O + base + (size_t)myq * d, o, 1.0f / l, d, part);
    if (part == 0) LSE[(size_t)bh * N + myq] = (m + log2_hw(l)) * kLn2;
  }
}

// dK and dV for a block of 64 key rows, looping over tiles of 32 queries.
template <bool CAUSAL>
__global__ void __launch_bounds__(NT)
bwd_dkdv_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
                    const float* __restrict__ LSE, const float* __restrict__ dO,
                    const float* __restrict__ delta, float* __restrict__ dK, float* __restrict__ dV,
                    int N, int d, int nkb, float c, float scale) {
  __shared__ __attribute__((aligned(16))) float Qs[TILE * 128];
  __shared__ __attribute__((aligned(16))) float Gs[TILE * 128];
  __shared__ float lse2[TILE], dl[TILE];
  const int tid = threadIdx.x, part = tid & 3;
  const int bh = blockIdx.x / nkb, kb = blockIdx.x % nkb;
  const int k0 = kb * ROWS, myk = k0 + (tid >> 2);
  const size_t base = (size_t)bh * N * d;
  float k[MAXC][4], v[MAXC][4], dk[MAXC][4], dv[MAXC][4];
  load_row(k, K + base + (size_t)myk * d, d, part, myk < N);
  load_row(v, V + base + (size_t)myk * d, d, part, myk < N);
#pragma unroll
  for (int i = 0; i < MAXC; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) dk[i][e] = dv[i][e] = 0.f;

  // Queries before k0 cannot see any key of this block under the causal mask.
  const int qstart = CAUSAL ? (k0 / TILE) * TILE : 0;
  for (int qt0 = qstart; qt0 < N; qt0 += TILE) {
    stage_rows(Qs, Q + base, qt0, N, d, tid);
    stage_rows(Gs, dO + base, qt0, N, d, tid);
    if (tid < TILE) {
      const int qi = qt0 + tid;
      lse2[tid] = qi < N ? LSE[(size_t)bh * N + qi] * kLog2e : INFINITY;
      dl[tid] = qi < N ? delta[(size_t)bh * N + qi] : 0.f;
    }
    __syncthreads();
    for (int i = 0; i < TILE; ++i) {
      const int qi = qt0 + i;
      const float s = dot_lds(k, Qs + i * 128, d, part);
      float p = exp2_hw(__builtin_fmaf(s, c, -lse2[i]));
      if (qi >= N || myk >= N || (CAUSAL && myk > qi)) p = 0.f;
      axpy_lds(dv, p, Gs + i * 128, d, part);
      const float dp = dot_lds(v, Gs + i * 128, d, part);
      const float ds = p * (dp - dl[i]);
      axpy_lds(dk, ds, Qs + i * 128, d, part);
    }
    __syncthreads();
  }
  if (myk < N) {
    store_row(dK + base + (size_t)myk * d, dk, scale, d, part);
    store_row(dV + base + (size_t)myk * d, dv, 1.0f, d, part);
  }
}

// dQ for a block of 64 query rows, looping over tiles of 32 keys.
template <bool CAUSAL>
__global__ void __launch_bounds__(NT)
bwd_dq_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
                  const float* __restrict__ LSE, const float* __restrict__ dO,
                  const float* __restrict__ delta, float* __restrict__ dQ, int N, int d, int nqb,
                  float c, float scale) {
  __shared__ __attribute__((aligned(16))) float Ks[TILE * 128];
  __shared__ __attribute__((aligned(16))) float Vs[TILE * 128];
  const int tid = threadIdx.x, part = tid & 3;
  const int bh = blockIdx.x / nqb, qb = blockIdx.x % nqb;
  const int q0 = qb * ROWS, myq = q0 + (tid >> 2);
  const size_t base = (size_t)bh * N * d;
  float q[MAXC][4], g[MAXC][4], dq[MAXC][4];
  load_row(q, Q + base + (size_t)myq * d, d, part, myq < N);
  load_row(g, dO + base + (size_t)myq * d, d, part, myq < N);
#pragma unroll
  for (int i = 0; i < MAXC; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) dq[i][e] = 0.f;
  const float lse2 = myq < N ? LSE[(size_t)bh * N + myq] * kLog2e : INFINITY;
  const float dl = myq < N ? delta[(size_t)bh * N + myq] : 0.f;

  const int kv_end = CAUSAL ? min(N, q0 + ROWS) : N;
  for (int kv0 = 0; kv0 < kv_end; kv0 += TILE) {
    stage_rows(Ks, K + base, kv0, N, d, tid);
    stage_rows(Vs, V + base, kv0, N, d, tid);
    __syncthreads();
    for (int j = 0; j < TILE; ++j) {
      const int key = kv0 + j;
      const float s = dot_lds(q, Ks + j * 128, d, part);
      float p = exp2_hw(__builtin_fmaf(s, c, -lse2));
      if (key >= N || myq >= N || (CAUSAL && key > myq)) p = 0.f;
      const float dp = dot_lds(g, Vs + j * 128, d, part);
      axpy_lds(dq, p * (dp - dl), Ks + j * 128, d, part);
    }
    __syncthreads();
  }
  if (myq < N) store_row(dQ + base + (size_t)myq * d, dq, scale, d, part);
}

// delta: 16 threads per row, each summing 16-byte chunks part, part+16, ...
// NEG stores -delta.  (float32 rows; bf16 rows use rowdot_bf16_kernel.)
template <typename T, bool NEG>
__global__ void __launch_bounds__(NT)
rowdot_kernel(const T* __restrict__ O, const T* __restrict__ G, float* __restrict__ delta,
              long long rows, int d) {
  static_assert(sizeof(T) == 4, "float32 rows");
  constexpr int EPC = 16 / sizeof(T);  // elements per 16-byte chunk
  const long long row = (long long)blockIdx.x * (NT / 16) + (threadIdx.x >> 4);
  const int part = threadIdx.x & 15;
  float acc = 0.f;
  if (row < rows) {
    const T* o = O + row * d;
    const T* g = G + row * d;
    for (int col = part * EPC; col < d; col += 16 * EPC) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(o + col);
      const u32x4 b = *reinterpret_cast<const u32x4*>(g + col);
#pragma unroll
      for (int w = 0; w < 4; ++w)
        acc = __builtin_fmaf(__uint_as_float(word_of(a, w)), __uint_as_float(word_of(b, w)), acc);
    }
  }
  acc += __shfl_xor(acc, 8);
  acc += __shfl_xor(acc, 4);
  acc += __shfl_xor(acc, 2);
  acc += __shfl_xor(acc, 1);
  if (row < rows && part == 0) delta[row] = NEG ? -acc : acc;
}

// bf16 delta (negated when NEG) in the order the dQ kernel uses for its own
// queries: per row, two halves (columns 16 k + 8 h .. + 7, h = 0, 1), each
// summed as one FMA chain in column order, then added.  One wave per 32
// rows: the rows are copied to LDS with consecutive lanes on consecutive
// 16-byte chunks, then lane 2 r + h sums half h of row r.
constexpr int RD_ROWS = 32;
template <bool NEG>
__global__ void __launch_bounds__(64)
rowdot_bf16_kernel(const uint16_t* __restrict__ O, const uint16_t* __restrict__ G, float* __restrict__ delta,
                   long long rows, int d) {
  __shared__ __attribute__((aligned(16))) uint16_t so[RD_ROWS * 128], sg[RD_ROWS * 128];
  const long long r0 = (long long)blockIdx.x * RD_ROWS;
  const int lane = threadIdx.x;
  const int cpr = d / 8;   // 16-byte chunks per row
  for (int ch = lane; ch < RD_ROWS * cpr; ch += 64) {
    const long long row = r0 + ch / cpr;
    u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
    if (row < rows) {
      a = *reinterpret_cast<const u32x4*>(O + row * d + (ch % cpr) * 8);
      b = *reinterpret_cast<const u32x4*>(G + row * d + (ch % cpr) * 8);
    }
    *reinterpret_cast<u32x4*>(so + ch * 8) = a;
    *reinterpret_cast<u32x4*>(sg + ch * 8) = b;
  }
  __syncthreads();
  const int rl = lane >> 1, h = lane & 1;
  float acc = 0.f;
  for (int k = 0; k < d / 16; ++k) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(so + rl * d + 16 * k + 8 * h);
    const u32x4 b = *reinterpret_cast<const u32x4*>(sg + rl * d + 16 * k + 8 * h);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t x = word_of(a, w), y = word_of(b, w);
      acc = __builtin_fmaf(bf16_lo(x), bf16_lo(y), acc);
      acc = __builtin_fmaf(bf16_hi(x), bf16_hi(y), acc);
    }
  }
  const float tot = acc + __shfl_xor(acc, 1);
  const long long row = r0 + rl;
  if (row < rows && h == 0) delta[row] = NEG ? -tot : tot;
}

template <typename T, bool NEG>
hipError_t launch_rowdot(const T* o, const T* g, float* delta, long long rows, int d, hipStream_t s) {
  const long long blocks = (rows + (NT / 16) - 1) / (NT / 16);
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((rowdot_kernel<T, NEG>), dim3((unsigned)blocks), dim3(NT), 0, s, o, g, delta, rows, d);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rowdot_bf16(const uint16_t* o, const uint16_t* dO, float* delta, long long rows,
                              int d, hipStream_t stream) {
  if (d % 16 != 0 || d > 128) return hipErrorInvalidValue;
  const long long blocks = (rows + RD_ROWS - 1) / RD_ROWS;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((rowdot_bf16_kernel<true>), dim3((unsigned)blocks), dim3(64), 0, stream, o, dO, delta, rows, d);
  return hipGetLastError();
}

hipError_t launch_rowdot_f32(const float* o, const float* dO, float* delta, long long rows, int d,
                             hipStream_t stream) {
  return launch_rowdot<float, false>(o, dO, delta, rows, d, stream);
}

hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                          int BH, int N, int d, bool causal, float scale, hipStream_t stream) {
  const int nqb = (N + ROWS - 1) / ROWS;
  const long long blocks = (long long)BH * nqb;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  const float c = scale * kLog2e;
  if (causal)
    hipLaunchKernelGGL(fwd_f32_kernel<true>, dim3((unsigned)blocks), dim3(NT), 0, stream, q, k, v, o,
                       lse, N, d, nqb, c);
  else
    hipLaunchKernelGGL(fwd_f32_kernel<false>, dim3((unsigned)blocks), dim3(NT), 0, stream, q, k, v, o,
                       lse, N, d, nqb, c);
  return hipGetLastError();
}

hipError_t launch_bwd_f32(const float* q, const float* k, const float* v, const float* o,
                          const float* lse, const float* dO, float* dq, float* dk, float* dv,
                          int BH, int N, int d, bool causal, float scale, float* delta,
                          hipStream_t stream) {
  const int nb = (N + ROWS - 1) / ROWS;
  const long long blocks = (long long)BH * nb;
  // checked before the row-dot pass is launched, so a refused problem
  // launches nothing
  if (blocks > 0x7fffffffLL || ((long long)BH * N + (NT / 16) - 1) / (NT / 16) > 0x7fffffffLL)
    return hipErrorInvalidValue;
  hipError_t e = launch_rowdot_f32(o, dO, delta, (long long)BH * N, d, stream);
  if (e != hipSuccess) return e;
  const float c = scale * kLog2e;
  if (causal) {
    hipLaunchKernelGGL(bwd_dkdv_f32_kernel<true>, dim3((unsigned)blocks), dim3(NT), 0, stream, q, k, v,
                       lse, dO, delta, dk, dv, N, d, nb, c, scale);
    hipLaunchKernelGGL(bwd_dq_f32_kernel<true>, dim3((unsigned)blocks), dim3(NT), 0, stream, q, k, v,
                       lse, dO, delta, dq, N, d, nb, c, scale);
  } else {
    hipLaunchKernelGGL(bwd_dkdv_f32_kernel<false>, dim3((unsigned)blocks), dim3(NT), 0, stream, q, k, v,
                       lse, dO, delta, dk, dv, N, d, nb, c, scale);
    hipLaunchKernelGGL(bwd_dq_f32_kernel<false>, dim3((unsigned)blocks), dim3(NT), 0, stream, q, k, v,
                       lse, dO, delta, dq, N, d, nb, c, scale);
  }
  return hipGetLastError();
}

}  // namespace fa
