// Decode-phase attention: a few new queries (1 <= nq <= 8) per (batch, head)
// over a long key/value cache of Nk rows, bf16 in/out, float32 arithmetic.
//
// With so few queries the work is a matrix-vector product per key: every key
// and value byte is read once and used for at most 2*nq multiply-adds, so the
// bound is HBM bandwidth, not the matrix cores.  The kernels therefore stream
// K and V with wide coalesced loads into the vector ALUs:
//
//  * split kernel: the keys of each (batch, head) are cut into chunks
//    (split-KV), one wavefront per chunk, so that B*H*chunks wavefronts fill
//    the chip even for B*H = 1.  Within a wavefront, a wave-wide 16-byte-per-
//    lane load covers 1024 contiguous bytes = 64/LPK whole keys (LPK = d/8
//    lanes per key).  Each lane keeps its own running max / sum / output for
//    its key slot (online softmax per slot); the slots are merged once at the
//    end of the chunk.  The chunk's partial (max, sum, unnormalised output)
//    goes to the workspace.
//  * merge kernel: combines the chunk partials of each query through their
//    maxima and sums (the same rescaling the online softmax uses between
//    tiles) and writes O and LSE.
//
// Scores live in the base-2 domain: x = scale*log2(e) * q.k, p = 2^(x - m).
#include "fa_common.h"
#include "launch.h"

namespace fa {
namespace {

constexpr int DEC_NT = 256;             // 4 wavefronts, each its own chunk
constexpr int DEC_WAVES = DEC_NT / 64;

// 16-byte buffer load with the non-temporal hint (`nt`): every K and V byte
// is read exactly once, so the caches need not keep it.  Measured on the
// B=8 H=16 Nk=16384 d=128 decode: 5.6 -> 6.3 TB/s; 3-17% on every decode
// shape tried.
__device__ __forceinline__ u32x4 buf_load16_stream(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  constexpr int kNonTemporal = 2;
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, kNonTemporal);
}

// a.lo*b.lo + a.hi*b.hi + acc for two bf16 pairs (v_dot2c_f32_bf16).
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), acc,
                                         false);
}

template <int D, int NQ, int U, bool CAUSAL>
struct DecodeState {
  static constexpr int LPK = D / 8;     // lanes per key (8 bf16 per lane)
  static constexpr int KPI = 64 / LPK;  // keys per wave-wide load
  static constexpr int UK = U * KPI;    // keys per step
};

// One step: UK keys starting at kb.  MASK hides keys >= k1 and, when causal,
// keys past each query's position.
template <int D, int NQ, int U, bool CAUSAL, bool MASK>
__device__ __forceinline__ void decode_step(__amdgpu_buffer_rsrc_t krs, __amdgpu_buffer_rsrc_t vrs, const u32x4* qv,
                                            float* m, float* l, f32x4 (*o)[2], int kb, int slot, int cc,
                                            int k1, int last_visible0, float c) {
  using S = DecodeState<D, NQ, U, CAUSAL>;
  u32x4 kr[U], vr[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t off = (uint32_t)(((kb + u * S::KPI + slot) * D + 8 * cc) * 2);
    kr[u] = buf_load16_stream(krs, off);
    vr[u] = buf_load16_stream(vrs, off);
  }
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    float s[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float a = dot2(qv[i][0], kr[u][0], 0.f);
      a = dot2(qv[i][1], kr[u][1], a);
      a = dot2(qv[i][2], kr[u][2], a);
      a = dot2(qv[i][3], kr[u][3], a);
      s[u] = group_sum<S::LPK>(a);
      if (MASK) {
        const int key = kb + u * S::KPI + slot;
        if (key >= k1 || (CAUSAL && key > last_visible0 + i)) s[u] = -INFINITY;
      }
    }
    float mx = s[0];
#pragma unroll
    for (int u = 1; u < U; ++u) mx = max_nan(mx, s[u]);
    const float mn = max_nan(m[i], mx * c);
    const float alpha = mn == m[i] ? 1.f : exp2_hw(m[i] - mn);
    const float mref = mn == -INFINITY ? 0.f : mn;
    m[i] = mn;
    float lsum = l[i] * alpha;
    f32x4 o0 = o[i][0] * alpha, o1 = o[i][1] * alpha;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float p = exp2_hw(__builtin_fmaf(s[u], c, -mref));
      lsum += p;
      o0 += p * f32x4{bf16_lo(vr[u][0]), bf16_hi(vr[u][0]), bf16_lo(vr[u][1]), bf16_hi(vr[u][1])};
      o1 += p * f32x4{bf16_lo(vr[u][2]), bf16_hi(vr[u][2]), bf16_lo(vr[u][3]), bf16_hi(vr[u][3])};
    }
    l[i] = lsum;
    o[i][0] = o0;
    o[i][1] = o1;
  }
}

// part_o:  [BH][nsplit][nq][D] float32, the chunk's output before division
//          by its sum, relative to its max;
// part_ml: [BH][nsplit][nq][2] float32, the chunk's (max, sum) in the base-2
//          domain (max = -inf and sum = 0 when no key of the chunk is visible).
template <int D, int NQ, int U, bool CAUSAL>
__global__ void __launch_bounds__(DEC_NT)
decode_split_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                    const uint16_t* __restrict__ V, float* __restrict__ part_o,
                    float* __restrict__ part_ml, int nq, int Nk, int chunk, int nsplit, int units,
                    float c) {
  using S = DecodeState<D, NQ, U, CAUSAL>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int unit = blockIdx.x * DEC_WAVES + wave;
  if (unit >= units) return;
  const int bh = unit / nsplit, split = unit - bh * nsplit;
  const int slot = lane / S::LPK, cc = lane % S::LPK;
  const int k0 = split * chunk, k1 = min(Nk, k0 + chunk);
  // Query i sits at position Nk - nq + i; causal, it sees keys <= that.
  const int last_visible0 = Nk - nq;

  const size_t kv_base = (size_t)bh * Nk * D;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(K + kv_base, (uint32_t)Nk * D * 2);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(V + kv_base, (uint32_t)Nk * D * 2);
  const __amdgpu_buffer_rsrc_t qrs = make_rsrc(Q + (size_t)bh * nq * D, (uint32_t)nq * D * 2);

  u32x4 qv[NQ];  // query slots past nq read as zero and are never stored
#pragma unroll
  for (int i = 0; i < NQ; ++i) qv[i] = buf_load16(qrs, (uint32_t)((i * D + 8 * cc) * 2));

  float m[NQ], l[NQ];
  f32x4 o[NQ][2];
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    m[i] = -INFINITY;
    l[i] = 0.f;
    o[i][0] = f32x4{};
    o[i][1] = f32x4{};
  }

  // Keys below `clean` are visible to every query of this chunk.
  const int clean = CAUSAL ? min(k1, last_visible0 + 1) : k1;
  int kb = k0;
  for (; kb + S::UK <= clean; kb += S::UK)
    decode_step<D, NQ, U, CAUSAL, false>(krs, vrs, qv, m, l, o, kb, slot, cc, k1, last_visible0, c);
  for (; kb < k1; kb += S::UK)
    decode_step<D, NQ, U, CAUSAL, true>(krs, vrs, qv, m, l, o, kb, slot, cc, k1, last_visible0, c);

  // Merge the KPI key slots of the wavefront (lanes LPK apart).
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    if (i >= nq) break;
    float M = m[i];
#pragma unroll
    for (int sh = S::LPK; sh < 64; sh <<= 1) M = max_nan(M, __shfl_xor(M, sh));
    const float f = m[i] == -INFINITY ? 0.f : exp2_hw(m[i] - M);
    float L = l[i] * f;
    f32x4 o0 = o[i][0] * f, o1 = o[i][1] * f;
#pragma unroll
    for (int sh = S::LPK; sh < 64; sh <<= 1) {
      L += __shfl_xor(L, sh);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o0[e] += __shfl_xor(o0[e], sh);
        o1[e] += __shfl_xor(o1[e], sh);
      }
    }
    const size_t row = (size_t)unit * nq + i;
    if (slot == 0) {
      f32x4* dst = reinterpret_cast<f32x4*>(part_o + row * D + 8 * cc);
      dst[0] = o0;
      dst[1] = o1;
    }
    if (lane == 0) *reinterpret_cast<f32x2*>(part_ml + row * 2) = f32x2{M, L};
  }
}

// One thread per (row, column pair); row = bh * nq + i.
template <int D>
__global__ void __launch_bounds__(256)
decode_merge_kernel(const float* __restrict__ part_o, const float* __restrict__ part_ml,
                    uint16_t* __restrict__ O, float* __restrict__ LSE, int nq, int nsplit, int rows) {
  constexpr int TPR = D / 2;  // threads per row
  const int row = blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
  if (row >= rows) return;
  const int c2 = 2 * (threadIdx.x % TPR);
  const int bh = row / nq, i = row - bh * nq;
  const size_t first = (size_t)bh * nsplit * nq + i;  // partial of split s: first + s * nq
  float M = -INFINITY;
  for (int s = 0; s < nsplit; ++s) M = max_nan(M, part_ml[(first + (size_t)s * nq) * 2]);
  float L = 0.f, a0 = 0.f, a1 = 0.f;
  if (M != -INFINITY) {
    for (int s = 0; s < nsplit; ++s) {
      const size_t p = first + (size_t)s * nq;
      const f32x2 ml = *reinterpret_cast<const f32x2*>(part_ml + p * 2);
      const float f = exp2_hw(ml[0] - M);  // 0 for a chunk with no visible key
      const f32x2 ov = *reinterpret_cast<const f32x2*>(part_o + p * D + c2);
      L += ml[1] * f;
      a0 += ov[0] * f;
      a1 += ov[1] * f;
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  *reinterpret_cast<uint32_t*>(O + (size_t)row * D + c2) = pack_bf16x2(a0 * inv, a1 * inv);
  if (c2 == 0) LSE[row] = L > 0.f ? (M + log2_hw(L)) * kLn2 : -INFINITY;
}

template <int D, int NQ, bool CAUSAL>
hipError_t launch_split(const uint16_t* q, const uint16_t* k, const uint16_t* v, float* po, float* pml, int BH,
                        int nq, int Nk, int chunk, int nsplit, float scale, hipStream_t stream) {
  constexpr int U = NQ <= 2 ? 16 : NQ <= 4 ? 8 : 4;  // wave-wide loads per step (register budget)
  const long long units = (long long)BH * nsplit;
  const unsigned blocks = (unsigned)((units + DEC_WAVES - 1) / DEC_WAVES);
  hipLaunchKernelGGL((decode_split_kernel<D, NQ, U, CAUSAL>), dim3(blocks), dim3(DEC_NT), 0, stream, q, k, v,
                     po, pml, nq, Nk, chunk, nsplit, (int)units, score_coef(scale));
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_split_nq(const uint16_t* q, const uint16_t* k, const uint16_t* v, float* po, float* pml,
                           int BH, int nq, int Nk, int chunk, int nsplit, float scale, hipStream_t s) {
  if (nq <= 1) return launch_split<D, 1, CAUSAL>(q, k, v, po, pml, BH, nq, Nk, chunk, nsplit, scale, s);
  if (nq <= 2) return launch_split<D, 2, CAUSAL>(q, k, v, po, pml, BH, nq, Nk, chunk, nsplit, scale, s);
  if (nq <= 4) return launch_split<D, 4, CAUSAL>(q, k, v, po, pml, BH, nq, Nk, chunk, nsplit, scale, s);
  return launch_split<D, 8, CAUSAL>(q, k, v, po, pml, BH, nq, Nk, chunk, nsplit, scale, s);
}

}  // namespace

DecodeSplit decode_split(long long BH, int nq, int Nk, int d) {
  // Keys per chunk: a multiple of 64 (a whole number of steps for every
  // instantiation) sized for a number of chunk wavefronts that all stay
  // resident, each streaming one long contiguous range: 1024 (one per SIMD)
  // for one query, 2048 for two, 3072 for three or four, 2048 for five to
  // eight.  Measured on MI355X, fewer longer streams beat more shorter ones
  // (16k chunks of 128 keys ran 25% slower on the B=8 H=16 Nk=16384 d=128
  // decode), and even one (batch, head) still fills the 256 compute units.
  // With one query a wave keeps 32 loads in flight and does little
  // arithmetic per key, so one wave per SIMD streams fastest (+4-13%); more
  // queries need more waves to overlap their arithmetic (1024 chunks ran
  // 25% slower at nq = 2; 3072 ran 14-15% faster than 2048 at nq = 3-4 and
  // 4-7% slower at nq = 6-8).
  DecodeSplit r;
  const long long target = nq == 1 ? 1024 : nq <= 2 ? 2048 : nq <= 4 ? 3072 : 2048;
  long long chunk = (BH * (long long)Nk + target - 1) / target;
  chunk = (chunk + 63) / 64 * 64;
  if (chunk < 64) chunk = 64;
  if (chunk > Nk) chunk = (Nk + 63) / 64 * 64;
  r.chunk = (int)chunk;
  r.nsplit = (int)((Nk + chunk - 1) / chunk);
  const size_t parts = (size_t)BH * r.nsplit * nq;
  r.o_bytes = (parts * d * sizeof(float) + 255) & ~(size_t)255;
  r.bytes = r.o_bytes + ((parts * 2 * sizeof(float) + 255) & ~(size_t)255);
  return r;
}

hipError_t launch_decode_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, float* lse,
                              int BH, int nq, int Nk, int d, bool causal, float scale, void* workspace,
                              hipStream_t stream) {
  if (nq < 1 || nq > 8 || (d != 64 && d != 128)) return hipErrorInvalidValue;
  // Buffer offsets are 32-bit: one head of K or V must stay below 2 GiB.
  if ((long long)Nk * d * 2 >= (1LL << 31)) return hipErrorInvalidValue;
  const DecodeSplit sp = decode_split(BH, nq, Nk, d);
  if ((long long)BH * sp.nsplit > 0x7fffffffLL - DEC_WAVES) return hipErrorInvalidValue;
  float* po = static_cast<float*>(workspace);
  float* pml = reinterpret_cast<float*>(static_cast<char*>(workspace) + sp.o_bytes);
  hipError_t e;
  if (d == 64)
    e = causal ? launch_split_nq<64, true>(q, k, v, po, pml, BH, nq, Nk, sp.chunk, sp.nsplit, scale, stream)
               : launch_split_nq<64, false>(q, k, v, po, pml, BH, nq, Nk, sp.chunk, sp.nsplit, scale, stream);
  else
    e = causal ? launch_split_nq<128, true>(q, k, v, po, pml, BH, nq, Nk, sp.chunk, sp.nsplit, scale, stream)
               : launch_split_nq<128, false>(q, k, v, po, pml, BH, nq, Nk, sp.chunk, sp.nsplit, scale, stream);
  if (e != hipSuccess) return e;
  const int rows = BH * nq;
  const int rpb = 256 / (d / 2);
  const unsigned blocks = (unsigned)((rows + rpb - 1) / rpb);
  if (d == 64)
    hipLaunchKernelGGL((decode_merge_kernel<64>), dim3(blocks), dim3(256), 0, stream, po, pml, o, lse, nq,
                       sp.nsplit, rows);
  else
    hipLaunchKernelGGL((decode_merge_kernel<128>), dim3(blocks), dim3(256), 0, stream, po, pml, o, lse, nq,
                       sp.nsplit, rows);
  return hipGetLastError();
}

}  // namespace fa
