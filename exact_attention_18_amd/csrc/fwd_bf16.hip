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
//    is fetched by direct HBM-to-LDS loads while tile j is computed (the
//    two-group kernel below does the same with 128-key tiles);
//  * S^T = K Q^T and O^T += V^T P^T on the bf16 matrix cores.  Computing the
//    transposed products puts one query per lane (two lanes per query), so
//    the row max, the row sum and the output rescale are per-lane values.
//    K and V sit in LDS row-major; the V^T operand comes from the LDS
//    transpose read;
//  * online softmax in the base-2 domain: scale*log2(e) is folded into one
//    multiply-add before v_exp_f32; the running max is only raised when a
//    tile's max exceeds it by more than 8 (log2 units; the numerator and
//    denominator share the reference, so the result is unchanged), which the
//    tile's exponentials themselves reveal (some p > 2^8), so the row max is
//    only computed in the rare tiles that need it; 1/l is applied once, in
//    the epilogue;
//  * causal: tiles above the diagonal are never loaded; the mask code runs
//    only on tiles that straddle the diagonal or the ragged end of N.
#include <type_traits>

#include "fa_common.h"
#include "launch.h"

namespace fa {
namespace {

constexpr int BR = 128;       // queries per workgroup
constexpr int BC = 64;        // keys per tile
constexpr int NT = 256;       // threads per workgroup (4 waves)
constexpr float TAU = 8.0f;   // lazy-rescale threshold, log2 units
constexpr float PMAX = 256.f;  // 2^TAU

// Row padding (elements) of the K and V tiles in LDS; tuning knobs.
#ifndef FA_FWD_KPAD
#define FA_FWD_KPAD 8
#endif
#ifndef FA_FWD_VPAD
#define FA_FWD_VPAD 32
#endif

template <int D>
struct Lds {
  // K rows are read 16 bytes per lane from 32 consecutive rows: a row stride
  // of D+8 elements spreads 16 consecutive rows over all 64 banks.  V rows
  // are read with the transpose read: two 16-lane groups each take 4
  // consecutive rows x 32 bytes; a row stride of D+32 elements (64 bytes
  // past a multiple of 256) puts those 8 segments on disjoint banks.
  static constexpr int KS = D + FA_FWD_KPAD;
  static constexpr int VS = D + FA_FWD_VPAD;
  static constexpr int K_ELEMS = BC * KS;
  static constexpr int STAGE = K_ELEMS + BC * VS;
  static constexpr int ELEMS = 2 * STAGE;              // double buffer
  // direct loads of 64 x 16 bytes fill a tile's padded rows in order
  static constexpr int KCPR = KS / 8, VCPR = VS / 8;   // chunks per padded row
  static constexpr int KLOADS = BC * KCPR / 64, VLOADS = BC * VCPR / 64;
  static_assert(KLOADS * 64 == BC * KCPR && VLOADS * 64 == BC * VCPR, "tiles must be whole loads");
};

// A K tile and a V tile of 64 rows by direct HBM -> LDS loads, shared out
// over NW waves: load j (K loads first, then V) is issued by wave j % NW, and
// lane l of a load fills 16-byte chunk 64 (its index within the tile) + l of
// the tile's padded rows.  Lanes on a row's padding get an offset past the
// buffer (zeros); rows at or past N read as zero as well.
template <int D, int NW>
struct TileDma {
  using L = Lds<D>;
  static constexpr int NL = L::KLOADS + L::VLOADS, PW = (NL + NW - 1) / NW;
  uint32_t voff[PW];
  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int u = 0; u < PW; ++u) {
      const int j = wave + NW * u;
      const bool isv = j >= L::KLOADS;
      const int cpr = isv ? L::VCPR : L::KCPR;
      const int p = 64 * (isv ? j - L::KLOADS : j) + lane, row = p / cpr, col = p % cpr;
      voff[u] = col < D / 8 ? (uint32_t)(row * D + col * 8) * 2 : 0x80000000u;
    }
  }
  // Tile starting at key kv0 into the stage at dst (K, then V at K_ELEMS).
  __device__ __forceinline__ void issue(const RowSrc<D>& ks, const RowSrc<D>& vs, int kv0, uint16_t* dst,
                                        int wave) const {
    const __amdgpu_buffer_rsrc_t kr = ks.from_row(kv0), vr = vs.from_row(kv0);
#pragma unroll
    for (int u = 0; u < PW; ++u) {
      const int j = wave + NW * u;
      if (j < L::KLOADS)
        lds_load16(kr, dst + j * 512, voff[u]);
      else if (j < NL)
        lds_load16(vr, dst + L::K_ELEMS + (j - L::KLOADS) * 512, voff[u]);
    }
  }
};

// Online-softmax bookkeeping for one wave's 64-key tile of S^T (element r of
// s[kb] is key 32*kb + 8*(r/4) + 4*g + r%4): optional mask (keys past `lim`
// get -inf), row max, and the lazy rescale of the reference max m, the row
// sum and the output accumulators.  FIRST: the wave's first tile, where m is
// still -inf and the row sum and accumulators are still zero, so the rescale
// by alpha = 2^-inf = 0 would leave them unchanged and is skipped.
template <int D, bool MASK, int NKB = 2, bool FIRST = false>
__device__ __forceinline__ void softmax_update(f32x16 (&s)[NKB], f32x16 (&oacc)[D / 32], float& m, float& lsum,
                                               float c, int lim) {
  if (MASK) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (kb * 32 + 8 * (r >> 2) + (r & 3) > lim) s[kb][r] = -INFINITY;
  }
  // Row max as a shallow tree (v_max3), not a 32-long dependent chain.
  // max_nan (NaN-propagating maximum) lowers to v_maximum3_f32 without the
  // operand canonicalisation that fmaxf needs in IEEE mode.
  float m8[2 * NKB];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = 8 * h;
      const float a = max_nan(max_nan(s[kb][r], s[kb][r + 1]), s[kb][r + 2]);
      const float b = max_nan(max_nan(s[kb][r + 3], s[kb][r + 4]), s[kb][r + 5]);
      m8[2 * kb + h] = max_nan(max_nan(a, b), max_nan(s[kb][r + 6], s[kb][r + 7]));
    }
  float mx = max_nan(max_nan(m8[0], m8[1]), max_nan(m8[2], m8[3]));
#pragma unroll
  for (int i = 4; i < 2 * NKB; i += 2) mx = max_nan(mx, max_nan(m8[i], m8[i + 1]));
  mx = max_halves(mx) * c;  // c > 0: the scaled row max over the tile (or -inf)

  // Raise the reference max only when some row's tile max exceeds it by
  // more than TAU; otherwise p stays below 2^TAU and nothing is rescaled.
  if (__any(mx > m + TAU)) {
    const float mn = fmaxf(m, mx);
    if constexpr (!FIRST) {
      const float alpha = exp2_hw(m - mn);
      lsum *= alpha;
#pragma unroll
      for (int i = 0; i < D / 32; ++i) oacc[i] *= alpha;
    }
    m = mn;
  }
}

// P = exp2(c s - m) for one wave's 64-key tile, packed to bf16 into pw
// (block b = 2 kb + t holds keys 32 kb + 16 t + ...), added to the row sum,
// with the lazy rescale of m.  Fast path: P with the current reference max.
// It stands when no p exceeds 2^TAU, which each block sum (at least its
// largest p) shows without a row max, and that is exactly when the lazy rule
// keeps m.  Otherwise (also while m is still -inf, which gives inf or NaN)
// the tile takes softmax_update and P is recomputed with the new m, as if
// the fast path had not run.  Sums are added in the same order either way.
// FIRST (the wave's first tile, m still -inf, where the fast path always
// fails): straight to softmax_update, with the same arithmetic and bits.
template <int D, bool MASK, int NKB = 2, bool FIRST = false>
__device__ __forceinline__ void softmax_probs(f32x16 (&s)[NKB], u32x4 (&pw)[2 * NKB], f32x16 (&oacc)[D / 32],
                                              float& m, float& lsum, float c, int lim) {
  if (MASK) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (kb * 32 + 8 * (r >> 2) + (r & 3) > lim) s[kb][r] = -INFINITY;
  }
  auto probs = [&](float& l) {
    float bmax = 0.f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        float ps[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 8 * t + 2 * e;
          const float p0 = exp2_hw(__builtin_fmaf(s[kb][r], c, -m));
          const float p1 = exp2_hw(__builtin_fmaf(s[kb][r + 1], c, -m));
          ps[e] = p0 + p1;
          pw[2 * kb + t][e] = pack_bf16x2(p0, p1);
        }
        const float bs = (ps[0] + ps[1]) + (ps[2] + ps[3]);
        l += bs;
        bmax = max_nan(bmax, bs);
      }
    return bmax;
  };
  float l = lsum;
  if constexpr (FIRST) {
    softmax_update<D, false, NKB, true>(s, oacc, m, lsum, c, 0);
    l = lsum;
    probs(l);
  } else {
    const float bmax = probs(l);
    if (__any(!(bmax <= PMAX))) {
      softmax_update<D, false, NKB>(s, oacc, m, lsum, c, 0);
      l = lsum;
      probs(l);
    }
  }
  lsum = l;
}

// One 64-key tile for one wave: S^T = K Q^T, (mask), online softmax update,
// O^T += V^T P^T.  MASK selects the variant for tiles that straddle the
// diagonal or the end of N; `lim` is the largest visible key offset within
// the tile for this lane's query, minus 4*g.  FIRST: the wave's first tile.
template <int D, bool MASK, bool FIRST = false>
__device__ __forceinline__ void tile_step(const uint16_t* Ks, const uint16_t* Vs, const bf16x8 (&qf)[D / 16],
                                          f32x16 (&oacc)[D / 32], float& m, float& lsum, float c, int lim,
                                          int lane) {
  using L = Lds<D>;
  constexpr int KSTEPS = D / 16, DB = D / 32;
  const int l32 = lane & 31, g = lane >> 5;

  // S^T tile: s[kb] element r is key 32*kb + 8*(r/4) + 4*g + r%4 of the tile.
  // The two 32-key blocks are independent chains; alternating them keeps
  // consecutive matrix-core instructions independent.
  f32x16 s[2];
  const uint16_t* krow = Ks + l32 * L::KS + 8 * g;
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const bf16x8 a = bf16x8_from(*reinterpret_cast<const u32x4*>(krow + kb * 32 * L::KS + ks * 16));
      s[kb] = mfma32(a, qf[ks], ks == 0 ? f32x16{} : s[kb]);
    }
  // Scheduling: up to 16 K-operand LDS reads (mask 0x100) in flight ahead of
  // the matrix-core instructions (mask 0x008), then alternate 2 and 2 (at
  // d = 128 all 16 reads go first: the direct tile loads left the registers
  // for it, measured 3% faster than 8 ahead).
  constexpr int NQK = 2 * KSTEPS, AHEAD = NQK < 16 ? NQK : 16;
  __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);
#pragma unroll
  for (int i = 0; i < (NQK - AHEAD) / 2; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, AHEAD, 0);

  u32x4 pw[4];
  softmax_probs<D, MASK, 2, FIRST>(s, pw, oacc, m, lsum, c, lim);

  const int tr_row = 4 * g + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const bf16x8 pb = __builtin_bit_cast(bf16x8, pw[2 * kb + t]);
      const uint16_t* vp = Vs + (kb * 32 + 16 * t + tr_row) * L::VS + tr_col;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const bf16x8 a = bf16x8_from(lds_read_tr16(vp + db * 32), lds_read_tr16(vp + 8 * L::VS + db * 32));
        oacc[db] = mfma32(a, pb, oacc[db]);
      }
    }
}

// tile_step on the stage at (Ks, Vs), with the direct loads of the next
// tile into the other stage (next) issued first.  The three stages are
// disjoint; passing them as restrict pointers of one inlined function gives
// the LDS accesses alias scopes, so the compiler can tell that the transpose
// reads of this tile do not read what the loads write and does not make
// them wait for the loads.
template <int D, bool MASK, int NW, bool FIRST = false>
__device__ __forceinline__ void tile_step_next(const uint16_t* __restrict__ Ks, const uint16_t* __restrict__ Vs,
                                               uint16_t* __restrict__ next, bool load_next,
                                               const TileDma<D, NW>& dma, const RowSrc<D>& krs,
                                               const RowSrc<D>& vrs, int kv_next, int wave,
                                               const bf16x8 (&qf)[D / 16], f32x16 (&oacc)[D / 32], float& m,
                                               float& lsum, float c, int lim, int lane) {
  if (load_next) dma.issue(krs, vrs, kv_next, next, wave);
  tile_step<D, MASK, FIRST>(Ks, Vs, qf, oacc, m, lsum, c, lim, lane);
}

#ifndef FA_FWD_WAVES_PER_SIMD
#define FA_FWD_WAVES_PER_SIMD 2
#endif
// Waves per SIMD of the one-group forward: at d = 64 a wave needs ~144 VGPRs
// and a workgroup 43 KB of LDS, so three workgroups share a CU (measured
// +14% over two); at d = 128 two.
template <int D>
constexpr int fwd_waves_per_simd() { return D == 64 ? 3 : FA_FWD_WAVES_PER_SIMD; }

// SPARSE: block-sparse variant.  bmask is a [ceil(N/128)][ceil(N/128)] byte
// mask shared by every (batch, head); key block kb is visible to query block
// qb iff bmask[qb][kb] != 0 (128 x 128 blocks, so one mask row per
// workgroup and one mask entry per two 64-key tiles).
template <int D, bool CAUSAL, bool SPARSE>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(fwd_waves_per_simd<D>(), fwd_waves_per_simd<D>())))
fwd_bf16_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
                float* __restrict__ LSE, int N, int nqb, int total, float c,
                const uint8_t* __restrict__ bmask) {
  using L = Lds<D>;
  constexpr int KSTEPS = D / 16, DB = D / 32;
  __shared__ __attribute__((aligned(16))) uint16_t smem[L::ELEMS];

  const int tid = threadIdx.x, lane = tid & 63;
  // wave-uniform, kept in an SGPR; the mask tells the compiler it is below 4,
  // which settles at compile time which tile loads each wave issues
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6) & (NT / 64 - 1);
  const int l32 = lane & 31, g = lane >> 5;
  int bh, qb;
  map_block_xcd(blockIdx.x, total, nqb, CAUSAL, bh, qb);
  const size_t base = (size_t)bh * N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  const RowSrc<D> krs{K + base, head_bytes}, vrs{V + base, head_bytes};
  const __amdgpu_buffer_rsrc_t qrs = make_rsrc(Q + base, head_bytes);
  const int q0 = qb * BR;
  const int qw = q0 + wave * 32;   // first query of this wave
  const int myq = qw + l32;        // query owned by this lane (with its partner lane)

  // Q fragment: lane holds Q[myq][16*ks + 8*g .. +8]; rows past N read as zero.
  bf16x8 qf[KSTEPS];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks)
    qf[ks] = bf16x8_from(buf_load16(qrs, (uint32_t)((myq * D + ks * 16 + 8 * g) * 2)));

  const int kv_end = CAUSAL ? min(N, q0 + BR) : N;
  const int ntiles = (kv_end + BC - 1) / BC;

  f32x16 oacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) oacc[i] = f32x16{};
  float m = -INFINITY;   // reference max of scale*log2e*s for query myq
  float lsum = 0.f;      // this lane's share of the row sum

  TileDma<D, NT / 64> dma;
  dma.init(wave, lane);
  if constexpr (SPARSE) {
    // Visit only the tiles of visible key blocks and prefetch the next
    // visible one.  A key block is two 64-key tiles.  The mask row is read
    // 64 entries at a time into a wave-uniform bit set (one ballot).
    // Every tile a wave visits holds key kv0 <= min(qw, N - 1), visible to
    // all its rows, so m is finite after the wave's first tile; rows of a
    // query block that visits no tile keep l = 0.
    const uint8_t* mrow = bmask + (size_t)qb * nqb;
    int win = -1;
    uint64_t bits = 0;
    auto first_visible_block = [&](int b) {  // smallest visible key block >= b, or nqb
      while (b < nqb) {
        if ((b >> 6) != win) {
          win = b >> 6;
          const int e = 64 * win + lane;
          bits = __ballot(e < nqb && mrow[e] != 0);
        }
        const uint64_t rest = bits >> (b & 63);
        if (rest) return b + (int)__builtin_ctzll(rest);
        b = 64 * (win + 1);
      }
      return nqb;
    };
    int j = 2 * first_visible_block(0);
    if (j < ntiles) dma.issue(krs, vrs, j * BC, smem, wave);
    wait_vmem();
    __syncthreads();
    int slot = 0;
    while (j < ntiles) {
      const int jn = (j & 1) == 0 ? j + 1 : 2 * first_visible_block((j >> 1) + 1);
      const uint16_t* Ks = smem + slot * L::STAGE;
      const uint16_t* Vs = Ks + L::K_ELEMS;
      const int kv0 = j * BC;
      if (!CAUSAL || kv0 <= qw + 31) {
        const int lim = (CAUSAL ? min(myq, N - 1) : N - 1) - kv0 - 4 * g;
        tile_step_next<D, true, NT / 64>(Ks, Vs, smem + (slot ^ 1) * L::STAGE, jn < ntiles, dma, krs, vrs, jn * BC,
                                        wave, qf, oacc, m, lsum, c, lim, lane);
      } else if (jn < ntiles) {
        dma.issue(krs, vrs, jn * BC, smem + (slot ^ 1) * L::STAGE, wave);
      }
      wait_vmem();
      __syncthreads();
      slot ^= 1;
      j = jn;
    }
  } else {
  dma.issue(krs, vrs, 0, smem, wave);
  wait_vmem();
  __syncthreads();

  // Interior tiles (no key of the tile is hidden from any query of the
  // workgroup) run the unmasked step; the remaining tiles (at most two on the
  // causal diagonal, or the ragged last tile) run the masked one.  Two loops
  // rather than a branch per tile keep the accumulators in place.  Tile 0
  // holds key 0, which every query sees, and is the first of every wave: it
  // takes the FIRST step (row max at once, m being still -inf).
  const int n_plain = min(CAUSAL ? q0 / BC : ntiles, N / BC);
  auto step = [&](int j, auto mask_tag, auto first_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    constexpr bool FIRST = decltype(first_tag)::value;
    const uint16_t* Ks = smem + (j & 1) * L::STAGE;
    const uint16_t* Vs = Ks + L::K_ELEMS;
    uint16_t* next = smem + ((j + 1) & 1) * L::STAGE;
    const int kv0 = j * BC;
    if constexpr (MASK) {
      if (!CAUSAL || kv0 <= qw + 31) {
        const int lim = (CAUSAL ? min(myq, N - 1) : N - 1) - kv0 - 4 * g;
        tile_step_next<D, true, NT / 64, FIRST>(Ks, Vs, next, j + 1 < ntiles, dma, krs, vrs, kv0 + BC, wave, qf,
                                               oacc, m, lsum, c, lim, lane);
      } else if (j + 1 < ntiles) {
        dma.issue(krs, vrs, kv0 + BC, next, wave);
      }
    } else {
      tile_step_next<D, false, NT / 64, FIRST>(Ks, Vs, next, j + 1 < ntiles, dma, krs, vrs, kv0 + BC, wave, qf,
                                              oacc, m, lsum, c, 0, lane);
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
  }

  // Epilogue: O = O^T / l, LSE = ln2 * (m + log2 l).
  // A row with no visible key (possible only under a block mask) gets
  // O = 0 and LSE = -inf.
  const float ltot = sum_halves(lsum);
  const float inv = ltot > 0.f ? rcp_hw(ltot) : 0.f;
  if (myq < N) {
    uint16_t* orow = O + base + (size_t)myq * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        u32x2 w = {pack_bf16x2(oacc[db][4 * a] * inv, oacc[db][4 * a + 1] * inv),
                   pack_bf16x2(oacc[db][4 * a + 2] * inv, oacc[db][4 * a + 3] * inv)};
        *reinterpret_cast<u32x2*>(orow + db * 32 + 8 * a + 4 * g) = w;
      }
    if (g == 0) LSE[(size_t)bh * N + myq] = ltot > 0.f ? (m + log2_hw(ltot)) * kLn2 : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// Dense forward, d = 128: two wave groups in alternation.
//
// The page "FlashAttention-3 — FlashAttention-3" (section on overlapping the
// softmax with the matrix products) describes two warpgroups that take turns:
// while one runs its matrix products, the other runs its softmax.  On gfx950
// the same idea maps onto the two waves that share a SIMD.  A workgroup of 8
// waves owns 256 queries; waves w and w+4 run on the same SIMD (the
// dispatcher places the waves of a workgroup on the 4 SIMDs in turn), group 0
// is waves 0-3 and group 1 waves 4-7.  Each wave alternates
//   matrix phase k:  O^T += V(k-1)^T P(k-1)^T and S(k) = K(k) Q^T (128 keys)
//   softmax phase k: mask, row max and lazy rescale on S(k), P(k) = exp2(...)
// and the groups run them one phase apart, with a workgroup barrier between
// phases: in every phase one wave per SIMD keeps the matrix core busy while
// the other wave's softmax runs on the vector ALU.
//
// Phase pair k: group 0 runs matrix phase k then softmax phase k; group 1
// runs softmax phase k-1 then matrix phase k.  Tiles K(k+1) and V(k) are
// loaded straight into LDS during pair k (every wave issues its share at the
// start of the pair and waits for it before the pair's last barrier); their
// slots held K(k-1) and V(k-2), whose last reads were in pair k-1.  The
// barriers are also scheduling fences, so no instruction migrates from one
// phase into the next.
constexpr int PP_BR = 256;              // queries per workgroup
constexpr int PP_NT = 512;              // 8 waves
constexpr int PP_MIN_CAUSAL_N = 2049;   // shorter causal problems use fwd_bf16_kernel

// Workgroup barrier that is also a scheduling fence.
__device__ __forceinline__ void pp_sync() {
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();
  __builtin_amdgcn_sched_barrier(0);
}

// Online softmax over a 128-key tile (four 32-key blocks of S^T, element r
// of s[kb] is key 32 kb + 8 (r/4) + 4 g + r%4), with P written back into the
// registers of S: word e of P block b = 2 kb + t (keys 32 kb + 16 t + ...)
// goes to s[kb][8 t + e].  The row max comes first (so S need not stay live
// beside P); the reference max m is raised only when the tile's max exceeds
// it by more than TAU, as in softmax_update, and the arithmetic per element
// is that of softmax_probs.
template <bool MASK>
__device__ __forceinline__ void softmax_inplace128(f32x16 (&s)[4], f32x16 (&oacc)[4], float& m, float& lsum, float c,
                                                   int lim) {
  softmax_update<128, MASK, 4>(s, oacc, m, lsum, c, lim);
  float l = lsum;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      float ps[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 8 * t + 2 * e;
        const float p0 = exp2_hw(__builtin_fmaf(s[kb][r], c, -m));
        const float p1 = exp2_hw(__builtin_fmaf(s[kb][r + 1], c, -m));
        ps[e] = p0 + p1;
        s[kb][8 * t + e] = __uint_as_float(pack_bf16x2(p0, p1));   // elements 8t+e <= r were read already
      }
      l += (ps[0] + ps[1]) + (ps[2] + ps[3]);
    }
  lsum = l;
}

// Tiles of 128 keys: a matrix phase is 64 products per wave, so the
// per-phase costs (the barrier, the first LDS reads of a phase, the first
// read of the new scores) are paid half as often per product as with 64-key
// tiles.  P(k-1) V(k-1) goes first so that P's registers (which are S's,
// see softmax_inplace128) are free before S(k) is written.
//
// One workgroup per (batch*head, 256-query block), dispatched heaviest
// first when the mask makes the work grow with the block index; when B*H is
// a multiple of 8 the workgroups of each XCD (id % 8) take only the heads h
// with h % 8 equal to their XCD, so a head's K and V are read through one L2.
constexpr int PP_BK = 128;   // keys per tile

struct PpLds {
  static constexpr int D = 128;
  static constexpr int KS = D + FA_FWD_KPAD;
  static constexpr int VS = D + FA_FWD_VPAD;
  static constexpr int K_ELEMS = PP_BK * KS;
  static constexpr int V_ELEMS = PP_BK * VS;
  static constexpr int V0 = 2 * K_ELEMS;                   // K slots 0, 1, then V slots 0, 1
  static constexpr int ELEMS = 2 * K_ELEMS + 2 * V_ELEMS;
  // direct loads of 64 x 16 bytes fill a tile's padded rows in order
  static constexpr int KCPR = KS / 8, VCPR = VS / 8;       // chunks per padded row
  static constexpr int KLOADS = PP_BK * KCPR / 64, VLOADS = PP_BK * VCPR / 64;
  static_assert(KLOADS * 64 == PP_BK * KCPR && VLOADS * 64 == PP_BK * VCPR, "tiles must be whole loads");
  static_assert(ELEMS * 2 <= 160 * 1024, "two K and two V tiles fit in the LDS");
};

// Direct HBM -> LDS loads of 128-row tiles shared out over the 8 waves: load
// j of a K tile (or of a V tile) is issued by wave j % 8; lane l of a load
// fills 16-byte chunk 64 (its index within the tile) + l of the tile's
// padded rows.  A lane on a row's padding loads the row's first chunk again
// (the padding is never read).  The buffer resource starts at the tile's
// first row and ends at row N, so rows at or past N read as zero and the
// per-lane offsets stay the same for every tile.
struct PpDma {
  using L = PpLds;
  static constexpr int PK = (L::KLOADS + 7) / 8, PV = (L::VLOADS + 7) / 8;
  uint32_t koff[PK], voff[PV];
  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int u = 0; u < PK; ++u) {
      const int p = 64 * (wave + 8 * u) + lane, row = p / L::KCPR, col = p % L::KCPR;
      koff[u] = (uint32_t)(row * L::D + (col < L::D / 8 ? col * 8 : 0)) * 2;
    }
#pragma unroll
    for (int u = 0; u < PV; ++u) {
      const int p = 64 * (wave + 8 * u) + lane, row = p / L::VCPR, col = p % L::VCPR;
      voff[u] = (uint32_t)(row * L::D + (col < L::D / 8 ? col * 8 : 0)) * 2;
    }
  }
  // rows kv0 .. of the head at src (N rows) into the tile at dst
  __device__ __forceinline__ void k_tile(const uint16_t* src, int N, int kv0, uint16_t* dst, int wave) const {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(src + (size_t)kv0 * L::D, (uint32_t)(N - kv0) * L::D * 2);
#pragma unroll
    for (int u = 0; u < PK; ++u)
      if (wave + 8 * u < L::KLOADS) lds_load16(rs, dst + (wave + 8 * u) * 512, koff[u]);
  }
  __device__ __forceinline__ void v_tile(const uint16_t* src, int N, int kv0, uint16_t* dst, int wave) const {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(src + (size_t)kv0 * L::D, (uint32_t)(N - kv0) * L::D * 2);
#pragma unroll
    for (int u = 0; u < PV; ++u)
      if (wave + 8 * u < L::VLOADS) lds_load16(rs, dst + (wave + 8 * u) * 512, voff[u]);
  }
};

// Matrix phase over one 128-key tile: O^T += V^T P^T on the tile at Vs (PV),
// then S = K Q^T on the tile at Ks (QK).
template <bool QK, bool PV>
__device__ __forceinline__ void pp_matrix(const uint16_t* Ks, const uint16_t* Vs, const bf16x8 (&qf)[8],
                                          f32x16 (&s)[4], f32x16 (&oacc)[4], int lane) {
  using L = PpLds;
  const int l32 = lane & 31, g = lane >> 5;
  if (PV) {
    const int tr_row = 4 * g + ((lane & 15) >> 2);
    const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const uint16_t* vp = Vs + ((b >> 1) * 32 + 16 * (b & 1) + tr_row) * L::VS + tr_col;
      {
        const int kb = b >> 1, t8 = 8 * (b & 1);
        const u32x4 pb = {__float_as_uint(s[kb][t8]), __float_as_uint(s[kb][t8 + 1]), __float_as_uint(s[kb][t8 + 2]),
                          __float_as_uint(s[kb][t8 + 3])};
#pragma unroll
        for (int db = 0; db < 4; ++db)
          oacc[db] = mfma32(bf16x8_from(lds_read_tr16(vp + db * 32), lds_read_tr16(vp + 8 * L::VS + db * 32)),
                            __builtin_bit_cast(bf16x8, pb), oacc[db]);
      }
    }
    // two reads per product, eight ahead
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    // P is dead once these products are issued; S is written only after
    __builtin_amdgcn_sched_barrier(0);
  }
  if (QK) {
    const uint16_t* krow = Ks + l32 * L::KS + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        s[kb] = mfma32(bf16x8_from(*reinterpret_cast<const u32x4*>(krow + kb * 32 * L::KS + ks * 16)), qf[ks],
                       ks == 0 ? f32x16{} : s[kb]);
  }
  if (QK) {
    // one read per product, eight ahead
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  }
}

// The loads of a pair and the LDS reads that follow them, with every LDS
// stage passed as a restrict pointer of one inlined function (K(k), V(k-1)
// read; K(k+1), V(k) written: four disjoint slots), so that the compiler can
// tell that the transpose reads do not read what the loads write and does
// not make them wait for the loads.  Group 0: loads, then its matrix phase.
// Group 1: loads, its softmax phase (sm), the barrier between the phases,
// then its matrix phase.
template <bool QK, bool PV>
__device__ __forceinline__ void pp_load_matrix(const uint16_t* __restrict__ Kr, const uint16_t* __restrict__ Vr,
                                               uint16_t* __restrict__ Kw, uint16_t* __restrict__ Vw, bool load_k,
                                               bool load_v, bool mat, const PpDma& dma, const uint16_t* K,
                                               const uint16_t* V, int N, int kv_k, int kv_v, int wave,
                                               const bf16x8 (&qf)[8], f32x16 (&s)[4], f32x16 (&oacc)[4], int lane) {
  if (load_k) dma.k_tile(K, N, kv_k, Kw, wave);
  if (load_v) dma.v_tile(V, N, kv_v, Vw, wave);
  if (mat) pp_matrix<QK, PV>(Kr, Vr, qf, s, oacc, lane);
}
template <bool QK, bool PV, class SM>
__device__ __forceinline__ void pp_load_softmax_matrix(const uint16_t* __restrict__ Kr,
                                                       const uint16_t* __restrict__ Vr, uint16_t* __restrict__ Kw,
                                                       uint16_t* __restrict__ Vw, bool load_k, bool load_v, bool mat,
                                                       const PpDma& dma, const uint16_t* K, const uint16_t* V, int N,
                                                       int kv_k, int kv_v, int wave, const bf16x8 (&qf)[8],
                                                       f32x16 (&s)[4], f32x16 (&oacc)[4], int lane, SM&& sm) {
  if (load_k) dma.k_tile(K, N, kv_k, Kw, wave);
  if (load_v) dma.v_tile(V, N, kv_v, Vw, wave);
  sm();
  pp_sync();
  if (mat) pp_matrix<QK, PV>(Kr, Vr, qf, s, oacc, lane);
}

template <bool CAUSAL>
__global__ void __launch_bounds__(PP_NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
fwd_pp_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
               uint16_t* __restrict__ O, float* __restrict__ LSE, int N, int nqb, int BH, float c) {
  constexpr int D = 128;
  using L = PpLds;
  constexpr int KSTEPS = D / 16, DB = D / 32;
  __shared__ __attribute__((aligned(16))) uint16_t smem[L::ELEMS];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6) & 7;
  const int grp = wave >> 2;
  const int g = lane >> 5, l32 = lane & 31;

  // this workgroup's item (see above)
  const int nx = BH % 8 == 0 ? 8 : 1;
  const int xg = blockIdx.x % nx, r = blockIdx.x / nx;
  const int hx = BH / nx;
  PpDma dma;
  dma.init(wave, lane);

  {
    const int hl = CAUSAL ? r % hx : r / nqb;
    const int qb = CAUSAL ? nqb - 1 - r / hx : r % nqb;
    const int bh = hl * nx + xg;

    const size_t base = (size_t)bh * N * D;
    const uint32_t head_bytes = (uint32_t)N * D * 2;
    const __amdgpu_buffer_rsrc_t qrs = make_rsrc(Q + base, head_bytes);
    const int q0 = qb * PP_BR;
    // The two waves of a SIMD take adjacent 32-query slices, so both groups
    // meet the causal diagonal in the same tiles.
    const int qw = q0 + 64 * (wave & 3) + 32 * grp;
    const int myq = qw + l32;

    bf16x8 qf[KSTEPS];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
      qf[ks] = bf16x8_from(buf_load16(qrs, (uint32_t)((myq * D + ks * 16 + 8 * g) * 2)));

    const int kv_end = CAUSAL ? min(N, q0 + PP_BR) : N;
    const int ntiles = (kv_end + PP_BK - 1) / PP_BK;
    // Last tile this wave sees, and the first one that needs the mask (it
    // has a key past one of the wave's queries, or past N).
    const int last_w = CAUSAL ? min(qw + 31, N - 1) / PP_BK : ntiles - 1;
    const int first_mask_w = min(CAUSAL ? (qw + 1) / PP_BK : ntiles, N / PP_BK);

    f32x16 oacc[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i) oacc[i] = f32x16{};
    float m = -INFINITY, lsum = 0.f;
    f32x16 s[4];   // S of the tile in flight, then its P (softmax_inplace128)
    auto kslot = [&](int j) { return smem + (j & 1) * L::K_ELEMS; };
    auto vslot = [&](int j) { return smem + L::V0 + (j & 1) * L::V_ELEMS; };
    // Loads of pair k (both groups, at its start): K(k+1) and V(k) into the
    // slots of K(k-1) and V(k-2), whose last reads were in pair k-1; each
    // wave waits for its own loads before the barrier that ends pair k.
    // Softmax phase i; a tile the wave does not see (causal) gives P = 0.
    auto softmax = [&](int i, auto mask_tag) {
      constexpr bool MASK = decltype(mask_tag)::value;
      if (i > last_w) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) s[kb] = f32x16{};
        return;
      }
      const int lim = MASK ? (CAUSAL ? min(myq, N - 1) : N - 1) - i * PP_BK - 4 * g : 0;
      softmax_inplace128<MASK>(s, oacc, m, lsum, c, lim);
    };
    // Group 0's pair k up to its first barrier: the loads, then matrix phase
    // k (P(k-1) V(k-1), then S(k)), if `mat`.
    auto g0_pair = [&](int k, auto qk_tag, auto pv_tag, bool mat) {
      pp_load_matrix<decltype(qk_tag)::value, decltype(pv_tag)::value>(
          kslot(k), vslot(k - 1), kslot(k + 1), vslot(k), k + 1 < ntiles, k < ntiles, mat, dma, K + base, V + base, N,
          (k + 1) * PP_BK, k * PP_BK, wave, qf, s, oacc, lane);
    };
    // Group 1's pair k up to its second barrier: the loads, softmax phase
    // k-1 (sm), the barrier, then matrix phase k if `mat`.
    auto g1_pair = [&](int k, auto qk_tag, auto pv_tag, bool mat, auto&& sm) {
      pp_load_softmax_matrix<decltype(qk_tag)::value, decltype(pv_tag)::value>(
          kslot(k), vslot(k - 1), kslot(k + 1), vslot(k), k + 1 < ntiles, k < ntiles, mat, dma, K + base, V + base, N,
          (k + 1) * PP_BK, k * PP_BK, wave, qf, s, oacc, lane, sm);
    };
    // The last matrix phase: P(ntiles-1) V(ntiles-1) only, no loads before it.
    auto matrix = [&](int k, auto qk_tag, auto pv_tag) {
      pp_matrix<decltype(qk_tag)::value, decltype(pv_tag)::value>(kslot(k), vslot(k - 1), qf, s, oacc, lane);
    };
    using T = std::true_type;
    using F = std::false_type;

    dma.k_tile(K + base, N, 0, kslot(0), wave);
    wait_vmem();
    pp_sync();

    // In the pairs whose softmax needs the mask (the causal diagonal, the
    // ragged end of N) a wave skips matrix phase k when neither tile k nor
    // tile k-1 holds a key it sees (P(k-1) is then zero and S(k) unused);
    // the barriers stay the same for every wave.
    const int k_mask = max(1, min(grp == 0 ? first_mask_w : first_mask_w + 1, ntiles));
    if (grp == 0) {
      g0_pair(0, T{}, F{}, true);
      pp_sync();
      if (0 < first_mask_w) softmax(0, F{}); else softmax(0, T{});
      wait_vmem();
      pp_sync();
      int k = 1;
      for (; k < k_mask; ++k) {
        g0_pair(k, T{}, T{}, true);
        pp_sync();
        softmax(k, F{});
        wait_vmem();
        pp_sync();
      }
      for (; k < ntiles; ++k) {
        g0_pair(k, T{}, T{}, k - 1 <= last_w);
        pp_sync();
        softmax(k, T{});
        wait_vmem();
        pp_sync();
      }
      if (ntiles - 1 <= last_w) matrix(ntiles, F{}, T{});
      pp_sync();
      pp_sync();
    } else {
      g1_pair(0, T{}, F{}, true, [] {});
      wait_vmem();
      pp_sync();
      int k = 1;
      for (; k < k_mask; ++k) {
        g1_pair(k, T{}, T{}, true, [&] { softmax(k - 1, F{}); });
        wait_vmem();
        pp_sync();
      }
      for (; k < ntiles; ++k) {
        g1_pair(k, T{}, T{}, k - 1 <= last_w, [&] { softmax(k - 1, T{}); });
        wait_vmem();
        pp_sync();
      }
      if (ntiles - 1 < first_mask_w) softmax(ntiles - 1, F{}); else softmax(ntiles - 1, T{});
      pp_sync();
      if (ntiles - 1 <= last_w) matrix(ntiles, F{}, T{});
      pp_sync();
    }

    const float ltot = sum_halves(lsum);
    const float inv = ltot > 0.f ? rcp_hw(ltot) : 0.f;
    if (myq < N) {
      uint16_t* orow = O + base + (size_t)myq * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          u32x2 w = {pack_bf16x2(oacc[db][4 * a] * inv, oacc[db][4 * a + 1] * inv),
                     pack_bf16x2(oacc[db][4 * a + 2] * inv, oacc[db][4 * a + 3] * inv)};
          *reinterpret_cast<u32x2*>(orow + db * 32 + 8 * a + 4 * g) = w;
        }
      if (g == 0) LSE[(size_t)bh * N + myq] = ltot > 0.f ? (m + log2_hw(ltot)) * kLn2 : -INFINITY;
    }
  }
}

template <int D, bool CAUSAL, bool SPARSE = false>
hipError_t launch(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, float* lse,
                  int BH, int N, float scale, hipStream_t stream, const uint8_t* bmask = nullptr) {
  // Buffer offsets are 32-bit: one head of K or V must stay below 2 GiB.
  if ((long long)N * D * 2 >= (1LL << 31)) return hipErrorInvalidValue;
  if constexpr (D == 128 && !SPARSE) {
    if (!CAUSAL || N >= PP_MIN_CAUSAL_N) {
      const int nqb = (N + PP_BR - 1) / PP_BR;
      const long long total = (long long)BH * nqb;
      if (total > 0x7fffffffLL) return hipErrorInvalidValue;
      hipLaunchKernelGGL((fwd_pp_kernel<CAUSAL>), dim3((unsigned)total), dim3(PP_NT), 0, stream, q, k, v, o, lse, N,
                         nqb, BH, score_coef(scale));
      return hipGetLastError();
    }
  }
  const int nqb = (N + BR - 1) / BR;
  const long long total = (long long)BH * nqb;
  if (total > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, SPARSE>), dim3((unsigned)total), dim3(NT), 0, stream,
                     q, k, v, o, lse, N, nqb, (int)total, score_coef(scale), bmask);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Balanced block-sparse forward.  A block mask can give some query blocks
// far more visible key blocks than others (a "global" query row sees them
// all); one workgroup per query block then leaves the whole launch waiting
// for the heaviest row.  A plan kernel counts every mask row and splits the
// rows holding more than twice the mean into parts of about the mean; a
// persistent kernel walks the list of (row, part) items; the parts of split
// rows leave partial results (unnormalised O, reference max, row sum) that a
// merge kernel combines exactly as the online softmax combines tiles.  Rows
// that are not split follow the same tile sequence as the one-pass kernel
// and give bit-identical results.
//
// plan (int32): [0] items per head P, [1] partial slots per head, [2] mean,
// [3] number of split rows, then row_cnt[nqb], row_parts[nqb],
// row_first[nqb], row_slot[nqb], item_qb[3 nqb], item_part[3 nqb],
// split_qb[nqb] (the split rows, in order).  With split iff cnt > 2 mean and
// parts = min(16, ceil(cnt / mean)): fewer than nqb / 2 rows split, so P < 2.5 nqb and
// the split rows use fewer than 1.5 nqb slots (2 nqb are allocated).

constexpr int SPARSE_MAX_PARTS = 16;   // parts per split row (bounds the merge's unrolled loads)
constexpr int SPARSE_PLAN_MAX_NQB = 4096;  // plan kept in LDS: 3 ints per query block

__global__ void __launch_bounds__(256)
sparse_plan_kernel(const uint8_t* __restrict__ bmask, int nqb, int causal, int* __restrict__ plan,
                   int* __restrict__ counters, int n_counters) {
  for (int i = threadIdx.x; i < n_counters; i += 256) counters[i] = 0;
  __shared__ int s_cnt[SPARSE_PLAN_MAX_NQB], s_parts[SPARSE_PLAN_MAX_NQB], s_first[SPARSE_PLAN_MAX_NQB];
  int* cnt = plan + 4;
  int* parts = cnt + nqb;
  int* first = parts + nqb;
  int* slot = first + nqb;
  int* item_qb = slot + nqb;
  int* item_part = item_qb + 3 * nqb;
  int* split_qb = item_part + 3 * nqb;
  for (int qb = threadIdx.x; qb < nqb; qb += 256) s_cnt[qb] = 0;
  __syncthreads();
  // Count the visible blocks of every row: the mask is read as a flat array,
  // 16 entries per thread per pass, with the loads of a pass issued together.
  const int cells = nqb * nqb;   // nqb <= 4096, so this fits in 32 bits
  for (int c0 = 16 * threadIdx.x; c0 < cells; c0 += 16 * 256) {
    uint8_t v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = c0 + i < cells ? bmask[c0 + i] : 0;
    int qb = c0 / nqb, kb = c0 - qb * nqb;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (v[i] != 0 && (!causal || kb <= qb)) atomicAdd(&s_cnt[qb], 1);
      if (++kb == nqb) {
        kb = 0;
        ++qb;
      }
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    long long total = 0;
    for (int qb = 0; qb < nqb; ++qb) total += s_cnt[qb];
    const int mean = (int)max(1LL, (total + nqb - 1) / nqb);
    int P = 0, S = 0, ns = 0;
    for (int qb = 0; qb < nqb; ++qb) {
      const int c = s_cnt[qb];
      const int p = c > 2 * mean ? min(SPARSE_MAX_PARTS, (c + mean - 1) / mean) : 1;
      s_parts[qb] = p;
      s_first[qb] = P;
      slot[qb] = p > 1 ? S : -1;
      if (p > 1) split_qb[ns++] = qb;
      P += p;
      if (p > 1) S += p;
    }
    plan[0] = P;
    plan[1] = S;
    plan[2] = mean;
    plan[3] = ns;
  }
  __syncthreads();
  for (int qb = threadIdx.x; qb < nqb; qb += 256) {
    cnt[qb] = s_cnt[qb];
    parts[qb] = s_parts[qb];
    first[qb] = s_first[qb];
    for (int p = 0; p < s_parts[qb]; ++p) {
      item_qb[s_first[qb] + p] = qb;
      item_part[s_first[qb] + p] = p;
    }
  }
}

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(FA_FWD_WAVES_PER_SIMD, FA_FWD_WAVES_PER_SIMD)))
fwd_sparse_balanced_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                           const uint16_t* __restrict__ V, uint16_t* __restrict__ O, float* __restrict__ LSE,
                           int N, int nqb, int BH, float c, const uint8_t* __restrict__ bmask,
                           const int* __restrict__ plan, float* __restrict__ part_o,
                           float* __restrict__ part_ml, int* __restrict__ counters) {
  using L = Lds<D>;
  constexpr int KSTEPS = D / 16, DB = D / 32;
  __shared__ __attribute__((aligned(16))) uint16_t smem[L::ELEMS];
  __shared__ long long s_item;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6) & (NT / 64 - 1);
  const int l32 = lane & 31, g = lane >> 5;
  const int P = plan[0];
  const int* row_cnt = plan + 4;
  const int* row_parts = row_cnt + nqb;
  const int* row_slot = row_parts + 2 * nqb;
  const int* item_qb = row_slot + nqb;
  const int* item_part = item_qb + 3 * nqb;
  const int slots = 2 * nqb;
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  const long long items = (long long)BH * P;

  // Items are split into 8 contiguous ranges, one per XCD (the dispatcher
  // hands workgroup ids to the XCDs round-robin), so the items of a head
  // share one XCD's L2 as in the one-pass grid; within its range a
  // workgroup takes the next item from that XCD's counter (zeroed by the
  // plan kernel), so the load evens out to within one item.  A grid of fewer
  // than 8 workgroups uses one counter over all items.
  const int x = gridDim.x >= 8 ? (int)(blockIdx.x & 7) : 0;
  const long long it0 = gridDim.x >= 8 ? x * items / 8 : 0;
  const long long it1 = gridDim.x >= 8 ? (x + 1) * items / 8 : items;
  while (true) {
    if (tid == 0) s_item = it0 + atomicAdd(&counters[x], 1);
    __syncthreads();
    const long long it = s_item;
    if (it >= it1) break;   // uniform: every wave read the same value
    const int bh = (int)(it / P), i = (int)(it - (long long)bh * P);
    const int qb = item_qb[i], part = item_part[i], parts = row_parts[qb], cnt = row_cnt[qb];
    // this item's visible blocks: ordinals [o0, o1) among the row's visible blocks
    const int o0 = (int)((long long)part * cnt / parts), o1 = (int)((long long)(part + 1) * cnt / parts);
    const size_t base = (size_t)bh * N * D;
    const RowSrc<D> krs{K + base, head_bytes}, vrs{V + base, head_bytes};
    const __amdgpu_buffer_rsrc_t qrs = make_rsrc(Q + base, head_bytes);
    const int q0 = qb * BR, qw = q0 + wave * 32, myq = qw + l32;
    bf16x8 qf[KSTEPS];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
      qf[ks] = bf16x8_from(buf_load16(qrs, (uint32_t)((myq * D + ks * 16 + 8 * g) * 2)));
    const int kend = CAUSAL ? qb + 1 : nqb;            // key blocks that can be visible
    const int kv_end = CAUSAL ? min(N, q0 + BR) : N;
    const int ntiles = (kv_end + BC - 1) / BC;
    f32x16 oacc[DB];
#pragma unroll
    for (int d = 0; d < DB; ++d) oacc[d] = f32x16{};
    float m = -INFINITY, lsum = 0.f;

    // Visible-block walk over the mask row (64 entries per ballot).
    const uint8_t* mrow = bmask + (size_t)qb * nqb;
    int win = -1;
    uint64_t bits = 0;
    auto window = [&](int w) {
      if (w != win) {
        win = w;
        const int e = 64 * w + lane;
        bits = __ballot(e < kend && mrow[e] != 0);
      }
      return bits;
    };
    auto next_visible = [&](int b) {  // smallest visible block >= b, or kend
      while (b < kend) {
        const uint64_t rest = window(b >> 6) >> (b & 63);
        if (rest) return b + (int)__builtin_ctzll(rest);
        b = 64 * ((b >> 6) + 1);
      }
      return kend;
    };
    auto nth_visible = [&](int o) {  // the o-th visible block (from 0), or kend
      for (int w = 0; 64 * w < kend; ++w) {
        uint64_t b = window(w);
        const int n = __builtin_popcountll(b);
        if (o < n) {
          for (int t = 0; t < o; ++t) b &= b - 1;
          return 64 * w + (int)__builtin_ctzll(b);
        }
        o -= n;
      }
      return kend;
    };
    int blk = o1 > o0 ? nth_visible(o0) : kend;
    int blocks_left = o1 - o0;                        // blocks of this item not yet finished
    int j = blk < kend ? 2 * blk : ntiles;
    TileDma<D, NT / 64> dma;
    dma.init(wave, lane);
    if (j < ntiles) dma.issue(krs, vrs, j * BC, smem, wave);
    wait_vmem();
    __syncthreads();
    int slot = 0;
    while (j < ntiles) {
      int jn;
      if ((j & 1) == 0 && j + 1 < ntiles) {
        jn = j + 1;
      } else {
        --blocks_left;
        jn = blocks_left > 0 ? 2 * next_visible((j >> 1) + 1) : ntiles;
        if (jn > ntiles) jn = ntiles;
      }
      const uint16_t* Ks = smem + slot * L::STAGE;
      const uint16_t* Vs = Ks + L::K_ELEMS;
      const int kv0 = j * BC;
      if (jn < ntiles) dma.issue(krs, vrs, jn * BC, smem + (slot ^ 1) * L::STAGE, wave);
      if (!CAUSAL || kv0 <= qw + 31) {
        const int lim = (CAUSAL ? min(myq, N - 1) : N - 1) - kv0 - 4 * g;
        tile_step<D, true>(Ks, Vs, qf, oacc, m, lsum, c, lim, lane);
      }
      wait_vmem();
      __syncthreads();
      slot ^= 1;
      j = jn;
    }

    const float ltot = sum_halves(lsum);
    if (myq < N) {
      if (parts == 1) {
        const float inv = ltot > 0.f ? rcp_hw(ltot) : 0.f;
        uint16_t* orow = O + base + (size_t)myq * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            u32x2 w = {pack_bf16x2(oacc[db][4 * a] * inv, oacc[db][4 * a + 1] * inv),
                       pack_bf16x2(oacc[db][4 * a + 2] * inv, oacc[db][4 * a + 3] * inv)};
            *reinterpret_cast<u32x2*>(orow + db * 32 + 8 * a + 4 * g) = w;
          }
        if (g == 0) LSE[(size_t)bh * N + myq] = ltot > 0.f ? (m + log2_hw(ltot)) * kLn2 : -INFINITY;
      } else {
        const size_t prow = ((size_t)bh * slots + row_slot[qb] + part) * BR + (myq - q0);
        float* po = part_o + prow * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int a = 0; a < 4; ++a)
            *reinterpret_cast<f32x4*>(po + db * 32 + 8 * a + 4 * g) =
                f32x4{oacc[db][4 * a], oacc[db][4 * a + 1], oacc[db][4 * a + 2], oacc[db][4 * a + 3]};
        if (g == 0) *reinterpret_cast<f32x2*>(part_ml + prow * 2) = f32x2{m, ltot};
      }
    }
  }
}

// Combine the parts of split rows: four workgroups per (batch*head, query
// block), 32 rows each; rows that were not split return at once.  Each
// thread merges 4 columns of one row, with the loads of all parts issued
// together.
template <int D>
__global__ void __launch_bounds__(256)
sparse_merge_kernel(const int* __restrict__ plan, const float* __restrict__ part_o,
                    const float* __restrict__ part_ml, uint16_t* __restrict__ O, float* __restrict__ LSE, int N,
                    int nqb, int BH) {
  // Items (head, split row, quarter of its 128 rows), walked by a grid of
  // fixed size: only the split rows have anything to merge.
  const int* row_parts = plan + 4 + nqb;
  const int* row_slot = row_parts + 2 * nqb;
  const int* split_qb = row_slot + nqb + 6 * nqb;
  const int ns = plan[3];
  const long long items = (long long)BH * ns * 4;
  for (long long it = blockIdx.x; it < items; it += gridDim.x) {
  const int quarter = (int)(it & 3);
  const long long hr = it >> 2;
  const int bh = (int)(hr / ns), qb = split_qb[hr - (long long)bh * ns];
  const int parts = row_parts[qb];
  const size_t s0 = (size_t)bh * 2 * nqb + row_slot[qb];
  constexpr int C4 = D / 4;
  for (int idx = threadIdx.x; idx < 32 * C4; idx += 256) {
    const int r = quarter * 32 + idx / C4, c4 = 4 * (idx % C4);
    const int q = qb * BR + r;
    if (q >= N) break;
    f32x2 ml[SPARSE_MAX_PARTS];
    f32x4 ov[SPARSE_MAX_PARTS];
#pragma unroll
    for (int p = 0; p < SPARSE_MAX_PARTS; ++p)
      if (p < parts) {
        const size_t pr = (s0 + p) * BR + r;
        ml[p] = *reinterpret_cast<const f32x2*>(part_ml + pr * 2);
        ov[p] = *reinterpret_cast<const f32x4*>(part_o + pr * D + c4);
      }
    float M = -INFINITY;
#pragma unroll
    for (int p = 0; p < SPARSE_MAX_PARTS; ++p)
      if (p < parts) M = max_nan(M, ml[p][0]);
    float Lsum = 0.f;
    f32x4 acc = {};
    if (M != -INFINITY) {
#pragma unroll
      for (int p = 0; p < SPARSE_MAX_PARTS; ++p)
        if (p < parts) {
          const float f = exp2_hw(ml[p][0] - M);   // 0 for a part with no visible key
          Lsum += ml[p][1] * f;
          acc += ov[p] * f;
        }
    }
    const float inv = Lsum > 0.f ? 1.f / Lsum : 0.f;
    u32x2 w = {pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv)};
    *reinterpret_cast<u32x2*>(O + ((size_t)bh * N + q) * D + c4) = w;
    if (c4 == 0) LSE[(size_t)bh * N + q] = Lsum > 0.f ? (M + log2_hw(Lsum)) * kLn2 : -INFINITY;
  }
  }
}

template <int D, bool CAUSAL>
hipError_t launch_sparse_balanced(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, float* lse,
                                  const uint8_t* bmask, int BH, int N, float scale, void* workspace,
                                  hipStream_t stream) {
  const int nqb = (N + BR - 1) / BR;
  if ((long long)N * D * 2 >= (1LL << 31) || nqb > SPARSE_PLAN_MAX_NQB || (long long)BH * nqb * 4 > 0x7fffffffLL)
    return hipErrorInvalidValue;
  const SparseWorkspace w = sparse_workspace_layout(BH, N, D);
  char* ws = static_cast<char*>(workspace);
  int* plan = reinterpret_cast<int*>(ws);
  float* po = reinterpret_cast<float*>(ws + w.part_o);
  float* pml = reinterpret_cast<float*>(ws + w.part_ml);
  int* counters = reinterpret_cast<int*>(ws + w.counters);
  hipLaunchKernelGGL(sparse_plan_kernel, dim3(1), dim3(256), 0, stream, bmask, nqb, CAUSAL ? 1 : 0, plan, counters,
                     8);
  long long wgs = min((long long)BH * nqb, 512LL);
  if (wgs >= 8) wgs &= ~7LL;   // a multiple of 8: the same number of workgroups per XCD
  hipLaunchKernelGGL((fwd_sparse_balanced_kernel<D, CAUSAL>), dim3((unsigned)wgs), dim3(NT), 0, stream, q, k, v, o,
                     lse, N, nqb, BH, score_coef(scale), bmask, plan, po, pml, counters);
  const unsigned mwgs = (unsigned)min((long long)BH * nqb * 4, 1024LL);
  hipLaunchKernelGGL((sparse_merge_kernel<D>), dim3(mwgs), dim3(256), 0, stream, plan, po, pml, o, lse, N, nqb, BH);
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

SparseWorkspace sparse_workspace_layout(long long BH, int N, int d) {
  SparseWorkspace w;
  const long long nqb = (N + BR - 1) / BR;
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  w.plan = 0;
  w.counters = up((size_t)(4 + 4 * nqb + 6 * nqb + nqb) * sizeof(int));
  w.part_o = up(w.counters + 8 * sizeof(int));
  w.part_ml = up(w.part_o + (size_t)BH * 2 * nqb * BR * d * sizeof(float));
  w.bytes = up(w.part_ml + (size_t)BH * 2 * nqb * BR * 2 * sizeof(float));
  return w;
}

hipError_t launch_fwd_bf16_block_sparse(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                        uint16_t* o, float* lse, const uint8_t* block_mask, int BH,
                                        int N, int d, bool causal, float scale, void* workspace,
                                        hipStream_t stream) {
  if (workspace != nullptr) {
    if (d == 64)
      return causal ? launch_sparse_balanced<64, true>(q, k, v, o, lse, block_mask, BH, N, scale, workspace, stream)
                    : launch_sparse_balanced<64, false>(q, k, v, o, lse, block_mask, BH, N, scale, workspace, stream);
    if (d == 128)
      return causal ? launch_sparse_balanced<128, true>(q, k, v, o, lse, block_mask, BH, N, scale, workspace, stream)
                    : launch_sparse_balanced<128, false>(q, k, v, o, lse, block_mask, BH, N, scale, workspace, stream);
    return hipErrorInvalidValue;
  }
  if (d == 64)
    return causal ? launch<64, true, true>(q, k, v, o, lse, BH, N, scale, stream, block_mask)
                  : launch<64, false, true>(q, k, v, o, lse, BH, N, scale, stream, block_mask);
  if (d == 128)
    return causal ? launch<128, true, true>(q, k, v, o, lse, BH, N, scale, stream, block_mask)
                  : launch<128, false, true>(q, k, v, o, lse, BH, N, scale, stream, block_mask);
  return hipErrorInvalidValue;
}

}  // namespace fa
