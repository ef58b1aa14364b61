// Backward exact attention, bf16 in/out, float32 accumulation, for gfx950.
//
// The probabilities are recomputed from Q, K and the saved LSE instead of
// being stored (page "Flash Attention 2で打破するローカルLLMの「メモリの壁」：IO最適化の
// 実践的エンジニアリング", section 「タイリング（Tiling）と再計算（Recomputation）の仕組み」).
// With P = exp(scale*Q K^T - LSE) (masked entries 0) and delta = rowsum(dO * O):
//     dV = P^T dO,   dP = dO V^T,   dS = P * (dP - delta),
//     dQ = scale * dS K,   dK = scale * dS^T Q.
// The default backward launches on one stream with no atomics, so its
// result is bit-reproducible:
//   1. -delta (row-dot pre-pass, in f32_path.hip; the negated sums let the
//      dP accumulators start from them), or computed by the dQ kernel for
//      its own queries when that kernel runs first;
//   2. dK/dV: one workgroup per (batch*head, 128 keys); each wave owns 32
//      keys (K rows in registers) and loops over query tiles of 32 (causal:
//      from the diagonal on);
//   3. dQ: one workgroup per (batch*head, 128 queries); each wave owns 32
//      queries (Q and dO rows in registers) and loops over key tiles of 64
//      (causal: up to the diagonal).
// The single-pass form (bwd_single_pass_kernel) runs step 2 only and adds
// each key block's share of dQ into a float32 accumulator with atomics; its
// dK and dV are those of step 2, its dQ depends on the order of the adds.
// Every product runs on the 32x32x16 bf16 matrix cores.  Each kernel picks
// the orientation (S or S^T) in which its register-resident rows sit on the
// lanes.  Tiles stay row-major in LDS; operands that need the other
// orientation come from the LDS transpose read.  Tiles are double-buffered:
// tile i+1 is fetched by direct HBM-to-LDS loads while tile i is computed.
//
// Ragged N needs no masks here: rows past N read as zero (buffer loads), a
// zero key row contributes nothing to dQ, a query past N has a zero dO row
// and delta (so dS = 0 and P^T dO = 0 whatever its P), and results for keys
// or queries past N are never stored.
#include <algorithm>
#include <type_traits>

#include "fa_common.h"
#include "launch.h"

namespace fa {
namespace {

constexpr int NT = 256;

// Waves per SIMD: at d = 64 both kernels fit 168 VGPRs and ~37 KB of LDS, so
// three workgroups share a CU (measured +8% over two); at d = 128 two.
template <int D>
constexpr int bwd_waves_per_simd() { return D == 64 ? 3 : 2; }

// Row stride (elements) of a tile that is read both with 16-byte row reads
// (32 rows, one column block) and with the transpose read (4 rows x 32
// bytes per 16 lanes).  The row reads are free of bank conflicts when 16
// consecutive rows start on 16 different 16-byte slots of a 256-byte bank
// line; 304 bytes (d=128) and 144 bytes (d=64) do that.  No stride also
// keeps 4 consecutive rows of a transpose read apart, so those reads take
// rows 4 apart instead (spread_row): rows x, x+4, x+8, x+12 start 0, 64,
// 128 and 192 bytes apart in the bank line at either stride.
template <int D>
constexpr int both_ways_stride() { return D == 128 ? D + 24 : D + 8; }

// Tile row that holds row x = 16t + 8s + 4g + j of a 32x32 MFMA operand
// (j = 0..3 the 4 rows one lane group of the transpose read covers, g the
// lane half, s the second read of the pair, t the half of a 32-row block):
// 16t + 4j + 2s + g, so one transpose read takes rows 4 apart.  Row reads
// use the same map (lane x reads tile row spread_row(x)), which keeps the
// accumulators of S and dP in the order the transpose reads expect.
__device__ __forceinline__ constexpr int spread_row(int x) {
  return (x & 16) | ((x & 3) << 2) | ((x >> 2) & 2) | ((x >> 2) & 1);
}
// Row stride of a tile read only with 16-byte row reads.
template <int D>
constexpr int row_read_stride() { return D + 8; }

// Global -> register staging of ROWS x D bf16 rows starting at row r0 of a
// buffer; rows past the buffer read as zero.
template <int ROWS, int D>
struct Rows {
  static constexpr int CPR = D / 8;
  static constexpr int CPT = ROWS * CPR / NT;
  static_assert(CPT * NT == ROWS * CPR, "tile must split evenly over the workgroup");
  u32x4 r[CPT];
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, int r0, int tid) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + NT * i;
      r[i] = buf_load16(rs, (uint32_t)(((r0 + c / CPR) * D + (c % CPR) * 8) * 2));
    }
  }
  template <int STRIDE>
  __device__ __forceinline__ void store(uint16_t* dst, int tid) const {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + NT * i;
      *reinterpret_cast<u32x4*>(dst + (c / CPR) * STRIDE + (c % CPR) * 8) = r[i];
    }
  }
};

// Row `row` of a row-major tile, 16-byte block ks*16 + 8*g: a 32x32x16
// operand whose rows sit on the lanes.
template <int STRIDE>
__device__ __forceinline__ bf16x8 row_operand(const uint16_t* tile, int row, int ks, int g) {
  return bf16x8_from(*reinterpret_cast<const u32x4*>(tile + row * STRIDE + ks * 16 + 8 * g));
}

// Transposed operand from a row-major tile: lane l gets column col0 + l%32
// of rows row0 + 16t + 8(v/4) + 4g + v%4 (slot v), the slot order of a
// 32x32x16 accumulator converted with acc_to_operand(.., t).
template <int STRIDE>
__device__ __forceinline__ bf16x8 tr_operand(const uint16_t* tile, int row0, int col0, int t, int lane) {
  const int g = lane >> 5;
  const uint16_t* p = tile + (row0 + 16 * t + 4 * g + ((lane & 15) >> 2)) * STRIDE + col0 +
                      16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  return bf16x8_from(lds_read_tr16(p), lds_read_tr16(p + 8 * STRIDE));
}

// tr_operand over a tile whose 32-row blocks are in spread_row order: slot v
// of lane l comes from tile row row0 + spread_row(16t + 8(v/4) + 4g + v%4).
template <int STRIDE>
__device__ __forceinline__ bf16x8 tr_operand_spread(const uint16_t* tile, int row0, int col0, int t, int lane) {
  const int g = lane >> 5;
  const uint16_t* p = tile + (row0 + 16 * t + 4 * ((lane & 15) >> 2) + g) * STRIDE + col0 +
                      16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  return bf16x8_from(lds_read_tr16(p), lds_read_tr16(p + 2 * STRIDE));
}

// Accumulator elements r = 8t .. 8t+7 of `x` as one bf16 operand.
__device__ __forceinline__ bf16x8 acc_to_operand(const f32x16& x, int t) {
  u32x4 u = {pack_bf16x2(x[8 * t + 0], x[8 * t + 1]), pack_bf16x2(x[8 * t + 2], x[8 * t + 3]),
             pack_bf16x2(x[8 * t + 4], x[8 * t + 5]), pack_bf16x2(x[8 * t + 6], x[8 * t + 7])};
  return __builtin_bit_cast(bf16x8, u);
}

// Store a [D][32] accumulator set (lane holds column l%32) as row `dst_row`
// of a [N][D] bf16 matrix: element r of block db is column
// 32*db + 8*(r/4) + 4*g + r%4.
template <int D>
__device__ __forceinline__ void store_acc_row(uint16_t* __restrict__ dst_row, const f32x16 (&acc)[D / 32],
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
// LDS reads the dK/dV step issues ahead of its products: row-operand reads
// ahead of the S / dP products, transpose reads ahead of the dV / dK
// products.  Measured (balanced A/B, B8 H16 N2048 d128 causal dK/dV): 7 and 8
// at d = 128 took 284 us against 292 for 4 and 4; at d = 64, 8 transpose
// reads ahead were 2% slower than 4.
template <int D>
constexpr int dkdv_row_reads_ahead() { return 7; }
template <int D>
constexpr int dkdv_tr_reads_ahead() { return D == 128 ? 8 : 4; }
constexpr int KV_BLK = 128;   // keys per dK/dV workgroup
constexpr int Q_TILE = 32;    // queries per dK/dV tile
constexpr int Q_BLK = 128;    // queries per dQ workgroup
constexpr int K_TILE = 64;    // keys per dQ tile

template <int D>
struct DkdvLds {
  static constexpr int QS = both_ways_stride<D>();   // Q and dO tiles
  static constexpr int VS = row_read_stride<D>();    // the workgroup's V rows
  // The Q and dO tiles are filled by direct loads of 64 x 16 bytes (one per
  // lane, in order), so each tile's region is a whole number of such blocks:
  // RI loads cover the Q_TILE padded rows, the rest of the last block is a
  // zero-filled gap.
  static constexpr int CPRP = QS / 8;                          // 16-byte chunks per padded row
  static constexpr int RI = (Q_TILE * CPRP + 63) / 64;         // loads per tile
  static constexpr int TILE = RI * 512;                        // region, elements
  // one stage: Q region, dO region, then LSE and delta (2 x 64 floats, the
  // first 32 of each used)
  static constexpr int STAGE = 2 * TILE + 2 * 64 * 2;
  static constexpr int V_ELEMS = KV_BLK * VS;
  static constexpr int ELEMS = V_ELEMS + 2 * STAGE;
};

template <int D>
struct DqLds {
  static constexpr int KS = both_ways_stride<D>();   // K tile: row reads and transpose reads
  static constexpr int VS = row_read_stride<D>();    // V tile: row reads
  static constexpr int K_ELEMS = K_TILE * KS;
  static constexpr int STAGE = K_ELEMS + K_TILE * VS;
  static constexpr int ELEMS = 2 * STAGE;
  // direct loads of 64 x 16 bytes fill each tile's padded rows in order
  static constexpr int KCPR = KS / 8, VCPR = VS / 8;
  static constexpr int KLOADS = K_TILE * KCPR / 64, VLOADS = K_TILE * VCPR / 64;
  static_assert(KLOADS * 64 == K_TILE * KCPR && VLOADS * 64 == K_TILE * VCPR, "tiles must be whole loads");
};

// One LDS buffer, big enough for either kernel's tiles, used by every
// backward kernel of one head dimension.
template <int D>
constexpr int bwd_lds_elems() { return DkdvLds<D>::ELEMS > DqLds<D>::ELEMS ? DkdvLds<D>::ELEMS : DqLds<D>::ELEMS; }
template <int D>
__device__ __forceinline__ uint16_t* bwd_lds() {
  constexpr int E = bwd_lds_elems<D>();
  __shared__ __attribute__((aligned(16))) uint16_t buf[E];
  return buf;
}

// Single-pass form (dK/dV with dQ added by atomics): after the dK/dV
// layout, the workgroup's K rows (read with the transpose read) and one
// tile's dS, [128 keys][32 query slots].
template <int D>
struct SinglePassLds {
  static constexpr int KS = row_read_stride<D>();
  static constexpr int SS = 32 + 8;
  static_assert(KS % 32 == 8 && SS % 32 == 8, "transpose reads 4 rows apart stay conflict free");
  static constexpr int K_OFF = DkdvLds<D>::ELEMS;
  static constexpr int S_OFF = K_OFF + KV_BLK * KS;
  static constexpr int ELEMS = S_OFF + KV_BLK * SS;
  static_assert(ELEMS * 2 <= 160 * 1024, "the single-pass tiles fit in the LDS");
};
// Dynamic LDS (SinglePassLds<D>::ELEMS elements, set at launch): with a
// static array the compiler would plan for the one workgroup per CU that
// 119 KB allows at d = 128 and spread into the accumulator registers.
__device__ __forceinline__ uint16_t* single_pass_lds() {
  extern __shared__ __attribute__((aligned(16))) uint16_t sp_dyn_lds[];
  return sp_dyn_lds;
}

// Barrier for LDS hazards only: this wave's LDS accesses are complete, its
// vector memory operations may still be in flight (__syncthreads would also
// wait for those).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// One workgroup's work for block id `wid` of a grid of `total` blocks.
// ATOMIC: the single-pass form, which also adds this block's share of
// dQ / scale (dS K over the block's 128 keys) into the float32 dQacc.
template <int D, bool CAUSAL, bool ATOMIC = false>
__device__ __forceinline__ void dkdv_block(int wid, const uint16_t* __restrict__ Q,
                                           const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                                           const float* __restrict__ LSE, const uint16_t* __restrict__ dO,
                                           const float* __restrict__ delta, uint16_t* __restrict__ dK,
                                           uint16_t* __restrict__ dV, int N, int nkb, int total, float c,
                                           float scale, float* __restrict__ dQacc = nullptr) {
  using L = DkdvLds<D>;
  constexpr int KSTEPS = D / 16, DB = D / 32;
  uint16_t* smem;
  if constexpr (ATOMIC)
    smem = single_pass_lds();
  else
    smem = bwd_lds<D>();
  uint16_t* Vs = smem;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6) & (NT / 64 - 1);  // wave-uniform, below 4
  const int l32 = lane & 31, g = lane >> 5;
  int bh, kb;
  map_block(wid, total, nkb, CAUSAL ? 2 : 0, bh, kb);  // causal: low key blocks carry the most work
  const size_t base = (size_t)bh * N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  const RowSrc<D> qrs{Q + base, head_bytes}, grs{dO + base, head_bytes};
  const RowSrc<1, float> lrs{LSE + (size_t)bh * N, (uint32_t)N * 4}, drs{delta + (size_t)bh * N, (uint32_t)N * 4};
  const __amdgpu_buffer_rsrc_t dqrs = make_rsrc(ATOMIC ? static_cast<const void*>(dQacc + base) : Q,
                                                ATOMIC ? (uint32_t)N * D * 4 : 0u);
  const int k0 = kb * KV_BLK;
  const int kw = k0 + wave * 32;
  const int myk = kw + l32;
  // element r of an accumulator is query row spread_row(8(r/4) + 4g + r%4)
  // of the tile, i.e. qrow(r) + g
  auto qrow = [](int r) { return spread_row(8 * (r >> 2) + (r & 3)); };

  // This lane's K row as the B operand of S = Q K^T (rows past N read as
  // zero).  The single-pass form reads it from its K tile in LDS instead.
  bf16x8 kf[ATOMIC ? 1 : KSTEPS];
  if constexpr (!ATOMIC) {
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(K + base, head_bytes);
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
      kf[ks] = bf16x8_from(buf_load16(krs, (uint32_t)((myk * D + ks * 16 + 8 * g) * 2)));
  }
  // The workgroup's V rows, staged once (B operand of dP = dO V^T): loaded
  // here, stored to LDS after the first tile's loads are issued.
  Rows<KV_BLK, D> vrows;
  vrows.load(make_rsrc(V + base, head_bytes), k0, tid);
  using SL = SinglePassLds<D>;
  uint16_t* Ks = smem + SL::K_OFF;
  uint16_t* Ss = smem + SL::S_OFF;
  if constexpr (ATOMIC) {
    // K rows for the dQ product (contracted over keys, so read transposed)
    Rows<KV_BLK, D> krows;
    krows.load(make_rsrc(K + base, head_bytes), k0, tid);
    krows.template store<SL::KS>(Ks, tid);
  }

  f32x16 dkt[DB], dvt[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) dkt[i] = dvt[i] = f32x16{};

  const int qstart = CAUSAL ? k0 : 0;
  const int ntiles = (N - qstart + Q_TILE - 1) / Q_TILE;

  // Per-tile loads, straight into LDS: the Q and dO rows and the delta of
  // the tile's queries; wave 2 loads their LSE into a register and stores
  // LSE * log2(e) at the end of the step.  Slot x of the LSE and delta
  // vectors holds query spread_row(x), the query of accumulator row x.  Queries past N read as zero throughout, which
  // makes their P = exp2(0) = 1 but their dO row, dP and delta zero, so they
  // add nothing to dV (P^T dO) or dK (dS^T Q with dS = P (dP - delta) = 0).
  // Load j of the 2 RI per tile (Q then dO) is issued by wave j % 4; lane l
  // of load jj of a matrix fills 16-byte chunk 64 jj + l of its region.
  constexpr int NJ = (2 * L::RI + 3) / 4;   // loads per wave, at most
  uint32_t voff[NJ];
#pragma unroll
  for (int u = 0; u < NJ; ++u) {
    const int jj = (wave + 4 * u) % L::RI;
    const int p = 64 * jj + lane, row = p / L::CPRP, col = p % L::CPRP;
    voff[u] = row < Q_TILE && col < D / 8 ? (uint32_t)(row * D + col * 8) * 2 : 0x80000000u;
  }
  uint32_t lse_bits = 0;
  const int srow = (lane & 32) | spread_row(l32);
  auto fetch = [&](int qt0, uint16_t* stage) {
    const __amdgpu_buffer_rsrc_t qr = qrs.from_row(qt0), gr = grs.from_row(qt0);
#pragma unroll
    for (int u = 0; u < NJ; ++u) {
      const int j = wave + 4 * u;
      if (j < 2 * L::RI) {
        const int m = j / L::RI, jj = j % L::RI;
        lds_load16(m ? gr : qr, stage + m * L::TILE + jj * 512, voff[u]);
      }
    }
    if (wave == 2)
      lse_bits = __builtin_amdgcn_raw_buffer_load_b32(lrs.from_row(qt0), (uint32_t)srow * 4, 0, 0);
    if (wave == 3) lds_load4(drs.from_row(qt0), stage + 2 * L::TILE + 128, (uint32_t)srow * 4);
  };
  auto put_lse = [&](uint16_t* stage) {
    if (wave == 2) reinterpret_cast<float*>(stage + 2 * L::TILE)[lane] = __uint_as_float(lse_bits) * kLog2e;
  };

  // With the causal mask, query tiles are visited from the last one down to
  // the diagonal, so that the workgroups of one head (all key blocks) start
  // on the same tile and read the same Q and dO tiles at about the same
  // time, each stopping at its own diagonal: the tiles are fetched once into
  // L2 and shared, rather than streamed by each block from a different
  // start.  Without the mask every block visits every tile, so the order does not
  // change what is shared; the ascending order then compiles without
  // spilling at d = 128 (the descending one spilled 12-16 bytes per lane).
  auto tile_of = [&](int p) { return CAUSAL ? ntiles - 1 - p : p; };
  fetch(qstart + tile_of(0) * Q_TILE, smem + L::V_ELEMS);
  vrows.template store<L::VS>(Vs, tid);
  put_lse(smem + L::V_ELEMS);
  wait_vmem();
  __syncthreads();

  // Query tile i, the p-th one visited, for this wave.  MASK: the tile may
  // straddle the diagonal of this wave's keys (some query < some key).
  auto step = [&](int p, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int i = tile_of(p);
    const int qt0 = qstart + i * Q_TILE;
    const uint16_t* Qs = smem + L::V_ELEMS + (p & 1) * L::STAGE;
    const uint16_t* Gs = Qs + L::TILE;
    const float* lse2 = reinterpret_cast<const float*>(Qs + 2 * L::TILE);   // LSE * log2(e)
    const float* dls = lse2 + 64;
    if (p + 1 < ntiles) fetch(qstart + tile_of(p + 1) * Q_TILE, smem + L::V_ELEMS + ((p + 1) & 1) * L::STAGE);

    // (The single-pass form also runs tiles with no visible query for the
    // wave, where P = 0 and the products add exact zeros: its dS rows must
    // be written either way, and a skip branch there spills.)
    if (ATOMIC || !CAUSAL || !MASK || qt0 + Q_TILE - 1 >= kw) {
      // S and dP: element r is query qt0 + qrow(r) + g, key myk.  At
      // d = 64 the dP accumulator starts from the tile's -delta values (the
      // workspace holds -delta), which saves a subtraction per element; at
      // d = 128 the extra live registers cost more than that saves, and the
      // -delta is added after the product.
      constexpr bool ND_INIT = D == 64;
      f32x16 s, dp, nd = {};
      if constexpr (ND_INIT) {
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(dls + 8 * a + 4 * g);
#pragma unroll
          for (int b = 0; b < 4; ++b) nd[4 * a + b] = d4[b];
        }
      }
      // d = 128: the wave in a product phase gets issue priority over the
      // other wave of its SIMD (1.4-3.2% faster dK/dV; at d = 64 ~1% slower)
      if constexpr (D == 128) __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        bf16x8 kop;
        if constexpr (ATOMIC)
          kop = row_operand<SL::KS>(Ks, wave * 32 + l32, ks, g);
        else
          kop = kf[ks];
        s = mfma32(row_operand<L::QS>(Qs, srow & 31, ks, g), kop, ks == 0 ? f32x16{} : s);
        dp = mfma32(row_operand<L::QS>(Gs, srow & 31, ks, g), row_operand<L::VS>(Vs, wave * 32 + l32, ks, g),
                    ks == 0 ? nd : dp);
      }
      // Scheduling: dkdv_row_reads_ahead row-operand LDS reads (mask 0x100)
      // ahead of the matrix-core instructions (mask 0x008), then 2 products
      // per 3 reads.  The single-pass form leaves the order to the compiler:
      // with a fourth read per step (its K rows) the fixed order spills at
      // d = 128.
      if constexpr (!ATOMIC) {
        constexpr int NM = 2 * KSTEPS, NR = 3 * KSTEPS, AH = dkdv_row_reads_ahead<D>(), STEPS = (NR - AH) / 3;
        __builtin_amdgcn_sched_group_barrier(0x100, AH, 0);
#pragma unroll
        for (int u = 0; u < STEPS; ++u) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, NM - 2 * STEPS, 0);
      }
      if constexpr (D == 128) {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
      }
      // hidden when key > query, i.e. query offset qrow(r) + g < myk - qt0
      const int lim = myk - qt0 - g;
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(lse2 + 8 * a + 4 * g);
        f32x4 d4 = {};
        if constexpr (!ND_INIT) d4 = *reinterpret_cast<const f32x4*>(dls + 8 * a + 4 * g);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int r = 4 * a + b;
          float p = exp2_hw(__builtin_fmaf(s[r], c, -l4[b]));
          if (CAUSAL && MASK && qrow(r) < lim) p = 0.f;
          s[r] = p;
          dp[r] = ND_INIT ? p * dp[r] : p * (dp[r] + d4[b]);
        }
      }
      if constexpr (D == 128) __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const bf16x8 pb = acc_to_operand(s, t);
        const bf16x8 dsb = acc_to_operand(dp, t);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          dvt[db] = mfma32(tr_operand_spread<L::QS>(Gs, 0, 32 * db, t, lane), pb, dvt[db]);
          dkt[db] = mfma32(tr_operand_spread<L::QS>(Qs, 0, 32 * db, t, lane), dsb, dkt[db]);
        }
      }
      // dkdv_tr_reads_ahead transpose reads ahead, then one product per 2 reads.
      {
        constexpr int NM = 4 * DB, AH = dkdv_tr_reads_ahead<D>();
        __builtin_amdgcn_sched_group_barrier(0x100, AH, 0);
#pragma unroll
        for (int u = 0; u < NM - AH / 2; ++u) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, AH / 2, 0);
      }
      if constexpr (D == 128) {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
      }
      if constexpr (ATOMIC) {
        // this wave's dS rows (the bf16 values of the dK product): row
        // 32 wave + l%32, slot 8(r/4) + 4g + r%4 holds element r
        __builtin_amdgcn_sched_barrier(0);
        uint16_t* srow_p = Ss + (wave * 32 + l32) * SL::SS + 4 * g;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const u32x4 w = __builtin_bit_cast(u32x4, acc_to_operand(dp, t));
          *reinterpret_cast<u32x2*>(srow_p + 16 * t) = u32x2{w[0], w[1]};
          *reinterpret_cast<u32x2*>(srow_p + 16 * t + 8) = u32x2{w[2], w[3]};
        }
      }
    }
    // dQ share of the tile: wave cb < D / 32 forms slots x columns
    // 32 cb .. 32 cb + 31 over all 128 keys of the block (at d = 64 waves 2
    // and 3 have no share: one atomic per element rather than two partial
    // sums).  Both operands come from the transpose read in the same
    // (spread) row order, so they pair key by key; rows 4 apart at these
    // strides (8 mod 32 elements) keep the reads free of bank conflicts.
    constexpr int NCB = D / 32;
    const bool has_dq = wave < NCB;
    if constexpr (ATOMIC) lds_barrier();
    if (ATOMIC && has_dq) {
      const int cb = wave;
      f32x16 dq = {};
#pragma unroll
      for (int j = 0; j < 8; ++j)
        dq = mfma32(tr_operand_spread<SL::SS>(Ss, 32 * (j >> 1), 0, j & 1, lane),
                    tr_operand_spread<SL::KS>(Ks, 32 * (j >> 1), 32 * cb, j & 1, lane), dq);
      // element r is slot m = 8(r/4) + 4g + r%4, i.e. query qt0 +
      // spread_row(m) = qt0 + g + 16(a/2) + 2(a%2) + 4b (r = 4a + b),
      // column 32 cb + l%32; rows past N fall outside the buffer and are
      // dropped.  Exactly 16 atomics per wave per tile (the wait below
      // counts on it).  The tile's base offset is opaque to the optimiser,
      // so each atomic's offset stays base + constant (the constant's low
      // 12 bits go to the instruction) instead of 16 offsets held across
      // the loop.
      uint32_t obase = (uint32_t)(((qt0 + g) * D + 32 * cb + l32) * 4);
      asm volatile("" : "+v"(obase));
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int a = r >> 2, b = r & 3;
        const uint32_t rows = 16 * (a >> 1) + 2 * (a & 1) + 4 * b;
        __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(dq[r], dqrs, obase + rows * D * 4, 0, 0);
      }
    }
    if (p + 1 < ntiles) put_lse(smem + L::V_ELEMS + ((p + 1) & 1) * L::STAGE);
    if constexpr (ATOMIC) {
      // Vector memory operations complete in issue order, so once at most
      // the 16 atomics just issued are outstanding, the next tile's loads
      // (issued before them) have landed; the atomics finish during the
      // next tile.  A wave without atomics waits for everything.
      if (has_dq)
        __builtin_amdgcn_s_waitcnt(0x4F70);   // vmcnt(16)
      else
        wait_vmem();
      lds_barrier();
    } else {
      wait_vmem();
      __syncthreads();
    }
  };
  // Causal: the first KV_BLK / Q_TILE tiles straddle the diagonals of the
  // workgroup's waves; every later tile is fully visible.
  const int n_diag = CAUSAL ? min(ntiles, KV_BLK / Q_TILE) : 0;
  if constexpr (ATOMIC) {
    // one loop of masked steps (the mask is a no-op away from the
    // diagonal): a second copy of the larger single-pass step spills
    for (int p = 0; p < ntiles; ++p) step(p, std::true_type{});
  } else {
    int p = 0;
    for (; p < ntiles - n_diag; ++p) step(p, std::false_type{});
    for (; p < ntiles; ++p) step(p, std::true_type{});
  }

  if (myk < N) {
    store_acc_row<D>(dK + base + (size_t)myk * D, dkt, scale, g);
    store_acc_row<D>(dV + base + (size_t)myk * D, dvt, 1.0f, g);
  }
}

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(bwd_waves_per_simd<D>(), bwd_waves_per_simd<D>())))
bwd_dkdv_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                const uint16_t* __restrict__ V, const float* __restrict__ LSE,
                const uint16_t* __restrict__ dO, const float* __restrict__ delta,
                uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int N, int nkb, int total,
                float c, float scale) {
  dkdv_block<D, CAUSAL>(blockIdx.x, Q, K, V, LSE, dO, delta, dK, dV, N, nkb, total, c, scale);
}

// ---------------------------------------------------------------- dQ
// DELTA: the workgroup first computes -delta of its own queries from O and
// dO (the row-dot pre-pass's arithmetic, in the same order, so the values
// are the same bits), writes it to nd_out for the dK/dV kernel that runs
// next, and uses it itself; `delta` is then not read.
template <int D, bool CAUSAL, bool DELTA = false>
__device__ __forceinline__ void dq_block(int wid, const uint16_t* __restrict__ Q,
                                         const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                                         const float* __restrict__ LSE, const uint16_t* __restrict__ dO,
                                         const float* __restrict__ delta, uint16_t* __restrict__ dQ, int N,
                                         int nqb, int total, float c, float scale,
                                         const uint16_t* __restrict__ O = nullptr, float* __restrict__ nd_out = nullptr) {
  using L = DqLds<D>;
  constexpr int KSTEPS = D / 16, DB = D / 32;
  uint16_t* smem = bwd_lds<D>();

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6) & (NT / 64 - 1);  // wave-uniform, below 4
  const int l32 = lane & 31, g = lane >> 5;
  int bh, qb;
  map_block_xcd(wid, total, nqb, CAUSAL, bh, qb);
  const size_t base = (size_t)bh * N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  const RowSrc<D> krs{K + base, head_bytes}, vrs{V + base, head_bytes};
  const int q0 = qb * Q_BLK;
  const int qw = q0 + wave * 32;
  const int myq = qw + l32;

  // This lane's Q and dO rows as B operands (rows past N read as zero).
  bf16x8 qf[KSTEPS], gf[KSTEPS];
  {
    const __amdgpu_buffer_rsrc_t qrs = make_rsrc(Q + base, head_bytes);
    const __amdgpu_buffer_rsrc_t grs = make_rsrc(dO + base, head_bytes);
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const uint32_t off = (uint32_t)((myq * D + ks * 16 + 8 * g) * 2);
      qf[ks] = bf16x8_from(buf_load16(qrs, off));
      gf[ks] = bf16x8_from(buf_load16(grs, off));
    }
  }
  const float lse2 = myq < N ? LSE[(size_t)bh * N + myq] * kLog2e : INFINITY;
  // K and V tiles come by direct HBM -> LDS loads: load j of a tile pair (K
  // loads first, then V) is issued by wave j % 4, and lane l of a load fills
  // the 16-byte chunk 64 (its index within the tile) + l of the padded rows;
  // lanes on a row's padding get an offset past the buffer (zeros).
  constexpr int NL = L::KLOADS + L::VLOADS, PW = (NL + 3) / 4;
  uint32_t voff[PW];
#pragma unroll
  for (int u = 0; u < PW; ++u) {
    const int j = wave + 4 * u;
    const bool isv = j >= L::KLOADS;
    const int cpr = isv ? L::VCPR : L::KCPR;
    const int p = 64 * (isv ? j - L::KLOADS : j) + lane, row = p / cpr, col = p % cpr;
    voff[u] = col < D / 8 ? (uint32_t)(row * D + col * 8) * 2 : 0x80000000u;
  }
  auto fetch = [&](int kv0, uint16_t* stage) {
    const __amdgpu_buffer_rsrc_t kr = krs.from_row(kv0), vr = vrs.from_row(kv0);
#pragma unroll
    for (int u = 0; u < PW; ++u) {
      const int j = wave + 4 * u;
      if (j < L::KLOADS)
        lds_load16(kr, stage + j * 512, voff[u]);
      else if (j < NL)
        lds_load16(vr, stage + L::K_ELEMS + (j - L::KLOADS) * 512, voff[u]);
    }
  };
  fetch(0, smem);   // the first tiles load while -delta is computed
  // -delta of this lane's query (the workspace holds -delta): the dP^T
  // accumulators start from it
  float ndl;
  if constexpr (DELTA) {
    // The lane holds columns 16 ks + 8 g .. + 7 of its dO row (gf); it
    // loads the same columns of its O row, sums their products as one FMA
    // chain in column order, and adds the other half from lane ^ 32.  The
    // row-dot pass (rowdot_bf16_kernel) sums in the same order, so both give
    // the same bits.
    const __amdgpu_buffer_rsrc_t ors = make_rsrc(O + base, head_bytes);
    u32x4 orow[KSTEPS];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) orow[ks] = buf_load16(ors, (uint32_t)((myq * D + ks * 16 + 8 * g) * 2));
    float part = 0.f;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const u32x4 gw = __builtin_bit_cast(u32x4, gf[ks]);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        part = __builtin_fmaf(bf16_lo(orow[ks][w]), bf16_lo(gw[w]), part);
        part = __builtin_fmaf(bf16_hi(orow[ks][w]), bf16_hi(gw[w]), part);
      }
    }
    const float tot = part + __shfl_xor(part, 32);
    ndl = myq < N ? -tot : 0.f;
    if (g == 0 && myq < N) nd_out[(size_t)bh * N + myq] = ndl;
  } else {
    ndl = myq < N ? delta[(size_t)bh * N + myq] : 0.f;
  }
  f32x16 ndv;
#pragma unroll
  for (int r = 0; r < 16; ++r) ndv[r] = ndl;
  f32x16 dqt[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) dqt[i] = f32x16{};

  const int kv_end = CAUSAL ? min(N, q0 + Q_BLK) : N;
  const int ntiles = (kv_end + K_TILE - 1) / K_TILE;
  wait_vmem();
  __syncthreads();

  const int srow = spread_row(l32);
  auto krow = [](int r) { return spread_row(8 * (r >> 2) + (r & 3)); };
  auto step = [&](int j, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int kv0 = j * K_TILE;
    const uint16_t* Ks = smem + (j & 1) * L::STAGE;
    const uint16_t* Vs = Ks + L::K_ELEMS;
    if (j + 1 < ntiles) fetch(kv0 + K_TILE, smem + ((j + 1) & 1) * L::STAGE);
    if (!CAUSAL || !MASK || kv0 <= qw + 31) {
      // hidden when key > myq, i.e. key offset 32kb + krow(r) > lim
      const int lim = myq - kv0 - g;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        // S^T and dP^T: element r is key kv0 + 32kb + krow(r) + g, query
        // myq, with the keys of each 32-row block in spread_row order.
        f32x16 s, dp;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
          s = mfma32(row_operand<L::KS>(Ks, kb * 32 + srow, ks, g), qf[ks], ks == 0 ? f32x16{} : s);
          dp = mfma32(row_operand<L::VS>(Vs, kb * 32 + srow, ks, g), gf[ks], ks == 0 ? ndv : dp);
        }
        // Scheduling: 4 row-operand LDS reads (mask 0x100) ahead of the
        // matrix-core instructions (mask 0x008), then 2 and 2 (measured 2-3%
        // faster than leaving the order to the compiler; 8 ahead was no better).
        {
          constexpr int NQ = 2 * KSTEPS, AH = NQ < 4 ? NQ : 4;
          __builtin_amdgcn_sched_group_barrier(0x100, AH, 0);
#pragma unroll
          for (int u = 0; u < (NQ - AH) / 2; ++u) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x008, AH, 0);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = exp2_hw(__builtin_fmaf(s[r], c, -lse2));
          if (CAUSAL && MASK && kb * 32 + krow(r) > lim) p = 0.f;
          dp[r] = p * dp[r];
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const bf16x8 dsb = acc_to_operand(dp, t);
#pragma unroll
          for (int db = 0; db < DB; ++db)
            dqt[db] = mfma32(tr_operand_spread<L::KS>(Ks, kb * 32, 32 * db, t, lane), dsb, dqt[db]);
        }
        // 4 transpose reads ahead, then one product per 2 reads.
        {
          constexpr int NM = 2 * DB, AH = 4;
          __builtin_amdgcn_sched_group_barrier(0x100, AH, 0);
#pragma unroll
          for (int u = 0; u < NM - AH / 2; ++u) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x008, AH / 2, 0);
        }
      }
    }
    wait_vmem();
    __syncthreads();
  };
  // Tiles below every query's diagonal run unmasked; the last (at most two)
  // causal tiles run masked.
  const int n_plain = CAUSAL ? min(ntiles, q0 / K_TILE) : ntiles;
  int j = 0;
  for (; j < n_plain; ++j) step(j, std::false_type{});
  for (; j < ntiles; ++j) step(j, std::true_type{});

  if (myq < N) store_acc_row<D>(dQ + base + (size_t)myq * D, dqt, scale, g);
}

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(bwd_waves_per_simd<D>(), bwd_waves_per_simd<D>())))
bwd_dq_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
              const uint16_t* __restrict__ V, const float* __restrict__ LSE,
              const uint16_t* __restrict__ dO, const float* __restrict__ delta,
              uint16_t* __restrict__ dQ, int N, int nqb, int total, float c, float scale) {
  dq_block<D, CAUSAL>(blockIdx.x, Q, K, V, LSE, dO, delta, dQ, N, nqb, total, c, scale);
}

// dQ together with -delta of its own queries (see dq_block); the dK/dV
// kernel launched after it on the same stream reads that -delta.
template <int D, bool CAUSAL>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(bwd_waves_per_simd<D>(), bwd_waves_per_simd<D>())))
bwd_dq_delta_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                    const uint16_t* __restrict__ V, const float* __restrict__ LSE,
                    const uint16_t* __restrict__ dO, const uint16_t* __restrict__ O, float* __restrict__ nd_out,
                    uint16_t* __restrict__ dQ, int N, int nqb, int total, float c, float scale) {
  dq_block<D, CAUSAL, true>(blockIdx.x, Q, K, V, LSE, dO, nullptr, dQ, N, nqb, total, c, scale, O, nd_out);
}

// dK/dV and dQ in one launch: ids 16j .. 16j+7 run dK/dV block 8j + (id % 8)
// and ids 16j+8 .. 16j+15 dQ block 8j + (id % 8), so both kinds of work sit
// on every XCD (id % 8) in the order each grid would dispatch them, and the
// dQ blocks fill in behind the dK/dV blocks' tail and the reverse.  The two
// grids have the same number of blocks (128 keys or 128 queries each).
template <int D, bool CAUSAL>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(bwd_waves_per_simd<D>(), bwd_waves_per_simd<D>())))
bwd_fused_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                 const uint16_t* __restrict__ V, const float* __restrict__ LSE,
                 const uint16_t* __restrict__ dO, const float* __restrict__ delta,
                 uint16_t* __restrict__ dQ, uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int N, int nb,
                 int total, float c, float scale) {
  const int w = blockIdx.x;
  const int vid = 8 * (w >> 4) + (w & 7);
  if (vid >= total) return;
  if ((w & 8) == 0)
    dkdv_block<D, CAUSAL>(vid, Q, K, V, LSE, dO, delta, dK, dV, N, nb, total, c, scale);
  else
    dq_block<D, CAUSAL>(vid, Q, K, V, LSE, dO, delta, dQ, N, nb, total, c, scale);
}

// Single pass: dK/dV as bwd_dkdv_kernel (the same bits) and dQ / scale
// added into dQacc (float32, zeroed beforehand) by atomics.  d = 128 holds
// 119 KB of LDS, one workgroup per CU; d = 64 67 KB, two.

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
bwd_single_pass_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                       const uint16_t* __restrict__ V, const float* __restrict__ LSE,
                       const uint16_t* __restrict__ dO, const float* __restrict__ delta,
                       uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, float* __restrict__ dQacc, int N,
                       int nkb, int total, float c, float scale) {
  dkdv_block<D, CAUSAL, true>(blockIdx.x, Q, K, V, LSE, dO, delta, dK, dV, N, nkb, total, c, scale, dQacc);
}

// n4 float4 of zeros.
__global__ void __launch_bounds__(256) zero_f32_kernel(f32x4* __restrict__ p, long long n4) {
  const long long stride = (long long)gridDim.x * 256;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) p[i] = f32x4{};
}

// dQ = bf16(scale * dQacc), 8 elements per thread (n8 groups).
__global__ void __launch_bounds__(256) dq_convert_kernel(const f32x4* __restrict__ acc, u32x4* __restrict__ dq,
                                                         long long n8, float scale) {
  const long long stride = (long long)gridDim.x * 256;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n8; i += stride) {
    const f32x4 a = acc[2 * i], b = acc[2 * i + 1];
    dq[i] = u32x4{pack_bf16x2(a[0] * scale, a[1] * scale), pack_bf16x2(a[2] * scale, a[3] * scale),
                  pack_bf16x2(b[0] * scale, b[1] * scale), pack_bf16x2(b[2] * scale, b[3] * scale)};
  }
}

template <int D, bool CAUSAL>
hipError_t launch_single_pass(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* lse,
                              const uint16_t* dO, const float* delta, uint16_t* dk, uint16_t* dv, float* dqacc,
                              int BH, int N, float scale, hipStream_t stream) {
  const int nkb = (N + KV_BLK - 1) / KV_BLK;
  const long long tk = (long long)BH * nkb;
  if (tk > 0x7fffffffLL || (long long)N * D * 2 >= (1LL << 31)) return hipErrorInvalidValue;
  constexpr size_t lds_bytes = SinglePassLds<D>::ELEMS * 2;
  // dynamic LDS above 64 KB: allowed once per kernel (thread-safe static)
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&bwd_single_pass_kernel<D, CAUSAL>),
      hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((bwd_single_pass_kernel<D, CAUSAL>), dim3((unsigned)tk), dim3(NT), lds_bytes, stream, q, k, v,
                     lse, dO, delta, dk, dv, dqacc, N, nkb, (int)tk, score_coef(scale), scale);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_dkdv(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* lse,
                       const uint16_t* dO, const float* delta, uint16_t* dk, uint16_t* dv, int BH,
                       int N, float scale, hipStream_t stream) {
  const int nkb = (N + KV_BLK - 1) / KV_BLK;
  const long long tk = (long long)BH * nkb;
  if (tk > 0x7fffffffLL || (long long)N * D * 2 >= (1LL << 31)) return hipErrorInvalidValue;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3((unsigned)tk), dim3(NT), 0, stream, q, k, v,
                     lse, dO, delta, dk, dv, N, nkb, (int)tk, score_coef(scale), scale);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_fused(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* lse,
                        const uint16_t* dO, const float* delta, uint16_t* dq, uint16_t* dk, uint16_t* dv, int BH,
                        int N, float scale, hipStream_t stream) {
  static_assert(KV_BLK == Q_BLK, "the fused grid pairs key blocks with query blocks");
  const int nb = (N + KV_BLK - 1) / KV_BLK;
  const long long total = (long long)BH * nb;
  const long long grid = 16 * ((total + 7) / 8);
  if (grid > 0x7fffffffLL || (long long)N * D * 2 >= (1LL << 31)) return hipErrorInvalidValue;
  hipLaunchKernelGGL((bwd_fused_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(NT), 0, stream, q, k, v, lse, dO,
                     delta, dq, dk, dv, N, nb, (int)total, score_coef(scale), scale);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_dq_delta(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* lse,
                           const uint16_t* dO, const uint16_t* o, float* nd, uint16_t* dq, int BH, int N,
                           float scale, hipStream_t stream) {
  const int nqb = (N + Q_BLK - 1) / Q_BLK;
  const long long tq = (long long)BH * nqb;
  if (tq > 0x7fffffffLL || (long long)N * D * 2 >= (1LL << 31)) return hipErrorInvalidValue;
  hipLaunchKernelGGL((bwd_dq_delta_kernel<D, CAUSAL>), dim3((unsigned)tq), dim3(NT), 0, stream, q, k, v, lse,
                     dO, o, nd, dq, N, nqb, (int)tq, score_coef(scale), scale);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_dq(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* lse,
                     const uint16_t* dO, const float* delta, uint16_t* dq, int BH, int N, float scale,
                     hipStream_t stream) {
  const int nqb = (N + Q_BLK - 1) / Q_BLK;
  const long long tq = (long long)BH * nqb;
  if (tq > 0x7fffffffLL || (long long)N * D * 2 >= (1LL << 31)) return hipErrorInvalidValue;
  hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3((unsigned)tq), dim3(NT), 0, stream, q, k, v, lse,
                     dO, delta, dq, N, nqb, (int)tq, score_coef(scale), scale);
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

hipError_t launch_bwd_dq_delta_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* o,
                                   const float* lse, const uint16_t* dO, float* delta, uint16_t* dq, int BH,
                                   int N, int d, bool causal, float scale, hipStream_t stream) {
  if (d == 64)
    return causal ? launch_dq_delta<64, true>(q, k, v, lse, dO, o, delta, dq, BH, N, scale, stream)
                  : launch_dq_delta<64, false>(q, k, v, lse, dO, o, delta, dq, BH, N, scale, stream);
  if (d == 128)
    return causal ? launch_dq_delta<128, true>(q, k, v, lse, dO, o, delta, dq, BH, N, scale, stream)
                  : launch_dq_delta<128, false>(q, k, v, lse, dO, o, delta, dq, BH, N, scale, stream);
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

hipError_t launch_bwd_single_pass_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* o,
                                      const float* lse, const uint16_t* dO, uint16_t* dq, uint16_t* dk,
                                      uint16_t* dv, int BH, int N, int d, bool causal, float scale, float* delta,
                                      float* dqacc, hipStream_t stream) {
  if (d != 64 && d != 128) return hipErrorInvalidValue;
  // the single-pass launch's limits, checked before anything is launched
  const long long tk = (long long)BH * ((N + KV_BLK - 1) / KV_BLK);
  if (tk > 0x7fffffffLL || (long long)N * d * 2 >= (1LL << 31)) return hipErrorInvalidValue;
  const long long n = (long long)BH * N * d;   // a multiple of 64
  const int cap = 256 * 8;
  hipError_t e = launch_rowdot_bf16(o, dO, delta, (long long)BH * N, d, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(zero_f32_kernel, dim3((unsigned)std::min<long long>(cap, (n / 4 + 255) / 256)), dim3(256), 0,
                     stream, reinterpret_cast<f32x4*>(dqacc), n / 4);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (d == 64)
    e = causal ? launch_single_pass<64, true>(q, k, v, lse, dO, delta, dk, dv, dqacc, BH, N, scale, stream)
               : launch_single_pass<64, false>(q, k, v, lse, dO, delta, dk, dv, dqacc, BH, N, scale, stream);
  else
    e = causal ? launch_single_pass<128, true>(q, k, v, lse, dO, delta, dk, dv, dqacc, BH, N, scale, stream)
               : launch_single_pass<128, false>(q, k, v, lse, dO, delta, dk, dv, dqacc, BH, N, scale, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(dq_convert_kernel, dim3((unsigned)std::min<long long>(cap, (n / 8 + 255) / 256)), dim3(256), 0,
                     stream, reinterpret_cast<const f32x4*>(dqacc), reinterpret_cast<u32x4*>(dq), n / 8, scale);
  return hipGetLastError();
}

hipError_t launch_bwd_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                           const uint16_t* o, const float* lse, const uint16_t* dO, uint16_t* dq,
                           uint16_t* dk, uint16_t* dv, int BH, int N, int d, bool causal,
                           float scale, float* delta, hipStream_t stream) {
  // While each kernel's grid fits on the chip at once (256 CUs x the waves
  // per SIMD), the two run better side by side in one launch than one after
  // the other; beyond that the separate launches are faster.
  if (d != 64 && d != 128) return hipErrorInvalidValue;
  const long long blocks = (long long)BH * ((N + KV_BLK - 1) / KV_BLK);
  if (blocks <= 256 * (d == 64 ? bwd_waves_per_simd<64>() : bwd_waves_per_simd<128>())) {
    hipError_t e = launch_rowdot_bf16(o, dO, delta, (long long)BH * N, d, stream);
    if (e != hipSuccess) return e;
    if (d == 64)
      return causal ? launch_fused<64, true>(q, k, v, lse, dO, delta, dq, dk, dv, BH, N, scale, stream)
                    : launch_fused<64, false>(q, k, v, lse, dO, delta, dq, dk, dv, BH, N, scale, stream);
    return causal ? launch_fused<128, true>(q, k, v, lse, dO, delta, dq, dk, dv, BH, N, scale, stream)
                  : launch_fused<128, false>(q, k, v, lse, dO, delta, dq, dk, dv, BH, N, scale, stream);
  }
  // Larger grids: dQ first, computing -delta on the way (no row-dot pass),
  // then dK/dV.
  hipError_t e = launch_bwd_dq_delta_bf16(q, k, v, o, lse, dO, delta, dq, BH, N, d, causal, scale, stream);
  if (e != hipSuccess) return e;
  return launch_bwd_dkdv_bf16(q, k, v, lse, dO, delta, dk, dv, BH, N, d, causal, scale, stream);
}

}  // namespace fa
