/*
 * fa.h - C ABI of the exact-attention library for AMD Instinct MI355X (gfx950).
 *
 * The library computes exact scaled dot-product attention,
 *     O = softmax(scale * Q K^T) V,
 * the formula given on the page "Flash Attention 2で打破するローカルLLMの「メモリの壁」：
 * IO最適化の実践的エンジニアリング", section 「標準的なAttention機構のメモリ挙動」, and its
 * backward pass.  It never forms the N x N score or probability matrix in device
 * memory: Q, K and V are processed in on-chip tiles with a running (online)
 * softmax, as the same page describes in section 「タイリング（Tiling）と再計算
 * （Recomputation）の仕組み」 and as the page "FlashAttention-2を読む：長い文脈の
 * アテンションをGPUで効率化する仕組み" describes in section 「タイル分割でも全体の
 * 正規化を保つ」.  Work is split over batch x heads x query blocks (same page,
 * section 「GPUの稼働率を高める三つの工夫」).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layout     All tensors are dense, contiguous [B][H][N][d] with d fastest
 *            (element (b,h,i,c) at offset ((b*H + h)*N + i)*d + c).  LSE and the
 *            backward workspace rows are [B][H][N] float32.
 * Precision  The bf16 entry points take bfloat16 as raw 16-bit storage
 *            (const void*), multiply in bf16 on the matrix cores and accumulate
 *            in float32; outputs are rounded to bf16 to nearest-even.  The _f32
 *            entry points take float32 everywhere (a slower debug path).
 * Shapes     B, H, N >= 1.  bf16: d in {64, 128}.  f32: 4 <= d <= 128 and
 *            d % 4 == 0.  Any N (a ragged last tile is masked).  N_q == N_k == N
 *            except for fa_decode (Nq new queries over Nk keys).
 * scale      Finite and >= 0 (0 gives uniform attention).  The caller chooses
 *            it; 1/sqrt(d) is the usual value.
 * causal     0 or 1.  1 hides key j from query i when j > i (top-left aligned).
 * LSE        lse[b][h][i] = log(sum_j exp(scale * q_i . k_j)) over the visible
 *            keys j, natural log, float32.
 * Ownership  The caller allocates and owns every buffer (device memory).  The
 *            library allocates nothing and keeps no state between calls, except
 *            for fa_backward_noalloc's static scratch buffer (see there).
 * Aliasing   q, k and v may alias one another.  Every output buffer (o, lse,
 *            dq, dk, dv, workspace) must not overlap any other buffer passed to
 *            the same call.
 * Alignment  Every tensor pointer must be 16-byte aligned.
 * Streams    Work is enqueued on `stream` (a hipStream_t passed as void*, NULL
 *            for the default stream).  Calls return without synchronising;
 *            results are valid once the stream has reached them.
 * Errors     Every entry point returns FA_OK (0) or a negative status.  All
 *            arguments are checked on the host before any HIP call; a failed
 *            check launches nothing and writes nothing.  FA_ERR_HIP reports a
 *            launch failure from the HIP runtime.  fa_status_string() names a
 *            status.  No C++ exception crosses this interface.
 *            Kernel faults surface asynchronously, at the caller's next
 *            synchronisation.  With the environment variable FA_SYNC_DEBUG=1
 *            every entry point also synchronises `stream` before it returns
 *            and reports any error the runtime then holds as FA_ERR_HIP
 *            (a debugging aid: it serialises the caller's work).
 * Threads    Stateless and re-entrant; calls on different streams may overlap.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_ABI_VERSION 6

enum fa_status {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = -1, /* null pointer, bad size, scale, causal flag,
                              misaligned or overlapping buffers, workspace too small */
  FA_ERR_UNSUPPORTED = -2, /* head dimension not supported by this entry point */
  FA_ERR_HIP = -3,         /* the HIP runtime reported a launch error */
  FA_ERR_TOO_LARGE = -4    /* the problem needs more scratch than the library's
                              static buffer holds (fa_backward_noalloc) */
};

/*
 * Forward pass, bf16 in/out, float32 accumulation.
 *   q, k, v : [B][H][N][d] bf16, read only.
 *   o       : [B][H][N][d] bf16, written: O = softmax(scale*QK^T (masked)) V.
 *   lse     : [B][H][N] float32, written: the row log-sum-exp defined above,
 *             which fa_backward needs.
 * The N x N matrices live only in registers, tile by tile (pages cited above).
 */
int fa_forward(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int N, int d, int causal, float scale, void* stream);

/* Side of the square blocks of a block-sparse mask (queries and keys). */
#define FA_BLOCK_SPARSE_BLOCK 128

/*
 * Block-sparse forward pass, bf16 in/out, float32 accumulation.  The page
 * "FlashAttention――GPUメモリの読み書きを減らし、注意機構を正確なまま高速・省メモリに"
 * (sections 要約 and 手法) extends FlashAttention to block-sparse attention:
 * only the key blocks a mask marks are read and computed, the rest are
 * skipped.  Here query i sees key j iff
 *     block_mask[(i / 128) * nb + j / 128] != 0,   nb = ceil(N / 128),
 * and, when causal, j <= i; the softmax runs over the visible keys only.
 *   q, k, v, o, lse : as for fa_forward.
 *   block_mask      : device, nb x nb bytes row-major (query block major),
 *                     nonzero = visible, read only, any alignment; one mask
 *                     shared by every (batch, head).
 *   workspace       : NULL, or device scratch of at least
 *                     fa_block_sparse_workspace_size() bytes, 16-byte
 *                     aligned (contents on entry ignored, on return
 *                     unspecified).  NULL: one workgroup per query block.
 *                     With a workspace the rows of the mask are counted on
 *                     the device first; rows with more than twice the mean
 *                     count of visible blocks are split over several
 *                     workgroups and their partial results merged, which
 *                     keeps a few dense rows (e.g. global tokens) from
 *                     setting the running time.  Rows that are not split
 *                     give the same bits either way.
 * A query row that sees no key gets o = 0 and lse = -inf.  Without a
 * workspace and with every block visible the result equals fa_forward's
 * (same arithmetic, tile by tile).
 */
int fa_forward_block_sparse(const void* q, const void* k, const void* v, void* o, float* lse,
                            const unsigned char* block_mask, int B, int H, int N, int d,
                            int causal, float scale, void* workspace, size_t workspace_bytes,
                            void* stream);

/* Bytes of workspace fa_forward_block_sparse uses to split heavy rows (0 if
 * a size is out of range; N above 4096 * 128 = 524288 takes no workspace).
 * Pure host function. */
size_t fa_block_sparse_workspace_size(int B, int H, int N, int d);

/* Largest number of new queries per (batch, head) fa_decode accepts. */
#define FA_DECODE_MAX_QUERIES 8

/*
 * Decode-phase forward, bf16 in/out, float32 arithmetic: Nq new queries per
 * (batch, head) attend over Nk cached keys.  The page "Flash Attention 2で打破
 * するローカルLLMの「メモリの壁」：IO最適化の実践的エンジニアリング" (section
 * 「実装上の差を検証可能な形で残す」) treats the prefill and decode phases as
 * separate workloads.  Here the queries are those of positions Nk-Nq .. Nk-1
 * of the sequence whose keys and values are k and v; with causal = 1 the
 * query at position p sees keys j <= p (the causal mask aligned at the bottom
 * right), with causal = 0 every key.  A query that sees no key (Nq > Nk,
 * causal) gets o = 0 and lse = -inf.
 *   q        : [B][H][Nq][d] bf16, read only, 1 <= Nq <= FA_DECODE_MAX_QUERIES.
 *   k, v     : [B][H][Nk][d] bf16, read only, Nk >= 1.
 *   o        : [B][H][Nq][d] bf16, written.
 *   lse      : [B][H][Nq] float32, written (natural-log row log-sum-exp).
 *   workspace: device scratch of at least fa_decode_workspace_size() bytes,
 *              16-byte aligned; contents on entry ignored, on return
 *              unspecified.  It holds the per-chunk partial results: the keys
 *              are split into chunks processed in parallel (split-KV) and
 *              merged through their log-sum-exp.
 * d in {64, 128}.  Deterministic (no atomics; the chunking depends only on
 * B, H, Nq, Nk and d).
 */
int fa_decode(const void* q, const void* k, const void* v, void* o, float* lse,
              int B, int H, int Nq, int Nk, int d, int causal, float scale,
              void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace fa_decode needs for these sizes (0 if a size is out of
 * range).  Pure host function. */
size_t fa_decode_workspace_size(int B, int H, int Nq, int Nk, int d);

/*
 * FP8 forward with incoherent processing (d = 128 only).  The page
 * "FlashAttention-3 — FlashAttention-3" (section 「3. 量子化誤差を低減した低精度
 * （FP8）」) multiplies Q and K by a random orthogonal matrix before quantising
 * them to FP8, which spreads outliers and lowers the FP8 error while leaving
 * Q K^T unchanged.  Here the matrix is diag(signs) H / sqrt(128) (H the
 * Sylvester Hadamard matrix); Q, K (rotated) and V are quantised to OCP E4M3,
 * round to nearest even, with one power-of-two scale per 32 elements (rows of
 * Q and K; 32 consecutive keys of each column of V), chosen so that nothing
 * saturates; the attention then runs on the block-scaled FP8 matrix cores,
 * with P rounded to E4M3 for the P V product and float32 accumulation.
 * Outputs o (bf16) and lse (float32) mean what they mean for fa_forward.
 *
 *   signs : device, 128 floats, each +1 or -1, read only; NULL quantises Q
 *           and K without rotation (plain FP8, for comparison).
 *   buf   : device buffer of at least fa_fp8_buffer_size() bytes, 16-byte
 *           aligned, that receives the quantised operands (layout below).
 *
 * fa_forward_fp8 = fa_fp8_prepare then fa_forward_fp8_prepared (rotated =
 * signs != NULL).  Calling the two halves separately lets a caller reuse the
 * quantised K and V, or time them apart.
 *
 * Layout of buf (sections in this order, each at a 256-byte boundary,
 * (batch, head) major, Np = N rounded up to 64; rows and keys past N are 0):
 *   Q8 [B*H][Np][128] E4M3 codes of the (rotated) Q rows;
 *   QE [B*H][Np][4]   E8M0 scale bytes (127 + t, value 2^t) of their 32-blocks;
 *   K8, KE            the same for K;
 *   V8 [B*H][Np/64][128][64]: row c of 64-key tile T holds, for b = 0, 1, the
 *                     codes of keys 32b .. 32b+31 of column c, key
 *                     32b + 8j + 4g + i at byte 32b + 16g + 4j + i;
 *   VE [B*H][Np/64][2][32][4]: VE[T][b][c % 32][c / 32] is the scale byte of
 *                     keys 32b .. 32b+31 of column c.
 */
size_t fa_fp8_buffer_size(int B, int H, int N, int d);
int fa_fp8_prepare(const void* q, const void* k, const void* v, const float* signs,
                   int B, int H, int N, int d, void* buf, size_t buf_bytes, void* stream);
int fa_forward_fp8_prepared(const void* buf, size_t buf_bytes, void* o, float* lse,
                            int B, int H, int N, int d, int causal, float scale, int rotated,
                            void* stream);
int fa_forward_fp8(const void* q, const void* k, const void* v, const float* signs,
                   void* o, float* lse, int B, int H, int N, int d, int causal, float scale,
                   void* buf, size_t buf_bytes, void* stream);

/*
 * Backward pass, bf16 in/out, float32 accumulation: the vector-Jacobian
 * product of O with respect to Q, K and V for the incoming gradient dO.
 * The probability matrix is recomputed from q, k and lse rather than stored
 * (page "Flash Attention 2で打破するローカルLLMの「メモリの壁」：IO最適化の実践的
 * エンジニアリング", section 「タイリング（Tiling）と再計算（Recomputation）の仕組み」).
 *   q, k, v, o, dO : [B][H][N][d] bf16, read only (o from fa_forward).
 *   lse            : [B][H][N] float32 from fa_forward with the same
 *                    causal flag and scale.
 *   dq, dk, dv     : [B][H][N][d] bf16, written.
 *   workspace      : device scratch of at least fa_backward_workspace_size()
 *                    bytes, 16-byte aligned; its contents on entry are ignored
 *                    and on return are unspecified.
 * Deterministic: the same inputs give bit-identical outputs (no atomics).
 */
int fa_backward(const void* q, const void* k, const void* v, const void* o,
                const float* lse, const void* dO, void* dq, void* dk, void* dv,
                int B, int H, int N, int d, int causal, float scale,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * The stages of fa_backward, as separate calls (bf16 only), so that callers
 * can time or schedule them one by one.  Either sequence on one stream with
 * the same workspace gives exactly what fa_backward gives:
 *   fa_backward_dq_delta, then fa_backward_dkdv (what fa_backward runs when
 *   the grids are large), or
 *   fa_backward_preprocess, then fa_backward_dkdv and fa_backward_dq in
 *   either order.
 * (For grids that fit on the device at once fa_backward runs the dK/dV and
 * dQ work in one launch, so that the two kinds of workgroup share the
 * compute units; the arithmetic per output is the same in every case.)
 * Arguments mean what they mean for fa_backward.
 *   fa_backward_preprocess: workspace rows -delta_i, the negated row sums
 *     delta_i = sum_c dO_ic * O_ic.
 *   fa_backward_dkdv: dK and dV, one workgroup per 128 keys, looping over
 *     query tiles (reads q, k, v, lse, dO and the workspace).
 *   fa_backward_dq: dQ, one workgroup per 128 queries, looping over key
 *     tiles (reads q, k, v, lse, dO and the workspace).
 *   fa_backward_dq_delta: dQ as fa_backward_dq, but each workgroup first
 *     computes -delta of its own queries from o and dO (the same values
 *     fa_backward_preprocess writes) and writes them to the workspace, so no
 *     preprocess pass is needed.
 * The same checks as fa_backward apply to every buffer each stage touches.
 */
int fa_backward_preprocess(const void* o, const void* dO, int B, int H, int N, int d,
                           void* workspace, size_t workspace_bytes, void* stream);
int fa_backward_dkdv(const void* q, const void* k, const void* v, const float* lse,
                     const void* dO, void* dk, void* dv, int B, int H, int N, int d,
                     int causal, float scale, const void* workspace, size_t workspace_bytes,
                     void* stream);
int fa_backward_dq(const void* q, const void* k, const void* v, const float* lse,
                   const void* dO, void* dq, int B, int H, int N, int d, int causal, float scale,
                   const void* workspace, size_t workspace_bytes, void* stream);
int fa_backward_dq_delta(const void* q, const void* k, const void* v, const void* o,
                         const float* lse, const void* dO, void* dq, int B, int H, int N, int d,
                         int causal, float scale, void* workspace, size_t workspace_bytes,
                         void* stream);

/* Bytes of workspace fa_backward and fa_backward_f32 need for these sizes
 * (0 if a size is not positive).  Pure host function. */
size_t fa_backward_workspace_size(int B, int H, int N, int d);

/*
 * Single-pass backward (bf16 only): dK, dV and dQ from one pass over the
 * (key block, query tile) pairs.  fa_backward's dQ pass recomputes S and dP
 * for its own tiles; here the dK/dV pass, which has dS already, also adds
 * each key block's share of dQ into a float32 accumulator with atomic adds.
 * That takes 5 products of N x N x d per head instead of 7, at the price of
 * the atomic traffic and of determinism (the recompute this replaces is the
 * one of page "Flash Attention 2で打破するローカルLLMの「メモリの壁」：IO最適化の
 * 実践的エンジニアリング", section 「タイリング（Tiling）と再計算（Recomputation）の
 * 仕組み」; page "FlashAttention-2 — FlashAttention-2", section
 * 「パフォーマンスと効率」, counts determinism among the method's properties,
 * which is why fa_backward stays the default).
 *   Arguments : as fa_backward; workspace of at least
 *               fa_backward_atomic_workspace_size() bytes, 16-byte aligned
 *               (the rows -delta_i, then a float32 [B][H][N][d] dQ
 *               accumulator); its contents on entry are ignored.
 *   Results   : dk and dv are bit-identical to fa_backward's.  dq =
 *               bf16(scale * sum of the key blocks' shares): the float32
 *               additions happen in the order the atomics arrive, so two
 *               calls may differ in the last bits of dq.
 *   Errors    : as fa_backward.
 */
size_t fa_backward_atomic_workspace_size(int B, int H, int N, int d);
int fa_backward_atomic(const void* q, const void* k, const void* v, const void* o,
                       const float* lse, const void* dO, void* dq, void* dk, void* dv,
                       int B, int H, int N, int d, int causal, float scale,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of the static device scratch buffer behind fa_backward_noalloc. */
#define FA_NOALLOC_SCRATCH_BYTES (16u << 20)

/*
 * fa_backward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  It computes exactly what
 * fa_backward computes (same kernels, bit-identical outputs) and calls no
 * allocating routine.  Its scratch (the rows -delta_i, 4*B*H*N bytes) is a
 * file-scope device array of FA_NOALLOC_SCRATCH_BYTES bytes that each GPU
 * the library runs on holds until the process ends; its address is looked
 * up once per device, on the first call with that device current.
 *   Arguments: as fa_backward, without workspace and workspace_bytes; the
 *   stream must belong to the current device.
 *   Returns FA_ERR_TOO_LARGE when 4*B*H*N (rounded up to 256) exceeds
 *   FA_NOALLOC_SCRATCH_BYTES (B*H*N up to 4194304 rows fits), after the
 *   same argument checks as fa_backward.
 * Every call on one GPU shares that GPU's scratch: calls that may overlap in
 * time on one GPU (different streams, or different host threads) race and
 * must be serialised by the caller.  Calls on one stream are ordered and
 * safe.
 */
int fa_backward_noalloc(const void* q, const void* k, const void* v, const void* o,
                        const float* lse, const void* dO, void* dq, void* dk, void* dv,
                        int B, int H, int N, int d, int causal, float scale, void* stream);

/* float32 debug twins of fa_forward / fa_backward: same arguments, same
 * layouts and semantics, float32 storage and arithmetic throughout. */
int fa_forward_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                   int B, int H, int N, int d, int causal, float scale, void* stream);
int fa_backward_f32(const float* q, const float* k, const float* v, const float* o,
                    const float* lse, const float* dO, float* dq, float* dk, float* dv,
                    int B, int H, int N, int d, int causal, float scale,
                    void* workspace, size_t workspace_bytes, void* stream);

/* Static text naming a status code (never NULL). */
const char* fa_status_string(int status);

/* FA_ABI_VERSION of the built library. */
int fa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
