// Internal launchers behind the C ABI.  Arguments are already validated:
// tensors are [BH][N][d] contiguous (BH = batch*heads), pointers are 16-byte
// aligned, sizes are positive and supported.  Each launcher enqueues its
// kernels on `stream` and returns the HIP status of the launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

hipError_t launch_fwd_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                           float* lse, int BH, int N, int d, bool causal, float scale,
                           hipStream_t stream);

// Block-sparse forward: block_mask is [ceil(N/128)][ceil(N/128)] bytes.
// With a workspace (laid out by sparse_workspace_layout) heavy mask rows are
// split over several workgroups and merged; without one, one workgroup per
// query block.
struct SparseWorkspace {
  size_t plan, counters, part_o, part_ml, bytes;
};
SparseWorkspace sparse_workspace_layout(long long BH, int N, int d);
hipError_t launch_fwd_bf16_block_sparse(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                        uint16_t* o, float* lse, const uint8_t* block_mask, int BH,
                                        int N, int d, bool causal, float scale, void* workspace,
                                        hipStream_t stream);

// Decode (1 <= nq <= 8 queries over Nk keys), split over key chunks.  The
// workspace layout and size follow decode_split(); both the launcher and the
// size query use it.
struct DecodeSplit {
  int chunk;       // keys per chunk
  int nsplit;      // chunks per (batch, head)
  size_t o_bytes;  // bytes of the partial outputs (256-byte multiple)
  size_t bytes;    // total workspace bytes
};
DecodeSplit decode_split(long long BH, int nq, int Nk, int d);
hipError_t launch_decode_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, float* lse,
                              int BH, int nq, int Nk, int d, bool causal, float scale, void* workspace,
                              hipStream_t stream);

// FP8 forward (d = 128): byte offsets of the sections of the prepared
// buffer, Np = N rounded up to 64, and its size.
struct Fp8Buffer {
  size_t q8, qe, k8, ke, v8, ve, bytes;
  int Np;
};
Fp8Buffer fp8_buffer_layout(long long BH, int N);
// Quantise Q, K (rotated by diag(signs) * Hadamard when signs != nullptr)
// and V into `buf`.
hipError_t launch_fp8_prepare(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* signs, int BH,
                              int N, void* buf, hipStream_t stream);
// Attention on a prepared buffer; `rotated` folds the rotation's 1/d into
// the softmax scale.
hipError_t launch_fwd_fp8(const void* buf, uint16_t* o, float* lse, int BH, int N, bool causal, float scale,
                          bool rotated, hipStream_t stream);

hipError_t launch_bwd_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                           const uint16_t* o, const float* lse, const uint16_t* dO, uint16_t* dq,
                           uint16_t* dk, uint16_t* dv, int BH, int N, int d, bool causal,
                           float scale, float* delta, hipStream_t stream);

// Single-pass backward: -delta (row-dot pass) into `delta`, dqacc
// (BH*N*d floats) zeroed, one dK/dV launch that also adds dS K into dqacc
// with float32 atomics, then dq = bf16(scale * dqacc).  dK and dV have the
// same bits as launch_bwd_bf16's; dQ depends on the order of the atomics.
hipError_t launch_bwd_single_pass_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* o,
                                      const float* lse, const uint16_t* dO, uint16_t* dq, uint16_t* dk,
                                      uint16_t* dv, int BH, int N, int d, bool causal, float scale, float* delta,
                                      float* dqacc, hipStream_t stream);

hipError_t launch_bwd_dkdv_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                const float* lse, const uint16_t* dO, const float* delta,
                                uint16_t* dk, uint16_t* dv, int BH, int N, int d, bool causal,
                                float scale, hipStream_t stream);

hipError_t launch_bwd_dq_delta_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* o,
                                   const float* lse, const uint16_t* dO, float* delta, uint16_t* dq, int BH,
                                   int N, int d, bool causal, float scale, hipStream_t stream);
hipError_t launch_bwd_dq_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              const float* lse, const uint16_t* dO, const float* delta,
                              uint16_t* dq, int BH, int N, int d, bool causal, float scale,
                              hipStream_t stream);

hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                          int BH, int N, int d, bool causal, float scale, hipStream_t stream);

hipError_t launch_bwd_f32(const float* q, const float* k, const float* v, const float* o,
                          const float* lse, const float* dO, float* dq, float* dk, float* dv,
                          int BH, int N, int d, bool causal, float scale, float* delta,
                          hipStream_t stream);

// delta[row] = sum_c dO[row][c] * O[row][c] over `rows` rows of width d.
hipError_t launch_rowdot_bf16(const uint16_t* o, const uint16_t* dO, float* delta, long long rows,
                              int d, hipStream_t stream);
hipError_t launch_rowdot_f32(const float* o, const float* dO, float* delta, long long rows, int d,
                             hipStream_t stream);

}  // namespace fa
