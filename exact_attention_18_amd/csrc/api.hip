// C ABI entry points (declared in include/fa.h): argument checks on the
// host, then dispatch to the launchers.  No allocation, no global state.
#include <math.h>
#include <stdlib.h>
#include <stdint.h>

#include <mutex>

#include "fa.h"
#include "launch.h"

extern "C" size_t fa_backward_workspace_size(int B, int H, int N, int d);

// Scratch of fa_backward_noalloc: a file-scope device array, one copy per GPU.
// Host code never uses this name as an address (on the host it names a
// stand-in object); the device address comes from hipGetSymbolAddress, once
// per device, with that device current, and is kept in noalloc_ptr.
static __device__ __attribute__((aligned(256))) unsigned char scratch[FA_NOALLOC_SCRATCH_BYTES];

namespace {

struct Span {
  uintptr_t lo, hi;  // [lo, hi)
};

Span span(const void* p, size_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Span{a, a + bytes};
}

bool overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Checks shared by every entry point.  Returns FA_OK or a status.
int check_common(int B, int H, int N, int d, int causal, float scale, bool bf16, size_t* elems) {
  if (B <= 0 || H <= 0 || N <= 0 || d <= 0) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  if (!isfinite(scale) || scale < 0.0f) return FA_ERR_INVALID_ARG;
  if (bf16) {
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  } else {
    if (d > 128 || d % 4 != 0) return FA_ERR_UNSUPPORTED;
  }
  const unsigned long long bh = (unsigned long long)B * (unsigned long long)H;
  if (bh > 0x7fffffffULL) return FA_ERR_INVALID_ARG;
  const unsigned long long n = bh * (unsigned long long)N * (unsigned long long)d;
  if (n / (unsigned long long)d / (unsigned long long)N != bh || n > (1ULL << 50))
    return FA_ERR_INVALID_ARG;
  *elems = (size_t)n;
  return FA_OK;
}

// Null, alignment and overlap checks.  `ins` are read-only (may alias each
// other); `outs` are written and must be disjoint from everything.
int check_buffers(const Span* ins, const void* const* in_ptrs, int n_in, const Span* outs,
                  const void* const* out_ptrs, int n_out) {
  for (int i = 0; i < n_in; ++i)
    if (in_ptrs[i] == nullptr || !aligned16(in_ptrs[i])) return FA_ERR_INVALID_ARG;
  for (int i = 0; i < n_out; ++i)
    if (out_ptrs[i] == nullptr || !aligned16(out_ptrs[i])) return FA_ERR_INVALID_ARG;
  for (int i = 0; i < n_out; ++i) {
    for (int j = 0; j < n_in; ++j)
      if (overlap(outs[i], ins[j])) return FA_ERR_INVALID_ARG;
    for (int j = i + 1; j < n_out; ++j)
      if (overlap(outs[i], outs[j])) return FA_ERR_INVALID_ARG;
  }
  return FA_OK;
}

// Status of a launch.  With FA_SYNC_DEBUG=1 in the environment the stream is
// also synchronised after every entry point and any error it reports
// (including a fault in the kernels just launched) is returned as
// FA_ERR_HIP; this serialises the caller's work and is meant for debugging.
bool sync_debug() {
  const char* v = getenv("FA_SYNC_DEBUG");
  return v != nullptr && v[0] == '1' && v[1] == '\0';
}

int hip_status(hipError_t e, void* stream) {
  if (e != hipSuccess) return FA_ERR_HIP;
  if (sync_debug()) {
    if (hipStreamSynchronize(static_cast<hipStream_t>(stream)) != hipSuccess) return FA_ERR_HIP;
    if (hipGetLastError() != hipSuccess) return FA_ERR_HIP;
  }
  return FA_OK;
}

template <typename T>
int forward_impl(const T* q, const T* k, const T* v, T* o, float* lse, int B, int H, int N, int d,
                 int causal, float scale, void* stream, bool bf16) {
  size_t elems = 0;
  int st = check_common(B, H, N, d, causal, scale, bf16, &elems);
  if (st != FA_OK) return st;
  const size_t tb = elems * sizeof(T), lb = (size_t)B * H * N * sizeof(float);
  const Span ins[3] = {span(q, tb), span(k, tb), span(v, tb)};
  const void* inp[3] = {q, k, v};
  const Span outs[2] = {span(o, tb), span(lse, lb)};
  const void* outp[2] = {o, lse};
  st = check_buffers(ins, inp, 3, outs, outp, 2);
  if (st != FA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if constexpr (sizeof(T) == 2)
    return hip_status(fa::launch_fwd_bf16(q, k, v, o, lse, B * H, N, d, causal != 0, scale, s), stream);
  else
    return hip_status(fa::launch_fwd_f32(q, k, v, o, lse, B * H, N, d, causal != 0, scale, s), stream);
}

template <typename T>
int backward_impl(const T* q, const T* k, const T* v, const T* o, const float* lse, const T* dO, T* dq,
                  T* dk, T* dv, int B, int H, int N, int d, int causal, float scale, void* workspace,
                  size_t workspace_bytes, void* stream, bool bf16) {
  size_t elems = 0;
  int st = check_common(B, H, N, d, causal, scale, bf16, &elems);
  if (st != FA_OK) return st;
  const size_t need = fa_backward_workspace_size(B, H, N, d);
  if (workspace_bytes < need) return FA_ERR_INVALID_ARG;
  const size_t tb = elems * sizeof(T), lb = (size_t)B * H * N * sizeof(float);
  const Span ins[6] = {span(q, tb), span(k, tb), span(v, tb), span(o, tb), span(lse, lb), span(dO, tb)};
  const void* inp[6] = {q, k, v, o, lse, dO};
  const Span outs[4] = {span(dq, tb), span(dk, tb), span(dv, tb), span(workspace, need)};
  const void* outp[4] = {dq, dk, dv, workspace};
  st = check_buffers(ins, inp, 6, outs, outp, 4);
  if (st != FA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* delta = static_cast<float*>(workspace);
  if constexpr (sizeof(T) == 2)
    return hip_status(fa::launch_bwd_bf16(q, k, v, o, lse, dO, dq, dk, dv, B * H, N, d, causal != 0,
                                          scale, delta, s), stream);
  else
    return hip_status(fa::launch_bwd_f32(q, k, v, o, lse, dO, dq, dk, dv, B * H, N, d, causal != 0,
                                         scale, delta, s), stream);
}

constexpr int kMaxDevices = 64;
std::mutex noalloc_mu;
void* noalloc_ptr[kMaxDevices] = {};

// Device address of the current device's scratch, looked up on first use.
int noalloc_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FA_ERR_HIP;
  std::lock_guard<std::mutex> lock(noalloc_mu);
  if (noalloc_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return FA_ERR_HIP;
    noalloc_ptr[dev] = p;
  }
  *out = noalloc_ptr[dev];
  return FA_OK;
}

// Shared checks of the bf16 backward stages.  `ws_written` says whether the
// stage writes the workspace (an output) or only reads it (an input).
int stage_checks(int B, int H, int N, int d, int causal, float scale, const void* const* in_ptrs,
                 const size_t* in_bytes, int n_in, const void* const* out_ptrs, int n_out,
                 const void* workspace, size_t workspace_bytes, bool ws_written) {
  size_t elems = 0;
  int st = check_common(B, H, N, d, causal, scale, true, &elems);
  if (st != FA_OK) return st;
  const size_t need = fa_backward_workspace_size(B, H, N, d);
  if (workspace_bytes < need) return FA_ERR_INVALID_ARG;
  const size_t tb = elems * 2;
  Span ins[8], outs[4];
  const void* inp[8];
  const void* outp[4];
  int ni = 0, no = 0;
  for (int i = 0; i < n_in; ++i) {
    ins[ni] = span(in_ptrs[i], in_bytes[i] ? in_bytes[i] : tb);
    inp[ni++] = in_ptrs[i];
  }
  for (int i = 0; i < n_out; ++i) {
    outs[no] = span(out_ptrs[i], tb);
    outp[no++] = out_ptrs[i];
  }
  if (ws_written) {
    outs[no] = span(workspace, need);
    outp[no++] = workspace;
  } else {
    ins[ni] = span(workspace, need);
    inp[ni++] = workspace;
  }
  return check_buffers(ins, inp, ni, outs, outp, no);
}

}  // namespace

extern "C" {

int fa_backward_preprocess(const void* o, const void* dO, int B, int H, int N, int d, void* workspace,
                           size_t workspace_bytes, void* stream) {
  const void* in[2] = {o, dO};
  const size_t ib[2] = {0, 0};
  int st = stage_checks(B, H, N, d, 0, 1.0f, in, ib, 2, nullptr, 0, workspace, workspace_bytes, true);
  if (st != FA_OK) return st;
  return hip_status(fa::launch_rowdot_bf16(static_cast<const uint16_t*>(o), static_cast<const uint16_t*>(dO),
                                           static_cast<float*>(workspace), (long long)B * H * N, d,
                                           static_cast<hipStream_t>(stream)), stream);
}

int fa_backward_dkdv(const void* q, const void* k, const void* v, const float* lse, const void* dO, void* dk,
                     void* dv, int B, int H, int N, int d, int causal, float scale, const void* workspace,
                     size_t workspace_bytes, void* stream) {
  const void* in[5] = {q, k, v, lse, dO};
  const size_t ib[5] = {0, 0, 0, (size_t)B * H * N * sizeof(float), 0};
  const void* out[2] = {dk, dv};
  int st = stage_checks(B, H, N, d, causal, scale, in, ib, 5, out, 2, workspace, workspace_bytes, false);
  if (st != FA_OK) return st;
  return hip_status(fa::launch_bwd_dkdv_bf16(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), lse,
      static_cast<const uint16_t*>(dO), static_cast<const float*>(workspace), static_cast<uint16_t*>(dk),
      static_cast<uint16_t*>(dv), B * H, N, d, causal != 0, scale, static_cast<hipStream_t>(stream)), stream);
}

int fa_backward_dq(const void* q, const void* k, const void* v, const float* lse, const void* dO, void* dq,
                   int B, int H, int N, int d, int causal, float scale, const void* workspace,
                   size_t workspace_bytes, void* stream) {
  const void* in[5] = {q, k, v, lse, dO};
  const size_t ib[5] = {0, 0, 0, (size_t)B * H * N * sizeof(float), 0};
  const void* out[1] = {dq};
  int st = stage_checks(B, H, N, d, causal, scale, in, ib, 5, out, 1, workspace, workspace_bytes, false);
  if (st != FA_OK) return st;
  return hip_status(fa::launch_bwd_dq_bf16(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), lse,
      static_cast<const uint16_t*>(dO), static_cast<const float*>(workspace), static_cast<uint16_t*>(dq), B * H,
      N, d, causal != 0, scale, static_cast<hipStream_t>(stream)), stream);
}

int fa_backward_dq_delta(const void* q, const void* k, const void* v, const void* o, const float* lse,
                         const void* dO, void* dq, int B, int H, int N, int d, int causal, float scale,
                         void* workspace, size_t workspace_bytes, void* stream) {
  const void* in[6] = {q, k, v, o, lse, dO};
  const size_t ib[6] = {0, 0, 0, 0, (size_t)B * H * N * sizeof(float), 0};
  const void* out[1] = {dq};
  int st = stage_checks(B, H, N, d, causal, scale, in, ib, 6, out, 1, workspace, workspace_bytes, true);
  if (st != FA_OK) return st;
  return hip_status(fa::launch_bwd_dq_delta_bf16(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
      static_cast<const uint16_t*>(o), lse, static_cast<const uint16_t*>(dO), static_cast<float*>(workspace),
      static_cast<uint16_t*>(dq), B * H, N, d, causal != 0, scale, static_cast<hipStream_t>(stream)), stream);
}

int fa_abi_version(void) { return FA_ABI_VERSION; }

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "FA_OK: success";
    case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG: invalid argument (pointer, size, scale, causal flag, alignment, overlap or workspace)";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: head dimension not supported by this entry point";
    case FA_ERR_HIP: return "FA_ERR_HIP: the HIP runtime reported a launch error";
    case FA_ERR_TOO_LARGE: return "FA_ERR_TOO_LARGE: the problem needs more than the static scratch buffer holds";
    default: return "unknown status";
  }
}

int fa_backward_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                        const void* dO, void* dq, void* dk, void* dv, int B, int H, int N, int d, int causal,
                        float scale, void* stream) {
  size_t elems = 0;
  int st = check_common(B, H, N, d, causal, scale, true, &elems);
  if (st != FA_OK) return st;
  const size_t need = fa_backward_workspace_size(B, H, N, d);
  if (need > FA_NOALLOC_SCRATCH_BYTES) return FA_ERR_TOO_LARGE;
  // the caller's buffers are checked before the first HIP call
  const size_t tb = elems * 2, lb = (size_t)B * H * N * sizeof(float);
  const Span ins[6] = {span(q, tb), span(k, tb), span(v, tb), span(o, tb), span(lse, lb), span(dO, tb)};
  const void* inp[6] = {q, k, v, o, lse, dO};
  const Span outs[3] = {span(dq, tb), span(dk, tb), span(dv, tb)};
  const void* outp[3] = {dq, dk, dv};
  st = check_buffers(ins, inp, 6, outs, outp, 3);
  if (st != FA_OK) return st;
  void* ws = nullptr;
  st = noalloc_scratch(&ws);
  if (st != FA_OK) return st;
  return backward_impl(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                       static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(o), lse,
                       static_cast<const uint16_t*>(dO), static_cast<uint16_t*>(dq), static_cast<uint16_t*>(dk),
                       static_cast<uint16_t*>(dv), B, H, N, d, causal, scale, ws, FA_NOALLOC_SCRATCH_BYTES, stream,
                       true);
}

size_t fa_backward_workspace_size(int B, int H, int N, int d) {
  if (B <= 0 || H <= 0 || N <= 0 || d <= 0) return 0;
  const size_t rows = (size_t)B * (size_t)H * (size_t)N;
  return (rows * sizeof(float) + 255) & ~(size_t)255;
}

int fa_forward(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
               int d, int causal, float scale, void* stream) {
  return forward_impl(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                      static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), lse, B, H, N, d,
                      causal, scale, stream, true);
}

size_t fa_block_sparse_workspace_size(int B, int H, int N, int d) {
  if (B <= 0 || H <= 0 || N <= 0 || (d != 64 && d != 128)) return 0;
  if (N > 4096 * FA_BLOCK_SPARSE_BLOCK) return 0;   // the row plan is built in one workgroup's LDS
  const unsigned long long bh = (unsigned long long)B * (unsigned long long)H;
  if (bh > 0x7fffffffULL) return 0;
  return fa::sparse_workspace_layout((long long)bh, N, d).bytes;
}

int fa_forward_block_sparse(const void* q, const void* k, const void* v, void* o, float* lse,
                            const unsigned char* block_mask, int B, int H, int N, int d, int causal,
                            float scale, void* workspace, size_t workspace_bytes, void* stream) {
  size_t elems = 0;
  int st = check_common(B, H, N, d, causal, scale, true, &elems);
  if (st != FA_OK) return st;
  if (block_mask == nullptr) return FA_ERR_INVALID_ARG;
  const size_t nb = ((size_t)N + FA_BLOCK_SPARSE_BLOCK - 1) / FA_BLOCK_SPARSE_BLOCK;
  const size_t tb = elems * 2, lb = (size_t)B * H * N * sizeof(float);
  const size_t need = workspace != nullptr ? fa_block_sparse_workspace_size(B, H, N, d) : 0;
  if (workspace != nullptr && (need == 0 || workspace_bytes < need)) return FA_ERR_INVALID_ARG;
  const Span ins[3] = {span(q, tb), span(k, tb), span(v, tb)};
  const void* inp[3] = {q, k, v};
  const Span outs[3] = {span(o, tb), span(lse, lb), span(workspace, need)};
  const void* outp[3] = {o, lse, workspace};
  st = check_buffers(ins, inp, 3, outs, outp, workspace != nullptr ? 3 : 2);
  if (st != FA_OK) return st;
  const Span ms = span(block_mask, nb * nb);
  for (int i = 0; i < (workspace != nullptr ? 3 : 2); ++i)
    if (overlap(ms, outs[i])) return FA_ERR_INVALID_ARG;
  return hip_status(fa::launch_fwd_bf16_block_sparse(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
      static_cast<uint16_t*>(o), lse, block_mask, B * H, N, d, causal != 0, scale, workspace,
      static_cast<hipStream_t>(stream)), stream);
}

size_t fa_decode_workspace_size(int B, int H, int Nq, int Nk, int d) {
  if (B <= 0 || H <= 0 || Nq <= 0 || Nq > FA_DECODE_MAX_QUERIES || Nk <= 0 || (d != 64 && d != 128)) return 0;
  const unsigned long long bh = (unsigned long long)B * (unsigned long long)H;
  if (bh > 0x7fffffffULL) return 0;
  return fa::decode_split((long long)bh, Nq, Nk, d).bytes;
}

int fa_decode(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq, int Nk,
              int d, int causal, float scale, void* workspace, size_t workspace_bytes, void* stream) {
  if (B <= 0 || H <= 0 || Nq <= 0 || Nk <= 0 || d <= 0) return FA_ERR_INVALID_ARG;
  if (Nq > FA_DECODE_MAX_QUERIES) return FA_ERR_UNSUPPORTED;
  size_t kelems = 0, qelems = 0;
  int st = check_common(B, H, Nk, d, causal, scale, true, &kelems);
  if (st != FA_OK) return st;
  st = check_common(B, H, Nq, d, causal, scale, true, &qelems);
  if (st != FA_OK) return st;
  if ((long long)Nk * d * 2 >= (1LL << 31)) return FA_ERR_INVALID_ARG;  // one head of K below 2 GiB
  if ((unsigned long long)B * H * Nq > 0x7fffffffULL) return FA_ERR_INVALID_ARG;
  const size_t need = fa_decode_workspace_size(B, H, Nq, Nk, d);
  if (need == 0 || workspace_bytes < need) return FA_ERR_INVALID_ARG;
  const size_t qb = qelems * 2, kb = kelems * 2, lb = (size_t)B * H * Nq * sizeof(float);
  const Span ins[3] = {span(q, qb), span(k, kb), span(v, kb)};
  const void* inp[3] = {q, k, v};
  const Span outs[3] = {span(o, qb), span(lse, lb), span(workspace, need)};
  const void* outp[3] = {o, lse, workspace};
  st = check_buffers(ins, inp, 3, outs, outp, 3);
  if (st != FA_OK) return st;
  return hip_status(fa::launch_decode_bf16(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                           static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), lse,
                                           B * H, Nq, Nk, d, causal != 0, scale, workspace,
                                           static_cast<hipStream_t>(stream)), stream);
}

size_t fa_fp8_buffer_size(int B, int H, int N, int d) {
  if (B <= 0 || H <= 0 || N <= 0 || d != 128) return 0;
  const unsigned long long bh = (unsigned long long)B * (unsigned long long)H;
  if (bh > 0x7fffffffULL) return 0;
  return fa::fp8_buffer_layout((long long)bh, N).bytes;
}

int fa_fp8_prepare(const void* q, const void* k, const void* v, const float* signs, int B, int H, int N, int d,
                   void* buf, size_t buf_bytes, void* stream) {
  size_t elems = 0;
  int st = check_common(B, H, N, d, 0, 1.0f, true, &elems);
  if (st != FA_OK) return st;
  if (d != 128) return FA_ERR_UNSUPPORTED;
  const size_t need = fa_fp8_buffer_size(B, H, N, d);
  if (need == 0 || buf_bytes < need) return FA_ERR_INVALID_ARG;
  const size_t tb = elems * 2;
  Span ins[4] = {span(q, tb), span(k, tb), span(v, tb), span(signs, 128 * sizeof(float))};
  const void* inp[4] = {q, k, v, signs};
  const Span outs[1] = {span(buf, need)};
  const void* outp[1] = {buf};
  st = check_buffers(ins, inp, signs != nullptr ? 4 : 3, outs, outp, 1);
  if (st != FA_OK) return st;
  return hip_status(fa::launch_fp8_prepare(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                           static_cast<const uint16_t*>(v), signs, B * H, N, buf,
                                           static_cast<hipStream_t>(stream)), stream);
}

int fa_forward_fp8_prepared(const void* buf, size_t buf_bytes, void* o, float* lse, int B, int H, int N, int d,
                            int causal, float scale, int rotated, void* stream) {
  size_t elems = 0;
  int st = check_common(B, H, N, d, causal, scale, true, &elems);
  if (st != FA_OK) return st;
  if (d != 128) return FA_ERR_UNSUPPORTED;
  if (rotated != 0 && rotated != 1) return FA_ERR_INVALID_ARG;
  const size_t need = fa_fp8_buffer_size(B, H, N, d);
  if (need == 0 || buf_bytes < need) return FA_ERR_INVALID_ARG;
  const Span ins[1] = {span(buf, need)};
  const void* inp[1] = {buf};
  const Span outs[2] = {span(o, elems * 2), span(lse, (size_t)B * H * N * sizeof(float))};
  const void* outp[2] = {o, lse};
  st = check_buffers(ins, inp, 1, outs, outp, 2);
  if (st != FA_OK) return st;
  return hip_status(fa::launch_fwd_fp8(buf, static_cast<uint16_t*>(o), lse, B * H, N, causal != 0, scale,
                                       rotated != 0, static_cast<hipStream_t>(stream)), stream);
}

int fa_forward_fp8(const void* q, const void* k, const void* v, const float* signs, void* o, float* lse, int B,
                   int H, int N, int d, int causal, float scale, void* buf, size_t buf_bytes, void* stream) {
  size_t elems = 0;
  int st = check_common(B, H, N, d, causal, scale, true, &elems);
  if (st != FA_OK) return st;
  if (d != 128) return FA_ERR_UNSUPPORTED;
  const size_t need = fa_fp8_buffer_size(B, H, N, d);
  if (need == 0 || buf_bytes < need) return FA_ERR_INVALID_ARG;
  const size_t tb = elems * 2;
  Span ins[4] = {span(q, tb), span(k, tb), span(v, tb), span(signs, 128 * sizeof(float))};
  const void* inp[4] = {q, k, v, signs};
  const Span outs[3] = {span(o, tb), span(lse, (size_t)B * H * N * sizeof(float)), span(buf, need)};
  const void* outp[3] = {o, lse, buf};
  st = check_buffers(ins, inp, signs != nullptr ? 4 : 3, outs, outp, 3);
  if (st != FA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = fa::launch_fp8_prepare(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                              static_cast<const uint16_t*>(v), signs, B * H, N, buf, s);
  if (e != hipSuccess) return FA_ERR_HIP;
  return hip_status(fa::launch_fwd_fp8(buf, static_cast<uint16_t*>(o), lse, B * H, N, causal != 0, scale,
                                       signs != nullptr, s), stream);
}

size_t fa_backward_atomic_workspace_size(int B, int H, int N, int d) {
  const size_t rows_bytes = fa_backward_workspace_size(B, H, N, d);
  if (rows_bytes == 0) return 0;
  return rows_bytes + (size_t)B * (size_t)H * (size_t)N * (size_t)d * sizeof(float);
}

int fa_backward_atomic(const void* q, const void* k, const void* v, const void* o, const float* lse,
                       const void* dO, void* dq, void* dk, void* dv, int B, int H, int N, int d, int causal,
                       float scale, void* workspace, size_t workspace_bytes, void* stream) {
  size_t elems = 0;
  int st = check_common(B, H, N, d, causal, scale, true, &elems);
  if (st != FA_OK) return st;
  const size_t need = fa_backward_atomic_workspace_size(B, H, N, d);
  if (workspace_bytes < need) return FA_ERR_INVALID_ARG;
  const size_t tb = elems * 2, lb = (size_t)B * H * N * sizeof(float);
  const Span ins[6] = {span(q, tb), span(k, tb), span(v, tb), span(o, tb), span(lse, lb), span(dO, tb)};
  const void* inp[6] = {q, k, v, o, lse, dO};
  const Span outs[4] = {span(dq, tb), span(dk, tb), span(dv, tb), span(workspace, need)};
  const void* outp[4] = {dq, dk, dv, workspace};
  st = check_buffers(ins, inp, 6, outs, outp, 4);
  if (st != FA_OK) return st;
  float* delta = static_cast<float*>(workspace);
  float* dqacc = reinterpret_cast<float*>(static_cast<char*>(workspace) + fa_backward_workspace_size(B, H, N, d));
  return hip_status(fa::launch_bwd_single_pass_bf16(
                        static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                        static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(o), lse,
                        static_cast<const uint16_t*>(dO), static_cast<uint16_t*>(dq), static_cast<uint16_t*>(dk),
                        static_cast<uint16_t*>(dv), B * H, N, d, causal != 0, scale, delta, dqacc,
                        static_cast<hipStream_t>(stream)),
                    stream);
}

int fa_forward_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H,
                   int N, int d, int causal, float scale, void* stream) {
  return forward_impl(q, k, v, o, lse, B, H, N, d, causal, scale, stream, false);
}

int fa_backward(const void* q, const void* k, const void* v, const void* o, const float* lse,
                const void* dO, void* dq, void* dk, void* dv, int B, int H, int N, int d, int causal,
                float scale, void* workspace, size_t workspace_bytes, void* stream) {
  return backward_impl(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                       static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(o), lse,
                       static_cast<const uint16_t*>(dO), static_cast<uint16_t*>(dq),
                       static_cast<uint16_t*>(dk), static_cast<uint16_t*>(dv), B, H, N, d, causal,
                       scale, workspace, workspace_bytes, stream, true);
}

int fa_backward_f32(const float* q, const float* k, const float* v, const float* o, const float* lse,
                    const float* dO, float* dq, float* dk, float* dv, int B, int H, int N, int d,
                    int causal, float scale, void* workspace, size_t workspace_bytes, void* stream) {
  return backward_impl(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, causal, scale, workspace,
                       workspace_bytes, stream, false);
}

}  // extern "C"
