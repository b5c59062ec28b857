// C-ABI entry points of libfa_mi355x.so: synchronous argument checks, then kernel
// launches on the caller's stream. Declarations and contracts: include/fa.h.
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#include <vector>

#include "fa.h"
#include "fa_decode.h"
#include "fa_internal.h"

#define FA_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

constexpr float kLog2e = 1.44269504088896340736f;
// (N + 256) * H * d limit: byte offsets of every row a kernel touches, including the
// padded rows of a ragged last tile, fit in 31 bits.
constexpr long kMaxSliceElems = 1L << 30;

// Exponent scale |softmax_scale| * log2(e), kept >= the smallest normal float so that it
// is strictly positive: masked scores (-inf) then give exp2(-inf) = 0 with no select, and
// a zero softmax_scale still gives uniform weights (exp2 of products below 2^-100 is
// exactly 1.0 in fp32).
float exp_scale(float softmax_scale) { return fmaxf(fabsf(softmax_scale) * kLog2e, FLT_MIN); }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool dtype_ok(int dt) { return dt == FA_F16 || dt == FA_BF16; }

fa_status to_status(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }

// FA_DEBUG set to anything but "" or "0" turns on the checks that need a device-to-host
// copy. Read at every call, so a process can switch it.
bool debug_checks() {
  const char* e = getenv("FA_DEBUG");
  return e != nullptr && e[0] != '\0' && !(e[0] == '0' && e[1] == '\0');
}

// Debug check of a packed batch's offsets: copies cu_seqlens to the host on the caller's
// stream (waiting for the stream) and accepts it only if cu[0] = 0, it never decreases and
// cu[num_seqs] = total_tokens. Lengths above max_seqlen are allowed (they are truncated).
fa_status check_cu_seqlens(const int32_t* cu, int num_seqs, int total_tokens,
                           hipStream_t stream) {
  std::vector<int32_t> h((size_t)num_seqs + 1);
  if (hipMemcpyAsync(h.data(), cu, h.size() * sizeof(int32_t), hipMemcpyDeviceToHost,
                     stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess) {
    (void)hipGetLastError();
    return FA_ERR_INVALID_ARG;
  }
  if (h[0] != 0 || h[num_seqs] != total_tokens) return FA_ERR_INVALID_ARG;
  for (int s = 0; s < num_seqs; ++s)
    if (h[s + 1] < h[s]) return FA_ERR_INVALID_ARG;
  return FA_OK;
}

// Shared checks of the scalar arguments. Returns FA_OK when the request is valid.
fa_status check_common(long B, long N, long H, int d, int dt, float scale) {
  if (B < 0 || N < 0 || H < 0) return FA_ERR_INVALID_ARG;
  if (!dtype_ok(dt) || !isfinite(scale)) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if ((N + 256) * H * d >= kMaxSliceElems) return FA_ERR_UNSUPPORTED;
  // workgroups of the largest launch (128-row blocks; packed launches round B·H up to 8)
  if ((B * H + 7) / 8 * 8 * ((N + 127) / 128) >= (1L << 31)) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

// Dense calls index their row terms by token (B * N of them) in 32-bit ints.
bool tokens_ok(long B, long N) { return B * N <= INT32_MAX; }

bool tensors_ok(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (p == nullptr || !aligned16(p)) return false;
  return true;
}

}  // namespace

FA_EXPORT const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_INVALID_ARG: return "invalid argument";
    case FA_ERR_UNSUPPORTED: return "unsupported configuration";
    case FA_ERR_HIP: return "HIP launch error";
  }
  return "unknown status";
}

FA_EXPORT fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int N, int H, int d, int dtype, float softmax_scale,
                           int causal, hipStream_t stream) {
  fa_status st = check_common(B, N, H, d, dtype, softmax_scale);
  if (st != FA_OK) return st;
  if (!tokens_ok(B, N)) return FA_ERR_UNSUPPORTED;
  if ((long)B * N * H == 0) return FA_OK;
  if (!tensors_ok({q, k, v, o}) || lse == nullptr || ((uintptr_t)lse & 3u))
    return FA_ERR_INVALID_ARG;
  fa::FwdArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<uint16_t*>(o);
  a.lse = lse;
  a.cu = nullptr;
  a.B = B;
  a.N = N;
  a.H = H;
  a.T = B * N;
  a.scale_log2 = exp_scale(softmax_scale);
  a.qsign = softmax_scale < 0.f ? 0x80008000u : 0u;
  return to_status(fa::launch_fwd(a, d, dtype == FA_BF16, causal != 0, false, stream));
}

FA_EXPORT fa_status fa_fwd_fp8(const void* q, const void* k, const void* v, void* o,
                               float* lse, int B, int N, int H, int d, float q_descale,
                               float k_descale, float v_descale, float softmax_scale,
                               int causal, hipStream_t stream) {
  // the size limits of the 16-bit path are kept (they bound element counts, so they also
  // cover the one-byte rows)
  fa_status st = check_common(B, N, H, d, FA_BF16, softmax_scale);
  if (st != FA_OK) return st;
  for (float x : {q_descale, k_descale, v_descale})
    if (!(isfinite(x) && x > 0.f)) return FA_ERR_INVALID_ARG;
  const float c = fabsf(softmax_scale) * q_descale * k_descale * kLog2e;
  if (!isfinite(c)) return FA_ERR_INVALID_ARG;
  if ((long)B * N * H == 0) return FA_OK;
  if (!tensors_ok({q, k, v, o}) || lse == nullptr || ((uintptr_t)lse & 3u))
    return FA_ERR_INVALID_ARG;
  fa::Fp8FwdArgs a{};
  a.q = static_cast<const uint8_t*>(q);
  a.k = static_cast<const uint8_t*>(k);
  a.v = static_cast<const uint8_t*>(v);
  a.o = static_cast<uint16_t*>(o);
  a.lse = lse;
  a.B = B;
  a.N = N;
  a.H = H;
  a.scale_log2 = fmaxf(c, FLT_MIN);
  a.qsign = softmax_scale < 0.f ? 0x80808080u : 0u;
  a.v_descale = v_descale;
  return to_status(fa::launch_fwd_fp8(a, d, causal != 0, stream));
}

FA_EXPORT fa_status fa_merge(float* o_acc, float* lse_acc, const void* o_part,
                             const float* lse_part, void* out, int B, int N, int H, int d,
                             int dtype, hipStream_t stream) {
  fa_status st = check_common(B, N, H, d, dtype, 1.0f);
  if (st != FA_OK) return st;
  // workgroups of the merge: B·N·H rows, at least 8 per workgroup, below 2^31
  if ((long)B * N * H >= (1L << 34)) return FA_ERR_UNSUPPORTED;
  if ((long)B * N * H == 0) return FA_OK;
  if (!tensors_ok({o_acc, o_part}) || (out != nullptr && !aligned16(out)) ||
      lse_acc == nullptr || lse_part == nullptr || ((uintptr_t)lse_acc & 3u) ||
      ((uintptr_t)lse_part & 3u))
    return FA_ERR_INVALID_ARG;
  fa::MergeArgs a{};
  a.o_acc = o_acc;
  a.lse_acc = lse_acc;
  a.o_part = static_cast<const uint16_t*>(o_part);
  a.lse_part = lse_part;
  a.out = static_cast<uint16_t*>(out);
  a.B = B;
  a.N = N;
  a.H = H;
  return to_status(fa::launch_merge(a, d, dtype == FA_BF16, stream));
}

FA_EXPORT size_t fa_bwd_workspace_size(int B, int N, int H, int d) {
  if (B < 0 || N < 0 || H < 0 || (d != 64 && d != 128)) return 0;
  return (size_t)8 * B * H * N;
}

namespace {

fa_status bwd_common(const void* q, const void* k, const void* v, const void* o,
                     const float* lse, const void* dout, void* dq, void* dk, void* dv,
                     void* workspace, int B, int N, int H, int d, int dtype,
                     float softmax_scale, int causal, int stage, hipStream_t stream) {
  fa_status st = check_common(B, N, H, d, dtype, softmax_scale);
  if (st != FA_OK) return st;
  if (!tokens_ok(B, N)) return FA_ERR_UNSUPPORTED;
  if ((long)B * N * H == 0) return FA_OK;
  if (!tensors_ok({q, k, v, o, dout, dq, dk, dv, workspace}) || lse == nullptr ||
      ((uintptr_t)lse & 3u))
    return FA_ERR_INVALID_ARG;
  fa::BwdArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<const uint16_t*>(o);
  a.lse = lse;
  a.dout = static_cast<const uint16_t*>(dout);
  a.dq = static_cast<uint16_t*>(dq);
  a.dk = static_cast<uint16_t*>(dk);
  a.dv = static_cast<uint16_t*>(dv);
  a.neg_delta = static_cast<float*>(workspace);
  a.neg_lse2 = a.neg_delta + (long)B * H * N;
  a.cu = nullptr;
  a.B = B;
  a.N = N;
  a.H = H;
  a.T = B * N;
  a.scale = softmax_scale;
  a.scale_log2 = exp_scale(softmax_scale);
  a.qsign = softmax_scale < 0.f ? 0x80008000u : 0u;
  return to_status(fa::launch_bwd(a, d, dtype == FA_BF16, causal != 0, false, stage, stream));
}

}  // namespace

#define FA_BWD_ENTRY(name, stage)                                                          \
  FA_EXPORT fa_status name(const void* q, const void* k, const void* v, const void* o,    \
                           const float* lse, const void* dout, void* dq, void* dk,        \
                           void* dv, void* workspace, int B, int N, int H, int d,         \
                           int dtype, float softmax_scale, int causal,               \
                           hipStream_t stream) {                                          \
    return bwd_common(q, k, v, o, lse, dout, dq, dk, dv, workspace, B, N, H, d, dtype,    \
                      softmax_scale, causal, stage, stream);                              \
  }

FA_BWD_ENTRY(fa_bwd, fa::kBwdAll)
FA_BWD_ENTRY(fa_bwd_prep, fa::kBwdPrep)
FA_BWD_ENTRY(fa_bwd_dkdv, fa::kBwdDkDv)
FA_BWD_ENTRY(fa_bwd_dq, fa::kBwdDq)

FA_EXPORT fa_status fa_fwd_varlen(const void* q, const void* k, const void* v, void* o,
                                  float* lse, const int32_t* cu_seqlens, int num_seqs,
                                  int total_tokens, int max_seqlen, int H, int d,
                                  int dtype, float softmax_scale, int causal,
                                  hipStream_t stream) {
  if (num_seqs < 0 || total_tokens < 0 || max_seqlen < 0) return FA_ERR_INVALID_ARG;
  fa_status st = check_common(num_seqs, max_seqlen, H, d, dtype, softmax_scale);
  if (st != FA_OK) return st;
  if (cu_seqlens == nullptr || ((uintptr_t)cu_seqlens & 3u)) return FA_ERR_INVALID_ARG;
  if ((long)num_seqs * max_seqlen * H == 0 || total_tokens == 0) return FA_OK;
  if (!tensors_ok({q, k, v, o}) || lse == nullptr || ((uintptr_t)lse & 3u))
    return FA_ERR_INVALID_ARG;
  if (debug_checks() &&
      (st = check_cu_seqlens(cu_seqlens, num_seqs, total_tokens, stream)) != FA_OK)
    return st;
  fa::FwdArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<uint16_t*>(o);
  a.lse = lse;
  a.cu = cu_seqlens;
  a.B = num_seqs;
  a.N = max_seqlen;
  a.H = H;
  a.T = total_tokens;
  a.scale_log2 = exp_scale(softmax_scale);
  a.qsign = softmax_scale < 0.f ? 0x80008000u : 0u;
  return to_status(fa::launch_fwd(a, d, dtype == FA_BF16, causal != 0, true, stream));
}

FA_EXPORT fa_status fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o,
                                  const float* lse, const void* dout, void* dq, void* dk,
                                  void* dv, void* workspace, const int32_t* cu_seqlens,
                                  int num_seqs, int total_tokens, int max_seqlen, int H, int d,
                                  int dtype, float softmax_scale, int causal,
                                  hipStream_t stream) {
  if (num_seqs < 0 || total_tokens < 0 || max_seqlen < 0) return FA_ERR_INVALID_ARG;
  fa_status st = check_common(num_seqs, max_seqlen, H, d, dtype, softmax_scale);
  if (st != FA_OK) return st;
  if (cu_seqlens == nullptr || ((uintptr_t)cu_seqlens & 3u)) return FA_ERR_INVALID_ARG;
  if ((long)num_seqs * max_seqlen * H == 0 || total_tokens == 0) return FA_OK;
  if (!tensors_ok({q, k, v, o, dout, dq, dk, dv, workspace}) || lse == nullptr ||
      ((uintptr_t)lse & 3u))
    return FA_ERR_INVALID_ARG;
  if (debug_checks() &&
      (st = check_cu_seqlens(cu_seqlens, num_seqs, total_tokens, stream)) != FA_OK)
    return st;
  fa::BwdArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<const uint16_t*>(o);
  a.lse = lse;
  a.dout = static_cast<const uint16_t*>(dout);
  a.dq = static_cast<uint16_t*>(dq);
  a.dk = static_cast<uint16_t*>(dk);
  a.dv = static_cast<uint16_t*>(dv);
  a.neg_delta = static_cast<float*>(workspace);
  a.neg_lse2 = a.neg_delta + (long)H * total_tokens;
  a.cu = cu_seqlens;
  a.B = num_seqs;
  a.N = max_seqlen;
  a.H = H;
  a.T = total_tokens;
  a.scale = softmax_scale;
  a.scale_log2 = exp_scale(softmax_scale);
  a.qsign = softmax_scale < 0.f ? 0x80008000u : 0u;
  return to_status(fa::launch_bwd(a, d, dtype == FA_BF16, causal != 0, true, fa::kBwdAll,
                                  stream));
}

namespace {

constexpr int kMaxSplits = 4096;

// Valid split-KV sizes: 0 when the request is fine, else the status to return.
fa_status splitkv_sizes(long B, long Nq, long Nk, long H, int d, int num_splits) {
  if (B < 0 || Nq < 0 || H < 0 || Nk < 1 || num_splits < 0 || num_splits > kMaxSplits)
    return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if ((Nk + 256) * H * d >= kMaxSliceElems || (Nq + 256) * H * d >= kMaxSliceElems)
    return FA_ERR_UNSUPPORTED;
  // workgroups of the launches: at most B·H·S·ceil(Nq / 32) for the partials (S key ranges)
  // and B·H·Nq for the merge, each below 2^31
  const long S = fa::decode_splits((int)B, (int)Nq, (int)Nk, (int)H, d, num_splits);
  if (B * H * S * ((Nq + 31) / 32) >= (1L << 31) || B * H * Nq >= (1L << 31))
    return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

}  // namespace

FA_EXPORT size_t fa_fwd_splitkv_workspace_size(int B, int Nq, int Nk, int H, int d,
                                               int num_splits) {
  if (splitkv_sizes(B, Nq, Nk, H, d, num_splits) != FA_OK) return 0;
  const long S = fa::decode_splits(B, Nq, Nk, H, d, num_splits);
  const long rows = (long)B * H * S * Nq;
  // partial outputs (rows x d), then the reference maxima and the sums (rows each)
  return (size_t)rows * (d + 2) * 4;
}

namespace {

// The checks and the launch of fa_fwd_splitkv; workspace is resolved by get_ws only after
// every argument check has passed.
template <class GetWs>
fa_status splitkv_impl(const void* q, const void* k, const void* v, void* o, float* lse,
                       GetWs get_ws, int B, int Nq, int Nk, int H, int d, int dtype,
                       float softmax_scale, int causal, int num_splits, hipStream_t stream) {
  fa_status st = splitkv_sizes(B, Nq, Nk, H, d, num_splits);
  if (st != FA_OK) return st;
  if (!dtype_ok(dtype) || !isfinite(softmax_scale)) return FA_ERR_INVALID_ARG;
  if ((long)B * Nq * H == 0) return FA_OK;
  if (!tensors_ok({q, k, v, o}) || lse == nullptr || ((uintptr_t)lse & 3u))
    return FA_ERR_INVALID_ARG;
  void* workspace = nullptr;
  if ((st = get_ws(&workspace)) != FA_OK) return st;
  if (!tensors_ok({workspace})) return FA_ERR_INVALID_ARG;
  fa::DecodeArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<uint16_t*>(o);
  a.lse = lse;
  a.B = B;
  a.Nq = Nq;
  a.Nk = Nk;
  a.H = H;
  a.S = fa::decode_splits(B, Nq, Nk, H, d, num_splits);
  a.span = fa::decode_span(Nk, a.S);
  const long rows = (long)B * H * a.S * Nq;
  a.opart = static_cast<float*>(workspace);
  a.mpart = a.opart + rows * d;
  a.lpart = a.mpart + rows;
  a.scale_log2 = exp_scale(softmax_scale);
  a.qsign = softmax_scale < 0.f ? 0x80008000u : 0u;
  return to_status(fa::launch_decode(a, d, dtype == FA_BF16, causal != 0, stream));
}

}  // namespace

FA_EXPORT fa_status fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o,
                                   float* lse, void* workspace, int B, int Nq, int Nk, int H,
                                   int d, int dtype, float softmax_scale, int causal,
                                   int num_splits, hipStream_t stream) {
  auto ws = [workspace](void** out) {
    *out = workspace;
    return FA_OK;
  };
  return splitkv_impl(q, k, v, o, lse, ws, B, Nq, Nk, H, d, dtype, softmax_scale, causal,
                      num_splits, stream);
}

FA_EXPORT size_t fa_noalloc_scratch_bytes(void) { return fa::kScratchBytes; }

FA_EXPORT fa_status fa_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o,
                                           float* lse, int B, int Nq, int Nk, int H, int d,
                                           int dtype, float softmax_scale, int causal,
                                           int num_splits, hipStream_t stream) {
  auto ws = [=](void** out) {
    // the partials must fit the library's scratch array (this check follows the argument
    // checks, so the size is well defined here)
    if (fa_fwd_splitkv_workspace_size(B, Nq, Nk, H, d, num_splits) > fa::kScratchBytes)
      return FA_ERR_UNSUPPORTED;
    return fa::scratch_buffer(out) == hipSuccess ? FA_OK : FA_ERR_HIP;
  };
  return splitkv_impl(q, k, v, o, lse, ws, B, Nq, Nk, H, d, dtype, softmax_scale, causal,
                      num_splits, stream);
}
