// Internal (non-exported) interface between the C-ABI entry points and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace fa {

// Compute units of the current device (queried once per device; 0 if the query fails).
inline int cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// One forward launch. Dense: B batches of N tokens. Varlen: B = number of sequences,
// N = max_seqlen, T = total tokens, cu = device cu_seqlens.
struct FwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  const int32_t* cu;
  int B, N, H, T;
  float scale_log2;  // |softmax_scale| * log2(e)
  uint32_t qsign;    // 0x80008000 flips the sign of q (negative softmax_scale), else 0
};

// One backward launch (dense or varlen, same conventions as FwdArgs).
struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const float* lse;
  const uint16_t* dout;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* neg_delta;  // workspace: -D_i = -<dO_i, O_i>, fp32, same layout as lse
  float* neg_lse2;   // workspace: -LSE_i * log2(e), fp32, same layout as lse
  const int32_t* cu;
  int B, N, H, T;
  float scale;       // softmax_scale (signed)
  float scale_log2;  // |softmax_scale| * log2(e)
  uint32_t qsign;
};

// One FP8 forward launch (dense). q, k, v: e4m3 codes [B, N, H, d]; o: bf16; lse: fp32.
struct Fp8FwdArgs {
  const uint8_t* q;
  const uint8_t* k;
  const uint8_t* v;
  uint16_t* o;
  float* lse;
  int B, N, H;
  float scale_log2;  // |softmax_scale| * q_descale * k_descale * log2(e)
  uint32_t qsign;    // 0x80808080 flips the sign of q (negative softmax_scale), else 0
  float v_descale;
};

// One merge of a partial result into a running one (same rows, disjoint key sets).
struct MergeArgs {
  float* o_acc;            // fp32 [B, N, H, d], in/out
  float* lse_acc;          // fp32 [B, H, N], in/out
  const uint16_t* o_part;  // [B, N, H, d], element type
  const float* lse_part;   // fp32 [B, H, N]
  uint16_t* out;           // [B, N, H, d], element type, or null
  int B, N, H;
};
__attribute__((visibility("hidden"))) hipError_t launch_merge(const MergeArgs& a, int d,
                                                              bool bf16, hipStream_t stream);

__attribute__((visibility("hidden"))) hipError_t launch_fwd_fp8(const Fp8FwdArgs& a, int d,
                                                                bool causal,
                                                                hipStream_t stream);
__attribute__((visibility("hidden"))) hipError_t launch_fwd(const FwdArgs& a, int d, bool bf16,
                                                            bool causal, bool varlen,
                                                            hipStream_t stream);
// Backward stages: row terms, dK/dV, dQ, or all three in that order.
enum { kBwdPrep = 0, kBwdDkDv = 1, kBwdDq = 2, kBwdAll = 3 };
__attribute__((visibility("hidden"))) hipError_t launch_bwd(const BwdArgs& a, int d, bool bf16,
                                                            bool causal, bool varlen, int stage,
                                                            hipStream_t stream);

// Scratch array of the allocation-free entry points (fa_scratch.hip): its size, and the
// device address of the current device's copy (looked up on the first call per device).
constexpr size_t kScratchBytes = (size_t)8 << 20;
__attribute__((visibility("hidden"))) hipError_t scratch_buffer(void** out);

}  // namespace fa
