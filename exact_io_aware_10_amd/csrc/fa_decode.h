// Internal interface of the split-KV decode forward (fa_decode.hip) for the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// One split-KV launch. q, o: [B, Nq, H, d]; k, v: [B, Nk, H, d]; lse: fp32 [B, H, Nq].
// The keys are cut into S ranges of `span` keys (a multiple of 32; trailing ranges may be
// empty). Per (b, h, split, query row) the first kernel writes, in fp32:
//   opart [B, H, S, Nq, d] : sum over the range of exp2(c s_j - mpart) v_j (c = |scale| log2 e,
//                            P rounded to the element type as in the forward)
//   mpart [B, H, S, Nq]    : the reference maximum of c s_j (-inf if the range sees no key)
//   lpart [B, H, S, Nq]    : sum over the range of the rounded exp2(c s_j - mpart)
// and the second merges the S parts of each row into o and lse.
struct DecodeArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  float* opart;
  float* mpart;
  float* lpart;
  int B, Nq, Nk, H, S, span;
  float scale_log2;  // |softmax_scale| * log2(e)
  uint32_t qsign;    // 0x80008000 flips the sign of q (negative softmax_scale), else 0
};

// Number of key ranges for a request of `requested` (0: chosen here from the shape so that
// the grid fills the GPU), and the keys per range.
int decode_splits(int B, int Nq, int Nk, int H, int d, int requested);
int decode_span(int Nk, int splits);

__attribute__((visibility("hidden"))) hipError_t launch_decode(const DecodeArgs& a, int d,
                                                               bool bf16, bool causal,
                                                               hipStream_t stream);

}  // namespace fa
