// Merge of a partial attention result into a running one (the per-device step of ring
// attention: "FlashAttention 与算子融合" lists ring attention, K/V blocks passed around a ring
// of devices with FlashAttention as the compute core, in its 代际演进 table and 工程实践
// section). Each device holds its query rows and, at every step of the ring, attends them to
// one K/V shard; the partial results over disjoint key sets are combined with the block-merge
// rule of the same page (section FlashAttention 的两个关键). For parts given as a normalised
// output and its log-sum-exp the rule reads
//   lse = ln(e^lse_acc + e^lse_part),
//   o   = o_acc e^(lse_acc - lse) + o_part e^(lse_part - lse).
// The running output is kept in fp32 so that many merges add no rounding of their own.
//
// Elementwise and HBM-bound: d/4 lanes per row (one wave holds whole rows), each lane updates
// four elements; every lane of a row computes the merged lse from the two row values, and
// the row's first lane writes it back after the row's loads (same wave, program order).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

template <int D, class T>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  constexpr int LPR = D / 4;            // lanes per row
  constexpr int RPB = 256 / LPR;        // rows per workgroup
  const long rows = (long)a.B * a.N * a.H;
  const long row = (long)blockIdx.x * RPB + threadIdx.x / LPR;
  if (row >= rows) return;
  const int c4 = (threadIdx.x % LPR) * 4;  // first of this lane's four elements
  const long h = row % a.H;
  const long bn = row / a.H;              // b * N + n
  const long n = bn % a.N, b = bn / a.N;
  const long li = (b * a.H + h) * a.N + n;
  const float la = a.lse_acc[li], lp = a.lse_part[li];
  const float mx = fmaxf(la, lp);
  float lse, wa, wp;
  if (mx == -__builtin_inff()) {  // neither part saw a key
    lse = mx;
    wa = wp = 0.f;
  } else {
    const float ea = expf(la - mx), ep = expf(lp - mx);  // one of them is 1
    lse = mx + logf(ea + ep);
    wa = ea / (ea + ep);
    wp = ep / (ea + ep);
  }
  const long e0 = row * D + c4;
  f32x4 acc = *reinterpret_cast<const f32x4*>(a.o_acc + e0);
  const u32x2 pbits = *reinterpret_cast<const u32x2*>(a.o_part + e0);
  const float p0 = to_f32<T>(pbits[0] & 0xffffu), p1 = to_f32<T>(pbits[0] >> 16);
  const float p2 = to_f32<T>(pbits[1] & 0xffffu), p3 = to_f32<T>(pbits[1] >> 16);
  // a part with weight 0 contributes nothing, whatever its (possibly non-finite) values
  acc[0] = (wa > 0.f ? wa * acc[0] : 0.f) + (wp > 0.f ? wp * p0 : 0.f);
  acc[1] = (wa > 0.f ? wa * acc[1] : 0.f) + (wp > 0.f ? wp * p1 : 0.f);
  acc[2] = (wa > 0.f ? wa * acc[2] : 0.f) + (wp > 0.f ? wp * p2 : 0.f);
  acc[3] = (wa > 0.f ? wa * acc[3] : 0.f) + (wp > 0.f ? wp * p3 : 0.f);
  *reinterpret_cast<f32x4*>(a.o_acc + e0) = acc;
  if (a.out != nullptr)
    *reinterpret_cast<u32x2*>(a.out + e0) = u32x2{pack2<T>(acc[0], acc[1]),
                                                  pack2<T>(acc[2], acc[3])};
  if (c4 == 0) a.lse_acc[li] = lse;
}

template <int D, class T>
hipError_t launch(const MergeArgs& a, hipStream_t st) {
  constexpr int RPB = 256 / (D / 4);
  const long rows = (long)a.B * a.N * a.H;
  const long blocks = (rows + RPB - 1) / RPB;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((merge_kernel<D, T>), dim3((unsigned)blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, int d, bool bf16, hipStream_t st) {
  if (d == 128) return bf16 ? launch<128, BF16>(a, st) : launch<128, F16>(a, st);
  return bf16 ? launch<64, BF16>(a, st) : launch<64, F16>(a, st);
}

}  // namespace fa
