// Backward attention kernels for gfx950: P is recomputed tile by tile from Q, K and the
// forward's per-row log-sum-exp instead of being stored ("FlashAttention 短片讲解稿",
// segment 第三招 · 反向重计算: keep the inputs, the output and a few row statistics, and
// recompute the needed block in the backward pass).
//
// The gradient formulas are the chain rule through O = softmax(scale Q K^T) V
// ("FlashAttention 详解（零基础入门）" §2.3-§2.6):
//   P_ij = exp(scale <q_i,k_j> - LSE_i)          (exact softmax, LSE is final)
//   D_i  = <dO_i, O_i>                             (= sum_j P_ij dP_ij)
//   dV_j = sum_i P_ij dO_i,  dP_ij = <dO_i, v_j>,  dS_ij = P_ij (dP_ij - D_i)
//   dQ_i = scale sum_j dS_ij k_j,                  dK_j = scale sum_i dS_ij q_i
//
// Three launches, no floating-point atomics (bitwise deterministic):
//   1. bwd_prep_kernel : per row, -D_i and -LSE_i log2(e) into the workspace.
//   2. bwd_dkdv_kernel : one workgroup of 8 waves per 128-key block; wave (kg, qh) owns 32
//                        keys (K in registers, V of the block in LDS) and one 32-query half
//                        of each 64-query tile of Q, dO and the two row terms, streamed from
//                        HBM/L2 straight into LDS, double buffered. S = Q K^T and dP = dO V^T
//                        are computed with lanes <-> keys, so P and dS leave the accumulators
//                        in the B-operand layout of dV^T += dO^T P and dK^T += Q^T dS; the two
//                        halves' partial dK, dV are summed through LDS at the end.
//   3. bwd_dq_kernel   : one workgroup of 8 waves per 256-query block (32 queries per wave;
//                        Q and dO in registers); streams 64-key tiles of K and V; S^T and
//                        dP^T with lanes <-> queries feed dQ^T += K^T dS^T.
// Under the causal mask both gradient kernels run the tiles that can meet the diagonal
// through a masked copy of their step and all others through the branch-free one.
// Each streamed tile is stored once, row-major, and read both as row fragments
// (ds_read_b128: operand rows = tile rows) and as transposed fragments
// (ds_read_b64_tr_b16: operand rows = tile columns; in each group of 16 lanes, lane i names
// 4 consecutive values and lane j receives column j%4 of rows j/4 + 4k, k = 0..3). The
// 16-byte chunks of row r are XOR-swizzled by f(r) = ((r&3)<<2)|((r>>2)&3) (d = 128), which
// makes both read patterns conflict-free.
// -D is loaded as the initial value of the dP accumulators, so dS = P * acc.
#include "fa_bwd_common.h"

namespace fa {
namespace bwd {
namespace {

// ---------------------------------------------------------------- 1. row terms
// ws[0 .. rows) = -D_i = -<dO_i, O_i>;  ws[rows .. 2 rows) = -LSE_i * log2(e)
template <int D, class T>
__global__ __launch_bounds__(kThreads) void bwd_prep_kernel(BwdArgs a, long rows) {
  constexpr int TPR = D / 8;  // threads per row, 8 elements each
  const long row = (long)blockIdx.x * (kThreads / TPR) + threadIdx.x / TPR;
  const int c = threadIdx.x % TPR;
  float acc = 0.f;
  const bool ok = row < rows;
  if (ok) {
    const u32x4 x = *reinterpret_cast<const u32x4*>(a.o + row * D + 8 * c);
    const u32x4 y = *reinterpret_cast<const u32x4*>(a.dout + row * D + 8 * c);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc += to_f32<T>(x[e] & 0xffffu) * to_f32<T>(y[e] & 0xffffu);
      acc += to_f32<T>(x[e] >> 16) * to_f32<T>(y[e] >> 16);
    }
  }
#pragma unroll
  for (int m = 1; m < TPR; m <<= 1) acc += __shfl_xor(acc, m, TPR);
  if (ok && c == 0) {
    // row = token * H + h  ->  stats layout
    const long tok = row / a.H;
    const int h = row % a.H;
    long idx;
    if (a.cu == nullptr) {
      const long b = tok / a.N, n = tok % a.N;
      idx = (b * a.H + h) * a.N + n;
    } else {
      idx = (long)h * a.T + tok;
    }
    a.neg_delta[idx] = -acc;
    a.neg_lse2[idx] = -a.lse[idx] * kLog2e;
  }
}

template <int D, class T>
hipError_t launch_prep(const BwdArgs& a, hipStream_t st) {
  const long rows = (long)a.T * a.H;
  constexpr int rows_per_block = kThreads / (D / 8);
  hipLaunchKernelGGL((bwd_prep_kernel<D, T>),
                     dim3((unsigned)((rows + rows_per_block - 1) / rows_per_block)),
                     dim3(kThreads), 0, st, a, rows);
  return hipGetLastError();
}

}  // namespace
}  // namespace bwd

hipError_t launch_bwd(const BwdArgs& a, int d, bool bf16, bool causal, bool varlen, int stage,
                      hipStream_t st) {
  if ((long)a.T * a.H == 0) return hipSuccess;
  if (stage == kBwdPrep || stage == kBwdAll) {
    const hipError_t e = d == 128 ? (bf16 ? bwd::launch_prep<128, BF16>(a, st)
                                          : bwd::launch_prep<128, F16>(a, st))
                                  : (bf16 ? bwd::launch_prep<64, BF16>(a, st)
                                          : bwd::launch_prep<64, F16>(a, st));
    if (e != hipSuccess) return e;
  }
  if (stage == kBwdDkDv || stage == kBwdAll) {
    const hipError_t e = bwd::launch_dkdv(a, d, bf16, causal, varlen, st);
    if (e != hipSuccess) return e;
  }
  if (stage == kBwdDq || stage == kBwdAll) return bwd::launch_dq(a, d, bf16, causal, varlen, st);
  return hipSuccess;
}

}  // namespace fa
