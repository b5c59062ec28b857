// Forward attention kernel for gfx950 (tiled exact attention with online softmax).
//
// Algorithm: "FlashAttention 详解（零基础入门）" §6.1-§6.2 (query blocks in the outer,
// parallel loop; key/value blocks streamed through on-chip memory in the inner loop; row
// max m, row sum l and the output accumulator kept on chip) and §5.2-§5.4 (online softmax
// rescale); the output is kept unnormalised and divided by l once at the end, as in
// "FlashAttention 短片讲解稿", segment 第二招 · 在线 Softmax. The causal mask is applied
// inside the kernel ("FlashAttention 与算子融合", fusion table).
//
// Mapping onto CDNA4:
//  - one workgroup = 4 waves = 128*CG query rows of one (batch or sequence, head); wave w
//    owns 32*CG consecutive rows, held as MFMA B operands in registers for the whole loop.
//  - key/value tiles of 64 rows are copied HBM/L2 -> registers -> LDS, double buffered:
//    the loads for tile t+1 are issued before tile t is computed.
//  - scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16: each lane then
//    holds 32 scores of ONE query row (the other 32 sit in lane l^32), so row max and row
//    sum need only per-lane work plus one v_permlane32_swap.
//  - P^T leaves the accumulators already in the B-operand layout of the next MFMA,
//    O^T += V^T P^T. V is written to LDS transposed, with key bits 2 and 3 swapped inside
//    each group of 16, so that the key order of each lane's P registers matches the key
//    order of a single 16-byte LDS read of V^T.
//  - exp2 domain: scores are multiplied by scale*log2(e) in the exponent's FMA. The
//    running max used as the exponent's reference is only moved when the true row max
//    exceeds it by more than 8 (in log2 units), so the rescale of the output accumulator is
//    rare; O = acc / l and LSE = (m_ref + log2 l) ln 2 are exact for any reference.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBK = 64;                   // keys per tile
constexpr float kRescaleSlack = 8.0f;     // log2 units the reference max may lag behind
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kNegInf = -__builtin_inff();

// Position of key k (0..63) inside a transposed V tile row: bits 2 and 3 swapped.
__device__ __forceinline__ int vpos(int k) { return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1); }

template <int D, class T, bool CAUSAL, bool VARLEN, int CG>
__global__ __launch_bounds__(kThreads, 1) void fwd_kernel(FwdArgs a) {
  constexpr int BQ = 32 * CG * kWaves;
  constexpr int KSTR = D + 8;    // LDS row stride of K (elements): +16 B against bank conflicts
  constexpr int VSTR = kBK + 8;  // LDS row stride of V^T (elements)
  constexpr int DC = D / 16;     // 16-wide d chunks of Q K^T
  constexpr int DB = D / 32;     // 32-wide d blocks of the output
  constexpr int KC = kBK * D / 8 / kThreads;  // 16-byte K chunks per thread
  constexpr int R = D / 32;                    // V rows per thread (transposed store)
  constexpr int VKG = kBK / R;                 // V key groups

  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][kBK * KSTR];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[2][D * VSTR];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, g = lane >> 5;

  // ---- work item: (query block, head, batch or sequence)
  const int nqb = (a.N + BQ - 1) / BQ;
  uint32_t w = blockIdx.x;
  if (!VARLEN) w = xcd_remap(w, gridDim.x);
  int qb = w % nqb;
  const int h = (w / nqb) % a.H;
  const int bs = w / (nqb * a.H);
  if (CAUSAL || VARLEN) qb = nqb - 1 - qb;  // longest rows first

  long tok0;
  int L;
  if (VARLEN) {
    int s0 = a.cu[bs], s1 = a.cu[bs + 1];
    s0 = s0 < 0 ? 0 : (s0 > a.T ? a.T : s0);
    s1 = s1 < s0 ? s0 : (s1 > a.T ? a.T : s1);
    L = s1 - s0 < a.N ? s1 - s0 : a.N;
    tok0 = s0;
  } else {
    L = a.N;
    tok0 = (long)bs * a.N;
  }
  const int q0 = qb * BQ;
  if (q0 >= L) return;

  const uint32_t rstride = (uint32_t)a.H * D * 2;  // bytes between consecutive tokens
  const long base = (tok0 * a.H + h) * D;
  const uint32_t nbytes = (uint32_t)(L - 1) * rstride + D * 2;
  const auto rq = make_rsrc(a.q + base, nbytes);
  const auto rk = make_rsrc(a.k + base, nbytes);
  const auto rv = make_rsrc(a.v + base, nbytes);
  const auto ro = make_rsrc(a.o + base, nbytes);
  float* lse = a.lse + (VARLEN ? (long)h * a.T + tok0 : ((long)bs * a.H + h) * a.N);

  const int wq0 = q0 + wave * 32 * CG;  // first query row of this wave
  const int kend = CAUSAL ? (L < q0 + BQ ? L : q0 + BQ) : L;
  const int ntiles = (kend + kBK - 1) / kBK;

  // ---- Q block into registers (B operand of S^T = K Q^T): lane holds row l32 of each
  // 32-row group, d = 16*dc + 8g .. +7.
  u32x4 qreg[CG][DC];
#pragma unroll
  for (int cg = 0; cg < CG; ++cg)
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
      u32x4 x = buf_load16(rq, (uint32_t)(wq0 + cg * 32 + l32) * rstride + (16 * dc + 8 * g) * 2);
      qreg[cg][dc] = x ^ a.qsign;
    }

  // ---- tile loaders
  u32x4 kr[KC], vr[R];
  const int vkg = tid % VKG, vc = tid / VKG;  // V: keys R*vkg.., dims 8*vc..
  auto gload = [&](int t) {
    const int kb0 = t * kBK;
#pragma unroll
    for (int i = 0; i < KC; ++i) {
      const int c = tid + kThreads * i, row = c / (D / 8), col = (c % (D / 8)) * 8;
      kr[i] = buf_load16(rk, (uint32_t)(kb0 + row) * rstride + col * 2);
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
      vr[r] = buf_load16(rv, (uint32_t)(kb0 + R * vkg + r) * rstride + vc * 16);
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KC; ++i) {
      const int c = tid + kThreads * i, row = c / (D / 8), col = (c % (D / 8)) * 8;
      *reinterpret_cast<u32x4*>(&Ks[buf][row * KSTR + col]) = kr[i];
    }
    const int p = vpos(R * vkg);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // dims 8*vc + 2e (low halves) and 8*vc + 2e + 1 (high halves)
      if constexpr (R == 4) {
        u32x2 lo = {__builtin_amdgcn_perm(vr[1][e], vr[0][e], 0x05040100u),
                    __builtin_amdgcn_perm(vr[3][e], vr[2][e], 0x05040100u)};
        u32x2 hi = {__builtin_amdgcn_perm(vr[1][e], vr[0][e], 0x07060302u),
                    __builtin_amdgcn_perm(vr[3][e], vr[2][e], 0x07060302u)};
        *reinterpret_cast<u32x2*>(&Vt[buf][(8 * vc + 2 * e) * VSTR + p]) = lo;
        *reinterpret_cast<u32x2*>(&Vt[buf][(8 * vc + 2 * e + 1) * VSTR + p]) = hi;
      } else {
        *reinterpret_cast<uint32_t*>(&Vt[buf][(8 * vc + 2 * e) * VSTR + p]) =
            __builtin_amdgcn_perm(vr[1][e], vr[0][e], 0x05040100u);
        *reinterpret_cast<uint32_t*>(&Vt[buf][(8 * vc + 2 * e + 1) * VSTR + p]) =
            __builtin_amdgcn_perm(vr[1][e], vr[0][e], 0x07060302u);
      }
    }
  };

  // ---- running state per 32-row group: reference max (log2 units), partial row sum
  // over this lane's keys, unnormalised output O^T (lane = row, registers = d).
  float mref[CG], lsum[CG];
  f32x16 oacc[CG][DB];
#pragma unroll
  for (int cg = 0; cg < CG; ++cg) {
    mref[cg] = kNegInf;
    lsum[cg] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[cg][db] = f32x16{};
  }
  const float c2 = a.scale_log2;

  gload(0);
  lstore(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) gload(t + 1);
    const int kt0 = t * kBK;
    const bool active = !CAUSAL || kt0 <= wq0 + 32 * CG - 1;
    if (active) {
      // S^T tile: two 32-key blocks x CG 32-query groups
      f32x16 s[CG][2];
#pragma unroll
      for (int cg = 0; cg < CG; ++cg) s[cg][0] = s[cg][1] = f32x16{};
#pragma unroll
      for (int dc = 0; dc < DC; ++dc)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const u32x4 ka =
              *reinterpret_cast<const u32x4*>(&Ks[buf][(kb * 32 + l32) * KSTR + 16 * dc + 8 * g]);
#pragma unroll
          for (int cg = 0; cg < CG; ++cg) s[cg][kb] = mfma32<T>(ka, qreg[cg][dc], s[cg][kb]);
        }

      const bool masked = kt0 + kBK > L || (CAUSAL && kt0 + kBK - 1 > wq0);
      u32x4 pf[CG][4];
#pragma unroll
      for (int cg = 0; cg < CG; ++cg) {
        const int qi = wq0 + cg * 32 + l32;
        if (masked) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = kt0 + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
              if (key >= L || (CAUSAL && key > qi)) s[cg][kb][r] = kNegInf;
            }
        }
        float mx = s[cg][0][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[cg][kb][r]);
        mx = pair_max(mx);
        const float mnew = mx == kNegInf ? kNegInf : mx * c2;
        const bool need = mnew > mref[cg] + kRescaleSlack;
        if (__any(need)) {
          const float alpha = need ? exp2f_hw(mref[cg] - mnew) : 1.0f;
          lsum[cg] *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db) oacc[cg][db] *= alpha;
          if (need) mref[cg] = mnew;
        }
        const float mu = mref[cg] == kNegInf ? 0.f : mref[cg];
        float p[32];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float sv = s[cg][kb][r];
            float e = exp2f_hw(fmaf(sv, c2, -mu));
            if (masked) e = sv == kNegInf ? 0.f : e;
            p[kb * 16 + r] = e;
          }
        float ls = 0.f;
#pragma unroll
        for (int i = 0; i < 32; ++i) ls += p[i];
        lsum[cg] += ls;
#pragma unroll
        for (int kc = 0; kc < 4; ++kc)
          pf[cg][kc] = u32x4{pack2<T>(p[8 * kc + 0], p[8 * kc + 1]),
                             pack2<T>(p[8 * kc + 2], p[8 * kc + 3]),
                             pack2<T>(p[8 * kc + 4], p[8 * kc + 5]),
                             pack2<T>(p[8 * kc + 6], p[8 * kc + 7])};
      }

      // O^T += V^T P^T over four 16-key chunks
#pragma unroll
      for (int kc = 0; kc < 4; ++kc)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const u32x4 va =
              *reinterpret_cast<const u32x4*>(&Vt[buf][(db * 32 + l32) * VSTR + 16 * kc + 8 * g]);
#pragma unroll
          for (int cg = 0; cg < CG; ++cg) oacc[cg][db] = mfma32<T>(va, pf[cg][kc], oacc[cg][db]);
        }
    }
    if (t + 1 < ntiles) lstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = acc / l (rows >= L are dropped by the buffer bounds), LSE
#pragma unroll
  for (int cg = 0; cg < CG; ++cg) {
    const int qi = wq0 + cg * 32 + l32;
    const float l = pair_sum(lsum[cg]);
    const float inv = l > 0.f ? 1.0f / l : 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const f32x16& o = oacc[cg][db];
        u32x2 v = {pack2<T>(o[4 * rr] * inv, o[4 * rr + 1] * inv),
                   pack2<T>(o[4 * rr + 2] * inv, o[4 * rr + 3] * inv)};
        buf_store8(ro, (uint32_t)qi * rstride + (db * 32 + 8 * rr + 4 * g) * 2, v);
      }
    if (g == 0 && qi < L) lse[qi] = l > 0.f ? (mref[cg] + log2f_hw(l)) * kLn2 : kNegInf;
  }
}

template <int D, class T, bool CAUSAL, bool VARLEN>
hipError_t launch(const FwdArgs& a, hipStream_t st) {
  constexpr int CG = 1;
  constexpr int BQ = 32 * CG * kWaves;
  const int nqb = (a.N + BQ - 1) / BQ;
  const long total = (long)nqb * a.H * a.B;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL((fwd_kernel<D, T, CAUSAL, VARLEN, CG>), dim3((unsigned)total),
                     dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

template <int D, class T>
hipError_t launch_d(const FwdArgs& a, bool causal, bool varlen, hipStream_t st) {
  if (varlen)
    return causal ? launch<D, T, true, true>(a, st) : launch<D, T, false, true>(a, st);
  return causal ? launch<D, T, true, false>(a, st) : launch<D, T, false, false>(a, st);
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a, int d, bool bf16, bool causal, bool varlen,
                      hipStream_t st) {
  if (d == 128)
    return bf16 ? launch_d<128, BF16>(a, causal, varlen, st) : launch_d<128, F16>(a, causal, varlen, st);
  return bf16 ? launch_d<64, BF16>(a, causal, varlen, st) : launch_d<64, F16>(a, causal, varlen, st);
}

}  // namespace fa
