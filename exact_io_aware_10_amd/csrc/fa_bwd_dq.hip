// dQ kernel of the backward pass (see fa_bwd.hip for the gradient formulas): one workgroup
// of 8 waves per 256-query block (one per CU), 32 queries per wave with Q and dO in
// registers; streams 64-key tiles of K and V into LDS; S^T and dP^T with lanes <-> queries
// feed dQ^T += K^T dS^T.
// Built with the MFMA results in VGPRs (the softmax-side VALU work reads them directly).
#include "fa_bwd_common.h"

namespace fa {
namespace bwd {
namespace {

// Eight waves share each streamed K/V tile: half the L2 -> LDS traffic of two 4-wave
// workgroups per CU, 1.3% faster (1.8% causal); 128-key tiles were no faster.
constexpr int kDqWaves = 8;                  // waves per workgroup, 32 queries each
constexpr int kDqThreads = 64 * kDqWaves;
constexpr int kDqTile = 64;                  // keys per streamed K/V tile

template <int D, class T, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(kDqThreads, 1) void bwd_dq_kernel(BwdArgs a) {
  constexpr int BQ = 32 * kDqWaves;
  constexpr int DC = D / 16, DB = D / 32;
  using TL = Tile<D, kDqWaves, kDqTile>;

  __shared__ __attribute__((aligned(1024))) uint8_t Ks0[TL::BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t Ks1[TL::BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t Vs0[TL::BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t Vs1[TL::BYTES];
  for (void* p : {(void*)Ks0, (void*)Ks1, (void*)Vs0, (void*)Vs1}) lds_poison(p, TL::BYTES);
  lds_poison_done();

  const int tid = threadIdx.x;
  const int lane = tid & 63, l32 = lane & 31, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  Lanes<D> ln(lane);
  const int nqb = (a.N + BQ - 1) / BQ;
  int qb, h, bs;
  if (!decode_work(a, nqb, VARLEN, CAUSAL, true, qb, h, bs)) return;
  const SliceInfo si = slice_info(a, bs, h);
  const int L = si.L;
  const int q0 = qb * BQ;
  if (q0 >= L) return;

  const uint32_t rstride = (uint32_t)a.H * D * 2;
  const long base = (si.tok0 * a.H + h) * D;
  const uint32_t nbytes = (uint32_t)(L - 1) * rstride + D * 2;
  const auto rq = make_rsrc(a.q + base, nbytes);
  const u32x4 rk = rsrc_words(a.k + base, nbytes);
  const u32x4 rv = rsrc_words(a.v + base, nbytes);
  const auto rdo = make_rsrc(a.dout + base, nbytes);
  const auto rdq = make_rsrc(a.dq + base, nbytes);

  const int wq0 = q0 + wave * 32;
  const int qi = wq0 + l32;  // the query row of this lane
  u32x4 qreg[DC], doreg[DC];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc) {
    qreg[dc] = buf_load16(rq, (uint32_t)qi * rstride + (16 * dc + 8 * g) * 2) ^ a.qsign;
    doreg[dc] = buf_load16(rdo, (uint32_t)qi * rstride + (16 * dc + 8 * g) * 2);
  }
  const float nlq = qi < L ? a.neg_lse2[si.stat + qi] : 0.f;
  const float ndq = qi < L ? a.neg_delta[si.stat + qi] : 0.f;

  f32x16 dqacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dqacc[db] = f32x16{};

  const int kend = CAUSAL ? (L < q0 + BQ ? L : q0 + BQ) : L;
  const int ntiles = (kend + kDqTile - 1) / kDqTile;
  const float c2 = a.scale_log2;

  // MASK: the step may meet the causal mask (key tiles from q0 on); earlier tiles lie wholly
  // below the diagonal and take the branch-free body
  auto step = [&](auto bsel, auto msel, int t) {
    constexpr int B = decltype(bsel)::value;
    constexpr bool MASK = decltype(msel)::value;
    const uint8_t* ks = B ? Ks1 : Ks0;
    const uint8_t* vs = B ? Vs1 : Vs0;
    if (t + 1 < ntiles) {
      TL::load(rk, B ? Ks0 : Ks1, (t + 1) * kDqTile, rstride, wave, lane);
      TL::load(rv, B ? Vs0 : Vs1, (t + 1) * kDqTile, rstride, wave, lane);
    }
    const int kt0 = t * kDqTile;
    const bool active = !MASK || kt0 <= wq0 + 31;
    if (active) {
      const bool masked = MASK && kt0 + kDqTile - 1 > wq0;
      // the tile's 32-key blocks, one after the other
#pragma unroll
      for (int kb = 0; kb < kDqTile / 32; ++kb) {
        ln.refresh();
        // S^T and dP^T - D (keys x queries; the dP accumulator starts at -D of the row)
        f32x16 s = f32x16{}, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) dp[r] = ndq;
        // the products run at raised wave priority, so that a wave ready to issue one wins
        // the SIMD's issue slot over the other wave's exponentials (0.9% faster at N = 8192)
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) {
          s = mfma32<T>(ln.row_frag(ks, kb * 32, dc), qreg[dc], s);
          dp = mfma32<T>(ln.row_frag(vs, kb * 32, dc), doreg[dc], dp);
        }
        __builtin_amdgcn_s_setprio(0);
        float p[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) p[r] = exp2f_hw(fmaf(s[r], c2, nlq));
        if (masked) {
          __builtin_amdgcn_sched_barrier(0);  // keep the mask a branch (diagonal tiles only)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (kt0 + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3) > qi) p[r] = 0.f;
        }
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          float ds[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) ds[j] = p[8 * hh + j] * dp[8 * hh + j];
          const u32x4 sf = {pack2<T>(ds[0], ds[1]), pack2<T>(ds[2], ds[3]),
                            pack2<T>(ds[4], ds[5]), pack2<T>(ds[6], ds[7])};
          const int kc = 2 * kb + hh;  // 16-key chunk of the tile
#pragma unroll
          for (int db = 0; db < DB; ++db)
            dqacc[db] = mfma32<T>(ln.tr_frag(ks, kc * 16, db), sf, dqacc[db]);
        }
        __builtin_amdgcn_s_setprio(0);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of the next tile have landed
    __syncthreads();
  };

  TL::load(rk, Ks0, 0, rstride, wave, lane);
  TL::load(rv, Vs0, 0, rstride, wave, lane);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  // first tile that can meet the mask: even (q0 is a multiple of 256), so the unmasked loop
  // ends on a whole pair and the buffers keep alternating from Ks0
  const int tmask = CAUSAL ? q0 / kDqTile : ntiles;
  int t = 0;
  for (; t < ntiles && t < tmask; t += 2) {
    step(B0{}, std::false_type{}, t);
    if (t + 1 < ntiles) step(B1{}, std::false_type{}, t + 1);
  }
  if constexpr (CAUSAL) {
    for (; t < ntiles; t += 2) {
      step(B0{}, std::true_type{}, t);
      if (t + 1 < ntiles) step(B1{}, std::true_type{}, t + 1);
    }
  }

  // dQ = scale * sum dS k  (signed scale)
  const float qs = a.scale;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const f32x16& x = dqacc[db];
      buf_store8(rdq, (uint32_t)qi * rstride + (db * 32 + 8 * rr + 4 * g) * 2,
                 u32x2{pack2<T>(x[4 * rr] * qs, x[4 * rr + 1] * qs),
                       pack2<T>(x[4 * rr + 2] * qs, x[4 * rr + 3] * qs)});
    }
}


template <int D, class T, bool CAUSAL, bool VARLEN>
hipError_t launch_t(const BwdArgs& a, hipStream_t st) {
  constexpr int BQ = 32 * kDqWaves;
  const int nqb = (a.N + BQ - 1) / BQ;
  const long nblk = VARLEN ? varlen_grid(nqb, a.H, a.B) : (long)nqb * a.H * a.B;
  hipLaunchKernelGGL((bwd_dq_kernel<D, T, CAUSAL, VARLEN>), dim3((unsigned)nblk),
                     dim3(kDqThreads), 0, st, a);
  return hipGetLastError();
}

template <int D, class T>
hipError_t launch_c(const BwdArgs& a, bool causal, bool varlen, hipStream_t st) {
  if (varlen)
    return causal ? launch_t<D, T, true, true>(a, st) : launch_t<D, T, false, true>(a, st);
  return causal ? launch_t<D, T, true, false>(a, st) : launch_t<D, T, false, false>(a, st);
}

}  // namespace

hipError_t launch_dq(const BwdArgs& a, int d, bool bf16, bool causal, bool varlen,
                     hipStream_t st) {
  if (d == 128)
    return bf16 ? launch_c<128, BF16>(a, causal, varlen, st) : launch_c<128, F16>(a, causal, varlen, st);
  return bf16 ? launch_c<64, BF16>(a, causal, varlen, st) : launch_c<64, F16>(a, causal, varlen, st);
}

}  // namespace bwd
}  // namespace fa
