// dK/dV kernel of the backward pass (see fa_bwd.hip for the gradient formulas): one
// workgroup per 128-key block; streams 64-query tiles of Q, dO and the row terms from HBM/L2
// straight into LDS, double buffered.
// S = Q K^T and dP = dO V^T are computed with lanes <-> keys, so P and dS leave the
// accumulators in the B-operand layout of dV^T += dO^T P and dK^T += Q^T dS.
#include "fa_bwd_common.h"

namespace fa {
namespace bwd {
namespace {

// Eight waves, two per SIMD. Wave (kg, qh) = (wave % 4, wave / 4) owns the 32 keys
// k0 + 32 kg .. and the 32-query half qh of every streamed tile; it holds K of its keys in
// registers and reads V of the block's 128 keys from LDS (loaded once), which keeps each
// wave within 256 registers. The two waves of a key group sum their partial dK and dV
// through LDS at the end.
template <int D, class T, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(512, 1) void bwd_dkdv_kernel(BwdArgs a) {
  constexpr int NW = 8;
  constexpr int BKV = 128;  // keys per workgroup
  constexpr int DC = D / 16, DB = D / 32;
  using TL = Tile<D, NW>;

  __shared__ __attribute__((aligned(1024))) uint8_t Qs0[TL::BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t Qs1[TL::BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t dOs0[TL::BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t dOs1[TL::BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t Vk0[TL::BYTES];  // V rows k0 .. k0+63
  __shared__ __attribute__((aligned(1024))) uint8_t Vk1[TL::BYTES];  // V rows k0+64 .. k0+127
  __shared__ __attribute__((aligned(256))) float nl0[kTile];  // -LSE log2(e)
  __shared__ __attribute__((aligned(256))) float nl1[kTile];
  __shared__ __attribute__((aligned(256))) float nd0[kTile];  // -D
  __shared__ __attribute__((aligned(256))) float nd1[kTile];
  for (void* p : {(void*)Qs0, (void*)Qs1, (void*)dOs0, (void*)dOs1, (void*)Vk0, (void*)Vk1})
    lds_poison(p, TL::BYTES);
  for (float* p : {nl0, nl1, nd0, nd1}) lds_poison(p, kTile * 4);
  lds_poison_done();

  const int tid = threadIdx.x;
  const int lane = tid & 63, l32 = lane & 31, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = wave & 3, qh = wave >> 2;
  Lanes<D> ln(lane);
  const int nkb = (a.N + BKV - 1) / BKV;
  int kb, h, bs;
  // per-head order even under the mask (key block 0, the longest, first within each head):
  // with 16 workgroups per CU the tail is short, and going longest first across the heads of
  // an XCD (as dQ does) streamed eight heads' Q and dO through its L2 at once and was 2-4%
  // slower at N = 8192
  if (!decode_work(a, nkb, VARLEN, false, false, kb, h, bs)) return;
  const SliceInfo si = slice_info(a, bs, h);
  const int L = si.L;
  const int k0 = kb * BKV;
  if (k0 >= L) return;

  const uint32_t rstride = (uint32_t)a.H * D * 2;
  const long base = (si.tok0 * a.H + h) * D;
  const uint32_t nbytes = (uint32_t)(L - 1) * rstride + D * 2;
  const u32x4 rq = rsrc_words(a.q + base, nbytes);
  const auto rk = make_rsrc(a.k + base, nbytes);
  const u32x4 rv = rsrc_words(a.v + base, nbytes);
  const u32x4 rdo = rsrc_words(a.dout + base, nbytes);
  const auto rdk = make_rsrc(a.dk + base, nbytes);
  const auto rdv = make_rsrc(a.dv + base, nbytes);
  const u32x4 rnl = rsrc_words(a.neg_lse2 + si.stat, (uint32_t)L * 4);
  const u32x4 rnd = rsrc_words(a.neg_delta + si.stat, (uint32_t)L * 4);

  const int wk0 = k0 + kg * 32;  // this wave's keys: wk0 .. wk0+31
  const int key = wk0 + l32;     // the key this lane's accumulators belong to

  // K of this wave's keys: B operand of S = Q K^T (negative scale folded into its sign)
  u32x4 kreg[DC];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc)
    kreg[dc] = buf_load16(rk, (uint32_t)key * rstride + (16 * dc + 8 * g) * 2) ^ a.qsign;
  // V of the block's keys into LDS (B operand of dP = dO V^T, row fragments)
  TL::load(rv, Vk0, k0, rstride, wave, lane);
  TL::load(rv, Vk1, k0 + kTile, rstride, wave, lane);
  const uint8_t* vk = kg < 2 ? Vk0 : Vk1;
  const int vrow0 = (kg & 1) * 32;

  f32x16 dkacc[DB], dvacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dkacc[db] = dvacc[db] = f32x16{};

  const int qt_begin = CAUSAL ? k0 / kTile : 0;
  const int qt_end = (L + kTile - 1) / kTile;
  const float c2 = a.scale_log2;

  auto load_tile = [&](int qt, uint8_t* qs, uint8_t* dos, float* nl, float* nd) {
    TL::load(rq, qs, qt * kTile, rstride, wave, lane);
    TL::load(rdo, dos, qt * kTile, rstride, wave, lane);
    if (wave == 0) {  // 64 lanes x 4 bytes: one row term per query of the tile
      dma4<0>(rnl, __builtin_amdgcn_readfirstlane(lds_addr(nl)), (qt * kTile + lane) * 4);
      dma4<0>(rnd, __builtin_amdgcn_readfirstlane(lds_addr(nd)), (qt * kTile + lane) * 4);
    }
  };

  // MASK: the step may meet the causal mask (the block's first two query tiles, queries
  // k0 .. k0+127); later tiles lie wholly below the diagonal and take the branch-free body,
  // which the compiler schedules as one block
  auto step = [&](auto bsel, auto msel, int qt) {
    constexpr int B = decltype(bsel)::value;
    constexpr bool MASK = decltype(msel)::value;
    const uint8_t* qs = B ? Qs1 : Qs0;
    const uint8_t* dos = B ? dOs1 : dOs0;
    const float* nl = B ? nl1 : nl0;
    const float* nd = B ? nd1 : nd0;
    if (qt + 1 < qt_end) load_tile(qt + 1, B ? Qs0 : Qs1, B ? dOs0 : dOs1, B ? nl0 : nl1,
                                   B ? nd0 : nd1);
    const int q0 = qt * kTile + qh * 32;  // this wave's 32 queries: q0 .. q0+31
    const bool active = !MASK || q0 + 31 >= wk0;
    if (active) {
      ln.refresh();
      // S (queries x keys) and dP - D (the accumulator starts at -D of each query)
      f32x16 s = f32x16{}, dp;
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(&nd[qh * 32 + 8 * a4 + 4 * g]);
#pragma unroll
        for (int j = 0; j < 4; ++j) dp[4 * a4 + j] = d4[j];
      }
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) {
        s = mfma32<T>(ln.row_frag(qs, qh * 32, dc), kreg[dc], s);
        dp = mfma32<T>(ln.row_frag(dos, qh * 32, dc), ln.row_frag(vk, vrow0, dc), dp);
      }
      float p[16];
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(&nl[qh * 32 + 8 * a4 + 4 * g]);
#pragma unroll
        for (int j = 0; j < 4; ++j) p[4 * a4 + j] = exp2f_hw(fmaf(s[4 * a4 + j], c2, l4[j]));
      }
      if (MASK && q0 < wk0 + 31) {
        __builtin_amdgcn_sched_barrier(0);  // keep the mask a branch (diagonal tiles only)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (key > q0 + 8 * (r >> 2) + 4 * g + (r & 3)) p[r] = 0.f;
      }
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        float ds[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) ds[j] = p[8 * hh + j] * dp[8 * hh + j];
        const u32x4 pf = {pack2<T>(p[8 * hh + 0], p[8 * hh + 1]),
                          pack2<T>(p[8 * hh + 2], p[8 * hh + 3]),
                          pack2<T>(p[8 * hh + 4], p[8 * hh + 5]),
                          pack2<T>(p[8 * hh + 6], p[8 * hh + 7])};
        const u32x4 sf = {pack2<T>(ds[0], ds[1]), pack2<T>(ds[2], ds[3]),
                          pack2<T>(ds[4], ds[5]), pack2<T>(ds[6], ds[7])};
        // dV^T += dO^T P and dK^T += Q^T dS over the 16-query chunk 2 qh + hh of the tile
        const int kc = 2 * qh + hh;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          dvacc[db] = mfma32<T>(ln.tr_frag(dos, kc * 16, db), pf, dvacc[db]);
          dkacc[db] = mfma32<T>(ln.tr_frag(qs, kc * 16, db), sf, dkacc[db]);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of the next tile have landed
    __syncthreads();
  };

  load_tile(qt_begin, Qs0, dOs0, nl0, nd0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  int qt = qt_begin;  // even: k0 is a multiple of 128, so the buffers alternate from Qs0
  if constexpr (CAUSAL) {
    step(B0{}, std::true_type{}, qt);
    if (qt + 1 < qt_end) step(B1{}, std::true_type{}, qt + 1);
    qt += 2;
  }
  for (; qt < qt_end; qt += 2) {
    step(B0{}, std::false_type{}, qt);
    if (qt + 1 < qt_end) step(B1{}, std::false_type{}, qt + 1);
  }

  // sum the two query halves' partial gradients of each key group through LDS (the tile
  // buffers are free now: one per key group, DB*16 floats per lane)
  uint8_t* red = kg == 0 ? Qs0 : (kg == 1 ? Qs1 : (kg == 2 ? dOs0 : dOs1));
  auto reduce = [&](f32x16 (&acc)[DB]) {
    if (qh == 1) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *reinterpret_cast<f32x4*>(red + ((db * 4 + q4) * 64 + lane) * 16) =
              f32x4{acc[db][4 * q4], acc[db][4 * q4 + 1], acc[db][4 * q4 + 2],
                    acc[db][4 * q4 + 3]};
    }
    __syncthreads();
    if (qh == 0) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4 o = *reinterpret_cast<const f32x4*>(red + ((db * 4 + q4) * 64 + lane) * 16);
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[db][4 * q4 + j] += o[j];
        }
    }
    __syncthreads();
  };
  reduce(dvacc);
  reduce(dkacc);
  if (qh != 0) return;

  // dK = scale * sum dS q (signed scale), dV = sum P dO
  const float ks = a.scale;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const uint32_t off = (uint32_t)key * rstride + (db * 32 + 8 * rr + 4 * g) * 2;
      const f32x16& x = dkacc[db];
      const f32x16& y = dvacc[db];
      buf_store8(rdk, off, u32x2{pack2<T>(x[4 * rr] * ks, x[4 * rr + 1] * ks),
                                 pack2<T>(x[4 * rr + 2] * ks, x[4 * rr + 3] * ks)});
      buf_store8(rdv, off, u32x2{pack2<T>(y[4 * rr], y[4 * rr + 1]),
                                 pack2<T>(y[4 * rr + 2], y[4 * rr + 3])});
    }
}

template <int D, class T, bool CAUSAL, bool VARLEN>
hipError_t launch_t(const BwdArgs& a, hipStream_t st) {
  const int nkb = (a.N + 127) / 128;
  const long nblk = VARLEN ? varlen_grid(nkb, a.H, a.B) : (long)nkb * a.H * a.B;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, T, CAUSAL, VARLEN>), dim3((unsigned)nblk), dim3(512),
                     0, st, a);
  return hipGetLastError();
}

template <int D, class T>
hipError_t launch_c(const BwdArgs& a, bool causal, bool varlen, hipStream_t st) {
  if (varlen)
    return causal ? launch_t<D, T, true, true>(a, st) : launch_t<D, T, false, true>(a, st);
  return causal ? launch_t<D, T, true, false>(a, st) : launch_t<D, T, false, false>(a, st);
}

}  // namespace

hipError_t launch_dkdv(const BwdArgs& a, int d, bool bf16, bool causal, bool varlen,
                       hipStream_t st) {
  if (d == 128)
    return bf16 ? launch_c<128, BF16>(a, causal, varlen, st) : launch_c<128, F16>(a, causal, varlen, st);
  return bf16 ? launch_c<64, BF16>(a, causal, varlen, st) : launch_c<64, F16>(a, causal, varlen, st);
}

}  // namespace bwd
}  // namespace fa
