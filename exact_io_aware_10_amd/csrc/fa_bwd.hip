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
//   1. bwd_delta_kernel : D_i for every row (reads O and dO once).
//   2. bwd_dkdv_kernel  : one workgroup per 128-key block (32 keys per wave, K and V held
//                         in registers); streams 64-query tiles of Q and dO through LDS,
//                         double buffered, each stored row-major and transposed.
//                         S = Q K^T and dP = dO V^T are computed with lanes <-> keys, so
//                         P and dS leave the accumulators in the B-operand layout of
//                         dV^T += dO^T P and dK^T += Q^T dS.
//   3. bwd_dq_kernel    : one workgroup per 128-query block (32 queries per wave, Q and
//                         dO in registers); streams 64-key tiles of K and V; S^T and dP^T
//                         with lanes <-> queries feed dQ^T += K^T dS^T.
// The transposed LDS copies use the same key/query bit permutation as the forward kernel
// (bits 2 and 3 swapped within groups of 16) so one 16-byte LDS read matches the row order
// of the P / dS registers.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 64;  // rows of the streamed tile (queries in dK/dV, keys in dQ)
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kInf = __builtin_inff();

__device__ __forceinline__ int tpos(int k) { return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1); }

// Per-slice addressing shared by the three kernels.
struct SliceInfo {
  long tok0;  // first token of the slice in the [tokens, H, d] tensors
  int L;      // rows in the slice
  long stat;  // offset of row 0 of the slice in lse / delta
};

__device__ __forceinline__ SliceInfo slice_info(const BwdArgs& a, int bs, int h) {
  SliceInfo s;
  if (a.cu != nullptr) {
    int s0 = a.cu[bs], s1 = a.cu[bs + 1];
    s0 = s0 < 0 ? 0 : (s0 > a.T ? a.T : s0);
    s1 = s1 < s0 ? s0 : (s1 > a.T ? a.T : s1);
    s.L = s1 - s0 < a.N ? s1 - s0 : a.N;
    s.tok0 = s0;
    s.stat = (long)h * a.T + s0;
  } else {
    s.L = a.N;
    s.tok0 = (long)bs * a.N;
    s.stat = ((long)bs * a.H + h) * a.N;
  }
  return s;
}

// ---------------------------------------------------------------- 1. D_i = <dO_i, O_i>
template <int D, class T>
__global__ __launch_bounds__(kThreads) void bwd_delta_kernel(BwdArgs a, long rows) {
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
    a.delta[idx] = acc;
  }
}

// ---------------------------------------------------------------- shared tile loader
// A tile of kTile rows x D of a [tokens, H, D] tensor, loaded so that each thread holds R
// consecutive rows x 8 columns; stored to LDS row-major (stride D+8) and/or transposed
// (stride kTile+8, rows permuted by tpos).
template <int D>
struct TileLoader {
  static constexpr int R = kTile * D / 8 / kThreads;  // rows per thread (4 or 2)
  static constexpr int KG = kTile / R;
  static constexpr int RSTR = D + 8;
  static constexpr int TSTR = kTile + 8;
  int kg, c;
  u32x4 r[R];
  __device__ TileLoader(int tid) : kg(tid % KG), c(tid / KG) {}
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, uint32_t rstride, int row0,
                                       uint32_t flip) {
#pragma unroll
    for (int i = 0; i < R; ++i)
      r[i] = buf_load16(rs, (uint32_t)(row0 + R * kg + i) * rstride + c * 16) ^ flip;
  }
  __device__ __forceinline__ void store_rows(uint16_t* lds) const {
#pragma unroll
    for (int i = 0; i < R; ++i)
      *reinterpret_cast<u32x4*>(&lds[(R * kg + i) * RSTR + 8 * c]) = r[i];
  }
  __device__ __forceinline__ void store_transposed(uint16_t* lds) const {
    const int p = tpos(R * kg);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (R == 4) {
        u32x2 lo = {__builtin_amdgcn_perm(r[1][e], r[0][e], 0x05040100u),
                    __builtin_amdgcn_perm(r[3][e], r[2][e], 0x05040100u)};
        u32x2 hi = {__builtin_amdgcn_perm(r[1][e], r[0][e], 0x07060302u),
                    __builtin_amdgcn_perm(r[3][e], r[2][e], 0x07060302u)};
        *reinterpret_cast<u32x2*>(&lds[(8 * c + 2 * e) * TSTR + p]) = lo;
        *reinterpret_cast<u32x2*>(&lds[(8 * c + 2 * e + 1) * TSTR + p]) = hi;
      } else {
        *reinterpret_cast<uint32_t*>(&lds[(8 * c + 2 * e) * TSTR + p]) =
            __builtin_amdgcn_perm(r[1][e], r[0][e], 0x05040100u);
        *reinterpret_cast<uint32_t*>(&lds[(8 * c + 2 * e + 1) * TSTR + p]) =
            __builtin_amdgcn_perm(r[1][e], r[0][e], 0x07060302u);
      }
    }
  }
};

// Work item of a dense or packed launch: (block index within the slice, head, batch/seq).
__device__ __forceinline__ void decode_work(const BwdArgs& a, int nblk, bool varlen, int& blk,
                                            int& h, int& bs) {
  uint32_t w = blockIdx.x;
  if (!varlen) w = xcd_remap(w, gridDim.x);
  blk = w % nblk;
  h = (w / nblk) % a.H;
  bs = w / (nblk * a.H);
}

// ---------------------------------------------------------------- 2. dK, dV
template <int D, class T, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_kernel(BwdArgs a) {
  constexpr int BKV = 32 * kWaves;  // keys per workgroup
  constexpr int DC = D / 16, DB = D / 32;
  using TL = TileLoader<D>;
  constexpr int RSTR = TL::RSTR, TSTR = TL::TSTR;

  __shared__ __attribute__((aligned(16))) uint16_t Qs[2][kTile * RSTR];
  __shared__ __attribute__((aligned(16))) uint16_t dOs[2][kTile * RSTR];
  __shared__ __attribute__((aligned(16))) uint16_t Qt[2][D * TSTR];
  __shared__ __attribute__((aligned(16))) uint16_t dOt[2][D * TSTR];
  __shared__ __attribute__((aligned(16))) float lse2s[2][kTile];
  __shared__ __attribute__((aligned(16))) float dds[2][kTile];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, g = lane >> 5;
  const int nkb = (a.N + BKV - 1) / BKV;
  int kb, h, bs;
  decode_work(a, nkb, VARLEN, kb, h, bs);
  const SliceInfo si = slice_info(a, bs, h);
  const int L = si.L;
  const int k0 = kb * BKV;
  if (k0 >= L) return;

  const uint32_t rstride = (uint32_t)a.H * D * 2;
  const long base = (si.tok0 * a.H + h) * D;
  const uint32_t nbytes = (uint32_t)(L - 1) * rstride + D * 2;
  const auto rq = make_rsrc(a.q + base, nbytes);
  const auto rk = make_rsrc(a.k + base, nbytes);
  const auto rv = make_rsrc(a.v + base, nbytes);
  const auto rdo = make_rsrc(a.dout + base, nbytes);
  const auto rdk = make_rsrc(a.dk + base, nbytes);
  const auto rdv = make_rsrc(a.dv + base, nbytes);
  const float* lse = a.lse + si.stat;
  const float* delta = a.delta + si.stat;

  const int wk0 = k0 + wave * 32;  // this wave's keys: wk0 .. wk0+31
  const int key = wk0 + l32;       // the key this lane's accumulators belong to

  // K and V of this wave's keys: B operands of S = Q K^T and dP = dO V^T
  u32x4 kreg[DC], vreg[DC];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc) {
    kreg[dc] = buf_load16(rk, (uint32_t)key * rstride + (16 * dc + 8 * g) * 2);
    vreg[dc] = buf_load16(rv, (uint32_t)key * rstride + (16 * dc + 8 * g) * 2);
  }

  f32x16 dkacc[DB], dvacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dkacc[db] = dvacc[db] = f32x16{};

  const int qt_begin = CAUSAL ? k0 / kTile : 0;
  const int qt_end = (L + kTile - 1) / kTile;
  const float c2 = a.scale_log2;

  TL tq(tid), tdo(tid);
  float lse2_next = 0.f, dd_next = 0.f;
  auto gload = [&](int qt) {
    const int r0 = qt * kTile;
    tq.load(rq, rstride, r0, a.qsign);
    tdo.load(rdo, rstride, r0, 0u);
    if (tid < kTile) {
      const int qi = r0 + tid;
      lse2_next = qi < L ? lse[qi] * kLog2e : kInf;
      dd_next = qi < L ? delta[qi] : 0.f;
    }
  };
  auto lstore = [&](int buf) {
    tq.store_rows(Qs[buf]);
    tq.store_transposed(Qt[buf]);
    tdo.store_rows(dOs[buf]);
    tdo.store_transposed(dOt[buf]);
    if (tid < kTile) {
      lse2s[buf][tid] = lse2_next;
      dds[buf][tid] = dd_next;
    }
  };

  if (qt_begin < qt_end) {
    gload(qt_begin);
    lstore(0);
  }
  __syncthreads();

  for (int qt = qt_begin; qt < qt_end; ++qt) {
    const int buf = (qt - qt_begin) & 1;
    if (qt + 1 < qt_end) gload(qt + 1);
    const int q0 = qt * kTile;
    const bool active = !CAUSAL || q0 + kTile - 1 >= wk0;
    if (active) {
      f32x16 s[2], dp[2];
      s[0] = s[1] = dp[0] = dp[1] = f32x16{};
#pragma unroll
      for (int dc = 0; dc < DC; ++dc)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const int off = (qb * 32 + l32) * RSTR + 16 * dc + 8 * g;
          const u32x4 qa = *reinterpret_cast<const u32x4*>(&Qs[buf][off]);
          const u32x4 da = *reinterpret_cast<const u32x4*>(&dOs[buf][off]);
          s[qb] = mfma32<T>(qa, kreg[dc], s[qb]);
          dp[qb] = mfma32<T>(da, vreg[dc], dp[qb]);
        }
      const bool diag = CAUSAL && q0 < wk0 + 31;
      u32x4 pf[4], sf[4];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        float p[16], ds[16];
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const int ql = qb * 32 + 8 * a4 + 4 * g;  // local query of registers 4*a4 ..
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(&lse2s[buf][ql]);
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(&dds[buf][ql]);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int r = 4 * a4 + j;
            float e = exp2f_hw(fmaf(s[qb][r], c2, -l4[j]));
            if (diag && key > q0 + ql + j) e = 0.f;
            p[r] = e;
            ds[r] = e * (dp[qb][r] - d4[j]);
          }
        }
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          pf[2 * qb + hh] = u32x4{pack2<T>(p[8 * hh + 0], p[8 * hh + 1]),
                                  pack2<T>(p[8 * hh + 2], p[8 * hh + 3]),
                                  pack2<T>(p[8 * hh + 4], p[8 * hh + 5]),
                                  pack2<T>(p[8 * hh + 6], p[8 * hh + 7])};
          sf[2 * qb + hh] = u32x4{pack2<T>(ds[8 * hh + 0], ds[8 * hh + 1]),
                                  pack2<T>(ds[8 * hh + 2], ds[8 * hh + 3]),
                                  pack2<T>(ds[8 * hh + 4], ds[8 * hh + 5]),
                                  pack2<T>(ds[8 * hh + 6], ds[8 * hh + 7])};
        }
      }
#pragma unroll
      for (int kc = 0; kc < 4; ++kc)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int off = (db * 32 + l32) * TSTR + 16 * kc + 8 * g;
          const u32x4 doa = *reinterpret_cast<const u32x4*>(&dOt[buf][off]);
          const u32x4 qa = *reinterpret_cast<const u32x4*>(&Qt[buf][off]);
          dvacc[db] = mfma32<T>(doa, pf[kc], dvacc[db]);
          dkacc[db] = mfma32<T>(qa, sf[kc], dkacc[db]);
        }
    }
    if (qt + 1 < qt_end) lstore(buf ^ 1);
    __syncthreads();
  }

  // dK = |scale| * sum dS q' (q' = q with the sign of scale folded in), dV = sum P dO
  const float ks = fabsf(a.scale);
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

// ---------------------------------------------------------------- 3. dQ
template <int D, class T, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(kThreads, 1) void bwd_dq_kernel(BwdArgs a) {
  constexpr int BQ = 32 * kWaves;
  constexpr int DC = D / 16, DB = D / 32;
  using TL = TileLoader<D>;
  constexpr int RSTR = TL::RSTR, TSTR = TL::TSTR;

  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][kTile * RSTR];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][kTile * RSTR];
  __shared__ __attribute__((aligned(16))) uint16_t Kt[2][D * TSTR];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, g = lane >> 5;
  const int nqb = (a.N + BQ - 1) / BQ;
  int qb, h, bs;
  decode_work(a, nqb, VARLEN, qb, h, bs);
  if (CAUSAL) qb = nqb - 1 - qb;  // longest rows first
  const SliceInfo si = slice_info(a, bs, h);
  const int L = si.L;
  const int q0 = qb * BQ;
  if (q0 >= L) return;

  const uint32_t rstride = (uint32_t)a.H * D * 2;
  const long base = (si.tok0 * a.H + h) * D;
  const uint32_t nbytes = (uint32_t)(L - 1) * rstride + D * 2;
  const auto rq = make_rsrc(a.q + base, nbytes);
  const auto rk = make_rsrc(a.k + base, nbytes);
  const auto rv = make_rsrc(a.v + base, nbytes);
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
  const float lse2 = qi < L ? a.lse[si.stat + qi] * kLog2e : kInf;
  const float dd = qi < L ? a.delta[si.stat + qi] : 0.f;

  f32x16 dqacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dqacc[db] = f32x16{};

  const int kend = CAUSAL ? (L < q0 + BQ ? L : q0 + BQ) : L;
  const int ntiles = (kend + kTile - 1) / kTile;
  const float c2 = a.scale_log2;

  TL tk(tid), tv(tid);
  auto gload = [&](int t) {
    tk.load(rk, rstride, t * kTile, 0u);
    tv.load(rv, rstride, t * kTile, 0u);
  };
  auto lstore = [&](int buf) {
    tk.store_rows(Ks[buf]);
    tk.store_transposed(Kt[buf]);
    tv.store_rows(Vs[buf]);
  };

  gload(0);
  lstore(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) gload(t + 1);
    const int kt0 = t * kTile;
    const bool active = !CAUSAL || kt0 <= wq0 + 31;
    if (active) {
      f32x16 s[2], dp[2];
      s[0] = s[1] = dp[0] = dp[1] = f32x16{};
#pragma unroll
      for (int dc = 0; dc < DC; ++dc)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int off = (kb * 32 + l32) * RSTR + 16 * dc + 8 * g;
          const u32x4 ka = *reinterpret_cast<const u32x4*>(&Ks[buf][off]);
          const u32x4 va = *reinterpret_cast<const u32x4*>(&Vs[buf][off]);
          s[kb] = mfma32<T>(ka, qreg[dc], s[kb]);
          dp[kb] = mfma32<T>(va, doreg[dc], dp[kb]);
        }
      const bool masked = kt0 + kTile > L || (CAUSAL && kt0 + kTile - 1 > wq0);
      float ds[32];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float e = exp2f_hw(fmaf(s[kb][r], c2, -lse2));
          if (masked) {
            const int kj = kt0 + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
            if (kj >= L || (CAUSAL && kj > qi)) e = 0.f;
          }
          ds[kb * 16 + r] = e * (dp[kb][r] - dd);
        }
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        const u32x4 sf = {pack2<T>(ds[8 * kc + 0], ds[8 * kc + 1]),
                          pack2<T>(ds[8 * kc + 2], ds[8 * kc + 3]),
                          pack2<T>(ds[8 * kc + 4], ds[8 * kc + 5]),
                          pack2<T>(ds[8 * kc + 6], ds[8 * kc + 7])};
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const u32x4 ka =
              *reinterpret_cast<const u32x4*>(&Kt[buf][(db * 32 + l32) * TSTR + 16 * kc + 8 * g]);
          dqacc[db] = mfma32<T>(ka, sf, dqacc[db]);
        }
      }
    }
    if (t + 1 < ntiles) lstore(buf ^ 1);
    __syncthreads();
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
hipError_t launch(const BwdArgs& a, hipStream_t st) {
  const long rows = (long)a.T * a.H;
  constexpr int rows_per_block = kThreads / (D / 8);
  hipLaunchKernelGGL((bwd_delta_kernel<D, T>), dim3((unsigned)((rows + rows_per_block - 1) /
                                                                rows_per_block)),
                     dim3(kThreads), 0, st, a, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long nblk = (long)((a.N + 127) / 128) * a.H * a.B;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, T, CAUSAL, VARLEN>), dim3((unsigned)nblk),
                     dim3(kThreads), 0, st, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dq_kernel<D, T, CAUSAL, VARLEN>), dim3((unsigned)nblk),
                     dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

template <int D, class T>
hipError_t launch_d(const BwdArgs& a, bool causal, bool varlen, hipStream_t st) {
  if (varlen)
    return causal ? launch<D, T, true, true>(a, st) : launch<D, T, false, true>(a, st);
  return causal ? launch<D, T, true, false>(a, st) : launch<D, T, false, false>(a, st);
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a, int d, bool bf16, bool causal, bool varlen,
                      hipStream_t st) {
  if ((long)a.T * a.H == 0) return hipSuccess;
  if (d == 128)
    return bf16 ? launch_d<128, BF16>(a, causal, varlen, st) : launch_d<128, F16>(a, causal, varlen, st);
  return bf16 ? launch_d<64, BF16>(a, causal, varlen, st) : launch_d<64, F16>(a, causal, varlen, st);
}

}  // namespace fa
