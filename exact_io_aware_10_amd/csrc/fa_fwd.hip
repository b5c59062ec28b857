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
//  - one workgroup = 4 waves = 128 query rows of one (batch or sequence, head); wave w
//    owns 32 consecutive rows, held as MFMA B operands in registers for the whole loop.
//  - key/value tiles of 64 rows go from HBM/L2 straight into LDS (buffer_load ... lds,
//    bounds-checked so rows past the sequence read as zero), double buffered: the loads
//    of tile t+1 are issued before tile t is computed. Rows are stored unpadded with an
//    XOR swizzle of their 16-byte chunks that keeps the operand reads conflict-free.
//  - scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16: each lane then
//    holds 32 scores of ONE query row (the other 32 sit in lane l^32), so row max and row
//    sum need only per-lane work plus one v_permlane32_swap.
//  - P^T leaves the accumulators already in the B-operand layout of the next MFMA,
//    O^T += V^T P^T. The V^T operand is read from the row-major V tile with
//    ds_read_b64_tr_b16: in each group of 16 lanes, lane i names 4 consecutive values
//    (row i of a 16x4 block) and lane j receives column j%4 of rows j/4, j/4+4, j/4+8,
//    j/4+12. Lane i addresses key k0 + i/4, dims d0 + 4(i%4), so lane j receives dim
//    d0 + j of keys k0..k0+3; two such reads give the 8 keys of one MFMA operand, in the
//    key order of the P^T registers.
//  - exp2 domain: scores are multiplied by scale*log2(e) in the exponent's FMA. The
//    running max used as the exponent's reference is only moved when the true row max
//    exceeds it by more than 8 (in log2 units), so the rescale of the output accumulator is
//    rare; O = acc / l and LSE = (m_ref + log2 l) ln 2 are exact for any reference.
#include <type_traits>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

#ifndef FA_FWD_OCC
#define FA_FWD_OCC 2  // workgroups per CU the register budget is sized for
#endif

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBK = 64;                   // keys per tile
constexpr float kRescaleSlack = 8.0f;     // log2 units the reference max may lag behind
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kNegInf = -__builtin_inff();

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

// 16-byte-chunk swizzles of a tile row r (D/8 chunks per row).
// K rows are read as 32 rows x one chunk (ds_read_b128): chunk c of row r sits at c ^ (r % D/8).
// V rows are read 4 rows x 4 chunks per 32 lanes (ds_read_b64_tr_b16).
template <int D>
__device__ __forceinline__ int kswz(int r) { return r & (D / 8 - 1); }
template <int D>
__device__ __forceinline__ int vswz(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }

template <int D, class T, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(kThreads, FA_FWD_OCC) void fwd_kernel(FwdArgs a) {
  constexpr int BQ = 32 * kWaves;
  constexpr int ROWB = D * 2;                 // bytes per K/V row in LDS
  constexpr int CPR = D / 8;                  // 16-byte chunks per row
  constexpr int TILEB = kBK * ROWB;           // bytes per tile
  constexpr int RPL = 1024 / ROWB;            // rows per 1 KiB direct load (one per wave)
  constexpr int LPW = TILEB / 1024 / kWaves;  // direct loads per wave per tile
  constexpr int DC = D / 16;                  // 16-wide d chunks of Q K^T
  constexpr int DB = D / 32;                  // 32-wide d blocks of the output

  // separate objects per buffer: the compiler can then see that the direct loads into one
  // buffer do not alias the reads of the other and need not wait for them
  __shared__ __attribute__((aligned(1024))) uint8_t Ks0[TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t Ks1[TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t Vs0[TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t Vs1[TILEB];

  const int tid = threadIdx.x;
  const int lane = tid & 63, l32 = lane & 31, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

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

  const int wq0 = q0 + wave * 32;  // first query row of this wave
  const int qi = wq0 + l32;        // this lane's query row
  const int kend = CAUSAL ? (L < q0 + BQ ? L : q0 + BQ) : L;
  const int ntiles = (kend + kBK - 1) / kBK;

  // ---- Q rows into registers (B operand of S^T = K Q^T): d = 16*dc + 8g .. +7
  u32x4 qreg[DC];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc)
    qreg[dc] = buf_load16(rq, (uint32_t)qi * rstride + (16 * dc + 8 * g) * 2) ^ a.qsign;

  // ---- direct HBM/L2 -> LDS tile loads: this wave fills LPW 1 KiB blocks of each tile;
  // lane l of a block writes row blk*RPL + l/CPR, physical chunk l%CPR.
  const int lrow = lane / CPR, lpc = lane % CPR;
  auto tload = [&](__amdgpu_buffer_rsrc_t rs, uint8_t* tile, int t, bool is_k) {
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      const int blk = wave * LPW + j;
      const int row = blk * RPL + lrow;
      const int c = lpc ^ (is_k ? kswz<D>(row) : vswz<D>(row));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (lds_void*)(tile + blk * 1024), 16,
          (uint32_t)(t * kBK + row) * rstride + c * 16, 0, 0, 0);
    }
  };

  // ---- per-lane LDS byte offsets of the MFMA operand reads
  // K (A operand of S^T): row kb*32 + l32, logical chunk 2*dc + g
  const int krow_off = l32 * ROWB;
  // V^T (A operand of O^T): tr reads of keys kc*16 + 4g + i/4 (+8), dims db*32 + 16G + 4(i%4)
  const int i16 = lane & 15, G = (lane >> 4) & 1;
  const int vkey = 4 * g + (i16 >> 2);
  const int vsw = vswz<D>(vkey);
  const int vhalf = 8 * (i16 & 1);

  float mref = kNegInf, lsum = 0.f;
  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
  const float c2 = a.scale_log2;

  // one pipeline step on tile t held in buffer B (B = t % 2): issue the direct loads of
  // tile t+1 into the other buffer, compute tile t, then wait for this wave's loads and
  // meet the other waves at the barrier.
  auto step = [&](auto bsel, int t) {
    constexpr int B = decltype(bsel)::value;
    const uint8_t* kt = B ? Ks1 : Ks0;
    const uint8_t* vt = B ? Vs1 : Vs0;
    if (t + 1 < ntiles) {
      tload(rk, B ? Ks0 : Ks1, t + 1, true);
      tload(rv, B ? Vs0 : Vs1, t + 1, false);
    }
    const int kt0 = t * kBK;
    const bool active = !CAUSAL || kt0 <= wq0 + 31;
    if (active) {
      // S^T tile: two 32-key blocks
      f32x16 s[2];
      s[0] = s[1] = f32x16{};
#pragma unroll
      for (int dc = 0; dc < DC; ++dc)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int c = (2 * dc + g) ^ kswz<D>(l32);  // row kb*32 + l32 has the same swizzle
          const u32x4 ka =
              *reinterpret_cast<const u32x4*>(kt + kb * 32 * ROWB + krow_off + c * 16);
          s[kb] = mfma32<T>(ka, qreg[dc], s[kb]);
        }

      const bool masked = kt0 + kBK > L || (CAUSAL && kt0 + kBK - 1 > wq0);
      if (masked) {
        // a real branch: keeps the per-element mask out of the unmasked tiles
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kt0 + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
            if (key >= L || (CAUSAL && key > qi)) s[kb][r] = kNegInf;
          }
      }
      float mx = s[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      const float mnew = pair_max(mx) * c2;  // c2 > 0: a fully masked row keeps -inf
      const bool need = mnew > mref + kRescaleSlack;
      if (__any(need)) {
        const float alpha = need ? exp2f_hw(mref - mnew) : 1.0f;
        lsum *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
        if (need) mref = mnew;
      }
      // masked scores are -inf and c2 > 0, so their exponent is exactly 0
      const float mu = mref == kNegInf ? 0.f : mref;
      u32x4 pf[4];
      float ls = lsum;
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        float p[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int r = 8 * kc + j;
          p[j] = exp2f_hw(fmaf(s[r >> 4][r & 15], c2, -mu));
        }
        // P rounded to the element type; the row sum adds exactly the rounded values
        pf[kc] = u32x4{pack2<T>(p[0], p[1]), pack2<T>(p[2], p[3]), pack2<T>(p[4], p[5]),
                       pack2<T>(p[6], p[7])};
#pragma unroll
        for (int e = 0; e < 4; ++e) ls = add_pair<T>(pf[kc][e], ls);
      }
      lsum = ls;

      // O^T += V^T P^T over four 16-key chunks
#pragma unroll
      for (int kc = 0; kc < 4; ++kc)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int c = (db * 4 + 2 * G + ((i16 & 3) >> 1)) ^ vsw;
          const int off = (kc * 16 + vkey) * ROWB + c * 16 + vhalf;
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vt + off));
          const i16x4 hi =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vt + off + 8 * ROWB));
          const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
          const u32x4 va = {lo2[0], lo2[1], hi2[0], hi2[1]};
          oacc[db] = mfma32<T>(va, pf[kc], oacc[db]);
        }
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's tile t+1 loads have landed in LDS
    __syncthreads();
  };

  tload(rk, Ks0, 0, true);
  tload(rv, Vs0, 0, false);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int t = 0; t < ntiles; t += 2) {
    step(std::integral_constant<int, 0>{}, t);
    if (t + 1 < ntiles) step(std::integral_constant<int, 1>{}, t + 1);
  }

  // ---- epilogue: O = acc / l (rows >= L are dropped by the buffer bounds), LSE
  const float l = pair_sum(lsum);
  const float inv = l > 0.f ? 1.0f / l : 0.f;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const f32x16& o = oacc[db];
      u32x2 v = {pack2<T>(o[4 * rr] * inv, o[4 * rr + 1] * inv),
                 pack2<T>(o[4 * rr + 2] * inv, o[4 * rr + 3] * inv)};
      buf_store8(ro, (uint32_t)qi * rstride + (db * 32 + 8 * rr + 4 * g) * 2, v);
    }
  if (g == 0 && qi < L) lse[qi] = l > 0.f ? (mref + log2f_hw(l)) * kLn2 : kNegInf;
}

template <int D, class T, bool CAUSAL, bool VARLEN>
hipError_t launch(const FwdArgs& a, hipStream_t st) {
  constexpr int BQ = 32 * kWaves;
  const int nqb = (a.N + BQ - 1) / BQ;
  const long total = (long)nqb * a.H * a.B;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL((fwd_kernel<D, T, CAUSAL, VARLEN>), dim3((unsigned)total),
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
