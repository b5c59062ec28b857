// Split-KV forward for decode shapes: a few query rows (Nq, e.g. the newest token of each
// sequence) against a long cached key/value sequence (Nk). The narration script ("FlashAttention
// 短片讲解稿", segment 适用范围与关键结论) notes that token-by-token decoding has a different shape
// from training and prefill; here the work is one pass over K and V, bound by HBM bandwidth,
// so it is spread over many independent key ranges, each reduced to a partial (O, m, l) by
// the online softmax, and the partials are combined with the block-merge rule of
// "FlashAttention 与算子融合" (section on the two keys of FlashAttention):
//   m = max_s m_s,  l = sum_s l_s exp(m_s - m),  O = sum_s O_s exp(m_s - m) / l.
//
// Query row i stands at position Nk - Nq + i of the sequence; the causal mask hides keys
// after it (for Nq = Nk this is the ordinary causal mask).
//
// Kernel 1 for a single query row (decode1_kernel, the decode step proper): one wave per key
// range on the vector units, loading K and V rows straight into registers (see the kernel).
// Kernel 1 for several query rows (decode_kernel): a workgroup is two (d = 128) or four
// (d = 64) independent waves, one key range each, over one block of 32 query rows of one (b, h). A wave holds the Q rows
// as MFMA B operands and streams its range in 32-key tiles of K and V from HBM straight into
// its own part of LDS (buffer_load_dwordx4 ... lds into a ring of four buffers, three tiles in
// flight, issued from inline assembly so that the compiler does not turn its conservative
// aliasing waits into a wait for the next tile; the wave waits for each tile itself). S^T = K Q^T and O^T += V^T P^T on MFMA as in the forward
// (the matrix cores have ample headroom at these shapes: the bound is the K/V stream).
// Tiles use the dual chunk swizzle of the backward kernels, which keeps both the row-fragment
// reads of K and the transposed reads of V conflict-free.
// Kernel 2 (combine_kernel): four waves per output row merge the S partials (their row
// statistics one per lane, their outputs as independent 16-byte loads over lane groups and
// waves) and write O and LSE.
#include "fa_bwd_common.h"
#include "fa_decode.h"

namespace fa {
namespace dec {
namespace {

using bwd::Lanes;
using bwd::swz;

constexpr int kTK = 32;  // keys per tile
// Independent waves (key ranges) per workgroup and tile buffers per wave: a wave keeps
// kBufs - 1 tiles in flight while it works on one, within 128 KiB of LDS per workgroup.
template <int D>
struct Cfg {
  static constexpr int kWaves = D == 128 ? 2 : 4;
  static constexpr int kBufs = 4;
};
constexpr float kNegInf = -__builtin_inff();
constexpr float kRescaleSlack = 8.0f;  // log2 units the reference max may lag behind
constexpr float kLn2 = 0.69314718055994530942f;

// acc + pair[0] + pair[1] for a packed pair of the element type, with the pair (1, 1) held in
// a register. The pair is taken by value: a bit cast applied directly to a vector element
// expression compiled to a cast of element 0.
template <class T>
__device__ __forceinline__ float add_pair_ones(uint32_t pair, uint32_t ones, float acc) {
  if constexpr (std::is_same_v<T, BF16>)
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair),
                                           __builtin_bit_cast(bf16x2, ones), acc, false);
  else
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pair),
                                  __builtin_bit_cast(f16x2, ones), acc, false);
}

template <int D, class T, bool CAUSAL>
__global__ __launch_bounds__(64 * Cfg<D>::kWaves, 1) void decode_kernel(DecodeArgs a) {
  constexpr int kWaves = Cfg<D>::kWaves, kBufs = Cfg<D>::kBufs;
  constexpr int ROWB = D * 2;          // bytes per K/V row
  constexpr int CPR = D / 8;           // 16-byte chunks per row
  constexpr int TB = kTK * ROWB;       // bytes per tile
  constexpr int RPL = 1024 / ROWB;     // rows per 1 KiB load
  constexpr int LPT = TB / 1024;       // loads per tile and tensor
  constexpr int DC = D / 16, DB = D / 32;
  static_assert(LPT == 4 || LPT == 8, "tile of 4 or 8 KiB");

  // per wave: kBufs buffers of a K tile and a V tile
  constexpr int WAVEB = kBufs * 2 * TB;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kWaves * WAVEB];
  lds_poison(smem, sizeof(smem));
  lds_poison_done();

  const int lane = threadIdx.x & 63, l32 = lane & 31, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nqb = (a.Nq + 31) / 32;
  const int G = (a.S + kWaves - 1) / kWaves;
  uint32_t w = blockIdx.x;
  const int gs = w % G;
  w /= G;
  const int qb = w % nqb;
  w /= nqb;
  const int h = w % a.H;
  const int b = w / a.H;
  const int s = gs * kWaves + wave;  // this wave's key range
  if (s >= a.S) return;
  const int j0 = min(s * a.span, a.Nk);
  const int j1 = min(j0 + a.span, a.Nk);
  const int ntile = (j1 - j0 + kTK - 1) / kTK;

  const uint32_t rstride = (uint32_t)a.H * D * 2;
  const auto rq = make_rsrc(a.q + ((long)b * a.Nq * a.H + h) * D,
                            (uint32_t)(a.Nq - 1) * rstride + D * 2);
  const long kvbase = ((long)b * a.Nk * a.H + h) * D;
  const uint32_t kvbytes = (uint32_t)(a.Nk - 1) * rstride + D * 2;
  const u32x4 rk = rsrc_words(a.k + kvbase, kvbytes);
  const u32x4 rv = rsrc_words(a.v + kvbase, kvbytes);

  const int q0 = qb * 32;
  const int qi = q0 + l32;  // this lane's query row
  u32x4 qreg[DC];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc)
    qreg[dc] = buf_load16(rq, (uint32_t)qi * rstride + (16 * dc + 8 * g) * 2) ^ a.qsign;

  // tile loads: block j (1 KiB) holds rows j*RPL + lane/CPR, physical chunk lane%CPR; one M0
  // per four blocks, the instruction offset selects the block within them
  const uint32_t mine = (uint32_t)(uintptr_t)(bwd::lds_void*)smem + wave * WAVEB;
  const int lrow = lane / CPR, lpc = lane % CPR;
  uint32_t vo[LPT];  // per-lane byte offset of block j relative to the tile's first row
#pragma unroll
  for (int j = 0; j < LPT; ++j) {
    const int row = j * RPL + lrow;
    vo[j] = (uint32_t)row * rstride + (uint32_t)((lpc ^ swz<D>(row)) * 16) - (j & 3) * 1024;
  }
  auto load_tile = [&](int t) __attribute__((always_inline)) {
    const uint32_t base = (uint32_t)(j0 + t * kTK) * rstride;
    const uint32_t lk = __builtin_amdgcn_readfirstlane(mine + (t % kBufs) * 2 * TB);
    const uint32_t lv = lk + TB;
    dma16<0>(rk, lk, base + vo[0]);
    dma16<1024>(rk, lk, base + vo[1]);
    dma16<2048>(rk, lk, base + vo[2]);
    dma16<3072>(rk, lk, base + vo[3]);
    if constexpr (LPT == 8) {
      dma16<0>(rk, lk + 4096, base + vo[4]);
      dma16<1024>(rk, lk + 4096, base + vo[5]);
      dma16<2048>(rk, lk + 4096, base + vo[6]);
      dma16<3072>(rk, lk + 4096, base + vo[7]);
    }
    dma16<0>(rv, lv, base + vo[0]);
    dma16<1024>(rv, lv, base + vo[1]);
    dma16<2048>(rv, lv, base + vo[2]);
    dma16<3072>(rv, lv, base + vo[3]);
    if constexpr (LPT == 8) {
      dma16<0>(rv, lv + 4096, base + vo[4]);
      dma16<1024>(rv, lv + 4096, base + vo[5]);
      dma16<2048>(rv, lv + 4096, base + vo[6]);
      dma16<3072>(rv, lv + 4096, base + vo[7]);
    }
  };

  const Lanes<D> ln(lane);
  constexpr bool kBf16 = std::is_same_v<T, BF16>;
  const uint32_t one2 = kBf16 ? 0x3f803f80u : 0x3c003c00u;
  uint32_t ones = one2;
  asm volatile("" : "+v"(ones));
  const float c2 = a.scale_log2;
  const int qpos = a.Nk - a.Nq + qi;  // position of this lane's query in the sequence

  float mref = kNegInf, lsum = 0.f;
  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};

  // tiles 0 .. kBufs-2 in flight before the loop; iteration t issues tile t + kBufs - 1 and
  // waits for tile t, leaving the later ones in flight (each tile is 2 * LPT loads)
#pragma unroll
  for (int u = 0; u < kBufs - 1; ++u)
    if (u < ntile) load_tile(u);
#pragma unroll 1
  for (int t = 0; t < ntile; ++t) {
    if (t + kBufs - 1 < ntile) load_tile(t + kBufs - 1);
    const int later = min(ntile - 1 - t, kBufs - 1);  // tiles issued after tile t
    if (later >= 3)
      wait_vmcnt<3 * 2 * LPT>();
    else if (later == 2)
      wait_vmcnt<2 * 2 * LPT>();
    else if (later == 1)
      wait_vmcnt<2 * LPT>();
    else
      wait_vmcnt<0>();
    const uint8_t* kt = smem + wave * WAVEB + (t % kBufs) * 2 * TB;
    const uint8_t* vt = kt + TB;
    // S^T = K Q^T: lane (l32, g) holds the scores of query qi for keys 8(r/4) + 4g + r%4
    f32x16 sc = f32x16{};
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) sc = mfma32<T>(ln.row_frag(kt, 0, dc), qreg[dc], sc);
    const int kt0 = j0 + t * kTK;
    const bool masked = kt0 + kTK > j1 || (CAUSAL && kt0 + kTK - 1 > a.Nk - a.Nq + q0);
    if (masked) {
      __builtin_amdgcn_sched_barrier(0);  // a real branch: tail and diagonal tiles only
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kt0 + 8 * (r >> 2) + 4 * g + (r & 3);
        const bool drop = key >= j1 || (CAUSAL && key > qpos);
        sc[r] = drop ? kNegInf : sc[r];
      }
    }
    float mx = sc[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sc[r]);
    const float mnew = pair_max(mx) * c2;  // c2 > 0: a row with no visible key keeps -inf
    const bool need = mnew > mref + kRescaleSlack;
    if (__any(need)) {
      const float alpha = need ? exp2f_hw(mref - mnew) : 1.0f;
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
      if (need) mref = mnew;
    }
    const float mu = mref == kNegInf ? 0.f : mref;
    u32x4 pf[2];
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      float p[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) p[j] = exp2f_hw(fmaf(sc[8 * kc + j], c2, -mu));
      pf[kc] = u32x4{pack2<T>(p[0], p[1]), pack2<T>(p[2], p[3]), pack2<T>(p[4], p[5]),
                     pack2<T>(p[6], p[7])};
#pragma unroll
      for (int e = 0; e < 4; ++e) lsum = add_pair_ones<T>(pf[kc][e], ones, lsum);
    }
    // O^T += V^T P^T over the two 16-key chunks of the tile
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int db = 0; db < DB; ++db)
        oacc[db] = mfma32<T>(ln.tr_frag(vt, kc * 16, db), pf[kc], oacc[db]);
  }

  // partial results of this key range (rows >= Nq are dropped by the buffer bounds)
  const long part = ((long)(b * a.H + h) * a.S + s) * a.Nq;
  const auto ro = make_rsrc(a.opart + part * D, (uint32_t)a.Nq * D * 4);
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const f32x16& x = oacc[db];
      const u32x4 val = {__float_as_uint(x[4 * rr]), __float_as_uint(x[4 * rr + 1]),
                         __float_as_uint(x[4 * rr + 2]), __float_as_uint(x[4 * rr + 3])};
      buf_store16(ro, ((uint32_t)qi * D + db * 32 + 8 * rr + 4 * g) * 4, val);
    }
  const float l = pair_sum(lsum);
  if (g == 0 && qi < a.Nq) {
    a.mpart[part + qi] = mref;
    a.lpart[part + qi] = l;
  }
}

// fdot2 of two packed pairs of the element type, accumulated in fp32.
template <class T>
__device__ __forceinline__ float dot2(uint32_t x, uint32_t y, float acc) {
  if constexpr (std::is_same_v<T, BF16>)
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x),
                                           __builtin_bit_cast(bf16x2, y), acc, false);
  else
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, x), __builtin_bit_cast(f16x2, y),
                                  acc, false);
}

// Sum over each group of N = 8 or 16 consecutive lanes, in every lane of the group: two quad
// permutations (lanes i^1, i^2), then the mirror within 8 lanes and the mirror within 16
// (row_half_mirror, row_mirror) each add the other half's (uniform) sum. Vector adds only.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  auto dpp = [](float v, auto ctrl) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                           decltype(ctrl)::value, 0xf, 0xf, false));
  };
  x += dpp(x, std::integral_constant<int, 0xB1>{});   // quad_perm [1,0,3,2]
  x += dpp(x, std::integral_constant<int, 0x4E>{});   // quad_perm [2,3,0,1]
  x += dpp(x, std::integral_constant<int, 0x141>{});  // row_half_mirror
  if constexpr (N == 16) x += dpp(x, std::integral_constant<int, 0x140>{});  // row_mirror
  return x;
}

// Kernel 1 for a single query row (Nq = 1, the decode step proper): one wave per (b, h, key
// range) on the vector units, no LDS. Lane (rg, c) = (lane / CPR, lane % CPR) takes 16-byte
// chunk c of rows j0 + rg, j0 + rg + RPW, ...: one load instruction brings RPW whole K (or V)
// rows, straight into registers, and a batch of U instructions per tensor is in flight while
// the previous batch is reduced (U = 4 measured up to 2% faster than 8, 12 or 16). The score of a row is four v_dot2 per lane and a sum over
// the row's CPR lanes; P is rounded to the element type as in the other kernels, and
// O += P V is two v_dot2 per pair of dims with the rounded P paired with zero. Each row group
// keeps its own lazily rescaled (O, m, l); the RPW groups are merged at the end. The matrix
// cores would use one of their 32 query columns here; the bound is the K/V stream, and
// without LDS buffers the loads in flight are bounded by registers, not by an LDS ring.
template <int D, class T>
__global__ __launch_bounds__(256) void decode1_kernel(DecodeArgs a) {
  constexpr int CPR = D / 8;      // lanes (16-byte chunks) per row
  constexpr int RPW = 64 / CPR;   // rows per load instruction
  constexpr int U = 4;            // load instructions per tensor and batch
  constexpr int BR = RPW * U;     // rows per batch
  const int lane = threadIdx.x & 63;
  const int rg = lane / CPR, c = lane % CPR;
  const long w = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= (long)a.B * a.H * a.S) return;
  // head-major: the four waves of a workgroup take four heads of one key range, so that
  // together they read adjacent 256-byte pieces of each token's K and V rows (2.4% faster
  // at B1 H16 Nk 131072 d128 than four ranges of one head)
  const int h = (int)(w % a.H);
  const int s = (int)((w / a.H) % a.S);
  const int b = (int)(w / ((long)a.S * a.H));
  const int j0 = min(s * a.span, a.Nk);
  const int j1 = min(j0 + a.span, a.Nk);
  const int nb = (j1 - j0 + BR - 1) / BR;

  const uint32_t rstride = (uint32_t)a.H * D * 2;
  const auto rq = make_rsrc(a.q + ((long)b * a.H + h) * D, D * 2);
  const long kvbase = ((long)b * a.Nk * a.H + h) * D;
  const uint32_t kvbytes = (uint32_t)(a.Nk - 1) * rstride + D * 2;
  const auto rk = make_rsrc(a.k + kvbase, kvbytes);
  const auto rv = make_rsrc(a.v + kvbase, kvbytes);
  const u32x4 qv = buf_load16(rq, c * 16) ^ a.qsign;

  constexpr bool kBf16 = std::is_same_v<T, BF16>;
  uint32_t ones = kBf16 ? 0x3f803f80u : 0x3c003c00u;
  asm volatile("" : "+v"(ones));
  const float c2 = a.scale_log2;
  float mref = kNegInf, lsum = 0.f, o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = 0.f;

  auto load = [&](u32x4 (&kb)[U], u32x4 (&vb)[U], int i) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t off = (uint32_t)(j0 + i * BR + u * RPW + rg) * rstride + c * 16;
      kb[u] = buf_load16(rk, off);
      vb[u] = buf_load16(rv, off);
    }
  };
  auto reduce = [&](const u32x4 (&kb)[U], const u32x4 (&vb)[U], int i)
                    __attribute__((always_inline)) {
    float sv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = dot2<T>(kb[u][e], qv[e], acc);
      sv[u] = group_sum<CPR>(acc);
      if (j0 + i * BR + u * RPW + rg >= j1) sv[u] = kNegInf;  // past the range
    }
    float mx = sv[0];
#pragma unroll
    for (int u = 1; u < U; ++u) mx = fmaxf(mx, sv[u]);
    const float mnew = mx * c2;  // c2 > 0: a group with no row in range keeps -inf
    const bool need = mnew > mref + kRescaleSlack;
    if (__any(need)) {
      const float alpha = need ? exp2f_hw(mref - mnew) : 1.0f;
      lsum *= alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] *= alpha;
      if (need) mref = mnew;
    }
    const float mu = mref == kNegInf ? 0.f : mref;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t plo = pack2<T>(exp2f_hw(fmaf(sv[u], c2, -mu)), 0.f);  // (p, 0)
      const uint32_t phi = plo << 16;                                       // (0, p)
      lsum = dot2<T>(plo, ones, lsum);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o[2 * e] = dot2<T>(vb[u][e], plo, o[2 * e]);
        o[2 * e + 1] = dot2<T>(vb[u][e], phi, o[2 * e + 1]);
      }
    }
  };

  u32x4 ka[U], va[U], kn[U], vn[U];
  if (nb > 0) load(ka, va, 0);
#pragma unroll 1
  for (int i = 0; i < nb; i += 2) {
    if (i + 1 < nb) load(kn, vn, i + 1);
    reduce(ka, va, i);
    if (i + 1 < nb) {
      if (i + 2 < nb) load(ka, va, i + 2);
      reduce(kn, vn, i + 1);
    }
  }

  // merge the RPW row groups (lanes c, c + CPR, ... hold the same dims)
  float m = mref;
#pragma unroll
  for (int x = CPR; x < 64; x *= 2) m = fmaxf(m, __shfl_xor(m, x));
  const float f = m == kNegInf ? 0.f : exp2f_hw(mref - m);
  lsum *= f;
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] *= f;
#pragma unroll
  for (int x = CPR; x < 64; x *= 2) {
    lsum += __shfl_xor(lsum, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] += __shfl_xor(o[e], x);
  }
  const long part = (long)(b * a.H + h) * a.S + s;  // Nq = 1
  if (rg == 0) {
    const auto ro = make_rsrc(a.opart + part * D, D * 4);
    buf_store16(ro, c * 32, u32x4{__float_as_uint(o[0]), __float_as_uint(o[1]),
                                  __float_as_uint(o[2]), __float_as_uint(o[3])});
    buf_store16(ro, c * 32 + 16, u32x4{__float_as_uint(o[4]), __float_as_uint(o[5]),
                                       __float_as_uint(o[6]), __float_as_uint(o[7])});
  }
  if (lane == 0) {
    a.mpart[part] = m;
    a.lpart[part] = lsum;
  }
}

// One workgroup of four waves per output row (b, q, h): merge the S partials. Every wave
// reduces the row statistics of all partials (one per lane, 64 at a time); the partial
// outputs are then split over the four waves and read as independent 16-byte loads, lane
// group j of a wave taking partials s = j, j + 64/LPR, ... of its share over D/4 lanes of four
// dims each. The groups' sums are added across lanes, the waves' sums through LDS. (One wave
// per row walking all partials was bound by the latency of its loads at large S.)
template <int D, class T>
__global__ __launch_bounds__(256) void combine_kernel(DecodeArgs a) {
  constexpr int LPR = D / 4;      // lanes per partial row (four dims each)
  constexpr int SPW = 64 / LPR;   // partials read side by side by one wave
  constexpr int NW = 4;           // waves per row
  __shared__ f32x4 wsum[NW][LPR];
  lds_poison(wsum, sizeof(wsum));
  lds_poison_done();
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const long row = blockIdx.x;
  const int qi = row % a.Nq;
  const long bh = row / a.Nq;  // b * H + h
  const int h = bh % a.H, b = bh / a.H;
  const long part0 = bh * a.S * a.Nq + qi;  // partial s of this row at part0 + s * Nq

  // m = max_s m_s, then l = sum_s l_s 2^(m_s - m) over the ranges that saw a key
  float m = kNegInf;
  for (int s = lane; s < a.S; s += 64) m = fmaxf(m, a.mpart[part0 + (long)s * a.Nq]);
#pragma unroll
  for (int x = 32; x >= 1; x >>= 1) m = fmaxf(m, __shfl_xor(m, x));
  float l = 0.f;
  if (m != kNegInf)
    for (int s = lane; s < a.S; s += 64) {
      const long p = part0 + (long)s * a.Nq;
      const float ls = a.lpart[p];
      if (ls > 0.f) l += ls * exp2f_hw(a.mpart[p] - m);
    }
#pragma unroll
  for (int x = 32; x >= 1; x >>= 1) l += __shfl_xor(l, x);

  const int c4 = (lane % LPR) * 4;  // this lane's first dim
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (m != kNegInf) {
#pragma unroll 8
    for (int s = wave * SPW + lane / LPR; s < a.S; s += NW * SPW) {
      const long p = part0 + (long)s * a.Nq;
      const float ls = a.lpart[p];
      const float wgt = ls > 0.f ? exp2f_hw(a.mpart[p] - m) : 0.f;
      const f32x4 op = *reinterpret_cast<const f32x4*>(a.opart + p * D + c4);
      acc += wgt * op;
    }
  }
#pragma unroll
  for (int x = LPR; x < 64; x <<= 1)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += __shfl_xor(acc[e], x);
  if (lane < LPR) wsum[wave][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
  if (lane < LPR) {
#pragma unroll
    for (int w2 = 1; w2 < NW; ++w2) acc += wsum[w2][lane];
  }
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  if (lane < LPR) {
    uint16_t* o = a.o + (((long)b * a.Nq + qi) * a.H + h) * D + c4;
    *reinterpret_cast<u32x2*>(o) = u32x2{pack2<T>(acc[0] * inv, acc[1] * inv),
                                         pack2<T>(acc[2] * inv, acc[3] * inv)};
  }
  if (lane == 0) a.lse[bh * a.Nq + qi] = l > 0.f ? (m + log2f_hw(l)) * kLn2 : kNegInf;
}

template <int D, class T, bool CAUSAL>
hipError_t launch(const DecodeArgs& a, hipStream_t st) {
  constexpr int kWaves = Cfg<D>::kWaves;
  if (a.Nq == 1) {  // query row Nk - 1 sees every key: the mask never applies
    const long waves = (long)a.B * a.H * a.S;
    hipLaunchKernelGGL((decode1_kernel<D, T>), dim3((unsigned)((waves + 3) / 4)), dim3(256), 0,
                       st, a);
  } else {
    const long nqb = (a.Nq + 31) / 32;
    const long G = (a.S + kWaves - 1) / kWaves;
    const long grid1 = G * nqb * a.H * a.B;
    hipLaunchKernelGGL((decode_kernel<D, T, CAUSAL>), dim3((unsigned)grid1), dim3(64 * kWaves),
                       0, st, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long rows = (long)a.B * a.H * a.Nq;
  hipLaunchKernelGGL((combine_kernel<D, T>), dim3((unsigned)rows), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int D, class T>
hipError_t launch_c(const DecodeArgs& a, bool causal, hipStream_t st) {
  return causal ? launch<D, T, true>(a, st) : launch<D, T, false>(a, st);
}

}  // namespace
}  // namespace dec

int decode_splits(int B, int Nq, int Nk, int H, int d, int requested) {
  const long tiles = (Nk + dec::kTK - 1) / dec::kTK;  // at least one tile per range
  if ((long)B * H * Nq <= 0 || tiles <= 0) return 1;   // nothing to split
  long s = requested;
  if (s <= 0 && Nq == 1) {
    // single-row kernel: about one wave per SIMD of a 256-CU part, each streaming a long
    // range with its own loads in flight (measured best: at decode_8k and decode_128k, 1024
    // waves beat 512, 2048 and 4096)
    const long units = (long)B * H;
    s = (1024 + units - 1) / units;
  } else if (s <= 0) {
    // about one workgroup per CU of a 256-CU part: long ranges keep each wave's stream of
    // tiles going, which is what the HBM bandwidth needs
    const long units = (long)B * H * ((Nq + 31) / 32);
    const int nw = d == 128 ? dec::Cfg<128>::kWaves : dec::Cfg<64>::kWaves;
    s = nw * ((256 + units - 1) / units);
  }
  if (s > tiles) s = tiles;
  return (int)(s < 1 ? 1 : s);
}

int decode_span(int Nk, int splits) {
  const int per = (Nk + splits - 1) / splits;
  return (per + dec::kTK - 1) / dec::kTK * dec::kTK;
}

hipError_t launch_decode(const DecodeArgs& a, int d, bool bf16, bool causal, hipStream_t st) {
  if ((long)a.B * a.H * a.Nq == 0) return hipSuccess;
  if (d == 128)
    return bf16 ? dec::launch_c<128, BF16>(a, causal, st) : dec::launch_c<128, F16>(a, causal, st);
  return bf16 ? dec::launch_c<64, BF16>(a, causal, st) : dec::launch_c<64, F16>(a, causal, st);
}

}  // namespace fa
