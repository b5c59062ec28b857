// FP8 forward attention for gfx950: q, k, v stored as OCP FP8 E4M3 codes with one fp32
// descale factor per tensor (stored value = descale * code value), output in bf16.
//
// The computation is the forward of fa_fwd.hip ("FlashAttention 详解（零基础入门）" §5-§6
// tiled loop with online softmax, deferred normalisation of "FlashAttention 短片讲解稿"
// segment 第二招, causal mask inside the kernel) on the FP8 path that "FlashAttention 与算子融合"
// lists for FlashAttention-3 (代际演进 table and 工程实践 precision note): both products run
// on the FP8 matrix cores, v_mfma_f32_32x32x64_f8f6f4 (e4m3 x e4m3, fp32 accumulation),
// which do twice the work per cycle of the 16-bit ones.
//
//  - S^T = K Q^T: the descales of q and k and the softmax scale fold into the exponent's
//    scale c = |scale| q_descale k_descale log2(e); the products of two e4m3 values are exact
//    in fp32, so the scores carry only the accumulation's rounding.
//  - P is rounded to e4m3 (nearest even, v_cvt_pk_fp8_f32) before O^T += V^T P^T. With the
//    lagging reference max (at most 8 log2 units behind the row max) P <= 2^8 < 448, the
//    largest e4m3 value, so nothing saturates.
//  - The row sum l is computed by the matrix cores too: an extra MFMA per 64 keys with an
//    all-ones A operand gives, in every accumulator row, the column sums of P^T, i.e. the
//    sum of exactly the rounded P values that enter P V, with no vector instructions.
//  - v_descale scales the output once, in the epilogue: O = v_descale * acc / l.
//
// Layout on the chip, as in the 16-bit kernel: 8 waves = 256 query rows per workgroup, the
// two groups of four waves ping-pong between matrix and vector phases, 128-key tiles of K
// and V (16 KiB each at d = 128) go HBM -> LDS with buffer_load ... lds, double buffered,
// issued by group A during its matrix phases. At these rates the vector phase (64 exp2 per
// lane per tile at a quarter of the vector rate, plus the max, the exponent's FMA and the
// conversions) is the longer one, so the kernel is bound by vector issue, not by the matrix
// cores.
//
// Operand layouts (lane l, l32 = l % 32, g = l / 32). The 32x32x64 MFMA takes 32 bytes per
// lane for A and for B; any assignment of (lane half, byte) to the contraction index that
// both operands share gives the same product. Here byte b of lane l is k = 32g + b for the
// scores (k = head dim), and for P V the keys of the S^T accumulators in register order:
// byte b of lane l is key kappa(g, b) = 32(b/16) + 8((b%16)/4) + 4g + b%4 of a 64-key half.
// The V^T operand is read from the row-major V tile with ds_read_b64_tr_b8, which works in
// groups of 16 lanes: lane j of a group receives byte j%8 of the eight 8-byte rows named by
// the group's even lanes (j < 8) or odd lanes (j >= 8). Even lane 2i names key kappa(g, 8p+i)
// at dims d0..d0+7 and odd lane 2i+1 the same key at dims d0+8..d0+15, so lane j of the group
// receives dim d0 + j of eight keys: 8 bytes of its A operand per read, four reads per MFMA.
#include <type_traits>
#include <utility>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace f8 {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBK = 128;        // keys per tile
constexpr int kKB = kBK / 32;   // 32-key blocks of S^T per tile
constexpr int kKH = kBK / 64;   // 64-key halves of P per tile (one MFMA k-step each)
constexpr float kRescaleSlack = 8.0f;  // log2 units the reference max may lag behind
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kNegInf = -__builtin_inff();
constexpr uint32_t kOnes = 0x38383838u;  // four e4m3 codes of 1.0

// C[32x32] += A[32x64] B[64x32], e4m3 operands, fp32 accumulation; C register r of lane l
// is C[8(r/4) + 4g + r%4][l32] as for the 16-bit MFMA. The scaled form of the instruction
// with zero scale operands compiles to the unscaled v_mfma_f32_32x32x64_f8f6f4.
__device__ __forceinline__ f32x16 mfma_f8(u32x8 a, u32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(__builtin_bit_cast(i32x8, a),
                                                         __builtin_bit_cast(i32x8, b), c, 0, 0,
                                                         0, 0, 0, 0);
}

// Four fp32 values -> four e4m3 codes in one dword (byte 0 = x0), round to nearest even.
// Each conversion writes one 16-bit half and keeps the other; the first one's kept half is
// overwritten by the second, so it starts from x0's own bits rather than a zeroed register.
__device__ __forceinline__ uint32_t pack4_e4m3(float x0, float x1, float x2, float x3) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, __builtin_bit_cast(int, x0), false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, w, true);
  return (uint32_t)w;
}

// 16-byte chunk swizzle of tile row r: logical chunk c is stored at c ^ swz(r). LDS serves
// 256 bytes per cycle from 64 banks; a 16-byte read is served 8 lanes at a time and an
// 8-byte read 16 or 32 lanes at a time. The swizzle keeps both operand reads conflict-free:
//  - K (ds_read_b128): 8 lanes read rows r0..r0+7 at one logical chunk;
//  - V (ds_read_b64_tr_b8): a 16-lane group reads 8 keys {k0..k0+3, k0+8..k0+11}
//    (k0 = 0 or 4 mod 16) at one logical chunk, two groups side by side read the next chunk.
// Both patterns depend on r % 16 only, so one swizzle serves every 16-row band.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128)  // 128-byte rows: rows r and r+1 are in different bank halves
    return 2 * (((r >> 1) & 3) ^ ((r >> 2) & 2));
  else  // 64-byte rows, 4 chunks: rows r, r+4, r+8, r+12 share banks
    return (2 * ((r >> 3) & 1)) ^ ((r >> 2) & 1);
}

#ifndef FA_FP8_PREFETCH
#define FA_FP8_PREFETCH 3  // MFMAs of look-ahead for the LDS operand reads (0: compiler order)
#endif

// Instruction order of one matrix phase: per 64-key half, DB MFMAs of O += P V (four
// transposed reads each) and the row-sum MFMA (no reads), then the score MFMAs (two reads
// each). Each MFMA's reads are issued PD MFMAs ahead, so their latency is covered by the
// wave's own matrix work; the other wave on the SIMD is in its vector phase.
template <int MASK, int N>
__device__ __forceinline__ void sched_group() {
  if constexpr (N > 0) __builtin_amdgcn_sched_group_barrier(MASK, N, 0);
}
constexpr int kSchedMfma = 0x008, kSchedDsRead = 0x100;
template <int DB>
constexpr int xreads(int m) { return m < kKH * (DB + 1) ? (m % (DB + 1) < DB ? 4 : 0) : 2; }
template <int DB>
constexpr int xreads_before(int n) {
  int r = 0;
  for (int m = 0; m < n; ++m) r += xreads<DB>(m);
  return r;
}
template <int DB, int NM, int PD, int M>
__device__ __forceinline__ void xsched_step() {
  sched_group<kSchedMfma, 1>();
  if constexpr (M + PD < NM) sched_group<kSchedDsRead, xreads<DB>(M + PD)>();
}
template <int DB, int PD, int... M>
__device__ __forceinline__ void xsched(std::integer_sequence<int, M...>) {
  constexpr int NM = sizeof...(M);
  sched_group<kSchedDsRead, xreads_before<DB>(PD < NM ? PD : NM)>();
  (xsched_step<DB, NM, PD, M>(), ...);
}

// STREAM (no mask): one workgroup per CU takes items blockIdx.x, blockIdx.x + G, ... of the
// XCD-remapped work list as one stream of key/value tiles (as the 16-bit forward's stream
// form): the loads run on into the next item's tiles, the next item's Q rows are loaded after
// their last use, and an item's output is stored in the vector phase that starts the next.
template <int D, bool CAUSAL, bool STREAM>
__global__ __launch_bounds__(kThreads, 1) void fwd_fp8_kernel(Fp8FwdArgs a) {
  static_assert(!STREAM || !CAUSAL, "the stream form is for unmasked launches");
  constexpr int BQ = 32 * kWaves;
  constexpr int ROWB = D;                     // bytes per K/V row in LDS
  constexpr int CPR = D / 16;                 // 16-byte chunks per row
  constexpr int TILEB = kBK * ROWB;           // bytes per tile
  constexpr int RPL = 1024 / ROWB;            // rows per 1 KiB direct load
  constexpr int LPW = TILEB / 1024 / (kWaves / 2);  // direct loads per group-B wave per tile
  constexpr int DC = D / 64;                  // 64-wide d chunks of Q K^T
  constexpr int DB = D / 32;                  // 32-wide d blocks of the output

  // four tile buffers: K at 0 and TILEB, V at 2 TILEB and 3 TILEB; switching buffers is an
  // XOR of bit log2(TILEB) of the per-lane offsets
  __shared__ __attribute__((aligned(1024))) uint8_t smem[4 * TILEB];
  lds_poison(smem, sizeof(smem));
  lds_poison_done();
  uint8_t* const Ks0 = smem;
  uint8_t* const Ks1 = smem + TILEB;
  uint8_t* const Vs0 = smem + 2 * TILEB;
  uint8_t* const Vs1 = smem + 3 * TILEB;

  const int tid = threadIdx.x;
  const int lane = tid & 63, l32 = lane & 31, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;                  // waves w and w+4 share a SIMD
  const int rb = 2 * (wave & 3) + grp;

  // ---- work item: (query block, head, batch)
  const int nqb = (a.N + BQ - 1) / BQ;
  const uint32_t total = (uint32_t)nqb * a.H * a.B;
  auto stream_item = [&](int j, int& iqb, int& ih, int& ibs) __attribute__((always_inline)) {
    const uint32_t w = xcd_remap(blockIdx.x + (uint32_t)j * gridDim.x, total);
    iqb = w % nqb;
    ih = (w / nqb) % a.H;
    ibs = w / (nqb * a.H);
  };
  const int nitems = STREAM ? (int)((total - blockIdx.x + gridDim.x - 1) / gridDim.x) : 1;
  int qb, h, bs;
  if (STREAM) {
    stream_item(0, qb, h, bs);
  } else if (CAUSAL) {  // longest rows first over whole slices per XCD
    int rank, bh;
    causal_order(blockIdx.x, a.B * a.H, rank, bh);
    qb = nqb - 1 - rank;
    h = bh % a.H;
    bs = bh / a.H;
  } else {
    const uint32_t w = xcd_remap(blockIdx.x, gridDim.x);
    qb = w % nqb;
    h = (w / nqb) % a.H;
    bs = w / (nqb * a.H);
  }
  const int L = a.N;
  const long tok0 = (long)bs * a.N;
  int q0 = qb * BQ;
  if (q0 >= L) return;

  const uint32_t rstride = (uint32_t)a.H * D;  // bytes between consecutive tokens (fp8)
  long base = (tok0 * a.H + h) * D;
  const uint32_t nbytes = (uint32_t)(L - 1) * rstride + D;
  auto ro = make_rsrc(a.o + base, 2 * nbytes);  // bf16 output: twice the byte offsets
  float* lse = a.lse + ((long)bs * a.H + h) * a.N;

  int wq0 = q0 + rb * 32;
  int qi = wq0 + l32;
  const int kend = CAUSAL ? (L < q0 + BQ ? L : q0 + BQ) : L;
  const int ntiles = (kend + kBK - 1) / kBK;
  const int nstream = nitems * ntiles;  // tiles of the whole stream

  // ---- Q rows into registers (B operand of S^T = K Q^T): d = 64 dc + 32 g + byte
  u32x8 qreg[DC];
  auto load_q = [&](long qbase, int row) __attribute__((always_inline)) {
    const auto rq = make_rsrc(a.q + qbase, nbytes);
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
      const uint32_t off = (uint32_t)row * rstride + 64 * dc + 32 * g;
      const u32x4 lo = buf_load16(rq, off) ^ a.qsign;
      const u32x4 hi = buf_load16(rq, off + 16) ^ a.qsign;
      qreg[dc] = u32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  };
  load_q(base, qi);

  // ---- direct HBM/L2 -> LDS tile loads: this wave fills LPW 1 KiB blocks of a tile; lane l
  // of a block writes row blk*RPL + l/CPR, physical chunk l%CPR.
  const int lrow = lane / CPR, lpc = lane % CPR;
  // The loads are issued from inline assembly (dma16): with the builtin the compiler would
  // make the matrix phase's LDS reads wait for these loads to land.
  const u32x4 wk = rsrc_words(a.k + base, nbytes), wv = rsrc_words(a.v + base, nbytes);
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
  auto tload_w = [&](u32x4 words, uint8_t* tile, int t) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      const int blk = (wave & 3) * LPW + j;
      const int row = blk * RPL + lrow;
      const int c = lpc ^ swz<D>(row);
      const uint32_t m0 =
          __builtin_amdgcn_readfirstlane(lds0 + (uint32_t)(tile - smem) + blk * 1024);
      dma16<0>(words, m0, (uint32_t)(t * kBK + row) * rstride + c * 16);
    }
  };
  // K or V resource words of item j of the stream form
  auto item_words = [&](int j, bool is_k) __attribute__((always_inline)) {
    int jqb, jh, jbs;
    stream_item(j, jqb, jh, jbs);
    return rsrc_words((is_k ? a.k : a.v) + ((long)jbs * a.N * a.H + jh) * D, nbytes);
  };

  // ---- per-lane LDS byte offsets of the operand reads (swizzle folded in; the 32-key block,
  // the 64-key half and the read index are immediates).
  // K (A operand of S^T): row 32 kb + l32, logical chunks 4 dc + 2 g + hh (hh = 0, 1).
  const int ksw = swz<D>(l32);
  int kcur[DC][2];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) kcur[dc][hh] = l32 * ROWB + ((4 * dc + 2 * g + hh) ^ ksw) * 16;
  // V^T (A operand of O^T): lane i of a 16-lane group G4 names key kappa(g, 8p + i/2), bytes
  // 8 (i%2) .. +7 of logical chunk 2 db + G4 % 2. The key is 64 kh + 32 (p/2) + 16 (p%2) + vkey
  // with vkey = 8 (i/8) + 4 g + (i/2) % 4; the swizzle only sees vkey (< 16).
  const int G4 = lane >> 4, i16 = lane & 15;
  const int vkey = 8 * (i16 >> 3) + 4 * g + ((i16 >> 1) & 3);
  const int vsw = swz<D>(vkey);
  int vcur[DB];  // V buffer 1 before tile 0
#pragma unroll
  for (int db = 0; db < DB; ++db)
    vcur[db] = 3 * TILEB + vkey * ROWB + ((2 * db + (G4 & 1)) ^ vsw) * 16 + 8 * (i16 & 1);

  float mref = kNegInf;
  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
  f32x16 lacc = f32x16{};  // every register holds the row sum of this lane's query
  u32x8 ones = u32x8{kOnes, kOnes, kOnes, kOnes, kOnes, kOnes, kOnes, kOnes};
  asm volatile("" : "+v"(ones));
  const float c2 = a.scale_log2;

  const int nt_w = CAUSAL ? min(ntiles, (wq0 + 31 + kBK) / kBK) : ntiles;  // this wave's tiles
  f32x16 s[kKB];
  u32x8 pf[kKH];

  // Matrix phase X(t) = [O += P(t-1) V(t-1), l += column sums of P(t-1); S(t) = K(t) Q^T].
  auto xphase = [&](auto HAS_PV, auto HAS_S) __attribute__((always_inline)) {
    if constexpr (decltype(HAS_PV)::value) {
#pragma unroll
      for (int kh = 0; kh < kKH; ++kh) {
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          u32x8 va;
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const uint8_t* src =
                smem + vcur[db] + (64 * kh + 32 * (p >> 1) + 16 * (p & 1)) * ROWB;
            const i32x2 r = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)src);
            va[2 * p] = (uint32_t)r[0];
            va[2 * p + 1] = (uint32_t)r[1];
          }
          oacc[db] = mfma_f8(va, pf[kh], oacc[db]);
        }
        lacc = mfma_f8(ones, pf[kh], lacc);
      }
    }
    if constexpr (decltype(HAS_S)::value) {
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb) s[kb] = f32x16{};
#pragma unroll
      for (int dc = 0; dc < DC; ++dc)
#pragma unroll
        for (int kb = 0; kb < kKB; ++kb) {
          const u32x4 lo = *reinterpret_cast<const u32x4*>(smem + kcur[dc][0] + kb * 32 * ROWB);
          const u32x4 hi = *reinterpret_cast<const u32x4*>(smem + kcur[dc][1] + kb * 32 * ROWB);
          const u32x8 ka = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          s[kb] = mfma_f8(ka, qreg[dc], s[kb]);
        }
    }
    if constexpr (decltype(HAS_PV)::value && decltype(HAS_S)::value && FA_FP8_PREFETCH > 0)
      xsched<DB, FA_FP8_PREFETCH>(
          std::make_integer_sequence<int, kKH * (DB + 1) + kKB * DC>{});
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
      kcur[dc][0] ^= TILEB;
      kcur[dc][1] ^= TILEB;
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) vcur[db] ^= TILEB;
  };

  // Y_t: online softmax of S(t) -> P(t) in e4m3, rescaling O and l (which hold tiles < t)
  auto yphase = [&](int t) __attribute__((always_inline)) {
    const int kt0 = t * kBK;
    const bool masked = kt0 + kBK > L || (CAUSAL && kt0 + kBK - 1 > wq0);
    if (masked) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kt0 + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
          const bool drop = key >= L || (CAUSAL && key > qi);
          s[kb][r] = drop ? kNegInf : s[kb][r];
        }
    }
    float sv[16 * kKB];
#pragma unroll
    for (int i = 0; i < 16 * kKB; ++i) sv[i] = s[i >> 4][i & 15];
    const float mnew = pair_max(max_tree3(sv)) * c2;  // c2 > 0: a fully masked row keeps -inf
    const bool need = mnew > mref + kRescaleSlack;
    if (__any(need)) {
      const float alpha = need ? exp2f_hw(mref - mnew) : 1.0f;
      lacc *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
      if (need) mref = mnew;
    }
    const float mu = mref == kNegInf ? 0.f : mref;
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float p[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) p[j] = exp2f_hw(fmaf(s[kb][4 * e + j], c2, -mu));
        // byte 16 (kb % 2) + 4 e + j of the 64-key half kb / 2 <-> register 4 e + j of s[kb]
        pf[kb >> 1][4 * (kb & 1) + e] = pack4_e4m3(p[0], p[1], p[2], p[3]);
      }
  };

  using I0 = std::integral_constant<bool, false>;
  using I1 = std::integral_constant<bool, true>;
  auto phase_barrier = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  // results a phase hands to the next are pinned on its side of the barrier
  auto pin_s = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb) asm volatile("" : "+v"(s[kb]));
  };
  auto pin_p = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int kh = 0; kh < kKH; ++kh) asm volatile("" : "+v"(pf[kh]));
  };
  // Group A issues the direct loads at the start of its matrix phase X(t): K(t+1) into K
  // buffer (t+1) % 2 and V(t) into V buffer t % 2, buffers whose tiles every wave finished
  // reading in X(t-1). It waits for them at the end of Y(t), before the barrier that precedes
  // their first reader X(t+1). The vector phases, which set the pace, issue no loads (issued
  // there, the loads lengthened them by a fifth).
  // Position of the next K tile (stream tile t + 1) and V tile (stream tile t) to load: item
  // and tile within it, with that item's resource words; advanced one tile per load.
  int kl_j = STREAM ? 1 / ntiles : 0, kl_t = STREAM ? 1 - kl_j * ntiles : 1;
  int vl_j = 0, vl_t = 0;
  u32x4 kl_w = wk, vl_w = wv;
  if (STREAM && kl_j > 0 && kl_j < nitems) kl_w = item_words(kl_j, true);
  auto advance = [&](int& lj, int& lt, u32x4& lw, bool is_k) __attribute__((always_inline)) {
    ++lt;
    if (STREAM && lt == ntiles) {
      lt = 0;
      if (++lj < nitems) lw = item_words(lj, is_k);
    }
  };
  auto issue = [&](int t) __attribute__((always_inline)) {
    if (grp == 0) {
      if (t + 1 < nstream) {
        tload_w(kl_w, ((t + 1) & 1) ? Ks1 : Ks0, kl_t);
        advance(kl_j, kl_t, kl_w, true);
      }
      if (t < nstream) {
        tload_w(vl_w, (t & 1) ? Vs1 : Vs0, vl_t);
        advance(vl_j, vl_t, vl_w, false);
      }
    }
  };
  auto land = [&]() __attribute__((always_inline)) {
    if (grp == 0) wait_vmcnt<0>();
  };
  auto step = [&](int t) __attribute__((always_inline)) {
    issue(t);
    xphase(I1{}, I1{});
    pin_s();
    phase_barrier();
    yphase(t);
    pin_p();
    land();
    phase_barrier();
  };

  // Phase p: group A runs X(p/2) for even p and Y(p/2) for odd p, group B one phase later.
  // A wave's own tiles end at nt_w; it then passes the remaining barriers idle (group A
  // still issuing its share of the loads).
  if (grp == 0) tload_w(wk, Ks0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  phase_barrier();
  if (grp == 1) phase_barrier();
  issue(0);
  xphase(I0{}, I1{});
  pin_s();
  phase_barrier();
  if (STREAM && ntiles == 1 && nitems > 1) {  // item 0's only S is done: Q of item 1
    int jqb, jh, jbs;
    stream_item(1, jqb, jh, jbs);
    load_q(((long)jbs * a.N * a.H + jh) * D, jqb * BQ + rb * 32 + l32);
  }
  yphase(0);
  pin_p();
  land();
  phase_barrier();
  // ---- epilogue of an item: O = v_descale * acc / l in bf16 (rows >= L dropped by the
  // bounds), LSE
  auto epilogue = [&]() __attribute__((always_inline)) {
    const float l = lacc[0];
    const float inv = l > 0.f ? a.v_descale / l : 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const f32x16& o = oacc[db];
        u32x2 v = {pack2<BF16>(o[4 * rr] * inv, o[4 * rr + 1] * inv),
                   pack2<BF16>(o[4 * rr + 2] * inv, o[4 * rr + 3] * inv)};
        buf_store8(ro, (uint32_t)qi * (2 * rstride) + (db * 32 + 8 * rr + 4 * g) * 2, v);
      }
    if (g == 0 && qi < L) lse[qi] = l > 0.f ? (mref + log2f_hw(l)) * kLn2 : kNegInf;
  };
  if constexpr (STREAM) {
    // stream step gs computes S of tile tin of item j (after the boundary, tile 0 of the
    // next item) and P V of the stream's previous tile
    int j = 0, tin = 1;
#pragma unroll 1
    for (int gs = 1; gs < nstream; ++gs) {
      const bool boundary = tin == ntiles;
      issue(gs);
      xphase(I1{}, I1{});
      pin_s();
      phase_barrier();
      if (boundary) {
        // item j is complete (its last P V and row sum ran in this matrix phase)
        epilogue();
        ++j;
        stream_item(j, qb, h, bs);
        q0 = qb * BQ;
        base = ((long)bs * a.N * a.H + h) * D;
        ro = make_rsrc(a.o + base, 2 * nbytes);
        lse = a.lse + ((long)bs * a.H + h) * a.N;
        wq0 = q0 + rb * 32;
        qi = wq0 + l32;
        mref = kNegInf;
        lacc = f32x16{};
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
        tin = 0;
      }
      if (tin == ntiles - 1 && j + 1 < nitems) {
        // Q is free after this step's S: load the next item's rows
        int jqb, jh, jbs;
        stream_item(j + 1, jqb, jh, jbs);
        load_q(((long)jbs * a.N * a.H + jh) * D, jqb * BQ + rb * 32 + l32);
      }
      yphase(tin);
      pin_p();
      land();
      phase_barrier();
      ++tin;
    }
    issue(nstream);
    xphase(I1{}, I0{});
    phase_barrier();
    if (grp == 0) {
      land();
      phase_barrier();
    }
    epilogue();
  } else {
    int t = 1;
#pragma unroll 1
    for (; t < nt_w; ++t) step(t);
    issue(t);
    xphase(I1{}, I0{});
    phase_barrier();
    for (; t < ntiles; ++t) {
      land();
      phase_barrier();
      issue(t + 1);
      phase_barrier();
    }
    if (grp == 0) {
      land();
      phase_barrier();
    }
    epilogue();
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const Fp8FwdArgs& a, hipStream_t st) {
  constexpr int BQ = 32 * kWaves;
  const int nqb = (a.N + BQ - 1) / BQ;
  const long total = (long)nqb * a.H * a.B;
  if (total == 0) return hipSuccess;
  if constexpr (!CAUSAL) {
    // one workgroup per CU (a multiple of the 8 XCDs) when there are at least two items each
    const int ncu = cu_count() / 8 * 8;
    if (ncu > 0 && total >= 2L * ncu) {
      hipLaunchKernelGGL((fwd_fp8_kernel<D, false, true>), dim3((unsigned)ncu), dim3(kThreads),
                         0, st, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((fwd_fp8_kernel<D, CAUSAL, false>), dim3((unsigned)total), dim3(kThreads),
                     0, st, a);
  return hipGetLastError();
}

}  // namespace
}  // namespace f8

hipError_t launch_fwd_fp8(const Fp8FwdArgs& a, int d, bool causal, hipStream_t st) {
  if (d == 128) return causal ? f8::launch<128, true>(a, st) : f8::launch<128, false>(a, st);
  return causal ? f8::launch<64, true>(a, st) : f8::launch<64, false>(a, st);
}

}  // namespace fa
