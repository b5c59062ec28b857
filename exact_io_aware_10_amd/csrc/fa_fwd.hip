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
//  - one workgroup = 8 waves = 256 query rows of one (batch or sequence, head); each wave
//    owns 32 rows, held as MFMA B operands in registers for the whole loop.
//  - ping-pong: the waves form two groups of four (one wave of each group per SIMD). Each
//    wave alternates an MFMA phase X_t = [O += P(t-1) V(t-1); S(t) = scores of tile t]
//    and a vector phase Y_t = [online softmax of S(t) -> P(t)], group B one phase behind
//    group A, with a workgroup barrier between phases; so on every SIMD one wave issues
//    matrix instructions while the other does the exp/max/convert work.
//  - key/value tiles of 128 rows go from HBM/L2 straight into LDS (buffer_load ... lds,
//    bounds-checked so rows past the sequence read as zero), K triple and V double buffered,
//    each group issuing one tile per step in its vector phase. Rows are stored unpadded with
//    an XOR swizzle of their 16-byte chunks that keeps the operand reads conflict-free.
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


constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
#ifndef FA_FWD_BK
#define FA_FWD_BK 128
#endif
constexpr int kBK = FA_FWD_BK;            // keys per tile
constexpr int kKB = kBK / 32;             // 32-key blocks of S^T per tile
constexpr int kKC = kBK / 16;             // 16-key chunks of P per tile (one MFMA k-step each)
static_assert(kBK == 64 || kBK == 128, "tile of 64 or 128 keys");
constexpr float kRescaleSlack = 8.0f;     // log2 units the reference max may lag behind
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kNegInf = -__builtin_inff();

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// 16-byte-chunk swizzles of a tile row r (D/8 chunks per row).
// K rows are read as 32 rows x one chunk (ds_read_b128): chunk c of row r sits at c ^ (r % D/8).
// V rows are read 4 rows x 4 chunks per 32 lanes (ds_read_b64_tr_b16).
template <int D>
__device__ __forceinline__ int kswz(int r) { return r & (D / 8 - 1); }
template <int D>
__device__ __forceinline__ int vswz(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }

#ifndef FA_FWD_PREFETCH
#define FA_FWD_PREFETCH 4  // MFMAs of look-ahead for the LDS operand reads of a matrix phase
#endif

// Instruction order of one matrix phase: NPV MFMAs with two LDS reads each (O += P V), then
// NS MFMAs with one read each (S = K Q^T). The reads run PD MFMAs ahead of their use, so the
// LDS latency is covered by the wave's own matrix work (the other wave on the SIMD is in its
// vector phase and cannot cover it).
template <int MASK, int N>
__device__ __forceinline__ void sched_group() {
  if constexpr (N > 0) __builtin_amdgcn_sched_group_barrier(MASK, N, 0);
}
constexpr int kSchedMfma = 0x008, kSchedDsRead = 0x100;
template <int NPV, int NM, int PD, int M>
__device__ __forceinline__ void xsched_step() {
  sched_group<kSchedMfma, 1>();
  if constexpr (M + PD < NM) sched_group<kSchedDsRead, (M + PD < NPV ? 2 : 1)>();
}
template <int NPV, int NS, int PD, int... M>
__device__ __forceinline__ void xsched(std::integer_sequence<int, M...>) {
  constexpr int NM = NPV + NS;
  constexpr int pd = PD < NM ? PD : NM;
  sched_group<kSchedDsRead, (pd <= NPV ? 2 * pd : 2 * NPV + (pd - NPV))>();
  (xsched_step<NPV, NM, PD, M>(), ...);
}

// STREAM (dense, no mask): one workgroup per CU takes items blockIdx.x, blockIdx.x + G, ...
// (G = gridDim.x) of the XCD-remapped work list, as one continuous stream of key/value tiles:
// the next item's first tiles are loaded through the same buffers and its Q rows into spare
// registers while the current item finishes, and an item's output is stored during the
// vector phase that starts the next item, so the pipeline never drains between items.
template <int D, class T, bool CAUSAL, bool VARLEN, bool STREAM>
__global__ __launch_bounds__(kThreads, 1) void fwd_kernel(FwdArgs a) {
  static_assert(!STREAM || (!CAUSAL && !VARLEN), "the stream form is for dense, unmasked launches");
  constexpr int BQ = 32 * kWaves;
  constexpr int ROWB = D * 2;                 // bytes per K/V row in LDS
  constexpr int CPR = D / 8;                  // 16-byte chunks per row
  constexpr int TILEB = kBK * ROWB;           // bytes per tile
  constexpr int RPL = 1024 / ROWB;            // rows per 1 KiB direct load (one per wave)
  constexpr int LPW = TILEB / 1024 / (kWaves / 2);  // direct loads per group-B wave per tile
  constexpr int DC = D / 16;                  // 16-wide d chunks of Q K^T
  constexpr int DB = D / 32;                  // 32-wide d blocks of the output

  // five tile buffers: V at 0 and TILEB (a V buffer's parity is bit log2(TILEB) of its
  // offset, so switching V buffers is an XOR of the per-lane offsets), K at 2, 3 and 4 TILEB
  // (three, so that a K tile can be loaded while both groups are still reading the two
  // before it). 160 KiB at d = 128.
  __shared__ __attribute__((aligned(1024))) uint8_t smem[5 * TILEB];
  lds_poison(smem, sizeof(smem));
  lds_poison_done();
  auto kbuf = [&](int i) __attribute__((always_inline)) { return smem + (2 + i) * TILEB; };
  auto vbuf = [&](int i) __attribute__((always_inline)) { return smem + i * TILEB; };

  const int tid = threadIdx.x;
  const int lane = tid & 63, l32 = lane & 31, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // group (0 = A, 1 = B) and this wave's 32-row block: the groups take alternate blocks so
  // that causal work is balanced between them; waves w and w+4 share a SIMD
  const int grp = wave >> 2;
  const int rb = 2 * (wave & 3) + grp;

  // ---- work item: (query block, head, batch or sequence)
  const int nqb = (a.N + BQ - 1) / BQ;
  const uint32_t total = (uint32_t)nqb * a.H * a.B;  // items of the launch
  // item j of this workgroup in the stream form
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
  } else if (CAUSAL && !VARLEN) {  // longest rows first over whole slices per XCD
    int rank, bh;
    causal_order(blockIdx.x, a.B * a.H, rank, bh);
    qb = nqb - 1 - rank;
    h = bh % a.H;
    bs = bh / a.H;
  } else if (VARLEN) {  // each (sequence, head) on one XCD, longest rows first
    if (!varlen_order(blockIdx.x, nqb, a.H, a.B, qb, h, bs)) return;
    qb = nqb - 1 - qb;
  } else {
    const uint32_t w = xcd_remap(blockIdx.x, gridDim.x);
    qb = w % nqb;
    h = (w / nqb) % a.H;
    bs = w / (nqb * a.H);
  }

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
  int q0 = qb * BQ;
  if (q0 >= L) return;

  const uint32_t rstride = (uint32_t)a.H * D * 2;  // bytes between consecutive tokens
  long base = (tok0 * a.H + h) * D;
  const uint32_t nbytes = (uint32_t)(L - 1) * rstride + D * 2;
  auto ro = make_rsrc(a.o + base, nbytes);
  float* lse = a.lse + (VARLEN ? (long)h * a.T + tok0 : ((long)bs * a.H + h) * a.N);

  int wq0 = q0 + rb * 32;  // first query row of this wave
  int qi = wq0 + l32;        // this lane's query row
  const int kend = CAUSAL ? (L < q0 + BQ ? L : q0 + BQ) : L;
  const int ntiles = (kend + kBK - 1) / kBK;
  const int ntiles_c = ntiles;             // tiles per item (the same for every item)
  const int nstream = nitems * ntiles;     // tiles of the whole stream

  // ---- Q rows into registers (B operand of S^T = K Q^T): d = 16*dc + 8g .. +7
  auto load_q = [&](u32x4 (&dst)[DC], long qbase, int row) __attribute__((always_inline)) {
    const auto rq = make_rsrc(a.q + qbase, nbytes);
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
      dst[dc] = buf_load16(rq, (uint32_t)row * rstride + (16 * dc + 8 * g) * 2) ^ a.qsign;
  };
  u32x4 qreg[DC];
  load_q(qreg, base, qi);

  // ---- direct HBM/L2 -> LDS tile loads: this wave fills LPW 1 KiB blocks of each tile;
  // lane l of a block writes row blk*RPL + l/CPR, physical chunk l%CPR. Issued from inline
  // assembly (dma16), so the compiler adds no wait of its own; the issuing waves wait
  // (vmcnt 0) before the barrier that precedes the tile's first reader.
  const int lrow = lane / CPR, lpc = lane % CPR;
  const u32x4 wk = rsrc_words(a.k + base, nbytes), wv = rsrc_words(a.v + base, nbytes);
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
  // Per-lane source offset of each load: the lane's row (the block's first row plus the lane's
  // row within the block) and its swizzled chunk, computed once. The tile's first row moves
  // the resource's base address and shrinks its size (tile_words), so every row offset stays
  // in the bounds-checked vector offset: rows past the sequence read as zero, and no load
  // touches memory past the end of the tensor. Issuing a load takes no vector work.
  uint32_t kof[LPW], vof[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int row = ((wave & 3) * LPW + j) * RPL + lrow;
    kof[j] = (uint32_t)row * rstride + (uint32_t)((lpc ^ kswz<D>(row)) * 16);
    vof[j] = (uint32_t)row * rstride + (uint32_t)((lpc ^ vswz<D>(row)) * 16);
  }
  auto tload_one = [&](u32x4 words, bool is_k, uint8_t* tile, int j)
      __attribute__((always_inline)) {
    const int blk = (wave & 3) * LPW + j;
    const uint32_t m0 =
        __builtin_amdgcn_readfirstlane(lds0 + (uint32_t)(tile - smem) + blk * 1024);
    dma16<0>(words, m0, is_k ? kof[j] : vof[j]);
  };
  // buffer resource words of K or V for item j of the stream form
  auto item_words = [&](int j, bool is_k) __attribute__((always_inline)) {
    int jqb, jh, jbs;
    stream_item(j, jqb, jh, jbs);
    return rsrc_words((is_k ? a.k : a.v) + ((long)jbs * a.N * a.H + jh) * D, nbytes);
  };
  auto tload_w = [&](u32x4 words, bool is_k, uint8_t* tile, int t) __attribute__((always_inline)) {
    const u32x4 tw = rsrc_advance(words, (uint32_t)(t * kBK) * rstride);
#pragma unroll
    for (int j = 0; j < LPW; ++j) tload_one(tw, is_k, tile, j);
  };
  // tile s of the stream (prologue): tile s of this item, or (stream form) tile s % ntiles
  // of item s / ntiles
  auto tload = [&](bool is_k, uint8_t* tile, int s) __attribute__((always_inline)) {
    if (STREAM) {
      const int j = s / ntiles_c;
      tload_w(item_words(j, is_k), is_k, tile, s - j * ntiles_c);
    } else {
      tload_w(is_k ? wk : wv, is_k, tile, s);
    }
  };

  // ---- per-lane LDS byte offsets of the MFMA operand reads, relative to a tile buffer.
  // The XOR swizzle is folded into one offset per d chunk (K) or d block (V), so every read
  // is one of these registers plus a constant.
  // K (A operand of S^T): row kb*32 + l32, logical chunk 2dc + g, stored at (2dc + g) ^ m,
  // m = l32 % (D/8); bit 0 comes from g alone, so this is 2(dc ^ m/2) + (g ^ m%2).
  const int km = kswz<D>(l32);
  int kcur[DC];  // offsets of the current tile's K buffer (starts at K buffer 0)
#pragma unroll
  for (int dc = 0; dc < DC; ++dc)
    kcur[dc] = 2 * TILEB + l32 * ROWB + (2 * (dc ^ (km >> 1)) + (g ^ (km & 1))) * 16;
  int kslot = 0;  // K buffer of the current tile (uniform)
  // V^T (A operand of O^T): tr reads of keys kc*16 + 4g + i/4 (+8), dims db*32 + 16G + 4(i%4)
  // (i = lane % 16): logical chunk 4db + x, x = 2G + (i%4)/2, stored at (4db + x) ^ vsw =
  // 4(db ^ vsw/4) + x, at byte 8(i%2) of the chunk.
  const int i16 = lane & 15, G = (lane >> 4) & 1;
  const int vkey = 4 * g + (i16 >> 2);
  const int vsw = vswz<D>(vkey);
  int vcur[DB];  // offsets into the V buffer of the previous tile (V buffer 1 before tile 0)
#pragma unroll
  for (int db = 0; db < DB; ++db)
    vcur[db] = TILEB + vkey * ROWB + (4 * (db ^ (vsw >> 2)) + 2 * G + ((i16 & 3) >> 1)) * 16 +
               8 * (i16 & 1);

  float mref = kNegInf, lsum = 0.f;
  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
  const float c2 = a.scale_log2;
  // the pair (1, 1) of the element type, kept in a register for the row-sum dot products
  uint32_t ones = one_pair<T>();
  asm volatile("" : "+v"(ones));

  const int nt_w = CAUSAL ? min(ntiles, (wq0 + 31 + kBK) / kBK) : ntiles;  // this wave's tiles
  f32x16 s[kKB];
  u32x4 pf[kKC];

  // Matrix phase X(t) = [O += P(t-1) V(t-1); S(t) = K(t) Q^T]; S^T has lanes <-> query rows.
  // It ends by moving the buffer offsets on to tile t+1.
  auto xphase = [&](auto HAS_PV, auto HAS_S) __attribute__((always_inline)) {
    if constexpr (decltype(HAS_PV)::value) {
#pragma unroll
      for (int kc = 0; kc < kKC; ++kc)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const uint8_t* src = smem + vcur[db] + kc * 16 * ROWB;
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)src);
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(src + 8 * ROWB));
          const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
          const u32x4 va = {lo2[0], lo2[1], hi2[0], hi2[1]};
          oacc[db] = mfma32<T>(va, pf[kc], oacc[db]);
        }
    }
    if constexpr (decltype(HAS_S)::value) {
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb) s[kb] = f32x16{};
#pragma unroll
      for (int dc = 0; dc < DC; ++dc)
#pragma unroll
        for (int kb = 0; kb < kKB; ++kb) {
          const u32x4 ka = *reinterpret_cast<const u32x4*>(smem + kcur[dc] + kb * 32 * ROWB);
          s[kb] = mfma32<T>(ka, qreg[dc], s[kb]);
        }
    }
    if constexpr (decltype(HAS_PV)::value && decltype(HAS_S)::value)
      xsched<kKC * DB, kKB * DC, FA_FWD_PREFETCH>(
          std::make_integer_sequence<int, kKC * DB + kKB * DC>{});
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) kcur[dc] += kslot == 2 ? -2 * TILEB : TILEB;
    kslot = kslot == 2 ? 0 : kslot + 1;
#pragma unroll
    for (int db = 0; db < DB; ++db) vcur[db] ^= TILEB;
  };

  // Y_t: online softmax of S(t) -> P(t), rescaling O (which holds P V up to tile t-1)
  auto yphase = [&](int t) __attribute__((always_inline)) {
    const int kt0 = t * kBK;
    const bool masked = kt0 + kBK > L || (CAUSAL && kt0 + kBK - 1 > wq0);
    if (masked) {
      // a real branch: keeps the per-element mask out of the unmasked tiles
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
    // Row max as a tree of three-input maxima: one wave runs this phase alone on its SIMD, so
    // the dependency depth, not only the instruction count, sets the phase length.
    float sv[16 * kKB];
#pragma unroll
    for (int i = 0; i < 16 * kKB; ++i) sv[i] = s[i >> 4][i & 15];
    const float mx = max_tree3(sv);
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
    float ls[kKC];  // independent partial row sums, one per 16-key chunk
#pragma unroll
    for (int kc = 0; kc < kKC; ++kc) {
      float p[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int r = 8 * kc + j;
        p[j] = exp2f_hw(fmaf(s[r >> 4][r & 15], c2, -mu));
      }
      // P rounded to the element type; the row sum adds exactly the rounded values
      pf[kc] = u32x4{pack2<T>(p[0], p[1]), pack2<T>(p[2], p[3]), pack2<T>(p[4], p[5]),
                     pack2<T>(p[6], p[7])};
      ls[kc] = kc == 0 ? lsum : 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) ls[kc] = add_pair_r<T>(pf[kc][e], ones, ls[kc]);
    }
#pragma unroll
    for (int w = kKC; w > 1; w >>= 1)
#pragma unroll
      for (int i = 0; i < w / 2; ++i) ls[i] = ls[2 * i] + ls[2 * i + 1];
    lsum = ls[0];
  };

  using I0 = std::integral_constant<bool, false>;
  using I1 = std::integral_constant<bool, true>;
  // workgroup barrier between phases; the scheduling barriers keep each phase's
  // instructions on their side of it
  auto phase_barrier = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  // Results a phase hands to the next one are pinned on its side of the barrier: without
  // this the compiler sinks their computation to the point of use, past the barrier.
  auto pin_s = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb) asm volatile("" : "+v"(s[kb]));
  };
  auto pin_p = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int kc = 0; kc < kKC; ++kc) asm volatile("" : "+v"(pf[kc]));
  };
  // Each group issues one tile's direct loads at the start of its vector phase Y(t), so the
  // load issue (the vector phases' largest extra cost) is split evenly between the phases:
  // group A loads K(t+2) into K buffer (t+2) % 3, which last held K(t-1), read by both groups
  // before the previous barrier; group B loads V(t+1) into V buffer (t+1) % 2, which last held
  // V(t-1), read by both groups in their matrix phases X(t). Every wave waits for its own
  // loads (vmcnt 0) at the end of its next matrix phase, one or two phases before the tile's
  // first reader.
  int kload_slot = 2;  // K buffer of tile t + 2 for the next loads(t) (uniform)
  // Position of the next tile each group loads (item, tile within the item) and that item's
  // resource words, advanced one tile per call: K from stream tile 2 on, V from tile 1 on.
  int kl_j = STREAM ? 2 / ntiles_c : 0, kl_t = STREAM ? 2 - kl_j * ntiles_c : 2;
  int vl_j = STREAM ? 1 / ntiles_c : 0, vl_t = STREAM ? 1 - vl_j * ntiles_c : 1;
  u32x4 kl_w = wk, vl_w = wv;
  if (STREAM) {
    if (grp == 0 && kl_j > 0 && kl_j < nitems) kl_w = item_words(kl_j, true);
    if (grp == 1 && vl_j > 0 && vl_j < nitems) vl_w = item_words(vl_j, false);
  }
  auto loads = [&](int t) __attribute__((always_inline)) {
    if (grp == 0) {
      if (t + 2 < nstream) {
        tload_w(kl_w, true, kbuf(kload_slot), kl_t);
        if (STREAM && ++kl_t == ntiles_c) {
          kl_t = 0;
          if (++kl_j < nitems) kl_w = item_words(kl_j, true);
        }
        if (!STREAM) ++kl_t;
      }
      kload_slot = kload_slot == 2 ? 0 : kload_slot + 1;
    } else if (t + 1 < nstream) {
      tload_w(vl_w, false, vbuf((t + 1) & 1), vl_t);
      if (STREAM && ++vl_t == ntiles_c) {
        vl_t = 0;
        if (++vl_j < nitems) vl_w = item_words(vl_j, false);
      }
      if (!STREAM) ++vl_t;
    }
  };
  auto finish_x = [&]() __attribute__((always_inline)) {
    wait_vmcnt<0>();
    phase_barrier();
  };

  // X(t) then Y(t), for 1 <= t < nt_w
  auto step = [&](int t) __attribute__((always_inline)) {
    xphase(I1{}, I1{});
    pin_s();
    finish_x();
    loads(t);
    yphase(t);
    pin_p();
    phase_barrier();
  };

  // ---- epilogue of an item: O = acc / l (rows >= L are dropped by the buffer bounds), LSE
  auto epilogue = [&]() __attribute__((always_inline)) {
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
  };

  // Phase p: group A runs X(p/2) for even p and Y(p/2) for odd p, group B one phase later.
  // A wave's own tiles end at nt_w; it then passes the remaining barriers idle.
  if (grp == 1) tload(true, kbuf(0), 0);
  wait_vmcnt<0>();
  phase_barrier();
  if (grp == 1) {
    if (nstream > 1) tload(true, kbuf(1), 1);
    tload(false, vbuf(0), 0);
    phase_barrier();
  }
  // stream form: once the matrix phase has computed S of an item's last tile, Q is free and
  // the next item's rows are loaded into it (the next matrix phase waits for them)
  auto next_q = [&](int j) __attribute__((always_inline)) {
    if (STREAM && j < nitems) {
      int jqb, jh, jbs;
      stream_item(j, jqb, jh, jbs);
      load_q(qreg, ((long)jbs * a.N * a.H + jh) * D, jqb * BQ + rb * 32 + l32);
    }
  };
  xphase(I0{}, I1{});
  pin_s();
  finish_x();
  loads(0);
  if (ntiles == 1) next_q(1);
  yphase(0);
  pin_p();
  phase_barrier();
  if constexpr (STREAM) {
    // stream step gs computes S of tile tin of item j (after the boundary, tile 0 of the
    // next item) and P V of the stream's previous tile
    int j = 0, tin = 1;
#pragma unroll 1
    for (int gs = 1; gs < nstream; ++gs) {
      const bool boundary = tin == ntiles;
      xphase(I1{}, I1{});
      pin_s();
      finish_x();
      loads(gs);
      if (boundary) {
        // item j is complete (its last P V ran in this matrix phase): store it, move on
        epilogue();
        ++j;
        stream_item(j, qb, h, bs);
        q0 = qb * BQ;
        base = ((long)bs * a.N * a.H + h) * D;
        ro = make_rsrc(a.o + base, nbytes);
        lse = a.lse + ((long)bs * a.H + h) * a.N;
        wq0 = q0 + rb * 32;
        qi = wq0 + l32;
        mref = kNegInf;
        lsum = 0.f;
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
        tin = 0;
      }
      if (tin == ntiles - 1) next_q(j + 1);
      yphase(tin);
      pin_p();
      phase_barrier();
      ++tin;
    }
    // the last P V of the last item
    xphase(I1{}, I0{});
    finish_x();
    if (grp == 0) phase_barrier();
    epilogue();
  } else {
    int t = 1;
#pragma unroll 1
    for (; t < nt_w; ++t) step(t);
    // t == nt_w: the last P V
    xphase(I1{}, I0{});
    finish_x();
    for (; t < ntiles; ++t) {
      loads(t);
      phase_barrier();
      finish_x();
    }
    if (grp == 0) phase_barrier();
    epilogue();
  }
}

template <int D, class T, bool CAUSAL, bool VARLEN>
hipError_t launch(const FwdArgs& a, hipStream_t st) {
  constexpr int BQ = 32 * kWaves;
  const int nqb = (a.N + BQ - 1) / BQ;
  const long total = (long)nqb * a.H * a.B;
  if (total == 0) return hipSuccess;
  if constexpr (!CAUSAL && !VARLEN) {
    // one workgroup per CU (a multiple of the 8 XCDs), each taking a stream of items, when
    // there are at least two items per workgroup
    const int ncu = cu_count() / 8 * 8;
    if (ncu > 0 && total >= 2L * ncu) {
      hipLaunchKernelGGL((fwd_kernel<D, T, false, false, true>), dim3((unsigned)ncu),
                         dim3(kThreads), 0, st, a);
      return hipGetLastError();
    }
  }
  const long grid = VARLEN ? varlen_grid(nqb, a.H, a.B) : total;
  hipLaunchKernelGGL((fwd_kernel<D, T, CAUSAL, VARLEN, false>), dim3((unsigned)grid),
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
