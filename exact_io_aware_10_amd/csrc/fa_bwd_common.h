// Shared device-side pieces of the backward kernels (fa_bwd.hip, fa_bwd_dkdv.hip,
// fa_bwd_dq.hip): slice addressing, work decoding, the tile swizzle, direct tile loads and
// the per-lane fragment addressing.
#pragma once

#include <type_traits>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace bwd {


constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 64;  // rows of the streamed tile (queries in dK/dV, keys in dQ)
constexpr float kLog2e = 1.44269504088896340736f;

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

// Chunk swizzle of tile row r, good for both row and transposed fragment reads.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// Per-slice addressing shared by the kernels.
struct SliceInfo {
  long tok0;  // first token of the slice in the [tokens, H, d] tensors
  int L;      // rows in the slice
  long stat;  // offset of row 0 of the slice in lse / the workspace row terms
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

// Work item of a dense or packed launch: (block index within the slice, head, batch/seq).
// With causal set, dense launches go longest first over whole slices per XCD (causal_order)
// and the costliest block is taken to be the last one (long_last: query blocks). Packed
// launches keep each (sequence, head) on one XCD (varlen_order), longest first under the mask.
// Returns false for a slot of a packed launch past the last (sequence, head) pair.
__device__ __forceinline__ bool decode_work(const BwdArgs& a, int nblk, bool varlen,
                                            bool causal, bool long_last, int& blk, int& h,
                                            int& bs) {
  if (varlen) {
    if (!varlen_order(blockIdx.x, nblk, a.H, a.B, blk, h, bs)) return false;
    if (causal && long_last) blk = nblk - 1 - blk;  // longest rows first within a sequence
    return true;
  }
  if (causal) {
    int rank, bh;
    causal_order(blockIdx.x, a.B * a.H, rank, bh);
    blk = long_last ? nblk - 1 - rank : rank;
    h = bh % a.H;
    bs = bh / a.H;
    return true;
  }
  const uint32_t w = xcd_remap(blockIdx.x, gridDim.x);
  blk = w % nblk;
  h = (w / nblk) % a.H;
  bs = w / (nblk * a.H);
  return true;
}

// ---------------------------------------------------------------- tile access helpers
template <int D, int NW = kWaves, int ROWS = kTile>
struct Tile {
  static constexpr int ROWB = D * 2;        // bytes per row
  static constexpr int CPR = D / 8;         // 16-byte chunks per row
  static constexpr int BYTES = ROWS * ROWB;
  static constexpr int RPL = 1024 / ROWB;   // rows per 1 KiB direct load
  static constexpr int LPW = BYTES / 1024 / NW;  // direct loads per wave per tile (NW waves)
  static_assert(LPW >= 1 && LPW * NW * 1024 == BYTES, "whole 1 KiB loads per wave");

  // direct HBM/L2 -> LDS load of tile rows [row0, row0 + ROWS) of a [tokens, H, D] tensor
  // (rs: the tensor's buffer resource words). Issued from inline assembly (dma16): with the
  // builtin the compiler makes the next LDS reads of the current tile wait for this
  // prefetch. The caller waits (vmcnt 0) before the barrier that precedes the tile's readers.
  static __device__ __forceinline__ void load(u32x4 rs, uint8_t* tile, int row0,
                                              uint32_t rstride, int wave, int lane) {
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      const int blk = wave * LPW + j;
      const int row = blk * RPL + lane / CPR;
      const int c = (lane % CPR) ^ swz<D>(row);
      dma16<0>(rs, __builtin_amdgcn_readfirstlane(lds_addr(tile) + blk * 1024),
               (uint32_t)(row0 + row) * rstride + c * 16);
    }
  }
};

// Per-lane constants of the fragment addressing. With them every fragment address is one
// xor-add, (compile-time offset ^ lane mask) + lane base, instead of a register per address.
//  row fragment (A operand rows = tile rows r0 + l32, 16-byte chunk 2*dc + g):
//    r0 * ROWB + ((dc << 5) ^ row_mask) + row_base
//  transposed fragment (A operand over tile rows k0..k0+15 and columns 32*db..32*db+31;
//    lane (l32, g) gets column 32*db + l32 of rows k0 + 4g + {0..3} and k0 + 8 + 4g + {0..3},
//    the row order of P / dS registers taken from a 32x32 accumulator):
//    k0 * ROWB + ((db << 6) ^ tr_mask[h]) + tr_base[h], h = 0 (first 4 rows), 1 (+8 rows)
template <int D>
struct Lanes {
  static constexpr int ROWB = D * 2;
  uint32_t row_base, row_mask, tr_base0, tr_base1, tr_mask0, tr_mask1;
  __device__ __forceinline__ explicit Lanes(int lane) {
    const int l32 = lane & 31, g = lane >> 5, i16 = lane & 15, G = (lane >> 4) & 1;
    // tile rows are 32-row aligned in row fragments: the swizzle of row r0 + l32 is that of l32
    row_base = l32 * ROWB;
    row_mask = (uint32_t)(g ^ swz<D>(l32)) << 4;
    const int r = 4 * g + (i16 >> 2);  // row within the 16-row group (k0 is 16-aligned)
    const int cl = 2 * G + ((i16 & 3) >> 1);  // chunk within the 4-chunk group of 32 columns
    tr_base0 = r * ROWB + 8 * (i16 & 1);
    tr_base1 = (r + 8) * ROWB + 8 * (i16 & 1);
    tr_mask0 = (uint32_t)(cl ^ swz<D>(r)) << 4;
    tr_mask1 = (uint32_t)(cl ^ swz<D>(r + 8)) << 4;
  }
  // keep the constants in registers but opaque, so the compiler recomputes each address
  // where it is used instead of holding one register per address across the loop
  __device__ __forceinline__ void refresh() {
    asm volatile("" : "+v"(row_base), "+v"(row_mask), "+v"(tr_base0), "+v"(tr_base1),
                 "+v"(tr_mask0), "+v"(tr_mask1));
  }
  __device__ __forceinline__ u32x4 row_frag(const uint8_t* tile, int r0, int dc) const {
    const uint32_t off = r0 * ROWB + ((((uint32_t)dc << 5) ^ row_mask) + row_base);
    return *reinterpret_cast<const u32x4*>(tile + off);
  }
  __device__ __forceinline__ u32x4 tr_frag(const uint8_t* tile, int k0, int db) const {
    const uint32_t o0 = k0 * ROWB + ((((uint32_t)db << 6) ^ tr_mask0) + tr_base0);
    const uint32_t o1 = k0 * ROWB + ((((uint32_t)db << 6) ^ tr_mask1) + tr_base1);
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + o0));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + o1));
    const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
    return u32x4{lo2[0], lo2[1], hi2[0], hi2[1]};
  }
};


hipError_t launch_dkdv(const BwdArgs& a, int d, bool bf16, bool causal, bool varlen,
                       hipStream_t st);
hipError_t launch_dq(const BwdArgs& a, int d, bool bf16, bool causal, bool varlen,
                     hipStream_t st);

}  // namespace bwd
}  // namespace fa
