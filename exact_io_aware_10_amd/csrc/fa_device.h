// Device-side building blocks for the gfx950 attention kernels: operand vector types,
// bf16/fp16 MFMA wrappers, buffer-resource loads with hardware bounds checks, exp2/log2,
// RNE conversions and the XCD-aware work remap.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Element type tags. Both are 16-bit storage; the tag picks the MFMA and the rounding.
struct BF16 {};
struct F16 {};

// C[32x32] += A[32x16] * B[16x32] with fp32 accumulation (v_mfma_f32_32x32x16_{bf16,f16}).
// Operand layout (lane l, g = l / 32): A holds A[l % 32][8g .. 8g+7], B holds
// B[8g .. 8g+7][l % 32]; C register r of lane l is C[8(r/4) + 4g + r%4][l % 32].
template <class T>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c);

template <>
__device__ __forceinline__ f32x16 mfma32<BF16>(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x16 mfma32<F16>(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Two fp32 values -> packed 16-bit pair, round to nearest even (low half = x).
template <class T>
__device__ __forceinline__ uint32_t pack2(float x, float y);
template <>
__device__ __forceinline__ uint32_t pack2<BF16>(float x, float y) {
  f32x2 v = {x, y};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
template <>
__device__ __forceinline__ uint32_t pack2<F16>(float x, float y) {
  f32x2 v = {x, y};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
}

// acc + lo + hi of a packed 16-bit pair (v_dot2c_f32_{bf16,f16} against (1, 1)).
template <class T>
__device__ __forceinline__ float add_pair(uint32_t pair, float acc);
template <>
__device__ __forceinline__ float add_pair<BF16>(uint32_t pair, float acc) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair), one, acc, false);
}
template <>
__device__ __forceinline__ float add_pair<F16>(uint32_t pair, float acc) {
  const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pair), one, acc, false);
}

// The pair (1, 1) of the element type as packed bits, and acc + pair[0] + pair[1] with the
// ones passed in (a register instead of a literal in every dot product).
template <class T>
__device__ __forceinline__ uint32_t one_pair();
template <>
__device__ __forceinline__ uint32_t one_pair<BF16>() { return 0x3f803f80u; }
template <>
__device__ __forceinline__ uint32_t one_pair<F16>() { return 0x3c003c00u; }
template <class T>
__device__ __forceinline__ float add_pair_r(uint32_t pair, uint32_t ones, float acc);
template <>
__device__ __forceinline__ float add_pair_r<BF16>(uint32_t pair, uint32_t ones, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair),
                                         __builtin_bit_cast(bf16x2, ones), acc, false);
}
template <>
__device__ __forceinline__ float add_pair_r<F16>(uint32_t pair, uint32_t ones, float acc) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pair), __builtin_bit_cast(f16x2, ones),
                                acc, false);
}

// 16-bit element -> fp32 (exact).
template <class T>
__device__ __forceinline__ float to_f32(uint32_t bits16);
template <>
__device__ __forceinline__ float to_f32<BF16>(uint32_t b) { return __uint_as_float(b << 16); }
template <>
__device__ __forceinline__ float to_f32<F16>(uint32_t b) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}

__device__ __forceinline__ float exp2f_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2f_hw(float x) { return __builtin_amdgcn_logf(x); }

// Buffer resource over [base, base + nbytes): loads past nbytes return 0 and stores past
// it are dropped, so ragged tails need no branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nbytes,
                                           0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ uint32_t buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ void buf_store8(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, off, 0, 0);
}
__device__ __forceinline__ void buf_store16(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0);
}
__device__ __forceinline__ void buf_store4(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, 0);
}

// Direct buffer -> LDS loads written in inline assembly. The builtin form tells the compiler
// that the instruction writes LDS, so it makes every later LDS read wait for the load to
// land (a wait on the HBM round trip). In assembly the load is opaque to the compiler: the
// caller waits explicitly (wait_vmcnt) before any wave reads the data.
// Words of a buffer resource over [base, base + nbytes), as make_rsrc.
__device__ __forceinline__ u32x4 rsrc_words(const void* base, uint32_t nbytes) {
  const uint64_t a = (uint64_t)base;
  return u32x4{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, nbytes, 0x00020000u};
}
// 16 bytes per lane from a buffer into LDS: lane l writes lds_addr + OFF + 16 l with the
// bytes at voff + OFF (zeros past the buffer's size). lds_addr is wave-uniform (M0).
template <int OFF>
__device__ __forceinline__ void dma16(u32x4 rs, uint32_t lds_addr, uint32_t voff) {
  static_assert(OFF >= 0 && OFF < 4096, "12-bit instruction offset");
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen offset:%3 lds"
               :
               : "{m0}"(lds_addr), "v"(voff), "s"(rs), "i"(OFF)
               : "memory");
}
// The resource words over [base + off, base + nbytes): the base address moves up by off
// bytes and the size shrinks by as much (to 0 if off >= nbytes), so a load at vector offset
// x reads the byte at base + off + x and is bounds-checked against the original end. (The
// instruction's scalar offset would not do: it is not part of the bounds check.)
// w and off must be wave-uniform; the words are read back from the first lane so that
// they stay in scalar registers, where the load instructions take them.
__device__ __forceinline__ u32x4 rsrc_advance(u32x4 w, uint32_t off) {
  const uint64_t a = (((uint64_t)(w[1] & 0xffffu) << 32) | w[0]) + off;
  const uint32_t n = w[2] > off ? w[2] - off : 0u;
  auto uni = [](uint32_t x) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)x); };
  return u32x4{uni((uint32_t)a), uni((uint32_t)(a >> 32) & 0xffffu), uni(n), uni(w[3])};
}
// 4 bytes per lane from a buffer into LDS: lane l writes lds_addr + OFF + 4 l.
template <int OFF>
__device__ __forceinline__ void dma4(u32x4 rs, uint32_t lds_addr, uint32_t voff) {
  static_assert(OFF >= 0 && OFF < 4096, "12-bit instruction offset");
  asm volatile("s_nop 0\n\tbuffer_load_dword %1, %2, 0 offen offset:%3 lds"
               :
               : "{m0}"(lds_addr), "v"(voff), "s"(rs), "i"(OFF)
               : "memory");
}
// LDS byte address of a pointer into a __shared__ array (the value M0 takes).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}
// Wait until at most N vector-memory operations of this wave are outstanding. Written in
// assembly with a memory clobber so that no LDS read moves above it.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Debug builds compiled with -DFA_LDS_POISON: every kernel first fills the LDS it declares
// with all-ones words (NaN as bf16, fp16 and fp32 data, 0xFF as e4m3: NaN), then passes a
// workgroup barrier, so an operand read from LDS that no load or store wrote shows up as
// NaN in the outputs. Without the macro both calls compile to nothing.
__device__ __forceinline__ void lds_poison(void* p, int bytes) {
#ifdef FA_LDS_POISON
  uint32_t* w = reinterpret_cast<uint32_t*>(p);
  for (int i = threadIdx.x; i < bytes / 4; i += blockDim.x) w[i] = 0xffffffffu;
#else
  (void)p;
  (void)bytes;
#endif
}
__device__ __forceinline__ void lds_poison_done() {
#ifdef FA_LDS_POISON
  __syncthreads();
#endif
}

// Workgroup barrier between phases that share LDS: waits for this wave's LDS accesses
// (lgkmcnt) but not for its outstanding buffer -> LDS loads. __syncthreads() would also wait
// for those (vmcnt 0), i.e. for every prefetch meant to stay in flight across the barrier;
// the kernels wait for each prefetch explicitly (wait_vmcnt) before the barrier that
// precedes its readers. The memory clobber keeps the compiler from moving memory accesses
// across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Row reductions across the lane pair (l, l ^ 32). v_permlane32_swap exchanges the upper
// half of its first operand with the lower half of its second; with both operands = x the
// two results hold, per lane, x and the partner's x (in an order that depends on the half),
// so a symmetric combination of the two is the pair's reduction in every lane.
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Maximum of N values by three-input maxima (v_max3_f32 from fmaxf(fmaxf(a, b), c)): for
// N = 64, 64 -> 22 -> 8 -> 3 -> 1 in 31 instructions, four levels deep.
template <int N>
__device__ __forceinline__ float max_tree3(const float (&x)[N]) {
  if constexpr (N == 1) {
    return x[0];
  } else {
    constexpr int M = (N + 2) / 3;
    float y[M];
#pragma unroll
    for (int i = 0; i < M; ++i) {
      if (3 * i + 2 < N)
        y[i] = fmaxf(fmaxf(x[3 * i], x[3 * i + 1]), x[3 * i + 2]);
      else if (3 * i + 1 < N)
        y[i] = fmaxf(x[3 * i], x[3 * i + 1]);
      else
        y[i] = x[3 * i];
    }
    return max_tree3<M>(y);
  }
}

// Workgroups are dispatched round-robin over the 8 XCDs (XCD = linear id % 8), each with
// its own L2. Remap the linear id so that XCD x receives a contiguous range of logical
// work items; neighbouring items (query blocks of one head) then share that XCD's L2.
__device__ __forceinline__ uint32_t xcd_remap(uint32_t lin, uint32_t total) {
  const uint32_t nx = 8;
  const uint32_t q = total / nx, r = total % nx;
  const uint32_t x = lin % nx, slot = lin / nx;
  return x * q + (x < r ? x : r) + slot;
}

// Work order of packed (varlen) launches over (sequence, head, block) items. The pairs
// p = s·H + h go to XCD p % 8, so every sequence's heads spread evenly over the XCDs, and each
// XCD takes its pairs one after another, all nblk blocks of a pair in a row: its CUs work on
// one head's keys and values at a time and share them in its L2 (dealing consecutive blocks of
// a pair to different XCDs made every XCD fetch the same keys and values from memory). The
// grid holds nblk slots for each of 8·ceil(H·nseq/8) pairs; slots past the last pair return
// false. Blocks past a sequence's length are left to the caller (they exit at once).
__device__ __forceinline__ bool varlen_order(uint32_t lin, int nblk, int H, int nseq, int& blk,
                                             int& h, int& s) {
  const uint32_t x = lin % 8, slot = lin / 8;
  const uint32_t p = x + 8 * (slot / (uint32_t)nblk);
  blk = (int)(slot % (uint32_t)nblk);
  if (p >= (uint32_t)H * (uint32_t)nseq) return false;
  h = (int)(p % (uint32_t)H);
  s = (int)(p / (uint32_t)H);
  return true;
}
// Grid size of a packed launch for varlen_order: nblk slots for each of 8·ceil(H·nseq/8) pairs.
__host__ __device__ __forceinline__ long varlen_grid(int nblk, int H, int nseq) {
  return (long)nblk * 8 * (((long)H * nseq + 7) / 8);
}

// Work order for causal launches over items (bh, r) whose cost falls with the rank r (r = 0
// is the longest). The hardware deals workgroups round-robin over the 8 XCDs and each XCD
// starts its share in order; here XCD x keeps a contiguous range of whole (b, h) slices (their
// K/V share its L2) and hands out all of their rank-0 items, then all rank-1 items, and so
// on: longest first across the slices, so no long item is left for the end. When the slices
// do not split evenly over the XCDs the order is rank-major over all slices.
__device__ __forceinline__ void causal_order(uint32_t lin, int nbh, int& rank, int& bh) {
  const uint32_t nx = 8;
  if (nbh % nx == 0) {
    const uint32_t per = nbh / nx;  // slices per XCD
    const uint32_t x = lin % nx, slot = lin / nx;
    rank = (int)(slot / per);
    bh = (int)(x * per + slot % per);
  } else {
    rank = (int)(lin / (uint32_t)nbh);
    bh = (int)(lin % (uint32_t)nbh);
  }
}

}  // namespace fa
