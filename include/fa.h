/*
 * fa.h - C ABI of the MI355X (gfx950) exact-attention library (libfa_mi355x.so).
 *
 * The library computes exact attention O = softmax(scale * Q K^T) V, tiled so that the
 * N x N score matrix S and probability matrix P exist only as on-chip tiles and are never
 * written to device memory. Definitions: "FlashAttention 详解（零基础入门）"
 * (https://blog-dist-2hw.pages.dev/2026/07/19/flashattention-guide/) §2.3-§2.6 for
 * S = Q K^T / sqrt(d), P = softmax(S), O = P V, §2.4 for the max-subtracted softmax, §5-§6
 * for online softmax and the tiled loop; "FlashAttention 短片讲解稿"
 * (https://xuujii.github.io/ai-infra-kb/videos/flashattention/讲解稿.md), segment 第三招 ·
 * 反向重计算, for the backward pass that recomputes P tiles from the inputs, the output and
 * per-row statistics; "FlashAttention 与算子融合"
 * (https://ai-infra-wiki.pages.dev/compilers-kernels/02-kernels/flash-attention/), fusion
 * table (mask fused into the kernel) and 工程实践 (varlen packing instead of padding).
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller. The library allocates
 *    nothing, keeps no global state, never synchronises, and enqueues its kernels on
 *    `stream` (a hipStream_t; NULL means the default stream). Kernels are launched on the
 *    calling thread's current HIP device, to which the tensors and the stream must belong.
 *    Calls on different streams may run concurrently.
 *  - Layout: q, k, v, o, dout, dq, dk, dv are [B, N, H, d] row-major (d contiguous, then
 *    heads, then tokens, then batch), 16-byte aligned. lse is fp32 [B, H, N].
 *    Packed (varlen) tensors are [T, H, d] with lse fp32 [H, T].
 *  - Element type: dtype FA_BF16 or FA_F16 for q, k, v, o, dout, dq, dk, dv. Products
 *    accumulate in fp32; P is rounded to the element type (nearest even) before P V.
 *  - head dim d must be 64 or 128.
 *  - softmax_scale multiplies the scores before the softmax; pass 1/sqrt(d) for the
 *    usual attention. Any finite value is accepted.
 *  - causal != 0 masks key j for query i when j > i (positions within the sequence).
 *  - lse[i] = m_i + ln(l_i), the natural-log log-sum-exp of row i's scaled, masked scores.
 *  - Errors: argument checks are synchronous and return a status without launching
 *    anything. FA_ERR_HIP reports a launch failure (hipGetLastError after the launch);
 *    faults inside a kernel surface at the caller's next synchronisation, as for any
 *    stream work.
 */
#ifndef FA_MI355X_H
#define FA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = 1, /* null pointer, negative size, non-finite scale, bad layout */
  FA_ERR_UNSUPPORTED = 2, /* valid request outside what the kernels handle (head dim, sizes) */
  FA_ERR_HIP = 3          /* a HIP launch reported an error */
} fa_status;

/* Element type codes, passed as the int argument dtype (any other value is rejected with
 * FA_ERR_INVALID_ARG). */
typedef enum { FA_F16 = 0, FA_BF16 = 1 } fa_dtype;

/* Short static description of a status code (an fa_status value; any other int gives
 * "unknown status"). Never NULL. */
const char* fa_status_string(int status);

/*
 * Forward pass (guide §6.2 tiled algorithm; narration 第二招 for the deferred
 * normalisation): for each (b, h), O = softmax(scale * Q K^T [+ causal mask]) V and the
 * per-row log-sum-exp.
 *   q, k, v : in,  [B, N, H, d], dtype
 *   o       : out, [B, N, H, d], dtype
 *   lse     : out, fp32 [B, H, N]
 * B, N, H >= 0 (B*N*H == 0 is a no-op returning FA_OK). Limits (else FA_ERR_UNSUPPORTED):
 * (N + 256) * H * d < 2^30 (row offsets of a slice fit in 31 bits), B * N < 2^31 tokens, and
 * 8 * ceil(B * H / 8) * ceil(N / 128) < 2^31 (the workgroup count of the largest launch).
 */
fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                 int N, int H, int d, int dtype, float softmax_scale, int causal,
                 hipStream_t stream);

/*
 * FP8 forward: the forward above with q, k, v stored as OCP FP8 E4M3 codes ("e4m3fn": 1 sign,
 * 4 exponent (bias 7), 3 mantissa bits; largest finite 448; no infinities) and one fp32
 * descale factor per tensor, so that the value of an element is descale * (code's value).
 * "FlashAttention 与算子融合" (代际演进 table, 工程实践 precision note) names FP8 as the path
 * FlashAttention-3 adds; the per-tensor descales and the output type are this library's.
 *   q, k, v : in,  [B, N, H, d], one byte per element (e4m3 codes), 16-byte aligned
 *   o       : out, [B, N, H, d], bf16
 *   lse     : out, fp32 [B, H, N], the log-sum-exp of the scaled scores
 *             softmax_scale * q_descale * k_descale * <q_i, k_j>
 * Computes O = v_descale * softmax(softmax_scale * q_descale * k_descale * Q K^T
 * [+ causal mask]) V with both products on the FP8 matrix cores (fp32 accumulation) and P
 * rounded to e4m3 (nearest even) before P V; the row sums add exactly those rounded values.
 * q_descale, k_descale, v_descale must be finite and > 0 (else FA_ERR_INVALID_ARG), as must
 * their product with |softmax_scale|; the other arguments and limits are fa_fwd's. The
 * per-element error against exact attention of the stored values is bounded by P's rounding:
 * each weight's relative error is at most 2^-4 (absolute 2^-10 of the row's largest weight
 * below e4m3's normal range), plus the bf16 rounding of the output.
 */
fa_status fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                     int N, int H, int d, float q_descale, float k_descale, float v_descale,
                     float softmax_scale, int causal, hipStream_t stream);

/*
 * Merge of a partial attention result into a running one: the per-device step of ring
 * (context-parallel) attention, where each device keeps its query rows and attends them to
 * one K/V shard per step ("FlashAttention 与算子融合", 代际演进 table and 工程实践: ring attention
 * with FlashAttention as the compute core), combined with the block-merge rule of the same
 * page (section FlashAttention 的两个关键). For the same query rows, (o_acc, lse_acc) hold the
 * result over the keys seen so far and (o_part, lse_part) the result over a disjoint set of
 * keys, e.g. fa_fwd on one shard. In place, per row:
 *   lse_acc <- ln(e^lse_acc + e^lse_part)
 *   o_acc   <- o_acc e^(lse_acc_old - lse_acc) + o_part e^(lse_part - lse_acc)
 * A side whose lse is -inf (no visible key) contributes nothing, whatever its o values;
 * both -inf gives o_acc = 0, lse_acc = -inf. Start a ring from lse_acc = -inf (o_acc's
 * contents are then ignored).
 *   o_acc    : in/out, fp32 [B, N, H, d], 16-byte aligned (kept in fp32 across merges)
 *   lse_acc  : in/out, fp32 [B, H, N]
 *   o_part   : in, [B, N, H, d], dtype
 *   lse_part : in, fp32 [B, H, N]
 *   out      : out, [B, N, H, d], dtype, or NULL: the merged output rounded to dtype
 * dtype FA_BF16 or FA_F16, d 64 or 128, sizes and limits as fa_fwd (B * N tokens aside),
 * and B * N * H < 2^34. Deterministic. For the backward, fa_bwd on each shard with the merged o (rounded) and lse gives that shard's dK,
 * dV and its share of dQ (the shares of dQ add up).
 */
fa_status fa_merge(float* o_acc, float* lse_acc, const void* o_part, const float* lse_part,
                   void* out, int B, int N, int H, int d, int dtype, hipStream_t stream);

/*
 * Bytes of device workspace fa_bwd needs: 8 * B * H * N (two fp32 row terms per query:
 * -D_i = -<dO_i, O_i> and -LSE_i * log2(e)). Linear in N: the backward never stores an
 * N x N matrix. Returns 0 for arguments fa_bwd would reject as sizes (negative sizes or a
 * head dim other than 64 or 128).
 */
size_t fa_bwd_workspace_size(int B, int N, int H, int d);

/*
 * Backward pass (narration 第三招 · 反向重计算: P is recomputed tile by tile from q, k and
 * the forward's lse instead of being stored). Gradients of the loss through O:
 *   P_ij = exp(scale <q_i,k_j> - lse_i), D_i = <dO_i, O_i>, dV_j = sum_i P_ij dO_i,
 *   dS_ij = P_ij (<dO_i, v_j> - D_i), dQ_i = scale sum_j dS_ij k_j,
 *   dK_j = scale sum_i dS_ij q_i.
 *   q, k, v, o, dout : in,  [B, N, H, d], dtype (o and lse from fa_fwd with the same
 *                      scale and causal flag)
 *   lse              : in,  fp32 [B, H, N]
 *   dq, dk, dv       : out, [B, N, H, d], dtype
 *   workspace        : scratch of fa_bwd_workspace_size(B, N, H, d) bytes, 16-byte
 *                      aligned; its contents are overwritten. May be NULL if that size is 0.
 * Deterministic: no floating-point atomics; repeated calls give identical bits.
 */
fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o,
                 const float* lse, const void* dout, void* dq, void* dk, void* dv,
                 void* workspace, int B, int N, int H, int d, int dtype,
                 float softmax_scale, int causal, hipStream_t stream);

/*
 * The three stages fa_bwd runs, in this order, for callers that schedule or time them
 * separately. Each takes exactly fa_bwd's arguments and validates them the same way.
 *   fa_bwd_prep : writes the row terms (-D_i and -LSE_i * log2(e)) into workspace; reads
 *                 o, dout, lse.
 *   fa_bwd_dkdv : dk and dv; reads q, k, v, dout and the workspace row terms.
 *   fa_bwd_dq   : dq; reads q, k, v, dout and the workspace row terms.
 * fa_bwd_dkdv and fa_bwd_dq need the row terms of an fa_bwd_prep call with the same
 * arguments, completed earlier on the stream (or otherwise ordered before them).
 */
fa_status fa_bwd_prep(const void* q, const void* k, const void* v, const void* o,
                      const float* lse, const void* dout, void* dq, void* dk, void* dv,
                      void* workspace, int B, int N, int H, int d, int dtype,
                      float softmax_scale, int causal, hipStream_t stream);
fa_status fa_bwd_dkdv(const void* q, const void* k, const void* v, const void* o,
                      const float* lse, const void* dout, void* dq, void* dk, void* dv,
                      void* workspace, int B, int N, int H, int d, int dtype,
                      float softmax_scale, int causal, hipStream_t stream);
fa_status fa_bwd_dq(const void* q, const void* k, const void* v, const void* o,
                    const float* lse, const void* dout, void* dq, void* dk, void* dv,
                    void* workspace, int B, int N, int H, int d, int dtype,
                    float softmax_scale, int causal, hipStream_t stream);

/*
 * Forward pass over packed sequences (fusion page, 工程实践: pack unequal lengths instead
 * of padding). Sequence s occupies tokens [cu_seqlens[s], cu_seqlens[s+1]) of the packed
 * tensors and is an independent attention problem; the causal mask is relative to the
 * start of each sequence.
 *   q, k, v     : in,  [total_tokens, H, d], dtype
 *   o           : out, [total_tokens, H, d], dtype
 *   lse         : out, fp32 [H, total_tokens]
 *   cu_seqlens  : in,  device int32 [num_seqs + 1], cu[0] = 0, non-decreasing,
 *                 cu[num_seqs] = total_tokens
 *   max_seqlen  : host-side upper bound on the sequence lengths (sizes the grid without a
 *                 device-to-host copy); lengths above it are not processed.
 * Limits: (max_seqlen + 256) * H * d < 2^30 and 8 * ceil(num_seqs * H / 8) *
 * ceil(max_seqlen / 128) < 2^31. Sequences longer than max_seqlen are treated as truncated
 * to max_seqlen tokens (their later rows are not written). A malformed cu_seqlens gives
 * undefined results (out-of-range rows are clamped by hardware bounds checks, never read or
 * written outside the packed tensors). With the environment variable FA_DEBUG set to anything but "" or
 * "0" (read at every call), the call first copies cu_seqlens to the host on `stream`,
 * waits for the stream, and returns FA_ERR_INVALID_ARG without launching anything if
 * cu[0] != 0, cu decreases anywhere or cu[num_seqs] != total_tokens (or the copy fails).
 */
fa_status fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                        const int32_t* cu_seqlens, int num_seqs, int total_tokens,
                        int max_seqlen, int H, int d, int dtype, float softmax_scale,
                        int causal, hipStream_t stream);

/*
 * Backward pass over packed sequences: fa_bwd's computation for each sequence of an
 * fa_fwd_varlen call (same cu_seqlens, max_seqlen, scale and causal flag).
 *   q, k, v, o, dout : in,  [total_tokens, H, d], dtype
 *   lse              : in,  fp32 [H, total_tokens] (from fa_fwd_varlen)
 *   dq, dk, dv       : out, [total_tokens, H, d], dtype; rows of tokens outside every
 *                      sequence are not written
 *   workspace        : fa_bwd_workspace_size(1, total_tokens, H, d) bytes, 16-byte aligned
 * Other arguments, limits, errors and the FA_DEBUG check as fa_fwd_varlen; deterministic
 * like fa_bwd.
 */
fa_status fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o,
                        const float* lse, const void* dout, void* dq, void* dk, void* dv,
                        void* workspace, const int32_t* cu_seqlens, int num_seqs,
                        int total_tokens, int max_seqlen, int H, int d, int dtype,
                        float softmax_scale, int causal, hipStream_t stream);

/*
 * Split-KV forward for decode shapes: Nq query rows (e.g. the newest tokens of each
 * sequence) against Nk cached keys and values. The keys are cut into num_splits contiguous
 * ranges processed in parallel; each range is reduced to a partial (O, m, l) by the online
 * softmax and the partials are combined with the block-merge rule of "FlashAttention 与算子
 * 融合" (section on the two keys of FlashAttention): m = max m_s, l = sum l_s exp(m_s - m),
 * O = sum O_s l_s exp(m_s - m) / l. The narration script ("FlashAttention 短片讲解稿",
 * segment 适用范围与关键结论) singles this shape out as different from training and prefill.
 *   q          : in,  [B, Nq, H, d], dtype
 *   k, v       : in,  [B, Nk, H, d], dtype
 *   o          : out, [B, Nq, H, d], dtype
 *   lse        : out, fp32 [B, H, Nq]
 *   workspace  : fa_fwd_splitkv_workspace_size(B, Nq, Nk, H, d, num_splits) bytes, 16-byte
 *                aligned; its contents are overwritten
 *   num_splits : key ranges per (b, h); 0 lets the library choose from the shape. Values
 *                above ceil(Nk / 32) are lowered to it. 0 <= num_splits <= 4096.
 *   causal     : query row i stands at position Nk - Nq + i and sees keys j <= Nk - Nq + i
 *                (none when Nk - Nq + i < 0: such rows get O = 0 and lse = -inf). With
 *                Nq = Nk this is fa_fwd's causal mask.
 * B, Nq, H >= 0 (B*Nq*H == 0 is a no-op returning FA_OK); Nk >= 1.
 * Limits: (Nk + 256) * H * d < 2^30, (Nq + 256) * H * d < 2^30, B * H * S * ceil(Nq / 32)
 * < 2^31 (S the number of key ranges used) and B * H * Nq < 2^31.
 * Deterministic: a fixed num_splits gives identical bits on every call.
 */
size_t fa_fwd_splitkv_workspace_size(int B, int Nq, int Nk, int H, int d, int num_splits);
fa_status fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                         void* workspace, int B, int Nq, int Nk, int H, int d, int dtype,
                         float softmax_scale, int causal, int num_splits, hipStream_t stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): fa_fwd_splitkv with its workspace in the
 * library's own scratch array instead of a workspace argument. Same arguments, results and
 * errors as fa_fwd_splitkv otherwise; the caller still passes q, k, v, o and lse.
 *   - The scratch array is a static device array of fa_noalloc_scratch_bytes() bytes
 *     (8 MiB), one copy per GPU, held until the process ends. A request whose
 *     fa_fwd_splitkv_workspace_size exceeds it returns FA_ERR_UNSUPPORTED before any launch.
 *   - The first call on a device looks up that device's copy (hipGetSymbolAddress, with the
 *     device current); a failure there returns FA_ERR_HIP. No call allocates or frees memory.
 *   - Every call on one GPU uses the same array: calls that overlap in time on one GPU (on
 *     different streams, or from several host threads) race on it and give undefined
 *     results. Calls in order on one stream are safe. Nothing in the array needs clearing:
 *     the first kernel writes every partial the second one reads.
 */
size_t fa_noalloc_scratch_bytes(void);
fa_status fa_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o,
                                 float* lse, int B, int Nq, int Nk, int H, int d, int dtype,
                                 float softmax_scale, int causal, int num_splits,
                                 hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_H */
