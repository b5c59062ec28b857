// Exact-attention oracle: plain fp64 CPU implementation of what the GPU path computes.
//
// TEST INFRASTRUCTURE ONLY. Nothing in the product library links, loads or calls this
// file; only the test suite, the smoke check and the benchmark's CPU-baseline leg do.
// It shares no source, header, table or helper with the GPU kernels.
//
// What it computes (pages: "FlashAttention 详解（零基础入门）" §2.3-§2.6 for the
// definition, §5.2-§5.4 and the §6.2 tiled algorithm for the blocked forms; the
// narration script "FlashAttention 短片讲解稿", segment 第二招 · 在线 Softmax, for the
// deferred-normalisation form; "FlashAttention 与算子融合" for the causal mask fused into
// the kernel and for varlen packing):
//
//   s_ij  = scale * <q_i, k_j>                       (definition of S, §2.3)
//   m_i   = max_{j in J(i)} s_ij                     (safe softmax, §2.4)
//   l_i   = sum_{j in J(i)} exp(s_ij - m_i)
//   O_i   = sum_{j in J(i)} exp(s_ij - m_i) v_j / l_i   (O = PV, §2.5)
//   LSE_i = m_i + ln l_i                              (natural log)
//
// J(i) = {0..L-1} without a mask, {0..i} with the causal mask. A row with no visible key
// (never produced by the supported inputs) is defined as O_i = 0, LSE_i = -inf.
//
// Backward: the pages state only that P is recomputed from Q, K, V, O and the saved row
// statistics; the gradients are the chain rule through the definition above:
//   P_ij = exp(s_ij - LSE_i), D_i = <dO_i, O_i>, dP_ij = <dO_i, v_j>,
//   dS_ij = P_ij (dP_ij - D_i), dV_j = sum_i P_ij dO_i,
//   dQ_i = scale sum_j dS_ij k_j, dK_j = scale sum_i dS_ij q_i.
//
// Layouts: q, k, v, o, dout, dq, dk, dv are [B, N, H, d] (d contiguous); lse is [B, H, N].
// Varlen: the same with B = 1 and N = total tokens ([T, H, d], lse [H, T]); sequence s
// occupies tokens [cu[s], cu[s+1]) and is an independent attention problem.
//
// Decode shapes (Nq query rows against Nk keys, e.g. the last Nq positions of a sequence
// whose keys and values are all cached): query row i stands at position Nk - Nq + i; with
// the causal mask it sees keys j <= Nk - Nq + i (none when that is negative), without it all
// Nk keys. For Nq = Nk this is the mask above. The split form cuts the keys into contiguous
// ranges, takes (m, l, O) of each range from the definition restricted to it, and combines
// them with the block-merge rule ("FlashAttention 与算子融合", section on the two keys of
// FlashAttention): m = max_s m_s, l = sum_s l_s exp(m_s - m), and the outputs rescaled the
// same way, O = sum_s O_s l_s exp(m_s - m) / l.
//
// Threads only split independent output rows (or heads); every sum is accumulated in
// natural index order, so results do not depend on the thread count.

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <limits>
#include <thread>
#include <vector>

namespace {

const double kNegInf = -std::numeric_limits<double>::infinity();

// One attention problem: a single (batch, head) or (sequence, head) slice.
struct Slice {
  const double* q;   // row i at q + i * rs
  const double* k;
  const double* v;
  double* o;
  double* lse;       // lse[i * ls]
  long rs;           // row stride in elements (H * d)
  long ls;           // lse stride (1)
  long L;            // rows (= keys) in this slice
};

long visible_end(long i, long L, int causal) { return causal ? std::min(i + 1, L) : L; }

double dot(const double* a, const double* b, long d) {
  double s = 0.0;
  for (long c = 0; c < d; ++c) s += a[c] * b[c];
  return s;
}

// Run fn(item) for item in [0, n) on up to nthreads threads.
template <class F>
void parallel_for(long n, int nthreads, F fn) {
  if (nthreads <= 1 || n <= 1) {
    for (long i = 0; i < n; ++i) fn(i);
    return;
  }
  std::atomic<long> next(0);
  int nt = (int)std::min<long>(nthreads, n);
  std::vector<std::thread> pool;
  for (int t = 0; t < nt; ++t)
    pool.emplace_back([&]() {
      for (long i = next.fetch_add(1); i < n; i = next.fetch_add(1)) fn(i);
    });
  for (auto& th : pool) th.join();
}

// Plain definition, rows [r0, r1) of one slice.
void fwd_rows(const Slice& s, long d, double scale, int causal, long r0, long r1) {
  std::vector<double> sc(s.L);
  for (long i = r0; i < r1; ++i) {
    const long je = visible_end(i, s.L, causal);
    const double* qi = s.q + i * s.rs;
    double m = kNegInf;
    for (long j = 0; j < je; ++j) {
      sc[j] = scale * dot(qi, s.k + j * s.rs, d);
      m = std::max(m, sc[j]);
    }
    double* oi = s.o + i * s.rs;
    for (long c = 0; c < d; ++c) oi[c] = 0.0;
    if (je == 0) {
      s.lse[i * s.ls] = kNegInf;
      continue;
    }
    double l = 0.0;
    for (long j = 0; j < je; ++j) {
      const double p = std::exp(sc[j] - m);
      l += p;
      const double* vj = s.v + j * s.rs;
      for (long c = 0; c < d; ++c) oi[c] += p * vj[c];
    }
    for (long c = 0; c < d; ++c) oi[c] /= l;
    s.lse[i * s.ls] = m + std::log(l);
  }
}

// Tiled algorithm: query block [i0, i0+Bq) against every key block of size Bk, keeping a
// running max m, running sum l and an output state per row (guide §5.4 and §6.2).
//   form 0 (normalised): the state is O itself, re-normalised by l after every block.
//   form 1 (deferred, as in the narration script): the state is the unnormalised
//           numerator sum exp(s - m) v, divided by l once after the last block.
// trace (nullable) receives, for row i0 only, one triple per key block:
//   (m, l, state[0]) after that block.
void fwd_block(const Slice& s, long d, double scale, int causal, long i0, long Bq, long Bk,
               int form, double* trace) {
  const long i1 = std::min(i0 + Bq, s.L);
  const long nb = (s.L + Bk - 1) / Bk;
  std::vector<double> m(i1 - i0, kNegInf), l(i1 - i0, 0.0), st((i1 - i0) * d, 0.0);
  std::vector<double> sblk(Bk), p(Bk);
  for (long jb = 0; jb < nb; ++jb) {
    const long j0 = jb * Bk, j1 = std::min(j0 + Bk, s.L);
    for (long i = i0; i < i1; ++i) {
      const long r = i - i0;
      const long je = std::min(j1, visible_end(i, s.L, causal));
      double mb = kNegInf;
      for (long j = j0; j < je; ++j) {
        sblk[j - j0] = scale * dot(s.q + i * s.rs, s.k + j * s.rs, d);
        mb = std::max(mb, sblk[j - j0]);
      }
      const double mn = std::max(m[r], mb);
      if (mn != kNegInf) {  // otherwise no key of this row has been visible yet
        const double alpha = std::exp(m[r] - mn);  // exp(-inf) = 0 on the first block
        double rowsum = 0.0;
        for (long j = j0; j < je; ++j) {
          p[j - j0] = std::exp(sblk[j - j0] - mn);
          rowsum += p[j - j0];
        }
        const double ln = l[r] * alpha + rowsum;
        double* sr = st.data() + r * d;
        for (long c = 0; c < d; ++c) {
          double pv = 0.0;
          for (long j = j0; j < je; ++j) pv += p[j - j0] * s.v[j * s.rs + c];
          if (form == 0)
            sr[c] = sr[c] * (l[r] / ln) * alpha + pv / ln;
          else
            sr[c] = sr[c] * alpha + pv;
        }
        m[r] = mn;
        l[r] = ln;
      }
      if (trace && i == i0) {
        trace[3 * jb + 0] = m[r];
        trace[3 * jb + 1] = l[r];
        trace[3 * jb + 2] = st[r * d];
      }
    }
  }
  for (long i = i0; i < i1; ++i) {
    const long r = i - i0;
    double* oi = s.o + i * s.rs;
    for (long c = 0; c < d; ++c) {
      if (l[r] == 0.0)
        oi[c] = 0.0;
      else
        oi[c] = form == 0 ? st[r * d + c] : st[r * d + c] / l[r];
    }
    s.lse[i * s.ls] = l[r] == 0.0 ? kNegInf : m[r] + std::log(l[r]);
  }
}

struct GradSlice {
  Slice f;
  const double* dout;
  double* dq;
  double* dk;
  double* dv;
};

// dQ for rows [r0, r1): dQ_i = scale * sum_j P_ij (dP_ij - D_i) k_j.
void bwd_dq_rows(const GradSlice& g, long d, double scale, int causal, long r0, long r1) {
  const Slice& s = g.f;
  for (long i = r0; i < r1; ++i) {
    const long je = visible_end(i, s.L, causal);
    const double* qi = s.q + i * s.rs;
    const double* doi = g.dout + i * s.rs;
    const double Di = dot(doi, s.o + i * s.rs, d);
    const double lse = s.lse[i * s.ls];
    double* dqi = g.dq + i * s.rs;
    for (long c = 0; c < d; ++c) dqi[c] = 0.0;
    for (long j = 0; j < je; ++j) {
      const double P = std::exp(scale * dot(qi, s.k + j * s.rs, d) - lse);
      const double dP = dot(doi, s.v + j * s.rs, d);
      const double dS = P * (dP - Di);
      const double* kj = s.k + j * s.rs;
      for (long c = 0; c < d; ++c) dqi[c] += dS * kj[c];
    }
    for (long c = 0; c < d; ++c) dqi[c] *= scale;
  }
}

// dK, dV for key rows [c0, c1): dV_j = sum_i P_ij dO_i, dK_j = scale * sum_i dS_ij q_i,
// over the query rows i that see key j.
void bwd_dkdv_rows(const GradSlice& g, long d, double scale, int causal, long c0, long c1) {
  const Slice& s = g.f;
  for (long j = c0; j < c1; ++j) {
    const double* kj = s.k + j * s.rs;
    const double* vj = s.v + j * s.rs;
    double* dkj = g.dk + j * s.rs;
    double* dvj = g.dv + j * s.rs;
    for (long c = 0; c < d; ++c) dkj[c] = dvj[c] = 0.0;
    for (long i = causal ? j : 0; i < s.L; ++i) {
      const double* qi = s.q + i * s.rs;
      const double* doi = g.dout + i * s.rs;
      const double Di = dot(doi, s.o + i * s.rs, d);
      const double P = std::exp(scale * dot(qi, kj, d) - s.lse[i * s.ls]);
      const double dP = dot(doi, vj, d);
      const double dS = P * (dP - Di);
      for (long c = 0; c < d; ++c) {
        dvj[c] += P * doi[c];
        dkj[c] += dS * qi[c];
      }
    }
    for (long c = 0; c < d; ++c) dkj[c] *= scale;
  }
}

const long kRowChunk = 32;

bool bad_sizes(long B, long N, long H, long d) { return B < 0 || N < 0 || H <= 0 || d <= 0; }

// ---------------------------------------------------------------- decode shapes
// Keys visible to query row i of Nq against Nk keys (see the header).
long decode_visible_end(long i, long Nq, long Nk, int causal) {
  if (!causal) return Nk;
  const long e = Nk - Nq + i + 1;
  return e < 0 ? 0 : (e > Nk ? Nk : e);
}

// One (batch, head) of a decode problem.
struct DecodeSlice {
  const double* q;  // query row i at q + i * rs
  const double* k;  // key row j at k + j * rs
  const double* v;
  long rs;          // row stride in elements (H * d)
  long Nq, Nk;
};

// (m, l, O) of query row i over the visible keys in [j0, j1): the plain definition restricted
// to those keys, O normalised by l. An empty range gives m = -inf, l = 0, O = 0.
void decode_partial(const DecodeSlice& s, long d, double scale, int causal, long i, long j0,
                    long j1, double* o, double& m, double& l) {
  const long je = std::min(j1, decode_visible_end(i, s.Nq, s.Nk, causal));
  const double* qi = s.q + i * s.rs;
  for (long c = 0; c < d; ++c) o[c] = 0.0;
  m = kNegInf;
  l = 0.0;
  if (je <= j0) return;
  std::vector<double> sc(je - j0);
  for (long j = j0; j < je; ++j) {
    sc[j - j0] = scale * dot(qi, s.k + j * s.rs, d);
    m = std::max(m, sc[j - j0]);
  }
  for (long j = j0; j < je; ++j) {
    const double p = std::exp(sc[j - j0] - m);
    l += p;
    const double* vj = s.v + j * s.rs;
    for (long c = 0; c < d; ++c) o[c] += p * vj[c];
  }
  for (long c = 0; c < d; ++c) o[c] /= l;
}

// Block-merge rule over n partial results (m_s, l_s, O_s), O_s normalised by l_s.
void merge_partials(long n, long d, const double* ms, const double* ls, const double* os,
                    double* o, double& lse) {
  double m = kNegInf;
  for (long t = 0; t < n; ++t) m = std::max(m, ms[t]);
  for (long c = 0; c < d; ++c) o[c] = 0.0;
  if (m == kNegInf) {  // no visible key in any part
    lse = kNegInf;
    return;
  }
  double l = 0.0;
  for (long t = 0; t < n; ++t) {
    if (ls[t] == 0.0) continue;
    const double w = ls[t] * std::exp(ms[t] - m);
    l += w;
    for (long c = 0; c < d; ++c) o[c] += w * os[t * d + c];
  }
  for (long c = 0; c < d; ++c) o[c] /= l;
  lse = m + std::log(l);
}

DecodeSlice decode_slice(const double* q, const double* k, const double* v, long Nq, long Nk,
                         long H, long d, long idx) {
  const long b = idx / H, h = idx % H;
  return DecodeSlice{q + (b * Nq * H + h) * d, k + (b * Nk * H + h) * d,
                     v + (b * Nk * H + h) * d, H * d, Nq, Nk};
}

// Slices of a dense [B, N, H, d] problem: slice index = b * H + h.
Slice dense_slice(const double* q, const double* k, const double* v, double* o, double* lse,
                  long N, long H, long d, long idx) {
  const long b = idx / H, h = idx % H;
  const long off = b * N * H * d + h * d;
  return Slice{q + off, k + off, v + off, o + off, lse + (b * H + h) * N, H * d, 1, N};
}

}  // namespace

extern "C" {

// Plain definition (O1-O4). Returns 0, or -1 on bad sizes.
int oracle_fwd(const double* q, const double* k, const double* v, double* o, double* lse,
               long B, long N, long H, long d, double scale, int causal, int nthreads) {
  if (bad_sizes(B, N, H, d)) return -1;
  const long chunks = (N + kRowChunk - 1) / kRowChunk;
  parallel_for(B * H * chunks, nthreads, [&](long it) {
    Slice s = dense_slice(q, k, v, o, lse, N, H, d, it / chunks);
    const long r0 = (it % chunks) * kRowChunk;
    fwd_rows(s, d, scale, causal, r0, std::min(r0 + kRowChunk, N));
  });
  return 0;
}

// Tiled algorithm with query blocks of Bq rows and key blocks of Bk rows (any sizes >= 1,
// divisors of N or not). form: 0 normalised update, 1 deferred normalisation.
// trace (nullable) gets (m, l, state[0]) after each key block for row 0 of slice (0, 0):
// 3 * ceil(N / Bk) doubles.
int oracle_fwd_blocked(const double* q, const double* k, const double* v, double* o,
                       double* lse, long B, long N, long H, long d, double scale, int causal,
                       long Bq, long Bk, int form, double* trace, int nthreads) {
  if (bad_sizes(B, N, H, d) || Bq < 1 || Bk < 1 || (form != 0 && form != 1)) return -1;
  const long qblocks = (N + Bq - 1) / Bq;
  parallel_for(B * H * qblocks, nthreads, [&](long it) {
    const long idx = it / qblocks, ib = it % qblocks;
    Slice s = dense_slice(q, k, v, o, lse, N, H, d, idx);
    fwd_block(s, d, scale, causal, ib * Bq, Bq, Bk, form, (idx == 0 && ib == 0) ? trace : nullptr);
  });
  return 0;
}

// Gradients from the saved O and LSE (B1-B4 of the chain rule above).
int oracle_bwd(const double* q, const double* k, const double* v, const double* o,
               const double* lse, const double* dout, double* dq, double* dk, double* dv,
               long B, long N, long H, long d, double scale, int causal, int nthreads) {
  if (bad_sizes(B, N, H, d)) return -1;
  const long chunks = (N + kRowChunk - 1) / kRowChunk;
  auto grad_slice = [&](long idx) {
    const long b = idx / H, h = idx % H;
    const long off = b * N * H * d + h * d;
    GradSlice g{Slice{q + off, k + off, v + off, const_cast<double*>(o + off),
                      const_cast<double*>(lse + (b * H + h) * N), H * d, 1, N},
                dout + off, dq + off, dk + off, dv + off};
    return g;
  };
  parallel_for(B * H * chunks, nthreads, [&](long it) {
    GradSlice g = grad_slice(it / chunks);
    const long r0 = (it % chunks) * kRowChunk;
    bwd_dq_rows(g, d, scale, causal, r0, std::min(r0 + kRowChunk, N));
  });
  parallel_for(B * H * chunks, nthreads, [&](long it) {
    GradSlice g = grad_slice(it / chunks);
    const long c0 = (it % chunks) * kRowChunk;
    bwd_dkdv_rows(g, d, scale, causal, c0, std::min(c0 + kRowChunk, N));
  });
  return 0;
}

// Packed sequences: q, k, v, o [T, H, d]; lse [H, T]; cu_seqlens int32 [nseq + 1].
// Returns -2 if cu_seqlens is not a valid prefix-sum array (cu[0] = 0, non-decreasing,
// cu[nseq] = T).
int oracle_fwd_varlen(const double* q, const double* k, const double* v, double* o,
                      double* lse, const int32_t* cu, long nseq, long T, long H, long d,
                      double scale, int causal, int nthreads) {
  if (nseq < 0 || T < 0 || H <= 0 || d <= 0) return -1;
  if (cu[0] != 0 || cu[nseq] != T) return -2;
  for (long s = 0; s < nseq; ++s)
    if (cu[s + 1] < cu[s]) return -2;
  // work items: (sequence, head, row chunk)
  std::vector<long> first(nseq + 1, 0);
  for (long s = 0; s < nseq; ++s)
    first[s + 1] = first[s] + H * ((cu[s + 1] - cu[s] + kRowChunk - 1) / kRowChunk);
  parallel_for(first[nseq], nthreads, [&](long it) {
    const long s = std::upper_bound(first.begin(), first.end(), it) - first.begin() - 1;
    const long L = cu[s + 1] - cu[s];
    const long chunks = (L + kRowChunk - 1) / kRowChunk;
    const long h = (it - first[s]) / chunks, r0 = ((it - first[s]) % chunks) * kRowChunk;
    const long off = (long)cu[s] * H * d + h * d;
    Slice sl{q + off, k + off, v + off, o + off, lse + h * T + cu[s], H * d, 1, L};
    fwd_rows(sl, d, scale, causal, r0, std::min(r0 + kRowChunk, L));
  });
  return 0;
}

// Packed-sequence gradients (same layouts as oracle_fwd_varlen; dout, dq, dk, dv [T, H, d]).
int oracle_bwd_varlen(const double* q, const double* k, const double* v, const double* o,
                      const double* lse, const double* dout, double* dq, double* dk,
                      double* dv, const int32_t* cu, long nseq, long T, long H, long d,
                      double scale, int causal, int nthreads) {
  if (nseq < 0 || T < 0 || H <= 0 || d <= 0) return -1;
  if (cu[0] != 0 || cu[nseq] != T) return -2;
  for (long s = 0; s < nseq; ++s)
    if (cu[s + 1] < cu[s]) return -2;
  parallel_for(nseq * H, nthreads, [&](long it) {
    const long s = it / H, h = it % H;
    const long L = cu[s + 1] - cu[s];
    const long off = (long)cu[s] * H * d + h * d;
    GradSlice g{Slice{q + off, k + off, v + off, const_cast<double*>(o + off),
                      const_cast<double*>(lse + h * T + cu[s]), H * d, 1, L},
                dout + off, dq + off, dk + off, dv + off};
    bwd_dq_rows(g, d, scale, causal, 0, L);
    bwd_dkdv_rows(g, d, scale, causal, 0, L);
  });
  return 0;
}

// Decode shapes: q, o [B, Nq, H, d]; k, v [B, Nk, H, d]; lse [B, H, Nq]. Plain definition
// with the decode visibility rule. Returns 0, or -1 on bad sizes.
int oracle_fwd_decode(const double* q, const double* k, const double* v, double* o,
                      double* lse, long B, long Nq, long Nk, long H, long d, double scale,
                      int causal, int nthreads) {
  if (B < 1 || Nq < 1 || Nk < 1 || H < 1 || d < 1) return -1;
  parallel_for(B * H * Nq, nthreads, [&](long it) {
    const long idx = it / Nq, i = it % Nq;
    const DecodeSlice s = decode_slice(q, k, v, Nq, Nk, H, d, idx);
    double* oi = o + ((idx / H) * Nq * H + i * H + idx % H) * d;
    double m, l;
    decode_partial(s, d, scale, causal, i, 0, Nk, oi, m, l);
    lse[idx * Nq + i] = l > 0.0 ? m + std::log(l) : kNegInf;
  });
  return 0;
}

// Split form: the keys cut into nsplit contiguous ranges of ceil(Nk / nsplit) (trailing
// ranges may be empty), each range's (m, l, O) from the definition, combined by the
// block-merge rule. Same layouts as oracle_fwd_decode.
int oracle_fwd_decode_split(const double* q, const double* k, const double* v, double* o,
                            double* lse, long B, long Nq, long Nk, long H, long d, double scale,
                            int causal, long nsplit, int nthreads) {
  if (B < 1 || Nq < 1 || Nk < 1 || H < 1 || d < 1 || nsplit < 1) return -1;
  const long span = (Nk + nsplit - 1) / nsplit;
  parallel_for(B * H * Nq, nthreads, [&](long it) {
    const long idx = it / Nq, i = it % Nq;
    const DecodeSlice s = decode_slice(q, k, v, Nq, Nk, H, d, idx);
    std::vector<double> ms(nsplit), ls(nsplit), os(nsplit * d);
    for (long t = 0; t < nsplit; ++t) {
      const long j0 = std::min(t * span, Nk), j1 = std::min(j0 + span, Nk);
      decode_partial(s, d, scale, causal, i, j0, j1, &os[t * d], ms[t], ls[t]);
    }
    double* oi = o + ((idx / H) * Nq * H + i * H + idx % H) * d;
    merge_partials(nsplit, d, ms.data(), ls.data(), os.data(), oi, lse[idx * Nq + i]);
  });
  return 0;
}

// Merge of partial results given as (O_s, LSE_s): part s holds the normalised output and
// the log-sum-exp of the same rows over its own disjoint set of keys (for instance one K/V
// shard of a ring of devices). In the block-merge rule's terms a part has m_s = LSE_s and
// l_s = 1 (l_s = 0 for a part that saw no key, LSE_s = -inf), so the merge is exactly
// merge_partials. Layout: o_parts [nparts][rows][d], lse_parts [nparts][rows]; o [rows][d],
// lse [rows]. Returns 0, or -1 on bad sizes.
int oracle_merge(const double* o_parts, const double* lse_parts, double* o, double* lse,
                 long nparts, long rows, long d, int nthreads) {
  if (nparts < 1 || rows < 0 || d < 1) return -1;
  parallel_for(rows, nthreads, [&](long r) {
    std::vector<double> ms(nparts), ls(nparts), os(nparts * d);
    for (long t = 0; t < nparts; ++t) {
      ms[t] = lse_parts[t * rows + r];
      ls[t] = ms[t] == kNegInf ? 0.0 : 1.0;
      for (long c = 0; c < d; ++c) os[t * d + c] = o_parts[(t * rows + r) * d + c];
    }
    merge_partials(nparts, d, ms.data(), ls.data(), os.data(), o + r * d, lse[r]);
  });
  return 0;
}

// Spot checks of problems too large for the whole-tensor functions, one (batch, head) slice
// at a time: q_rows, dout_rows [R, d] are R query rows at positions pos[r] of a slice whose
// keys and values k, v are [N, d]. For each row, by the plain definition: O, LSE and, when
// dout_rows is given, dQ = scale * sum_j P_ij (dP_ij - D_i) k_j with D_i = <dO_i, O_i>.
int oracle_rows(const double* q_rows, const double* k, const double* v, const double* dout_rows,
                const long* pos, double* o, double* lse, double* dq, long R, long N, long d,
                double scale, int causal, int nthreads) {
  if (R < 0 || N < 0 || d <= 0) return -1;
  for (long r = 0; r < R; ++r)
    if (pos[r] < 0 || pos[r] >= N) return -2;
  parallel_for(R, nthreads, [&](long r) {
    const long je = visible_end(pos[r], N, causal);
    const double* qr = q_rows + r * d;
    double* orow = o + r * d;
    for (long c = 0; c < d; ++c) orow[c] = 0.0;
    if (dout_rows != nullptr)
      for (long c = 0; c < d; ++c) dq[r * d + c] = 0.0;
    if (je == 0) {
      lse[r] = kNegInf;
      return;
    }
    std::vector<double> sc(je);
    double m = kNegInf;
    for (long j = 0; j < je; ++j) {
      sc[j] = scale * dot(qr, k + j * d, d);
      m = std::max(m, sc[j]);
    }
    double l = 0.0;
    for (long j = 0; j < je; ++j) {
      const double p = std::exp(sc[j] - m);
      l += p;
      for (long c = 0; c < d; ++c) orow[c] += p * v[j * d + c];
    }
    for (long c = 0; c < d; ++c) orow[c] /= l;
    lse[r] = m + std::log(l);
    if (dout_rows == nullptr) return;
    const double* dor = dout_rows + r * d;
    const double Di = dot(dor, orow, d);
    double* dqr = dq + r * d;
    for (long j = 0; j < je; ++j) {
      const double P = std::exp(sc[j] - lse[r]);
      const double dS = P * (dot(dor, v + j * d, d) - Di);
      for (long c = 0; c < d; ++c) dqr[c] += dS * k[j * d + c];
    }
    for (long c = 0; c < d; ++c) dqr[c] *= scale;
  });
  return 0;
}

// Under the causal mask, key j is seen only by query rows i >= j, so the gradients of the
// last R keys of a slice need only its last R rows. Given those rows (q_tail, dout_tail
// [R, d], rows N - R .. N - 1) with their O and LSE (o_tail [R, d], lse_tail [R], e.g. from
// oracle_rows) and the slice's k, v [N, d]: dV_j = sum_{i >= j} P_ij dO_i and
// dK_j = scale * sum_{i >= j} dS_ij q_i for j = N - R .. N - 1, into dk, dv [R, d].
int oracle_tail_keys(const double* q_tail, const double* k, const double* v,
                     const double* dout_tail, const double* o_tail, const double* lse_tail,
                     double* dk, double* dv, long R, long N, long d, double scale, int nthreads) {
  if (R < 0 || R > N || d <= 0) return -1;
  const long t0 = N - R;
  parallel_for(R, nthreads, [&](long c) {
    const long j = t0 + c;
    const double* kj = k + j * d;
    const double* vj = v + j * d;
    double* dkj = dk + c * d;
    double* dvj = dv + c * d;
    for (long e = 0; e < d; ++e) dkj[e] = dvj[e] = 0.0;
    for (long r = c; r < R; ++r) {  // rows i = t0 + r >= j
      const double* qi = q_tail + r * d;
      const double* doi = dout_tail + r * d;
      const double Di = dot(doi, o_tail + r * d, d);
      const double P = std::exp(scale * dot(qi, kj, d) - lse_tail[r]);
      const double dS = P * (dot(doi, vj, d) - Di);
      for (long e = 0; e < d; ++e) {
        dvj[e] += P * doi[e];
        dkj[e] += dS * qi[e];
      }
    }
    for (long e = 0; e < d; ++e) dkj[e] *= scale;
  });
  return 0;
}

}  // extern "C"
