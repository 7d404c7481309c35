/*
 * Plain fp64 CPU oracle for Gated Linear Attention (GLA).  TEST INFRASTRUCTURE:
 * only the tests, the smoke check and the benchmark's CPU-baseline leg load
 * this; the product path never does.  It shares no code with the HIP library.
 *
 * What it computes (page "Gated Linear Attention (GLA): Mathematical
 * Foundations ...", section "The Gated Recurrent Update"): for every
 * independent unit (sequence n, head h) and every token t of that sequence,
 *
 *     S_t = diag(alpha_t) S_{t-1} + k_t^T v_t,      alpha_t = exp(g_t),
 *     o_t = q_t S_t                                  (uses the updated state),
 *
 * with S_0 the caller's initial state (zeros when absent).  The state is a
 * d_k x d_v matrix; g_t = log(alpha_t) is one value per key channel.  Nothing
 * is chunked, reordered or fused: one token at a time, in sequence order.
 *
 * The single-token decode step of the same page (and of the "O(1) Inference
 * Memory" section of the FlashLinearAttention page) is one iteration of the
 * same loop, so it is this function with one token per sequence.
 *
 * Inputs are float32 arrays holding the exact values the device read (every
 * bf16 and fp32 value is exactly representable in float32); all arithmetic is
 * fp64.  Layout, row-major, last index fastest:
 *   q, k, g : [B, H, T, dk]      v : [B, H, T, dv]      o : [B, H, T, dv] (fp64)
 *   s0, s_final : [num_units_n, H, dk, dv] fp64 (either may be NULL)
 * Fixed length: cu_seqlens == NULL, sequences n = 0..B-1 each of length T.
 * Packed variable length: cu_seqlens[0..num_seqs] (non-decreasing, first 0,
 * last T) and B == 1; sequence n owns tokens [cu_seqlens[n], cu_seqlens[n+1]).
 *
 * Returns 0 on success, a negative value for invalid arguments.  *threads_used
 * (if non-NULL) receives the number of OpenMP threads of the parallel region.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int gla_oracle_recurrence(const float* q, const float* k, const float* v,
                          const float* g, const double* s0, double* o,
                          double* s_final, const int32_t* cu_seqlens,
                          int num_seqs, int B, int H, int T, int dk, int dv,
                          int nthreads, int* threads_used) {
  if (!q || !k || !v || !g || !o) return -1;
  if (B <= 0 || H <= 0 || T < 0 || dk <= 0 || dv <= 0) return -2;
  int nseq = B;
  if (cu_seqlens) {
    if (B != 1 || num_seqs <= 0) return -3;
    if (cu_seqlens[0] != 0 || cu_seqlens[num_seqs] != T) return -4;
    for (int n = 0; n < num_seqs; ++n)
      if (cu_seqlens[n + 1] < cu_seqlens[n]) return -5;
    nseq = num_seqs;
  }
  const long units = (long)nseq * H;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
  int used = 1;
  int failed = 0;
#pragma omp parallel
  {
#ifdef _OPENMP
#pragma omp single
    used = omp_get_num_threads();
#endif
    double* S = (double*)malloc(sizeof(double) * (size_t)dk * dv);
    double* a = (double*)malloc(sizeof(double) * (size_t)dk);
    if (!S || !a) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (long u = 0; u < units; ++u) {
      if (!S || !a) continue;
      const long n = u / H, h = u % H;
      long b, t0, t1;
      if (cu_seqlens) {
        b = 0;
        t0 = cu_seqlens[n];
        t1 = cu_seqlens[n + 1];
      } else {
        b = n;
        t0 = 0;
        t1 = T;
      }
      const size_t row_k = (size_t)(b * H + h) * T;  /* first row of (b, h) */
      if (s0)
        memcpy(S, s0 + (size_t)u * dk * dv, sizeof(double) * (size_t)dk * dv);
      else
        memset(S, 0, sizeof(double) * (size_t)dk * dv);
      for (long t = t0; t < t1; ++t) {
        const float* qt = q + (row_k + t) * dk;
        const float* kt = k + (row_k + t) * dk;
        const float* gt = g + (row_k + t) * dk;
        const float* vt = v + (row_k + t) * dv;
        double* ot = o + (row_k + t) * dv;
        for (int c = 0; c < dk; ++c) a[c] = exp((double)gt[c]);
        /* S_t = diag(alpha_t) S_{t-1} + k_t^T v_t */
        for (int c = 0; c < dk; ++c) {
          double* Sc = S + (size_t)c * dv;
          const double kc = (double)kt[c];
          for (int j = 0; j < dv; ++j) Sc[j] = a[c] * Sc[j] + kc * (double)vt[j];
        }
        /* o_t = q_t S_t */
        for (int j = 0; j < dv; ++j) ot[j] = 0.0;
        for (int c = 0; c < dk; ++c) {
          const double qc = (double)qt[c];
          const double* Sc = S + (size_t)c * dv;
          for (int j = 0; j < dv; ++j) ot[j] += qc * Sc[j];
        }
      }
      if (s_final)
        memcpy(s_final + (size_t)u * dk * dv, S, sizeof(double) * (size_t)dk * dv);
    }
    free(S);
    free(a);
  }
  if (threads_used) *threads_used = used;
  return failed ? -6 : 0;
}

/*
 * Gated DeltaNet (GDN), the second recurrence of the pages (page "Qwen Team
 * Releases FlashQLA for High-Performance Linear Attention", sections on the
 * GDN state update and "Core Technical Principles"): a forget gate alpha_t in
 * (0, 1] and an update gate beta_t in (0, 1), one value of each per token and
 * head, acting on the transition alpha_t (I - beta_t k_t^T k_t):
 *
 *     S_t = alpha_t (I - beta_t k_t^T k_t) S_{t-1} + beta_t k_t^T v_t,
 *     o_t = q_t S_t,                     alpha_t = exp(g_t),
 *
 * with k_t a row vector (1 x dk), S a dk x dv matrix and S_0 the caller's
 * initial state (zeros when absent).  The product (k^T k) S is evaluated as
 * k^T (k S), the same matrix.  One token at a time, fp64, OpenMP only across
 * independent (sequence, head) units.
 *   q, k : [B, H, T, dk]   v : [B, H, T, dv]   g, beta : [B, H, T]
 *   o : [B, H, T, dv] fp64; s0, s_final : [nseq, H, dk, dv] fp64 (NULL allowed)
 * Varlen exactly as gla_oracle_recurrence.  Returns 0 or a negative code.
 */
int gdn_oracle_recurrence(const float* q, const float* k, const float* v,
                          const float* g, const float* beta, const double* s0,
                          double* o, double* s_final, const int32_t* cu_seqlens,
                          int num_seqs, int B, int H, int T, int dk, int dv,
                          int nthreads, int* threads_used) {
  if (!q || !k || !v || !g || !beta || !o) return -1;
  if (B <= 0 || H <= 0 || T < 0 || dk <= 0 || dv <= 0) return -2;
  int nseq = B;
  if (cu_seqlens) {
    if (B != 1 || num_seqs <= 0) return -3;
    if (cu_seqlens[0] != 0 || cu_seqlens[num_seqs] != T) return -4;
    for (int n = 0; n < num_seqs; ++n)
      if (cu_seqlens[n + 1] < cu_seqlens[n]) return -5;
    nseq = num_seqs;
  }
  const long units = (long)nseq * H;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
  int used = 1;
  int failed = 0;
#pragma omp parallel
  {
#ifdef _OPENMP
#pragma omp single
    used = omp_get_num_threads();
#endif
    double* S = (double*)malloc(sizeof(double) * (size_t)dk * dv);
    double* kS = (double*)malloc(sizeof(double) * (size_t)dv);
    if (!S || !kS) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (long u = 0; u < units; ++u) {
      if (!S || !kS) continue;
      const long n = u / H, h = u % H;
      long b, t0, t1;
      if (cu_seqlens) {
        b = 0;
        t0 = cu_seqlens[n];
        t1 = cu_seqlens[n + 1];
      } else {
        b = n;
        t0 = 0;
        t1 = T;
      }
      const size_t row = (size_t)(b * H + h) * T;  /* first row of (b, h) */
      if (s0)
        memcpy(S, s0 + (size_t)u * dk * dv, sizeof(double) * (size_t)dk * dv);
      else
        memset(S, 0, sizeof(double) * (size_t)dk * dv);
      for (long t = t0; t < t1; ++t) {
        const float* qt = q + (row + t) * dk;
        const float* kt = k + (row + t) * dk;
        const float* vt = v + (row + t) * dv;
        double* ot = o + (row + t) * dv;
        const double a = exp((double)g[row + t]);
        const double bt = (double)beta[row + t];
        /* kS = k_t S_{t-1} */
        for (int j = 0; j < dv; ++j) kS[j] = 0.0;
        for (int c = 0; c < dk; ++c) {
          const double kc = (double)kt[c];
          const double* Sc = S + (size_t)c * dv;
          for (int j = 0; j < dv; ++j) kS[j] += kc * Sc[j];
        }
        /* S_t = a (S_{t-1} - b k^T kS) + b k^T v_t */
        for (int c = 0; c < dk; ++c) {
          double* Sc = S + (size_t)c * dv;
          const double kc = (double)kt[c];
          for (int j = 0; j < dv; ++j)
            Sc[j] = a * (Sc[j] - bt * kc * kS[j]) + bt * kc * (double)vt[j];
        }
        /* o_t = q_t S_t */
        for (int j = 0; j < dv; ++j) ot[j] = 0.0;
        for (int c = 0; c < dk; ++c) {
          const double qc = (double)qt[c];
          const double* Sc = S + (size_t)c * dv;
          for (int j = 0; j < dv; ++j) ot[j] += qc * Sc[j];
        }
      }
      if (s_final)
        memcpy(s_final + (size_t)u * dk * dv, S, sizeof(double) * (size_t)dk * dv);
    }
    free(S);
    free(kS);
  }
  if (threads_used) *threads_used = used;
  return failed ? -6 : 0;
}
