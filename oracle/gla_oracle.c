/*
 * fp64 token-by-token oracle for the gated linear attention prefill forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header or constant with the HIP
 * library.
 *
 * What it computes (plain definition, no chunking, no reordering):
 *
 *   for every (b, h) independently
 *     S <- h0[b,h]  (K x V, or 0 when h0 is NULL)
 *     for t = 0 .. T-1
 *       S[d, :] <- exp(g[t, d]) * S[d, :]      for every key dim d
 *       S       <- S + k_t^T v_t                 (rank-1 write)
 *       o[t, :] <- scale * (q_t . S)             (uses S after token t)
 *     h_final[b,h] <- S
 *
 * Sources: the state update "h <- h*g + k^T v" with a D x D state
 * (blog "Linear Attention 在 GPU 上到底慢在哪", section 学长的反馈); the
 * update-then-output recurrence in the pseudocode of "线性注意力GPU算子库的定义
 * 与技术解析" (section 四, 工作原理); the high-precision token-by-token
 * reference asked for in "面向长序列大模型的线性注意力算子性能评测方法与优化实践"
 * (section 六.1).  The gate is a log-decay applied on the key (row) axis:
 * decay = exp(g).
 *
 * Optional: `states` receives the state *before* token n*record_every, for
 * n = 0 .. ceil(T/record_every)-1, i.e. the chunk-start states of a chunked
 * evaluation with chunk = record_every.  That is still the plain recurrence,
 * only observed at fixed token indices.
 *
 * Layouts (row-major, contiguous): q,k,g [B,H,T,K]; v,o [B,H,T,V];
 * h0,h_final [B,H,K,V]; states [B,H,N,K,V].  All doubles.
 * Parallelised with OpenMP over (b, h, block of 16 value columns): the value
 * columns of S are independent because the decay acts on rows only.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_VBLK 16

int gla_oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

int gla_oracle_f64(const double *q, const double *k, const double *v,
                   const double *g, const double *h0, double *o,
                   double *h_final, double *states, long B, long H, long T,
                   long K, long V, double scale, long record_every,
                   int threads) {
    if (B < 0 || H < 0 || T < 0 || K <= 0 || V <= 0) return -1;
    if (states && record_every <= 0) return -1;
    const long BH = B * H;
    const long nvb = (V + ORACLE_VBLK - 1) / ORACLE_VBLK;
    const long nrec = (states && T > 0) ? (T + record_every - 1) / record_every : 0;
    int status = 0;
#ifdef _OPENMP
    if (threads > 0) omp_set_num_threads(threads);
#else
    (void)threads;
#endif

#pragma omp parallel for schedule(dynamic, 1)
    for (long job = 0; job < BH * nvb; ++job) {
        const long bh = job / nvb;
        const long vb = job % nvb;
        const long c0 = vb * ORACLE_VBLK;
        const long nc = (V - c0) < ORACLE_VBLK ? (V - c0) : ORACLE_VBLK;
        double *S = (double *)malloc(sizeof(double) * (size_t)(K * nc));
        double *decay = (double *)malloc(sizeof(double) * (size_t)K);
        if (!S || !decay) {
            free(S);
            free(decay);
#pragma omp atomic write
            status = -2;
            continue;
        }
        for (long d = 0; d < K; ++d)
            for (long c = 0; c < nc; ++c)
                S[d * nc + c] = h0 ? h0[(bh * K + d) * V + c0 + c] : 0.0;

        for (long t = 0; t < T; ++t) {
            const double *qt = q + (bh * T + t) * K;
            const double *kt = k + (bh * T + t) * K;
            const double *gt = g + (bh * T + t) * K;
            const double *vt = v + (bh * T + t) * V + c0;
            if (states && t % record_every == 0) {
                double *dst = states + ((bh * nrec + t / record_every) * K) * V;
                for (long d = 0; d < K; ++d)
                    for (long c = 0; c < nc; ++c) dst[d * V + c0 + c] = S[d * nc + c];
            }
            for (long d = 0; d < K; ++d) decay[d] = exp(gt[d]);
            /* S[d,:] = exp(g[t,d]) * S[d,:] + k[t,d] * v[t,:] */
            for (long d = 0; d < K; ++d) {
                const double a = decay[d], kd = kt[d];
                double *row = S + d * nc;
                for (long c = 0; c < nc; ++c) row[c] = a * row[c] + kd * vt[c];
            }
            /* o[t,:] = scale * sum_d q[t,d] * S[d,:] */
            double *ot = o + (bh * T + t) * V + c0;
            for (long c = 0; c < nc; ++c) ot[c] = 0.0;
            for (long d = 0; d < K; ++d) {
                const double qd = qt[d];
                const double *row = S + d * nc;
                for (long c = 0; c < nc; ++c) ot[c] += qd * row[c];
            }
            for (long c = 0; c < nc; ++c) ot[c] *= scale;
        }
        if (h_final)
            for (long d = 0; d < K; ++d)
                for (long c = 0; c < nc; ++c)
                    h_final[(bh * K + d) * V + c0 + c] = S[d * nc + c];
        free(S);
        free(decay);
    }
    return status;
}

/*
 * fp64 backward of the same recurrence: reverse-mode chain rule, token by
 * token.  TEST INFRASTRUCTURE ONLY, like the forward above.
 *
 * Given do = dL/do [B,H,T,V] and dh_final = dL/dh_final [B,H,K,V] (NULL:
 * zero), for every (b, h):
 *
 *   R <- dh_final                          (dL/dS_t from tokens after t)
 *   for t = T-1 .. 0
 *     R        <- R + scale * q_t^T do_t   (now the full dL/dS_t)
 *     dq[t, d] <- scale * sum_v S_t[d, v] do_t[v]
 *     dk[t, d] <- sum_v R[d, v] v_t[v]
 *     dv[t, v] <- sum_d k_t[d] R[d, v]
 *     dg[t, d] <- exp(g[t, d]) * sum_v R[d, v] S_{t-1}[d, v]
 *     R[d, :]  <- exp(g[t, d]) * R[d, :]   (dL/dS_{t-1})
 *   dh0 <- R
 *
 * with S_t the forward state after token t and S_{-1} = h0 (or 0).  The
 * forward states are kept at every `ckpt`-th token and recomputed block by
 * block with the same forward steps as gla_oracle_f64 (a memory bound, not a
 * change of arithmetic).  Layouts as above; do [B,H,T,V], dq, dk, dg
 * [B,H,T,K], dv [B,H,T,V], dh0 [B,H,K,V] (NULL: not written).  Parallel over
 * (b, h).
 */
int gla_oracle_bwd_f64(const double *q, const double *k, const double *v,
                       const double *g, const double *h0, const double *dout,
                       const double *dh_final, double *dq, double *dk,
                       double *dv, double *dg, double *dh0, long B, long H,
                       long T, long K, long V, double scale, long ckpt,
                       int threads) {
    if (B < 0 || H < 0 || T < 0 || K <= 0 || V <= 0 || ckpt <= 0) return -1;
    const long BH = B * H;
    const long KV = K * V;
    const long nblk = T > 0 ? (T + ckpt - 1) / ckpt : 0;
    int status = 0;
#ifdef _OPENMP
    if (threads > 0) omp_set_num_threads(threads);
#else
    (void)threads;
#endif

#pragma omp parallel for schedule(dynamic, 1)
    for (long bh = 0; bh < BH; ++bh) {
        /* cp: state before each block's first token; blk: states after each
           token of one block; R: the running gradient */
        double *cp = (double *)malloc(sizeof(double) * (size_t)((nblk > 0 ? nblk : 1) * KV));
        double *blk = (double *)malloc(sizeof(double) * (size_t)(ckpt * KV));
        double *R = (double *)malloc(sizeof(double) * (size_t)KV);
        double *S = (double *)malloc(sizeof(double) * (size_t)KV);
        if (!cp || !blk || !R || !S) {
            free(cp); free(blk); free(R); free(S);
#pragma omp atomic write
            status = -2;
            continue;
        }
        for (long i = 0; i < KV; ++i) S[i] = h0 ? h0[bh * KV + i] : 0.0;
        /* forward, keeping the state before every block */
        for (long t = 0; t < T; ++t) {
            if (t % ckpt == 0) memcpy(cp + (t / ckpt) * KV, S, sizeof(double) * (size_t)KV);
            const double *kt = k + (bh * T + t) * K;
            const double *gt = g + (bh * T + t) * K;
            const double *vt = v + (bh * T + t) * V;
            for (long d = 0; d < K; ++d) {
                const double a = exp(gt[d]), kd = kt[d];
                for (long c = 0; c < V; ++c) S[d * V + c] = a * S[d * V + c] + kd * vt[c];
            }
        }
        for (long i = 0; i < KV; ++i) R[i] = dh_final ? dh_final[bh * KV + i] : 0.0;

        for (long b = nblk - 1; b >= 0; --b) {
            const long t0 = b * ckpt;
            const long t1 = (t0 + ckpt < T) ? t0 + ckpt : T;
            /* recompute the block's states: blk[t - t0] = S_t */
            memcpy(S, cp + b * KV, sizeof(double) * (size_t)KV);
            for (long t = t0; t < t1; ++t) {
                const double *kt = k + (bh * T + t) * K;
                const double *gt = g + (bh * T + t) * K;
                const double *vt = v + (bh * T + t) * V;
                for (long d = 0; d < K; ++d) {
                    const double a = exp(gt[d]), kd = kt[d];
                    for (long c = 0; c < V; ++c) S[d * V + c] = a * S[d * V + c] + kd * vt[c];
                }
                memcpy(blk + (t - t0) * KV, S, sizeof(double) * (size_t)KV);
            }
            for (long t = t1 - 1; t >= t0; --t) {
                const double *St = blk + (t - t0) * KV;
                const double *Sp = t > t0 ? blk + (t - 1 - t0) * KV : cp + b * KV;
                const double *qt = q + (bh * T + t) * K;
                const double *kt = k + (bh * T + t) * K;
                const double *gt = g + (bh * T + t) * K;
                const double *vt = v + (bh * T + t) * V;
                const double *dot = dout + (bh * T + t) * V;
                for (long d = 0; d < K; ++d)
                    for (long c = 0; c < V; ++c) R[d * V + c] += scale * qt[d] * dot[c];
                for (long d = 0; d < K; ++d) {
                    double sq = 0.0, sk = 0.0, sg = 0.0;
                    for (long c = 0; c < V; ++c) {
                        sq += St[d * V + c] * dot[c];
                        sk += R[d * V + c] * vt[c];
                        sg += R[d * V + c] * Sp[d * V + c];
                    }
                    const double a = exp(gt[d]);
                    dq[(bh * T + t) * K + d] = scale * sq;
                    dk[(bh * T + t) * K + d] = sk;
                    dg[(bh * T + t) * K + d] = a * sg;
                }
                for (long c = 0; c < V; ++c) {
                    double s = 0.0;
                    for (long d = 0; d < K; ++d) s += kt[d] * R[d * V + c];
                    dv[(bh * T + t) * V + c] = s;
                }
                for (long d = 0; d < K; ++d) {
                    const double a = exp(gt[d]);
                    for (long c = 0; c < V; ++c) R[d * V + c] *= a;
                }
            }
        }
        if (dh0)
            for (long i = 0; i < KV; ++i) dh0[bh * KV + i] = R[i];
        free(cp); free(blk); free(R); free(S);
    }
    return status;
}

/*
 * fp64 token-by-token oracle for the gated delta rule (Gated DeltaNet
 * forward).  TEST INFRASTRUCTURE ONLY, like the functions above.
 *
 * The evaluation page names the Gated Delta Network class as gating plus an
 * incremental ("delta") update of the recurrent state ("面向长序列大模型的线性
 * 注意力算子性能评测方法与优化实践", sections 一 and 三.3) and gives no formula;
 * the reading taken is the published gated delta rule: per (b, h),
 *
 *   S <- h0 (or 0)                                   K x V
 *   for t = 0 .. T-1
 *     S <- exp(g[t]) * S                             (scalar gate per token)
 *     S <- S + beta[t] * k_t^T (v_t - k_t S)         (delta update)
 *     o[t, :] <- scale * q_t S
 *   h_final <- S
 *
 * Layouts: q, k [B,H,T,K]; v, o [B,H,T,V]; g, beta [B,H,T]; h0, h_final
 * [B,H,K,V].  Value columns of S are independent (the update of column c
 * only reads column c), so the work is split over (b, h, block of 16
 * columns) as in gla_oracle_f64.
 */
int gdn_oracle_f64(const double *q, const double *k, const double *v,
                   const double *g, const double *beta, const double *h0,
                   double *o, double *h_final, long B, long H, long T, long K,
                   long V, double scale, int threads) {
    if (B < 0 || H < 0 || T < 0 || K <= 0 || V <= 0) return -1;
    const long BH = B * H;
    const long nvb = (V + ORACLE_VBLK - 1) / ORACLE_VBLK;
    int status = 0;
#ifdef _OPENMP
    if (threads > 0) omp_set_num_threads(threads);
#else
    (void)threads;
#endif

#pragma omp parallel for schedule(dynamic, 1)
    for (long job = 0; job < BH * nvb; ++job) {
        const long bh = job / nvb;
        const long c0 = (job % nvb) * ORACLE_VBLK;
        const long nc = (V - c0) < ORACLE_VBLK ? (V - c0) : ORACLE_VBLK;
        double *S = (double *)malloc(sizeof(double) * (size_t)(K * nc));
        if (!S) {
#pragma omp atomic write
            status = -2;
            continue;
        }
        for (long d = 0; d < K; ++d)
            for (long c = 0; c < nc; ++c) S[d * nc + c] = h0 ? h0[(bh * K + d) * V + c0 + c] : 0.0;
        for (long t = 0; t < T; ++t) {
            const double *qt = q + (bh * T + t) * K;
            const double *kt = k + (bh * T + t) * K;
            const double *vt = v + (bh * T + t) * V + c0;
            const double a = exp(g[bh * T + t]), b = beta[bh * T + t];
            for (long i = 0; i < K * nc; ++i) S[i] *= a;
            for (long c = 0; c < nc; ++c) {
                double ks = 0.0;   /* (k_t S)[c] */
                for (long d = 0; d < K; ++d) ks += kt[d] * S[d * nc + c];
                const double r = b * (vt[c] - ks);
                for (long d = 0; d < K; ++d) S[d * nc + c] += kt[d] * r;
            }
            double *ot = o + (bh * T + t) * V + c0;
            for (long c = 0; c < nc; ++c) {
                double s = 0.0;
                for (long d = 0; d < K; ++d) s += qt[d] * S[d * nc + c];
                ot[c] = scale * s;
            }
        }
        if (h_final)
            for (long d = 0; d < K; ++d)
                for (long c = 0; c < nc; ++c) h_final[(bh * K + d) * V + c0 + c] = S[d * nc + c];
        free(S);
    }
    return status;
}
