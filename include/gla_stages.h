/*
 * gla_stages.h — per-stage entry points of libgla.so, for testing each step
 * of the chunked path on its own.  They run the same device code as gla_fwd
 * (bf16 q/k/v, fp32 g), one stage at a time, and write fp32 results.  The
 * stages are the ones the blog "Linear Attention 在 GPU 上到底慢在哪"
 * profiles (section 实验结果, Kernel Profiling): gate cumsum, intra-chunk
 * scores, inter-chunk state recurrence and output.
 *
 * Conventions as in gla.h (row-major device buffers, 16-byte aligned base
 * pointers, K == V in {64, 128}, chunk 0 = default, asynchronous on
 * `stream`, negative GLA_ERR_* on bad arguments with nothing enqueued).
 * N = ceil(T / chunk) chunks per (batch, head).
 */
#ifndef GLA_STAGES_H
#define GLA_STAGES_H

#include "gla.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Chunk-local inclusive cumsum of the log-gates (restarting at each chunk
 * start): gc [B,H,T,K] with gc[n*C+i] = sum_{j<=i} g[n*C+j], and gamma
 * [B,H,N,K] = gc at each chunk's last valid row.  Natural-log units.
 */
int gla_stage_cumsum(const float *g, float *gc, float *gamma,
                     int B, int H, int T, int K, int chunk, void *stream);

/*
 * Intra-chunk decayed causal scores, scaled:
 *   A[b,h,n,i,j] = scale * sum_d q[nC+i,d] k[nC+j,d] exp(Gc[nC+i,d] - Gc[nC+j,d])
 * for j <= i, 0 above the diagonal; [B,H,N,C,C] fp32 (the accumulator values
 * before the bf16 rounding the fused path applies).  Rows and columns past T
 * in the last chunk hold values of zero-padded tokens.
 */
int gla_stage_intra(const gla_bf16 *q, const gla_bf16 *k, const float *g,
                    float *A, int B, int H, int T, int K, int chunk,
                    float scale, void *stream);

/*
 * The full forward (same arguments and outputs as gla_fwd) that also writes
 * the inter-chunk recurrence's chunk-start states: states[b,h,n] = S before
 * token n*C, [B,H,N,K,V] fp32.
 */
int gla_stage_states(const gla_bf16 *q, const gla_bf16 *k, const gla_bf16 *v,
                     const float *g, const float *h0, gla_bf16 *o,
                     float *h_final, float *states, int B, int H, int T, int K,
                     int V, int chunk, float scale, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GLA_STAGES_H */
