/*
 * gla_scalar.h — the scalar-gate variant of the prefill forward: one
 * log-decay per token and head, shared by every key dim.
 *
 *     S_t = exp(g_t) S_{t-1} + k_t^T v_t        S_{-1} = h0 (or 0)
 *     o_t = scale * q_t S_t                     h_final = S_{T-1}
 *
 * The blog "Linear Attention 在 GPU 上到底慢在哪" (section 正确的 baseline 和
 * 下一步) ranks Mamba-2's SSD / semiseparable block second after GLA as a
 * target, and names Lightning Attention among the kernels its baselines
 * measure; both decay the whole state by one factor per token and head.
 * This is the recurrence of gla.h with g_t broadcast
 * over the key dims, so every result equals gla_fwd's with g expanded to
 * [B,H,T,K], and the chunk form is the same reordering: intra-chunk scores
 * become (q_i . k_j) exp(G_i - G_j) for j <= i, with G the chunk-local
 * prefix sum of g.
 *
 * Layout: as gla.h, except g:
 *     q, k [B, H, T, K]    v, o [B, H, T, V]    g [B, H, T] fp32
 *     h0, h_final [B, H, K, V] fp32
 * gla_fwd_scalar: q, k, v, o bfloat16; gla_fwd_scalar_f32: float32.
 * Supported shapes, chunk sizes, ownership (the same cached workspace),
 * nullability, aliasing, the g <= 0 precondition, determinism and error
 * codes are those of gla_fwd / gla_fwd_f32 in gla.h; g's extent for the
 * aliasing checks is B*H*T floats.
 */
#ifndef GLA_SCALAR_H
#define GLA_SCALAR_H

#include "gla.h"

#ifdef __cplusplus
extern "C" {
#endif

int gla_fwd_scalar(const gla_bf16 *q, const gla_bf16 *k, const gla_bf16 *v,
                   const float *g, const float *h0, gla_bf16 *o, float *h_final,
                   int B, int H, int T, int K, int V, int chunk, float scale,
                   void *stream);

int gla_fwd_scalar_f32(const float *q, const float *k, const float *v,
                       const float *g, const float *h0, float *o, float *h_final,
                       int B, int H, int T, int K, int V, int chunk, float scale,
                       void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GLA_SCALAR_H */
