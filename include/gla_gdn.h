/*
 * gla_gdn.h — forward of the gated delta rule (the Gated DeltaNet class of
 * linear attention), causal, in chunk form on gfx950.
 *
 * Operation (per batch row b and head h; one gate g_t and one write strength
 * beta_t per token and head):
 *
 *     S_t = exp(g_t) (I - beta_t k_t^T k_t) S_{t-1} + beta_t k_t^T v_t
 *     o_t = scale * q_t S_t            S_{-1} = h0 (or 0), h_final = S_{T-1}
 *
 * The evaluation page "面向长序列大模型的线性注意力算子性能评测方法与优化实践"
 * (sections 一 and 三.3) names the Gated Delta Network class as linear
 * attention with gating and an incremental ("delta") update of the recurrent
 * state, without a formula; this is the published gated delta rule.  The
 * chunk form solves one unit lower-triangular system per chunk of 64 tokens;
 * every decay factor it forms is at most 1.
 *
 * Layout (dense, row-major, device memory, 16-byte aligned):
 *     q, k [B, H, T, K] bf16     v, o [B, H, T, V] bf16
 *     g, beta [B, H, T] fp32     h0, h_final [B, H, K, V] fp32
 * Supported: K == V in {64, 128}; T >= 0; chunk 0 (default) or 64.
 * Preconditions (not checked): g finite and <= 0, 0 <= beta <= 1; rows of k
 * L2-normalised, as the delta rule assumes (the bf16 error bound of the
 * matrix products relies on it).
 *
 * One work-group per (batch, head) walks the sequence: this build has no
 * sequence parallelism for the gated delta rule, so B*H should fill the GPU
 * (256 work-groups, one per CU) for full speed.
 *
 * Ownership, nullability (h0 NULL = zero state, h_final NULL = not written),
 * aliasing (o, h_final must not overlap the inputs or each other), streams,
 * determinism and error codes: as gla_fwd in gla.h.  No workspace is used.
 */
#ifndef GLA_GDN_H
#define GLA_GDN_H

#include "gla.h"

#ifdef __cplusplus
extern "C" {
#endif

int gla_gdn_fwd(const gla_bf16 *q, const gla_bf16 *k, const gla_bf16 *v,
            const float *g, const float *beta, const float *h0, gla_bf16 *o,
            float *h_final, int B, int H, int T, int K, int V, int chunk,
            float scale, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GLA_GDN_H */
