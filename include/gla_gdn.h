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
 * Two evaluation forms, same results up to rounding:
 *   one launch  — one work-group per (batch, head, block of value columns)
 *                 forms each chunk's system and walks the state through the
 *                 chunks; used when B*H fills the GPU;
 *   two launches — a chunk-parallel prep forms, for every chunk at once, the
 *                 chunk-local products (T, W, U~ and the output terms that do
 *                 not involve the state) into a per-chunk record, then a walk
 *                 with one wave per (batch, head, 16 value columns) carries the
 *                 state through the records; used when B*H is small.  The
 *                 records (117 KiB per chunk and head at
 *                 K = 128, 61 KiB at 64) live in the library's cached per-device
 *                 workspace (grown with hipMalloc, freed by gla_release());
 *                 long sequences are processed in windows of at most 1 GiB of
 *                 records, the state carried between windows in the workspace.
 *
 * Ownership, nullability (h0 NULL = zero state, h_final NULL = not written),
 * aliasing (o, h_final must not overlap the inputs or each other), streams,
 * determinism and error codes: as gla_fwd in gla.h (GLA_ERR_ALLOC when the
 * workspace of the two-launch form cannot be grown).  Calls on one device
 * must not overlap in time.
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

/*
 * gla_gdn_set_path — which form gla_gdn_fwd uses (process-wide; a schedule
 * knob with no effect on results beyond rounding): GLA_GDN_AUTO (default:
 * two launches when B*H*K/16, the walk's one-wave work-groups, is at most
 * the work-group target of gla_set_tuning, 256 by default: B*H <= 32 at
 * K = 128, B*H <= 64 at K = 64), GLA_GDN_ONE_LAUNCH, GLA_GDN_TWO_LAUNCH.  window_chunks > 0 caps
 * the two-launch form's windows at that many 64-token chunks (0 = only the
 * 1 GiB record cap).  Returns GLA_OK, or GLA_ERR_SHAPE for another path or a
 * negative window.
 */
#define GLA_GDN_AUTO       0
#define GLA_GDN_ONE_LAUNCH 1
#define GLA_GDN_TWO_LAUNCH 2
int gla_gdn_set_path(int path, int window_chunks);

#ifdef __cplusplus
}
#endif

#endif /* GLA_GDN_H */
