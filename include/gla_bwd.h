/*
 * gla_bwd.h — backward of the prefill forward of gla.h: the gradients of a
 * loss L with respect to q, k, v, the log-gates g and the initial state h0,
 * given dL/do and dL/dh_final.
 *
 * The pages define the forward only (the recurrence S_t = diag(exp g_t)
 * S_{t-1} + k_t^T v_t, o_t = scale q_t S_t: blog "Linear Attention 在 GPU 上到
 * 底慢在哪", section 学长的反馈; "线性注意力GPU算子库的定义与技术解析", section
 * 四) and ask the operator library for autodiff support (same page, section
 * 七).  This is the exact chain rule of that recurrence:
 *
 *   R_t     = dL/dS_t = scale q_t^T do_t + diag(exp g_{t+1}) R_{t+1},
 *             R_{T-1} = dh_final + scale q_{T-1}^T do_{T-1}
 *   dq_t    = scale S_t do_t^T          dk_t = R_t v_t^T      dv_t = k_t R_t
 *   dg_t[d] = exp(g_t[d]) sum_v R_t[d, v] S_{t-1}[d, v]      dh0 = diag(exp g_0) R_0
 *
 * evaluated in chunk form on the GPU (chunk-start states of the forward,
 * a reverse state recurrence over chunks, per-chunk matrix products).
 * Every call recomputes the forward's chunk-start states itself.
 *
 * Layout (dense, row-major, device memory, 16-byte aligned):
 *     q, k, g, dq, dk, dg   [B, H, T, K]
 *     v, do, dv             [B, H, T, V]
 *     h0, dh_final, dh0     [B, H, K, V] fp32
 * gla_bwd: q, k, v, do, dq, dk, dv bfloat16 (outputs rounded to nearest
 * even); gla_bwd_f32: float32.  g and dg are float32 in both.
 * Supported shapes are those of gla_fwd / gla_fwd_f32; chunk sizes: 32 and 64
 * for gla_bwd, 32 and 64 for gla_bwd_f32 at K = 64 and 32 at K = 128 (chunk
 * 0 picks 64 where supported, else 32).  Any other chunk returns
 * GLA_ERR_UNSUPPORTED before anything is enqueued.
 *
 * Nullability: h0 NULL = zero initial state; dh_final NULL = zero; dh0 NULL =
 * not written.  q, k, v, g, do, dq, dk, dv, dg are required when T > 0.
 * Aliasing: no output may overlap an input or another output.
 *
 * Ownership: the caller owns every buffer.  The library keeps a second
 * cached workspace per device for the backward (the forward chunk-start
 * states, B*H*ceil(T/chunk)*K*V*4 bytes, plus segment states), grown on
 * demand with hipMalloc and freed by gla_release(); the forward's workspace
 * is used too.  Calls on one device must not overlap in time.  Work is
 * enqueued on `stream`; results are deterministic.
 *
 * Precondition (not checked): g finite and <= 0.  Chunks whose gates decay
 * by more than a factor 2^80 in some key dim are evaluated elementwise with
 * running products of decays (exact, slower).
 *
 * Errors: as gla.h (GLA_ERR_SHAPE, GLA_ERR_UNSUPPORTED, GLA_ERR_NULL,
 * GLA_ERR_ALIGN, GLA_ERR_ALIAS, GLA_ERR_ALLOC, GLA_ERR_DEVICE,
 * GLA_ERR_LAUNCH), checked before anything is enqueued.
 */
#ifndef GLA_BWD_H
#define GLA_BWD_H

#include "gla.h"

#ifdef __cplusplus
extern "C" {
#endif

int gla_bwd(const gla_bf16 *q, const gla_bf16 *k, const gla_bf16 *v,
            const float *g, const float *h0, const gla_bf16 *dout,
            const float *dh_final, gla_bf16 *dq, gla_bf16 *dk, gla_bf16 *dv,
            float *dg, float *dh0, int B, int H, int T, int K, int V,
            int chunk, float scale, void *stream);

int gla_bwd_f32(const float *q, const float *k, const float *v,
                const float *g, const float *h0, const float *dout,
                const float *dh_final, float *dq, float *dk, float *dv,
                float *dg, float *dh0, int B, int H, int T, int K, int V,
                int chunk, float scale, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GLA_BWD_H */
