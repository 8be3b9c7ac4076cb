/*
 * gla_decode.h — one decode step of gated linear attention: a single new
 * token per (batch, head) against a carried fp32 state, the state updated in
 * place.  Same recurrence as gla_fwd (gla.h), one token at a time:
 *
 *     S <- diag(exp(g)) S + k^T v        o = scale * q S
 *
 * (the D x D state update "h <- h*g + k^T v" of the blog "Linear Attention 在
 * GPU 上到底慢在哪", section 学长的反馈, which also notes that decode is the case
 * its prefill study leaves out; the update-then-read order of
 * "线性注意力GPU算子库的定义与技术解析", section 四).  A call is exactly gla_fwd
 * with T = 1, h0 = state and h_final = state, except that the state is
 * updated in place: the h_final of a gla_fwd prefill is the state to carry
 * into the first decode step.
 *
 * Layout (dense, row-major, device memory, 16-byte aligned base pointers):
 *     q, k, g  [B, H, K]      v, o  [B, H, V]      state  [B, H, K, V] fp32
 * gla_decode: q, k, v, o bfloat16 (o rounded to nearest-even from fp32);
 * gla_decode_f32: q, k, v, o float32.  g (log-decay, precondition: finite
 * and <= 0, not checked) is float32 in both.  Supported: K == V in {64, 128}.
 *
 * Ownership: the caller owns every buffer; nothing is kept after the call.
 * No workspace is used.  Work is enqueued on `stream` (hipStream_t, NULL =
 * the null stream) and runs asynchronously; each (batch, head) row is
 * independent and the result is deterministic.
 *
 * Errors: GLA_OK, or GLA_ERR_SHAPE (B, H, K or V <= 0, or B * H > 2^30), GLA_ERR_UNSUPPORTED
 * (K != V or K not in {64, 128}), GLA_ERR_NULL (any pointer NULL),
 * GLA_ERR_ALIGN, GLA_ERR_ALIAS (o or state overlapping an input, or each
 * other), GLA_ERR_DEVICE, GLA_ERR_LAUNCH.  Arguments are checked before
 * anything is enqueued.
 */
#ifndef GLA_DECODE_H
#define GLA_DECODE_H

#include "gla.h"

#ifdef __cplusplus
extern "C" {
#endif

int gla_decode(const gla_bf16 *q, const gla_bf16 *k, const gla_bf16 *v,
               const float *g, float *state, gla_bf16 *o,
               int B, int H, int K, int V, float scale, void *stream);

int gla_decode_f32(const float *q, const float *k, const float *v,
                   const float *g, float *state, float *o,
                   int B, int H, int K, int V, float scale, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GLA_DECODE_H */
