/*
 * gla.h — C ABI of libgla.so: causal prefill forward of gated linear
 * attention (GLA) in chunk form, hand-written HIP kernels for gfx950.
 *
 * Operation (per batch row b and head h, independently):
 *
 *     S_t = diag(exp(g_t)) S_{t-1} + k_t^T v_t        S_{-1} = h0 (or 0)
 *     o_t = scale * q_t S_t                           h_final = S_{T-1}
 *
 * S is a K x V fp32 state; g is a per-key-dim log-decay (g <= 0).  Sources:
 * the D x D state update "h <- h*g + k^T v" (blog "Linear Attention 在 GPU 上
 * 到底慢在哪", section 学长的反馈); the update-then-read recurrence
 * ("线性注意力GPU算子库的定义与技术解析", section 四); the chunk form — split the
 * sequence into chunks, pass states between chunks, compute the within-chunk
 * part with matrix units (same page, sections 三.1, 三.3 and 四); the five
 * kernels the blog profiles (cumsum, intra-chunk scores, state recurrence,
 * output; section 实验结果, Kernel Profiling).  The chunked evaluation is a
 * reordering of the same sums: the result does not depend on `chunk` beyond
 * rounding.
 *
 * Layout: all tensors dense, row-major, device memory:
 *     q, k, g   [B, H, T, K]        v, o   [B, H, T, V]
 *     h0, h_final [B, H, K, V] fp32
 * q, k, v, o are bfloat16 (gla_fwd) or float32 (gla_fwd_f32); g is float32
 * in both.  Every base pointer must be 16-byte aligned.
 *
 * Supported shapes: K == V in {64, 128}; T >= 0; B, H >= 1; any T (the last
 * chunk may be partial) with T * K < 2^29 and B * H <= 2^30, since each
 * (batch, head) row is addressed with 32-bit byte offsets; larger sizes return
 * GLA_ERR_SHAPE.  chunk: 0 picks the default (64 for gla_fwd, 32 for
 * gla_fwd_f32); gla_fwd accepts 32, 64 and 128; gla_fwd_f32 accepts 32 and 64.
 * Anything else returns GLA_ERR_UNSUPPORTED, never a silent fallback.
 *
 * Ownership: the caller owns every buffer.  The library keeps no pointer to
 * them after the call returns.  It owns an internal workspace (fp32 segment
 * states, about (B*H) * (segments-1) * K*(V+1) * 4 bytes) cached per device
 * and grown on demand with hipMalloc; gla_release() frees it.  Work is
 * enqueued on `stream` (a hipStream_t; NULL means the null stream) and runs
 * asynchronously; the call returns after enqueueing.  Calls that share a
 * device share its workspace: calls on one device must not overlap in time
 * (issue them on one stream, or synchronise between streams).
 *
 * Nullability / aliasing: h0 == NULL means a zero initial state; h_final ==
 * NULL means the final state is not written.  o must not overlap q, k, v, g
 * or h0; h_final must not overlap any input or o.  Precondition (not
 * checked): g finite and <= 0.  Results are deterministic (no atomics) and
 * finite for finite inputs with g <= 0, including extreme gates.
 *
 * Errors: every entry point returns GLA_OK (0) or a negative code below.
 * Arguments are validated before anything is enqueued, so nothing is
 * written on error.  The library never aborts or prints.  Faults of enqueued
 * kernels surface at the caller's next synchronisation.
 */
#ifndef GLA_H
#define GLA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GLA_OK               0
#define GLA_ERR_NULL        -1  /* a required pointer is NULL                  */
#define GLA_ERR_SHAPE       -2  /* B/H <= 0, T < 0, K != V, or past the limits */
#define GLA_ERR_UNSUPPORTED -3  /* K/V or chunk outside the supported set      */
#define GLA_ERR_ALIGN       -4  /* a base pointer is not 16-byte aligned       */
#define GLA_ERR_LAUNCH      -5  /* a kernel launch failed (hipGetLastError)    */
#define GLA_ERR_ALLOC       -6  /* workspace allocation failed                 */
#define GLA_ERR_ALIAS       -7  /* an output overlaps an input                 */
#define GLA_ERR_DEVICE      -8  /* no usable HIP device / wrong architecture   */
#define GLA_ERR_WORKSPACE   -9  /* gla_fwd_noalloc: the call needs more
                                   workspace than the static scratch holds    */

/* bfloat16 values are passed as their 16-bit storage. */
typedef uint16_t gla_bf16;

/*
 * gla_fwd — bf16 in/out, fp32 gates and state.  Writes o [B,H,T,V] (bf16,
 * round-to-nearest-even from the fp32 accumulators) and, if h_final is not
 * NULL, the fp32 final state.  `scale` multiplies the whole output
 * (typically K^-0.5).
 */
int gla_fwd(const gla_bf16 *q, const gla_bf16 *k, const gla_bf16 *v,
            const float *g, const float *h0, gla_bf16 *o, float *h_final,
            int B, int H, int T, int K, int V, int chunk, float scale,
            void *stream);

/* gla_fwd_f32 — the same operation with fp32 q, k, v and o. */
int gla_fwd_f32(const float *q, const float *k, const float *v,
                const float *g, const float *h0, float *o, float *h_final,
                int B, int H, int T, int K, int V, int chunk, float scale,
                void *stream);

/*
 * gla_fwd_noalloc — gla_fwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same operation, arguments, layout, results and errors as
 * gla_fwd, but the call allocates nothing.  Its segment-state workspace is a
 * static device array of GLA_NOALLOC_SCRATCH_BYTES (64 MiB) that the library
 * holds on each device it runs on until the process ends; its address is
 * looked up on the first call on a device.  That covers the default schedule
 * at every supported shape (at most 32.25 MiB, for K = 128 with chunk 32: the
 * segment states of about 512 state-pass work-groups); a call whose schedule
 * needs more (raised target_wgs in gla_set_tuning) returns GLA_ERR_WORKSPACE
 * before anything is enqueued.
 * Every call on a device shares that device's array, whose contents are
 * whatever the last call left (each call writes what it reads first), so
 * calls that overlap in time on one device race: issue them on one stream or
 * synchronise between them.
 */
#define GLA_NOALLOC_SCRATCH_BYTES (64u << 20)
int gla_fwd_noalloc(const gla_bf16 *q, const gla_bf16 *k, const gla_bf16 *v,
                    const float *g, const float *h0, gla_bf16 *o, float *h_final,
                    int B, int H, int T, int K, int V, int chunk, float scale,
                    void *stream);

/*
 * gla_set_tuning — schedule knobs (no effect on results beyond rounding of
 * the segment boundaries' fp32 states).  target_wgs: work-groups the
 * segment split aims for (0 = default 256, one per CU); head_group: heads
 * processed per pass of the three-launch pipeline (0 = all at once).
 * Returns GLA_OK, or GLA_ERR_SHAPE for negative values.
 */
int gla_set_tuning(int target_wgs, int head_group);

/*
 * Launch tracing.  Between gla_profile_start and gla_profile_stop every
 * kernel the library enqueues is bracketed by two HIP events recorded on
 * the launch stream, so its device duration can be read back.  Kinds:
 * GLA_KERNEL_OUTPUT (the fused chunk pass that writes o), GLA_KERNEL_STATES
 * (the backward's states-only forward chunk pass), GLA_KERNEL_SEGMENT
 * (segment end states), GLA_KERNEL_SCAN (segment-state scan),
 * GLA_KERNEL_DECODE (a gla_decode step, gla_decode.h), GLA_KERNEL_BWD_SEGMENT
 * and GLA_KERNEL_BWD (the backward's segment pass and chunk pass,
 * gla_bwd.h), GLA_KERNEL_GDN, GLA_KERNEL_GDN_PREP and GLA_KERNEL_GDN_WALK
 * (gla_gdn_fwd's one-launch form and the two launches of its other form,
 * gla_gdn.h), GLA_KERNEL_OTHER.
 * gla_profile_start(capacity) creates the events
 * (capacity launches; more are not traced) and returns GLA_OK or
 * GLA_ERR_ALLOC.  gla_profile_stop waits for the traced work, writes up to
 * `max` records in launch order to `out`, stores the number written in
 * *count, destroys the events and returns GLA_OK (GLA_ERR_NULL if out or
 * count is NULL while records exist).  Not thread-safe with concurrent
 * gla_fwd calls.
 */
#define GLA_KERNEL_OUTPUT  0
#define GLA_KERNEL_SEGMENT 1
#define GLA_KERNEL_SCAN    2
#define GLA_KERNEL_OTHER   3
#define GLA_KERNEL_DECODE  4
#define GLA_KERNEL_BWD_SEGMENT 5
#define GLA_KERNEL_BWD     6
#define GLA_KERNEL_GDN     7
#define GLA_KERNEL_GDN_PREP 8
#define GLA_KERNEL_GDN_WALK 9
#define GLA_KERNEL_STATES  10
typedef struct {
    int kind;     /* GLA_KERNEL_* */
    float ms;     /* device time between the bracketing events */
} gla_kernel_time;

int gla_profile_start(int capacity);
int gla_profile_stop(gla_kernel_time *out, int max, int *count);

/* Human-readable text for a return code (static storage, never NULL). */
const char *gla_strerror(int code);

/* Library version: major*10000 + minor*100 + patch. */
int gla_version(void);

/*
 * Bytes of device workspace the library holds on the current device (the
 * forward's segment states plus the backward's chunk-start states), as
 * grown by the calls so far; 0 when none is held.  Reported next to the
 * caller's own buffers as the library's share of peak device memory.
 */
long long gla_workspace_bytes(void);

/* Free the cached workspace on every device.  Call with no work pending. */
void gla_release(void);

#ifdef __cplusplus
}
#endif

#endif /* GLA_H */
