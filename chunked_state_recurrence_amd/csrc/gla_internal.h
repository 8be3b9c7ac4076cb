// gla_internal.h — shared between the kernels and the C-ABI layer of libgla.so.
#pragma once

#include <hip/hip_runtime.h>

namespace gla {

enum { DTYPE_BF16 = 0, DTYPE_F32 = 1 };

// MODE_OUT: output pass from given segment start states (writes o, h_final,
//           and optionally the chunk-start states into `dump`).
// MODE_SEG: end state of each segment from a zero start (writes ws_E, ws_G).
// MODE_INTRA / MODE_CUMSUM: single stages written to `dump` / `dump2`.
// MODE_STATES: the chunk-start states only (into `dump` or `dump16`, and
//           h_final), from given segment start states; no scores, no o.
enum { MODE_OUT = 0, MODE_SEG = 1, MODE_INTRA = 2, MODE_CUMSUM = 3, MODE_STATES = 4 };

struct KernelParams {
    const void *q, *k, *v;
    const float *g;
    const float *h0;
    void *o;
    float *h_final;
    float *ws_E;   // [nbh][ws_slots][D][D]  state-pass end states, then start states
    float *ws_G;   // [nbh][ws_slots][D]     state-pass total log2-decay
    float *dump;   // stage outputs
    float *dump2;
    void *dump16;  // chunk-start states in bf16 (the backward's, see bwd_states_bf16)
    int T;         // tokens per (batch, head)
    int N;         // chunks per (batch, head)
    int cps;       // chunks per segment
    int P;         // work-groups along T in this launch
    int ws_slots;  // state-pass units per (batch, head) in the workspace
    int sub;       // state-pass units per output segment (output pass reads slot seg*sub - 1)
    long bh0;      // first (batch, head) row of this launch
    float scale;
};

// The backward keeps the forward's chunk-start states in bf16 (they enter the
// dq product as bf16 MFMA operands in any case) where a state slot still
// holds the exact path's fp32 staging of one chunk's C x D sums, D >= 2 C;
// fp32 otherwise.
constexpr bool bwd_states_bf16(int dtype, int D, int C) { return dtype == DTYPE_BF16 && D >= 2 * C; }

// backward chunk kernel (gla_bwd.hip)
struct BwdParams {
    const void *q, *k, *v, *dout;
    const float *g;
    const void *states;    // forward chunk-start states [heads][N][D][D], fp32 or bf16 (bwd_states_bf16)
    const float *dhf;      // dL/dh_final [heads][D][D] or null (zero)
    void *dq, *dk, *dv;
    float *dg;
    float *dh0;            // or null
    float *ws_E;           // [nbh][ws_slots][D][D]  segment contributions, then U at segment ends
    float *ws_G;           // [nbh][ws_slots][D]     segment total log2-decays
    int T, N, cps, P, ws_slots;
    long bh0;              // first (batch, head) row of this launch
    float scale;
};

// gated delta rule (gla_gdn.hip): one work-group per (batch, head)
struct GdnParams {
    const void *q, *k, *v;     // bf16 [heads][T][D]
    const float *g, *beta;     // [heads][T]
    const float *h0;           // [heads][D][D] or null
    void *o;                   // bf16 [heads][T][D]
    float *h_final;            // [heads][D][D] or null
    int T;
    float scale;
    int nvb;                   // value-column blocks per (batch, head): 1, 2, 4 or 8 (D / 16 at most)
    // two-launch form (chunk-parallel prep, then the sequential walk) over the
    // window of chunks [c0, c0 + nc): per-chunk records and gamma_C per chunk
    void *ws;                  // [heads][nc] records of gdn_record_bytes(D)
    float *ws_gc;              // [heads][nc]
    int c0, nc;
    int nbh;                   // batch x heads
};
hipError_t launch_gdn(int D, const GdnParams &p, long nbh, hipStream_t s);
// the backward's segment pass on the state-pass kernel (bf16; p.k = q, p.v = do,
// p.ws_slots = segments - 1, grid_x = p.ws_slots)
hipError_t launch_bwd_segments(int D, int C, const KernelParams &p, int grid_x, int grid_y, hipStream_t s);
size_t gdn_record_bytes(int D);
hipError_t launch_gdn_prep(int D, const GdnParams &p, int slices, hipStream_t s);
hipError_t launch_gdn_walk(int D, const GdnParams &p, hipStream_t s);

bool chunk_supported(int dtype, int D, int C);
// chunk sizes the backward has kernels for (a subset of the forward's)
bool bwd_chunk_supported(int dtype, int D, int C);
// chunk length of the state pass for an output-pass chunk of C tokens (it
// divides C, so state units end on output-chunk boundaries)
int state_chunk(int dtype, int C);
// work-groups of the state pass that fit on one CU (LDS bound), 1 or 2
int state_units_per_cu(int dtype, int D, int C);
// scalar_gate: g is [B,H,T] (one log-decay per token), MODE_OUT / MODE_SEG only
hipError_t launch_chunk_kernel(int dtype, int D, int C, int mode, bool scalar_gate,
                               const KernelParams &p, int grid_x, int grid_y, hipStream_t s);
hipError_t launch_scan(float *ws_E, const float *ws_G, const float *h0, long bh0, int nbh,
                       int slots, int D, hipStream_t s);
hipError_t launch_copy_state(float *dst, const float *src, long n, hipStream_t s);
// backward: full = false, the segment contributions (grid: P - 1 slots x
// heads); full = true, the per-segment chunk walk (grid: P segments x heads)
hipError_t launch_bwd(int dtype, int D, int C, bool full, const BwdParams &p, int gx, int gy,
                      hipStream_t s);
// one decode step for nbh (batch, head) rows, state [nbh][D][D] updated in place
hipError_t launch_decode(int dtype, int D, const void *q, const void *k, const void *v, const float *g,
                         float *state, void *o, long nbh, float scale, hipStream_t s);

}  // namespace gla
