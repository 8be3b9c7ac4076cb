// gla_api.hip — C ABI of libgla.so: argument validation, segment scheduling,
// workspace, launches.  Declarations and contracts: include/gla.h,
// include/gla_scalar.h, include/gla_bwd.h, include/gla_gdn.h,
// include/gla_decode.h and include/gla_stages.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <vector>

#include "gla.h"
#include "gla_bwd.h"
#include "gla_decode.h"
#include "gla_gdn.h"
#include "gla_scalar.h"
#include "gla_stages.h"
#include "gla_internal.h"

// Workspace of gla_fwd_noalloc: a file-scope device array, one copy per
// device, held until the process ends.  Host code never uses its name as an
// address (on the host it is only a stand-in for the symbol): the device
// address comes from hipGetSymbolAddress, resolved once per device with that
// device current, and only that address is passed to kernels.
static constexpr size_t kScratchBytes = GLA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kVersion = 100;  // 0.1.0
constexpr int kDefaultTargetWgs = 256;


struct DeviceState {
    int arch_ok = -1;  // -1 unknown, 0 not gfx950, 1 gfx950
    void *ws = nullptr;    // forward: segment states
    size_t ws_bytes = 0;
    float *scratch = nullptr;   // this device's copy of `scratch` (gla_fwd_noalloc), once resolved
    void *bws = nullptr;   // backward: forward chunk-start states, final states, segment states
    size_t bws_bytes = 0;
};

std::mutex g_mu;
std::vector<DeviceState> g_dev;
int g_target_wgs = kDefaultTargetWgs;
int g_head_group = 0;
int g_gdn_path = GLA_GDN_AUTO;
int g_gdn_window = 0;   // chunks per window of the two-launch form (0 = by the record cap)
// records of the gated delta rule's two-launch form are made for windows of
// chunks whose records take at most this many bytes
constexpr size_t kGdnRecordCap = size_t(1) << 30;

// launch tracing (gla_profile_start / gla_profile_stop)
struct Trace {
    bool active = false;
    int capacity = 0;
    int used = 0;
    std::vector<hipEvent_t> ev;   // 2 per launch
    std::vector<int> kind;
};
Trace g_trace;

// Run `launch` bracketed by trace events when tracing is active.
template <typename F>
hipError_t traced(int kind, hipStream_t s, F &&launch) {
    int slot = -1;
    {
        std::lock_guard<std::mutex> lk(g_mu);
        if (g_trace.active && g_trace.used < g_trace.capacity) slot = g_trace.used++;
    }
    if (slot >= 0) {
        g_trace.kind[slot] = kind;
        (void)hipEventRecord(g_trace.ev[2 * slot], s);
    }
    const hipError_t e = launch();
    if (slot >= 0) (void)hipEventRecord(g_trace.ev[2 * slot + 1], s);
    return e;
}

int current_device(DeviceState **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return GLA_ERR_DEVICE;
    std::lock_guard<std::mutex> lk(g_mu);
    if (size_t(dev) >= g_dev.size()) g_dev.resize(dev + 1);
    DeviceState &d = g_dev[dev];
    if (d.arch_ok < 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return GLA_ERR_DEVICE;
        d.arch_ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 0;
    }
    if (d.arch_ok != 1) return GLA_ERR_DEVICE;
    *out = &d;
    return GLA_OK;
}

// This device's address of `scratch`, resolved on the first use on the
// device (which is current here) and kept.
int device_scratch(DeviceState *d, float **out) {
    std::lock_guard<std::mutex> lk(g_mu);
    if (!d->scratch) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return GLA_ERR_DEVICE;
        }
        d->scratch = static_cast<float *>(p);
    }
    *out = d->scratch;
    return GLA_OK;
}

int grow(void **buf, size_t *have, size_t bytes, float **out) {
    std::lock_guard<std::mutex> lk(g_mu);
    if (*have < bytes) {
        if (*buf) {
            (void)hipFree(*buf);  // hipFree waits for work that may still use it
            *buf = nullptr;
            *have = 0;
        }
        void *p = nullptr;
        if (hipMalloc(&p, bytes) != hipSuccess || !p) {
            (void)hipGetLastError();
            return GLA_ERR_ALLOC;
        }
        *buf = p;
        *have = bytes;
    }
    *out = static_cast<float *>(*buf);
    return GLA_OK;
}

int ensure_workspace(DeviceState *d, size_t bytes, float **out) { return grow(&d->ws, &d->ws_bytes, bytes, out); }
int ensure_bwd_workspace(DeviceState *d, size_t bytes, float **out) {
    return grow(&d->bws, &d->bws_bytes, bytes, out);
}

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

bool misaligned(const void *p) { return p && (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

struct Call {
    int dtype;
    const void *q, *k, *v;
    const float *g, *h0;
    void *o;
    float *h_final;
    float *states;  // stage output (chunk-start states) or nullptr
    int B, H, T, K, V, chunk;
    float scale;
    hipStream_t stream;
    bool scalar_gate = false;  // g is [B,H,T] instead of [B,H,T,K]
    bool need_o = true;        // false: only states / h_final are wanted (backward)
    void *states16 = nullptr;  // the backward's chunk-start states in bf16, or nullptr
};

// chunk 0: 64 for bf16; 32 for fp32, which ran faster than (D = 64) or as fast
// as (D = 128) chunk 64 at H = 16, T = 4K and 16K
int default_chunk(int dtype, int D) {
    if (dtype == gla::DTYPE_BF16 && gla::chunk_supported(dtype, D, 64)) return 64;
    return 32;
}

int validate(Call &c) {
    if (c.B <= 0 || c.H <= 0 || c.T < 0 || c.K <= 0 || c.V <= 0) return GLA_ERR_SHAPE;
    if (long(c.B) * c.H > (1L << 30) || long(c.T) * c.K >= (1L << 29)) return GLA_ERR_SHAPE;
    if (c.K != c.V || (c.K != 64 && c.K != 128)) return GLA_ERR_UNSUPPORTED;
    if (c.chunk < 0) return GLA_ERR_UNSUPPORTED;
    if (c.chunk == 0) c.chunk = default_chunk(c.dtype, c.K);
    if (!gla::chunk_supported(c.dtype, c.K, c.chunk)) return GLA_ERR_UNSUPPORTED;
    if (c.T > 0 && (!c.q || !c.k || !c.v || !c.g || (c.need_o && !c.o))) return GLA_ERR_NULL;
    const void *ptrs[] = {c.q, c.k, c.v, c.g, c.h0, c.o, c.h_final, c.states};
    for (const void *p : ptrs)
        if (misaligned(p)) return GLA_ERR_ALIGN;
    const size_t es = c.dtype == gla::DTYPE_BF16 ? 2 : 4;
    const size_t bht = size_t(c.B) * c.H * c.T;
    const size_t nqk = bht * c.K * es, nv = bht * c.V * es, ng = bht * (c.scalar_gate ? 1 : c.K) * 4;
    const size_t nst = size_t(c.B) * c.H * c.K * c.V * 4;
    const size_t nchunks = c.T > 0 ? size_t((c.T + c.chunk - 1) / c.chunk) : 0;
    const size_t nstates = size_t(c.B) * c.H * nchunks * c.K * c.V * 4;
    struct R { const void *p; size_t n; } ins[] = {{c.q, nqk}, {c.k, nqk}, {c.v, nv}, {c.g, ng}, {c.h0, nst}};
    for (const R &r : ins) {
        if (overlaps(c.o, nv, r.p, r.n)) return GLA_ERR_ALIAS;
        if (overlaps(c.h_final, nst, r.p, r.n)) return GLA_ERR_ALIAS;
        if (overlaps(c.states, nstates, r.p, r.n)) return GLA_ERR_ALIAS;
    }
    if (overlaps(c.h_final, nst, c.o, nv)) return GLA_ERR_ALIAS;
    if (overlaps(c.states, nstates, c.o, nv) || overlaps(c.states, nstates, c.h_final, nst))
        return GLA_ERR_ALIAS;
    return GLA_OK;
}

struct Plan {
    int P;      // output-pass segments along T
    int cps;    // chunks per output segment
    int sub;    // state-pass units per output segment (divides cps)
    int slots;  // state-pass units before the last output segment: (P - 1) * sub
};

// Output pass: about `target` work-groups (one per CU).  State pass: units
// that end on segment boundaries, about state_per_cu work-groups per CU.
Plan plan_segments(int nbh, int N, int target, int state_per_cu) {
    int P = std::max(1, (target + nbh - 1) / nbh);
    P = std::min(P, N);
    const int cps = (N + P - 1) / P;
    P = (N + cps - 1) / cps;
    int sub = 1;
    if (P > 1) {   // state units: about state_per_cu work-groups per CU target
        const int want = std::max(1, (state_per_cu * target) / (nbh * (P - 1)));
        for (int m = std::min(want, cps); m >= 1; --m)
            if (cps % m == 0) { sub = m; break; }
    }
    return {P, cps, sub, (P - 1) * sub};
}

// Bytes of segment-state workspace a validated forward call needs with the
// current schedule knobs (host arithmetic only).
size_t forward_workspace_bytes(const Call &c) {
    if (c.T == 0) return 0;
    const int D = c.K;
    const long BH = long(c.B) * c.H;
    const int N = (c.T + c.chunk - 1) / c.chunk;
    int target, hg;
    {
        std::lock_guard<std::mutex> lk(g_mu);
        target = g_target_wgs;
        hg = g_head_group;
    }
    const int spc = gla::state_units_per_cu(c.dtype, D, gla::state_chunk(c.dtype, c.chunk));
    long group = hg > 0 ? std::min<long>(hg, BH) : BH;
    group = std::min<long>(group, 65535);
    size_t need = 0;
    for (long g0 = 0; g0 < BH; g0 += group) {
        const int nbh = int(std::min(group, BH - g0));
        const Plan pl = plan_segments(nbh, N, target, spc);
        need = std::max(need, size_t(nbh) * size_t(pl.slots) * size_t(D) * (D + 1) * 4);
    }
    return need;
}

// fixed_ws != nullptr: use that workspace of fixed_cap bytes (no allocation);
// a call that needs more returns GLA_ERR_WORKSPACE.
int run_forward(Call &c, float *fixed_ws = nullptr, size_t fixed_cap = 0) {
    int rc = validate(c);
    if (rc != GLA_OK) return rc;
    DeviceState *dev = nullptr;
    if ((rc = current_device(&dev)) != GLA_OK) return rc;
    const int D = c.K;
    const long BH = long(c.B) * c.H;
    if (c.T == 0) {
        if (c.h_final && traced(GLA_KERNEL_OTHER, c.stream, [&] {
                return gla::launch_copy_state(c.h_final, c.h0, BH * D * D, c.stream);
            }) != hipSuccess)
            return GLA_ERR_LAUNCH;
        return GLA_OK;
    }
    const int N = (c.T + c.chunk - 1) / c.chunk;
    int target, hg;
    {
        std::lock_guard<std::mutex> lk(g_mu);
        target = g_target_wgs;
        hg = g_head_group;
    }
    // chunk length of the state pass (state units end on output-chunk
    // boundaries, so it may differ from the output pass's)
    const int cs = gla::state_chunk(c.dtype, c.chunk);
    const int spc = gla::state_units_per_cu(c.dtype, D, cs);
    long group = hg > 0 ? std::min<long>(hg, BH) : BH;
    group = std::min<long>(group, 65535);

    // workspace: the largest group's (P-1) segment states and decays
    const size_t need = forward_workspace_bytes(c);
    float *ws = nullptr;
    if (fixed_ws) {
        if (need > fixed_cap) return GLA_ERR_WORKSPACE;
        ws = fixed_ws;
    } else if (need > 0 && (rc = ensure_workspace(dev, need, &ws)) != GLA_OK) {
        return rc;
    }

    for (long g0 = 0; g0 < BH; g0 += group) {
        const int nbh = int(std::min(group, BH - g0));
        const Plan pl = plan_segments(nbh, N, target, spc);
        gla::KernelParams p{};
        p.q = c.q; p.k = c.k; p.v = c.v; p.g = c.g; p.h0 = c.h0;
        p.o = c.o; p.h_final = c.h_final;
        p.ws_E = ws;
        p.ws_G = ws ? ws + size_t(nbh) * pl.slots * D * D : nullptr;
        p.dump = c.states; p.dump2 = nullptr; p.dump16 = c.states16;
        p.T = c.T; p.N = N; p.bh0 = g0; p.scale = c.scale;
        p.ws_slots = pl.slots; p.sub = pl.sub;
        if (pl.P > 1) {
            gla::KernelParams ps = p;   // state pass over the chunks before the last segment
            ps.cps = pl.cps / pl.sub * (c.chunk / cs);
            ps.N = (c.T + cs - 1) / cs;
            ps.P = pl.slots;
            if (traced(GLA_KERNEL_SEGMENT, c.stream, [&] {
                    return gla::launch_chunk_kernel(c.dtype, D, cs, gla::MODE_SEG, c.scalar_gate, ps, pl.slots,
                                                    nbh, c.stream);
                }) != hipSuccess)
                return GLA_ERR_LAUNCH;
            if (traced(GLA_KERNEL_SCAN, c.stream, [&] {
                    return gla::launch_scan(p.ws_E, p.ws_G, c.h0, g0, nbh, pl.slots, D, c.stream);
                }) != hipSuccess)
                return GLA_ERR_LAUNCH;
        }
        p.cps = pl.cps;
        p.P = pl.P;
        // no o wanted (the backward's chunk-start states): the states-only
        // mode, which forms no scores
        const int mode = !c.need_o && (c.states || c.states16) ? gla::MODE_STATES : gla::MODE_OUT;
        if (traced(mode == gla::MODE_STATES ? GLA_KERNEL_STATES : GLA_KERNEL_OUTPUT, c.stream, [&] {
                return gla::launch_chunk_kernel(c.dtype, D, c.chunk, mode, c.scalar_gate, p, pl.P, nbh, c.stream);
            }) != hipSuccess)
            return GLA_ERR_LAUNCH;
    }
    return GLA_OK;
}

struct BwdCall {
    int dtype;
    const void *q, *k, *v;
    const float *g, *h0;
    const void *dout;
    const float *dhf;
    void *dq, *dk, *dv;
    float *dg, *dh0;
    int B, H, T, K, V, chunk;
    float scale;
    hipStream_t stream;
};

int run_backward(BwdCall &b) {
    // the backward's own chunk set and default (64 where it has kernels, else
    // 32), checked before anything is enqueued
    if (b.chunk == 0 && (b.K == 64 || b.K == 128))
        b.chunk = gla::bwd_chunk_supported(b.dtype, b.K, 64) ? 64 : 32;
    Call c{b.dtype, b.q, b.k, b.v, b.g, b.h0, nullptr, nullptr, nullptr, b.B, b.H, b.T, b.K, b.V,
           b.chunk, b.scale, b.stream};
    c.need_o = false;
    int rc = validate(c);   // shapes, chunk, input pointers and alignment
    if (rc != GLA_OK) return rc;
    b.chunk = c.chunk;
    if (!gla::bwd_chunk_supported(b.dtype, b.K, b.chunk)) return GLA_ERR_UNSUPPORTED;
    if (b.T > 0 && (!b.dout || !b.dq || !b.dk || !b.dv || !b.dg)) return GLA_ERR_NULL;
    const void *ptrs[] = {b.dout, b.dhf, b.dq, b.dk, b.dv, b.dg, b.dh0};
    for (const void *p : ptrs)
        if (misaligned(p)) return GLA_ERR_ALIGN;
    const size_t es = b.dtype == gla::DTYPE_BF16 ? 2 : 4;
    const size_t bht = size_t(b.B) * b.H * b.T;
    const size_t nqk = bht * b.K * es, nv = bht * b.V * es, ng = bht * b.K * 4;
    const size_t nst = size_t(b.B) * b.H * b.K * b.V * 4;
    struct R { const void *p; size_t n; };
    const R ins[] = {{b.q, nqk}, {b.k, nqk}, {b.v, nv}, {b.g, ng}, {b.h0, nst}, {b.dout, nv}, {b.dhf, nst}};
    const R outs[] = {{b.dq, nqk}, {b.dk, nqk}, {b.dv, nv}, {b.dg, ng}, {b.dh0, nst}};
    for (const R &o : outs) {
        for (const R &i : ins)
            if (overlaps(o.p, o.n, i.p, i.n)) return GLA_ERR_ALIAS;
        for (const R &o2 : outs)
            if (&o2 != &o && overlaps(o.p, o.n, o2.p, o2.n)) return GLA_ERR_ALIAS;
    }
    DeviceState *dev = nullptr;
    if ((rc = current_device(&dev)) != GLA_OK) return rc;
    const int D = b.K;
    const long BH = long(b.B) * b.H;
    if (b.T == 0) {   // dh0 = dh_final
        if (b.dh0 && traced(GLA_KERNEL_OTHER, b.stream, [&] {
                return gla::launch_copy_state(b.dh0, b.dhf, BH * D * D, b.stream);
            }) != hipSuccess)
            return GLA_ERR_LAUNCH;
        return GLA_OK;
    }
    const int N = (b.T + b.chunk - 1) / b.chunk;
    int target;
    {
        std::lock_guard<std::mutex> lk(g_mu);
        target = g_target_wgs;
    }
    const long group = std::min<long>(BH, 65535);
    // workspace: chunk-start states, then the largest group's segment states
    size_t seg_need = 0;
    for (long g0 = 0; g0 < BH; g0 += group) {
        const int nbh = int(std::min(group, BH - g0));
        const Plan pl = plan_segments(nbh, N, target, 1);
        seg_need = std::max(seg_need, size_t(nbh) * size_t(pl.P - 1) * size_t(D) * (D + 1) * 4);
    }
    const size_t n_states = size_t(BH) * N * D * D;
    const bool s16 = gla::bwd_states_bf16(b.dtype, D, b.chunk);
    const size_t states_bytes = n_states * (s16 ? 2 : 4);
    float *bws = nullptr;
    if ((rc = ensure_bwd_workspace(dev, states_bytes + seg_need, &bws)) != GLA_OK) return rc;
    void *states = bws;
    float *segws = reinterpret_cast<float *>(reinterpret_cast<unsigned char *>(bws) + states_bytes);

    // forward chunk-start states (no o, no final state)
    if (s16) c.states16 = states;
    else c.states = static_cast<float *>(states);
    if ((rc = run_forward(c)) != GLA_OK) return rc;

    for (long g0 = 0; g0 < BH; g0 += group) {
        const int nbh = int(std::min(group, BH - g0));
        const Plan pl = plan_segments(nbh, N, target, 1);
        gla::BwdParams p{};
        p.q = b.q; p.k = b.k; p.v = b.v; p.dout = b.dout; p.g = b.g;
        p.states = states; p.dhf = b.dhf;
        p.dq = b.dq; p.dk = b.dk; p.dv = b.dv; p.dg = b.dg; p.dh0 = b.dh0;
        p.ws_E = segws;
        p.ws_G = segws + size_t(nbh) * (pl.P - 1) * D * D;
        p.T = b.T; p.N = N; p.cps = pl.cps; p.P = pl.P; p.ws_slots = pl.P - 1;
        p.bh0 = g0; p.scale = b.scale;
        if (pl.P > 1) {
            // bf16: the state-pass kernel, pipelined, walking each segment first
            // chunk first (its last rows are the chunk pass's first); fp32: the
            // chunk kernel's segment mode
            gla::KernelParams kp{};
            kp.k = b.q; kp.v = b.dout; kp.g = b.g;
            kp.ws_E = p.ws_E; kp.ws_G = p.ws_G;
            kp.T = b.T; kp.N = N; kp.cps = pl.cps; kp.P = pl.P - 1; kp.ws_slots = pl.P - 1;
            kp.bh0 = g0; kp.scale = b.scale;
            if (traced(GLA_KERNEL_BWD_SEGMENT, b.stream, [&] {
                    return b.dtype == gla::DTYPE_BF16
                               ? gla::launch_bwd_segments(D, b.chunk, kp, pl.P - 1, nbh, b.stream)
                               : gla::launch_bwd(b.dtype, D, b.chunk, false, p, pl.P - 1, nbh, b.stream);
                }) != hipSuccess)
                return GLA_ERR_LAUNCH;
            if (traced(GLA_KERNEL_SCAN, b.stream, [&] {
                    return gla::launch_scan(p.ws_E, p.ws_G, b.dhf, g0, nbh, pl.P - 1, D, b.stream);
                }) != hipSuccess)
                return GLA_ERR_LAUNCH;
        }
        if (traced(GLA_KERNEL_BWD, b.stream, [&] {
                return gla::launch_bwd(b.dtype, D, b.chunk, true, p, pl.P, nbh, b.stream);
            }) != hipSuccess)
            return GLA_ERR_LAUNCH;
    }
    return GLA_OK;
}

}  // namespace

extern "C" {

int gla_bwd(const gla_bf16 *q, const gla_bf16 *k, const gla_bf16 *v, const float *g, const float *h0,
            const gla_bf16 *dout, const float *dh_final, gla_bf16 *dq, gla_bf16 *dk, gla_bf16 *dv,
            float *dg, float *dh0, int B, int H, int T, int K, int V, int chunk, float scale,
            void *stream) {
    BwdCall b{gla::DTYPE_BF16, q, k, v, g, h0, dout, dh_final, dq, dk, dv, dg, dh0, B, H, T, K, V,
              chunk, scale, static_cast<hipStream_t>(stream)};
    return run_backward(b);
}

int gla_bwd_f32(const float *q, const float *k, const float *v, const float *g, const float *h0,
                const float *dout, const float *dh_final, float *dq, float *dk, float *dv, float *dg,
                float *dh0, int B, int H, int T, int K, int V, int chunk, float scale, void *stream) {
    BwdCall b{gla::DTYPE_F32, q, k, v, g, h0, dout, dh_final, dq, dk, dv, dg, dh0, B, H, T, K, V,
              chunk, scale, static_cast<hipStream_t>(stream)};
    return run_backward(b);
}


int gla_fwd(const gla_bf16 *q, const gla_bf16 *k, const gla_bf16 *v, const float *g,
            const float *h0, gla_bf16 *o, float *h_final, int B, int H, int T, int K, int V,
            int chunk, float scale, void *stream) {
    Call c{gla::DTYPE_BF16, q, k, v, g, h0, o, h_final, nullptr, B, H, T, K, V, chunk, scale,
           static_cast<hipStream_t>(stream)};
    return run_forward(c);
}

int gla_fwd_f32(const float *q, const float *k, const float *v, const float *g, const float *h0,
                float *o, float *h_final, int B, int H, int T, int K, int V, int chunk, float scale,
                void *stream) {
    Call c{gla::DTYPE_F32, q, k, v, g, h0, o, h_final, nullptr, B, H, T, K, V, chunk, scale,
           static_cast<hipStream_t>(stream)};
    return run_forward(c);
}

int gla_fwd_noalloc(const gla_bf16 *q, const gla_bf16 *k, const gla_bf16 *v, const float *g,
                    const float *h0, gla_bf16 *o, float *h_final, int B, int H, int T, int K, int V,
                    int chunk, float scale, void *stream) {
    Call c{gla::DTYPE_BF16, q, k, v, g, h0, o, h_final, nullptr, B, H, T, K, V, chunk, scale,
           static_cast<hipStream_t>(stream)};
    int rc = validate(c);
    if (rc != GLA_OK) return rc;
    // the size check is host arithmetic and comes before any device call
    if (forward_workspace_bytes(c) > kScratchBytes) return GLA_ERR_WORKSPACE;
    DeviceState *dev = nullptr;
    if ((rc = current_device(&dev)) != GLA_OK) return rc;
    float *ws = nullptr;
    if ((rc = device_scratch(dev, &ws)) != GLA_OK) return rc;
    return run_forward(c, ws, kScratchBytes);
}

// Scalar-gate forward (include/gla_scalar.h): g is [B,H,T].
int gla_fwd_scalar(const gla_bf16 *q, const gla_bf16 *k, const gla_bf16 *v, const float *g,
                   const float *h0, gla_bf16 *o, float *h_final, int B, int H, int T, int K, int V,
                   int chunk, float scale, void *stream) {
    Call c{gla::DTYPE_BF16, q, k, v, g, h0, o, h_final, nullptr, B, H, T, K, V, chunk, scale,
           static_cast<hipStream_t>(stream), true};
    return run_forward(c);
}

int gla_fwd_scalar_f32(const float *q, const float *k, const float *v, const float *g, const float *h0,
                       float *o, float *h_final, int B, int H, int T, int K, int V, int chunk, float scale,
                       void *stream) {
    Call c{gla::DTYPE_F32, q, k, v, g, h0, o, h_final, nullptr, B, H, T, K, V, chunk, scale,
           static_cast<hipStream_t>(stream), true};
    return run_forward(c);
}

// Gated delta rule forward (include/gla_gdn.h).
int gla_gdn_fwd(const gla_bf16 *q, const gla_bf16 *k, const gla_bf16 *v, const float *g, const float *beta,
            const float *h0, gla_bf16 *o, float *h_final, int B, int H, int T, int K, int V, int chunk,
            float scale, void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (B <= 0 || H <= 0 || T < 0 || K <= 0 || V <= 0) return GLA_ERR_SHAPE;
    if (long(B) * H > (1L << 30) || long(T) * K >= (1L << 29)) return GLA_ERR_SHAPE;
    if (K != V || (K != 64 && K != 128) || (chunk != 0 && chunk != 64)) return GLA_ERR_UNSUPPORTED;
    if (T > 0 && (!q || !k || !v || !g || !beta || !o)) return GLA_ERR_NULL;
    const void *ptrs[] = {q, k, v, g, beta, h0, o, h_final};
    for (const void *p : ptrs)
        if (misaligned(p)) return GLA_ERR_ALIGN;
    const size_t bh = size_t(B) * H, bht = bh * T;
    const size_t nx = bht * K * 2, ns = bht * 4, nst = bh * K * V * 4;
    struct R { const void *p; size_t n; } ins[] = {{q, nx}, {k, nx}, {v, nx}, {g, ns}, {beta, ns}, {h0, nst}};
    for (const R &r : ins) {
        if (overlaps(o, nx, r.p, r.n)) return GLA_ERR_ALIAS;
        if (overlaps(h_final, nst, r.p, r.n)) return GLA_ERR_ALIAS;
    }
    if (overlaps(h_final, nst, o, nx)) return GLA_ERR_ALIAS;
    DeviceState *dev = nullptr;
    int rc = current_device(&dev);
    if (rc != GLA_OK) return rc;
    if (T == 0) {
        if (h_final && traced(GLA_KERNEL_OTHER, s, [&] {
                return gla::launch_copy_state(h_final, h0, long(bh) * K * V, s);
            }) != hipSuccess)
            return GLA_ERR_LAUNCH;
        return GLA_OK;
    }
    int target, path, wcap;
    {
        std::lock_guard<std::mutex> lk(g_mu);
        target = g_target_wgs;
        path = g_gdn_path;
        wcap = g_gdn_window;
    }
    const int N = (T + 63) / 64;
    // The walk runs K / 16 one-wave work-groups per (batch, head), one per CU;
    // while they all fit at once the two launches win, beyond that the walk
    // takes a second round (T = 4K, K = 128: two launches 0.149 / 0.202 ms
    // against one 0.301 / 0.309 ms at B*H = 16 / 32; from B*H = 40 one launch,
    // 0.312 against 0.390 ms)
    const bool two = path == GLA_GDN_TWO_LAUNCH || (path == GLA_GDN_AUTO && long(bh) * (K / 16) <= target);
    if (!two) {
        // split value columns over work-groups while batch x heads leaves CUs idle
        int nvb = 1;
        while (nvb < K / 16 && long(bh) * nvb * 2 <= target) nvb *= 2;
        gla::GdnParams p{q, k, v, g, beta, h0, o, h_final, T, scale, nvb};
        p.nbh = int(bh);
        if (traced(GLA_KERNEL_GDN, s, [&] { return gla::launch_gdn(K, p, long(bh), s); }) != hipSuccess)
            return GLA_ERR_LAUNCH;
        return GLA_OK;
    }
    // two launches per window of chunks: the chunk-local prep (all chunks at
    // once), then the sequential walk carrying the state
    const size_t rec = gla::gdn_record_bytes(K);
    int window = int(std::max<size_t>(1, std::min<size_t>(size_t(N), kGdnRecordCap / (bh * rec))));
    if (wcap > 0) window = std::min(window, wcap);
    const bool multi = window < N;
    const size_t nrec = bh * size_t(window);
    const size_t need = nrec * rec + nrec * 4 + (multi ? nst : 0);
    float *ws = nullptr;
    if ((rc = ensure_workspace(dev, need, &ws)) != GLA_OK) return rc;
    unsigned char *wsb = reinterpret_cast<unsigned char *>(ws);
    float *ws_gc = reinterpret_cast<float *>(wsb + nrec * rec);
    float *carry = multi ? reinterpret_cast<float *>(wsb + nrec * rec + nrec * 4) : nullptr;
    const int slices_max = int(std::min<long>(65535, std::max<long>(1, (target + long(bh) - 1) / long(bh))));
    for (int c0 = 0; c0 < N; c0 += window) {
        const int nc = std::min(window, N - c0);
        const bool last = c0 + nc >= N;
        gla::GdnParams p{q, k, v, g, beta, c0 == 0 ? h0 : carry, o, last ? h_final : carry, T, scale, 1};
        p.ws = wsb;
        p.ws_gc = ws_gc;
        p.c0 = c0;
        p.nc = nc;
        p.nbh = int(bh);
        const int slices = std::min(nc, slices_max);
        if (traced(GLA_KERNEL_GDN_PREP, s, [&] { return gla::launch_gdn_prep(K, p, slices, s); }) != hipSuccess)
            return GLA_ERR_LAUNCH;
        if (traced(GLA_KERNEL_GDN_WALK, s, [&] { return gla::launch_gdn_walk(K, p, s); }) != hipSuccess)
            return GLA_ERR_LAUNCH;
    }
    return GLA_OK;
}

int gla_gdn_set_path(int path, int window_chunks) {
    if (path != GLA_GDN_AUTO && path != GLA_GDN_ONE_LAUNCH && path != GLA_GDN_TWO_LAUNCH) return GLA_ERR_SHAPE;
    if (window_chunks < 0) return GLA_ERR_SHAPE;
    std::lock_guard<std::mutex> lk(g_mu);
    g_gdn_path = path;
    g_gdn_window = window_chunks;
    return GLA_OK;
}

// One decode step (include/gla_decode.h).
static int decode_call(int dtype, const void *q, const void *k, const void *v, const float *g,
                       float *state, void *o, int B, int H, int K, int V, float scale, hipStream_t stream) {
    if (B <= 0 || H <= 0 || K <= 0 || V <= 0) return GLA_ERR_SHAPE;
    if (long(B) * H > (1L << 30)) return GLA_ERR_SHAPE;
    if (K != V || (K != 64 && K != 128)) return GLA_ERR_UNSUPPORTED;
    if (!q || !k || !v || !g || !state || !o) return GLA_ERR_NULL;
    const void *ptrs[] = {q, k, v, g, state, o};
    for (const void *p : ptrs)
        if (misaligned(p)) return GLA_ERR_ALIGN;
    const size_t es = dtype == gla::DTYPE_BF16 ? 2 : 4;
    const size_t bh = size_t(B) * H;
    const size_t nvec = bh * K * es, ng = bh * K * 4, nst = bh * K * V * 4;
    struct R { const void *p; size_t n; } ins[] = {{q, nvec}, {k, nvec}, {v, nvec}, {g, ng}};
    for (const R &r : ins) {
        if (overlaps(o, nvec, r.p, r.n)) return GLA_ERR_ALIAS;
        if (overlaps(state, nst, r.p, r.n)) return GLA_ERR_ALIAS;
    }
    if (overlaps(state, nst, o, nvec)) return GLA_ERR_ALIAS;
    DeviceState *dev = nullptr;
    int rc = current_device(&dev);
    if (rc != GLA_OK) return rc;
    if (traced(GLA_KERNEL_DECODE, stream, [&] {
            return gla::launch_decode(dtype, K, q, k, v, g, state, o, long(bh), scale, stream);
        }) != hipSuccess)
        return GLA_ERR_LAUNCH;
    return GLA_OK;
}

int gla_decode(const gla_bf16 *q, const gla_bf16 *k, const gla_bf16 *v, const float *g, float *state,
               gla_bf16 *o, int B, int H, int K, int V, float scale, void *stream) {
    return decode_call(gla::DTYPE_BF16, q, k, v, g, state, o, B, H, K, V, scale,
                       static_cast<hipStream_t>(stream));
}

int gla_decode_f32(const float *q, const float *k, const float *v, const float *g, float *state,
                   float *o, int B, int H, int K, int V, float scale, void *stream) {
    return decode_call(gla::DTYPE_F32, q, k, v, g, state, o, B, H, K, V, scale,
                       static_cast<hipStream_t>(stream));
}

int gla_stage_states(const gla_bf16 *q, const gla_bf16 *k, const gla_bf16 *v, const float *g,
                     const float *h0, gla_bf16 *o, float *h_final, float *states, int B, int H,
                     int T, int K, int V, int chunk, float scale, void *stream) {
    if (T > 0 && !states) return GLA_ERR_NULL;
    Call c{gla::DTYPE_BF16, q, k, v, g, h0, o, h_final, states, B, H, T, K, V, chunk, scale,
           static_cast<hipStream_t>(stream)};
    return run_forward(c);
}

static int run_stage(int mode, const void *q, const void *k, const float *g, float *out,
                     float *out2, int B, int H, int T, int K, int chunk, float scale, void *stream) {
    Call c{gla::DTYPE_BF16, q, k, q, g, nullptr, out, nullptr, nullptr, B, H, T, K, K, chunk, scale,
           static_cast<hipStream_t>(stream)};
    if (B <= 0 || H <= 0 || T < 0 || K <= 0) return GLA_ERR_SHAPE;
    if (long(B) * H > (1L << 30) || long(T) * K >= (1L << 29)) return GLA_ERR_SHAPE;
    if (K != 64 && K != 128) return GLA_ERR_UNSUPPORTED;
    if (chunk < 0) return GLA_ERR_UNSUPPORTED;
    if (chunk == 0) c.chunk = default_chunk(c.dtype, K);
    if (!gla::chunk_supported(c.dtype, K, c.chunk)) return GLA_ERR_UNSUPPORTED;
    if (T == 0) return GLA_OK;
    if (!g || !out || (mode == gla::MODE_INTRA && (!q || !k)) || (mode == gla::MODE_CUMSUM && !out2))
        return GLA_ERR_NULL;
    const void *ptrs[] = {q, k, g, out, out2};
    for (const void *p : ptrs)
        if (misaligned(p)) return GLA_ERR_ALIGN;
    DeviceState *dev = nullptr;
    int rc = current_device(&dev);
    if (rc != GLA_OK) return rc;
    const int N = (T + c.chunk - 1) / c.chunk;
    const long BH = long(B) * H;
    gla::KernelParams p{};
    p.q = q; p.k = k; p.v = q; p.g = g;
    p.dump = out; p.dump2 = out2;
    p.T = T; p.N = N; p.cps = 1; p.P = N; p.scale = scale;
    for (long g0 = 0; g0 < BH; g0 += 65535) {
        p.bh0 = g0;
        const int nbh = int(std::min<long>(65535, BH - g0));
        if (traced(GLA_KERNEL_OTHER, c.stream, [&] {
                return gla::launch_chunk_kernel(c.dtype, K, c.chunk, mode, false, p, N, nbh, c.stream);
            }) != hipSuccess)
            return GLA_ERR_LAUNCH;
    }
    return GLA_OK;
}

int gla_stage_cumsum(const float *g, float *gc, float *gamma, int B, int H, int T, int K, int chunk,
                     void *stream) {
    return run_stage(gla::MODE_CUMSUM, nullptr, nullptr, g, gc, gamma, B, H, T, K, chunk, 1.0f, stream);
}

int gla_stage_intra(const gla_bf16 *q, const gla_bf16 *k, const float *g, float *A, int B, int H,
                    int T, int K, int chunk, float scale, void *stream) {
    return run_stage(gla::MODE_INTRA, q, k, g, A, nullptr, B, H, T, K, chunk, scale, stream);
}

int gla_set_tuning(int target_wgs, int head_group) {
    if (target_wgs < 0 || head_group < 0) return GLA_ERR_SHAPE;
    std::lock_guard<std::mutex> lk(g_mu);
    g_target_wgs = target_wgs > 0 ? target_wgs : kDefaultTargetWgs;
    g_head_group = head_group;
    return GLA_OK;
}

static void trace_clear() {
    for (hipEvent_t e : g_trace.ev)
        if (e) (void)hipEventDestroy(e);
    g_trace = Trace{};
}

int gla_profile_start(int capacity) {
    if (capacity < 0) return GLA_ERR_SHAPE;
    std::lock_guard<std::mutex> lk(g_mu);
    trace_clear();
    g_trace.ev.assign(2 * size_t(capacity), nullptr);
    g_trace.kind.assign(size_t(capacity), GLA_KERNEL_OTHER);
    for (hipEvent_t &e : g_trace.ev) {
        if (hipEventCreate(&e) != hipSuccess) {
            (void)hipGetLastError();
            trace_clear();
            return GLA_ERR_ALLOC;
        }
    }
    g_trace.capacity = capacity;
    g_trace.active = true;
    return GLA_OK;
}

int gla_profile_stop(gla_kernel_time *out, int max, int *count) {
    std::lock_guard<std::mutex> lk(g_mu);
    g_trace.active = false;
    const int n = g_trace.used;
    if (n > 0 && (!out || !count)) {
        trace_clear();
        return GLA_ERR_NULL;
    }
    int written = 0;
    for (int i = 0; i < n && i < max; ++i) {
        float ms = -1.f;
        if (hipEventSynchronize(g_trace.ev[2 * i + 1]) == hipSuccess)
            (void)hipEventElapsedTime(&ms, g_trace.ev[2 * i], g_trace.ev[2 * i + 1]);
        out[written++] = gla_kernel_time{g_trace.kind[i], ms};
    }
    if (count) *count = written;
    trace_clear();
    return GLA_OK;
}

const char *gla_strerror(int code) {
    switch (code) {
        case GLA_OK: return "ok";
        case GLA_ERR_NULL: return "a required pointer is NULL";
        case GLA_ERR_SHAPE: return "invalid shape (B, H >= 1, T >= 0, sizes within limits)";
        case GLA_ERR_UNSUPPORTED: return "unsupported head dim or chunk size";
        case GLA_ERR_ALIGN: return "a base pointer is not 16-byte aligned";
        case GLA_ERR_LAUNCH: return "kernel launch failed";
        case GLA_ERR_ALLOC: return "workspace allocation failed";
        case GLA_ERR_ALIAS: return "an output buffer overlaps an input buffer";
        case GLA_ERR_DEVICE: return "no usable gfx950 HIP device";
        case GLA_ERR_WORKSPACE: return "the call needs more workspace than the static scratch holds";
        default: return "unknown error code";
    }
}

int gla_version(void) { return kVersion; }

long long gla_workspace_bytes(void) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
    std::lock_guard<std::mutex> lk(g_mu);
    if (size_t(dev) >= g_dev.size()) return 0;
    return (long long)(g_dev[dev].ws_bytes + g_dev[dev].bws_bytes);
}

void gla_release(void) {
    std::lock_guard<std::mutex> lk(g_mu);
    int cur = -1;
    (void)hipGetDevice(&cur);
    for (size_t i = 0; i < g_dev.size(); ++i) {
        if (g_dev[i].ws || g_dev[i].bws) {
            (void)hipSetDevice(int(i));
            if (g_dev[i].ws) (void)hipFree(g_dev[i].ws);
            if (g_dev[i].bws) (void)hipFree(g_dev[i].bws);
            g_dev[i].ws = nullptr;
            g_dev[i].ws_bytes = 0;
            g_dev[i].bws = nullptr;
            g_dev[i].bws_bytes = 0;
        }
    }
    if (cur >= 0) (void)hipSetDevice(cur);
}

}  // extern "C"
