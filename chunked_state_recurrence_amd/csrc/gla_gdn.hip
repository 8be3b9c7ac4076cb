// gla_gdn.hip — gfx950 kernel for the gated delta rule (Gated DeltaNet
// forward), chunk form.
//
// Recurrence (per batch row and head; scalar gate and write strength per
// token): S_t = exp(g_t) (I - beta_t k_t^T k_t) S_{t-1} + beta_t k_t^T v_t,
// o_t = scale q_t S_t.  The evaluation page "面向长序列大模型的线性注意力算子
// 性能评测方法与优化实践" (sections 一 and 三.3) describes the GDN class as
// gating plus an incremental state update without a formula; this is the
// published gated delta rule.
//
// Chunk form (rows i, j of a chunk; gamma_i = exp of the chunk-local
// inclusive cumsum of g; S the chunk-start state).  The rows written into the
// state, u_i = beta_i (v_i - exp(g_i) k_i S_{i-1}), satisfy
//     (I + A) U = diag(beta) V - diag(beta gamma) K S,
//     A_ij = beta_i (gamma_i / gamma_j) (k_i . k_j)        (j < i),
// so with T = (I + A)^{-1}:  U = T diag(beta) (V - (gamma K) S) = U~ - W S with
// U~ = T diag(beta) V and W = T diag(beta) (gamma K), and
//     o_i    = scale [ gamma_i q_i S + sum_{j<=i} (gamma_i / gamma_j) (q_i . k_j) u_j ]
//     S_next = gamma_C S + sum_j (gamma_C / gamma_j) k_j^T u_j.
// Every factor is at most 1 (gamma_i / gamma_j with j <= i), so extreme gates
// need no special path.  T is formed by blocks: the 16 x 16 diagonal blocks
// by forward substitution (one lane per column), the others level by level,
// T_IJ = -T_II sum_{J<=K<I} A_IK T_KJ, with fp32 MFMA.
//
// One work-group per (batch, head, block of value columns) walks the chunks
// in order.  Value columns of S evolve independently (the state is mixed only
// along its key rows), so when batch x heads would leave CUs idle the value
// columns are split over several work-groups; each one forms the chunk-local
// A, P and T for all key dims and U, o, S for its own columns.  The products
// that need S but not T, V - (gamma K) S and (scale gamma q) S, run while one
// wave solves T's diagonal blocks and three more its off-diagonal ones; U is
// then T diag(beta) times the first, and W is never formed.  S stays in
// MFMA accumulators (the block's value columns are spread 16 per wave over
// its first waves) and is fed to the S products straight from them (the row
// operand's columns are permuted in LDS, as in the forward output pass).
//
// Two-launch form, for few (batch, head) pairs: the chain of phases above is
// long and only the state products depend on S, so a prep launch (the same
// kernel, PREP = true) forms every chunk's state-independent half at once and
// stores it as a record: -W, Q' = scale gamma q - P W, K^ = (gamma_C / gamma) k,
// U~ and O0 = P U~ (with bf16 W and U~ as the MFMA operands), and gamma_C.  A
// walk (gdn_walk_kernel) then carries S through the records:
//     U = U~ - W S,   o = O0 + Q' S,   S <- gamma_C S + K^T U,
// the same o as above since q^ S + P (U~ - W S) = (q^ - P W) S + P U~.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gla_device.h"
#include "gla_internal.h"

namespace gla {

// v moved between lanes by DPP control CTRL, written only in the rows of
// ROW_MASK; lanes with no source, and rows outside the mask, read 0
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float wave_dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf, false));
}

// WIDE (the one-launch kernel): permuted rows padded by 32 bytes (288 / 160
// bytes), on which a 16-row fragment read takes one LDS pass instead of two;
// the prep kernel keeps 16-byte pads, since its tiles are the byte images of
// the records, whose size bounds the walk's direct loads per chunk.
template <int D, int C, bool WIDE = false> struct GdnLayout {
    static constexpr int QP = D + (WIDE ? 16 : 8);   // permuted-row tiles, bf16 elements per row
    static constexpr int PD = 2 * D + 32;            // bank-spread bf16 tiles, bytes per row
    static constexpr int PC = 2 * C + 32;            // bank-spread bf16 C x C tiles
    static constexpr int PF = C + 4;                 // fp32 C x C tiles, floats per row
    static constexpr int TD = BF16::tile_bytes(C, PD);
    static constexpr int TQ = C * QP * 2;
    static constexpr int R = TD > TQ ? TD : TQ;      // a region holding either layout
    // Three LDS arrays: the targets of the direct loads that run ahead of their
    // chunk (the fp32 A / T area, which stages the next chunk's q and k rows,
    // and the v tile) are kept apart from the tiles in use meanwhile.
    // main: kr raw k rows, later -W (permuted);  qr raw q rows, later U or W
    // (bank-spread);  kg gamma k, later (gamma_C / gamma) k;  qh scale gamma q
    // (permuted);  pp P (bf16, rows i, columns j <= i);  tb T diag(beta) (bf16)
    static constexpr int kr = 0, qr = kr + R, kg = qr + R, qh = kg + TD, pp = qh + TQ;
    static constexpr int tb = pp + BF16::tile_bytes(C, PC);
    static constexpr int main_bytes = tb + BF16::tile_bytes(C, PC);
    static constexpr int at_bytes = 2 * C * PF * 4;            // A then T (fp32)
    static constexpr int v_bytes = TD;                          // v rows (bank-spread)
    static constexpr int bytes = main_bytes + at_bytes + v_bytes;
};

// Per-chunk record that the prep pass leaves for the walk (device memory,
// [heads][chunks of the window] records).  The three operand tiles are byte
// images of the LDS tiles the walk reads them from (pads included), so the
// walk stages them with plain 16-byte direct loads:
//   wi: -W rows, permuted columns          qi: Q' = scale gamma q - P W rows, permuted
//   ki: (gamma_C / gamma) k rows, bank-spread
//   ut, ot: U~ = T diag(beta) V and O0 = P U~ (fp32) in the MFMA accumulator
//   layout, [value block of 16][row tile of 16][lane][4]: one value block's
//   tiles are 4 KB of contiguous bytes.
template <int D, int C> struct GdnRec {
    using L = GdnLayout<D, C>;
    static constexpr int IW = C * L::QP * 2;
    static constexpr int IK = L::TD;
    static constexpr int wi = 0, qi = IW, ki = 2 * IW, ut = ki + IK, ot = ut + C * D * 4;
    static constexpr int bytes = ot + C * D * 4;
    static constexpr int images = ut;                 // bytes of the three tile images
    static constexpr int blk = (C / 16) * 1024;       // one value block of ut or ot
    static_assert(IW % 1024 == 0 && IK % 1024 == 0 && bytes % 1024 == 0, "1 KB direct-load granules");
};

size_t gdn_record_bytes(int D) { return D == 128 ? GdnRec<128, 64>::bytes : GdnRec<64, 64>::bytes; }

// 16 x 16 x 16 fp32 product from LDS blocks (row-major, `pa` / `pb` floats per
// row): acc[e] += sum_m A[4 q4 + e][m] B[m][n16]... with the operands supplied
// as v_mfma_f32_16x16x4f32 takes them (lane (n16, q4) gives A[n16][4i + q4]
// and B[4i + q4][n16] in step i).
__device__ __forceinline__ f32x4_t mma16_f32(const float *A, int pa, const float *B, int pb,
                                             int n16, int q4, f32x4_t acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(A[n16 * pa + 4 * i + q4], B[(4 * i + q4) * pb + n16],
                                                   acc, 0, 0, 0);
    return acc;
}

__device__ __forceinline__ void wave_lds_fence() { __asm__ __volatile__("s_waitcnt lgkmcnt(0)" ::: "memory"); }

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

// four consecutive bf16 of an LDS row (8 bytes) from fp32
__device__ __forceinline__ void st_row4(__bf16 *dst, f32x4_t x) {
    bf16x4_t b;
#pragma unroll
    for (int e = 0; e < 4; ++e) b[e] = (__bf16)x[e];
    *reinterpret_cast<bf16x4_t *>(dst) = b;
}

// PREP = false: the whole recurrence, one work-group per (batch, head, value
// block) walking every chunk.  PREP = true: the chunk-local half only (no
// state), work-group (head, slice) taking chunks slice, slice + slices, ... of
// the window [c0, c0 + nc) and writing each chunk's record for the walk.
template <int D, int C, bool PREP>
__global__ void __launch_bounds__((Shape<D, C>::NW * 64))
gdn_kernel(const GdnParams p) {
    using E = BF16;
    using L = GdnLayout<D, C, !PREP>;
    using frag_t = E::frag_t;
    constexpr int NW = Shape<D, C>::NW;
    constexpr int RPW = Shape<D, C>::RPW;
    constexpr int NB = C / 16;
    constexpr int CPL = D / 64;
    constexpr int VS = D / NW;
    constexpr int NTW = VS / 16;
    constexpr int MT = D / 16;
    constexpr int KS = D / 32;
    constexpr int TS = C / 32;
    constexpr int NTILE = NB * (NB + 1) / 2;
    static_assert(C == 64 && NB == 4, "the blocked inverse is written for 64-row chunks");
    static_assert(NW >= NB, "one wave per column of T's off-diagonal blocks, another for its diagonal");
    static_assert(L::bytes + 2 * C * 4 <= 163840, "LDS");

    __shared__ __attribute__((aligned(16))) unsigned char smem[L::main_bytes];
    __shared__ __attribute__((aligned(16))) unsigned char sAT[L::at_bytes];
    __shared__ __attribute__((aligned(16))) unsigned char sVV[L::v_bytes];
    __shared__ __attribute__((aligned(16))) float sGc[C];   // chunk-local inclusive cumsum of g, log2 units
    __shared__ float sBeta[C];

    unsigned char *tKr = smem + L::kr;   // raw k, row-major (then -W, permuted)
    unsigned char *tQr = smem + L::qr;   // raw q, row-major (then U, bank-spread)
    unsigned char *tKg = smem + L::kg;   // gamma k, then (gamma_C / gamma) k
    __bf16 *tQh = reinterpret_cast<__bf16 *>(smem + L::qh);   // scale gamma q, permuted columns
    unsigned char *tV = sVV;
    unsigned char *tP = smem + L::pp;
    unsigned char *tTb = smem + L::tb;
    float *tA = reinterpret_cast<float *>(sAT);
    float *tT = tA + C * L::PF;
    __bf16 *tW = reinterpret_cast<__bf16 *>(tKr);
    __bf16 *tKh = reinterpret_cast<__bf16 *>(tKg);   // one launch: gamma k, permuted columns
    static_assert(L::TQ <= L::TD, "permuted gamma k over the gamma k tile");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int n16 = lane & 15;
    const int q4 = lane >> 4;
    const long bh = blockIdx.x;
    const int T = p.T;
    const int N = PREP ? p.nc : (T + C - 1) / C;   // chunks walked, counted from chunk cb
    const int cb = PREP ? p.c0 : 0;
    const int cfirst = PREP ? int(blockIdx.y) : 0, cstep = PREP ? int(gridDim.y) : 1;
    const int kcb = w * VS;                         // this wave's key columns of W
    const int VB = PREP ? D : D / p.nvb;            // value columns of this work-group
    const bool vw = kcb < VB;                       // does this wave own value columns?
    const int vb = (PREP ? 0 : int(blockIdx.y)) * VB + kcb;   // its first value column
    const int r0 = RPW * w;

    const rsrc_t bo = make_rsrc(reinterpret_cast<uint16_t *>(p.o) + bh * long(T) * D, long(T) * D * 2);
    const rsrc_t bg = make_rsrc(p.g + bh * long(T), long(T) * 4);
    const rsrc_t bb = make_rsrc(p.beta + bh * long(T), long(T) * 4);
    const u32x4_t wq = rsrc_words(reinterpret_cast<const uint16_t *>(p.q) + bh * long(T) * D, long(T) * D * 2);
    const u32x4_t wk = rsrc_words(reinterpret_cast<const uint16_t *>(p.k) + bh * long(T) * D, long(T) * D * 2);
    const u32x4_t wv = rsrc_words(reinterpret_cast<const uint16_t *>(p.v) + bh * long(T) * D, long(T) * D * 2);

    auto rowp = [&](unsigned char *tile, int r, int pitch) {
        return reinterpret_cast<__bf16 *>(tile + E::rowoff(r, pitch));
    };

    // ---- state ---------------------------------------------------------------
    f32x4_t S[MT][NTW];
    if constexpr (!PREP) {
        if (p.h0 && vw) {   // one branch around all loads, so they are in flight together
            const float *src = p.h0 + bh * long(D) * D;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
                    for (int e = 0; e < 4; ++e) S[mt][nt][e] = src[(16 * mt + 4 * q4 + e) * D + vb + 16 * nt + n16];
        } else {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt) S[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
    }
    // entries above the diagonal of P and T diag(beta) are never written
    for (int i = tid; i < 2 * E::tile_bytes(C, L::PC) / 4; i += NW * 64) reinterpret_cast<uint32_t *>(tP)[i] = 0u;

    // Loads of chunk cn: q and k rows into the staging area over the fp32 A / T
    // tiles (each wave its own rows, 16-byte lanes), v rows into the bank-spread
    // tile, gates of the chunk into wave 0's registers.  Chunk c + 1 is requested
    // while chunk c still works, once those areas are free.
    unsigned char *stq = sAT;
    unsigned char *stk = stq + C * D * 2;
    constexpr int NSL = RPW * D * 2 / 1024;   // 16-byte-lane loads per wave and operand
    static_assert(NSL * 1024 == RPW * D * 2 && 2 * C * D * 2 <= 2 * C * L::PF * 4, "staging");
    float gx = 0.f, gb = 0.f;
    auto issue_qk = [&](int cn) {
        const int row0 = __builtin_amdgcn_readfirstlane((cb + cn) * C + r0);
        const int lr0 = __builtin_amdgcn_readfirstlane(r0);
        mem_fence_compiler();
#pragma unroll
        for (int i = 0; i < NSL; ++i) {
            dma_untracked<16>(wq, lds_addr(stq) + lr0 * D * 2 + i * 1024, lane * 16, row0 * D * 2 + i * 1024);
            dma_untracked<16>(wk, lds_addr(stk) + lr0 * D * 2 + i * 1024, lane * 16, row0 * D * 2 + i * 1024);
        }
        mem_fence_compiler();
    };
    auto issue_vg = [&](int cn) {
        const int row0 = __builtin_amdgcn_readfirstlane((cb + cn) * C + r0);
        const int lr0 = __builtin_amdgcn_readfirstlane(r0);
        mem_fence_compiler();
#pragma unroll
        for (int i = 0; i < RPW; ++i)   // 4 bytes per lane: a 64-wide row takes lanes 0..31
            if (CPL == 2 || lane < 32)
                dma_untracked<4>(wv, lds_addr(sVV) + E::rowoff(lr0 + i, L::PD), lane * 4, (row0 + i) * D * 2);
        mem_fence_compiler();
        if (w == 0) {
            gx = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(bg, ((cb + cn) * C + lane) * 4, 0, 0));
            gb = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(bb, ((cb + cn) * C + lane) * 4, 0, 0));
        }
    };
    if (cfirst < N) {
        issue_qk(cfirst);
        issue_vg(cfirst);
    }

    for (int c = cfirst; c < N; c += cstep) {
        const int t0 = (cb + c) * C;
        const int cn = c + cstep;
        // ---- gates of the chunk scanned (log2 units), one row per lane -------------
        if (w == 0) {
            // inclusive scan over the wave by DPP: within each 16-lane row
            // (lane - 1, 2, 4, 8; 0 before the row's start), then the running
            // totals of the rows before (lane 15 into rows 1 and 3, lane 31
            // into rows 2 and 3; the other rows add 0)
            float x = gx * kLog2e;
            x += wave_dpp<0x111, 0xf>(x);
            x += wave_dpp<0x112, 0xf>(x);
            x += wave_dpp<0x114, 0xf>(x);
            x += wave_dpp<0x118, 0xf>(x);
            x += wave_dpp<0x142, 0xa>(x);
            x += wave_dpp<0x143, 0xc>(x);
            sGc[lane] = x;
            sBeta[lane] = gb;
        }
        wait_vmem<0>();   // this chunk's rows (requested one chunk ahead)
        block_sync();  // B1: gates, v rows

        // ---- operand rows ----------------------------------------------------------
        const float gcl = sGc[C - 1];
        Raw<E, CPL> rq[RPW], rk[RPW];
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            rq[i].x = reinterpret_cast<const decltype(rq[i].x) *>(stq + (r0 + i) * D * 2)[lane];
            rk[i].x = reinterpret_cast<const decltype(rk[i].x) *>(stk + (r0 + i) * D * 2)[lane];
        }
        // a lane's CPL columns stay adjacent in every layout (perm_col keeps the
        // pair 2l, 2l + 1 together), so each row of each tile is one store
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            const int r = r0 + i;
            const float gr = sGc[r];
            const float gam = fexp2(gr);
            const int col = lane * CPL;
            float kv[CPL], qv[CPL], kgv[CPL], qhv[CPL];
#pragma unroll
            for (int u = 0; u < CPL; ++u) {
                kv[u] = rk[i].get(u);
                qv[u] = rq[i].get(u);
                kgv[u] = kv[u] * gam;
                qhv[u] = qv[u] * gam * p.scale;
            }
            using raw_t = decltype(rk[i].x);   // the raw rows as loaded, no conversion
            *reinterpret_cast<raw_t *>(reinterpret_cast<__bf16 *>(tKr) + r * L::QP + col) = rk[i].x;
            *reinterpret_cast<raw_t *>(reinterpret_cast<__bf16 *>(tQr) + r * L::QP + col) = rq[i].x;
            if constexpr (PREP) st_lds_cols<E>(rowp(tKg, r, L::PD) + col, kgv);
            else st_lds_cols<E>(tKh + r * L::QP + perm_col(col), kgv);
            st_lds_cols<E>(tQh + r * L::QP + perm_col(col), qhv);
        }
        block_sync();  // B2: operand tiles

        // ---- A = beta_i (gamma_i / gamma_j) (k_i . k_j) (j < i, fp32) and
        //      P = (gamma_i / gamma_j) (q_i . k_j) (j <= i, bf16), causal tiles ----------
        const __bf16 *kraw = reinterpret_cast<const __bf16 *>(tKr);
        const __bf16 *qraw = reinterpret_cast<const __bf16 *>(tQr);
#pragma unroll
        for (int t = 0; t < NTILE; ++t) {
            if (t % NW != w) continue;
            int I = 0, J = t;
#pragma unroll
            for (int r = 0; r < NB; ++r)
                if (J > r) { J -= r + 1; I = r + 1; }
            f32x4_t kk = {0.f, 0.f, 0.f, 0.f}, qk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int pos = ks * 32 + 8 * q4;
                const frag_t kj = E::ld_frag(kraw + (16 * J + n16) * L::QP + pos);
                kk = E::mma(kj, E::ld_frag(kraw + (16 * I + n16) * L::QP + pos), kk);
                qk = E::mma(kj, E::ld_frag(qraw + (16 * I + n16) * L::QP + pos), qk);
            }
            // acc[e] = (. . k_j)[i = 16I + n16][j = 16J + 4q4 + e]; the factors are
            // formed for every j and masked by selects (no branches), and the four
            // values go out as one store per tile
            const int i = 16 * I + n16;
            const float gi = sGc[i], bi = sBeta[i];
            const f32x4_t gj = *reinterpret_cast<const f32x4_t *>(sGc + 16 * J + 4 * q4);
            f32x4_t av;
            float pv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = 16 * J + 4 * q4 + e;
                const float rt = fexp2(gi - gj[e]);   // may overflow above the diagonal: never used there
                const float ratio = j <= i ? rt : 0.f;
                av[e] = j < i ? bi * ratio * kk[e] : 0.f;
                pv[e] = p.scale * ratio * qk[e];
            }
            *reinterpret_cast<f32x4_t *>(tA + i * L::PF + 16 * J + 4 * q4) = av;
            st_lds_cols<E>(rowp(tP, i, L::PC) + 16 * J + 4 * q4, pv);
        }
        block_sync();  // B3: A, P

        // One launch: the products that do not need T run while it is formed, in
        // each wave that owns value columns and is not making T at the time:
        //   O = (scale gamma q) S  and  V' = V - (gamma K) S  for its columns, S
        //   straight from its accumulators, V' (bf16) into the former raw q tile;
        // after T, U = T diag(beta) V' replaces U~ - W S, so W is never formed.
        f32x4_t O[NTW][NB];
        auto resid_and_o = [&]() {
            f32x4_t G[NTW][NB];
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
                for (int m = 0; m < NB; ++m) {
                    O[nt][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                    G[nt][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                }
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                frag_t sf[NTW];
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt) {
                    float x[8];
#pragma unroll
                    for (int e = 0; e < 4; ++e) { x[e] = S[2 * ks][nt][e]; x[4 + e] = S[2 * ks + 1][nt][e]; }
                    sf[nt] = E::pack(x);
                }
#pragma unroll
                for (int m = 0; m < NB; ++m) {
                    const frag_t kf = E::ld_frag(tKh + (16 * m + n16) * L::QP + ks * 32 + 8 * q4);
                    const frag_t qf = E::ld_frag(tQh + (16 * m + n16) * L::QP + ks * 32 + 8 * q4);
#pragma unroll
                    for (int nt = 0; nt < NTW; ++nt) {
                        G[nt][m] = E::mma(sf[nt], kf, G[nt][m]);
                        O[nt][m] = E::mma(sf[nt], qf, O[nt][m]);
                    }
                }
            }
            // acc[e] = X[row 16m + n16][col vb + 16nt + 4q4 + e]
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
                for (int m = 0; m < NB; ++m) {
                    const int co = vb + 16 * nt + 4 * q4;
                    const bf16x4_t v = *reinterpret_cast<const bf16x4_t *>(rowp(tV, 16 * m + n16, L::PD) + co);
                    f32x4_t r;
#pragma unroll
                    for (int e = 0; e < 4; ++e) r[e] = float(v[e]) - G[nt][m][e];
                    st_row4(rowp(tQr, 16 * m + n16, L::PD) + co, r);
                }
        };

        // ---- T = (I + A)^{-1}: diagonal blocks by substitution (the last wave, one
        //      lane per column of each of the four blocks) ----------------------------
        if (w == NW - 1) {
            const int blk = lane >> 4, col = lane & 15;
            float tcol[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float x = i == col ? 1.f : 0.f;
#pragma unroll
                for (int j = 0; j < i; ++j) x -= tA[(16 * blk + i) * L::PF + 16 * blk + j] * tcol[j];
                tcol[i] = x;
            }
            const float bc = sBeta[16 * blk + col];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                tT[(16 * blk + i) * L::PF + 16 * blk + col] = tcol[i];
                rowp(tTb, 16 * blk + i, L::PC)[16 * blk + col] = (__bf16)(tcol[i] * bc);
            }
        } else if constexpr (!PREP) {
            if (vw) resid_and_o();
        }
        block_sync();  // B4: diagonal blocks of T
        // off-diagonal blocks: wave NW - NB + J makes column J of T, T_{J+1,J},
        // T_{J+2,J}, ... in turn; each needs only the diagonal blocks, A and the
        // column's own earlier blocks (this wave's stores, seen after its LDS
        // fence), so the levels need no barrier between them
        if (w >= NW - NB && w < NW - 1) {
#pragma unroll
            for (int d = 1; d < NB; ++d) {
                const int J = w - (NW - NB), I = J + d;
                if (I >= NB) break;
                f32x4_t x = {0.f, 0.f, 0.f, 0.f};
                for (int Kb = J; Kb < I; ++Kb)
                    x = mma16_f32(tA + (16 * I) * L::PF + 16 * Kb, L::PF, tT + (16 * Kb) * L::PF + 16 * J, L::PF,
                                  n16, q4, x);
                // x[e] = X[4q4 + e][n16]; park X in T's (I, J) block, then T_IJ = -T_II X
                float *blkIJ = tT + (16 * I) * L::PF + 16 * J;
#pragma unroll
                for (int e = 0; e < 4; ++e) blkIJ[(4 * q4 + e) * L::PF + n16] = x[e];
                wave_lds_fence();
                f32x4_t y = {0.f, 0.f, 0.f, 0.f};
                float av[4], bv4[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    av[i] = tT[(16 * I + n16) * L::PF + 16 * I + 4 * i + q4];
                    bv4[i] = blkIJ[(4 * i + q4) * L::PF + n16];
                }
                wave_lds_fence();
#pragma unroll
                for (int i = 0; i < 4; ++i) y = __builtin_amdgcn_mfma_f32_16x16x4f32(av[i], bv4[i], y, 0, 0, 0);
                const float bc = sBeta[16 * J + n16];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    blkIJ[(4 * q4 + e) * L::PF + n16] = -y[e];
                    rowp(tTb, 16 * I + 4 * q4 + e, L::PC)[16 * J + n16] = (__bf16)(-y[e] * bc);
                }
                wave_lds_fence();   // T_IJ visible to this wave's next block
            }
        } else if constexpr (!PREP) {
            if (w == NW - 1 && vw) resid_and_o();
        }
        block_sync();  // B5: T complete
        if constexpr (PREP) {
        if (cn < N) issue_qk(cn);   // the A / T tiles are no longer read

        // ---- W = T diag(beta) (gamma K) and U~ = T diag(beta) V for this wave's
        //      columns; acc[e] = X[row 16m + n16][col + 4q4 + e] -------------------------
        f32x4_t Wa[NTW][NB], Ua[NTW][NB];
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
            for (int m = 0; m < NB; ++m) {
                Wa[nt][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                Ua[nt][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
        for (int ts = 0; ts < TS; ++ts)
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt) {
                const frag_t kf = E::ld_col8(tKg, L::PD, ts * 32 + 8 * q4, kcb + 16 * nt, n16);
#pragma unroll
                for (int m = 0; m < NB; ++m) {
                    if (ts * 32 > 16 * m + 15) continue;   // T is lower triangular
                    const frag_t tf = E::ld_frag(rowp(tTb, 16 * m + n16, L::PC) + ts * 32 + 8 * q4);
                    Wa[nt][m] = E::mma(kf, tf, Wa[nt][m]);
                }
                if (vw) {
                    const frag_t vf = E::ld_col8(tV, L::PD, ts * 32 + 8 * q4, vb + 16 * nt, n16);
#pragma unroll
                    for (int m = 0; m < NB; ++m) {
                        if (ts * 32 > 16 * m + 15) continue;
                        const frag_t tf = E::ld_frag(rowp(tTb, 16 * m + n16, L::PC) + ts * 32 + 8 * q4);
                        Ua[nt][m] = E::mma(vf, tf, Ua[nt][m]);
                    }
                }
            }
        block_sync();  // B8: gamma k and v no longer read
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
            for (int m = 0; m < NB; ++m)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    tW[(16 * m + n16) * L::QP + perm_col(kcb + 16 * nt + 4 * q4 + e)] = (__bf16)(-Wa[nt][m][e]);
#pragma unroll
        for (int i = 0; i < RPW; ++i) {   // (gamma_C / gamma) k over gamma k
            const int r = r0 + i;
            const float gk = fexp2(gcl - sGc[r]);
            float kv[CPL];
#pragma unroll
            for (int u = 0; u < CPL; ++u) kv[u] = rk[i].get(u) * gk;
            st_lds_cols<E>(rowp(tKg, r, L::PD) + lane * CPL, kv);
        }
        using R = GdnRec<D, C>;
        unsigned char *rec = nullptr;
        if constexpr (PREP) {
            // W (bf16, bank-spread, over raw q) and U~ (bf16, over v) as operands of
            // P W and P U~; U~ in fp32 into the record
            rec = static_cast<unsigned char *>(p.ws) + (size_t(bh) * p.nc + c) * R::bytes;
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
                for (int m = 0; m < NB; ++m) {
                    __bf16 *dw = rowp(tQr, 16 * m + n16, L::PD) + kcb + 16 * nt + 4 * q4;
                    __bf16 *du = rowp(tV, 16 * m + n16, L::PD) + vb + 16 * nt + 4 * q4;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        dw[e] = (__bf16)Wa[nt][m][e];
                        du[e] = (__bf16)Ua[nt][m][e];
                    }
                    *reinterpret_cast<f32x4_t *>(rec + R::ut + ((vb + 16 * nt) / 16) * R::blk + m * 1024 + lane * 16) =
                        Ua[nt][m];
                }
        }
        block_sync();  // B9: -W and the state-update rows visible

            // ---- Q' = scale gamma q - P W (in place over the permuted q tile) and
            //      O0 = P U~ (fp32, into the record); acc[e] = X[row 16m + n16][col + 4q4 + e]
            f32x4_t Qa[NTW][NB], Oa[NTW][NB];
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
                for (int m = 0; m < NB; ++m) {
                    Qa[nt][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                    Oa[nt][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                }
#pragma unroll
            for (int m = 0; m < NB; ++m)
#pragma unroll
                for (int ts = 0; ts < TS; ++ts) {
                    if (ts * 32 > 16 * m + 15) continue;   // P is lower triangular
                    const frag_t pf = E::ld_frag(rowp(tP, 16 * m + n16, L::PC) + ts * 32 + 8 * q4);
#pragma unroll
                    for (int nt = 0; nt < NTW; ++nt) {
                        Qa[nt][m] = E::mma(E::ld_col8(tQr, L::PD, ts * 32 + 8 * q4, kcb + 16 * nt, n16), pf, Qa[nt][m]);
                        Oa[nt][m] = E::mma(E::ld_col8(tV, L::PD, ts * 32 + 8 * q4, vb + 16 * nt, n16), pf, Oa[nt][m]);
                    }
                }
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
                for (int m = 0; m < NB; ++m) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        __bf16 &x = tQh[(16 * m + n16) * L::QP + perm_col(kcb + 16 * nt + 4 * q4 + e)];
                        x = (__bf16)(float(x) - Qa[nt][m][e]);
                    }
                    *reinterpret_cast<f32x4_t *>(rec + R::ot + ((vb + 16 * nt) / 16) * R::blk + m * 1024 + lane * 16) =
                        Oa[nt][m];
                }
            block_sync();  // B10: the three tile images complete, v and raw q free
            if (cn < N) issue_vg(cn);
            // tile images to the record, 16 bytes per lane
            {
                const unsigned char *src[3] = {tKr, reinterpret_cast<const unsigned char *>(tQh), tKg};
                const int off[3] = {R::wi, R::qi, R::ki};
                const int len[3] = {R::IW, R::IW, R::IK};
#pragma unroll
                for (int a = 0; a < 3; ++a)
                    for (int o = tid * 16; o < len[a]; o += NW * 64 * 16)
                        *reinterpret_cast<u32x4_t *>(rec + off[a] + o) =
                            *reinterpret_cast<const u32x4_t *>(src[a] + o);
            }
            if (tid == 0) p.ws_gc[size_t(bh) * p.nc + c] = fexp2(gcl);
        } else {

        // ---- U = T diag(beta) V' for this wave's columns (V' formed while T was),
        //      into the former raw k tile; (gamma_C / gamma) k over gamma k;
        //      O += P U; o rows to HBM; S <- gamma_C S + ((gamma_C / gamma) k)^T U ------
        if (cn < N) {   // the A / T area and the v tile are no longer read
            issue_qk(cn);
            issue_vg(cn);
        }
        if (vw) {
            f32x4_t Ua[NTW][NB];
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
                for (int m = 0; m < NB; ++m) Ua[nt][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ts = 0; ts < TS; ++ts)
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt) {
                    const frag_t vf = E::ld_col8(tQr, L::PD, ts * 32 + 8 * q4, vb + 16 * nt, n16);
#pragma unroll
                    for (int m = 0; m < NB; ++m) {
                        if (ts * 32 > 16 * m + 15) continue;   // T is lower triangular
                        const frag_t tf = E::ld_frag(rowp(tTb, 16 * m + n16, L::PC) + ts * 32 + 8 * q4);
                        Ua[nt][m] = E::mma(vf, tf, Ua[nt][m]);
                    }
                }
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
                for (int m = 0; m < NB; ++m) st_row4(rowp(tKr, 16 * m + n16, L::PD) + vb + 16 * nt + 4 * q4, Ua[nt][m]);
        }
#pragma unroll
        for (int i = 0; i < RPW; ++i) {   // (gamma_C / gamma) k over gamma k
            const int r = r0 + i;
            const float gk = fexp2(gcl - sGc[r]);
            float kv[CPL];
#pragma unroll
            for (int u = 0; u < CPL; ++u) kv[u] = rk[i].get(u) * gk;
            st_lds_cols<E>(rowp(tKg, r, L::PD) + lane * CPL, kv);
        }
        wave_lds_fence();   // this wave's U columns, read back below
        const float gC = fexp2(gcl);
        if (vw) {
#pragma unroll
            for (int m = 0; m < NB; ++m)
#pragma unroll
                for (int ts = 0; ts < TS; ++ts) {
                    if (ts * 32 > 16 * m + 15) continue;
                    const frag_t pf = E::ld_frag(rowp(tP, 16 * m + n16, L::PC) + ts * 32 + 8 * q4);
#pragma unroll
                    for (int nt = 0; nt < NTW; ++nt)
                        O[nt][m] = E::mma(E::ld_col8(tKr, L::PD, ts * 32 + 8 * q4, vb + 16 * nt, n16), pf, O[nt][m]);
                }
#pragma unroll
            for (int m = 0; m < NB; ++m)
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt) E::st4(bo, ((t0 + 16 * m + n16) * D + vb + 16 * nt + 4 * q4) * 2, O[nt][m]);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
                    for (int e = 0; e < 4; ++e) S[mt][nt][e] *= gC;
        }
        block_sync();  // B10: the (gamma_C / gamma) k rows complete
        if (vw) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int ts = 0; ts < TS; ++ts) {
                    const frag_t a = E::ld_col8(tKg, L::PD, ts * 32 + 8 * q4, 16 * mt, n16);
#pragma unroll
                    for (int nt = 0; nt < NTW; ++nt)
                        S[mt][nt] = E::mma(a, E::ld_col8(tKr, L::PD, ts * 32 + 8 * q4, vb + 16 * nt, n16), S[mt][nt]);
                }
        }
        }
        block_sync();  // B11: tiles free for the next chunk
    }

    if constexpr (!PREP) {
        if (p.h_final && vw) {
            float *dst = p.h_final + bh * long(D) * D;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
                    for (int e = 0; e < 4; ++e) dst[(16 * mt + 4 * q4 + e) * D + vb + 16 * nt + n16] = S[mt][nt][e];
        }
    }
}

// The sequential half: one wave per (batch, head, 16 value columns) walks the
// chunks of the window with its columns of S in MFMA accumulators,
//     U = U~ - W S,   o = O0 + Q' S,   S <- gamma_C S + ((gamma_C / gamma) k)^T U,
// reading each chunk's record (staged by direct loads into LDS one chunk ahead).
// The D / 16 waves of one head are placed on one XCD (work-groups are dealt to
// the XCDs round-robin), so they share the records through that XCD's L2.
// p.h0 is the state at the window start (null = zero), p.h_final receives the
// state at its end (null = not written); they may be the same buffer.
template <int D, int C>
__global__ void __launch_bounds__(64)
gdn_walk_kernel(const GdnParams p) {
    using E = BF16;
    using L = GdnLayout<D, C>;
    using R = GdnRec<D, C>;
    using frag_t = E::frag_t;
    constexpr int NB = C / 16;
    constexpr int MT = D / 16;
    constexpr int KS = D / 32;
    constexpr int TS = C / 32;
    constexpr int NVB = D / 16;
    constexpr int OU = R::images, OO = OU + R::blk, OG = OO + R::blk;
    constexpr int BUF = OG + 256;                              // one chunk's staged record
    constexpr int NIMG = R::images / 1024, NBLK = R::blk / 1024;
    constexpr int NISSUE = NIMG + 2 * NBLK + 1;                // direct loads per chunk
    static_assert(NISSUE <= 63, "vmcnt range");
    static_assert(2 * BUF <= 163840, "LDS");
    __shared__ __attribute__((aligned(16))) unsigned char smem[2 * BUF];

    const int lane = threadIdx.x;
    const int n16 = lane & 15;
    const int q4 = lane >> 4;
    const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
    const long bh = long(j / NVB) * 8 + xcd;
    if (bh >= p.nbh) return;
    const int vb = (j % NVB) * 16;
    const int nc = p.nc;
    const int T = p.T;

    const u32x4_t wrec = rsrc_words(static_cast<const unsigned char *>(p.ws) + size_t(bh) * nc * R::bytes,
                                    long(nc) * R::bytes);
    const u32x4_t wgc = rsrc_words(p.ws_gc + size_t(bh) * nc, long(nc) * 4);
    const rsrc_t bo = make_rsrc(reinterpret_cast<uint16_t *>(p.o) + bh * long(T) * D, long(T) * D * 2);

    f32x4_t S[MT];
    if (p.h0) {
        const float *src = p.h0 + bh * long(D) * D;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int e = 0; e < 4; ++e) S[mt][e] = src[(16 * mt + 4 * q4 + e) * D + vb + n16];
    } else {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) S[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    auto issue = [&](int c) {
        const uint32_t lb = lds_addr(smem) + (c & 1) * BUF;
        const int base = __builtin_amdgcn_readfirstlane(c * R::bytes);
        const int vblk = __builtin_amdgcn_readfirstlane(vb / 16);
        mem_fence_compiler();
#pragma unroll
        for (int i = 0; i < NIMG; ++i) dma_untracked<16, true>(wrec, lb + i * 1024, lane * 16, base + i * 1024);
#pragma unroll
        for (int i = 0; i < NBLK; ++i) {
            dma_untracked<16, true>(wrec, lb + OU + i * 1024, lane * 16, base + R::ut + vblk * R::blk + i * 1024);
            dma_untracked<16, true>(wrec, lb + OO + i * 1024, lane * 16, base + R::ot + vblk * R::blk + i * 1024);
        }
        dma_untracked<4, true>(wgc, lb + OG, lane * 4, c * 4);   // gamma_C of chunks c.. (lane 0's is used)
        mem_fence_compiler();
    };

    if (nc > 0) issue(0);
    for (int c = 0; c < nc; ++c) {
        __asm__ __volatile__("s_waitcnt lgkmcnt(0)" ::: "memory");   // reads of the buffer reloaded next
        if (c + 1 < nc) {
            issue(c + 1);
            wait_vmem<NISSUE>();
        } else {
            wait_vmem<0>();
        }
        mem_fence_compiler();
        const unsigned char *buf = smem + (c & 1) * BUF;
        const __bf16 *wi = reinterpret_cast<const __bf16 *>(buf + R::wi);
        const __bf16 *qi = reinterpret_cast<const __bf16 *>(buf + R::qi);
        // O^T tiles as the record holds them (lane: one token, four value
        // columns); U in the other orientation (lane: four tokens 16 m + 4 q4 + e
        // of value column n16), so that it feeds the state update from its
        // accumulators: U~ is read transposed out of the staged record
        f32x4_t U[NB], O[NB];
#pragma unroll
        for (int m = 0; m < NB; ++m) {
            O[m] = *reinterpret_cast<const f32x4_t *>(buf + OO + m * 1024 + lane * 16);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                U[m][e] = *reinterpret_cast<const float *>(buf + OU + m * 1024 + ((n16 >> 2) * 16 + 4 * q4 + e) * 16 +
                                                          (n16 & 3) * 4);
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            float x[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) { x[e] = S[2 * ks][e]; x[4 + e] = S[2 * ks + 1][e]; }
            const frag_t sf = E::pack(x);
#pragma unroll
            for (int m = 0; m < NB; ++m) {
                U[m] = E::mma(E::ld_frag(wi + (16 * m + n16) * L::QP + ks * 32 + 8 * q4), sf, U[m]);
                O[m] = E::mma(sf, E::ld_frag(qi + (16 * m + n16) * L::QP + ks * 32 + 8 * q4), O[m]);
            }
        }
        const int t0 = (p.c0 + c) * C;
#pragma unroll
        for (int m = 0; m < NB; ++m) E::st4(bo, ((t0 + 16 * m + n16) * D + vb + 4 * q4) * 2, O[m]);
        const float gC = *reinterpret_cast<const float *>(buf + OG);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int e = 0; e < 4; ++e) S[mt][e] *= gC;
        // U straight from its accumulators: lane (q4, n16) holds tokens
        // 32 ts + 4 q4 + e and 32 ts + 16 + 4 q4 + e of column n16, and the
        // k^ operand is read in the same token order
#pragma unroll
        for (int ts = 0; ts < TS; ++ts) {
            float x[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) { x[e] = U[2 * ts][e]; x[4 + e] = U[2 * ts + 1][e]; }
            const frag_t uf = E::pack(x);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                S[mt] = E::mma(E::ld_col4x2(buf + R::ki, L::PD, ts * 32 + 4 * q4, ts * 32 + 16 + 4 * q4, 16 * mt, n16),
                               uf, S[mt]);
        }
    }
    if (p.h_final) {
        float *dst = p.h_final + bh * long(D) * D;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int e = 0; e < 4; ++e) dst[(16 * mt + 4 * q4 + e) * D + vb + n16] = S[mt][e];
    }
}

hipError_t launch_gdn(int D, const GdnParams &p, long nbh, hipStream_t s) {
    if (nbh <= 0) return hipSuccess;
    // value blocks of at least 16 columns, a power of two, at most one wave's worth each
    if (p.nvb < 1 || p.nvb > D / 16 || (p.nvb & (p.nvb - 1)) != 0) return hipErrorInvalidValue;
    const dim3 grid(unsigned(nbh), unsigned(p.nvb));
    if (D == 128)
        hipLaunchKernelGGL((gdn_kernel<128, 64, false>), grid, dim3(Shape<128, 64>::NW * 64), 0, s, p);
    else if (D == 64)
        hipLaunchKernelGGL((gdn_kernel<64, 64, false>), grid, dim3(Shape<64, 64>::NW * 64), 0, s, p);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_gdn_prep(int D, const GdnParams &p, int slices, hipStream_t s) {
    if (p.nbh <= 0 || p.nc <= 0) return hipSuccess;
    if (slices < 1 || slices > p.nc || slices > 65535 || !p.ws || !p.ws_gc) return hipErrorInvalidValue;
    const dim3 grid(unsigned(p.nbh), unsigned(slices));
    if (D == 128)
        hipLaunchKernelGGL((gdn_kernel<128, 64, true>), grid, dim3(Shape<128, 64>::NW * 64), 0, s, p);
    else if (D == 64)
        hipLaunchKernelGGL((gdn_kernel<64, 64, true>), grid, dim3(Shape<64, 64>::NW * 64), 0, s, p);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_gdn_walk(int D, const GdnParams &p, hipStream_t s) {
    if (p.nbh <= 0 || p.nc <= 0) return hipSuccess;
    if (!p.ws || !p.ws_gc) return hipErrorInvalidValue;
    // the D / 16 waves of a head on one XCD: 8 x ceil(heads / 8) x (D / 16) work-groups
    const long wgs = 8L * ((p.nbh + 7) / 8) * (D / 16);
    if (wgs > 0x7fffffffL) return hipErrorInvalidValue;
    if (D == 128)
        hipLaunchKernelGGL((gdn_walk_kernel<128, 64>), dim3(unsigned(wgs)), dim3(64), 0, s, p);
    else if (D == 64)
        hipLaunchKernelGGL((gdn_walk_kernel<64, 64>), dim3(unsigned(wgs)), dim3(64), 0, s, p);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace gla
