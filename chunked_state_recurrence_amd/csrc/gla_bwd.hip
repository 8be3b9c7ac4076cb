// gla_bwd.hip — gfx950 kernels for the backward of the chunked
// gated-linear-attention forward (recurrence of gla_kernels.hip).
//
// Loss gradients do = dL/do, dh_final = dL/dh_final.  U_n denotes dL/dS_n,
// the gradient flowing into the state at the start of chunk n from every
// later token (U_N = dh_final).  Reverse-mode of the chunk form, per chunk
// (rows i, j; Gc chunk-local inclusive cumsum of g, Gamma its total):
//
//   U_n   = diag(e^Gamma) U_{n+1} + scale (q e^Gc)^T dO
//   dq_i  = scale e^{Gc_i} * [ do_i S_n^T + sum_{j<=i} (do_i . v_j) k_j e^{-Gc_j} ]
//   dk_j  = sum_{i>=j} scale (do_i . v_j) q_i e^{Gc_i - Gc_j} + e^{Gamma - Gc_j} * (v_j U_{n+1}^T)
//   dv_j  = sum_{i>=j} scale A_ij do_i + (k_j e^{Gamma - Gc_j}) U_{n+1}
//   dg_t  = sum_{t' >= t} (q_t' * dq_t' - k_t' * dk_t')        (log-space gates)
//
// with S_n the forward chunk-start state and A the forward intra-chunk
// scores.  The gate gradient at a chunk start equals sum_v U_n[d, v] S_n[d, v]
// (the gradient of exp(g) at that token times the state it multiplies), so
// inside chunk n dg_t = (sum over the chunk's rows t' >= t of q*dq - k*dk)
// + sum_v U_{n+1} S_{n+1}, and no pass over the whole sequence is needed.
// Expanding S_{n+1} = diag(e^Gamma) S_n + sum_j (k_j e^{Gamma-Gc_j})^T v_j
// turns the last term into e^Gamma * sum_v U_{n+1} S_n + sum_j k_j * dk2_j,
// with dk2_j = e^{Gamma-Gc_j} * (v_j U_{n+1}^T) the state part of dk_j; its
// rows t' >= t cancel against the same part inside the first sum, leaving
//   dg_t = e^Gamma * sum_v U_{n+1} S_n + sum_{t'>=t} (q*dq - k*dk1)_t'
//          + sum_{j<t} k_j * dk2_j,
// dk1 = dk - dk2 the intra-chunk part, which is what is evaluated.  The sources give the forward only (blog "Linear Attention 在 GPU
// 上到底慢在哪", section 学长的反馈; "线性注意力GPU算子库的定义与技术解析",
// sections 四 and 七, which asks for autodiff support); the backward is the
// chain rule of that recurrence.
//
// Likewise the j = i terms of dq and dk, scale (do_i . v_i) k_i and
// scale (do_i . v_i) q_i, cancel exactly in q * dq - k * dk; they are kept
// out of the accumulated sums and added to dq and dk at the end.  Both
// rearrangements matter for strongly decaying gates, where dg is many orders
// of magnitude below the terms that cancel.
//
// Sequence parallelism mirrors the forward in reverse:
//   BM_SEG:  each segment's contribution to U at its start from a zero U at
//            its end, and its total log-decay (segments 1 .. P-1, stored last
//            segment first);
//   scan:    U at every segment end, seeded with dh_final (the forward's scan
//            kernel over the reversed slots);
//   BM_FULL: every segment walks its chunks backwards from its end U, writing
//            dq, dk, dv, dg, and dh0 from the first segment.
// The forward chunk-start states S_n come from the forward output pass.
//
// Work-group = NW waves; wave w owns chunk rows [RPW w, RPW (w+1)) for the
// gate sums, the scaled operand rows and the dq / dk / dg epilogue, and
// columns [VS w, VS (w+1)) of dq, dk, dv and of U (U in MFMA accumulators).
// Chunks whose gates decay by more than 2^kSpanGuard in some key dim take an
// exact path: the scores and the two decayed intra-chunk sums are formed
// elementwise with running products of per-token decays (factors <= 1).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "gla_device.h"
#include "gla_internal.h"

namespace gla {

enum { BM_SEG = 0, BM_FULL = 1 };

template <typename E, int D, int C> struct BwdLayout {
    static constexpr int es = sizeof(typename E::lds_t);
    // row pitches (bytes): bf16 rows padded by 32 bytes for the transposing
    // reads (see E::rowoff), fp32 rows by 16 bytes
    static constexpr int PD = es == 2 ? D * 2 + 32 : D * 4 + 16;   // C x D and D x D tiles
    static constexpr int PC = es == 2 ? C * 2 + 32 : C * 4 + 16;   // C x C tiles
    static constexpr int TD = E::tile_bytes(C, PD);
    static constexpr int TU = E::tile_bytes(D, PD);
    static constexpr int TA = E::tile_bytes(C, PC);
    // operand tiles: scale q e^Gc, k e^-Gc (or k e^{Gamma-Gc}), v, do, U (or
    // e^Gamma U), then scale A and do v^T (rows i, columns j <= i)
    static constexpr int q = 0, k = q + TD, v = k + TD, o = v + TD, u = o + TD, a = u + TU, da = a + TA;
    static constexpr int bytes = da + TA;
    // dq, dk1, dk2 before their row factors, fp32 [C][RP], over the q .. U tiles
    static constexpr int RP = D + 4;
    static_assert(3 * C * RP * 4 <= a, "result tiles must not reach the score tiles");
};

// CPL consecutive values of one row, stored in the element type / fp32
template <typename E, int CPL>
__device__ __forceinline__ void store_row(rsrc_t r, int off, const float *x) {
    if constexpr (std::is_same<E, BF16>::value) {
        if constexpr (CPL == 2) {
            const uint32_t lo = __builtin_bit_cast(uint16_t, (__bf16)x[0]);
            const uint32_t hi = __builtin_bit_cast(uint16_t, (__bf16)x[1]);
            __builtin_amdgcn_raw_buffer_store_b32(lo | (hi << 16), r, off, 0, 0);
        } else {
            __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (__bf16)x[0]), r, off, 0, 0);
        }
    } else {
        if constexpr (CPL == 2)
            __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{__float_as_uint(x[0]), __float_as_uint(x[1])}, r, off, 0, 0);
        else
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x[0]), r, off, 0, 0);
    }
}
template <int CPL>
__device__ __forceinline__ void store_row_f32(rsrc_t r, int off, const float *x) {
    if constexpr (CPL == 2)
        __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{__float_as_uint(x[0]), __float_as_uint(x[1])}, r, off, 0, 0);
    else
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x[0]), r, off, 0, 0);
}

template <typename E, int D, int C, int BM>
__global__ void __launch_bounds__((Shape<D, C>::NW * 64))
bwd_kernel(const BwdParams p) {
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
    static_assert(NTW >= 1 && TS >= 1 && CPL >= 1, "unsupported tile shape");
    constexpr bool kFull = BM == BM_FULL;
    using L = BwdLayout<E, D, C>;
    using lds_t = typename E::lds_t;
    using gmem_t = typename E::gmem_t;
    using frag_t = typename E::frag_t;
    constexpr int es = sizeof(gmem_t);
    static_assert(L::bytes + (3 * NW * D + D + C) * 4 <= 163840, "LDS");

    __shared__ __attribute__((aligned(16))) unsigned char smem[L::bytes];
    __shared__ __attribute__((aligned(16))) float sBt[NW * D];    // wave totals: gates, then q dq - k dk1
    __shared__ __attribute__((aligned(16))) float sXt[NW * D];    // wave totals of k dk2
    __shared__ __attribute__((aligned(16))) float sEG[D];         // exp2(Gamma)
    __shared__ __attribute__((aligned(16))) float sDot[NW * D];   // per-wave parts of e^Gamma sum_v U_{n+1} S_n
    __shared__ __attribute__((aligned(16))) float sDiag[C];       // do_i . v_i
    unsigned char *tQ = smem + L::q;
    unsigned char *tK = smem + L::k;
    unsigned char *tV = smem + L::v;
    unsigned char *tO = smem + L::o;
    unsigned char *tU = smem + L::u;
    unsigned char *tA = smem + L::a;
    unsigned char *tdA = smem + L::da;
    float *rDq = reinterpret_cast<float *>(smem);
    float *rDk1 = rDq + C * L::RP;
    float *rDk2 = rDk1 + C * L::RP;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int n16 = lane & 15;
    const int q4 = lane >> 4;
    const long bhl = blockIdx.y;
    const long bh = p.bh0 + bhl;
    const int T = p.T;
    const int N = p.N;
    // BM_FULL: block x is the segment; BM_SEG: block x is the slot, the
    // segment is counted from the end (slot 0 = last segment)
    const int seg = kFull ? int(blockIdx.x) : p.P - 1 - int(blockIdx.x);
    const int c_begin = seg * p.cps;
    const int c_end = min(N, c_begin + p.cps);
    const int cb = w * VS;        // this wave's first output column
    const int r0 = RPW * w;       // this wave's first chunk row

    const rsrc_t bq = make_rsrc(reinterpret_cast<const gmem_t *>(p.q) + bh * long(T) * D, long(T) * D * es);
    const rsrc_t bk = make_rsrc(reinterpret_cast<const gmem_t *>(p.k) + bh * long(T) * D, long(T) * D * es);
    const rsrc_t bv = make_rsrc(reinterpret_cast<const gmem_t *>(p.v) + bh * long(T) * D, long(T) * D * es);
    const rsrc_t bo = make_rsrc(reinterpret_cast<const gmem_t *>(p.dout) + bh * long(T) * D, long(T) * D * es);
    const rsrc_t bg = make_rsrc(p.g + bh * long(T) * D, long(T) * D * 4);

    // ---- U at the segment end --------------------------------------------
    f32x4_t U[MT][NTW];
    {
        const float *src = nullptr;
        if constexpr (kFull) {
            if (seg == p.P - 1) src = p.dhf ? p.dhf + bh * long(D) * D : nullptr;
            else src = p.ws_E + (bhl * p.ws_slots + (p.P - 2 - seg)) * long(D) * D;
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    U[mt][nt][e] = src ? src[(16 * mt + 4 * q4 + e) * D + cb + 16 * nt + n16] : 0.f;
    }
    // per-wave parts of sum_v U S_c over this wave's columns
    auto dot_us = [&](int c, float *dst) {
        const float *S = p.states + (bh * long(N) + c) * long(D) * D;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float part = 0.f;
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt)
                    part += U[mt][nt][e] * S[(16 * mt + 4 * q4 + e) * D + cb + 16 * nt + n16];
#pragma unroll
                for (int m = 1; m < 16; m <<= 1) part += __shfl_xor(part, m, 64);
                if (n16 == 0) dst[w * D + 16 * mt + 4 * q4 + e] = part;
            }
    };
    if constexpr (kFull) {   // entries above the diagonal of the score tiles are never written
        for (int i = tid; i < 2 * L::TA / 4; i += NW * 64) reinterpret_cast<uint32_t *>(tA)[i] = 0u;
    }
    float seg_gamma[CPL];
#pragma unroll
    for (int u = 0; u < CPL; ++u) seg_gamma[u] = 0.f;

    // row r of a tile
    auto row_ptr = [&](unsigned char *tile, int r, int pitch) {
        return reinterpret_cast<lds_t *>(tile + E::rowoff(r, pitch));
    };

    for (int c = c_end - 1; c >= c_begin; --c) {
        const int t0 = c * C;
        // ---- this chunk's rows: gates, q, k into registers; v, do into LDS ----
        RawG<CPL> rg[RPW];
        Raw<E, CPL> rq[RPW], rk[RPW];
        {
            const int eoff = (t0 + r0) * D + lane * CPL;
#pragma unroll
            for (int i = 0; i < RPW; ++i) {
                rg[i].load(bg, eoff * 4, i * D * 4);
                rq[i].load(bq, eoff * es, i * D * es);
                if constexpr (kFull) rk[i].load(bk, eoff * es, i * D * es);
            }
            const int row0 = __builtin_amdgcn_readfirstlane(t0 + r0);
            const int lr0 = __builtin_amdgcn_readfirstlane(r0);
            mem_fence_compiler();
#pragma unroll
            for (int i = 0; i < RPW; ++i) {
                if constexpr (es == 2) {   // 4 bytes per lane: a 64-wide row takes lanes 0..31
                    if (CPL == 2 || lane < 32) {
                        if constexpr (kFull) dma<4>(bv, tV + E::rowoff(lr0 + i, L::PD), lane * 4, (row0 + i) * D * 2);
                        dma<4>(bo, tO + E::rowoff(lr0 + i, L::PD), lane * 4, (row0 + i) * D * 2);
                    }
                } else {                   // 16 bytes per lane, D / 4 lanes per row
                    if (lane < D / 4) {
                        if constexpr (kFull) dma<16>(bv, tV + E::rowoff(lr0 + i, L::PD), lane * 16, (row0 + i) * D * 4);
                        dma<16>(bo, tO + E::rowoff(lr0 + i, L::PD), lane * 16, (row0 + i) * D * 4);
                    }
                }
            }
            mem_fence_compiler();
            wait_vmem<0>();
        }

        // ---- gate sums (log2 units) over this wave's rows --------------------
        float Pf[RPW][CPL];   // inclusive prefix within the wave's rows
        float Sw[RPW][CPL];   // suffix after the row within the wave's rows
#pragma unroll
        for (int u = 0; u < CPL; ++u) {
            float run = 0.f;
#pragma unroll
            for (int i = 0; i < RPW; ++i) {
                run = __builtin_fmaf(rg[i].get(u), kLog2e, run);
                Pf[i][u] = run;
            }
            float suf = 0.f;
#pragma unroll
            for (int i = RPW - 1; i >= 0; --i) {
                Sw[i][u] = suf;
                suf = __builtin_fmaf(rg[i].get(u), kLog2e, suf);
            }
            sBt[w * D + lane * CPL + u] = run;
        }
        block_sync();  // B1: wave totals and the v / do rows visible

        float rw[CPL], aw[CPL], gam[CPL];   // rows before the wave's, after, all
#pragma unroll
        for (int u = 0; u < CPL; ++u) {
            float before = 0.f, after = 0.f, tot = 0.f;
#pragma unroll
            for (int j = 0; j < NW; ++j) {
                const float b = sBt[j * D + lane * CPL + u];
                if (j < w) before += b;
                if (j > w) after += b;
                tot += b;
            }
            rw[u] = before;
            aw[u] = after;
            gam[u] = tot;
            seg_gamma[u] += tot;
            if (w == 0) sEG[lane * CPL + u] = fexp2(tot);
        }
        bool wide = false;
#pragma unroll
        for (int u = 0; u < CPL; ++u) wide |= -gam[u] > kSpanGuard;
        const bool fast = !kFull || __ballot(wide) == 0;

        // ---- scaled operand rows ---------------------------------------------
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            lds_t *qrow = row_ptr(tQ, r0 + i, L::PD) + lane * CPL;
            lds_t *krow = row_ptr(tK, r0 + i, L::PD) + lane * CPL;
#pragma unroll
            for (int u = 0; u < CPL; ++u) {
                const float gc = rw[u] + Pf[i][u];                      // log2 Gc_i <= 0
                qrow[u] = E::f2l(rq[i].get(u) * (p.scale * fexp2(gc)));  // scale q e^Gc
                if constexpr (kFull) {
                    if (fast) krow[u] = E::f2l(rk[i].get(u) * fexp2(-gc));               // k e^-Gc
                    else krow[u] = E::f2l(rk[i].get(u) * fexp2(aw[u] + Sw[i][u]));     // k e^{Gamma-Gc}
                }
            }
        }
        block_sync();  // B2: exp2(Gamma) visible

        // ---- U tile (U_{n+1}, times e^Gamma on the fast path), then decay U ----
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const f32x4_t egv = *reinterpret_cast<const f32x4_t *>(sEG + 16 * mt + 4 * q4);
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if constexpr (kFull) {
                        const float x = fast ? U[mt][nt][e] * egv[e] : U[mt][nt][e];
                        row_ptr(tU, 16 * mt + 4 * q4 + e, L::PD)[cb + 16 * nt + n16] = E::f2l(x);
                    }
                    U[mt][nt][e] *= egv[e];
                }
        }
        if constexpr (kFull) dot_us(c, sDot);   // e^Gamma sum_v U_{n+1} S_n
        block_sync();  // B3: operand tiles complete

        float dq2x[RPW][CPL], dk1x[RPW][CPL];   // exact path: the decayed intra-chunk sums
        if constexpr (kFull) {
            // ---- do v^T and (fast path) scale A, causal 16x16 tiles -------------
#pragma unroll
            for (int t = 0; t < NTILE; ++t) {
                if (t % NW != w) continue;
                int I = 0, J = t;
#pragma unroll
                for (int r = 0; r < NB; ++r)
                    if (J > r) { J -= r + 1; I = r + 1; }
                f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const int pos = ks * 32 + 8 * q4;
                    acc = E::mma(E::ld_frag(row_ptr(tV, 16 * J + n16, L::PD) + pos),
                                 E::ld_frag(row_ptr(tO, 16 * I + n16, L::PD) + pos), acc);
                }
                f32x4_t aa = {0.f, 0.f, 0.f, 0.f};
                if (fast) {
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {
                        const int pos = ks * 32 + 8 * q4;
                        aa = E::mma(E::ld_frag(row_ptr(tK, 16 * J + n16, L::PD) + pos),
                                    E::ld_frag(row_ptr(tQ, 16 * I + n16, L::PD) + pos), aa);
                    }
                }
                if (I == J) {   // scores keep the diagonal; do v^T keeps j < i only
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        if (4 * q4 + e == n16) sDiag[16 * I + n16] = acc[e];
                        if (4 * q4 + e >= n16) acc[e] = 0.f;
                        if (4 * q4 + e > n16) aa[e] = 0.f;
                    }
                }
                // acc[e] = (do v^T)[16I + n16][16J + 4q4 + e]
                lds_t *da_row = row_ptr(tdA, 16 * I + n16, L::PC) + 16 * J + 4 * q4;
                lds_t *a_row = row_ptr(tA, 16 * I + n16, L::PC) + 16 * J + 4 * q4;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    da_row[e] = E::f2l(acc[e]);
                    if (fast) a_row[e] = E::f2l(aa[e]);
                }
            }
            block_sync();  // B4: do v^T tiles visible

            if (!fast) {
                // exact path, this wave's rows: running products of per-token
                // decays, A_ij = scale sum_d q_i k_j prod_{r=j+1..i} e^{g_r},
                // dq2_i = sum_{j<i} (do_i.v_j) k_j prod(..), dk1_j = sum_{i>j} (do_i.v_j) q_i prod(..)
                // (the do v^T tile is zero on its diagonal)
#pragma unroll
                for (int il = 0; il < RPW; ++il)
#pragma unroll
                    for (int u = 0; u < CPL; ++u) { dq2x[il][u] = 0.f; dk1x[il][u] = 0.f; }
                const int col0 = lane * CPL;
#pragma unroll
                for (int il = 0; il < RPW; ++il) {
                    const int i = r0 + il;
                    float pr[CPL];
#pragma unroll
                    for (int u = 0; u < CPL; ++u) pr[u] = 1.f;
                    for (int j = i; j >= 0; --j) {
                        Raw<E, CPL> kj;
                        RawG<CPL> gj;
                        kj.load(bk, ((t0 + j) * D + col0) * es, 0);
                        gj.load(bg, ((t0 + j) * D + col0) * 4, 0);
                        const float dav = E::l2f(row_ptr(tdA, i, L::PC)[j]);
                        float part = 0.f;
#pragma unroll
                        for (int u = 0; u < CPL; ++u) {
                            const float kd = kj.get(u) * pr[u];
                            part += rq[il].get(u) * kd;
                            dq2x[il][u] += dav * kd;
                            pr[u] *= fexp2(gj.get(u) * kLog2e);
                        }
                        const float s = wave_sum(part) * p.scale;
                        if (lane == 0) row_ptr(tA, i, L::PC)[j] = E::f2l(s);
                    }
#pragma unroll
                    for (int u = 0; u < CPL; ++u) pr[u] = 1.f;
                    for (int i2 = i; i2 < C; ++i2) {   // rows of the chunk at or after row i
                        Raw<E, CPL> qi;
                        qi.load(bq, ((t0 + i2) * D + col0) * es, 0);
                        const float dav = E::l2f(row_ptr(tdA, i2, L::PC)[i]);
#pragma unroll
                        for (int u = 0; u < CPL; ++u) dk1x[il][u] += dav * qi.get(u) * pr[u];
                        if (i2 + 1 < C) {
                            RawG<CPL> gn;
                            gn.load(bg, ((t0 + i2 + 1) * D + col0) * 4, 0);
#pragma unroll
                            for (int u = 0; u < CPL; ++u) pr[u] *= fexp2(gn.get(u) * kLog2e);
                        }
                    }
                }
                block_sync();  // B5: exact scores visible
            }

            // ---- dq, dk, dv column slices of this wave ----------------------------
            f32x4_t Dq[NTW][NB], Dk1[NTW][NB], Dk2[NTW][NB], Dv[NTW][NB];
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
                for (int m = 0; m < NB; ++m) {
                    Dq[nt][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                    Dk1[nt][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                    Dk2[nt][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                    Dv[nt][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                }
            // do S_n^T: S_n rows d of this wave's slice, straight from HBM
            const float *Sn = p.states + (bh * long(N) + c) * long(D) * D;
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const float *src = Sn + (cb + 16 * nt + n16) * D + ks * 32 + 8 * q4;
                    const f32x4_t lo = *reinterpret_cast<const f32x4_t *>(src);
                    const f32x4_t hi = *reinterpret_cast<const f32x4_t *>(src + 4);
                    const float xs[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    const frag_t sf = E::pack(xs);
#pragma unroll
                    for (int m = 0; m < NB; ++m)
                        Dq[nt][m] = E::mma(sf, E::ld_frag(row_ptr(tO, 16 * m + n16, L::PD) + ks * 32 + 8 * q4), Dq[nt][m]);
                }
            // v U^T (U tile rows d along v)
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const frag_t uf = E::ld_frag(row_ptr(tU, cb + 16 * nt + n16, L::PD) + ks * 32 + 8 * q4);
#pragma unroll
                    for (int m = 0; m < NB; ++m)
                        Dk2[nt][m] = E::mma(uf, E::ld_frag(row_ptr(tV, 16 * m + n16, L::PD) + ks * 32 + 8 * q4), Dk2[nt][m]);
                }
            // k~ U~ (or k^ U): U tile columns of this wave along d
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const frag_t uf = E::ld_col8(tU, L::PD, ks * 32 + 8 * q4, cb + 16 * nt, n16);
#pragma unroll
                    for (int m = 0; m < NB; ++m)
                        Dv[nt][m] = E::mma(uf, E::ld_frag(row_ptr(tK, 16 * m + n16, L::PD) + ks * 32 + 8 * q4), Dv[nt][m]);
                }
            // causal intra-chunk terms over 32-deep token steps
#pragma unroll
            for (int m = 0; m < NB; ++m)
#pragma unroll
                for (int ts = 0; ts < TS; ++ts) {
                    const bool lower = ts * 32 <= 16 * m + 15;   // some j <= i in the step (dq)
                    const bool upper = ts * 32 + 31 >= 16 * m;   // some i >= j in the step (dk, dv)
                    if (fast && lower) {   // dq += (do v^T) k e^-Gc
                        const frag_t af = E::ld_frag(row_ptr(tdA, 16 * m + n16, L::PC) + ts * 32 + 8 * q4);
#pragma unroll
                        for (int nt = 0; nt < NTW; ++nt)
                            Dq[nt][m] = E::mma(E::ld_col8(tK, L::PD, ts * 32 + 8 * q4, cb + 16 * nt, n16), af, Dq[nt][m]);
                    }
                    if (upper) {
                        const frag_t at = E::ld_col8(tA, L::PC, ts * 32 + 8 * q4, 16 * m, n16);
                        const frag_t dat = E::ld_col8(tdA, L::PC, ts * 32 + 8 * q4, 16 * m, n16);
#pragma unroll
                        for (int nt = 0; nt < NTW; ++nt) {
                            // dv += (scale A)^T do
                            Dv[nt][m] = E::mma(E::ld_col8(tO, L::PD, ts * 32 + 8 * q4, cb + 16 * nt, n16), at, Dv[nt][m]);
                            // dk += (do v^T)^T scale q e^Gc   (fast path)
                            if (fast)
                                Dk1[nt][m] = E::mma(E::ld_col8(tQ, L::PD, ts * 32 + 8 * q4, cb + 16 * nt, n16), dat, Dk1[nt][m]);
                        }
                    }
                }
            // dv rows straight to HBM (rows past T are dropped)
            const rsrc_t bdv = make_rsrc(reinterpret_cast<gmem_t *>(p.dv) + bh * long(T) * D, long(T) * D * es);
#pragma unroll
            for (int m = 0; m < NB; ++m)
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt)
                    E::st4(bdv, ((t0 + 16 * m + n16) * D + cb + 16 * nt + 4 * q4) * es, Dv[nt][m]);

            // ---- U_n = e^Gamma U_{n+1} + (scale q e^Gc)^T do ------------------------
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int ts = 0; ts < TS; ++ts) {
                    const frag_t a = E::ld_col8(tQ, L::PD, ts * 32 + 8 * q4, 16 * mt, n16);
#pragma unroll
                    for (int nt = 0; nt < NTW; ++nt)
                        U[mt][nt] = E::mma(a, E::ld_col8(tO, L::PD, ts * 32 + 8 * q4, cb + 16 * nt, n16), U[mt][nt]);
                }
            block_sync();  // B6: every wave is done with the operand tiles

            // dq, dk1, dk2 (before their row factors) over the operand tiles
#pragma unroll
            for (int m = 0; m < NB; ++m)
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt) {
                    const int off = (16 * m + n16) * L::RP + cb + 16 * nt + 4 * q4;
                    *reinterpret_cast<f32x4_t *>(rDq + off) = Dq[nt][m];
                    *reinterpret_cast<f32x4_t *>(rDk1 + off) = Dk1[nt][m];
                    *reinterpret_cast<f32x4_t *>(rDk2 + off) = Dk2[nt][m];
                }
            block_sync();  // B7: results visible

            // ---- epilogue on this wave's rows: dq, dk, then dg -------------------
            float dqo[RPW][CPL], dko[RPW][CPL], w1[RPW][CPL], xk[RPW][CPL];
#pragma unroll
            for (int il = 0; il < RPW; ++il) {
                const int i = r0 + il;
                const float dgl = p.scale * sDiag[i];   // scale do_i . v_i
#pragma unroll
                for (int u = 0; u < CPL; ++u) {
                    const int col = lane * CPL + u;
                    const float gc = rw[u] + Pf[il][u];
                    const float dqv = rDq[i * L::RP + col];
                    const float k1v = rDk1[i * L::RP + col], k2v = rDk2[i * L::RP + col];
                    float dk1, dk2;
                    if (fast) {
                        const float ek = fexp2(-gc);
                        dqo[il][u] = p.scale * fexp2(gc) * dqv;
                        dk1 = ek * k1v;
                        dk2 = ek * k2v;
                    } else {
                        dqo[il][u] = p.scale * (fexp2(gc) * dqv + dq2x[il][u]);
                        dk1 = p.scale * dk1x[il][u];
                        dk2 = fexp2(aw[u] + Sw[il][u]) * k2v;
                    }
                    const float qv = rq[il].get(u), kv = rk[il].get(u);
                    w1[il][u] = qv * dqo[il][u] - kv * dk1;
                    xk[il][u] = kv * dk2;
                    // the j = i terms, which cancel in q dq - k dk, added after
                    dqo[il][u] += dgl * kv;
                    dko[il][u] = dk1 + dk2 + dgl * qv;
                }
            }
            // within the wave: rows t' >= t of w1 (inclusive), rows j < t of k dk2
            float dgo[RPW][CPL];
#pragma unroll
            for (int u = 0; u < CPL; ++u) {
                float suf = 0.f, pre = 0.f;
#pragma unroll
                for (int il = RPW - 1; il >= 0; --il) {
                    suf += w1[il][u];
                    dgo[il][u] = suf;
                }
#pragma unroll
                for (int il = 0; il < RPW; ++il) {
                    dgo[il][u] += pre;
                    pre += xk[il][u];
                }
                sBt[w * D + lane * CPL + u] = suf;
                sXt[w * D + lane * CPL + u] = pre;
            }
            block_sync();  // B8: wave totals visible
            float later[CPL];   // later waves' w1, earlier waves' k dk2, the state term
#pragma unroll
            for (int u = 0; u < CPL; ++u) {
                const int col = lane * CPL + u;
                float x = 0.f;
#pragma unroll
                for (int j = 0; j < NW; ++j) {
                    if (j > w) x += sBt[j * D + col];
                    if (j < w) x += sXt[j * D + col];
                    x += sDot[j * D + col];
                }
                later[u] = x;
            }
            const rsrc_t bdq = make_rsrc(reinterpret_cast<gmem_t *>(p.dq) + bh * long(T) * D, long(T) * D * es);
            const rsrc_t bdk = make_rsrc(reinterpret_cast<gmem_t *>(p.dk) + bh * long(T) * D, long(T) * D * es);
            const rsrc_t bdg = make_rsrc(p.dg + bh * long(T) * D, long(T) * D * 4);
#pragma unroll
            for (int il = 0; il < RPW; ++il) {
                const int e0 = (t0 + r0 + il) * D + lane * CPL;
                float dgv[CPL];
#pragma unroll
                for (int u = 0; u < CPL; ++u) dgv[u] = dgo[il][u] + later[u];
                store_row<E, CPL>(bdq, e0 * es, dqo[il]);
                store_row<E, CPL>(bdk, e0 * es, dko[il]);
                store_row_f32<CPL>(bdg, e0 * 4, dgv);
            }
        } else {
            // state units: only U_n = e^Gamma U_{n+1} + (scale q e^Gc)^T do
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int ts = 0; ts < TS; ++ts) {
                    const frag_t a = E::ld_col8(tQ, L::PD, ts * 32 + 8 * q4, 16 * mt, n16);
#pragma unroll
                    for (int nt = 0; nt < NTW; ++nt)
                        U[mt][nt] = E::mma(a, E::ld_col8(tO, L::PD, ts * 32 + 8 * q4, cb + 16 * nt, n16), U[mt][nt]);
                }
        }
        block_sync();  // B9: tiles and totals free for the next chunk
    }

    // ---- segment start ------------------------------------------------------
    float *dst = nullptr;
    if constexpr (kFull) {
        if (seg == 0 && p.dh0) dst = p.dh0 + bh * long(D) * D;
    } else {
        const int slot = int(blockIdx.x);
        dst = p.ws_E + (bhl * p.ws_slots + slot) * long(D) * D;
        if (w == 0)
#pragma unroll
            for (int u = 0; u < CPL; ++u) p.ws_G[(bhl * p.ws_slots + slot) * D + lane * CPL + u] = seg_gamma[u];
    }
    if (dst) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    dst[(16 * mt + 4 * q4 + e) * D + cb + 16 * nt + n16] = U[mt][nt][e];
    }
}

template <typename E, int D, int C>
static hipError_t launch_bwd_t(int bm, const BwdParams &p, int gx, int gy, hipStream_t s) {
    if (gx <= 0 || gy <= 0) return hipSuccess;
    const dim3 block(Shape<D, C>::NW * 64);
    if (bm == BM_SEG) hipLaunchKernelGGL((bwd_kernel<E, D, C, BM_SEG>), dim3(gx, gy), block, 0, s, p);
    else hipLaunchKernelGGL((bwd_kernel<E, D, C, BM_FULL>), dim3(gx, gy), block, 0, s, p);
    return hipGetLastError();
}

hipError_t launch_bwd(int dtype, int D, int C, bool full, const BwdParams &p, int gx, int gy,
                      hipStream_t s) {
    const int bm = full ? BM_FULL : BM_SEG;
    if (dtype == DTYPE_BF16) {
        if (D == 128 && C == 64) return launch_bwd_t<BF16, 128, 64>(bm, p, gx, gy, s);
        if (D == 128 && C == 32) return launch_bwd_t<BF16, 128, 32>(bm, p, gx, gy, s);
        if (D == 64 && C == 64) return launch_bwd_t<BF16, 64, 64>(bm, p, gx, gy, s);
        if (D == 64 && C == 32) return launch_bwd_t<BF16, 64, 32>(bm, p, gx, gy, s);
    } else if (dtype == DTYPE_F32) {
        if (D == 64 && C == 64) return launch_bwd_t<F32, 64, 64>(bm, p, gx, gy, s);
        if (D == 64 && C == 32) return launch_bwd_t<F32, 64, 32>(bm, p, gx, gy, s);
        if (D == 128 && C == 32) return launch_bwd_t<F32, 128, 32>(bm, p, gx, gy, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace gla
