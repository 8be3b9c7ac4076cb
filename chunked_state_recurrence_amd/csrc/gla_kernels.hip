// gla_kernels.hip — gfx950 kernels for the chunked gated-linear-attention
// prefill forward.
//
// Math (per batch row and head): S_t = diag(exp g_t) S_{t-1} + k_t^T v_t,
// o_t = scale q_t S_t (blog "Linear Attention 在 GPU 上到底慢在哪", section
// 学长的反馈; pseudocode of "线性注意力GPU算子库的定义与技术解析", section 四).
// The chunk form follows the GPU flow of that page (section 四, steps 1-3):
// per chunk of C tokens,
//   Gc      = chunk-local inclusive cumsum of g            (stage "cumsum")
//   A[i,j]  = sum_d q_i k_j exp(Gc_i - Gc_j), j <= i        (intra-chunk scores)
//   o_i     = scale (q_i exp(Gc_i)) S_n + scale sum_j A_ij v_j   (output)
//   S_{n+1} = diag(exp Gamma) S_n + (k exp(Gamma - Gc))^T V      (state pass)
// which are the five kernels the blog profiles (section 实验结果, Kernel
// Profiling: cumsum, intra_sub_inter, intra_sub_intra, chunk_fwd_kernel_h,
// chunk_gla_fwd_kernel_o), fused here into one pass per sequence segment.
//
// Sequence parallelism (same page, section 三.1: chunks processed in
// parallel, states merged across them): the T axis is split into P segments.
//   launch 1 (MODE_SEG): each segment's end state from a zero start, E_r,
//                        and its total log-decay;
//   launch 2 (scan):     S_start(r+1) = diag(exp Gamma_r) S_start(r) + E_r;
//   launch 3 (MODE_OUT): every segment replays its chunks from S_start(r),
//                        writing o (and h_final for the last segment).
//
// Work-group = NW waves (8 chunk rows each, 16 when the head dim is 64);
// wave w owns its rows for the gate cumsum and the exponentials, and value
// columns [w*D/NW, (w+1)*D/NW) of the state S and of the output.  S lives in
// MFMA accumulators for a whole segment.  Exponentials use exp2 with
// log2-scaled gates.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>

#include "gla_device.h"
#include "gla_internal.h"

namespace gla {

// LDS carve-up (bytes) per mode; pitches pad rows against bank conflicts.
// bf16 rows are padded by 32 bytes: the MFMA fragment reads (16 rows of a
// tile, four 16-byte groups per row, one group per quarter-wave) then run
// without conflicts on gfx950 (measured with an LDS probe: a 16-byte pad
// costs every 16-byte read a second pass).  Only the tiles a mode uses are
// allocated, so the state-only pass fits several work-groups per CU.
template <typename E, int D, int C, int MODE> struct Layout {
    static constexpr int es = sizeof(typename E::lds_t);
    static constexpr int NW = Shape<D, C>::NW;
    static constexpr int RPW = Shape<D, C>::RPW;
    // gate-sum units: each wave's rows, in pieces of at most 16 (one score block)
    static constexpr int NU = C / (RPW < 16 ? RPW : 16);
    static constexpr bool scores = MODE == MODE_OUT || MODE == MODE_INTRA;
    static constexpr bool state = MODE == MODE_OUT || MODE == MODE_SEG || MODE == MODE_STATES;
    static constexpr bool vreg = MODE == MODE_SEG || MODE == MODE_STATES;   // v^T tile
    // The large tiles (bf16 at C = 128, fp32 at D = 128 and C = 64) fit only
    // with up to three savings: the exact path's block-referenced q^ written
    // over the q tile (the output phase rescales its fragments), the gate rows
    // loaded into registers instead of LDS, and (bf16, D = C = 128) the score
    // tile written over the key tile once every wave has read it.
    static constexpr bool qb_in_qh = C == 128 || (es == 4 && D == 128 && C == 64);
    static constexpr bool greg = (es == 2 && D == 128 && C == 128) || (es == 4 && D == 128 && C == 64);
    static constexpr bool a_in_kt = es == 2 && D == 128 && C == 128;
    static constexpr int PAD = es == 2 ? 32 : 16;   // row pad (bytes)
    static constexpr int QP = D + PAD / es;  // Qh / Kt row pitch (elements)
    static constexpr int TP = C + PAD / es;  // Kht / Vt / A row pitch (elements)
    // output pass: v rows staged row-major by direct loads; bf16 rows padded
    // by 32 bytes so the transposing fragment reads hit distinct banks
    static constexpr int VP = es == 2 ? D * 2 + 32 : D * 4;   // bytes
    // (the direct-load targets, gate rows and output-pass value rows, are
    // arrays of their own)
    static constexpr int qh = 0;
    static constexpr int kt = qh + (scores ? C * QP * es : 0);
    static constexpr int kht = kt + (scores ? C * QP * es : 0);
    static constexpr int vt = kht + (state ? D * TP * es : 0);             // state pass: v^T
    static constexpr int a = vt + (vreg ? D * TP * es : 0);
    static constexpr int qb = a + (MODE == MODE_OUT && !a_in_kt ? C * TP * es : 0);   // exact path: q^ (block references)
    static constexpr int btot = qb + (scores && !qb_in_qh ? C * QP * es : 0);   // float [2][NU][D]
    static constexpr int eg = btot + 2 * NU * D * 4;              // float [D] exp2(Gamma)
    static constexpr int bytes = eg + D * 4;
    static constexpr int aoff = a_in_kt ? kt : a;                  // score tile
    static constexpr int qboff = qb_in_qh ? qh : qb;               // exact path's q^ tile
    static constexpr int gbytes = greg ? 16 : C * D * 4;            // gate rows
    static constexpr int vbytes = MODE == MODE_OUT ? E::tile_bytes(C, VP) : 16;   // output pass: v rows
    static_assert(bytes + gbytes + vbytes <= 163840, "LDS");
};


// The sums over the 64 lanes of eight values part[0..7], one transposing
// butterfly in VALU cross-lane operations (no LDS permutes): at the xor-32,
// -16 and -8 steps each lane keeps the half of its values its lane bit
// selects and adds the partner's copy of them.  A permlane32 (permlane16)
// swap of the two halves' registers exchanges the upper 32 lanes of the
// first with the lower 32 of the second (odd with even 16-lane rows), after
// which the two registers hold exactly the kept values and the partner's
// copy; the xor-8 partner is a DPP rotate by 8 within each row.  Each 8-lane
// group is then summed by DPP (xor 1, xor 2, the mirror within 8 lanes).
// Returns the total of part[t] for t = (lane >> 3) & 7, in every lane.
__device__ __forceinline__ float reduce8(const float (&part)[8], int lane) {
    float r4[4], r2[2];
#pragma unroll
    for (int k2 = 0; k2 < 4; ++k2) {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[k2]), __float_as_uint(part[k2 + 4]),
                                                         false, false);
        r4[k2] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
        const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(r4[k2]), __float_as_uint(r4[k2 + 2]),
                                                         false, false);
        r2[k2] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
    const bool h3 = (lane >> 3) & 1;
    const float keep = h3 ? r2[1] : r2[0];
    const float send = h3 ? r2[0] : r2[1];
    float sum = keep + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(send), 0x128 /* row_ror:8 */,
                                                                  0xf, 0xf, false));
    sum += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(sum), 0xB1 /* quad_perm 1,0,3,2 */, 0xf, 0xf, false));
    sum += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(sum), 0x4E /* quad_perm 2,3,0,1 */, 0xf, 0xf, false));
    sum += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(sum), 0x141 /* row_half_mirror */, 0xf, 0xf, false));
    return sum;
}

// Two ways to form a chunk's scores, chosen per chunk (uniformly over the
// work-group: every wave holds all key dims of the chunk totals):
//  * fast: one reference point at the chunk start, q exp(Gc) and k exp(-Gc),
//    when every key dim decays by at most 2^kSpanGuard over the chunk; the
//    score tiles are then plain MFMA products;
//  * exact: otherwise A[i][j] = sum_d q_i k_j prod_{r=j+1..i} exp(g_r) is
//    formed elementwise from running products of per-token decays (factors
//    in (0, 1], so nothing overflows and underflow is the true value).
// Q and the state-update operand are bounded (exponents <= 0) on both paths.
// SG: scalar gate, g [B,H,T] (one log-decay per token, shared by every key
// dim); each wave stages its rows' gates and reads them back broadcast over
// the key dims, after which the arithmetic is the per-key-dim one.
template <typename E, int D, int C, int MODE, bool SG>
__global__ void __launch_bounds__((Shape<D, C>::NW * 64))
chunk_kernel(const KernelParams p) {
    constexpr int NW = Shape<D, C>::NW;    // waves
    constexpr int RPW = Shape<D, C>::RPW;  // chunk rows per wave
    constexpr int NB = C / 16;             // 16-row token tiles per chunk
    constexpr int CPL = D / 64;            // key/value columns per lane in the row mapping
    constexpr int VS = D / NW;             // value columns per wave
    constexpr int NTW = VS / 16;           // 16-wide value tiles per wave
    constexpr int MT = D / 16;             // 16-row key tiles of S
    constexpr int KS = D / 32;             // 32-deep key steps
    constexpr int TS = C / 32;             // 32-deep token steps
    constexpr int NTILE = NB * (NB + 1) / 2;   // causal 16x16 score tiles
    constexpr int UR = RPW < 16 ? RPW : 16;    // rows per gate-sum unit
    constexpr int NU = C / UR;                 // gate-sum units per chunk
    constexpr int UPW = RPW / UR;              // units per wave (1, or 2 at 32 rows)
    constexpr int UPB = 16 / UR;               // units per 16-row block (2 at 8 rows per wave)
    static_assert(NTW >= 1 && TS >= 1 && CPL >= 1, "unsupported tile shape");
    constexpr bool kOut = MODE == MODE_OUT;
    constexpr bool kSeg = MODE == MODE_SEG;
    constexpr bool kIntra = MODE == MODE_INTRA;
    constexpr bool kCumsum = MODE == MODE_CUMSUM;
    constexpr bool kStates = MODE == MODE_STATES;
    constexpr bool kScores = kOut || kIntra;     // needs the score matrix
    constexpr bool kState = kOut || kSeg || kStates;   // carries S
    constexpr bool kFrom = kOut || kStates;      // S starts from h0 / the scanned segment states
    constexpr bool kEnd = kSeg || kStates;       // update operand k exp(Gamma - Gc) from suffix sums
    using L = Layout<E, D, C, MODE>;
    using lds_t = typename E::lds_t;
    using gmem_t = typename E::gmem_t;
    using frag_t = typename E::frag_t;

    __shared__ __attribute__((aligned(16))) unsigned char smem[L::bytes];
    lds_t *sQh = reinterpret_cast<lds_t *>(smem + L::qh);    // scale q exp(Gc), permuted cols
    lds_t *sKt = reinterpret_cast<lds_t *>(smem + L::kt);    // fast: k exp(-Gc) (permuted); exact: raw k
    lds_t *sKht = reinterpret_cast<lds_t *>(smem + L::kht);  // (k exp(Gamma - Gc))^T
    lds_t *sVt = reinterpret_cast<lds_t *>(smem + L::vt);    // state pass: v^T
    // Direct-load targets in arrays of their own, so the compiler can tell
    // that fragment reads elsewhere do not touch loads still landing here.
    __shared__ __attribute__((aligned(16))) float sG[L::greg ? 4 : (SG ? C : C * D)];   // gate rows
    __shared__ __attribute__((aligned(16))) unsigned char sV[L::vbytes];       // v rows (pitch L::VP)
    lds_t *sA = reinterpret_cast<lds_t *>(smem + L::aoff);   // scaled scores, row-major
    lds_t *sQb = reinterpret_cast<lds_t *>(smem + L::qboff); // exact path: scale q exp(Gc - r_block), permuted cols
    float *sBtot = reinterpret_cast<float *>(smem + L::btot);
    float *sEG = reinterpret_cast<float *>(smem + L::eg);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int n16 = lane & 15;
    const int q4 = lane >> 4;
    const int seg = blockIdx.x;
    const long bhl = blockIdx.y;               // index inside this launch's head group
    const long bh = p.bh0 + bhl;               // absolute (batch, head) row
    const int T = p.T;
    const int c_begin = seg * p.cps;
    const int c_end = min(p.N, c_begin + p.cps);
    const int vb = w * VS;                     // this wave's first value column
    const int r0 = RPW * w;                    // this wave's first chunk row

    const gmem_t *gq = reinterpret_cast<const gmem_t *>(p.q) + bh * long(T) * D;
    const gmem_t *gk = reinterpret_cast<const gmem_t *>(p.k) + bh * long(T) * D;
    const gmem_t *gv = reinterpret_cast<const gmem_t *>(p.v) + bh * long(T) * D;
    constexpr int GD = SG ? 1 : D;            // gates per token
    const float *gg = p.g + bh * long(T) * GD;

    // ---- state init ---------------------------------------------------------
    f32x4_t S[MT][NTW];
    if constexpr (kState) {
        const float *src = nullptr;
        if constexpr (kFrom) {
            if (seg == 0) src = p.h0 ? p.h0 + bh * D * D : nullptr;
            else src = p.ws_E + (bhl * p.ws_slots + seg * p.sub - 1) * long(D) * D;
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    S[mt][nt][e] = src ? src[(16 * mt + 4 * q4 + e) * D + vb + 16 * nt + n16] : 0.f;
    }
    if constexpr (kOut) {  // entries above the diagonal of A are never written: zero them once
        for (int i = tid; i < C * L::TP; i += NW * 64) sA[i] = E::f2l(0.f);
    }
    float seg_gamma[CPL];
#pragma unroll
    for (int u = 0; u < CPL; ++u) seg_gamma[u] = 0.f;

    // ---- raw rows of the current chunk (this wave's RPW rows, CPL columns) --
    constexpr bool kVreg = kEnd;   // v through registers into v^T (state-only passes)
    constexpr bool kVdma = kOut;   // v straight into LDS rows (output pass)
    Raw<E, CPL> rq[RPW], rk[RPW], rv[RPW];
    constexpr int es = sizeof(gmem_t);
    const rsrc_t bq = make_rsrc(gq, long(T) * D * es);
    const rsrc_t bk = make_rsrc(gk, long(T) * D * es);
    const rsrc_t bv = make_rsrc(gv, long(T) * D * es);
    const rsrc_t bg = make_rsrc(gg, long(T) * GD * 4);
    // Issue counts per wave, for the explicit waits: gate rows (direct, 1 KB
    // per load; one load of RPW floats for scalar gates), register rows of
    // q / k (/ v in the state pass), v rows.
    constexpr int NG = L::greg ? RPW : (SG ? 1 : RPW * D * 4 / 1024);
    constexpr int NQK = (kScores ? RPW : 0) + (kCumsum ? 0 : RPW) + (kVreg ? RPW : 0);
    constexpr int NV = !kVdma ? 0 : (es == 2 ? RPW : RPW * D * 4 / 1024);
    static_assert(RPW * D * 4 % 1024 == 0, "gate rows per wave must fill whole loads");
    // this wave's gate rows of chunk c into its rows of sG, or into registers
    // (rows past T read 0)
    RawG<CPL> rgn[RPW];
    auto load_g = [&](int c) {
        if constexpr (L::greg) {
#pragma unroll
            for (int i = 0; i < RPW; ++i) {
                if constexpr (SG) rgn[i].load_one(bg, (c * C + r0) * 4, i * 4);
                else rgn[i].load(bg, ((c * C + r0) * D + lane * CPL) * 4, i * D * 4);
            }
            mem_fence_compiler();
        } else {
            const int rbase = __builtin_amdgcn_readfirstlane((c * C + r0) * GD * 4);
            float *dst = sG + __builtin_amdgcn_readfirstlane(r0 * GD);
            mem_fence_compiler();
            if constexpr (SG) {
                if (lane < RPW) dma<4>(bg, reinterpret_cast<unsigned char *>(dst), lane * 4, rbase);
            } else {
#pragma unroll
                for (int i = 0; i < NG; ++i)
                    dma<16>(bg, reinterpret_cast<unsigned char *>(dst) + i * 1024, lane * 16, rbase + i * 1024);
            }
            mem_fence_compiler();
        }
    };
    // rows past T read as zero; row offsets go in the uniform soffset
    auto load_qkv = [&](int c) {
        const int eoff = (c * C + r0) * D + lane * CPL;
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            if constexpr (kScores) rq[i].load(bq, eoff * es, i * D * es);
            if constexpr (!kCumsum) rk[i].load(bk, eoff * es, i * D * es);
            if constexpr (kVreg) rv[i].load(bv, eoff * es, i * D * es);
        }
        mem_fence_compiler();
    };
    // this wave's v rows of chunk c into sV
    auto load_v = [&](int c) {
        if constexpr (kVdma) {
            const int row0 = __builtin_amdgcn_readfirstlane(c * C + r0);
            const int lr0 = __builtin_amdgcn_readfirstlane(r0);
            if constexpr (es == 2) {   // one load per row, padded pitch; 4 bytes per lane
                // (narrower direct loads still occupy 4 bytes of LDS per lane), so
                // a 64-wide row takes lanes 0..31 only
#pragma unroll
                for (int i = 0; i < RPW; ++i)
                    if (CPL == 2 || lane < 32) dma<4>(bv, sV + E::rowoff(lr0 + i, L::VP), lane * 4, (row0 + i) * D * 2);
            } else {                   // dense rows, 1 KB per load
#pragma unroll
                for (int i = 0; i < NV; ++i)
                    dma<16>(bv, sV + lr0 * L::VP + i * 1024, lane * 16, row0 * D * 4 + i * 1024);
            }
            mem_fence_compiler();
        }
    };
    if (c_begin < c_end) {
        load_g(c_begin);
        load_qkv(c_begin);
        load_v(c_begin);
    }

    // RPW consecutive tokens of column `col` into a transposed tile
    auto store_col = [&](lds_t *tile, int col, const float *x) {
#pragma unroll
        for (int h = 0; h < RPW / 8; ++h) E::st_frag(tile + col * L::TP + r0 + 8 * h, E::pack(x + 8 * h));
    };
    auto store_v_cols = [&]() {
#pragma unroll
        for (int u = 0; u < CPL; ++u)
#pragma unroll
            for (int h = 0; h < RPW / 8; ++h)
                E::st_frag(sVt + (lane * CPL + u) * L::TP + r0 + 8 * h, Raw<E, CPL>::col8(rv + 8 * h, u));
    };
    auto store_row = [&](lds_t *tile, int row, const float *x) {   // permuted columns
        const int pc = perm_col(lane * CPL);
        if constexpr (CPL == 2) {
            typedef lds_t l2_t __attribute__((ext_vector_type(2)));
            l2_t a;
            a[0] = E::f2l(x[0]);
            a[1] = E::f2l(x[1]);
            *reinterpret_cast<l2_t *>(tile + row * L::QP + pc) = a;
        } else {
            tile[row * L::QP + pc] = E::f2l(x[0]);
        }
    };
    auto sink_tile = [&](int c, int I, int J, f32x4_t acc) {
        // acc[e] = A[16I + n16][16J + 4q4 + e]
        if constexpr (kOut) {
            typedef lds_t l4_t __attribute__((ext_vector_type(4)));
            l4_t v4;
#pragma unroll
            for (int e = 0; e < 4; ++e) v4[e] = E::f2l(acc[e]);
            *reinterpret_cast<l4_t *>(sA + (16 * I + n16) * L::TP + 16 * J + 4 * q4) = v4;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                p.dump[((bh * long(p.N) + c) * C + 16 * I + n16) * C + 16 * J + 4 * q4 + e] = acc[e];
        }
    };

    // chunk c's start state S into `dump` (fp32, row-major D x D per chunk)
    // or, states-only mode, `dump16` (bf16 in 16 x 16 tiles, the layout of
    // bf16_state_offset: a 4 x 4 transpose within each lane quad (DPP) gives
    // a lane four consecutive columns of one row, so a wave stores a whole
    // 512-byte tile with one 8-byte store per lane)
    auto dump_start = [&](int c) {
        if (p.dump) {
            float *dst = p.dump + (bh * long(p.N) + c) * long(D) * D;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        dst[(16 * mt + 4 * q4 + e) * D + vb + 16 * nt + n16] = S[mt][nt][e];
        } else if (kStates && p.dump16) {
            unsigned char *dst = static_cast<unsigned char *>(p.dump16) + (bh * long(p.N) + c) * long(D) * D * 2;
            const int j = n16 & 3;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt) {
                    float x[4] = {S[mt][nt][0], S[mt][nt][1], S[mt][nt][2], S[mt][nt][3]};
                    quad_transpose4(x, j);
                    // x[b] = S[16 mt + 4 q4 + j][vb + 16 nt + 4 (n16 / 4) + b]
                    const uint32_t lo = pack_bf16x2(x[0], x[1]), hi = pack_bf16x2(x[2], x[3]);
                    *reinterpret_cast<u32x2_t *>(dst + 2 * bf16_state_offset<D>(16 * mt + 4 * q4 + j, vb + 16 * nt + 4 * (n16 >> 2))) =
                        u32x2_t{lo, hi};
                }
        }
    };

    int buf = 0;
    for (int c = c_begin; c < c_end; ++c) {
        const int t0 = c * C;
        // ---- a1: gate cumsum (log2 units) over this wave's RPW rows.  Every
        // exponent formed below is a sum of gates of one sign (a prefix, a
        // suffix, a run of wave totals), never a difference of two prefix
        // sums, so huge gates cannot cancel into large exponent errors.
        // The next chunk's loads are issued on every chunk (the last one
        // reloads its own rows), so each wait below counts the same loads on
        // every path.
        const int cn = min(c + 1, c_end - 1);
        // this wave's gate rows arrived (loads after them: q / k / v rows)
        wait_vmem<NQK + NV>();
        RawG<CPL> rg[RPW];   // each wave reads back only the rows it loaded itself
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            if constexpr (L::greg) rg[i] = rgn[i];
            else if constexpr (SG) rg[i].fill(sG[r0 + i]);
            else rg[i].x = *reinterpret_cast<const decltype(rg[i].x) *>(sG + (r0 + i) * D + lane * CPL);
        }
        float Pf[RPW][CPL];   // inclusive prefix within the wave's rows
        float Pu[UPW > 1 ? RPW : 1][CPL];   // 32-row waves: inclusive prefix within the row's unit
        float Sw[RPW][CPL];   // state pass: suffix after the row within the wave's rows
#pragma unroll
        for (int u = 0; u < CPL; ++u) {
            float run = 0.f, urun = 0.f;
#pragma unroll
            for (int i = 0; i < RPW; ++i) {
                run = __builtin_fmaf(rg[i].get(u), kLog2e, run);
                Pf[i][u] = run;
                if constexpr (UPW > 1) {   // each unit's total goes to its own slot
                    urun = __builtin_fmaf(rg[i].get(u), kLog2e, i % UR == 0 ? 0.f : urun);
                    Pu[i][u] = urun;
                    if (i % UR == UR - 1) sBtot[(buf * NU + w * UPW + i / UR) * D + lane * CPL + u] = urun;
                }
            }
            if constexpr (kEnd) {
                float suf = 0.f;
#pragma unroll
                for (int i = RPW - 1; i >= 0; --i) {
                    Sw[i][u] = suf;
                    suf = __builtin_fmaf(rg[i].get(u), kLog2e, suf);
                }
            }
            if constexpr (UPW == 1) sBtot[(buf * NU + w) * D + lane * CPL + u] = run;
        }
        // the gates are in registers: the next chunk's gate rows load during
        // the rest of this chunk (gate rows into registers wait for the q / k
        // prefetch below, which keeps them out of the operand phase's registers)
        if constexpr (!kCumsum && !L::greg) load_g(cn);
        block_sync();  // B1: wave totals visible

        // rows before the wave's, after them, all: before and all from one
        // running sum over the wave totals (the same additions in the same
        // order as separate sums); after, a sum of its own, is formed only
        // where it is used (the state-only pass here, the exact path below)
        float rw[CPL], aw[CPL], gam[CPL];
        auto rows_after = [&](int u) {
            float after = 0.f;
#pragma unroll
            for (int j = 0; j < NU; ++j)
                if (j >= (w + 1) * UPW) after += sBtot[(buf * NU + j) * D + lane * CPL + u];
            return after;
        };
#pragma unroll
        for (int u = 0; u < CPL; ++u) {
            float pre = 0.f, before = 0.f;
#pragma unroll
            for (int j = 0; j < NU; ++j) {
                if (j == w * UPW) before = pre;
                pre += sBtot[(buf * NU + j) * D + lane * CPL + u];
            }
            rw[u] = before;
            gam[u] = pre;
            if constexpr (!kScores) aw[u] = rows_after(u);
        }

        if constexpr (kCumsum) {
#pragma unroll
            for (int i = 0; i < RPW; ++i) {
                const int t = t0 + r0 + i;
                if (t < T)
#pragma unroll
                    for (int u = 0; u < CPL; ++u)
                        p.dump[(bh * long(T) + t) * D + lane * CPL + u] = (rw[u] + Pf[i][u]) * kLn2;
            }
            if (w == 0)
#pragma unroll
                for (int u = 0; u < CPL; ++u)
                    p.dump2[(bh * long(p.N) + c) * D + lane * CPL + u] = gam[u] * kLn2;
            load_g(cn);
            buf ^= 1;
            continue;
        }

        // fast path unless some key dim decays by more than 2^kSpanGuard
        bool wide = false;
#pragma unroll
        for (int u = 0; u < CPL; ++u) wide |= -gam[u] > kSpanGuard;
        const bool fast = __ballot(wide) == 0;

        // exact path: the chunk's 16-row blocks.  Wave w's rows lie in block
        // w / WPB; the block's waves before / after it contribute gate sums
        // (log2) to the block-referenced exponents below.
        constexpr int WPB = RPW < 16 ? 16 / RPW : 1;   // waves per 16-row block
        constexpr int BPW = RPW > 16 ? RPW / 16 : 1;   // 16-row blocks per wave
        const int hw = w % WPB;         // this wave's place in its block
        // per-block sums of the chunk's gates (log2), B_K = sum of the units of
        // block K, for key dims d0..d0+3 (f32x4)
        auto blk4 = [&](int K, int d0) {
            f32x4_t t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < UPB; ++j)
                t += *reinterpret_cast<const f32x4_t *>(sBtot + (buf * NU + K * UPB + j) * D + d0);
            return t;
        };
        // ---- operand tiles into LDS -----------------------------------------
        float eg[CPL];
#pragma unroll
        for (int u = 0; u < CPL; ++u) {
            eg[u] = fexp2(gam[u]);
            if constexpr (kState) if (w == 0) sEG[lane * CPL + u] = eg[u];
        }
        if constexpr (kScores) {
            float kh[CPL][RPW];
            float kb_[RPW][CPL];   // exact path: k^_j (block-end reference)
            if (fast) {
#pragma unroll
                for (int i = 0; i < RPW; ++i) {
                    float qh[CPL], kt[CPL];
#pragma unroll
                    for (int u = 0; u < CPL; ++u) {
                        const float t = rw[u] + Pf[i][u];           // Gc_i in [-kSpanGuard, 0]
                        qh[u] = rq[i].get(u) * (p.scale * fexp2(t)); // scale q exp(Gc)
                        kt[u] = rk[i].get(u) * fexp2(-t);            // k exp(-Gc)
                        kh[u][i] = kt[u] * eg[u];                    // k exp(Gamma - Gc)
                    }
                    store_row(sQh, r0 + i, qh);
                    store_row(sKt, r0 + i, kt);
                }
            } else {
                // Sub-block references (every factor <= 1): per 16-row block I,
                // r_I = Gc at the row before the block, and per row
                //   q^_i = scale q_i exp2(Gc_i - r_I)     (tile sQb, permuted),
                //   k^_j = k_j exp2(r_{J+1} - Gc_j)       (tile sKt, permuted),
                // so a score tile (I, J) is q^_I diag(exp2(r_I - r_{J+1})) k^_J^T;
                // the inter-chunk term and the state update keep the chunk-start
                // and chunk-end references (sQh, sKht), which are <= 1 for any gates.
                // Exponents are sums of gates of one sign, never differences.
                float bef[CPL], aft[CPL];   // gates of the block's rows before / after this wave's
#pragma unroll
                for (int u = 0; u < CPL; ++u) {
                    bef[u] = 0.f;
                    aft[u] = 0.f;
#pragma unroll
                    for (int j = 0; j < WPB; ++j) {
                        const float t = sBtot[(buf * NU + (w - hw + j)) * D + lane * CPL + u];
                        if (j < hw) bef[u] += t;
                        if (j > hw) aft[u] += t;
                    }
                    aw[u] = rows_after(u);
                }
#pragma unroll
                for (int u = 0; u < CPL; ++u) {
                    float suf = aw[u], sufb = aft[u];   // rows after i: in the chunk / in the block
#pragma unroll
                    for (int i = RPW - 1; i >= 0; --i) {
                        if constexpr (UPW > 1)   // a unit's rows see only the gates after them in the unit
                            if (i % UR == UR - 1) sufb = 0.f;
                        kh[u][i] = rk[i].get(u) * fexp2(suf);
                        kb_[i][u] = rk[i].get(u) * fexp2(sufb);
                        const float gl = rg[i].get(u) * kLog2e;
                        suf += gl;
                        sufb += gl;
                    }
                }
#pragma unroll
                for (int i = 0; i < RPW; ++i) {
                    float qh[CPL], qb[CPL];
#pragma unroll
                    for (int u = 0; u < CPL; ++u) {
                        qh[u] = rq[i].get(u) * (p.scale * fexp2(rw[u] + Pf[i][u]));
                        qb[u] = rq[i].get(u) * (p.scale * fexp2(bef[u] + (UPW > 1 ? Pu[i][u] : Pf[i][u])));
                    }
                    if constexpr (!L::qb_in_qh) store_row(sQh, r0 + i, qh);
                    store_row(sQb, r0 + i, qb);   // over the q tile when qb_in_qh
                    store_row(sKt, r0 + i, kb_[i]);
                }
            }
            if constexpr (kOut) {
#pragma unroll
                for (int u = 0; u < CPL; ++u) store_col(sKht, lane * CPL + u, kh[u]);
            }
        }
        if constexpr (kEnd) {
#pragma unroll
            for (int u = 0; u < CPL; ++u) {
                float kk[RPW];
#pragma unroll
                for (int i = 0; i < RPW; ++i)   // k exp(Gamma - Gc_i): two sums of gates <= 0
                    kk[i] = rk[i].get(u) * fexp2(aw[u] + Sw[i][u]);
                store_col(sKht, lane * CPL + u, kk);
            }
            store_v_cols();
        }
#pragma unroll
        for (int u = 0; u < CPL; ++u) seg_gamma[u] += gam[u];

        // prefetch the next chunk's gates (score modes) and q / k rows; the
        // loads fly during the matrix work below
        load_qkv(cn);
        if constexpr (L::greg && !kCumsum) load_g(cn);
        if constexpr (kVdma) wait_vmem<NG + NQK>();   // this chunk's v rows arrived (loads after them: next gates, q, k)
        block_sync();  // B2: operand tiles visible

        // ---- a2: causal score tiles -------------------------------------------
        // With the score tile over the key tile, a wave holds its tiles in
        // registers until every wave has read the key tile, then stores them
        // with zero tiles right of the even diagonal tiles (the output phase's
        // 32-deep token steps read those, and key rows are still there).
        constexpr bool kHold = kOut && L::a_in_kt;
        constexpr int MAXT = (NTILE + NW - 1) / NW;   // tiles per wave, at most
        // body(slot, I, J) for this wave's tiles t = w, w + NW, ... (tile t is
        // (I, J) in row-major order of the lower triangle).  Up to 10 tiles the
        // loop runs over all of them with constant indices; the 36 tiles of a
        // 128-token chunk would then put 36 tile bodies in every wave's code,
        // so each wave walks only its own slots there.
        auto for_my_tiles = [&](auto &&body) {
            if constexpr (NB <= 4) {
#pragma unroll
                for (int t = 0; t < NTILE; ++t) {
                    if (t % NW != w) continue;
                    int I = 0, J = t;
#pragma unroll
                    for (int r = 0; r < NB; ++r)
                        if (J > r) { J -= r + 1; I = r + 1; }
                    body(t / NW, I, J);
                }
            } else {
#pragma unroll
                for (int sl = 0; sl < MAXT; ++sl) {
                    const int t = w + sl * NW;
                    if (t >= NTILE) break;
                    int I = 0, J = t;
#pragma unroll
                    for (int r = 0; r < NB; ++r)
                        if (J > r) { J -= r + 1; I = r + 1; }
                    body(sl, I, J);
                }
            }
        };
        f32x4_t held[kHold ? MAXT : 1];
        auto put_tile = [&](int slot, int I, int J, f32x4_t acc) {
            if constexpr (kHold) held[slot] = acc;
            else sink_tile(c, I, J, acc);
        };
        auto flush_tiles = [&](unsigned diag_done) {
            if constexpr (kHold) {
                block_sync();   // every wave is done with the key tile
                for_my_tiles([&](int slot, int I, int J) {
                    if (I == J && !((diag_done >> I) & 1u)) return;
                    sink_tile(c, I, J, held[slot]);
                });
#pragma unroll
                for (int I = 0; I + 1 < NB; I += 2)
                    if ((I * NB + I + 1) % NW == w) sink_tile(c, I, I + 1, f32x4_t{0.f, 0.f, 0.f, 0.f});
            }
        };
        if constexpr (kScores) {
            if (fast) {
                // tile (I, J) = Kt[J] Qh[I]^T; tiles dealt round-robin to the waves
                for_my_tiles([&](int slot, int I, int J) {
                    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {
                        const int pos = ks * 32 + 8 * q4;
                        acc = E::mma(E::ld_frag(sKt + (16 * J + n16) * L::QP + pos),
                                     E::ld_frag(sQh + (16 * I + n16) * L::QP + pos), acc);
                    }
                    if (I == J) {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (4 * q4 + e > n16) acc[e] = 0.f;
                    }
                    put_tile(slot, I, J, acc);
                });
                flush_tiles(~0u);
                if constexpr (kIntra) {  // zero tiles above the diagonal
#pragma unroll
                    for (int I = 0; I < NB; ++I)
#pragma unroll
                        for (int J = I + 1; J < NB; ++J)
                            if ((I * NB + J) % NW == w) sink_tile(c, I, J, f32x4_t{0.f, 0.f, 0.f, 0.f});
                }
            } else {
                // Diagonal blocks whose own span stays within the guard in every
                // key dim take the MFMA form too (one bit per block, the same in
                // every wave); the others are formed elementwise by their rows' waves.
                unsigned diag_mma = 0;
#pragma unroll
                for (int I = 0; I < NB; ++I) {
                    bool wide_blk = false;
#pragma unroll
                    for (int u = 0; u < CPL; ++u) {
                        float t = 0.f;
#pragma unroll
                        for (int j = 0; j < UPB; ++j) t += sBtot[(buf * NU + I * UPB + j) * D + lane * CPL + u];
                        wide_blk |= -t > kSpanGuard;
                    }
                    if (__ballot(wide_blk) == 0) diag_mma |= 1u << I;
                }
                // tile (I, J) = k^_J diag(m) q^_I^T with m = exp2(r_I - r_{J+1}) per key
                // dim: 1 for I = J + 1, the gates of blocks J+1 .. I-1 (<= 1) further
                // below, exp2(-B_I) (<= 2^kSpanGuard) on the diagonal; m scales the
                // k^ fragment (its 8 positions are key dims d0..d0+3, d0+16..d0+19)
                for_my_tiles([&](int slot, int I, int J) {
                    if (I == J && !((diag_mma >> I) & 1u)) return;
                    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {
                        const int pos = ks * 32 + 8 * q4;
                        frag_t kf = E::ld_frag(sKt + (16 * J + n16) * L::QP + pos);
                        if (I != J + 1) {
                            const int d0 = ks * 32 + 4 * q4;
                            f32x4_t x0 = {0.f, 0.f, 0.f, 0.f}, x1 = {0.f, 0.f, 0.f, 0.f};
                            if (I == J) {
                                x0 = -blk4(I, d0);
                                x1 = -blk4(I, d0 + 16);
                            } else {
                                for (int K = J + 1; K < I; ++K) {
                                    x0 += blk4(K, d0);
                                    x1 += blk4(K, d0 + 16);
                                }
                            }
                            float kv[8];
                            E::unpack(kf, kv);
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                kv[e] *= fexp2(x0[e]);
                                kv[4 + e] *= fexp2(x1[e]);
                            }
                            kf = E::pack(kv);
                        }
                        acc = E::mma(kf, E::ld_frag(sQb + (16 * I + n16) * L::QP + pos), acc);
                    }
                    if (I == J) {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (4 * q4 + e > n16) acc[e] = 0.f;
                    }
                    put_tile(slot, I, J, acc);
                });
                flush_tiles(diag_mma);
                if constexpr (kIntra) {  // zero tiles above the diagonal
#pragma unroll
                    for (int I = 0; I < NB; ++I)
#pragma unroll
                        for (int J = I + 1; J < NB; ++J)
                            if ((I * NB + J) % NW == w) sink_tile(c, I, J, f32x4_t{0.f, 0.f, 0.f, 0.f});
                }
                // The wave's block, elementwise, when its span passes the guard:
                // A_ij = sum_d q_i k_j prod_{r=j+1..i} exp(g_r) for columns j of
                // the block up to i, from the raw rows of the block (re-read from
                // the cache; rows past T read 0) with running products of
                // per-token decays (factors in (0, 1]).  The block's waves take
                // its rows in turn (row li to wave li % WPB), which evens out
                // their column counts; each wave's rows are unrolled so that
                // every column bound is a constant.  (A 32-row wave takes its two
                // blocks in turn.)
                constexpr int RIB = 16 / WPB;   // rows of the block per wave
#pragma unroll 1
                for (int bb = 0; bb < BPW; ++bb) {
                const int Iw = (w * RPW) / 16 + bb;
                const int rb = 16 * Iw;   // the block's first chunk row
                if (!((diag_mma >> Iw) & 1u)) {
                    Raw<E, CPL> kr[16], qr[RIB];
                    RawG<CPL> gr[16];
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        kr[r].load(bk, ((c * C + rb + r) * D + lane * CPL) * es, 0);
                        if constexpr (SG) gr[r].load_one(bg, (c * C + rb + r) * 4, 0);
                        else gr[r].load(bg, ((c * C + rb + r) * D + lane * CPL) * 4, 0);
                    }
#pragma unroll
                    for (int il = 0; il < RIB; ++il)
                        qr[il].load(bq, ((c * C + rb + hw + WPB * il) * D + lane * CPL) * es, 0);
                    float dc[16][CPL];
#pragma unroll
                    for (int r = 0; r < 16; ++r)
#pragma unroll
                        for (int u = 0; u < CPL; ++u) dc[r][u] = fexp2(gr[r].get(u) * kLog2e);
                    auto rows = [&](auto hc) {
                        constexpr int HW = decltype(hc)::value;
#pragma unroll
                        for (int il = 0; il < RIB; ++il) {
                            const int li = HW + WPB * il;   // row within the block
                            const int i = rb + li;
                            float qp[CPL];   // q_i times the running decay product
#pragma unroll
                            for (int u = 0; u < CPL; ++u) qp[u] = qr[il].get(u);
                            // columns jl = li .. 0 in two groups of 8, group g holding
                            // columns 15 - 8 g - t (t = 0..7); rows in the block's
                            // first half have no column in group 0, and once every
                            // q-scaled running product has underflowed to 0 the rest
                            // of the row is exactly 0.  A group's columns past li
                            // sum to 0, the value those causal-mask entries hold, so
                            // every lane stores (the 8 lanes of a column the same value)
                            auto emit = [&](int g2, float sum) {
                                const int jl = 15 - 8 * g2 - (lane >> 3);
                                const float sc = sum * p.scale;
                                if constexpr (kOut) sA[i * L::TP + rb + jl] = E::f2l(sc);
                                else p.dump[((bh * long(p.N) + c) * C + i) * C + rb + jl] = sc;
                            };
                            auto run_group = [&](auto gc) {
                                constexpr int G2 = decltype(gc)::value;
                                float part[8];
#pragma unroll
                                for (int t = 0; t < 8; ++t) {
                                    const int jl = 15 - 8 * G2 - t;
                                    part[t] = 0.f;
                                    if (jl <= li) {
#pragma unroll
                                        for (int u = 0; u < CPL; ++u) {
                                            part[t] = __builtin_fmaf(qp[u], kr[jl].get(u), part[t]);
                                            qp[u] *= dc[jl][u];   // times exp(g_jl): the factor for column jl-1
                                        }
                                    }
                                }
                                emit(G2, reduce8(part, lane));
                            };
                            bool live = true;
                            if (li < 8) {
                                // the block's columns 8..15 lie right of the diagonal: zero,
                                // which the key tile's rows under the score tile are not
                                if constexpr (kHold) emit(0, 0.f);
                            } else {
                                run_group(std::integral_constant<int, 0>{});
                                bool any = false;
#pragma unroll
                                for (int u = 0; u < CPL; ++u) any |= qp[u] != 0.f;
                                live = __ballot(any) != 0;
                            }
                            if (live) run_group(std::integral_constant<int, 1>{});
                            else emit(1, 0.f);
                            if constexpr (kIntra) {
                                for (int j = i + 1 + lane; j < C; j += 64)
                                    if (j < rb + 16) p.dump[((bh * long(p.N) + c) * C + i) * C + j] = 0.f;
                            }
                        }
                    };
                    if (WPB == 1 || hw == 0) rows(std::integral_constant<int, 0>{});
                    else rows(std::integral_constant<int, WPB - 1>{});
                }
                }
            }
        }
        if constexpr (kIntra) {
            buf ^= 1;
            block_sync();  // LDS reuse by the next chunk
            continue;
        }

        frag_t vf[NTW][TS];
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
            for (int ts = 0; ts < TS; ++ts)
                if constexpr (kVdma) vf[nt][ts] = E::ld_col8(sV, L::VP, ts * 32 + 8 * q4, vb + 16 * nt, n16);
                else vf[nt][ts] = E::ld_frag(sVt + (vb + 16 * nt + n16) * L::TP + ts * 32 + 8 * q4);

        if constexpr (kStates) dump_start(c);
        if constexpr (kOut) {
            block_sync();  // B3: score tiles visible
            dump_start(c);   // chunk-start states, when asked for (stage output)
            // every wave holds its v fragments: the next chunk's v rows may land
            load_v(cn);
            // ---- a4: O^T tiles (value tile nt, token tile m) ---------------------
            f32x4_t O[NTW][NB];
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
                for (int m = 0; m < NB; ++m) O[nt][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            // inter-chunk: O^T += S^T (scale q exp Gc)^T, S straight from its accumulators
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
                if (!L::qb_in_qh || fast) {
#pragma unroll
                    for (int m = 0; m < NB; ++m) {
                        const frag_t b = E::ld_frag(sQh + (16 * m + n16) * L::QP + ks * 32 + 8 * q4);
#pragma unroll
                        for (int nt = 0; nt < NTW; ++nt) O[nt][m] = E::mma(sf[nt], b, O[nt][m]);
                    }
                } else {
                    // exact chunk with q^ over the q tile: block m's rows hold
                    // scale q exp2(Gc - r_m); times exp2(r_m) per key dim (r_m, the
                    // gates of the blocks before m, <= 0) gives the chunk-start form
                    const int d0 = ks * 32 + 4 * q4;
                    f32x4_t x0 = {0.f, 0.f, 0.f, 0.f}, x1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int m = 0; m < NB; ++m) {
                        float qv[8];
                        E::unpack(E::ld_frag(sQh + (16 * m + n16) * L::QP + ks * 32 + 8 * q4), qv);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            qv[e] *= fexp2(x0[e]);
                            qv[4 + e] *= fexp2(x1[e]);
                        }
                        const frag_t b = E::pack(qv);
#pragma unroll
                        for (int nt = 0; nt < NTW; ++nt) O[nt][m] = E::mma(sf[nt], b, O[nt][m]);
                        x0 += blk4(m, d0);
                        x1 += blk4(m, d0 + 16);
                    }
                }
            }
            // intra-chunk: O^T += V^T A^T over causal token steps
#pragma unroll
            for (int m = 0; m < NB; ++m) {
#pragma unroll
                for (int ts = 0; ts < TS; ++ts) {
                    if (ts * 32 > 16 * m + 15) continue;
                    const frag_t b = E::ld_frag(sA + (16 * m + n16) * L::TP + ts * 32 + 8 * q4);
#pragma unroll
                    for (int nt = 0; nt < NTW; ++nt) O[nt][m] = E::mma(vf[nt][ts], b, O[nt][m]);
                }
            }
            if (p.o) {   // no o when only the chunk-start states are wanted (backward)
                const rsrc_t bo = make_rsrc(reinterpret_cast<gmem_t *>(p.o) + bh * long(T) * D, long(T) * D * es);
#pragma unroll
                for (int m = 0; m < NB; ++m) {
                    const int row = t0 + 16 * m + n16;   // rows past T are dropped
#pragma unroll
                    for (int nt = 0; nt < NTW; ++nt)
                        E::st4(bo, (row * D + vb + 16 * nt + 4 * q4) * es, O[nt][m]);
                }
            }
        }

        // ---- a3: S <- diag(exp2 Gamma) S + Kht^T V ------------------------------
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const f32x4_t egv = *reinterpret_cast<const f32x4_t *>(sEG + 16 * mt + 4 * q4);
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
                for (int e = 0; e < 4; ++e) S[mt][nt][e] *= egv[e];
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
            for (int ts = 0; ts < TS; ++ts) {
                const frag_t a = E::ld_frag(sKht + (16 * mt + n16) * L::TP + ts * 32 + 8 * q4);
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt) S[mt][nt] = E::mma(a, vf[nt][ts], S[mt][nt]);
            }
        }
        buf ^= 1;
    }
    wait_vmem<0>();   // no direct load may land after the work-group ends

    // ---- segment end --------------------------------------------------------
    if constexpr (kState) {
        float *dst = nullptr;
        if constexpr (kFrom) {
            if (seg == p.P - 1 && p.h_final) dst = p.h_final + bh * long(D) * D;
        } else {
            dst = p.ws_E + (bhl * p.ws_slots + seg) * long(D) * D;
            if (w == 0)
#pragma unroll
                for (int u = 0; u < CPL; ++u)
                    p.ws_G[(bhl * p.ws_slots + seg) * D + lane * CPL + u] = seg_gamma[u];
        }
        if (dst) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        dst[(16 * mt + 4 * q4 + e) * D + vb + 16 * nt + n16] = S[mt][nt][e];
        }
    }
}

// ---------------------------------------------------------------------------
// State pass, bf16: the end state of each state unit (a run of chunks) from a
// zero start, S <- diag(exp2 Gamma) S + (k exp2(Gamma - Gc))^T V per chunk,
// and the unit's total log2-decay.  NST-stage pipeline (four stages at
// D = 128, C = 64, else three), so that NST - 1 chunks' rows are on their way
// from HBM while one is worked on: key and value rows go straight into LDS
// (NST buffers each), gate rows into registers (NST sets); chunk c + NST - 1
// is requested at the first barrier of chunk c, once every wave is done with
// chunk c - 1's buffers.  The compiler adds its own wait for the gate
// registers at the start of a step, counting the loads it knows were issued
// after them.  Four stages issue the key and value rows with the builtin
// direct loads, which it counts, so that wait holds only for chunk c (chunks
// c + 1 and c + 2 stay in flight; in the generated code it is vmcnt(46), and
// no other wait precedes the transposing reads).  Three stages issue them
// untracked (below), and the compiler's wait, blind to them, then also holds
// for chunk c + 1's rows.
// Wave w owns the gate / key rows [r0, r0 + RPW) for the exponent sums and
// value columns [w*D/NW, (w+1)*D/NW) of S.  The k~^T and V operands of the
// update are read as MFMA fragments with transposing LDS reads.
// ---------------------------------------------------------------------------
template <int D, int C> struct StateLayout {
    static constexpr int NW = Shape<D, C>::NW;
    static constexpr int VP = D * 2 + 32;    // padded bf16 row pitch (bytes) of the v tiles
    static constexpr int KB = C * D * 2;     // raw key tile, dense rows
    static constexpr int VB = BF16::tile_bytes(C, VP);   // value tile
    // D = 128, C = 64: four stages (three chunks in flight), which fit only
    // with the scaled key tile in dense swizzled rows (KKB = KB); other shapes
    // keep three stages and the padded layout for that tile
    static constexpr bool kFour = D == 128 && C == 64;
    static constexpr int NST = kFour ? 4 : 3;
    static constexpr int KKB = kFour ? KB : VB;
    static constexpr int bytes = NST * (KB + VB) + KKB + NW * D * 4;
    static_assert(bytes <= 163840, "state pass LDS");
};

// Scaled key tile of the four-stage state pass: dense 256-byte rows (D = 128
// bf16) whose 8-byte units are permuted by row, unit u of row r stored at
// u ^ (4 (r % 4) + 16 ((r / 8) % 2)).  A transposing read touches rows
// k0..k0+3 (k0 a multiple of 4) and four aligned units of each: the XOR
// with 4 (r % 4) spreads them over 16 distinct units, and rows eight apart
// (the next 16-lane group) go to the other half of the row's units.
__device__ __forceinline__ int kk_swz(int r) { return ((r & 3) << 2) | (((r >> 3) & 1) << 4); }
__device__ __forceinline__ int kk_off(int r, int u) { return r * 256 + ((u ^ kk_swz(r)) << 3); }
// 8 consecutive tokens (k0 a multiple of 8) of column c0 + (lane % 16) of that tile
__device__ __forceinline__ bf16x8_t kk_col8(const unsigned char *tile, int k0, int c0, int n16) {
    typedef short s4_t __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s4_t *lds_s4_p;
    const int r = k0 + (n16 >> 2), u = (c0 >> 2) + (n16 & 3);
    const s4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4_p)(tile + kk_off(r, u)));
    const s4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4_p)(tile + kk_off(r + 4, u)));
    typedef short s8_t __attribute__((ext_vector_type(8)));
    const s8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8_t, v);
}

// BWD = true: the backward's segment pass with the same machinery.  Fed with
// k := q, v := do, it forms each segment's contribution to the gradient of
// the state before the segment, sum_t scale (q_t e^{gates from the segment
// start through t})^T do_t (rows of the first chunk in the segment first, the
// prefix decay folded into the q rows), for segments P-1 .. 1 into slots
// 0 .. P-2 (slot = block x, segment = ws_slots - slot), plus the segment's
// total log2-decay: what the backward scan takes.
template <int D, int C, bool SG, bool BWD>
__global__ void __launch_bounds__((Shape<D, C>::NW * 64))
state_kernel(const KernelParams p) {
    using E = BF16;
    using L = StateLayout<D, C>;
    constexpr int NW = Shape<D, C>::NW;
    constexpr int RPW = Shape<D, C>::RPW;
    constexpr int CPL = D / 64;
    constexpr int VS = D / NW;
    constexpr int NTW = VS / 16;
    constexpr int MT = D / 16;
    constexpr int TS = C / 32;
    constexpr int NKL = RPW * D * 2 / 1024;   // direct loads per wave and chunk: keys
    constexpr int NVL = RPW;                  // values (one per row)
    constexpr int NCH = RPW + NKL + NVL;      // vector-memory operations per wave and chunk
    constexpr int NST = L::NST;               // pipeline stages (chunks in flight: NST - 1)
    static_assert(RPW * D * 2 % 1024 == 0, "key rows per wave must fill whole loads");
    // (waits past 63 are clamped, which only waits longer; the four-stage
    // shape keeps every count exact)
    static_assert(NST == 3 || NVL + (NST - 1) * NCH <= 63, "four stages: loads in flight must fit the vmcnt counter");
    typedef typename E::frag_t frag_t;

    // Separate arrays per buffer: the compiler can then tell that fragment
    // reads of one buffer do not touch the loads landing in another.
    constexpr int KB3 = NST == 4 ? L::KB : 16, VB3 = NST == 4 ? L::VB : 16;   // fourth stage
    __shared__ __attribute__((aligned(16))) unsigned char sK0[L::KB], sK1[L::KB], sK2[L::KB], sK3[KB3];
    __shared__ __attribute__((aligned(16))) unsigned char sV0[L::VB], sV1[L::VB], sV2[L::VB], sV3[VB3];
    __shared__ __attribute__((aligned(16))) unsigned char sKK[L::KKB];  // k exp2(Gamma - Gc), rows
    __shared__ __attribute__((aligned(16))) float sBt[NW * D];          // wave totals

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int n16 = lane & 15;
    const int q4 = lane >> 4;
    static_assert(!(BWD && SG), "the backward takes per-key-dim gates");
    const int slot = blockIdx.x;
    const int seg = BWD ? p.ws_slots - slot : slot;
    const long bhl = blockIdx.y;
    const long bh = p.bh0 + bhl;
    const int T = p.T;
    const int c_begin = seg * p.cps;
    const int c_end = min(p.N, c_begin + p.cps);
    const int vb = w * VS;
    const int r0 = RPW * w;

    const rsrc_t bk = make_rsrc(reinterpret_cast<const uint16_t *>(p.k) + bh * long(T) * D, long(T) * D * 2);
    const rsrc_t bv = make_rsrc(reinterpret_cast<const uint16_t *>(p.v) + bh * long(T) * D, long(T) * D * 2);
    constexpr int GD = SG ? 1 : D;   // gates per token (SG: one scalar gate per token)
    const rsrc_t bg = make_rsrc(p.g + bh * long(T) * GD, long(T) * GD * 4);
    const u32x4_t wk = rsrc_words(reinterpret_cast<const uint16_t *>(p.k) + bh * long(T) * D, long(T) * D * 2);
    const u32x4_t wv = rsrc_words(reinterpret_cast<const uint16_t *>(p.v) + bh * long(T) * D, long(T) * D * 2);

    RawG<CPL> rg0[RPW], rg1[RPW], rg2[RPW], rg3[NST == 4 ? RPW : 1];   // gate rows per stage

    // this wave's gate rows (registers), key and value rows (LDS) of chunk c
    // (rows past T read as zero).  Issue order g, k, v is what the waits count on.
    // Three stages: the key and value rows are untracked direct loads
    // (dma_untracked): an earlier three-stage build with the builtin form had
    // the compiler wait for all loads in flight, the next two chunks'
    // included, before the first transposing read of each step.
    auto issue = [&](int c, RawG<CPL> *tg, unsigned char *tk, unsigned char *tv) {
        const int row0 = __builtin_amdgcn_readfirstlane(c * C + r0);
        const int lr0 = __builtin_amdgcn_readfirstlane(r0);
        mem_fence_compiler();
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            if constexpr (SG) tg[i].load_one(bg, row0 * 4, i * 4);   // same address in every lane
            else tg[i].load(bg, (row0 * D + lane * CPL) * 4, i * D * 4);
        }
        if constexpr (L::kFour) {   // tracked: the compiler's own waits then count them
#pragma unroll
            for (int i = 0; i < NKL; ++i) dma<16>(bk, tk + lr0 * D * 2 + i * 1024, lane * 16, row0 * D * 2 + i * 1024);
#pragma unroll
            for (int i = 0; i < NVL; ++i) dma<4>(bv, tv + E::rowoff(lr0 + i, L::VP), lane * 4, (row0 + i) * D * 2);
        } else {
#pragma unroll
            for (int i = 0; i < NKL; ++i)
                dma_untracked<16>(wk, lds_addr(tk) + lr0 * D * 2 + i * 1024, lane * 16, row0 * D * 2 + i * 1024);
#pragma unroll
            for (int i = 0; i < NVL; ++i)   // 4 bytes per lane: a 64-wide row takes lanes 0..31
                if (CPL == 2 || lane < 32) dma_untracked<4>(wv, lds_addr(tv) + E::rowoff(lr0 + i, L::VP), lane * 4, (row0 + i) * D * 2);
        }
        mem_fence_compiler();
    };

    f32x4_t S[MT][NTW];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) S[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float seg_gamma[CPL];
#pragma unroll
    for (int u = 0; u < CPL; ++u) seg_gamma[u] = 0.f;

    // Steps c_begin .. c_end - 1 take the unit's chunks last to first:
    //     E = sum_c diag(exp(gates after chunk c)) (k_c exp(Gamma_c - Gc))^T V_c,
    // with the decays after the chunk (seg_gamma, log2 units) folded into the
    // key rows, so the accumulators are never rescaled.  The unit's first
    // chunks are then the ones read last, which the output pass reads first.
    // (BWD: first chunk first, the decay of every earlier chunk folded in)
    auto chunk_of = [&](int c) { return BWD ? c : c_end - 1 - (c - c_begin); };
    auto stage_g = [&](auto bsel) -> RawG<CPL> * {
        constexpr int B = decltype(bsel)::value;
        if constexpr (B == 0) return rg0; else if constexpr (B == 1) return rg1;
        else if constexpr (B == 2) return rg2; else return rg3;
    };
    auto stage_k = [&](auto bsel) -> unsigned char * {
        constexpr int B = decltype(bsel)::value;
        if constexpr (B == 0) return sK0; else if constexpr (B == 1) return sK1;
        else if constexpr (B == 2) return sK2; else return sK3;
    };
    auto stage_v = [&](auto bsel) -> unsigned char * {
        constexpr int B = decltype(bsel)::value;
        if constexpr (B == 0) return sV0; else if constexpr (B == 1) return sV1;
        else if constexpr (B == 2) return sV2; else return sV3;
    };
    // one chunk from stage B while the next NST - 1 chunks load into the others
    auto step = [&](int c, auto bsel) {
        RawG<CPL> *rg = stage_g(bsel);
        unsigned char *kt = stage_k(bsel);
        unsigned char *vt = stage_v(bsel);
        // this wave's key rows of chunk c arrived (after them: its value rows
        // and all of chunks c + 1 .. c + NST - 2); the gate registers are
        // waited for by the compiler
        wait_vmem<NVL + (NST - 2) * NCH>();
        Raw<E, CPL> rk[RPW];
#pragma unroll
        for (int i = 0; i < RPW; ++i)
            rk[i].x = *reinterpret_cast<const decltype(rk[i].x) *>(kt + ((r0 + i) * D + lane * CPL) * 2);
        // gate sums in log2 units, per wave: the suffix after each row (BWD: the
        // prefix through each row) and the total
        float Sw[RPW][CPL];
#pragma unroll
        for (int u = 0; u < CPL; ++u) {
            float run = 0.f;
            if constexpr (BWD) {
#pragma unroll
                for (int i = 0; i < RPW; ++i) {
                    run = __builtin_fmaf(rg[i].get(u), kLog2e, run);
                    Sw[i][u] = run;
                }
            } else {
#pragma unroll
                for (int i = RPW - 1; i >= 0; --i) {
                    Sw[i][u] = run;
                    run = __builtin_fmaf(rg[i].get(u), kLog2e, run);
                }
            }
            sBt[w * D + lane * CPL + u] = run;
        }
        block_sync();  // B1: wave totals visible; every wave is done with chunk c - 1
        // chunk c - 1's stage is free: request chunk c + NST - 1 (near the end
        // the last chunk is requested again, so the waits count the same loads)
        {
            constexpr int N2 = (decltype(bsel)::value + NST - 1) % NST;
            const auto nsel = std::integral_constant<int, N2>{};
            issue(chunk_of(min(c + NST - 1, c_end - 1)), stage_g(nsel), stage_k(nsel), stage_v(nsel));
        }

        // gates after the wave's rows: the rest of the chunk and every later chunk
        // (BWD: before them, the earlier waves' rows and every earlier chunk)
        float aw[CPL];
#pragma unroll
        for (int u = 0; u < CPL; ++u) {
            float other = 0.f, tot = 0.f;
#pragma unroll
            for (int j = 0; j < NW; ++j) {
                const float t = sBt[j * D + lane * CPL + u];
                if (BWD ? j < w : j > w) other += t;
                tot += t;
            }
            aw[u] = other + seg_gamma[u];
            seg_gamma[u] += tot;
        }
        // k exp2(gates after row i) (BWD: scale q exp2(gates through row i)):
        // sums of gates <= 0, rows into the k~ tile
        const float rs = BWD ? p.scale : 1.f;
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            float kk[CPL];
#pragma unroll
            for (int u = 0; u < CPL; ++u) kk[u] = rk[i].get(u) * (rs * fexp2(aw[u] + Sw[i][u]));
            __bf16 *dst = L::kFour
                              ? reinterpret_cast<__bf16 *>(sKK + kk_off(r0 + i, lane >> 1) + (lane & 1) * 4)
                              : reinterpret_cast<__bf16 *>(sKK + E::rowoff(r0 + i, L::VP)) + lane * CPL;
            if constexpr (CPL == 2) {
                typedef __bf16 b2_t __attribute__((ext_vector_type(2)));
                *reinterpret_cast<b2_t *>(dst) = b2_t{(__bf16)kk[0], (__bf16)kk[1]};
            } else {
                dst[0] = (__bf16)kk[0];
            }
        }
        wait_vmem<(NST - 1) * NCH>();   // this chunk's value rows arrived (after them: chunks c + 1 .. c + NST - 1)
        block_sync();  // B2: k~ tile, value rows and decays visible

        frag_t vf[NTW][TS];
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
            for (int ts = 0; ts < TS; ++ts) vf[nt][ts] = E::ld_col8(vt, L::VP, ts * 32 + 8 * q4, vb + 16 * nt, n16);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int ts = 0; ts < TS; ++ts) {
                const frag_t a = L::kFour ? kk_col8(sKK, ts * 32 + 8 * q4, 16 * mt, n16)
                                          : E::ld_col8(sKK, L::VP, ts * 32 + 8 * q4, 16 * mt, n16);
#pragma unroll
                for (int nt = 0; nt < NTW; ++nt) S[mt][nt] = E::mma(a, vf[nt][ts], S[mt][nt]);
            }
    };

    if (c_begin < c_end) {   // prologue: the first NST - 1 chunks
        issue(chunk_of(c_begin), rg0, sK0, sV0);
        issue(chunk_of(min(c_begin + 1, c_end - 1)), rg1, sK1, sV1);
        if constexpr (NST == 4) issue(chunk_of(min(c_begin + 2, c_end - 1)), rg2, sK2, sV2);
    }
    // whole rounds of NST, then the remainder, so that every path into a
    // step has issued the same loads (the waits stay tight)
    const auto s0 = std::integral_constant<int, 0>{};
    const auto s1 = std::integral_constant<int, 1>{};
    const auto s2 = std::integral_constant<int, 2>{};
    const auto s3 = std::integral_constant<int, NST == 4 ? 3 : 0>{};
    int c = c_begin;
    for (; c + NST <= c_end; c += NST) {
        step(c, s0);
        step(c + 1, s1);
        step(c + 2, s2);
        if constexpr (NST == 4) step(c + 3, s3);
    }
    // nested, so that each remainder step is reached only through the one
    // before it (the compiler's wait counts then see every load issued)
    if (c < c_end) {
        step(c, s0);
        if (c + 1 < c_end) {
            step(c + 1, s1);
            if constexpr (NST == 4) if (c + 2 < c_end) step(c + 2, s2);
        }
    }
    wait_vmem<0>();   // no direct load may land after the work-group ends

    float *dst = p.ws_E + (bhl * p.ws_slots + slot) * long(D) * D;
    if (w == 0)
#pragma unroll
        for (int u = 0; u < CPL; ++u) p.ws_G[(bhl * p.ws_slots + slot) * D + lane * CPL + u] = seg_gamma[u];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
            for (int e = 0; e < 4; ++e) dst[(16 * mt + 4 * q4 + e) * D + vb + 16 * nt + n16] = S[mt][nt][e];
}

// Exclusive scan of the state-pass maps: E_j <- S_start(j+1) in place.
// One thread per (head, key dim, value column).
__global__ void __launch_bounds__(256)
scan_kernel(float *__restrict__ ws_E, const float *__restrict__ ws_G,
            const float *__restrict__ h0, long bh0, int nbh, int slots, int D) {
    const long idx = long(blockIdx.x) * 256 + threadIdx.x;
    const long DD = long(D) * D;
    if (idx >= long(nbh) * DD) return;
    const long bhl = idx / DD;
    const long dv = idx - bhl * DD;
    const int d = int(dv / D);
    float s = h0 ? h0[(bh0 + bhl) * DD + dv] : 0.f;
    float *e = ws_E + bhl * (slots) * DD + dv;
    const float *gm = ws_G + bhl * (slots) * D + d;
    constexpr int U = 8;   // segment states loaded ahead of the dependent chain
    for (int r0 = 0; r0 < slots; r0 += U) {
        float ev[U], gv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (r0 + u < slots) {
                ev[u] = e[long(r0 + u) * DD];
                gv[u] = gm[long(r0 + u) * D];
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (r0 + u < slots) {
                s = fexp2(gv[u]) * s + ev[u];
                e[long(r0 + u) * DD] = s;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Decode step: one new token per (batch, head), the state updated in place,
//   S <- diag(exp g) S + k^T v,   o = scale q S   (update, then read out)
// the same recurrence one token at a time (blog "Linear Attention 在 GPU 上到底
// 慢在哪", section 学长的反馈; "线性注意力GPU算子库的定义与技术解析", section 四).
// Bound by the state traffic: each (batch, head) reads and writes D*D fp32.
// Work-group = one (batch, head), 256 threads: thread t owns value columns
// 4 (t % QN) .. +3 (QN = D / 4 column quads) and state rows t / QN + RB i
// (RB = 256 / QN row groups), each row piece one 16-byte load and store.
// Whole rows per work-group measured faster than 32 or 64 columns (fewer,
// longer work-groups with more state in flight each).
// ---------------------------------------------------------------------------
template <typename E, int D>
__global__ void __launch_bounds__(256)
decode_kernel(const void *__restrict__ q, const void *__restrict__ k, const void *__restrict__ v,
              const float *__restrict__ g, float *__restrict__ state, void *__restrict__ o, float scale) {
    using gmem_t = typename E::gmem_t;
    constexpr int QN = D / 4;       // column quads
    constexpr int RB = 256 / QN;    // row groups
    static_assert(QN <= 64 && D % RB == 0, "decode tile");
    const long bh = blockIdx.x;
    const int t = threadIdx.x;
    const int cq = t % QN;
    const int rb = t / QN;
    const gmem_t *qp = reinterpret_cast<const gmem_t *>(q) + bh * D;
    const gmem_t *kp = reinterpret_cast<const gmem_t *>(k) + bh * D;
    const gmem_t *vp = reinterpret_cast<const gmem_t *>(v) + bh * D;
    const float *gp = g + bh * D;
    float *S = state + bh * D * D + 4 * cq;
    float vv[4], acc[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        vv[e] = E::g2f(vp[4 * cq + e]);
        acc[e] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < D / RB; ++i) {
        const int r = rb + RB * i;
        const float dec = fexp2(gp[r] * kLog2e);
        const float kr = E::g2f(kp[r]), qr = E::g2f(qp[r]);
        f32x4_t sv = *reinterpret_cast<const f32x4_t *>(S + r * D);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            sv[e] = __builtin_fmaf(kr, vv[e], dec * sv[e]);
            acc[e] = __builtin_fmaf(qr, sv[e], acc[e]);
        }
        *reinterpret_cast<f32x4_t *>(S + r * D) = sv;
    }
    // sum over the row groups: 64 / QN per wave (lane / QN), then over the 4 waves
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int m = QN; m <= 32; m <<= 1) acc[e] += __shfl_xor(acc[e], m, 64);
    __shared__ float red[4][D];
    if ((t & 63) < QN)
#pragma unroll
        for (int e = 0; e < 4; ++e) red[t >> 6][4 * cq + e] = acc[e];
    __syncthreads();
    if (t < D) {
        const float x = scale * (red[0][t] + red[1][t] + red[2][t] + red[3][t]);
        if constexpr (sizeof(gmem_t) == 2) reinterpret_cast<__bf16 *>(o)[bh * D + t] = (__bf16)x;
        else reinterpret_cast<float *>(o)[bh * D + t] = x;
    }
}

// T == 0: h_final <- h0 (or 0).
__global__ void __launch_bounds__(256)
copy_state_kernel(float *__restrict__ dst, const float *__restrict__ src, long n) {
    const long i = long(blockIdx.x) * 256 + threadIdx.x;
    if (i < n) dst[i] = src ? src[i] : 0.f;
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <typename E, int D, int C, int MODE, bool SG>
static hipError_t launch_one(const KernelParams &p, int grid_x, int grid_y, hipStream_t s) {
    if (grid_x <= 0 || grid_y <= 0) return hipSuccess;
    hipLaunchKernelGGL((chunk_kernel<E, D, C, MODE, SG>), dim3(grid_x, grid_y), dim3(Shape<D, C>::NW * 64), 0, s, p);
    return hipGetLastError();
}

template <int D, int C, bool SG, bool BWD = false>
static hipError_t launch_state(const KernelParams &p, int grid_x, int grid_y, hipStream_t s) {
    if (grid_x <= 0 || grid_y <= 0) return hipSuccess;
    hipLaunchKernelGGL((state_kernel<D, C, SG, BWD>), dim3(grid_x, grid_y), dim3(Shape<D, C>::NW * 64), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_bwd_segments(int D, int C, const KernelParams &p, int grid_x, int grid_y, hipStream_t s) {
    if (D == 128 && C == 64) return launch_state<128, 64, false, true>(p, grid_x, grid_y, s);
    if (D == 128 && C == 32) return launch_state<128, 32, false, true>(p, grid_x, grid_y, s);
    if (D == 64 && C == 64) return launch_state<64, 64, false, true>(p, grid_x, grid_y, s);
    if (D == 64 && C == 32) return launch_state<64, 32, false, true>(p, grid_x, grid_y, s);
    return hipErrorInvalidValue;
}

// Chunk 128 has no state pass of its own: its state units run on 64-token
// chunks (state_chunk below).
template <typename E, int D, int C>
static hipError_t dispatch_mode(int mode, bool sg, const KernelParams &p, int gx, int gy, hipStream_t s) {
    constexpr bool seg_ok = C <= 64;
    if (sg) {   // scalar gates: the fused output pass and the state pass only
        switch (mode) {
            case MODE_OUT: return launch_one<E, D, C, MODE_OUT, true>(p, gx, gy, s);
            case MODE_SEG:
                if constexpr (!seg_ok) return hipErrorInvalidValue;
                else if constexpr (std::is_same<E, BF16>::value) return launch_state<D, C, true>(p, gx, gy, s);
                else return launch_one<E, D, C, MODE_SEG, true>(p, gx, gy, s);
            default: return hipErrorInvalidValue;
        }
    }
    switch (mode) {
        case MODE_OUT: return launch_one<E, D, C, MODE_OUT, false>(p, gx, gy, s);
        case MODE_SEG:
            if constexpr (!seg_ok) return hipErrorInvalidValue;
            else if constexpr (std::is_same<E, BF16>::value) return launch_state<D, C, false>(p, gx, gy, s);
            else return launch_one<E, D, C, MODE_SEG, false>(p, gx, gy, s);
        case MODE_STATES:
            if constexpr (!seg_ok) return hipErrorInvalidValue;
            else return launch_one<E, D, C, MODE_STATES, false>(p, gx, gy, s);
        case MODE_INTRA: return launch_one<E, D, C, MODE_INTRA, false>(p, gx, gy, s);
        case MODE_CUMSUM: return launch_one<E, D, C, MODE_CUMSUM, false>(p, gx, gy, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_chunk_kernel(int dtype, int D, int C, int mode, bool scalar_gate,
                               const KernelParams &p, int gx, int gy, hipStream_t s) {
    const bool sg = scalar_gate;
    if (dtype == DTYPE_BF16) {
        if (D == 128 && C == 128) return dispatch_mode<BF16, 128, 128>(mode, sg, p, gx, gy, s);
        if (D == 128 && C == 64) return dispatch_mode<BF16, 128, 64>(mode, sg, p, gx, gy, s);
        if (D == 128 && C == 32) return dispatch_mode<BF16, 128, 32>(mode, sg, p, gx, gy, s);
        if (D == 64 && C == 64) return dispatch_mode<BF16, 64, 64>(mode, sg, p, gx, gy, s);
        if (D == 64 && C == 32) return dispatch_mode<BF16, 64, 32>(mode, sg, p, gx, gy, s);
        if (D == 64 && C == 128) return dispatch_mode<BF16, 64, 128>(mode, sg, p, gx, gy, s);
    } else if (dtype == DTYPE_F32) {
        if (D == 64 && C == 64) return dispatch_mode<F32, 64, 64>(mode, sg, p, gx, gy, s);
        if (D == 64 && C == 32) return dispatch_mode<F32, 64, 32>(mode, sg, p, gx, gy, s);
        if (D == 128 && C == 32) return dispatch_mode<F32, 128, 32>(mode, sg, p, gx, gy, s);
        if (D == 128 && C == 64) return dispatch_mode<F32, 128, 64>(mode, sg, p, gx, gy, s);
    }
    return hipErrorInvalidValue;
}

int state_units_per_cu(int dtype, int D, int C) {
    int bytes = 0;
    if (dtype == DTYPE_BF16) {
        if (D == 128 && C == 64) bytes = StateLayout<128, 64>::bytes;
        if (D == 128 && C == 32) bytes = StateLayout<128, 32>::bytes;
        if (D == 64 && C == 64) bytes = StateLayout<64, 64>::bytes;
        if (D == 64 && C == 32) bytes = StateLayout<64, 32>::bytes;
    } else if (dtype == DTYPE_F32) {
        if (D == 64 && C == 64) bytes = Layout<F32, 64, 64, MODE_SEG>::bytes;
        if (D == 64 && C == 32) bytes = Layout<F32, 64, 32, MODE_SEG>::bytes;
        if (D == 128 && C == 32) bytes = Layout<F32, 128, 32, MODE_SEG>::bytes;
        if (D == 128 && C == 64) bytes = Layout<F32, 128, 64, MODE_SEG>::bytes;
    }
    if (bytes <= 0) return 1;
    return std::max(1, std::min(2, 163840 / bytes));
}

bool chunk_supported(int dtype, int D, int C) {
    if (dtype == DTYPE_BF16) return (D == 128 || D == 64) && (C == 128 || C == 64 || C == 32);
    if (dtype == DTYPE_F32) return (D == 64 || D == 128) && (C == 64 || C == 32);
    return false;
}

int state_chunk(int dtype, int C) { return dtype == DTYPE_BF16 && C == 128 ? 64 : C; }

hipError_t launch_scan(float *ws_E, const float *ws_G, const float *h0, long bh0, int nbh,
                       int slots, int D, hipStream_t s) {
    const long n = long(nbh) * D * D;
    const long blocks = (n + 255) / 256;
    hipLaunchKernelGGL(scan_kernel, dim3(unsigned(blocks)), dim3(256), 0, s, ws_E, ws_G, h0, bh0, nbh, slots, D);
    return hipGetLastError();
}

hipError_t launch_decode(int dtype, int D, const void *q, const void *k, const void *v, const float *g,
                         float *state, void *o, long nbh, float scale, hipStream_t s) {
    if (nbh <= 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>(nbh));
    if (dtype == DTYPE_BF16) {
        if (D == 128) hipLaunchKernelGGL((decode_kernel<BF16, 128>), grid, dim3(256), 0, s, q, k, v, g, state, o, scale);
        else if (D == 64) hipLaunchKernelGGL((decode_kernel<BF16, 64>), grid, dim3(256), 0, s, q, k, v, g, state, o, scale);
        else return hipErrorInvalidValue;
    } else {
        if (D == 128) hipLaunchKernelGGL((decode_kernel<F32, 128>), grid, dim3(256), 0, s, q, k, v, g, state, o, scale);
        else if (D == 64) hipLaunchKernelGGL((decode_kernel<F32, 64>), grid, dim3(256), 0, s, q, k, v, g, state, o, scale);
        else return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_copy_state(float *dst, const float *src, long n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    const long blocks = (n + 255) / 256;
    hipLaunchKernelGGL(copy_state_kernel, dim3(unsigned(blocks)), dim3(256), 0, s, dst, src, n);
    return hipGetLastError();
}

}  // namespace gla
